// Backward: causal packed-document attention on token-block MXFP8 operands
// (jaehun.me review §1.2 gradient products, §3.1 operand formats, §3.2 dQ prescale,
//  §3.3 recomputation with the same quantised operands and block-scaled dS, §3.4 backward pass,
//  packed documents and work scheduling).
//
// Three launches.
//
// Prologue: one workgroup per query head computes the dQ prescale exponent pi of every row and
// zeroes the gradients of rows outside every document; one more workgroup lays out the dShat
// store (a prefix sum over documents) and checks that it fits the workspace.
//
// Key-stationary kernel (dK, dV, dShat): persistent grid, one 256-thread workgroup per compute
// unit.  A work unit is (backward item = 128-key tile kappa of a document, KV head).  Wave w owns
// keys 32w..32w+31; K^T and V for those keys stay in registers as MFMA operands, dK^T and dV^T
// accumulate in registers over all query heads of the group and all 64-query steps from the
// diagonal to the document end.  Per step:
//   S  (queries x keys) = Q K^T  and  dP = dO V^T          (A from the row-major Q / dO tiles)
//     -> the score t is bit-identical to the forward's: same codes, scales, instruction and
//        K ordering (the instruction gives identical results with its operands swapped);
//   P = 2^(t - LSE), dS = P (dP - D); each wave's 32x32 blocks of P and dS get a round-up E8M0
//     exponent from a wave-wide amax and E4M3 codes, already in operand order;
//   dV^T += dO^T Phat,  dK^T += Q^T dShat                   (A via transpose reads of the tiles)
//   dShat codes and exponents -> workspace, one 8 KiB block per (64-query tile, key tile, head).
// Steps whose 64 x 128 pairs are all visible skip the mask.  The Q / dO tiles of the next step
// are loaded while the current one computes (two LDS buffers, one barrier per step).
// A document with a single key tile has only one dQ contribution per row: its unit computes
// dQ = K^T dShat^T itself (dShat staged in LDS) and writes it, and nothing is stored.
//
// Query-stationary kernel (dQ of documents with two or more key tiles): a work unit is
// (half of a forward item = 128 queries of a document, query head), two workgroups of four
// waves per CU (twice the loads in flight of one larger workgroup); wave w owns 32 queries.
// Over the key
// tiles kappa = 0, 1, ... in ascending order it reads the stored dShat blocks and the K tile,
// forms partial = K^T dShat^T (FP32) and accumulates acc16 = FP16(acc16 + FP16(2^pi partial))
// in registers; at the end dQ = BF16(softmax_scale 2^-pi acc16).  The reduction order is fixed,
// so results are bit-reproducible, and no workgroup waits for another.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace flamia {

namespace {

constexpr int BWD_WAVES = 8;   // 4 producer + 4 consumer waves, one of each per SIMD
constexpr int BWD_THREADS = 64 * BWD_WAVES;
constexpr int QT = 64;                 // queries per step / per stored dShat block
constexpr int DS_BLOCK = KV_TILE * QT;  // code bytes of one stored dShat block
constexpr int NBUF = 4;                 // step tile buffers of the key-stationary pass
// codes, then the 8 exponent bytes in a 128-byte line of their own: every block starts on a cache
// line, so its 1 KiB stores and loads cover whole lines
constexpr int DS_STRIDE = DS_BLOCK + 128;
constexpr int DQ_QT = 2;               // 64-query tiles per dQ workgroup (two workgroups per CU)
constexpr int DQ_WAVES = 2 * DQ_QT;
constexpr int DQ_THREADS = 64 * DQ_WAVES;

// Query offset (within a 64-query tile) held at byte position pos of a dShat row as assembled in
// LDS by the dQ pass: the row of key j holds, for lane group hh of the wave that owns j, the 32
// bytes of its P-operand register order (query 32 qb + 8 w4 + 4 hh + e in byte 4 (4 qb + w4) + e).
__device__ __forceinline__ int ds_pos_query(int pos) {
  const int s = pos >> 5, n = pos & 31;
  return 32 * (n >> 4) + 8 * ((n >> 2) & 3) + 4 * s + (n & 3);
}

template <int D>
struct BwdSmem {
  uint8_t q[NBUF][QT * D];    // step s in buffer s % 4: in phase k producers form the products of
  uint8_t dO[NBUF][QT * D];   // step k + 1, consumers read step k - 1, the loads fill step k + 2
  uint8_t k[KV_TILE * D];
  uint8_t v[KV_TILE * D];
  int4 xp[2][4][2][64];       // Phat operand of (key group) in lane order, 2 x 16 bytes per lane
  int4 xd[2][4][2][64];       // dShat operand
  uint8_t ds[2][KV_TILE * QT];  // dShat [key][query], single-tile documents only
  uint8_t sk[KV_TILE];
  uint8_t sv[KV_TILE];
  float lse[NBUF][QT];
  float dd[NBUF][QT];
  int2 sqdo[NBUF][2];           // block scale bytes {Q, dO} of the step's two query blocks
  int xs_p[2][2][4], xs_d[2][2][4];  // block exponent bytes of (query block, key group)
  uint8_t q4[3][QT * D / 2];   // 4-bit scores: the step's 4-bit Q rows (step s in buffer s % 3)
  union {
    // per-token scales (the precision options), per step row: Q's exponent byte and 2^e(dO_i);
    // dd then holds D_i 2^(e(Q_i) - e(dO_i))
    struct {
      uint8_t sqr[NBUF][QT];
      alignas(16) float pf[NBUF][QT];
    } pr;
    uint8_t sq4[3][QT * D / 32];  // 4-bit scores: each step row's d/32 exponent bytes
  } rt;
};

// Step tiles go from global memory straight into LDS (16-byte direct loads: lane l of a wave
// writes bytes 16 l .. 16 l + 15 of the wave's 1 KiB LDS block), issued by the four consumer
// waves two phases ahead.  Each lane fetches the global chunk that belongs at its LDS position
// under the tile's swizzle.  Rows past the document end repeat its last row, and 1 KiB blocks
// wholly past it are zero-filled instead of loaded: every use of those rows is masked to zero,
// and the values are finite.
template <int D, bool PRECISE, bool QK4>
__device__ __forceinline__ void issue_step_loads(const BwdParams& p, BwdSmem<D>& sm, int b, int doc_start, int L,
                                                 int h, int qt, int cw, int lane, int b3) {
  constexpr int CPR = D / 16;                    // 16-byte chunks per row
  constexpr int BLOCKS = QT * D / 1024;          // 1 KiB wave blocks per tile (4 or 8)
  constexpr int PER_WAVE = 2 * BLOCKS / 4;       // Q and dO blocks per consumer wave
  const int q0 = QT * qt;
  if (q0 + QT <= L) {
    // a tile wholly inside the document: no row clamp, so the wave's blocks (consecutive, of one
    // tensor) are one scalar base each plus the lane's fixed offset; block i sits 64 i / CPR rows
    // below block 0, and the swizzle, a bit permutation of row bits below that step, moves its
    // chunk by the swizzle of the row step alone
    static_assert(BLOCKS % PER_WAVE == 0, "no wave's blocks span both tensors");
    const bool is_do = cw * PER_WAVE >= BLOCKS;
    const int blk0 = cw * PER_WAVE - (is_do ? BLOCKS : 0);
    const uint8_t* base = (is_do ? p.dO : p.q) + ((int64_t)(doc_start + q0 + blk0 * (64 / CPR)) * p.Hq + h) * D;
    const uint32_t voff0 = (uint32_t)((lane / CPR) * p.Hq * D + 16 * ((lane % CPR) ^ lds_swizzle<D>(lane / CPR)));
    uint8_t* dst = (is_do ? sm.dO[b] : sm.q[b]) + blk0 * 1024;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i)
      dma_load16_sv(base + (int64_t)i * (64 / CPR) * p.Hq * D, voff0 ^ (16 * lds_swizzle<D>(i * (64 / CPR))),
                    lds_addr(dst + i * 1024));
  } else {
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int wb = cw * PER_WAVE + i;            // 0 .. 2 BLOCKS - 1: Q blocks, then dO blocks
    const bool is_do = wb >= BLOCKS;
    const int blk = is_do ? wb - BLOCKS : wb;
    const int pos = blk * 64 + lane;             // 16-byte chunk position in the tile
    const int row = pos / CPR, pc = pos % CPR;
    const int lc = pc ^ lds_swizzle<D>(row);     // logical chunk stored at this position
    uint8_t* dst = (is_do ? sm.dO[b] : sm.q[b]) + blk * 1024;
    if (q0 + blk * (1024 / D) < L) {
      const int qr = min(q0 + row, L - 1);
      const uint8_t* src = (is_do ? p.dO : p.q) + ((int64_t)(doc_start + qr) * p.Hq + h) * D + 16 * lc;
      dma_load16(src, lds_addr(dst));
    } else {
      // a block wholly past the document end: zeros (its rows only need to be finite)
      *reinterpret_cast<uint4*>(dst + 16 * lane) = make_uint4(0, 0, 0, 0);
    }
  }
  }
  if constexpr (QK4) {
    // the 4-bit Q rows (d/2 bytes each) into buffer b3: one 1 KiB block per consumer wave
    constexpr int K4B = D / 2, BQ = QT * K4B / 1024, CPR = K4B / 16, RQ = 1024 / K4B;
    if (cw < BQ && QT * qt + QT <= L) {
      // a tile inside the document: one wave-uniform base, and a lane offset that the block's
      // row step (16 or 32 rows) leaves unswizzled
      const int row = lane / CPR;
      const uint32_t voff = (uint32_t)(row * p.Hq * K4B + 16 * ((lane % CPR) ^ lds_swizzle<K4B>(row)));
      const uint8_t* base = p.q4 + ((int64_t)(doc_start + QT * qt + cw * RQ) * p.Hq + h) * K4B;
      dma_load16_sv(base, voff, lds_addr(sm.q4[b3] + cw * 1024));
    } else if (cw < BQ) {
      const int pos = cw * 64 + lane, row = pos / CPR;
      const int lc = (pos % CPR) ^ lds_swizzle<K4B>(row);
      uint8_t* dst = sm.q4[b3] + cw * 1024;
      if (QT * qt + cw * (1024 / K4B) < L) {
        const int qr = min(QT * qt + row, L - 1);
        dma_load16(p.q4 + ((int64_t)(doc_start + qr) * p.Hq + h) * K4B + 16 * lc, lds_addr(dst));
      } else {
        *reinterpret_cast<uint4*>(dst + 16 * lane) = make_uint4(0, 0, 0, 0);
      }
    }
  }
  if (cw == 0 || (cw == 1 && !PRECISE)) {  // row statistics: one float per lane (D: PRECISE, rescaled first)
    const int qr = min(q0 + lane, L - 1);
    const float* src = (cw == 0 ? p.lse : p.Dv) + (int64_t)h * p.T + doc_start + qr;
    dma_load4(src, lds_addr(cw == 0 ? sm.lse[b] : sm.dd[b]));
  }
}

// Key-stationary pass.  Producer wave w (0..3) owns keys 32 w .. 32 w + 31 of the tile: per
// 64-query step it forms S and dP, the softmax terms, and the E4M3 Phat / dShat operands with
// their 32 x 32 block exponents and hands them over in LDS.  Its matrix products run one query
// block ahead of its softmax terms, so the two overlap.
// Consumer wave 4 + w holds dK^T and dV^T of the same keys and runs the gradient products one
// step behind, so its matrix instructions overlap the producer's vector work on the same SIMD;
// it also stores the step's dShat codes and exponents to the workspace.  A wave issues one
// instruction at a time, and the producer's stream is the longer one (it sets the phase
// length), so work that either role can do is given to the consumer.
// Phase k: producers finish step k and form the products of step k + 1, consumers work on step
// k - 1 and load step k + 2; one barrier per phase.
// CAUSAL: keys after the query are masked (else every key of the document is visible).
// PRECISE (the precision options, causal, per-token scales): the products that contract over
// queries take Q and dO with their bare codes, their exponents moving into the other operand
// before it is block-quantised, P'' = P 2^e(dO_i) for dV and dS'' = dS 2^e(Q_i) for dK, so no
// later query changes a block's shared exponent except through values it adds itself; dQ is
// left to a query-stationary pass of its own (nothing is stored).  The folds are exact: D - dP
// comes out as (D - dP) 2^(e(Q_i) - e(dO_i)) from dO's products taken with Q's exponent and an
// accumulator started at D 2^(e(Q_i) - e(dO_i)), and P is multiplied by 2^e(dO_i) after the
// exponential, so their product is dS''.
// QK4 (4-bit scores): S is recomputed from the forward's E2M1 copies of Q (step tiles) and K
// (operand registers), their exponent bytes per 32 channels as the instruction's scales; every
// other product keeps the 8-bit operands.
template <int D, bool CAUSAL, bool PRECISE, bool QK4>
__global__ __launch_bounds__(BWD_THREADS) void bwd_kernel(BwdParams p) {
  static_assert(CAUSAL || !PRECISE, "the precision options are causal");
  static_assert(!(PRECISE && QK4), "separate paths");
  constexpr int NC = D / 64;
  constexpr int NDB = D / 32;
  __shared__ BwdSmem<D> sm;

  if (p.status[0] || p.chunk >= p.status[1]) return;  // not laid out, or a chunk past the last
  const int tid = threadIdx.x;
  // the wave index is uniform: in a scalar register, everything derived from it stays scalar
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const bool producer = wave < 4;
  const int kw = wave & 3;  // key group of both roles
  // this chunk's items: a contiguous range of the backward list
  const int u_lo = p.chunk_start[p.chunk], u_hi = p.chunk_start[p.chunk + 1];
  const int4* items = reinterpret_cast<const int4*>(p.list + 4) + u_lo;
  const int grp = p.Hq / p.Hkv;
  const float c = p.c;
  const int T = p.T;

  // units (item, KV head) are taken dynamically: the list is sorted by descending cost, so the
  // longest left go first to whichever workgroup of the partition is free
  const UnitPartition up = unit_partition(p.Hkv);
  const int n_units = (u_hi - u_lo) * up.kv_per;
  __shared__ int unit_slot;
  int32_t* const counter = p.counters + 16 * p.chunk + up.part;
  for (int u = up.rank; u < n_units; u = next_unit(counter, &unit_slot, up.first)) {
    const int4 it = items[u / up.kv_per];
    const int g = partition_kv(up, u % up.kv_per);
    // unit values are the same in every lane: kept in scalar registers (vector loads would
    // leave them in vector registers for the whole unit)
    const int doc = __builtin_amdgcn_readfirstlane(it.x), kappa = __builtin_amdgcn_readfirstlane(it.y);
    const int doc_start = __builtin_amdgcn_readfirstlane(p.cu[doc]);
    const int L = __builtin_amdgcn_readfirstlane(p.cu[doc + 1]) - doc_start;
    const int n_qt = (L + QT - 1) / QT;
    // two or more key tiles: dQ in the query-stationary kernel (PRECISE: always, from its own
    // recomputation)
    const bool store_ds = !PRECISE && L > KV_TILE;
    int64_t ds_base = 0;  // the item's first block in the chunk's store
    if (store_ds) {
      const int64_t v = p.kv_off[__builtin_amdgcn_readfirstlane(p.tile_base[doc]) + kappa];
      ds_base = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(v >> 32)) << 32) |
                          (uint32_t)__builtin_amdgcn_readfirstlane((int)v));
    }
    const int key_rel = KV_TILE * kappa + 32 * kw + n;
    const bool key_valid = key_rel < L;

    // Steps run over (query head of the group, 64-query tile from the diagonal to the
    // document end).
    // query tiles that see this key tile: from its diagonal on (causal) or all of them
    const int qt_first = CAUSAL ? 2 * kappa : 0;
    const int nq = n_qt - qt_first;  // query tiles per head
    const int n_steps = grp * nq;

    // ---- K / V tiles and the first step's tiles into LDS
    lds_barrier();  // the previous unit no longer reads LDS
    const int cw = wave - 4;  // consumer index (loads)
    // block scales of the two 32-row query blocks of a step: two lanes of consumer 2 load them
    // into registers and store them to LDS at the end of the phase.  PRECISE: consumer 1 loads
    // the per-token exponents and D of the step's 64 rows (one per lane; rows past the document
    // end repeat its last row) and stores the row tables
    auto scale_loads = [&](int h, int qt, int& rsq, int& rsdo, float& rd, uint32_t& rq4) {
      if constexpr (QK4) {
        if (cw == 3) {  // the 4-bit Q exponent bytes of the step's rows, one row per lane
          const int qr = min(QT * qt + lane, L - 1);
          const uint8_t* e4 = p.sq4 + ((int64_t)h * T + doc_start + qr) * (D / 32);
          rq4 = D == 128 ? *reinterpret_cast<const uint32_t*>(e4) : (uint32_t)*reinterpret_cast<const uint16_t*>(e4);
        }
      }
      if constexpr (PRECISE) {
        if (cw == 1) {
          const int qr = min(QT * qt + lane, L - 1);
          const int64_t ti = (int64_t)h * T + doc_start + qr;
          rsq = p.sq[ti];
          rsdo = p.sdo[ti];
          rd = p.Dv[ti];
        }
      } else if (cw == 2 && lane < 2) {
        const int qr = min(QT * qt + 32 * lane, L - 1);
        const int64_t ti = (int64_t)h * T + doc_start + qr;
        rsq = p.sq[ti];
        rsdo = p.sdo[ti];
      }
    };
    auto scale_store = [&](int b, int b3, int qt, int rsq, int rsdo, float rd, uint32_t rq4) {
      if constexpr (QK4) {
        if (cw == 3) {
          if constexpr (D == 128) *reinterpret_cast<uint32_t*>(&sm.rt.sq4[b3][4 * lane]) = rq4;
          else *reinterpret_cast<uint16_t*>(&sm.rt.sq4[b3][2 * lane]) = (uint16_t)rq4;
        }
      }
      if constexpr (PRECISE) {
        if (cw == 1) {
          sm.rt.pr.sqr[b][lane] = (uint8_t)rsq;
          sm.rt.pr.pf[b][lane] = __builtin_ldexpf(1.0f, rsdo - 127);
          sm.dd[b][lane] = __builtin_ldexpf(rd, rsq - rsdo);
        }
      } else if (cw == 2 && lane < 2) {
        int l = lane;
        asm volatile("" : "+v"(l));  // address formed here, not kept in a register all along
        const bool valid = QT * qt + 32 * l < L;
        sm.sqdo[b][l] = make_int2(valid ? rsq : 127, valid ? rsdo : 127);
      }
    };
    // query head and 64-query tile of step st
    auto step_qt = [&](int st, int& h) {
      const int hi = st / nq;
      h = g * grp + hi;
      return qt_first + (st - hi * nq);
    };
    int rsq = 127, rsdo = 127, rsq1 = 127, rsdo1 = 127;
    float rd = 0.f, rd1 = 0.f;
    uint32_t rq4 = 0x7F7F7F7Fu, rq41 = 0x7F7F7F7Fu;
    if (!producer) {
      issue_step_loads<D, PRECISE, QK4>(p, sm, 0, doc_start, L, g * grp, qt_first, cw, lane, 0);
      scale_loads(g * grp, qt_first, rsq, rsdo, rd, rq4);
      if (n_steps > 1) {
        int h1;
        const int qt1 = step_qt(1, h1);
        issue_step_loads<D, PRECISE, QK4>(p, sm, 1, doc_start, L, h1, qt1, cw, lane, 1);
        scale_loads(h1, qt1, rsq1, rsdo1, rd1, rq41);
      }
    }
    {
      constexpr int CPR = D / 16;
      // consumer threads only: the producers' dShat stores stay outside the wait for these loads
      for (int chunk = tid - BWD_THREADS / 2; chunk >= 0 && chunk < KV_TILE * CPR; chunk += BWD_THREADS / 2) {
        const int row = chunk / CPR, col = (chunk % CPR) * 16;
        const int key = KV_TILE * kappa + row;
        uint4 k4 = make_uint4(0, 0, 0, 0), v4 = make_uint4(0, 0, 0, 0);
        if (key < L) {
          const int64_t off = ((int64_t)(doc_start + key) * p.Hkv + g) * D + col;
          k4 = *reinterpret_cast<const uint4*>(p.k + off);
          v4 = *reinterpret_cast<const uint4*>(p.v + off);
          // V is kept negated (E4M3 sign bits flipped, exact): the dP products then come out as
          // D - dP on top of an accumulator that starts at D
          v4.x ^= 0x80808080u; v4.y ^= 0x80808080u; v4.z ^= 0x80808080u; v4.w ^= 0x80808080u;
        }
        *reinterpret_cast<uint4*>(&sm.k[lds_off<D>(row, col)]) = k4;
        *reinterpret_cast<uint4*>(&sm.v[lds_off<D>(row, col)]) = v4;
      }
      if (tid >= BWD_THREADS / 2 && tid < BWD_THREADS / 2 + KV_TILE) {
        const int r = tid - BWD_THREADS / 2;
        const int key = KV_TILE * kappa + r;
        sm.sk[r] = key < L ? p.sk[(int64_t)g * T + doc_start + key] : (uint8_t)127;
        sm.sv[r] = key < L ? p.sv[(int64_t)g * T + doc_start + key] : (uint8_t)127;
      }
    }
    if (!producer) {
      __builtin_amdgcn_s_waitcnt(0);  // the direct loads have landed
      scale_store(0, 0, qt_first, rsq, rsdo, rd, rq4);
      if (n_steps > 1) {
        int h1;
        scale_store(1, 1, step_qt(1, h1), rsq1, rsdo1, rd1, rq41);
      }
    }
    lds_barrier();
    const int k_scale = sm.sk[32 * kw + n];
    const int v_scale = sm.sv[32 * kw + n];

    // Each role runs its own phase loop (the same number of barriers in both), so the
    // consumers' accumulators are not live in the producers' code.
    if (producer) {
      // lane-dependent values re-derived from an opaque copy of the lane index: addresses
      // built from them are local to this role instead of shared with (and kept alive
      // through) the other role's code
      int lane_r = lane;
      asm volatile("" : "+v"(lane_r));
      const int lane = lane_r, n = lane_r & 31, hh = lane_r >> 5;
      const int key_rel = KV_TILE * kappa + 32 * kw + n;
      // this wave's K and (negated) V operand rows, the same in every step of the unit
      v8i kreg[NC], vreg[NC];
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        if constexpr (!QK4) kreg[cc] = lds_read_row32<D>(sm.k, 32 * kw + n, 64 * cc + 32 * hh);
        vreg[cc] = lds_read_row32<D>(sm.v, 32 * kw + n, 64 * cc + 32 * hh);
      }
      // QK4: the key's 4-bit row (16 bytes per chunk) and its exponent byte per 32 channels
      v4i kreg4[NC];
      int ks4[NC];
      if constexpr (QK4) {
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          kreg4[cc] = v4i{0, 0, 0, 0};
          ks4[cc] = 127;
          if (key_rel < L) {
            const int64_t kt = (int64_t)doc_start + key_rel;
            kreg4[cc] = *reinterpret_cast<const v4i*>(p.k4 + (kt * p.Hkv + g) * (D / 2) + 32 * cc + 16 * hh);
            ks4[cc] = p.sk4[((int64_t)g * T + kt) * (D / 32) + 2 * cc + hh];
          }
        }
      }
      // S and D - dP of query block qb of step st (tiles in buffer st % 4).  The dP accumulator
      // starts at D of its rows: accumulator register 4 j + e holds row 32 qb + 8 j + 4 hh + e,
      // the float4 at that row.
      auto products = [&](int st, int qb, v16f& sa, v16f& pa) {
        const int bb = st & (NBUF - 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 d4 = *reinterpret_cast<const float4*>(&sm.dd[bb][32 * qb + 8 * j + 4 * hh]);
          pa[4 * j] = d4.x; pa[4 * j + 1] = d4.y; pa[4 * j + 2] = d4.z; pa[4 * j + 3] = d4.w;
        }
        // A scales: the block bytes, or PRECISE the row's Q exponent for both products
        const int sq_a = PRECISE ? (int)sm.rt.pr.sqr[bb][32 * qb + n] : sm.sqdo[bb][qb].x;
        const int sdo_a = PRECISE ? sq_a : sm.sqdo[bb][qb].y;
        int sq4p[NC];
        if constexpr (QK4)
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) sq4p[cc] = sm.rt.sq4[st % 3][(32 * qb + n) * (D / 32) + 2 * cc + hh];
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          if constexpr (QK4) {
            const int b3 = st % 3, row = 32 * qb + n;
            const v4i aq = lds_read_row16<D / 2>(sm.q4[b3], row, 32 * cc + 16 * hh);
            sa = mfma_scaled_fp4(aq, kreg4[cc], cc ? sa : v16f{}, sq4p[cc], ks4[cc]);
          } else {
            const v8i aq = lds_read_row32<D>(sm.q[bb], 32 * qb + n, 64 * cc + 32 * hh);
            sa = mfma_scaled(aq, kreg[cc], cc ? sa : v16f{}, sq_a, k_scale);
          }
          const v8i ad = lds_read_row32<D>(sm.dO[bb], 32 * qb + n, 64 * cc + 32 * hh);
          pa = mfma_scaled(ad, vreg[cc], pa, sdo_a, v_scale);
        }
      };
      // One block's softmax terms fused with another block's products.  Softmax of query block
      // qs of step ss from (sa, pa): P = 2^(c S - LSE), dS = P (dP - D), the 32 x 32 block
      // exponents and the E4M3 codes (four words each).  Products of query block qp of step sp
      // into (ns, np).  The code runs in chunks fenced off from each other: each chunk issues
      // one matrix instruction, the operand read of the next one and a slice of the softmax
      // elements, so the matrix unit works while the vector unit does, and only one operand is
      // in flight at a time.
      // bp, bs: the step buffers of the products' and the softmax's steps (constants of the
      // unrolled phase loop, so the buffer offsets fold into the LDS instructions)
      auto fused = [&](int sp_st, int qp, v16f& ns, v16f& np, int ss, int qs, int q0, int sh, v16f& sa, v16f& pa,
                       int* pp4, int* pd4, uint32_t& sp, uint32_t& sds, auto masked, int bp, int bs) {
        constexpr bool MASK = decltype(masked)::value;
        constexpr int NM = 2 * NC;     // matrix instructions of the products
        constexpr int EPM = 16 / NM;   // softmax elements per chunk
        float4 lse4[4];  // rows acc_row(4 j + e, hh) = 32 qs + 8 j + 4 hh + e
#pragma unroll
        for (int j = 0; j < 4; ++j)
          lse4[j] = *reinterpret_cast<const float4*>(&sm.lse[bs][32 * qs + 8 * j + 4 * hh]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 d4 = *reinterpret_cast<const float4*>(&sm.dd[bp][32 * qp + 8 * j + 4 * hh]);
          np[4 * j] = d4.x; np[4 * j + 1] = d4.y; np[4 * j + 2] = d4.z; np[4 * j + 3] = d4.w;
        }
        int sq_s, sdo_s;
        if constexpr (PRECISE) {
          sq_s = sdo_s = sm.rt.pr.sqr[bp][32 * qp + n];
        } else {
          const int2 sqdo = sm.sqdo[bp][qp];  // one 8-byte read
          sq_s = sqdo.x;
          sdo_s = sqdo.y;
        }
        float4 pf4[4];  // PRECISE: 2^e(dO) of the same rows as lse4
        if constexpr (PRECISE)
#pragma unroll
          for (int j = 0; j < 4; ++j) pf4[j] = *reinterpret_cast<const float4*>(&sm.rt.pr.pf[bs][32 * qs + 8 * j + 4 * hh]);
        // operand m: Q rows (m even) or dO rows (m odd) of column chunk m / 2; two in flight.
        // QK4: the Q rows are the 4-bit copy (16 bytes, in the first half of the operand)
        const int bp3 = sp_st % 3;
        int sq4s[NC];
        if constexpr (QK4)
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) sq4s[cc] = sm.rt.sq4[bp3][(32 * qp + n) * (D / 32) + 2 * cc + hh];
        auto read_op = [&](int m) {
          if (QK4 && !(m & 1)) {
            const v4i t = lds_read_row16<D / 2>(sm.q4[bp3], 32 * qp + n, 32 * (m >> 1) + 16 * hh);
            return v8i{t[0], t[1], t[2], t[3], 0, 0, 0, 0};
          }
          return lds_read_row32<D>((m & 1) ? sm.dO[bp] : sm.q[bp], 32 * qp + n, 64 * (m >> 1) + 32 * hh);
        };
        v8i opnd[2];
        opnd[0] = read_op(0);
        opnd[1] = read_op(1);
        __builtin_amdgcn_sched_barrier(0);
        float pmax = 0.f, dmax = 0.f;
        // element i sits in row 32 qs + 4 hh + r_i (r_i = 8 (i / 4) + i % 4, a constant): it is
        // visible when lo <= r_i < hi (non-causally every row is when the key is in the document)
        const int lo = CAUSAL ? key_rel - (q0 + 32 * qs + 4 * hh) : (key_rel < L ? -QT : QT);
        const int hi = L - (q0 + 32 * qs + 4 * hh);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const int cc = m / 2;
          if (m % 2 == 0) {
            if constexpr (QK4)
              ns = mfma_scaled_fp4(v4i{opnd[0][0], opnd[0][1], opnd[0][2], opnd[0][3]}, kreg4[cc], cc ? ns : v16f{},
                                   sq4s[cc], ks4[cc]);
            else ns = mfma_scaled(opnd[0], kreg[cc], cc ? ns : v16f{}, sq_s, k_scale);
          }
          else np = mfma_scaled(opnd[1], vreg[cc], np, sdo_s, v_scale);  // D - dP
          if (m + 2 < NM) opnd[m & 1] = read_op(m + 2);
#pragma unroll
          for (int i = m * EPM; i < (m + 1) * EPM; ++i) {
            const float lse_i = i % 4 == 0 ? lse4[i / 4].x : i % 4 == 1 ? lse4[i / 4].y : i % 4 == 2 ? lse4[i / 4].z : lse4[i / 4].w;
            float arg = fmaf(sa[i], c, -lse_i);
            if constexpr (MASK) {
              const int r = 8 * (i / 4) + i % 4;  // unrolled: an immediate
              arg = (lo <= r && r < hi) ? arg : -__builtin_inff();  // 2^-inf = +0
            }
#ifdef FLAMIA_DEBUG_DUMP
            if (p.dbg.bwd_s || p.dbg.bwd_dp) {  // test builds: the two accumulators, masked as used
              const int r = 8 * (i / 4) + i % 4, row_rel = q0 + 32 * qs + 4 * hh + r;
              const int64_t x = (row_rel < L && key_rel < L)
                                    ? dbg_index(p.dbg, sh, doc_start + row_rel, doc_start + key_rel) : -1;
              if (x >= 0) {
                if (p.dbg.bwd_s) p.dbg.bwd_s[x] = (MASK && !(lo <= r && r < hi)) ? -__builtin_inff() : sa[i];
                if (p.dbg.bwd_dp) p.dbg.bwd_dp[x] = pa[i];
              }
            }
#endif
            float pv = __builtin_amdgcn_exp2f(arg);
            if constexpr (PRECISE) {  // P'' = P 2^e(dO_i), exact
              const float4 f = pf4[i / 4];
              pv *= i % 4 == 0 ? f.x : i % 4 == 1 ? f.y : i % 4 == 2 ? f.z : f.w;
            }
            const float dsv = -(pv * pa[i]);  // P (dP - D), PRECISE P'' (D - dP)'' = dS 2^e(Q_i)
            sa[i] = pv;
            pa[i] = dsv;
            pmax = fmaxf(pmax, pv);
            dmax = fmaxf(dmax, fabsf(dsv));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        float fp, fd;  // the scales 2^(byte - 127)
        float pm, dm;
        wave_max2_nonneg(pmax, dmax, pm, dm);
        sp = e8m0_byte_uniform(pm, fp);  // E8M0 bytes of the block exponents
        sds = e8m0_byte_uniform(dm, fd);
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          pp4[w4] = pack4_fp8_scalef(sa[4 * w4], sa[4 * w4 + 1], sa[4 * w4 + 2], sa[4 * w4 + 3], fp);
          pd4[w4] = pack4_fp8_scalef(pa[4 * w4], pa[4 * w4 + 1], pa[4 * w4 + 2], pa[4 * w4 + 3], fd);
        }
#ifdef FLAMIA_DEBUG_DUMP
        if (p.dbg.bwd_p || p.dbg.bwd_ds) {  // test builds: codes and block exponent bytes
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int row_rel = q0 + 32 * qs + acc_row(i, hh);
            const int64_t x = (row_rel < L && key_rel < L)
                                  ? dbg_index(p.dbg, sh, doc_start + row_rel, doc_start + key_rel) : -1;
            if (x < 0) continue;
            if (p.dbg.bwd_p) { p.dbg.bwd_p[x] = (uint8_t)(pp4[i / 4] >> (8 * (i % 4))); p.dbg.bwd_ps[x] = (uint8_t)sp; }
            if (p.dbg.bwd_ds) { p.dbg.bwd_ds[x] = (uint8_t)(pd4[i / 4] >> (8 * (i % 4))); p.dbg.bwd_dss[x] = (uint8_t)sds; }
          }
        }
#endif
      };
      // Phase ph works on step ph (step buffer BB = ph mod 4, a constant of the unrolled loop).
      // Block 0's products were made in the phase before (cs, cp); block 1's are issued while
      // block 0's softmax terms are formed, and block 0 of the next step while block 1's are.
      // The last step has no successor: its block-0 products read the next buffer's stale tiles
      // (finite, or whatever LDS held) into registers that are never used.
      v16f cs, cp, xs, xq;
      auto phase_body = [&](int ph, int h, int qt, auto masked, auto BB) {
        constexpr int bb = decltype(BB)::value, bn = (bb + 1) & (NBUF - 1);
        const int q0 = QT * qt;
        constexpr int x2 = bb & 1;
        int pp[8], pd[8];
        uint32_t sp[2], sds[2];  // E8M0 bytes
        // hand over query block qb's operands as soon as they exist, so the writes retire under
        // the next block's work instead of before the barrier (the consumer stores dShat to the
        // workspace)
        auto hand_over = [&](int qb) {
          sm.xp[x2][kw][qb][lane] = make_int4(pp[4 * qb], pp[4 * qb + 1], pp[4 * qb + 2], pp[4 * qb + 3]);
          sm.xd[x2][kw][qb][lane] = make_int4(pd[4 * qb], pd[4 * qb + 1], pd[4 * qb + 2], pd[4 * qb + 3]);
          if (!PRECISE && !store_ds) {
            int l = lane;
            asm volatile("" : "+v"(l));  // addresses formed here, not kept in registers all along
            const int nl = l & 31, hl = l >> 5;
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
              const int qcol = 32 * qb + 8 * w4 + 4 * hl;
              *reinterpret_cast<int*>(&sm.ds[x2][lds_off<QT>(32 * kw + nl, qcol)]) = pd[4 * qb + w4];
            }
          }
        };
        fused(ph, 1, xs, xq, ph, 0, q0, h, cs, cp, pp, pd, sp[0], sds[0], masked, bb, bb);
        // empty uses of freshly issued products keep their matrix instructions among the vector
        // work they overlap, instead of sunk past the hand-over towards their next use
        asm volatile("" ::"v"(xs), "v"(xq));
        hand_over(0);
        fused(min(ph + 1, n_steps - 1), 0, cs, cp, ph, 1, q0, h, xs, xq, pp + 4, pd + 4, sp[1], sds[1], masked, bn, bb);
        asm volatile("" ::"v"(cs), "v"(cp));
        hand_over(1);
        if (lane == 0) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            sm.xs_p[x2][qb][kw] = sp[qb];
            sm.xs_d[x2][qb][kw] = sds[qb];
          }
        }
      };
      products(0, 0, cs, cp);
      // once per unit: the loop's paths (a step-less one among them, never taken) may touch these
      // registers soon after the products are issued
      mfma_drain(cs);
      mfma_drain(cp);
      int cur_h = g * grp, cur_qt = qt_first;  // head and query tile of step ph
      // all 64 x 128 pairs of a step are visible when the query tile lies wholly inside the
      // document and, causally, below the key tile (then every key of the tile is inside the
      // document too) or, non-causally, when the key tile is wholly inside it as well
      const bool keys_full = !CAUSAL && KV_TILE * kappa + KV_TILE <= L;
      // phase ph, or false past the last one (n_steps + 1 phases, one barrier each)
      auto phase = [&](int ph, auto BB) {
        if (ph > n_steps) return false;
        if (ph < n_steps) {
          // all 64 x 128 pairs visible: the query tile lies wholly below the key tile and
          // inside the document (then every key of the tile is inside it too)
          if ((CAUSAL ? cur_qt >= 2 * kappa + 2 : keys_full) && QT * cur_qt + QT <= L)
            phase_body(ph, cur_h, cur_qt, std::false_type{}, BB);
          else phase_body(ph, cur_h, cur_qt, std::true_type{}, BB);
          if (++cur_qt == n_qt) {
            cur_qt = qt_first;
            ++cur_h;
          }
        }
        lds_barrier();  // phase done: operands handed over, the next tiles in place
        return true;
      };
      static_assert(NBUF == 4, "the phase loop is unrolled over the four step buffers");
      for (int ph = 0;; ph += NBUF) {
        if (!phase(ph, std::integral_constant<int, 0>{})) break;
        if (!phase(ph + 1, std::integral_constant<int, 1>{})) break;
        if (!phase(ph + 2, std::integral_constant<int, 2>{})) break;
        if (!phase(ph + 3, std::integral_constant<int, 3>{})) break;
      }
    } else {
      // lane-dependent values re-derived from an opaque copy of the lane index: addresses
      // built from them are local to this role instead of shared with (and kept alive
      // through) the other role's code
      int lane_r = lane;
      asm volatile("" : "+v"(lane_r));
      const int lane = lane_r, n = lane_r & 31, hh = lane_r >> 5;
      const int key_rel = KV_TILE * kappa + 32 * kw + n;
      v16f dkacc[NDB], dvacc[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) { dkacc[db] = v16f{}; dvacc[db] = v16f{}; }
      int ld_h = 0, ld_qt = 0;  // head and query tile of step ph + 2 (the next to load)
      if (n_steps > 2) ld_qt = step_qt(2, ld_h);
      int st_h = g * grp, st_qt = qt_first;  // head and query tile of step ph - 1
      for (int ph = 0; ph <= n_steps; ++ph) {
        const int qtn = ld_qt;
        const int bn = (ph + 2) & (NBUF - 1);
        const int bn3 = (ph + 2) % 3;
        if (ph + 2 < n_steps) {  // step ph + 2's tiles, straight into LDS
          issue_step_loads<D, PRECISE, QK4>(p, sm, bn, doc_start, L, ld_h, qtn, cw, lane, bn3);
          scale_loads(ld_h, qtn, rsq, rsdo, rd, rq4);
          if (++ld_qt == n_qt) {
            ld_qt = qt_first;
            ++ld_h;
          }
        }
        if (ph >= 1) {
          // ---- gradient products of step ph - 1
          const int st = ph - 1;
          const int b = st & (NBUF - 1), xb = st & 1;
          {
            const int4 p0 = sm.xp[xb][kw][0][lane], p1 = sm.xp[xb][kw][1][lane];
            const int4 d0 = sm.xd[xb][kw][0][lane], d1 = sm.xd[xb][kw][1][lane];
            if (store_ds) {
              // dShat codes and block exponents of step ph - 1 to the workspace, from the operand
              // registers (the producer's wave stream is the longer one).  Stored layout: the
              // 2 KiB of key group kw hold query block qb's operand bytes at 1 KiB qb, lane by
              // lane, so each store instruction writes 1 KiB contiguously.  Non-temporal: the
              // store is read back once, by another kernel, and would otherwise push the step
              // tiles (re-read once per key tile) out of L2
              uint8_t* bbase = p.ds_store + ((ds_base + (st_qt - qt_first)) * p.Hq + st_h) * DS_STRIDE;
              v4i* dst = reinterpret_cast<v4i*>(bbase + 2048 * kw + 16 * lane);
              __builtin_nontemporal_store(v4i{d0.x, d0.y, d0.z, d0.w}, dst);
              __builtin_nontemporal_store(v4i{d1.x, d1.y, d1.z, d1.w}, dst + 64);
              if (lane == 0) {
                __builtin_nontemporal_store((uint8_t)sm.xs_d[xb][0][kw], bbase + DS_BLOCK + kw);
                __builtin_nontemporal_store((uint8_t)sm.xs_d[xb][1][kw], bbase + DS_BLOCK + 4 + kw);
              }
            }
            if (++st_qt == n_qt) {
              st_qt = qt_first;
              ++st_h;
            }
            const v8i bp = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
            const v8i bd = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
            // A scales: the query block's bytes, or PRECISE the bare codes (the exponents are in
            // P'' and dS'')
            const int2 sqdo_h = PRECISE ? make_int2(127, 127) : sm.sqdo[b][hh];
            const int sdo_h = sqdo_h.y, sq_h = sqdo_h.x;
            const int sp_h = sm.xs_p[xb][hh][kw], sds_h = sm.xs_d[xb][hh][kw];
            // Operand k (dO^T for even k, Q^T for odd k, d-block k / 2) is read AHEAD matrix
            // instructions early, so each one finds its operand in registers instead of waiting
            // out an LDS round trip; at most 4 AHEAD reads are outstanding, within the range of
            // the LDS wait counter.
            constexpr int NOP = 2 * NDB, AHEAD = 3;
            auto read_op = [&](int k) { return lds_read_tr32<D>((k & 1) ? sm.q[b] : sm.dO[b], 0, 32 * (k >> 1), lane); };
            v8i ring[AHEAD];
#pragma unroll
            for (int k = 0; k < AHEAD; ++k) ring[k] = read_op(k);
#pragma unroll
            for (int k = 0; k < NOP; ++k) {
              const v8i a = ring[k % AHEAD];
              if (k & 1) dkacc[k >> 1] = mfma_scaled(a, bd, dkacc[k >> 1], sq_h, sds_h);
              else dvacc[k >> 1] = mfma_scaled(a, bp, dvacc[k >> 1], sdo_h, sp_h);
              if (k + AHEAD < NOP) ring[k % AHEAD] = read_op(k + AHEAD);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          if (!PRECISE && !store_ds) {
            // single key tile: dQ^T = K^T dShat^T here, the only contribution of its rows;
            // consumer w computes d-block w (d = 128) or w % 2 (d = 64) of its query blocks
            const int hi = st / nq;
            const int h = g * grp + hi;
            const int q0 = QT * (qt_first + (st - hi * nq));
            constexpr int NQB = (D == 128) ? 2 : 1;
            const int dblk = (D == 128) ? kw : (kw & 1);
            const int qb0 = (D == 128) ? 0 : (kw >> 1);
#pragma unroll
            for (int x = 0; x < NQB; ++x) {
              const int qb = qb0 + x;
              v16f dq = v16f{};
#pragma unroll
              for (int ci = 0; ci < 2; ++ci) {
                const v8i ak = lds_read_tr32<D>(sm.k, 64 * ci, 32 * dblk, lane);
                const v8i bs = lds_read_tr32<QT>(sm.ds[xb], 64 * ci, 32 * qb, lane);
                dq = mfma_scaled(ak, bs, dq, sm.sk[64 * ci + 32 * hh], sm.xs_d[xb][qb][2 * ci + hh]);
              }
              mfma_drain(dq);
              const int qi = 32 * qb + n;
              const int qr = q0 + qi;
              if (qr < L) {
                const int pi = p.pi[(int64_t)h * T + doc_start + qr];
                const float up = exp2i(pi), down = exp2i(-pi) * p.softmax_scale;
#ifdef FLAMIA_DEBUG_DUMP
                if (p.dbg.dq_part) {  // test builds: the partial as converted to FP16 (key tile 0)
                  const int64_t x = dbg_row(p.dbg, h, doc_start + qr);
                  if (x >= 0)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                      p.dbg.dq_part[(x * p.dbg.n_tiles) * D + 32 * dblk + acc_row(i, hh)] = dq[i] * up;
                }
#endif
                uint16_t* row = p.dq + (int64_t)(doc_start + qr) * p.dqst + (int64_t)h * p.dqsh;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  // the FP16 sum of one partial: acc16 = +0 + FP16(partial), so a partial that
                  // rounds to -0 gives +0, as the sums of longer documents do
                  const _Float16 z = 0;
                  const _Float16 a0 = z + (_Float16)(dq[4 * j + 0] * up), a1 = z + (_Float16)(dq[4 * j + 1] * up);
                  const _Float16 a2 = z + (_Float16)(dq[4 * j + 2] * up), a3 = z + (_Float16)(dq[4 * j + 3] * up);
                  uint2 w;
                  w.x = pack_bf16_int((float)a0 * down, (float)a1 * down);
                  w.y = pack_bf16_int((float)a2 * down, (float)a3 * down);
                  *reinterpret_cast<uint2*>(row + 32 * dblk + 8 * j + 4 * hh) = w;
                }
              }
            }
          }
        }
        if (ph + 2 < n_steps) {
          __builtin_amdgcn_s_waitcnt(0);  // the direct loads have landed
          scale_store(bn, bn3, qtn, rsq, rsdo, rd, rq4);
        }
        lds_barrier();  // phase done: operands consumed, the next step's tiles stored
      }

      // ---- dK, dV of this consumer's keys
#pragma unroll
      for (int db = 0; db < NDB; ++db) { mfma_drain(dkacc[db]); mfma_drain(dvacc[db]); }
      if (key_valid) {
        uint16_t* krow = p.dk + (int64_t)(doc_start + key_rel) * p.dkst + (int64_t)g * p.dksh;
        uint16_t* vrow = p.dv + (int64_t)(doc_start + key_rel) * p.dvst + (int64_t)g * p.dvsh;
        const float ss = p.softmax_scale;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d0 = 32 * db + 8 * j + 4 * hh;
            uint2 wk, wv;
            wk.x = pack_bf16(dkacc[db][4 * j] * ss, dkacc[db][4 * j + 1] * ss);
            wk.y = pack_bf16(dkacc[db][4 * j + 2] * ss, dkacc[db][4 * j + 3] * ss);
            wv.x = pack_bf16(dvacc[db][4 * j], dvacc[db][4 * j + 1]);
            wv.y = pack_bf16(dvacc[db][4 * j + 2], dvacc[db][4 * j + 3]);
            *reinterpret_cast<uint2*>(krow + d0) = wk;
            *reinterpret_cast<uint2*>(vrow + d0) = wv;
          }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Query-stationary dQ.
template <int D>
struct DqSmem {
  uint8_t k[2][KV_TILE * D];
  uint8_t ds[2][DQ_QT][DS_BLOCK];
  uint8_t sk[2][KV_TILE];
  uint8_t dsc[2][DQ_QT][8];
};

// The next key tile's K rows, dShat blocks and exponents, in registers between the global loads
// and the LDS stores.
typedef unsigned int v4u __attribute__((ext_vector_type(4)));  // plain vector: stays in registers
template <int D>
struct DqRegs {
  static constexpr int KCH = KV_TILE * D / 16 / DQ_THREADS;  // K chunks per thread
  static constexpr int CPB = DS_BLOCK / 16 / DQ_THREADS;    // chunks of one dShat block per thread
  static_assert(CPB * DQ_THREADS * 16 == DS_BLOCK && (DQ_QT & (DQ_QT - 1)) == 0, "dQ tiling");
  v4u k[KCH], s[DQ_QT * CPB];
  uint2 sc;       // threads 0..DQ_QT-1: exponents of query tile `tid`
  uint32_t skb;   // threads 0..127: K scale byte of key `tid`
  int nkeys;      // keys of the tile inside the document (scale 127 beyond)
};

// Every thread issues the same loads whatever the tile (rows past the document end repeat its
// last row, tiles outside the item's range re-read a block that exists and are not used), so
// the number of loads in flight is the same on every path and the wait before the LDS store
// can leave the following tile's loads outstanding.
template <int D>
__device__ __forceinline__ void dq_load(DqRegs<D>& r, const BwdParams& p, int doc_start, int L, int n_qt,
                                        int64_t base, int qt0, int g, int h, int kappa) {
  const int tid = threadIdx.x;
  constexpr int CPR = D / 16;
#pragma unroll
  for (int i = 0; i < DqRegs<D>::KCH; ++i) {
    const int chunk = tid + i * DQ_THREADS;
    const int row = chunk / CPR, col = (chunk % CPR) * 16;
    const int key = min(KV_TILE * kappa + row, L - 1);
    r.k[i] = *reinterpret_cast<const v4u*>(p.k + ((int64_t)(doc_start + key) * p.Hkv + g) * D + col);
  }
  // block of query tile qt0 + t (clamped into the key tile's range [qt_lo, n_qt - 1], qt_lo its
  // diagonal query tile, or 0 non-causally); `base` is the key tile's first block in the chunk's
  // store
  const int qt_lo = p.causal_mask ? 2 * kappa : 0;
  auto block = [&](int t) {
    const int qt = min(max(qt0 + t, qt_lo), n_qt - 1);
    return p.ds_store + ((base + (qt - qt_lo)) * p.Hq + h) * DS_STRIDE;
  };
#pragma unroll
  for (int t = 0; t < DQ_QT; ++t)  // read once: non-temporal, so L2 keeps the K tiles
#pragma unroll
    for (int j = 0; j < DqRegs<D>::CPB; ++j)
      r.s[t * DqRegs<D>::CPB + j] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(block(t)) + tid + j * DQ_THREADS);
  r.sc = *reinterpret_cast<const uint2*>(block(tid & (DQ_QT - 1)) + DS_BLOCK);  // used by threads 0..DQ_QT-1
  r.skb = p.sk[(int64_t)g * p.T + doc_start + min(KV_TILE * kappa + (tid & (KV_TILE - 1)), L - 1)];
  r.nkeys = L - KV_TILE * kappa;  // the value is tested at the store, not here: no wait for it
}

template <int D>
__device__ __forceinline__ void dq_store(const DqRegs<D>& r, DqSmem<D>& sm, int b) {
  const int tid = threadIdx.x;
  constexpr int CPR = D / 16;
#pragma unroll
  for (int i = 0; i < DqRegs<D>::KCH; ++i) {
    const int chunk = tid + i * DQ_THREADS;
    const int row = chunk / CPR, col = (chunk % CPR) * 16;
    *reinterpret_cast<v4u*>(&sm.k[b][lds_off<D>(row, col)]) = r.k[i];
  }
  // stored chunk tid (key group kw = tid / 128, query block qb, producer lane (n, hh)) is the
  // 16-byte piece of key row 32 kw + n at byte 32 hh + 16 qb
#pragma unroll
  for (int j = 0; j < DqRegs<D>::CPB; ++j) {
    const int c = tid + j * DQ_THREADS;
    const int off = lds_off<QT>(32 * (c >> 7) + (c & 31), 32 * ((c >> 5) & 1) + 16 * ((c >> 6) & 1));
#pragma unroll
    for (int t = 0; t < DQ_QT; ++t) *reinterpret_cast<v4u*>(&sm.ds[b][t][off]) = r.s[t * DqRegs<D>::CPB + j];
  }
  if (tid < DQ_QT) *reinterpret_cast<uint2*>(&sm.dsc[b][tid][0]) = r.sc;
  if (tid < KV_TILE) sm.sk[b][tid] = tid < r.nkeys ? (uint8_t)r.skb : (uint8_t)127;
}

// Causality is a run-time flag here (p.causal_mask): two instantiations allocate registers
// differently enough that one keeps a spill reload inside the key-tile loop.
template <int D>
__global__ __launch_bounds__(DQ_THREADS, 2) void dq_kernel(BwdParams p) {  // two workgroups per CU
  constexpr int NDB = D / 32;
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  __shared__ DqSmem<D> sm;

  if (p.status[0] || p.chunk >= p.status[1]) return;  // not laid out, or a chunk past the last
  const int chunk = p.chunk;
  const int n_chunks = p.status[1];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int n_items = list_walk_items(p.fwd_list, p.T, p.small);
  const int4* items = reinterpret_cast<const int4*>(p.fwd_list + 4);
  constexpr int PARTS = ITEM_Q / (QT * DQ_QT);  // workgroup units per work item and head
  const int grp = p.Hq / p.Hkv;
  // units (part of an item, query head) of the partition's KV heads, in list order
  const UnitPartition up = unit_partition(p.Hkv);
  const int hq_per = up.kv_per * grp;           // query heads per partition
  const int n_units = n_items * PARTS * hq_per;
  const int t4 = wave >> 1, s = wave & 1;     // query tile of the unit, byte-position half
  const int qrow = ds_pos_query(32 * s + n);  // query offset in the tile held by this lane
  int lane_zero;                              // 0, opaque: keeps a load's result in vector registers
  asm volatile("v_mov_b32 %0, 0" : "=v"(lane_zero));
  const int qb_l = n >> 4;                    // its 32-query block

  __shared__ int unit_slot;
  int32_t* const counter = p.counters + 16 * p.chunk + 8 + up.part;
  for (int u = up.rank; u < n_units; u = next_unit(counter, &unit_slot, up.first)) {  // dynamic, as in the key-tile pass
    const int4 it = items[u / (PARTS * hq_per)];
    if (it.z < 2) break;  // single key tile from here on (the list is sorted by cost)
    const int j = u % hq_per;
    const int g = partition_kv(up, j / grp), h = g * grp + j % grp, part = (u / hq_per) % PARTS;
    const int doc = it.x, item = it.y;
    const int doc_start = p.cu[doc];
    const int L = p.cu[doc + 1] - doc_start;
    const int n_qt = (L + QT - 1) / QT;
    const int qt0 = (ITEM_Q / QT) * item + DQ_QT * part;
    if (qt0 >= n_qt) continue;  // the item ends before this part (uniform over the workgroup)
    // This unit's key tiles in this chunk: the key tiles 0 .. K of the unit's last row have
    // chunk numbers that do not decrease along the document, so the ones in this chunk are
    // [k_lo, kappa_hi] with k_lo = #(chunk < this one) and kappa_hi + 1 = #(chunk <= this one).
    // Rows whose last key tile lies in an earlier chunk are complete already.
    const int tb = p.tile_base[doc];
    const int last_qt = min(qt0 + DQ_QT, n_qt) - 1;
    // the last key tile the unit's rows see: that of its last query tile, or non-causally the
    // document's last one
    const int K = p.causal_mask ? last_qt / 2 : (L - 1) / KV_TILE;
    int k_lo = 0, kappa_hi = K;  // one chunk: every key tile is in it
    if (n_chunks > 1) {
    if (p.kv_chunk[tb + K] < chunk) continue;  // (uniform over the workgroup)
    kappa_hi = -1;
    for (int k0 = 0; k0 <= K; k0 += 64 * 8) {  // each lane reads up to 8 entries, all in flight
      int ch[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        const int kk = k0 + 64 * x + lane;
        ch[x] = kk <= K ? p.kv_chunk[tb + kk] : 0x7FFFFFFF;
      }
#pragma unroll
      for (int x = 0; x < 8; ++x) {
        k_lo += __popcll(__ballot(ch[x] < chunk));
        kappa_hi += __popcll(__ballot(ch[x] <= chunk));
      }
    }
    if (k_lo > kappa_hi) continue;  // no key tile of this unit's rows in this chunk (uniform)
    }
    const int qt = qt0 + t4;
    const bool active = qt < n_qt;
    const int q_rel = QT * qt + qrow;
    const bool row_valid = q_rel < L;
    // the wave's rows (one 64-query tile, whose last key tile is qt / 2, or K non-causally) take
    // part in this chunk when that tile is at or after k_lo, and are complete after it when it
    // is at or before kappa_hi (the unit's last key tile in this chunk)
    const int w_last = p.causal_mask ? qt / 2 : K;
    const bool w_on = active && row_valid && w_last >= k_lo;
    const bool w_final = w_last <= kappa_hi;
    int pi = 0;
    if (row_valid) pi = p.pi[(int64_t)h * p.T + doc_start + q_rel];
    const float up = exp2i(pi);
    uint16_t* const row = p.dq + (int64_t)(doc_start + q_rel) * p.dqst + (int64_t)h * p.dqsh;

    // the FP16 sums: from +0, or as an earlier chunk left them (kept in the dQ output rows)
    h2 acc16[NDB][8];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc16[db][j] = h2{0, 0};
    if (w_on && k_lo > 0) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint2 w = *reinterpret_cast<const uint2*>(row + 32 * db + 8 * j + 4 * hh);
          acc16[db][2 * j] = __builtin_bit_cast(h2, w.x);
          acc16[db][2 * j + 1] = __builtin_bit_cast(h2, w.y);
        }
    }

    // Key tile kappa's operands go global -> registers two tiles ahead and registers -> LDS one
    // tile ahead (two register sets, two LDS buffers), so each load has a whole tile's compute
    // to arrive.
    auto compute = [&](int kappa) __attribute__((always_inline)) {
      const int b = kappa & 1;
      if (active && (!p.causal_mask || qt >= 2 * kappa)) {
        v8i bs[2];
        int sb[2];
#pragma unroll
        for (int ci = 0; ci < 2; ++ci) {
          bs[ci] = lds_read_tr32<QT>(sm.ds[b][t4], 64 * ci, 32 * s, lane);
          sb[ci] = sm.dsc[b][t4][4 * qb_l + 2 * ci + hh];
        }
        // K^T operand k (d-block k / 2, key half k % 2) read three products ahead; the partial
        // of d-block db is added to the FP16 sums while the products of d-block db + 1 run.
        // The prescale 2^pi of the lane's query is folded into the dShat operand's scale byte
        // when every such byte stays a finite E8M0 exponent: the instruction then returns
        // partial * 2^pi itself (a power-of-two scale commutes with the rounding; the results
        // are far inside the normal range, |partial * 2^pi| <= 2^15), and no multiply is needed.
        // Otherwise (a rare block exponent near either end of the range) the partial is
        // multiplied by 2^pi as it stands.
        constexpr int NOP = 2 * NDB, AHEAD = 3;
        auto read_k = [&](int k) { return lds_read_tr32<D>(sm.k[b], 64 * (k & 1), 32 * (k >> 1), lane); };
        const int f0 = sb[0] + pi, f1 = sb[1] + pi;
        const bool fold_ok = (unsigned)f0 <= 254u && (unsigned)f1 <= 254u;
        auto run = [&](auto fold) {
          constexpr bool FOLD = decltype(fold)::value;
          const int sc[2] = {FOLD ? f0 : sb[0], FOLD ? f1 : sb[1]};
          auto add_partial = [&](v16f& part, int db) {
            mfma_drain(part);
#ifdef FLAMIA_DEBUG_DUMP
            if (p.dbg.dq_part && row_valid) {  // test builds: the partial as converted to FP16
              const int64_t x = dbg_row(p.dbg, h, doc_start + q_rel);
              if (x >= 0 && kappa < p.dbg.n_tiles)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                  p.dbg.dq_part[(x * p.dbg.n_tiles + kappa) * D + 32 * db + acc_row(i, hh)] = FOLD ? part[i] : part[i] * up;
            }
#endif
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const h2 x = FOLD ? h2{(_Float16)part[2 * j], (_Float16)part[2 * j + 1]}
                                : h2{(_Float16)(part[2 * j] * up), (_Float16)(part[2 * j + 1] * up)};
              acc16[db][j] = acc16[db][j] + x;
            }
          };
          v8i ring[AHEAD];
#pragma unroll
          for (int k = 0; k < AHEAD; ++k) ring[k] = read_k(k);
          v16f part[2];
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int ci = 0; ci < 2; ++ci) {
              const int k = 2 * db + ci;
              part[db & 1] = mfma_scaled(ring[k % AHEAD], bs[ci], ci ? part[db & 1] : v16f{},
                                         sm.sk[b][64 * ci + 32 * hh], sc[ci]);
              if (k + AHEAD < NOP) ring[k % AHEAD] = read_k(k + AHEAD);
            }
            if (db >= 1) add_partial(part[(db - 1) & 1], db - 1);
            __builtin_amdgcn_sched_barrier(0);
          }
          add_partial(part[(NDB - 1) & 1], NDB - 1);
        };
        if (__all(fold_ok)) run(std::true_type{});
        else run(std::false_type{});
      }
    };
    // one tile: loads of kappa + 2 into `spare`, compute kappa, `next` (kappa + 1) into LDS.  The
    // loads are issued on every tile (the last two re-read tile kappa_hi, unused) so that the
    // count of loads in flight does not depend on the path.
    // The store offset of tile kappa + 3 is read one tile ahead of its loads and before this
    // tile's loads, so waiting for it at the next tile leaves those in flight.  Its index goes
    // through a register that differs per lane in the compiler's view (zero in every lane): a
    // uniform value would be moved to scalar registers at once, which waits for every load
    // issued before that point, this tile's included.
    int64_t off_n = 0;
    auto tile = [&](int kappa, DqRegs<D>& next, DqRegs<D>& spare) __attribute__((always_inline)) {
      const int64_t off = off_n;
      off_n = p.kv_off[tb + min(kappa + 3, kappa_hi) + lane_zero];
      dq_load<D>(spare, p, doc_start, L, n_qt, off, qt0, g, h, min(kappa + 2, kappa_hi));
      compute(kappa);
      if (kappa + 1 <= kappa_hi) dq_store<D>(next, sm, (kappa + 1) & 1);
      lds_barrier();
    };
    DqRegs<D> ra, rb;
    lds_barrier();  // the previous unit no longer reads LDS
    dq_load<D>(ra, p, doc_start, L, n_qt, p.kv_off[tb + k_lo], qt0, g, h, k_lo);
    dq_load<D>(rb, p, doc_start, L, n_qt, p.kv_off[tb + min(k_lo + 1, kappa_hi)], qt0, g, h, min(k_lo + 1, kappa_hi));
    off_n = p.kv_off[tb + min(k_lo + 2, kappa_hi) + lane_zero];
    dq_store<D>(ra, sm, k_lo & 1);
    lds_barrier();
    for (int kappa = k_lo;; kappa += 2) {  // two tiles per trip: the register sets trade roles
      tile(kappa, rb, ra);
      if (kappa + 1 > kappa_hi) break;
      tile(kappa + 1, ra, rb);
      if (kappa + 2 > kappa_hi) break;
    }

    if (w_on && w_final) {
      const float down = exp2i(-pi) * p.softmax_scale;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const h2 lo = acc16[db][2 * j], hi2 = acc16[db][2 * j + 1];
          uint2 w;
          w.x = pack_bf16((float)lo[0] * down, (float)lo[1] * down);
          w.y = pack_bf16((float)hi2[0] * down, (float)hi2[1] * down);
          *reinterpret_cast<uint2*>(row + 32 * db + 8 * j + 4 * hh) = w;
        }
    } else if (w_on) {  // rows continued in a later chunk: the FP16 sums wait in the dQ rows
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint2 w;
          w.x = __builtin_bit_cast(uint32_t, acc16[db][2 * j]);
          w.y = __builtin_bit_cast(uint32_t, acc16[db][2 * j + 1]);
          *reinterpret_cast<uint2*>(row + 32 * db + 8 * j + 4 * hh) = w;
        }
    }
  }
}

// ------------------------------------------------------------------------------------------
// Prologue: pi per (head, row) and zero rows outside every document (workgroups 0..Hq-1);
// dShat store layout and capacity check (workgroup Hq).
constexpr int PRO_THREADS = 1024;
constexpr int PRO_CHUNK = 4 * PRO_THREADS;

struct Seg {  // segmented running maximum: f = a segment starts inside, v/k = running maxima
  int f, v, k;
};
__device__ __forceinline__ Seg seg_op(Seg a, Seg b) {
  return Seg{a.f | b.f, b.f ? b.v : max(a.v, b.v), b.f ? b.k : max(a.k, b.k)};
}

// Stored dShat blocks (per query head) of the backward item (document of length L, key tile
// kappa): one per 64-query tile from the key tile's diagonal to the document end; none for a
// document of a single key tile (its dQ is formed in the key-tile pass).
__device__ __forceinline__ int64_t item_blocks(int L, int kappa, int causal_mask) {
  return L > KV_TILE ? (int64_t)((L + QT - 1) / QT - (causal_mask ? 2 * kappa : 0)) : 0;
}

// Inclusive scan of part[0 .. PRO_THREADS) in place (all threads take part).
__device__ __forceinline__ void block_scan(int64_t* part) {
  const int tid = threadIdx.x;
  for (int off = 1; off < PRO_THREADS; off <<= 1) {
    const int64_t add = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
}

// Layout of the key-tile chunks (one workgroup).
//  1. tile_base: exclusive prefix sum over the documents of their key tiles (the row of each
//     document in the (document, key tile) tables);
//  2. over the backward list (sorted by descending cost, so the key tiles of one document appear
//     in ascending order): each item's stored blocks and their exclusive prefix P(u); item u
//     belongs to the chunk of its last block, floor(max(P(u) + blocks(u) - 1, 0) / chunk_cap),
//     so a chunk holds fewer than chunk_cap + (largest item) blocks and consecutive items differ
//     by at most one chunk; chunk_start / chunk_first record each chunk's first item and prefix;
//  3. each item's chunk and its first block within the chunk's store, P(u) - chunk_first, go into
//     the (document, key tile) tables.
// Chunks run in list order, so every query row still meets its key tiles in ascending order and
// the dQ sums are the same as with one chunk.
__device__ void layout_chunks(const BwdParams& p) {
  __shared__ int64_t part[PRO_THREADS];
  const int tid = threadIdx.x;
  {
    // each wave takes a contiguous span of documents in groups of 64 (lane l: document
    // base + l), so the bounds' loads and the table's stores are coalesced; the waves' totals
    // give each span its start
    constexpr int NWV = PRO_THREADS / 64;
    const int lane = tid & 63, wave = tid >> 6;
    const int nd = p.n_docs;
    const int per_w = ((nd + NWV - 1) / NWV + 63) / 64 * 64;
    const int w_lo = min(nd, wave * per_w), w_hi = min(nd, w_lo + per_w);
    auto tiles = [&](int k) { return (int64_t)((p.cu[k + 1] - p.cu[k] + KV_TILE - 1) / KV_TILE); };
    int64_t tot = 0;
    for (int k = w_lo + lane; k < w_hi; k += 64) tot += tiles(k);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off, 64);
    if (lane == 0) part[wave] = tot;
    __syncthreads();
    if (tid == 0) {
      int64_t run = 0;
      for (int w = 0; w < NWV; ++w) {
        const int64_t t = part[w];
        part[w] = run;
        run += t;
      }
      part[NWV] = run;
    }
    __syncthreads();
    int64_t run = part[wave];
    for (int k0 = w_lo; k0 < w_hi; k0 += 64) {
      const int k = k0 + lane;
      const int64_t v = k < w_hi ? tiles(k) : 0;
      int64_t incl = v;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int64_t y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      if (k < w_hi) p.tile_base[k] = (int32_t)(run + incl - v);
      run += __shfl(incl, 63, 64);
    }
    if (tid == 0) p.tile_base[nd] = (int32_t)part[NWV];
    __syncthreads();
  }
  const int n_items = list_walk_items(p.list, p.T, p.small);  // short documents: the small-document pass
  const int4* items = reinterpret_cast<const int4*>(p.list + 4);
  // the precision options store nothing (their dQ pass recomputes): one chunk
  auto blocks_of = [&](int u) {
    const int4 it = items[u];
    return p.precise ? (int64_t)0 : item_blocks(p.cu[it.x + 1] - p.cu[it.x], it.y, p.causal_mask);
  };
  auto chunk_of = [&](int64_t P, int64_t b) {
    const int64_t last = P + b - 1;
    return (int)(last > 0 ? last / p.chunk_cap : 0);
  };
  const int per = (n_items + PRO_THREADS - 1) / PRO_THREADS;
  const int lo = min(n_items, tid * per), hi = min(n_items, lo + per);
  int64_t sum = 0;
  for (int u = lo; u < hi; ++u) sum += blocks_of(u);
  part[tid] = sum;
  __syncthreads();
  block_scan(part);
  const int64_t base = part[tid] - sum;  // prefix of item lo
  __shared__ int any_bad;
  if (tid == 0) any_bad = 0;
  __syncthreads();
  int bad = 0;
  {
    int64_t P = base;
    int prev = -1;
    if (lo > 0 && lo < hi) {
      const int64_t bp = blocks_of(lo - 1);
      prev = chunk_of(P - bp, bp);
    }
    for (int u = lo; u < hi; ++u) {
      const int64_t b = blocks_of(u);
      const int c = chunk_of(P, b);
      if (c >= p.max_chunks) {  // more blocks than any documents of T tokens have: bad cu_seqlens
        bad = 1;
        break;
      }
      if (c != prev) {
        p.chunk_start[c] = u;
        p.chunk_first[c] = P;
      }
      if (u == n_items - 1) {  // the last item: the chunk count, and empty chunks start at the end
        p.status[1] = c + 1;
        for (int x = c + 1; x <= p.max_chunks; ++x) p.chunk_start[x] = n_items;
      }
      prev = c;
      P += b;
    }
  }
  if (n_items == 0 && tid == 0) {
    p.status[1] = 0;
    for (int x = 0; x <= p.max_chunks; ++x) p.chunk_start[x] = 0;
  }
  {
    // table rows of this thread's items (documents longer than the tables allow: bad cu_seqlens)
    for (int u = lo; u < hi && !bad; ++u) {
      const int4 it = items[u];
      const int x = p.tile_base[it.x] + it.y;
      if (x < 0 || x >= p.n_tab) bad = 1;
    }
    if (bad) any_bad = 1;
  }
  __syncthreads();  // chunk_first written, any_bad settled
  if (any_bad) {
    if (tid == 0) p.status[0] = 3;  // every later kernel of the backward exits
    return;
  }
  {
    int64_t P = base;
    for (int u = lo; u < hi; ++u) {
      const int64_t b = blocks_of(u);
      const int c = chunk_of(P, b);
      const int4 it = items[u];
      const int x = p.tile_base[it.x] + it.y;
      p.kv_chunk[x] = c;
      p.kv_off[x] = P - p.chunk_first[c];
      P += b;
    }
  }
  if (tid == 0) p.status[0] = 0;
}

template <int D>
__global__ __launch_bounds__(PRO_THREADS) void bwd_prologue(BwdParams p) {
  __shared__ uint8_t flags[PRO_CHUNK];
  __shared__ int wv[PRO_THREADS / 64][3];
  __shared__ int red[3][PRO_THREADS / 64];
  __shared__ int kstart;
  __shared__ Seg carry_sh;

  if ((int)blockIdx.x == p.Hq) {
    for (int x = threadIdx.x; x < 16 * (p.max_chunks + 1); x += PRO_THREADS) p.counters[x] = 0;
    layout_chunks(p);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, grp = p.Hq / p.Hkv, g = h / grp;
  const int T = p.T;
  const int C = (D == 128) ? 35 : 34;  // smallest C with 2 d 448^3 <= 2^C
  const int c_lo = p.n_docs > 0 ? p.cu[0] : T;
  const int c_hi = p.n_docs > 0 ? p.cu[p.n_docs] : T;
  const uint8_t* sdo = p.sdo + (int64_t)h * T;
  const uint8_t* sv = p.sv + (int64_t)g * T;
  const uint8_t* sk = p.sk + (int64_t)g * T;
  int16_t* pi = p.pi + (int64_t)h * T;

  // zero rows outside every document
  {
    const int64_t n_out = (int64_t)c_lo + (T - c_hi);
    for (int64_t x = tid; x < n_out * D; x += PRO_THREADS) {
      const int r = (int)(x / D), dd = (int)(x % D);
      const int t = r < c_lo ? r : c_hi + (r - c_lo);
      p.dq[(int64_t)t * p.dqst + (int64_t)h * p.dqsh + dd] = 0;
      if (h % grp == 0) {
        p.dk[(int64_t)t * p.dkst + (int64_t)g * p.dksh + dd] = 0;
        p.dv[(int64_t)t * p.dvst + (int64_t)g * p.dvsh + dd] = 0;
      }
    }
  }

  if (!p.causal) {
    int mdo = 0, mv = 0, mk = 0;
    for (int t = c_lo + tid; t < c_hi; t += PRO_THREADS) {
      mdo = max(mdo, (int)sdo[t]);
      mv = max(mv, (int)sv[t]);
      mk = max(mk, (int)sk[t]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      mdo = max(mdo, __shfl_xor(mdo, off, 64));
      mv = max(mv, __shfl_xor(mv, off, 64));
      mk = max(mk, __shfl_xor(mk, off, 64));
    }
    if (lane == 0) { red[0][wave] = mdo; red[1][wave] = mv; red[2][wave] = mk; }
    __syncthreads();
    int a = 0, b = 0, cc = 0;
    for (int w = 0; w < PRO_THREADS / 64; ++w) { a = max(a, red[0][w]); b = max(b, red[1][w]); cc = max(cc, red[2][w]); }
    int val = 15 - C - ((a - 127) + (b - 127) + (cc - 127));
    val = min(64, max(-64, val));
    for (int t = tid; t < T; t += PRO_THREADS) {
      const int16_t x = (t >= c_lo && t < c_hi) ? (int16_t)val : (int16_t)0;
      pi[t] = x;
      if (p.pi_out) p.pi_out[(int64_t)h * T + t] = x;
    }
    return;
  }

  // causal: running maxima of the V and K block exponents from each document's start
  __shared__ int n_marked;
  if (tid == 0) {
    carry_sh = Seg{0, -1, -1};
    kstart = 0;  // first document starting at or after C0: 0 for C0 = 0 (cu[0] >= 0)
    n_marked = 0;
  }
  for (int C0 = 0; C0 < T; C0 += PRO_CHUNK) {
    for (int x = tid; x < PRO_CHUNK; x += PRO_THREADS) flags[x] = 0;
    __syncthreads();
    // every document starting in the chunk is marked once (a thread stops at its first document
    // past the chunk; the ones after it start later still), so the next chunk's first document
    // is kstart plus their number
    int marked = 0;
    for (int k = kstart + tid; k < p.n_docs && p.cu[k] < C0 + PRO_CHUNK; k += PRO_THREADS) {
      flags[p.cu[k] - C0] = 1;
      ++marked;
    }
    if (marked) atomicAdd(&n_marked, marked);
    __syncthreads();
    // thread-local inclusive scan of 4 tokens
    Seg loc[4];
    Seg run{0, -1, -1};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = C0 + 4 * tid + e;
      Seg x{0, -1, -1};
      if (t < T) x = Seg{(int)flags[4 * tid + e], (int)sv[t], (int)sk[t]};
      run = seg_op(run, x);
      loc[e] = run;
    }
    // workgroup exclusive scan of the per-thread aggregates
    Seg incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      Seg y{__shfl_up(incl.f, off, 64), __shfl_up(incl.v, off, 64), __shfl_up(incl.k, off, 64)};
      if (lane >= off) incl = seg_op(y, incl);
    }
    if (lane == 63) { wv[wave][0] = incl.f; wv[wave][1] = incl.v; wv[wave][2] = incl.k; }
    __syncthreads();
    Seg pre = carry_sh;  // everything before this chunk
    for (int w = 0; w < wave; ++w) pre = seg_op(pre, Seg{wv[w][0], wv[w][1], wv[w][2]});
    Seg ex_lane{__shfl_up(incl.f, 1, 64), __shfl_up(incl.v, 1, 64), __shfl_up(incl.k, 1, 64)};
    if (lane > 0) pre = seg_op(pre, ex_lane);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = C0 + 4 * tid + e;
      if (t >= T) continue;
      const Seg s = seg_op(pre, loc[e]);
      int16_t x = 0;
      if (t >= c_lo && t < c_hi) {
        int val = 15 - C - (((int)sdo[t] - 127) + (s.v - 127) + (s.k - 127));
        x = (int16_t)min(64, max(-64, val));
      }
      pi[t] = x;
      if (p.pi_out) p.pi_out[(int64_t)h * T + t] = x;
    }
    __syncthreads();
    if (tid == PRO_THREADS - 1) carry_sh = seg_op(pre, run);
    if (tid == 0) {
      kstart += n_marked;
      n_marked = 0;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int d, int grid, hipStream_t s) {
  // the prologue lays out the chunks; then each chunk's key-tile pass fills the store and its
  // dQ pass consumes it (stream order keeps the two apart and the chunks in sequence)
  if (d == 128) hipLaunchKernelGGL(bwd_prologue<128>, dim3(p.Hq + 1), dim3(PRO_THREADS), 0, s, p);
  else hipLaunchKernelGGL(bwd_prologue<64>, dim3(p.Hq + 1), dim3(PRO_THREADS), 0, s, p);
  if (p.small) {  // the short documents' rows (after the prologue: pi, and the layout's status)
    const hipError_t e = launch_small_bwd(p, d, s);
    if (e != hipSuccess) return e;
  }
  auto chunks = [&](auto bk, auto dk) {
    for (int c = 0; c < p.max_chunks; ++c) {
      BwdParams q = p;
      q.chunk = c;
      hipLaunchKernelGGL(bk, dim3(grid), dim3(BWD_THREADS), 0, s, q);
      hipLaunchKernelGGL(dk, dim3(2 * grid), dim3(DQ_THREADS), 0, s, q);
    }
  };
  if (p.precise) {  // causal only (checked by the caller); one chunk, nothing stored
    BwdParams q = p;
    q.chunk = 0;
    if (d == 128) hipLaunchKernelGGL((bwd_kernel<128, true, true, false>), dim3(grid), dim3(BWD_THREADS), 0, s, q);
    else hipLaunchKernelGGL((bwd_kernel<64, true, true, false>), dim3(grid), dim3(BWD_THREADS), 0, s, q);
    const hipError_t e = hipGetLastError();
    return e != hipSuccess ? e : launch_dq_precise(q, d, grid, s);
  }
  const bool f4 = p.q4 != nullptr;  // 4-bit scores
  if (d == 128) {
    if (p.causal_mask) {
      if (f4) chunks(bwd_kernel<128, true, false, true>, dq_kernel<128>);
      else chunks(bwd_kernel<128, true, false, false>, dq_kernel<128>);
    } else {
      if (f4) chunks(bwd_kernel<128, false, false, true>, dq_kernel<128>);
      else chunks(bwd_kernel<128, false, false, false>, dq_kernel<128>);
    }
  } else {
    if (p.causal_mask) {
      if (f4) chunks(bwd_kernel<64, true, false, true>, dq_kernel<64>);
      else chunks(bwd_kernel<64, true, false, false>, dq_kernel<64>);
    } else {
      if (f4) chunks(bwd_kernel<64, false, false, true>, dq_kernel<64>);
      else chunks(bwd_kernel<64, false, false, false>, dq_kernel<64>);
    }
  }
  return hipGetLastError();
}

}  // namespace flamia
