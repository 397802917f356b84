// Forward: causal packed-document attention on token-block MXFP8 operands
// (jaehun.me review §1.2 online softmax, §3.1 token-block scales and score factorisation,
//  §3.4 packed documents and work scheduling).
//
// Persistent grid, one 512-thread workgroup per compute unit.  A work unit is (forward item,
// query head): 256 consecutive queries of one document.  Wave w (of 8) owns queries
// 32w..32w+31 of the item.  Per 128-key tile (visited from the diagonal tile down to tile 0):
//   S^T (keys x queries) = K Q^T   : scaled MFMA, A = K rows from LDS, B = Q held in registers;
//                                    the hardware applies 2^(e(K) + e(Q)), the score scale
//                                    softmax_scale*log2(e) is one FMA per element;
//   online softmax per query       : each lane holds 64 of a query's 128 scores, the other 64
//                                    sit in lane l ^ 32 (one permlane swap per reduction);
//   P operand                      : E4M3(2^8 p) from the score registers, which already are in
//                                    the MFMA operand order (no data movement between lanes);
//   O^T += V^T P^T                 : A = V^T read from the row-major V tile with transpose reads.
// One E4M3 copy of K and V serves both products; only the LDS read instruction differs.  K/V
// tiles arrive by direct global-to-LDS loads one tile ahead (two buffers each).  A wave issues
// its instructions one at a time, so the PV product's matrix instructions are spread between
// the vector instructions of the exponentials and the row sum, where they run underneath them.
#include "device_common.h"
#include "kernels.h"

namespace flamia {

namespace {

// Workgroup shapes: W = 8 waves (a 256-query unit, one workgroup per CU) for long documents, or
// W = 4 (a 128-query unit, two workgroups per CU, whose barriers and loads interleave) where
// documents are short and a unit covers few key tiles.  Both compute the same values.
template <int W>
constexpr int fwd_threads() { return 64 * W; }

template <int D>
struct FwdSmem {
  uint8_t k[2][KV_TILE * D];  // 4-bit scores: the 4-bit K tile in the first half
  uint8_t v[2][KV_TILE * D];
  uint8_t sk[2][KV_TILE];
  uint8_t sv[2][KV_TILE];
  uint8_t sk4[2][KV_TILE * D / 32];  // 4-bit scores: each key's d/32 exponent bytes
};

// Tile i of a unit (key tile kappa_hi - i) sits in K and V buffers i % 2: while tile i is current,
// tile i + 1 is being loaded.
// K and V rows go global -> LDS with direct loads, each lane fetching the 16-byte chunk that
// belongs at its LDS position under the tile's swizzle; rows past the document end repeat its
// last row (their scores are masked, their probabilities are zero, and the values are finite).
// The scale bytes go through a register, returned here and stored by store_scales: thread
// t < 128 holds the K scale of key t, 128 <= t < 256 the V scale of key t - 128.
template <int D, int W>
__device__ __forceinline__ uint32_t issue_tile(const FwdParams& p, FwdSmem<D>& sm, int kb, int vb, int g,
                                               int doc_start, int L, int kappa, int wave, int lane) {
  constexpr int CPR = D / 16;                        // 16-byte chunks per row
  constexpr int BLOCKS = KV_TILE * D / 1024;         // 1 KiB wave blocks per tensor
  constexpr int PER_WAVE = 2 * BLOCKS / W;           // K and V blocks per wave
  static_assert(PER_WAVE * W == 2 * BLOCKS, "blocks split evenly over the waves");
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int wb = wave * PER_WAVE + i;              // K blocks, then V blocks
    const bool is_v = wb >= BLOCKS;
    const int blk = is_v ? wb - BLOCKS : wb;
    const int pos = blk * 64 + lane;                 // chunk position in the tile
    const int row = pos / CPR, pc = pos % CPR;
    const int lc = pc ^ lds_swizzle<D>(row);         // logical chunk stored there
    uint8_t* dst = (is_v ? sm.v[vb] : sm.k[kb]) + blk * 1024;
    if (KV_TILE * kappa + blk * (1024 / D) < L) {
      const int key = min(KV_TILE * kappa + row, L - 1);
      const uint8_t* src = (is_v ? p.v : p.k) + ((int64_t)(doc_start + key) * p.Hkv + g) * D + 16 * lc;
      dma_load16(src, lds_addr(dst));
    } else if (is_v) {
      // a block wholly past the document end: its V rows meet zero probabilities and only need
      // to be finite; its K rows are masked and are not loaded at all
      *reinterpret_cast<uint4*>(dst + 16 * lane) = make_uint4(0, 0, 0, 0);
    }
  }
  const int tid = threadIdx.x;
  uint32_t sc = 127;
  if (tid < 2 * KV_TILE) {
    const int key = KV_TILE * kappa + (tid & (KV_TILE - 1));
    if (key < L) sc = (tid < KV_TILE ? p.sk : p.sv)[(int64_t)g * p.T + doc_start + key];
  }
  return sc;
}

// A tile wholly inside the document (every tile after a unit's first): no row needs clamping,
// so each of the wave's blocks is one wave-uniform base address plus a per-lane offset. Within a
// wave the blocks are consecutive and of one tensor; block i sits 64 i / CPR rows below block 0,
// and since the swizzle is a bit permutation of row bits below that step, its chunk differs
// from block 0's by the swizzle of that row step alone, whatever the lane.
template <int D, int W>
__device__ __forceinline__ uint32_t issue_full_tile(const FwdParams& p, FwdSmem<D>& sm, int kb, int vb, int g,
                                                    int doc_start, int kappa, int wave, uint32_t voff0) {
  constexpr int CPR = D / 16;
  constexpr int BLOCKS = KV_TILE * D / 1024;
  constexpr int PER_WAVE = 2 * BLOCKS / W;
  static_assert(BLOCKS % PER_WAVE == 0, "no wave's blocks span both tensors");
  static_assert(16 * CPR <= D && (D & (D - 1)) == 0, "chunk offsets stay below the row stride");
  const bool is_v = wave * PER_WAVE >= BLOCKS;
  const int blk0 = wave * PER_WAVE - (is_v ? BLOCKS : 0);
  uint8_t* dst = (is_v ? sm.v[vb] : sm.k[kb]) + blk0 * 1024;
  // the base address from the wave index read as a scalar (the LDS address above keeps the
  // per-lane form, which the compiler turns into a scalar itself)
  const int ws = __builtin_amdgcn_readfirstlane(wave);
  const bool vs = ws * PER_WAVE >= BLOCKS;
  const uint8_t* base =
      (vs ? p.v : p.k) + ((int64_t)(doc_start + KV_TILE * kappa + (ws * PER_WAVE - (vs ? BLOCKS : 0)) * (64 / CPR)) * p.Hkv + g) * D;
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const uint32_t dsw = 16 * lds_swizzle<D>(i * (64 / CPR));
    dma_load16_sv(base + (int64_t)i * (64 / CPR) * p.Hkv * D, voff0 ^ dsw, lds_addr(dst + i * 1024));
  }
  const int tid = threadIdx.x;
  uint32_t sc = 127;
  if (tid < 2 * KV_TILE)
    sc = (tid < KV_TILE ? p.sk : p.sv)[(int64_t)g * p.T + doc_start + KV_TILE * kappa + (tid & (KV_TILE - 1))];
  return sc;
}
// Per-lane byte offset, from its first row, of the chunk the lane fetches in the wave's first
// block of a full tile.
template <int D>
__device__ __forceinline__ uint32_t tile_offset(const FwdParams& p, int lane) {
  constexpr int CPR = D / 16;
  const int row = lane / CPR, pc = lane % CPR;
  return (uint32_t)(row * p.Hkv * D + 16 * (pc ^ lds_swizzle<D>(row)));
}

// 4-bit scores: tile kappa's 4-bit K rows (d/2 bytes each) and its V rows into buffers kb, vb by
// direct loads, the 1 KiB wave blocks dealt round robin over the waves; rows past the document end
// repeat its last row and blocks wholly past it are zero-filled, as in issue_tile.  Returns the
// scale word: thread t < 128 the d/32 K exponent bytes of key t, 128 <= t < 256 the V byte of key
// t - 128.
template <int D, int W>
__device__ __forceinline__ uint32_t issue_tile4(const FwdParams& p, FwdSmem<D>& sm, int kb, int vb, int g,
                                                int doc_start, int L, int kappa, int wave, int lane) {
  constexpr int K4B = D / 2;                // bytes per 4-bit K row
  constexpr int BK = KV_TILE * K4B / 1024;  // 1 KiB blocks of the K tile
  constexpr int BV = KV_TILE * D / 1024;    // and of the V tile
  for (int wb = __builtin_amdgcn_readfirstlane(wave); wb < BK + BV; wb += W) {
    if (wb < BK) {
      constexpr int CPR = K4B / 16;
      const int pos = wb * 64 + lane, row = pos / CPR;
      const int lc = (pos % CPR) ^ lds_swizzle<K4B>(row);
      uint8_t* dst = sm.k[kb] + wb * 1024;
      if (KV_TILE * kappa + wb * (1024 / K4B) < L) {
        const int key = min(KV_TILE * kappa + row, L - 1);
        dma_load16(p.k4 + ((int64_t)(doc_start + key) * p.Hkv + g) * K4B + 16 * lc, lds_addr(dst));
      } else {
        *reinterpret_cast<uint4*>(dst + 16 * lane) = make_uint4(0, 0, 0, 0);
      }
    } else {
      constexpr int CPR = D / 16;
      const int blk = wb - BK, pos = blk * 64 + lane, row = pos / CPR;
      const int lc = (pos % CPR) ^ lds_swizzle<D>(row);
      uint8_t* dst = sm.v[vb] + blk * 1024;
      if (KV_TILE * kappa + blk * (1024 / D) < L) {
        const int key = min(KV_TILE * kappa + row, L - 1);
        dma_load16(p.v + ((int64_t)(doc_start + key) * p.Hkv + g) * D + 16 * lc, lds_addr(dst));
      } else {
        *reinterpret_cast<uint4*>(dst + 16 * lane) = make_uint4(0, 0, 0, 0);
      }
    }
  }
  const int tid = threadIdx.x;
  uint32_t sc = 127;
  if (tid < 2 * KV_TILE) {
    const int key = KV_TILE * kappa + (tid & (KV_TILE - 1));
    if (tid < KV_TILE) {
      sc = 0x7F7F7F7Fu;
      if (key < L) {
        const uint8_t* e4 = p.sk4 + ((int64_t)g * p.T + doc_start + key) * (D / 32);
        sc = D == 128 ? *reinterpret_cast<const uint32_t*>(e4) : (uint32_t)*reinterpret_cast<const uint16_t*>(e4);
      }
    } else if (key < L) {
      sc = p.sv[(int64_t)g * p.T + doc_start + key];
    }
  }
  return sc;
}

// A tile wholly inside the document (every tile after a unit's first), 4-bit scores: each block
// is one wave-uniform base address plus a per-lane offset.  Within a K block the row step of
// the block leaves the swizzle unchanged (rows 16 or 32 apart), so one K offset serves every
// block; V blocks take issue_full_tile's offset with the swizzle of their row step.
template <int D, int W>
__device__ __forceinline__ uint32_t issue_full_tile4(const FwdParams& p, FwdSmem<D>& sm, int kb, int vb, int g,
                                                     int doc_start, int kappa, int wave, uint32_t voff_k,
                                                     uint32_t voff_v) {
  constexpr int K4B = D / 2, BK = KV_TILE * K4B / 1024, BV = KV_TILE * D / 1024;
  constexpr int RK = 1024 / K4B, RV = 1024 / D;  // rows per block
  const int64_t row0 = doc_start + KV_TILE * kappa;
  for (int wb = __builtin_amdgcn_readfirstlane(wave); wb < BK + BV; wb += W) {
    if (wb < BK) {
      const uint8_t* base = p.k4 + ((row0 + wb * RK) * p.Hkv + g) * K4B;
      dma_load16_sv(base, voff_k, lds_addr(sm.k[kb] + wb * 1024));
    } else {
      const int blk = wb - BK;
      const uint8_t* base = p.v + ((row0 + blk * RV) * p.Hkv + g) * D;
      dma_load16_sv(base, voff_v ^ (16 * lds_swizzle<D>(blk * RV)), lds_addr(sm.v[vb] + blk * 1024));
    }
  }
  const int tid = threadIdx.x;
  uint32_t sc = 127;
  if (tid < 2 * KV_TILE) {
    const int64_t key = row0 + (tid & (KV_TILE - 1));
    if (tid < KV_TILE) {
      const uint8_t* e4 = p.sk4 + ((int64_t)g * p.T + key) * (D / 32);
      sc = D == 128 ? *reinterpret_cast<const uint32_t*>(e4) : (uint32_t)*reinterpret_cast<const uint16_t*>(e4);
    } else {
      sc = p.sv[(int64_t)g * p.T + key];
    }
  }
  return sc;
}
// Per-lane byte offset, from its block's first row, of the chunk the lane fetches in a 4-bit K
// block of a full tile.
template <int D>
__device__ __forceinline__ uint32_t tile_offset4(const FwdParams& p, int lane) {
  constexpr int K4B = D / 2, CPR = K4B / 16;
  const int row = lane / CPR, pc = lane % CPR;
  return (uint32_t)(row * p.Hkv * K4B + 16 * (pc ^ lds_swizzle<K4B>(row)));
}

template <int D>
__device__ __forceinline__ void store_scales4(FwdSmem<D>& sm, int kb, int vb, uint32_t sc) {
  const int tid = threadIdx.x;
  if (tid < KV_TILE) {
    if constexpr (D == 128) *reinterpret_cast<uint32_t*>(&sm.sk4[kb][4 * tid]) = sc;
    else *reinterpret_cast<uint16_t*>(&sm.sk4[kb][2 * tid]) = (uint16_t)sc;
  } else if (tid < 2 * KV_TILE) {
    sm.sv[vb][tid - KV_TILE] = (uint8_t)sc;
  }
}

template <int D>
__device__ __forceinline__ void store_scales(FwdSmem<D>& sm, int kb, int vb, uint32_t sc) {
  const int tid = threadIdx.x;
  if (tid < KV_TILE) sm.sk[kb][tid] = (uint8_t)sc;
  else if (tid < 2 * KV_TILE) sm.sv[vb][tid - KV_TILE] = (uint8_t)sc;
}

// CAUSAL: keys after the query are masked (else every key of the document is visible).
// PRECISE (the precision options, with per-token scales): V's exponent is folded into the
// probability operand against the row's running maximum of visited V exponents, and V enters
// the product with its bare codes.
// QK4 (4-bit scores, [J] §3.1 "Mixed NVFP4/FP8 path", §3.4 "Softmax throughput"): S^T takes the
// E2M1 copies of K and Q (one exponent per 32 channels of a token, per lane as the instruction's
// scale bytes), and the probability operand is quantised in the log domain: each 32-key group of
// the tile gets the round-up exponent of its largest probability, found from the group's largest
// score (one exponential per group), and its codes are E4M3(p 2^-e) with operand scale 2^e.
template <int D, int W, bool CAUSAL, bool PRECISE, bool QK4>
__global__ __launch_bounds__(fwd_threads<W>(), 8 / W) void fwd_kernel(FwdParams p) {
  static_assert(!(PRECISE && QK4), "separate paths");
  constexpr int FWD_THREADS = fwd_threads<W>();
  constexpr int NC = D / 64;   // 64-wide d chunks of the score contraction
  constexpr int NDB = D / 32;  // 32-wide d blocks of the output
  __shared__ FwdSmem<D> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int n_items = list_walk_items(p.list, p.T, p.small);  // short documents: the small-document pass
  const int4* items = reinterpret_cast<const int4*>(p.list + 4);
  constexpr int QU = 32 * W;                 // queries per workgroup unit
  constexpr int PARTS = ITEM_Q / QU;         // units per work item and head
  const int n_units = n_items * PARTS * p.Hq;
  const int G = gridDim.x, wg = blockIdx.x;
  const int grp = p.Hq / p.Hkv;
  const float c = p.c;
  const uint32_t voff0 = tile_offset<D>(p, lane);
  const uint32_t voff4 = QK4 ? tile_offset4<D>(p, lane) : 0u;

  // Units: the static serpentine walk (round r of workgroup w takes r G + w, or r G + G - 1 - w on
  // odd rounds), or, for a list whose header word 3 gives the position of its unit counters,
  // dynamically: each workgroup takes its first unit by index and each next one from the counter
  // ([0]) when it has finished the last; [1] counts the workgroups done
  const int ctr_pos = p.list[3];
  const bool dyn = ctr_pos != 0;
  int32_t* const ctr = p.list + ctr_pos;
  __shared__ int unit_slot;
  int u = wg;
  for (int round = 0;; ++round) {
    if (!dyn) u = round * G + ((round & 1) ? (G - 1 - wg) : wg);
    else if (round > 0) u = next_unit(ctr, &unit_slot, G);
    if (u >= n_units) break;
    const int4 it = items[u / (PARTS * p.Hq)];
    const int h = u % p.Hq, g = h / grp, part = (u / p.Hq) % PARTS;
    const int doc = it.x, b = it.y;
    const int doc_start = p.cu[doc];
    const int L = p.cu[doc + 1] - doc_start;
    const int q0 = ITEM_Q * b + QU * part;             // first query (document offset) of the unit
    if (q0 >= L) continue;                              // the item ends before this part (uniform)
    const int q_wave = q0 + 32 * wave;                  // first query of this wave
    const bool wave_active = q_wave < L;
    const int q_rel = q_wave + n;
    const bool row_valid = q_rel < L;
    // this wave's first (diagonal) tile: causal, the tile of its queries; non-causal, the
    // document's last key tile, the one every row starts from
    const int kd = CAUSAL ? q_wave / KV_TILE : (L - 1) / KV_TILE;
    const int last_row = min(q0 + QU, L) - 1;
    const int kappa_hi = CAUSAL ? last_row / KV_TILE : (L - 1) / KV_TILE;

    // Q operand (B of S^T): lane (n, hh) holds d = 64c + 32hh .. +31 of query n.
    v8i qop[NC];
    int q_scale = 127;
    // QK4: the 4-bit Q operand, the same d range as 16 bytes, and its exponent byte per chunk
    v4i qop4[NC];
    int q_scale4[NC];
    if constexpr (QK4) {
      const int64_t qa = (int64_t)(doc_start + q_rel);
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        qop4[cc] = v4i{0, 0, 0, 0};
        q_scale4[cc] = 127;
        if (row_valid) {
          qop4[cc] = *reinterpret_cast<const v4i*>(p.q4 + (qa * p.Hq + h) * (D / 2) + 32 * cc + 16 * hh);
          q_scale4[cc] = p.sq4[((int64_t)h * p.T + qa) * (D / 32) + 2 * cc + hh];
        }
      }
    } else {
      const int64_t qa = (int64_t)(doc_start + q_rel);
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        if (row_valid) {
          const uint4* src = reinterpret_cast<const uint4*>(p.q + (qa * p.Hq + h) * D + 64 * cc + 32 * hh);
          const uint4 a = src[0], bb = src[1];
          qop[cc][0] = a.x; qop[cc][1] = a.y; qop[cc][2] = a.z; qop[cc][3] = a.w;
          qop[cc][4] = bb.x; qop[cc][5] = bb.y; qop[cc][6] = bb.z; qop[cc][7] = bb.w;
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) qop[cc][i] = 0;
        }
      }
      if (row_valid) q_scale = p.sq[(int64_t)h * p.T + doc_start + q_rel];
    }

    v16f oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = v16f{};
    float m = -__builtin_inff();  // running max, score units
    float l = 0.f;                // this lane's share of the row sum of 2^8 p
    int vref = -119;              // PRECISE: largest V exponent among the keys visited so far

    lds_barrier();  // the previous unit's readers are done with every buffer
    {
      const uint32_t sc = QK4 ? issue_tile4<D, W>(p, sm, 0, 0, g, doc_start, L, kappa_hi, wave, lane)
                              : issue_tile<D, W>(p, sm, 0, 0, g, doc_start, L, kappa_hi, wave, lane);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
      if constexpr (QK4) store_scales4<D>(sm, 0, 0, sc);
      else store_scales<D>(sm, 0, 0, sc);
    }
    lds_barrier();
    for (int kappa = kappa_hi, it = 0; kappa >= 0; --kappa, ++it) {
      const int kb = it & 1;
      uint32_t scn = 127;
      if (kappa > 0) {
        if constexpr (QK4) scn = issue_full_tile4<D, W>(p, sm, kb ^ 1, kb ^ 1, g, doc_start, kappa - 1, wave, voff4, voff0);
        else scn = issue_full_tile<D, W>(p, sm, kb ^ 1, kb ^ 1, g, doc_start, kappa - 1, wave, voff0);
      }
      if (wave_active && kappa <= kd) {
        const uint8_t* kt = sm.k[kb];
        // ---- S^T for the 4 key blocks of the tile.  K operand k (key block k / NC, d chunk
        // k % NC) is read SAHEAD matrix instructions early into a ring of registers, so each
        // instruction finds its operand loaded instead of waiting out an LDS round trip.
        v16f s[4];
        if constexpr (QK4) {
          // S^T from the 4-bit copies: A = K rows (16 bytes per lane and chunk), the key's
          // exponent byte of d-block 2 cc + hh as the A scale
          constexpr int K4B = D / 2, NS = 4 * NC, SAHEAD = 3;
          auto read_k = [&](int k) { return lds_read_row16<K4B>(kt, 32 * (k / NC) + n, 32 * (k % NC) + 16 * hh); };
          v4i kring[SAHEAD];
#pragma unroll
          for (int k = 0; k < SAHEAD; ++k) kring[k] = read_k(k);
          int ks[NS];  // all read ahead: an instruction never waits for its scale byte
#pragma unroll
          for (int k = 0; k < NS; ++k) ks[k] = sm.sk4[kb][(32 * (k / NC) + n) * (D / 32) + 2 * (k % NC) + hh];
#pragma unroll
          for (int k = 0; k < NS; ++k) {
            const int kb4 = k / NC, cc = k % NC;
            s[kb4] = mfma_scaled_fp4(kring[k % SAHEAD], qop4[cc], cc ? s[kb4] : v16f{}, ks[k], q_scale4[cc]);
            if (k + SAHEAD < NS) kring[k % SAHEAD] = read_k(k + SAHEAD);
            __builtin_amdgcn_sched_barrier(0);
          }
          // the group maxima read these right away: a fixed margin after the last product
#pragma unroll
          for (int kb4 = 0; kb4 < 4; ++kb4) mfma_drain(s[kb4]);
        } else {
          constexpr int NS = 4 * NC, SAHEAD = 3;
          auto read_k = [&](int k) { return lds_read_row32<D>(kt, 32 * (k / NC) + n, 64 * (k % NC) + 32 * hh); };
          v8i kring[SAHEAD];
#pragma unroll
          for (int k = 0; k < SAHEAD; ++k) kring[k] = read_k(k);
          int ks[4];
#pragma unroll
          for (int kb4 = 0; kb4 < 4; ++kb4) ks[kb4] = sm.sk[kb][32 * kb4 + n];
#pragma unroll
          for (int k = 0; k < NS; ++k) {
            const int kb4 = k / NC, cc = k % NC;
            s[kb4] = mfma_scaled(kring[k % SAHEAD], qop[cc], cc ? s[kb4] : v16f{}, ks[kb4], q_scale);
            if (k + SAHEAD < NS) kring[k % SAHEAD] = read_k(k + SAHEAD);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // ---- mask on the first tile: keys after the query (causal) or past the document end
        // (non-causal; causally those lie after the query too)
        if (kappa == kd) {
          // key 128 kappa + 32 kb4 + acc_row(i, hh) is masked when the constant part
          // 32 kb4 + acc_row(i, 0) exceeds lim; lim is formed here, opaque to the compiler, so
          // the 64 comparisons stay in this branch instead of held as lane masks in scalar
          // registers across the loop
          int lim = (CAUSAL ? q_rel : L - 1) - KV_TILE * kappa - 4 * hh;
          asm volatile("" : "+v"(lim));
#pragma unroll
          for (int kb4 = 0; kb4 < 4; ++kb4) mfma_drain(s[kb4]);  // the mask may follow the last product closely
#pragma unroll
          for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (32 * kb4 + acc_row(i, 0) > lim) s[kb4][i] = -__builtin_inff();
        }
#ifdef FLAMIA_DEBUG_DUMP
        if (row_valid && p.dbg.fwd_s) {  // test builds: the score accumulator after the mask
#pragma unroll
          for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key_rel = KV_TILE * kappa + 32 * kb4 + acc_row(i, hh);
              const int64_t x = key_rel < L ? dbg_index(p.dbg, h, doc_start + q_rel, doc_start + key_rel) : -1;
              if (x >= 0) p.dbg.fwd_s[x] = s[kb4][i];
            }
        }
#endif
        // ---- running max (raw accumulator units, then scaled once); QK4 keeps each 32-key
        // group's maximum for its exponent
        float mx = -__builtin_inff();
        float gmx[4];
        if constexpr (QK4) {
#pragma unroll
          for (int kb4 = 0; kb4 < 4; ++kb4) {
            gmx[kb4] = -__builtin_inff();
#pragma unroll
            for (int i = 0; i < 16; ++i) gmx[kb4] = fmaxf(gmx[kb4], s[kb4][i]);
            gmx[kb4] = halves_max(gmx[kb4]);
            mx = fmaxf(mx, gmx[kb4]);
          }
        } else {
#pragma unroll
          for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb4][i]);
          mx = halves_max(mx);
        }
        const float m_new = fmaxf(m, mx * c);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        if (__any(alpha != 1.0f)) {
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
          l *= alpha;
        }
        m = m_new;
        // ---- p = 2^(t - m), scaled by 2^8 for the E4M3 operand, packed into operand order;
        // O^T += V^T P^T in two halves of 64 keys.  A wave issues one instruction at a time, so
        // the eight matrix instructions are spread between vector instructions instead of
        // issued in a burst: the first half's run between the exponentials of key blocks 2 and
        // 3 (the probabilities overwrite their scores), the second half's between those blocks'
        // additions to the row sum, which come last (the order of the additions is unchanged).
        // QK4: the probabilities unshifted, each group's exponent byte from its largest one
        const float bias = QK4 ? -m_new : (float)P_SHIFT - m_new;
        uint32_t pe[4];
        if constexpr (QK4)
#pragma unroll
          for (int kb4 = 0; kb4 < 4; ++kb4) pe[kb4] = e8m0_byte_nonneg(__builtin_amdgcn_exp2f(fmaf(gmx[kb4], c, -m_new)));
        const uint8_t* vt = sm.v[kb];
        v8i pop[2];
        int vs[2];
#pragma unroll
        for (int ci = 0; ci < 2; ++ci) vs[ci] = sm.sv[kb][64 * ci + 32 * hh];
        // PRECISE: the V exponent bytes of element group (kb4, w4), keys 32 kb4 + 8 w4 + 4 hh + e
        auto ev_word = [&](int kb4, int w4) {
          return *reinterpret_cast<const uint32_t*>(&sm.sv[kb][32 * kb4 + 8 * w4 + 4 * hh]);
        };
        if constexpr (PRECISE) {
          // the row's reference: the largest exponent among its visible keys (finite scores; the
          // mask has made the others -inf) and the keys of earlier tiles, at least -119
          uint32_t tmax = 0;
#pragma unroll
          for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
              const uint32_t wv = ev_word(kb4, w4);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (s[kb4][4 * w4 + e] > -__builtin_inff()) tmax = max(tmax, (wv >> (8 * e)) & 0xFFu);
            }
          const auto sw = __builtin_amdgcn_permlane32_swap((int)tmax, (int)tmax, false, false);
          tmax = max((uint32_t)sw[0], (uint32_t)sw[1]);  // both lanes of the query
          vref = max(vref, (int)tmax - 127);
        }
        // the probability codes: E4M3 of 2^8 p, PRECISE times 2^(e(V_j) - vref) (exact)
        auto pcode = [&](float a0, float a1, float a2, float a3, int kb4, int w4) {
          if constexpr (PRECISE) {
            const uint32_t wv = ev_word(kb4, w4);
            return pack4_fp8(__builtin_ldexpf(a0, (int)(wv & 0xFFu) - 127 - vref),
                             __builtin_ldexpf(a1, (int)((wv >> 8) & 0xFFu) - 127 - vref),
                             __builtin_ldexpf(a2, (int)((wv >> 16) & 0xFFu) - 127 - vref),
                             __builtin_ldexpf(a3, (int)(wv >> 24) - 127 - vref));
          } else if constexpr (QK4) {
            return pack4_fp8_scaled(a0, a1, a2, a3, pe[kb4]);
          } else {
            return pack4_fp8(a0, a1, a2, a3);
          }
        };
        const int v_scale = PRECISE ? 127 : 0;          // bare V codes (PRECISE)
        const int p_scale = 127 - P_SHIFT + (PRECISE ? vref : 0);
        auto read_v = [&](int k) { return lds_read_tr32<D>(vt, 64 * (k / NDB), 32 * (k % NDB), lane); };
        constexpr int NPV = 2 * NDB;  // matrix instructions: (64-key half ci, d-block db)
        v8i ring[2];
        // QK4: lane (n, hh) scales key half hh of the 64-key chunk: group 2 ci + hh
        int psc[2] = {p_scale, p_scale};
        if constexpr (QK4) {
          psc[0] = (int)(hh ? pe[1] : pe[0]);
          psc[1] = (int)(hh ? pe[3] : pe[2]);
        }
        auto pv_step = [&](int k) {
          oacc[k % NDB] = mfma_scaled(ring[k & 1], pop[k / NDB], oacc[k % NDB], PRECISE ? v_scale : vs[k / NDB],
                                      QK4 ? psc[k / NDB] : p_scale);
          if (k + 2 < NPV) ring[k & 1] = read_v(k + 2);
        };
        // blocks 0, 1: probabilities, row sum, codes
#pragma unroll
        for (int kb4 = 0; kb4 < 2; ++kb4)
#pragma unroll
          for (int w4 = 0; w4 < 4; ++w4) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb4][4 * w4 + 0], c, bias));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb4][4 * w4 + 1], c, bias));
            const float p2 = __builtin_amdgcn_exp2f(fmaf(s[kb4][4 * w4 + 2], c, bias));
            const float p3 = __builtin_amdgcn_exp2f(fmaf(s[kb4][4 * w4 + 3], c, bias));
            l += (p0 + p1) + (p2 + p3);
            pop[0][4 * kb4 + w4] = pcode(p0, p1, p2, p3, kb4, w4);
          }
        ring[0] = read_v(0);
        ring[1] = read_v(1);
        asm volatile("" : "+v"(l));  // this part of the row sum formed here, not sunk below
        __builtin_amdgcn_sched_barrier(0);
        // blocks 2, 3: probabilities (in place) and codes, one matrix instruction per half block
#pragma unroll
        for (int kb4 = 2; kb4 < 4; ++kb4)
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
            for (int w4 = 2 * hb; w4 < 2 * hb + 2; ++w4) {
#pragma unroll
              for (int e = 0; e < 4; ++e) s[kb4][4 * w4 + e] = __builtin_amdgcn_exp2f(fmaf(s[kb4][4 * w4 + e], c, bias));
              pop[1][4 * (kb4 - 2) + w4] =
                  pcode(s[kb4][4 * w4], s[kb4][4 * w4 + 1], s[kb4][4 * w4 + 2], s[kb4][4 * w4 + 3], kb4, w4);
            }
            // first half, instructions 0 .. NDB - 1, spread over the four half blocks
            const int j = 2 * (kb4 - 2) + hb;
            if ((j + 1) * NDB / 4 > j * NDB / 4) pv_step(j * NDB / 4);
            __builtin_amdgcn_sched_barrier(0);
          }
        // second half's instructions between the remaining row-sum additions
#pragma unroll
        for (int k = NDB; k < NPV; ++k) {
          pv_step(k);
#pragma unroll
          for (int j = 0; j < 8 / NDB; ++j) {
            const int w = (k - NDB) * (8 / NDB) + j;  // word 0..7 of blocks 2, 3
            const int kb4 = 2 + w / 4, w4 = w % 4;
            l += (s[kb4][4 * w4] + s[kb4][4 * w4 + 1]) + (s[kb4][4 * w4 + 2] + s[kb4][4 * w4 + 3]);
          }
          asm volatile("" : "+v"(l));
          __builtin_amdgcn_sched_barrier(0);
        }
#ifdef FLAMIA_DEBUG_DUMP
        if (row_valid && (p.dbg.fwd_p || p.dbg.fwd_m)) {  // test builds: codes and the running max
#pragma unroll
          for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key_rel = KV_TILE * kappa + 32 * kb4 + acc_row(i, hh);
              const int64_t x = key_rel < L ? dbg_index(p.dbg, h, doc_start + q_rel, doc_start + key_rel) : -1;
              if (x < 0) continue;
              const int word = pop[kb4 >> 1][4 * (kb4 & 1) + i / 4];
              if (p.dbg.fwd_p) p.dbg.fwd_p[x] = (uint8_t)(word >> (8 * (i % 4)));
              if (p.dbg.fwd_m) p.dbg.fwd_m[x] = m_new;
              if (QK4 && p.dbg.fwd_ps) p.dbg.fwd_ps[x] = (uint8_t)pe[kb4];
            }
        }
#endif
      }
      if (kappa > 0) {
        __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
        if constexpr (QK4) store_scales4<D>(sm, kb ^ 1, kb ^ 1, scn);
        else store_scales<D>(sm, kb ^ 1, kb ^ 1, scn);
        lds_barrier();
      }
    }

    // ---- epilogue: O = acc / l, LSE = m + log2 l (l in units of 2^-8; QK4: of 1)
    constexpr int L_SHIFT = QK4 ? 0 : P_SHIFT;
    if (wave_active) {
      const float lt = halves_sum(l);
      if (row_valid) {
        const float inv = (float)(1 << L_SHIFT) / lt;
        uint16_t* orow = p.o + (int64_t)(doc_start + q_rel) * p.ost + (int64_t)h * p.osh;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int d0 = 32 * db + 8 * j + 4 * hh;
            uint2 w;
            w.x = pack_bf16(oacc[db][4 * j + 0] * inv, oacc[db][4 * j + 1] * inv);
            w.y = pack_bf16(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
            *reinterpret_cast<uint2*>(orow + d0) = w;
          }
        if (hh == 0) p.lse[(int64_t)h * p.T + doc_start + q_rel] = m + __builtin_amdgcn_logf(lt) - (float)L_SHIFT;
      }
    }
  }
  // dynamic lists: every workgroup has taken its last unit (its counter value came back before
  // this add), so the last one to get here clears the counters for the next call on the list
  if (dyn && tid == 0 && atomicAdd(&ctr[1], 1) == G - 1) {
    atomicExch(&ctr[0], 0);
    atomicExch(&ctr[1], 0);
  }

  // ---- rows outside every document: O = 0, LSE = +inf
  const int c_lo = p.n_docs > 0 ? p.cu[0] : p.T;
  const int c_hi = p.n_docs > 0 ? p.cu[p.n_docs] : p.T;
  const int per = (p.T + G - 1) / G;
  const int t0 = wg * per, t1 = min(t0 + per, p.T);
  for (int t = t0; t < t1; ++t) {
    if (t >= c_lo && t < c_hi) continue;
    for (int x = tid; x < p.Hq * D; x += FWD_THREADS) {
      const int hh2 = x / D, dd = x % D;
      p.o[(int64_t)t * p.ost + (int64_t)hh2 * p.osh + dd] = 0;
    }
    for (int x = tid; x < p.Hq; x += FWD_THREADS) p.lse[(int64_t)x * p.T + t] = __builtin_inff();
  }
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int d, int grid, hipStream_t s) {
  // documents of fewer than 4096 tokens on average: 128-query units, two workgroups per CU
  const bool short_docs = (int64_t)p.n_docs * 4096 > (int64_t)p.T;
  auto go = [&](auto c, auto pr, auto f4) {
    constexpr bool C = decltype(c)::value, PR = decltype(pr)::value, F4 = decltype(f4)::value;
    if (short_docs) {
      if (d == 128) hipLaunchKernelGGL((fwd_kernel<128, 4, C, PR, F4>), dim3(2 * grid), dim3(fwd_threads<4>()), 0, s, p);
      else hipLaunchKernelGGL((fwd_kernel<64, 4, C, PR, F4>), dim3(2 * grid), dim3(fwd_threads<4>()), 0, s, p);
    } else {
      if (d == 128) hipLaunchKernelGGL((fwd_kernel<128, 8, C, PR, F4>), dim3(grid), dim3(fwd_threads<8>()), 0, s, p);
      else hipLaunchKernelGGL((fwd_kernel<64, 8, C, PR, F4>), dim3(grid), dim3(fwd_threads<8>()), 0, s, p);
    }
  };
  const std::true_type y{};
  const std::false_type n{};
  if (p.precise) go(y, y, n);  // causal only (checked by the caller)
  else if (p.q4) {
    if (p.causal) go(y, n, y);
    else go(n, n, y);
  } else if (p.causal) go(y, n, n);
  else go(n, n, n);
  const hipError_t e = hipGetLastError();
  return (e == hipSuccess && p.small) ? launch_small_fwd(p, d, s) : e;
}

}  // namespace flamia
