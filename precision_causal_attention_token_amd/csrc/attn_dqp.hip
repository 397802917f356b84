// dQ under the precision options: query-stationary recomputation with query-row-wise dS
// exponents (jaehun.me review §3.2 "dQ prescale" and the precision options listed there:
// per-token operand scales, each product's other operand's exponent folded into the quantised
// gradient operand; §3.3 recomputation from the same quantised operands).
//
// With per-token scales, dQ_i = softmax_scale sum_j dS_ij K_j contracts over keys, so K's
// exponent moves into the dS operand: dS'_ij = dS_ij 2^e(K_j), quantised to E4M3 with one
// round-up E8M0 exponent per (query row, 32-key block).  No other row enters a row's rounding,
// and no later key enters any row's values (causal), so dQ_i depends on tokens up to i alone.
// K then enters the product with its bare codes.  The dQ prescale 2^pi_i (pi from the prefix
// maxima of the V and K exponents up to row i) and the FP16 accumulation of the key tiles'
// partials in ascending tile order are those of the key-stationary backward.
//
// Persistent grid, two 256-thread workgroups per compute unit.  A work unit is (half of a
// forward item = 128 queries of a document, query head); wave w owns queries 32w..32w+31, its Q
// and dO rows held in registers as MFMA operands.  Per 128-key tile kappa = 0, 1, ... up to the
// wave's diagonal tile, visited in ascending order:
//   S^T = K Q^T and dP^T = V dO^T       (A = K / V rows from LDS, B = Q / dO in registers; the
//                                        score is bit-identical to the forward's)
//   P = 2^(c S - LSE), dS' = P (dP - D) 2^e(K_j), per (query, 32-key block) exponents and codes
//                                       (already in operand order, as the forward's P)
//   partial^T = K^T dS'^T               (A = K^T from transpose reads of the same K tile)
//   acc16 = FP16(acc16 + FP16(2^pi partial))
// and dQ = BF16(softmax_scale 2^-pi acc16) at the end.  K and V tiles arrive by direct
// global-to-LDS loads one tile ahead (two buffers).
#include "device_common.h"
#include "kernels.h"

namespace flamia {

namespace {

constexpr int DQP_WAVES = 4;
constexpr int DQP_THREADS = 64 * DQP_WAVES;
constexpr int DQP_QU = 32 * DQP_WAVES;  // queries per unit

template <int D>
struct DqpSmem {
  uint8_t k[2][KV_TILE * D];
  uint8_t v[2][KV_TILE * D];
  uint8_t sk[2][KV_TILE];
  uint8_t sv[2][KV_TILE];
  alignas(16) int ek[2][KV_TILE];  // e(K_j) = scale byte - 127, the fold's exponent
};

// Key tile kappa's K and V rows into buffer b, global -> LDS with direct loads; each lane
// fetches the 16-byte chunk that belongs at its LDS position under the tile's swizzle.  Rows
// past the document end repeat its last row, and 1 KiB blocks wholly past it are zero-filled:
// those keys are masked (their dS' is zero), and both K and V only need to be finite there.
// Returns the scale byte thread t < 128 holds for key t's K, 128 <= t < 256 for key t - 128's V.
template <int D>
__device__ __forceinline__ uint32_t dqp_issue_tile(const BwdParams& p, DqpSmem<D>& sm, int b, int g, int doc_start,
                                                   int L, int kappa, int wave, int lane) {
  constexpr int CPR = D / 16;
  constexpr int BLOCKS = KV_TILE * D / 1024;
  constexpr int PER_WAVE = 2 * BLOCKS / DQP_WAVES;
  static_assert(PER_WAVE * DQP_WAVES == 2 * BLOCKS, "blocks split evenly over the waves");
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int wb = wave * PER_WAVE + i;  // K blocks, then V blocks
    const bool is_v = wb >= BLOCKS;
    const int blk = is_v ? wb - BLOCKS : wb;
    const int pos = blk * 64 + lane;
    const int row = pos / CPR, pc = pos % CPR;
    const int lc = pc ^ lds_swizzle<D>(row);
    uint8_t* dst = (is_v ? sm.v[b] : sm.k[b]) + blk * 1024;
    if (KV_TILE * kappa + blk * (1024 / D) < L) {
      const int key = min(KV_TILE * kappa + row, L - 1);
      const uint8_t* src = (is_v ? p.v : p.k) + ((int64_t)(doc_start + key) * p.Hkv + g) * D + 16 * lc;
      dma_load16(src, lds_addr(dst));
    } else {
      *reinterpret_cast<uint4*>(dst + 16 * lane) = make_uint4(0, 0, 0, 0);
    }
  }
  const int tid = threadIdx.x;
  uint32_t sc = 127;
  const int key = KV_TILE * kappa + (tid & (KV_TILE - 1));
  if (key < L) sc = (tid < KV_TILE ? p.sk : p.sv)[(int64_t)g * p.T + doc_start + key];
  return sc;
}

template <int D>
__device__ __forceinline__ void dqp_store_scales(DqpSmem<D>& sm, int b, uint32_t sc) {
  const int tid = threadIdx.x;
  if (tid < KV_TILE) {
    sm.sk[b][tid] = (uint8_t)sc;
    sm.ek[b][tid] = (int)sc - 127;
  } else {
    sm.sv[b][tid - KV_TILE] = (uint8_t)sc;
  }
}

template <int D>
__global__ __launch_bounds__(DQP_THREADS, 2) void dqp_kernel(BwdParams p) {
  constexpr int NC = D / 64;
  constexpr int NDB = D / 32;
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  static_assert(DQP_THREADS == 2 * KV_TILE, "one scale byte per thread");
  __shared__ DqpSmem<D> sm;

  if (p.status[0]) return;  // cu_seqlens did not fit the sizes the host gave
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int n_items = p.fwd_list[0];
  const int4* items = reinterpret_cast<const int4*>(p.fwd_list + 4);
  constexpr int PARTS = ITEM_Q / DQP_QU;
  const int grp = p.Hq / p.Hkv;
  const UnitPartition up = unit_partition(p.Hkv);  // as in the key-tile pass
  const int hq_per = up.kv_per * grp;
  const int n_units = n_items * PARTS * hq_per;
  const float c = p.c;
  const int T = p.T;

  __shared__ int unit_slot;
  int32_t* const counter = p.counters + 8 + up.part;  // the dQ counters of the one chunk
  for (int u = up.rank; u < n_units; u = next_unit(counter, &unit_slot, up.first)) {
    const int4 it = items[u / (PARTS * hq_per)];
    const int j = u % hq_per;
    const int g = partition_kv(up, j / grp), h = g * grp + j % grp, part = (u / hq_per) % PARTS;
    const int doc_start = p.cu[it.x];
    const int L = p.cu[it.x + 1] - doc_start;
    const int q0 = ITEM_Q * it.y + DQP_QU * part;
    if (q0 >= L) continue;  // the item ends before this part (uniform over the workgroup)
    const int q_wave = q0 + 32 * wave;
    const bool wave_active = q_wave < L;
    const int q_rel = q_wave + n;
    const bool row_valid = q_rel < L;
    const int kd = q_wave / KV_TILE;                  // the wave's diagonal (last) key tile
    const int kappa_hi = (min(q0 + DQP_QU, L) - 1) / KV_TILE;

    // Q and dO operands (B of S^T and dP^T): lane (n, hh) holds d = 64 cc + 32 hh .. + 31 of
    // query n; rows past the document end are zero with LSE = +inf (P = 0)
    v8i qop[NC], dop[NC];
    int q_scale = 127, do_scale = 127, pi = 0;
    float lse = __builtin_inff(), dd = 0.f;
    {
      const int64_t ra = ((int64_t)(doc_start + q_rel) * p.Hq + h) * D;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        uint4 a = make_uint4(0, 0, 0, 0), bq = a, e = a, f = a;
        if (row_valid) {
          const uint4* sq = reinterpret_cast<const uint4*>(p.q + ra + 64 * cc + 32 * hh);
          const uint4* sd = reinterpret_cast<const uint4*>(p.dO + ra + 64 * cc + 32 * hh);
          a = sq[0]; bq = sq[1]; e = sd[0]; f = sd[1];
        }
        qop[cc] = v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)bq.x, (int)bq.y, (int)bq.z, (int)bq.w};
        dop[cc] = v8i{(int)e.x, (int)e.y, (int)e.z, (int)e.w, (int)f.x, (int)f.y, (int)f.z, (int)f.w};
      }
      if (row_valid) {
        const int64_t ti = (int64_t)h * T + doc_start + q_rel;
        q_scale = p.sq[ti];
        do_scale = p.sdo[ti];
        lse = p.lse[ti];
        dd = p.Dv[ti];
        pi = p.pi[ti];
      }
    }
    const float up = exp2i(pi);
    h2 acc16[NDB][8];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc16[db][j] = h2{0, 0};

    lds_barrier();  // the previous unit's readers are done with every buffer
    {
      const uint32_t sc = dqp_issue_tile<D>(p, sm, 0, g, doc_start, L, 0, wave, lane);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
      dqp_store_scales<D>(sm, 0, sc);
    }
    lds_barrier();
    for (int kappa = 0; kappa <= kappa_hi; ++kappa) {
      const int b = kappa & 1;
      uint32_t scn = 127;
      if (kappa < kappa_hi) scn = dqp_issue_tile<D>(p, sm, b ^ 1, g, doc_start, L, kappa + 1, wave, lane);
      if (wave_active && kappa <= kd) {
        const uint8_t* kt = sm.k[b];
        const uint8_t* vt = sm.v[b];
        v8i dsop[2];  // dS' codes of keys 64 ci .. 64 ci + 63 in operand order
        int srb[2];   // the lane's scale byte for them: its K half's 32-key block
#pragma unroll
        for (int ci = 0; ci < 2; ++ci) {
          v16f s[2], dp[2];
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) {
            const int kb4 = 2 * ci + bb;
            const int ks = sm.sk[b][32 * kb4 + n], vs = sm.sv[b][32 * kb4 + n];
#pragma unroll
            for (int cc = 0; cc < NC; ++cc) {
              const v8i kr = lds_read_row32<D>(kt, 32 * kb4 + n, 64 * cc + 32 * hh);
              s[bb] = mfma_scaled(kr, qop[cc], cc ? s[bb] : v16f{}, ks, q_scale);
              const v8i vr = lds_read_row32<D>(vt, 32 * kb4 + n, 64 * cc + 32 * hh);
              dp[bb] = mfma_scaled(vr, dop[cc], cc ? dp[bb] : v16f{}, vs, do_scale);
            }
            mfma_drain(s[bb]);
            mfma_drain(dp[bb]);
          }
          if (kappa == kd) {
            // causal mask on the diagonal tile: key 128 kappa + 32 kb4 + acc_row(i, hh) after the
            // query (keys past the document end lie after every query of it)
            int lim = q_rel - KV_TILE * kappa - 4 * hh;
            asm volatile("" : "+v"(lim));
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
              for (int i = 0; i < 16; ++i)
                if (32 * (2 * ci + bb) + acc_row(i, 0) > lim) s[bb][i] = -__builtin_inff();
          }
#ifdef FLAMIA_DEBUG_DUMP
          if (row_valid && (p.dbg.dq_s || p.dbg.dq_dp)) {  // test builds: S (masked) and dP - D
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int key_rel = KV_TILE * kappa + 32 * (2 * ci + bb) + acc_row(i, hh);
                const int64_t x = key_rel < L ? dbg_index(p.dbg, h, doc_start + q_rel, doc_start + key_rel) : -1;
                if (x < 0) continue;
                if (p.dbg.dq_s) p.dbg.dq_s[x] = s[bb][i];
                if (p.dbg.dq_dp) p.dbg.dq_dp[x] = dp[bb][i] - dd;
              }
          }
#endif
          int sr[2];
#pragma unroll
          for (int bb = 0; bb < 2; ++bb) {
            const int kb4 = 2 * ci + bb;
            float rmax = 0.f;
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4) {
              // e(K_j) of keys 32 kb4 + 8 w4 + 4 hh + e
              const int4 ek = *reinterpret_cast<const int4*>(&sm.ek[b][32 * kb4 + 8 * w4 + 4 * hh]);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int i = 4 * w4 + e;
                const float pv = __builtin_amdgcn_exp2f(fmaf(s[bb][i], c, -lse));
                const float ds = pv * (dp[bb][i] - dd);  // dS = P (dP - D)
                const float dsk = __builtin_ldexpf(ds, e == 0 ? ek.x : e == 1 ? ek.y : e == 2 ? ek.z : ek.w);
                s[bb][i] = dsk;
                rmax = fmaxf(rmax, fabsf(dsk));
              }
            }
            // the row's exponent for this 32-key block: both lane halves hold 16 keys each
            sr[bb] = (int)e8m0_byte_nonneg(halves_max(rmax));
#pragma unroll
            for (int w4 = 0; w4 < 4; ++w4)
              dsop[ci][4 * bb + w4] =
                  pack4_fp8_scaled(s[bb][4 * w4], s[bb][4 * w4 + 1], s[bb][4 * w4 + 2], s[bb][4 * w4 + 3], sr[bb]);
#ifdef FLAMIA_DEBUG_DUMP
            if (row_valid && p.dbg.dq_ds) {  // test builds: dS' codes and the row's block exponent
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int key_rel = KV_TILE * kappa + 32 * kb4 + acc_row(i, hh);
                const int64_t x = key_rel < L ? dbg_index(p.dbg, h, doc_start + q_rel, doc_start + key_rel) : -1;
                if (x < 0) continue;
                p.dbg.dq_ds[x] = (uint8_t)(dsop[ci][4 * bb + i / 4] >> (8 * (i % 4)));
                p.dbg.dq_dss[x] = (uint8_t)sr[bb];
              }
            }
#endif
          }
          srb[ci] = hh ? sr[1] : sr[0];
        }
        // partial^T = K^T dS'^T (K with its bare codes), then the FP16 sums
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          v16f part = v16f{};
#pragma unroll
          for (int ci = 0; ci < 2; ++ci)
            part = mfma_scaled(lds_read_tr32<D>(kt, 64 * ci, 32 * db, lane), dsop[ci], part, 127, srb[ci]);
          mfma_drain(part);
#ifdef FLAMIA_DEBUG_DUMP
          if (p.dbg.dq_part && row_valid) {  // test builds: the partial times 2^pi, as converted to FP16
            const int64_t x = dbg_row(p.dbg, h, doc_start + q_rel);
            if (x >= 0 && kappa < p.dbg.n_tiles)
#pragma unroll
              for (int i = 0; i < 16; ++i)
                p.dbg.dq_part[(x * p.dbg.n_tiles + kappa) * D + 32 * db + acc_row(i, hh)] = part[i] * up;
          }
#endif
#pragma unroll
          for (int j = 0; j < 8; ++j)
            acc16[db][j] = acc16[db][j] + h2{(_Float16)(part[2 * j] * up), (_Float16)(part[2 * j + 1] * up)};
        }
      }
      if (kappa < kappa_hi) {
        __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
        dqp_store_scales<D>(sm, b ^ 1, scn);
      }
      lds_barrier();
    }

    if (row_valid) {
      const float down = exp2i(-pi) * p.softmax_scale;
      uint16_t* const row = p.dq + (int64_t)(doc_start + q_rel) * p.dqst + (int64_t)h * p.dqsh;
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
    }
  }
}

}  // namespace

hipError_t launch_dq_precise(const BwdParams& p, int d, int grid, hipStream_t s) {
  if (d == 128) hipLaunchKernelGGL(dqp_kernel<128>, dim3(2 * grid), dim3(DQP_THREADS), 0, s, p);
  else hipLaunchKernelGGL(dqp_kernel<64>, dim3(2 * grid), dim3(DQP_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace flamia
