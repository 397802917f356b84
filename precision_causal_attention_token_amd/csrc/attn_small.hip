// Small-document pass: forward and backward of documents of 1 .. SMALL_DOC (8) tokens on the
// default 8-bit path (jaehun.me review §3.4 "Packed documents": the quantiser's statistics stay
// inside a document, so every operand of such a document is one token block with one exponent;
// §3.3 recomputation with the same quantised operands and block-scaled dS).
//
// The tile kernels give every document at least one 128-key tile unit per head, whose fixed
// work (a mostly empty tile, barriers, dependent loads) dominates for documents this short:
// 131072 one-token documents are 131072 units per head.  Here one wave takes the documents
// that start in a window of 56 tokens; its 64 lanes are the tokens w0 .. w0 + 63, which hold
// every token of those documents.  Lane i is query i (scores, softmax, O, dQ) and key i
// (dK, dV) of its own document.  The products run on the vector unit in FP32 from the codes and
// exponents (products of two E4M3 values are exact; sums run in ascending d or token order);
// every E4M3 decision uses the conversions, exponent rule and score formula of the tile kernels:
//   forward:  t_ij = Q_i . K_j, m = c max_j t_ij, p = 2^fma(t, c, 8 - m), l = sum_j p,
//             Phat = E4M3(p) (operand scale 2^-8), O = (sum_j Phat V_j) 2^-8 (2^8 / l),
//             LSE = m + log2 l - 8;
//   backward: P = 2^fma(t, c, -LSE), D - dP, dS = P (dP - D); the document's 32 x 32 block (its
//             only one) takes the round-up E8M0 exponents of max P and max |dS|; dQ = dShat K
//             (a single key tile: FP16(2^pi partial), then 2^-pi softmax_scale), dK =
//             softmax_scale sum dShat^T Q and dV = sum Phat^T dO over the group's query heads.
// Keys after the query are masked (causal), or every key of the document is visible.
#include <climits>

#include "device_common.h"
#include "kernels.h"

namespace flamia {

namespace {

constexpr int NL = 64;              // lanes: tokens w0 .. w0 + 63
constexpr int SW = NL - SMALL_DOC;  // window of document starts per unit: such a document ends by w0 + 63
constexpr int HEADS_PER_WAVE = 4;  // heads of one window per wave: query heads forward, KV heads backward

// Documents of 1 .. SMALL_DOC tokens in a work list (counter word 2, written by the list build).
__device__ __forceinline__ int small_docs_of(const int32_t* list, int T) {
  return list[worklist_ctr_offset(list[2], T) / 4 + 2];
}

// First k in [0, n) with cu[k] > x (n if none), searched by the 64 lanes together: each round
// probes the last entry of 64 equal pieces and keeps the piece where the comparison turns.
__device__ __forceinline__ int wave_upper(const int32_t* __restrict__ cu, int n, int x, int lane) {
  int lo = 0, hi = n;  // the answer lies in [lo, hi]
  while (hi - lo > NL) {
    const int step = (hi - lo + NL - 1) / NL;
    const int pos = lo + (lane + 1) * step - 1;
    const uint64_t m = __ballot(pos >= hi || cu[pos] > x);
    if (m == 0) return hi;
    const int f = __ffsll((unsigned long long)m) - 1;
    const int nlo = lo + f * step;
    hi = min(lo + (f + 1) * step - 1, hi);
    lo = nlo;
  }
  const int pos = lo + lane;
  const uint64_t m = __ballot(pos >= hi || cu[pos] > x);
  return m == 0 ? hi : min(lo + __ffsll((unsigned long long)m) - 1, hi);
}

// The lane's token w0 + lane and its document [a, b): true when that document has 1 .. SMALL_DOC
// tokens and starts in the window [w0, w0 + SW).  Called by the whole wave: the documents around
// the window are found once (entries cu[u - 1 ..] in cw, u the first entry past w0), then each
// lane looks its token up there; a lane whose token lies more than 63 entries on (empty
// documents) searches the whole table.
__device__ __forceinline__ bool window_docs(const int32_t* __restrict__ cu, int n_docs, int w0, int lane, int* cw,
                                            int& a, int& b) {
  a = b = 0;
  if (n_docs <= 0) return false;
  const int u = wave_upper(cu, n_docs + 1, w0, lane);  // cu[u - 1] <= w0 < cu[u]
  const int e = u - 1 + lane;
  cw[lane] = e < 0 ? INT_MIN : (e <= n_docs ? cu[e] : INT_MAX);
  __syncthreads();
  const int t = w0 + lane;
  int k;
  if (cw[NL - 1] > t) {
    int lo = 0, hi = NL - 1;  // first idx with cw[idx] > t (cw[0] <= t)
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (cw[mid] > t) hi = mid;
      else lo = mid + 1;
    }
    k = u - 1 + lo - 1;
  } else {
    int lo = 0, hi = n_docs + 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (cu[mid] <= t) lo = mid + 1;
      else hi = mid;
    }
    k = lo - 1;
  }
  if (k < 0 || k >= n_docs) return false;
  a = cu[k];
  b = cu[k + 1];
  return a >= w0 && a < w0 + SW && b - a <= SMALL_DOC && t < b;
}

// Rows of tokens w0 .. w0 + 63 (those before T) of one head of a [T, H, D] code tensor into LDS
// (row stride D + 16 bytes), and their exponent bytes from [H, T].
template <int D>
__device__ __forceinline__ void stage_rows(const uint8_t* __restrict__ x, const uint8_t* __restrict__ sx, int H,
                                           int h, int T, int w0, int lane, uint8_t* rows, uint8_t* sc) {
  const int t = w0 + lane;
  if (t < T) {
    const uint4* src = reinterpret_cast<const uint4*>(x + ((int64_t)t * H + h) * D);
    uint4 v[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) v[c] = src[c];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) reinterpret_cast<uint4*>(rows + lane * (D + 16))[c] = v[c];
    sc[lane] = sx[(int64_t)h * T + t];
  }
}

// E4M3 code (round to nearest even) of x, and of x / scale with scale 2^(byte - 127).
__device__ __forceinline__ uint32_t fp8_code(float x) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false) & 0xFFu;
}
__device__ __forceinline__ uint32_t fp8_code_scaled(float x, float scale) {
  typedef short v2s __attribute__((ext_vector_type(2)));
  const v2s r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, x, 0.f, scale, false);
  return (uint32_t)(uint16_t)r[0] & 0xFFu;
}
__device__ __forceinline__ float fp8_value(uint32_t code) { return __builtin_amdgcn_cvt_pk_f32_fp8((int)code, false)[0]; }

// Sum over d ascending of dec(x_d) dec(y_d) for two rows of D E4M3 codes (x in registers, y
// read from memory), started at acc.
template <int D>
__device__ __forceinline__ float dot_codes(const uint32_t (&x)[D / 4], const uint8_t* __restrict__ y, float acc) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const uint4 v = reinterpret_cast<const uint4*>(y)[c];
    const uint32_t yw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // converted here, in every call: hoisted out of the callers' key loops, the floats of a
      // whole row would take D registers
      int xe = (int)x[4 * c + e];
      asm volatile("" : "+v"(xe));
      const auto x01 = __builtin_amdgcn_cvt_pk_f32_fp8(xe, false);
      const auto x23 = __builtin_amdgcn_cvt_pk_f32_fp8(xe, true);
      const auto y01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)yw[e], false);
      const auto y23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)yw[e], true);
      acc = fmaf(x01[0], y01[0], acc);
      acc = fmaf(x01[1], y01[1], acc);
      acc = fmaf(x23[0], y23[0], acc);
      acc = fmaf(x23[1], y23[1], acc);
    }
  }
  return acc;
}

template <int D>
__device__ __forceinline__ void load_row(uint32_t (&x)[D / 4], const uint8_t* __restrict__ src) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const uint4 v = reinterpret_cast<const uint4*>(src)[c];
    x[4 * c] = v.x; x[4 * c + 1] = v.y; x[4 * c + 2] = v.z; x[4 * c + 3] = v.w;
  }
}

// acc[0..N-1] += f dec(y_0..N-1): N codes of a row chunk (N a multiple of 16)
template <int N>
__device__ __forceinline__ void axpy_codes(float* acc, float f, const uint8_t* __restrict__ y) {
#pragma unroll
  for (int c = 0; c < N / 16; ++c) {
    const uint4 v = reinterpret_cast<const uint4*>(y)[c];
    const uint32_t yw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto y01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)yw[e], false);
      const auto y23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)yw[e], true);
      const int d = 16 * c + 4 * e;
      acc[d] = fmaf(f, y01[0], acc[d]);
      acc[d + 1] = fmaf(f, y01[1], acc[d + 1]);
      acc[d + 2] = fmaf(f, y23[0], acc[d + 2]);
      acc[d + 3] = fmaf(f, y23[1], acc[d + 3]);
    }
  }
}
__device__ __forceinline__ void axpy32(float (&acc)[32], float f, const uint8_t* __restrict__ y) { axpy_codes<32>(acc, f, y); }

// 32 BF16 values (x[d] * s) to dst (64 bytes, 16-byte aligned rows)
__device__ __forceinline__ void store_bf16x32(uint16_t* dst, const float* x, float s) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 w;
    w.x = pack_bf16(x[8 * c] * s, x[8 * c + 1] * s);
    w.y = pack_bf16(x[8 * c + 2] * s, x[8 * c + 3] * s);
    w.z = pack_bf16(x[8 * c + 4] * s, x[8 * c + 5] * s);
    w.w = pack_bf16(x[8 * c + 6] * s, x[8 * c + 7] * s);
    *reinterpret_cast<uint2*>(dst + 8 * c) = make_uint2(w.x, w.y);
    *reinterpret_cast<uint2*>(dst + 8 * c + 4) = make_uint2(w.z, w.w);
  }
}

// ---- forward: one wave per (window, four query heads)
template <int D>
__global__ __launch_bounds__(NL) void small_fwd_kernel(FwdParams p) {
  constexpr int RS = D + 16;  // LDS row stride
  __shared__ __align__(16) uint8_t kr[NL * RS], vr[NL * RS];  // K, V rows of the window's tokens
  __shared__ uint8_t ks[NL], vs[NL];
  __shared__ int cw[NL];
  __shared__ float s_row[NL][SMALL_DOC + 1];   // the lane's scores (row i, key a + jo)
  __shared__ uint8_t p_row[NL][SMALL_DOC + 4];  // its probability codes
  if (small_docs_of(p.list, p.T) == 0) return;  // uniform: the list has no short documents
  const int lane = threadIdx.x, w0 = SW * (int)blockIdx.x;
  int a, b;
  const bool own = window_docs(p.cu, p.n_docs, w0, lane, cw, a, b);
  if (!__any(own)) return;  // uniform
  const int i = w0 + lane, L = b - a;
  const int key_end = p.causal ? i + 1 : b;  // visible keys a .. key_end - 1
  const float c = p.c;
  const int grp = p.Hq / p.Hkv;
  const int h0 = HEADS_PER_WAVE * (int)blockIdx.y, h_end = min(p.Hq, h0 + HEADS_PER_WAVE);
  int g_rows = -1;
#pragma unroll 1
  for (int h = h0; h < h_end; ++h) {
    const int g = h / grp;
    if (g != g_rows) {  // uniform: the KV head's rows into LDS
      __syncthreads();
      stage_rows<D>(p.k, p.sk, p.Hkv, g, p.T, w0, lane, kr, ks);
      stage_rows<D>(p.v, p.sv, p.Hkv, g, p.T, w0, lane, vr, vs);
      __syncthreads();
      g_rows = g;
    }
    if (!own) continue;
    uint32_t qw[D / 4];
    load_row<D>(qw, p.q + ((int64_t)i * p.Hq + h) * D);
    const int eq = p.sq[(int64_t)h * p.T + i];
    float mx = -__builtin_inff();
#pragma unroll 1
    for (int jo = 0; jo < L; ++jo) {
      const int j = a + jo;
      float s = -__builtin_inff();
      if (j < key_end) {
        const float acc = dot_codes<D>(qw, kr + (j - w0) * RS, 0.f);
        s = __builtin_ldexpf(acc, eq + (int)ks[j - w0] - 254);
      }
      s_row[lane][jo] = s;
      mx = fmaxf(mx, s);
    }
    const float m = mx * c;
    const float bias = (float)P_SHIFT - m;
    float l = 0.f;
#pragma unroll 1
    for (int jo = 0; jo < L; ++jo) {
      const float s = s_row[lane][jo];
      const float pv = __builtin_amdgcn_exp2f(fmaf(s, c, bias));
      l += pv;
      const uint32_t code = fp8_code(pv);
      p_row[lane][jo] = (uint8_t)code;
#ifdef FLAMIA_DEBUG_DUMP
      const int64_t x = dbg_index(p.dbg, h, i, a + jo);
      if (x >= 0) {
        if (p.dbg.fwd_s) p.dbg.fwd_s[x] = s;
        if (p.dbg.fwd_m) p.dbg.fwd_m[x] = m;
        if (p.dbg.fwd_p) p.dbg.fwd_p[x] = (uint8_t)code;
      }
#endif
    }
    const float inv = (float)(1 << P_SHIFT) / l;
    uint16_t* orow = p.o + (int64_t)i * p.ost + (int64_t)h * p.osh;
#pragma unroll 1
    for (int c0 = 0; c0 < D; c0 += 32) {
      float acc[32];
#pragma unroll
      for (int d = 0; d < 32; ++d) acc[d] = 0.f;
#pragma unroll 1
      for (int j = a; j < key_end; ++j) {
        const float f = __builtin_ldexpf(fp8_value(p_row[lane][j - a]), (int)vs[j - w0] - 127 - P_SHIFT);
        axpy32(acc, f, vr + (j - w0) * RS + c0);
      }
      store_bf16x32(orow + c0, acc, inv);
    }
    p.lse[(int64_t)h * p.T + i] = m + __builtin_amdgcn_logf(l) - (float)P_SHIFT;
  }
}

// ---- backward: one wave per (window, four KV heads); for each KV head and each 64 columns of
// the gradients, over the group's query heads (every column pass forms the same P, dS and codes,
// since the scores need all of d, and writes its own columns of dQ, dK and dV: all 128 columns in
// registers at once would spill)
template <int D>
__global__ __launch_bounds__(NL) void small_bwd_kernel(BwdParams p) {
  constexpr int RS = D + 16;  // LDS row stride of K, V
  constexpr int DC = 64;      // gradient columns per wave
  constexpr int RC = DC + 16; // LDS row stride of the Q, dO columns
  __shared__ __align__(16) uint8_t kr[NL * RS], vr[NL * RS];
  __shared__ uint8_t ks[NL], vs[NL], qs[NL], dos[NL];
  __shared__ int cw[NL];
  __shared__ float rmax_p[NL], rmax_d[NL];
  __shared__ uint8_t cp[NL][SMALL_DOC], cd[NL][SMALL_DOC];  // Phat, dShat codes of the current head
  // P and dS of (row lane, key a + jo) until the block exponents are known, then the rows' Q and
  // dO codes
  __shared__ __align__(16) union {
    struct { float pv[NL][SMALL_DOC + 1], ds[NL][SMALL_DOC + 1]; } f;
    struct { uint8_t q[NL * RC], dO[NL * RC]; } r;
  } u;
  // uniform exits: the prologue found cu_seqlens that do not fit, or the list has no short
  // documents (the call's waves then end after one load)
  if (p.status[0] || small_docs_of(p.list, p.T) == 0) return;
  const int lane = threadIdx.x, w0 = SW * (int)blockIdx.x;
  int a, b;
  const bool own = window_docs(p.cu, p.n_docs, w0, lane, cw, a, b);
  if (!__any(own)) return;  // uniform: no barrier is left waiting
  const int t = w0 + lane, L = b - a;
  const float c = p.c, ss = p.softmax_scale;
  const int grp = p.Hq / p.Hkv;
  const int g_end = min(p.Hkv, HEADS_PER_WAVE * ((int)blockIdx.y + 1));
#pragma unroll 1
  for (int g = HEADS_PER_WAVE * (int)blockIdx.y; g < g_end; ++g) {
  __syncthreads();  // the previous KV head's readers are done with the rows
  stage_rows<D>(p.k, p.sk, p.Hkv, g, p.T, w0, lane, kr, ks);
  stage_rows<D>(p.v, p.sv, p.Hkv, g, p.T, w0, lane, vr, vs);
  __syncthreads();
#pragma unroll 1
  for (int d0 = 0; d0 < D; d0 += DC) {
  const bool dump = d0 == 0;  // test builds: one column pass dumps the decisions

  float ak[DC], av[DC];  // dK, dV of key t, these columns, summed over the group's heads
#pragma unroll
  for (int d = 0; d < DC; ++d) { ak[d] = 0.f; av[d] = 0.f; }
  uint32_t sp = 0, sd = 0;  // the document's block exponent bytes, current head

#pragma unroll 1
  for (int hi = 0; hi < grp; ++hi) {
    const int h = g * grp + hi;
    float pmax = 0.f, dmax = 0.f;
    if (own) {
      // row i = t: P, D - dP and dS against every key of the document (masked ones give P = 0)
      const int i = t;
      const int key_end = p.causal_mask ? i + 1 : b;
      uint32_t qw[D / 4], ow[D / 4];
      load_row<D>(qw, p.q + ((int64_t)i * p.Hq + h) * D);
      load_row<D>(ow, p.dO + ((int64_t)i * p.Hq + h) * D);
      const int eq = p.sq[(int64_t)h * p.T + i], edo = p.sdo[(int64_t)h * p.T + i];
      const float lse = p.lse[(int64_t)h * p.T + i], Di = p.Dv[(int64_t)h * p.T + i];
#pragma unroll 1
    for (int jo = 0; jo < L; ++jo) {
        const int j = a + jo, r = j - w0;
        const float sacc = dot_codes<D>(qw, kr + r * RS, 0.f);
        const float s = j < key_end ? __builtin_ldexpf(sacc, eq + (int)ks[r] - 254) : -__builtin_inff();
        const float dacc = dot_codes<D>(ow, vr + r * RS, 0.f);
        const float dpd = Di - __builtin_ldexpf(dacc, edo + (int)vs[r] - 254);  // D - dP
        const float pv = __builtin_amdgcn_exp2f(fmaf(s, c, -lse));
        const float dsv = -(pv * dpd);
        u.f.pv[lane][jo] = pv;
        u.f.ds[lane][jo] = dsv;
        pmax = fmaxf(pmax, pv);
        dmax = fmaxf(dmax, fabsf(dsv));
#ifdef FLAMIA_DEBUG_DUMP
        const int64_t x = dump ? dbg_index(p.dbg, h, i, j) : -1;
        if (x >= 0) {
          if (p.dbg.bwd_s) p.dbg.bwd_s[x] = s;
          if (p.dbg.bwd_dp) p.dbg.bwd_dp[x] = dpd;
        }
#endif
      }
    }
    rmax_p[lane] = pmax;
    rmax_d[lane] = dmax;
    __syncthreads();
    if (own) {
      // the document's block: its rows are lanes a - w0 .. b - w0 - 1
      float bp = 0.f, bd = 0.f;
      for (int x = a - w0; x < b - w0; ++x) {
        bp = fmaxf(bp, rmax_p[x]);
        bd = fmaxf(bd, rmax_d[x]);
      }
      sp = e8m0_byte_nonneg(bp);
      sd = e8m0_byte_nonneg(bd);
      const float fp = __uint_as_float(sp << 23), fd = __uint_as_float(sd << 23);
#pragma unroll 1
    for (int jo = 0; jo < L; ++jo) {
        const uint32_t kp = fp8_code_scaled(u.f.pv[lane][jo], fp), kd = fp8_code_scaled(u.f.ds[lane][jo], fd);
        cp[lane][jo] = (uint8_t)kp;
        cd[lane][jo] = (uint8_t)kd;
#ifdef FLAMIA_DEBUG_DUMP
        const int64_t x = dump ? dbg_index(p.dbg, h, t, a + jo) : -1;
        if (x >= 0) {
          if (p.dbg.bwd_p) { p.dbg.bwd_p[x] = (uint8_t)kp; p.dbg.bwd_ps[x] = (uint8_t)sp; }
          if (p.dbg.bwd_ds) { p.dbg.bwd_ds[x] = (uint8_t)kd; p.dbg.bwd_dss[x] = (uint8_t)sd; }
        }
#endif
      }
    }
    __syncthreads();  // P and dS read: their space takes the Q and dO rows
    if (t < p.T) {
      const uint4* qsrc = reinterpret_cast<const uint4*>(p.q + ((int64_t)t * p.Hq + h) * D + d0);
      const uint4* osrc = reinterpret_cast<const uint4*>(p.dO + ((int64_t)t * p.Hq + h) * D + d0);
      uint4 qv[DC / 16], ov[DC / 16];
#pragma unroll
      for (int x = 0; x < DC / 16; ++x) { qv[x] = qsrc[x]; ov[x] = osrc[x]; }
#pragma unroll
      for (int x = 0; x < DC / 16; ++x) {
        reinterpret_cast<uint4*>(u.r.q + lane * RC)[x] = qv[x];
        reinterpret_cast<uint4*>(u.r.dO + lane * RC)[x] = ov[x];
      }
      qs[lane] = p.sq[(int64_t)h * p.T + t];
      dos[lane] = p.sdo[(int64_t)h * p.T + t];
    }
    if (own) {
      // dQ of row t, this wave's columns: the only key tile's partial sum_j dShat_tj K_j, FP16
      // with the prescale
      const int i = t;
      const int key_end = p.causal_mask ? i + 1 : b;
      const int pi = p.pi[(int64_t)h * p.T + i];
      const float up = exp2i(pi), down = exp2i(-pi) * ss;
      uint16_t* qrow = p.dq + (int64_t)i * p.dqst + (int64_t)h * p.dqsh;
#pragma unroll 1
      for (int c0 = d0; c0 < d0 + DC; c0 += 32) {
        float acc[32];
#pragma unroll
        for (int d = 0; d < 32; ++d) acc[d] = 0.f;
#pragma unroll 1
        for (int j = a; j < key_end; ++j) {
          const float f = __builtin_ldexpf(fp8_value(cd[lane][j - a]), (int)sd - 127 + (int)ks[j - w0] - 127);
          axpy32(acc, f, kr + (j - w0) * RS + c0);
        }
#ifdef FLAMIA_DEBUG_DUMP
        if (p.dbg.dq_part) {  // test builds: the partial as converted to FP16 (key tile 0)
          const int64_t x = dbg_row(p.dbg, h, i);
          if (x >= 0)
            for (int d = 0; d < 32; ++d) p.dbg.dq_part[(x * p.dbg.n_tiles) * D + c0 + d] = acc[d] * up;
        }
#endif
        // the FP16 sum of one partial: +0 + FP16(2^pi partial), as the tile kernels form it
        const _Float16 z = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const _Float16 a0 = z + (_Float16)(acc[4 * e] * up), a1 = z + (_Float16)(acc[4 * e + 1] * up);
          const _Float16 a2 = z + (_Float16)(acc[4 * e + 2] * up), a3 = z + (_Float16)(acc[4 * e + 3] * up);
          *reinterpret_cast<uint2*>(qrow + c0 + 4 * e) =
              make_uint2(pack_bf16((float)a0 * down, (float)a1 * down), pack_bf16((float)a2 * down, (float)a3 * down));
        }
      }
    }
    __syncthreads();  // the codes and rows of this head are in place
    if (own) {
      // dK, dV of key j = t: the rows of its document that see it
      const int j = t, jo = j - a;
      const int row_lo = p.causal_mask ? j : a;
#pragma unroll 1
      for (int i = row_lo; i < b; ++i) {
        const int r = i - w0;
        const float fv = __builtin_ldexpf(fp8_value(cp[r][jo]), (int)sp - 127 + (int)dos[r] - 127);
        const float fk = __builtin_ldexpf(fp8_value(cd[r][jo]), (int)sd - 127 + (int)qs[r] - 127);
        axpy_codes<DC>(av, fv, u.r.dO + r * RC);
        axpy_codes<DC>(ak, fk, u.r.q + r * RC);
      }
    }
    __syncthreads();  // the next head rewrites the codes and rows
  }
  if (own) {
    uint16_t* krow = p.dk + (int64_t)t * p.dkst + (int64_t)g * p.dksh + d0;
    uint16_t* vrow = p.dv + (int64_t)t * p.dvst + (int64_t)g * p.dvsh + d0;
#pragma unroll
    for (int c0 = 0; c0 < DC; c0 += 32) {
      store_bf16x32(krow + c0, ak + c0, ss);
      store_bf16x32(vrow + c0, av + c0, 1.f);
    }
  }
  }  // column passes
  }  // KV heads
}

}  // namespace

hipError_t launch_small_fwd(const FwdParams& p, int d, hipStream_t s) {
  if (p.T <= 0 || p.n_docs <= 0) return hipSuccess;
  const dim3 grid((p.T + SW - 1) / SW, (p.Hq + HEADS_PER_WAVE - 1) / HEADS_PER_WAVE);
  if (d == 128) hipLaunchKernelGGL(small_fwd_kernel<128>, grid, dim3(NL), 0, s, p);
  else hipLaunchKernelGGL(small_fwd_kernel<64>, grid, dim3(NL), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_small_bwd(const BwdParams& p, int d, hipStream_t s) {
  if (p.T <= 0 || p.n_docs <= 0) return hipSuccess;
  if (p.Hq / p.Hkv > SMALL_MAX_GROUP) return hipErrorInvalidValue;  // the caller keeps such calls on the tile kernels
  const dim3 grid((p.T + SW - 1) / SW, (p.Hkv + HEADS_PER_WAVE - 1) / HEADS_PER_WAVE);
  if (d == 128) hipLaunchKernelGGL(small_bwd_kernel<128>, grid, dim3(NL), 0, s, p);
  else hipLaunchKernelGGL(small_bwd_kernel<64>, grid, dim3(NL), 0, s, p);
  return hipGetLastError();
}

}  // namespace flamia
