// Token-block quantiser (FLAMIA MXFP8 path: jaehun.me review §3.1, §3.2, §3.3, §3.4).
//
// One workgroup owns the 32-token document blocks that START inside its 128-token window of
// one head of one tensor.  Such a block may run up to 31 tokens past the window, so the
// workgroup reads rows [W0, W0 + 159).  Each input row is loaded exactly once (kept in
// registers between the amax and the code pass) by the workgroup that owns its block;
// loads are 16 bytes per lane and a row of d BF16 values is covered by d/8 consecutive lanes.
// The window is small so that a workgroup holds few rows in registers and more workgroups fit
// on a compute unit (more loads in flight; measured faster than 256- and 64-token windows).
#include "device_common.h"
#include "kernels.h"

namespace flamia {

namespace {

constexpr int WIN = 128;            // window of block starts per workgroup
constexpr int ROWS = WIN + BLK - 1; // rows a workgroup may touch

// ---- Hadamard rotation of the head dimension (jaehun.me §3.4 "Hadamard rotation", "Quantization
// fusion").  A row x of D values becomes x H / sqrt(D), H the Sylvester Hadamard matrix.  Fixed
// arithmetic, so that codes decided on the rotated values are reproducible: FP32 butterflies
// for strides 1, 2, ..., D/2 in that order, a pair (a, b) at distance `stride` (a the lower
// index) becoming (a + b, a - b), then the multiply by RN32(1 / sqrt(D)).
// The row is held 8 values per lane by D/8 consecutive lanes (lane lc: elements 8 lc .. 8 lc + 7),
// so strides 1, 2, 4 stay in the lane and strides 8 .. D/2 pair lane lc with lane lc ^ (stride / 8).
template <int M>
__device__ __forceinline__ float xor_lane(float x) {
  if constexpr (M == 1) return dpp<0xB1>(x);  // quad_perm [1,0,3,2]
  else if constexpr (M == 2) return dpp<0x4E>(x);  // quad_perm [2,3,0,1]
  else if constexpr (M == 4) return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x101F));
  else return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x201F));  // lane ^ 8
}
template <int M>
__device__ __forceinline__ void cross_stage(float (&v)[8], int lc) {
  const bool upper = (lc & M) != 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float other = xor_lane<M>(v[e]);
    v[e] = upper ? __fsub_rn(other, v[e]) : __fadd_rn(v[e], other);
  }
}
template <int D>
__device__ __forceinline__ void hadamard_row(float (&v)[8], int lc) {
#pragma unroll
  for (int st = 1; st < 8; st *= 2)
#pragma unroll
    for (int i = 0; i < 8; i += 2 * st)
#pragma unroll
      for (int j = i; j < i + st; ++j) {
        const float a = v[j], b = v[j + st];
        v[j] = __fadd_rn(a, b);
        v[j + st] = __fsub_rn(a, b);
      }
  cross_stage<1>(v, lc);
  cross_stage<2>(v, lc);
  cross_stage<4>(v, lc);
  if constexpr (D == 128) cross_stage<8>(v, lc);
  constexpr float c = (D == 128) ? 0x1.6a09e6p-4f : 0.125f;  // RN32(1 / sqrt(D))
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = __fmul_rn(v[e], c);
}
// E2M1 codes (values 0, 0.5, 1, 1.5, 2, 3, 4, 6) come from the hardware conversion
// v_cvt_scalef32_pk_fp4_f32 with scale 1 on values already scaled exactly by 2^-s: it rounds to
// nearest even and keeps the sign on zero (checked on the hardware against the definition,
// every midpoint and its float neighbours included); values never exceed 6 under the round-up
// exponent.
// Smallest s with amax <= 6 2^s for amax = 1.f 2^E (f in [1, 2)): s = E - 2 + (f > 1.5); adding
// 2^22 - 1 carries into the exponent field exactly when the mantissa exceeds 0.5.  Clamped to
// >= -127 (zero and subnormal amax).
__device__ __forceinline__ int e2m1_exponent(float amax) {
  const int s = (int)((__float_as_uint(amax) + 0x3FFFFFu) >> 23) - 129;
  return s < -127 ? -127 : s;
}
__device__ __forceinline__ void bf16x8_to_f32(const uint4& w, float (&v)[8]) {
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf16_lo(a[i]);
    v[2 * i + 1] = bf16_hi(a[i]);
  }
}

template <int D>
__global__ __launch_bounds__(256) void quantize_kernel(QuantParams p) {
  constexpr int LPR = D / 8;            // lanes per row
  constexpr int RPP = 256 / LPR;        // rows per pass
  constexpr int NPASS = (ROWS + RPP - 1) / RPP;
  __shared__ int16_t own_start[ROWS];   // block start (relative) of an owned row, -1: not owned, -2: outside row to clear
  __shared__ int16_t blk_len[ROWS];
  __shared__ float rmax[ROWS];
  __shared__ int16_t bexp[ROWS];        // exponent for every owned row

  const int tid = threadIdx.x;
  // One grid over every tensor's (window, head) units, tensor after tensor (no idle workgroups
  // for tensors with fewer heads).  Heads vary fastest, so the workgroups running at one time
  // read whole token rows ([T, H, d] packs a token's heads together) rather than one head's
  // slice of many rows.
  int ti = 0;
  while (ti + 1 < p.n_tensors && (int)blockIdx.x >= p.wg_base[ti + 1]) ++ti;
  const QTensorDev& X = p.t[ti];
  const int local = (int)blockIdx.x - p.wg_base[ti];
  const int h = local % X.H;
  const int W0 = (local / X.H) * WIN;
  const int T = p.T;

  // ---- ownership of each row of the window
  for (int r = tid; r < ROWS; r += 256) {
    const int tau = W0 + r;
    int16_t st = -1, len = 0;
    if (tau < T) {
      const int k = find_doc(p.cu, p.n_docs, tau);
      if (k >= 0 && X.per_token) {  // every token is its own block: the window's rows own themselves
        if (r < WIN) {
          st = (int16_t)r;
          len = 1;
        }
      } else if (k >= 0) {
        const int c0 = p.cu[k], c1 = p.cu[k + 1];
        const int bs = c0 + ((tau - c0) / BLK) * BLK;
        if (bs >= W0 && bs < W0 + WIN) {
          st = (int16_t)(bs - W0);
          len = (int16_t)min(BLK, c1 - bs);
        }
      } else if (r < WIN) {
        st = -2;
      }
    }
    own_start[r] = st;
    blk_len[r] = len;
  }
  __syncthreads();

  // ---- pass 1: load owned rows, per-row amax
  const int lr = tid / LPR, lc = tid % LPR;
  uint4 vals[NPASS];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int r = ps * RPP + lr;
    float m = 0.f;
    vals[ps] = make_uint4(0, 0, 0, 0);
    if (r < ROWS && own_start[r] >= 0) {
      const int64_t tau = W0 + r;
      vals[ps] = *reinterpret_cast<const uint4*>(X.x + tau * X.st + (int64_t)h * X.sh + 8 * lc);
      if (X.hadamard) {  // (uniform over the row's lanes, which exchange values)
        float v[8];
        bf16x8_to_f32(vals[ps], v);
        hadamard_row<D>(v, lc);
#pragma unroll
        for (int e = 0; e < 8; ++e) m = (fabsf(v[e]) <= 3.4028235e38f) ? fmaxf(m, fabsf(v[e])) : __int_as_float(0x7F800000);
      } else {
        const uint32_t w[4] = {vals[ps].x, vals[ps].y, vals[ps].z, vals[ps].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
        // a NaN element makes the block's exponent NaN (byte 0xFF)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (((w[i] & 0x7F80u) == 0x7F80u) || ((w[i] & 0x7F800000u) == 0x7F800000u)) m = __int_as_float(0x7F800000);
        }
      }
    }
    if constexpr (LPR == 16) {
      m = row16_max(m);
    } else {
      m = fmaxf(m, dpp<0xB1>(m));
      m = fmaxf(m, dpp<0x4E>(m));
      m = fmaxf(m, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(m), 0x101F)));  // xor 4
    }
    if (lc == 0 && r < ROWS) rmax[r] = m;
  }
  __syncthreads();

  // ---- block exponents (thread per block start)
  for (int r = tid; r < ROWS; r += 256) {
    if (own_start[r] == r) {
      // all 32 reads issued at once (independent, one wait), rows past the block masked off
      float m = 0.f;
      const int len = blk_len[r];
#pragma unroll
      for (int i = 0; i < BLK; ++i) {
        const float x = rmax[min(r + i, ROWS - 1)];
        m = i < len ? fmaxf(m, x) : m;
      }
      bexp[r] = (int16_t)e8m0_roundup(m);
    }
  }
  __syncthreads();
  // ---- scale bytes (thread per row)
  for (int r = tid; r < ROWS; r += 256) {
    const int st = own_start[r];
    const int tau = W0 + r;
    if (st >= 0) {
      const int s = bexp[st];
      X.scales[(int64_t)h * T + tau] = (uint8_t)(s + 127);
    } else if (st == -2) {
      X.scales[(int64_t)h * T + tau] = 0;
    }
  }

  // ---- pass 2: codes (+ D for the dO pass)
  const bool with_d = p.o != nullptr;
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
    const int r = ps * RPP + lr;
    const int st = r < ROWS ? own_start[r] : -1;
    const int64_t tau = W0 + r;
    float dsum = 0.f;
    if (st >= 0) {
      // d = 128: the row again (an L2 hit: this workgroup read it a moment ago) instead of
      // holding every pass's values in registers across the block maxima, which takes the kernel
      // from 84 to 50 registers and from 5 to 8 waves per SIMD (Q/K/V pass 10% faster; at
      // d = 64 the values fit at 8 waves and a reload only costs)
      if constexpr (D == 128) vals[ps] = *reinterpret_cast<const uint4*>(X.x + tau * X.st + (int64_t)h * X.sh + 8 * lc);
      const int s = bexp[st];
      uint2 out;
      if (s == 128) {
        out = make_uint2(0x7F7F7F7Fu, 0x7F7F7F7Fu);
      } else if (X.hadamard) {  // the rotation again (the same arithmetic), then the codes
        const float f = exp2i_neg(s);
        float v[8];
        bf16x8_to_f32(vals[ps], v);
        hadamard_row<D>(v, lc);
        out.x = (uint32_t)pack4_fp8(v[0] * f, v[1] * f, v[2] * f, v[3] * f);
        out.y = (uint32_t)pack4_fp8(v[4] * f, v[5] * f, v[6] * f, v[7] * f);
      } else {
        const float f = exp2i_neg(s);
        const uint32_t w[4] = {vals[ps].x, vals[ps].y, vals[ps].z, vals[ps].w};
        out.x = (uint32_t)pack4_fp8(bf16_lo(w[0]) * f, bf16_hi(w[0]) * f, bf16_lo(w[1]) * f, bf16_hi(w[1]) * f);
        out.y = (uint32_t)pack4_fp8(bf16_lo(w[2]) * f, bf16_hi(w[2]) * f, bf16_lo(w[3]) * f, bf16_hi(w[3]) * f);
        if (with_d) {
          const uint4 ov = *reinterpret_cast<const uint4*>(p.o + tau * p.ost + (int64_t)h * p.osh + 8 * lc);
          const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w};
          const float sc = exp2i(s);
          const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)out.x, false);
          const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)out.x, true);
          const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)out.y, false);
          const auto f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)out.y, true);
          dsum += (f0[0] * sc) * bf16_lo(ow[0]);
          dsum += (f0[1] * sc) * bf16_hi(ow[0]);
          dsum += (f1[0] * sc) * bf16_lo(ow[1]);
          dsum += (f1[1] * sc) * bf16_hi(ow[1]);
          dsum += (f2[0] * sc) * bf16_lo(ow[2]);
          dsum += (f2[1] * sc) * bf16_hi(ow[2]);
          dsum += (f3[0] * sc) * bf16_lo(ow[3]);
          dsum += (f3[1] * sc) * bf16_hi(ow[3]);
        }
      }
      *reinterpret_cast<uint2*>(X.codes + (tau * X.H + h) * D + 8 * lc) = out;
      if (X.codes4) {
        // the 4-bit copy from the same FP32 values: a 32-channel group is the quad of lanes
        // 4 (lc / 4) .. + 3 (rows are whole quads of lanes)
        float v[8];
        bf16x8_to_f32(vals[ps], v);
        if (X.hadamard) hadamard_row<D>(v, lc);
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
        m = fmaxf(m, dpp<0xB1>(m));
        m = fmaxf(m, dpp<0x4E>(m));
        const int s4 = e2m1_exponent(m);
        const float f = exp2i_neg(s4);  // exact scaling here; the conversion then takes scale 1
        uint32_t w = 0;
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0] * f, v[1] * f, 1.0f, 0);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2] * f, v[3] * f, 1.0f, 1);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4] * f, v[5] * f, 1.0f, 2);
        w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6] * f, v[7] * f, 1.0f, 3);
        *reinterpret_cast<uint32_t*>(X.codes4 + (tau * X.H + h) * (D / 2) + 4 * lc) = w;
        if ((lc & 3) == 0) X.scales4[((int64_t)h * T + tau) * (D / 32) + lc / 4] = (uint8_t)(s4 + 127);
      }
    } else if (st == -2) {
      *reinterpret_cast<uint2*>(X.codes + (tau * X.H + h) * D + 8 * lc) = make_uint2(0, 0);
      if (X.codes4) {
        *reinterpret_cast<uint32_t*>(X.codes4 + (tau * X.H + h) * (D / 2) + 4 * lc) = 0;
        if ((lc & 3) == 0) X.scales4[((int64_t)h * T + tau) * (D / 32) + lc / 4] = 0;
      }
    }
    if (with_d) {
      if constexpr (LPR == 16) {
        dsum = row16_sum(dsum);
      } else {
        dsum = dsum + dpp<0xB1>(dsum);
        dsum = dsum + dpp<0x4E>(dsum);
        dsum = dsum + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(dsum), 0x101F));
      }
      if (lc == 0 && (st >= 0 || st == -2)) p.D[(int64_t)h * T + tau] = dsum;
    }
  }
}

// Rows of gradients of rotated operands back to the inputs' basis, in place: BF16 -> FP32, the
// rotation above (its own inverse), BF16 round to nearest even.  One row per D/8 lanes.
template <int D>
__global__ __launch_bounds__(256) void unrotate_kernel(uint16_t* x, int64_t st, int64_t sh, int T, int H) {
  constexpr int LPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int lc = threadIdx.x % LPR;
  if (row >= (int64_t)T * H) return;  // whole rows leave together: the exchanges stay within a row
  const int64_t t = row / H, h = row % H;
  uint4* ptr = reinterpret_cast<uint4*>(x + t * st + h * sh + 8 * lc);
  float v[8];
  bf16x8_to_f32(*ptr, v);
  hadamard_row<D>(v, lc);
  *ptr = make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7]));
}

}  // namespace

hipError_t launch_unrotate(uint16_t* x, int64_t st, int64_t sh, int T, int H, int d, hipStream_t s) {
  const int64_t rows = (int64_t)T * H;
  if (rows == 0) return hipSuccess;
  const int rpb = 256 / (d / 8);  // rows per workgroup
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
  if (d == 128) hipLaunchKernelGGL(unrotate_kernel<128>, grid, dim3(256), 0, s, x, st, sh, T, H);
  else hipLaunchKernelGGL(unrotate_kernel<64>, grid, dim3(256), 0, s, x, st, sh, T, H);
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantParams& p, int d, hipStream_t s) {
  if (p.T == 0) return hipSuccess;
  const dim3 grid(p.wg_base[p.n_tensors]);  // every tensor's (window, head) units
  if (d == 128) hipLaunchKernelGGL(quantize_kernel<128>, grid, dim3(256), 0, s, p);
  else hipLaunchKernelGGL(quantize_kernel<64>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace flamia
