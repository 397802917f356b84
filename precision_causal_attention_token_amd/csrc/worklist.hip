// GPU work-list builder (jaehun.me review §3.4 "Work scheduling"; agihunt.info: the list for
// 131,072 one-token documents).
//
// Items are (document, block) pairs stably sorted by descending cost.  The sort is a counting
// sort done by one 1024-thread workgroup, using one property of these lists: inside a document
// every item has a different cost.
//   FWD: a document of length L with n = ceil(L/256) items and m = ceil(L/128) key tiles has
//        the costs {2, 4, ..., 2n-2} and m, so it has an item of cost c iff
//        (c even and c <= m) or c == m.
//   BWD: key tile kappa costs m - kappa, so the costs are exactly 1..m.
// Hence the position of item (document k, cost c) is
//   #items of cost > c  +  #documents k' < k that have an item of cost c.
// Non-causal lists (kinds 2 = FWD, 3 = BWD): every item of a document costs m, so a document's
// items (n = ceil(L/256), or m) sit together, in block order, at
//   #items of cost > m  +  #items of documents k' < k of cost m.
// Cost-1 items come from documents with m == 1 (FWD) or m >= 1 (BWD) and are placed by a
// prefix count over documents: those of documents longer than SMALL_DOC tokens first, then
// those of the shorter ones (every kind gives such a document one item of cost 1), which
// therefore close the list; their number goes to word 2 of the counters after the items, so
// the attention kernels can leave them to the small-document pass.  Items of cost >= 2 exist only in "long" documents (m >= 2,
// at most T/129 of them), which are listed in LDS; for every cost c one thread walks that
// list in document order and emits the items of cost c.
#include "device_common.h"
#include "kernels.h"

namespace flamia {

namespace {

constexpr int NT = 1024;

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Exclusive scan of one int per thread across the workgroup; returns the prefix, writes the
// total to *total.  `scratch` holds NT/64 ints.
__device__ int wg_exclusive_scan(int x, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < NT / 64; ++w) {
      const int t = scratch[w];
      scratch[w] = run;
      run += t;
    }
    scratch[NT / 64] = run;
  }
  __syncthreads();
  const int res = scratch[wave] + incl - x;
  *total = scratch[NT / 64];
  __syncthreads();
  return res;
}

__device__ __forceinline__ int serpentine(int i, int G) {
  const int r = i / G, w = i - r * G;
  return (r & 1) ? (G - 1 - w) : w;
}

template <int KIND>
__device__ __forceinline__ bool has_cost(int m, int c) {
  if constexpr (KIND == 0) return ((c & 1) == 0 && c <= m) || c == m;
  else if constexpr (KIND == 1) return c <= m;
  else return c == m;
}
// Items of a document of length L (m key tiles) in a list of this kind.
template <int KIND>
__device__ __forceinline__ int n_items_of(int L, int m) {
  return (KIND % 2 == 0) ? ceil_div(L, 256) : m;
}

// The list's schedule ([J] §3.4 "Work scheduling"): a non-causal list is taken dynamically when
// its longest document is at least 4 times the average document length (over all n_docs
// documents): longest * n_docs >= 4 * total, in integers.  Header word 3 then holds the position
// (in int32 words from the list's start) of the forward's unit counters `ctr`, after the room
// for the items, cleared here; causal lists keep 0 (the forward walks them statically; the
// backward takes its units dynamically whatever the word).
template <int KIND>
__global__ __launch_bounds__(NT) void worklist_kernel(const int32_t* __restrict__ cu, int n_docs, int max_cost,
                                                      int max_long, int G, int32_t* __restrict__ list,
                                                      int32_t* __restrict__ ctr) {
  extern __shared__ int smem[];
  int* hist = smem;                        // [max_cost + 2]: items per cost
  int* before = hist + (max_cost + 2);     // [max_cost + 2]: items of larger cost
  int* long_doc = before + (max_cost + 2); // [max_long]
  int* long_m = long_doc + max_long;       // [max_long]
  int* scratch = long_m + max_long;        // [NT/64 + 1]

  const int tid = threadIdx.x;
  __shared__ int longest;
  for (int c = tid; c < max_cost + 2; c += NT) hist[c] = 0;
  if (tid == 0) longest = 0;
  if (tid < FWD_CTR_WORDS) ctr[tid] = 0;
  __syncthreads();

  // ---- phase A: each wave takes a contiguous span of documents, 64 at a time (lane l: document
  // g0 + l), so the bounds' loads here and the items' stores of phase C1 are coalesced; positions
  // inside a group come from ballots (lanes below with the same kind of item)
  constexpr int NWV = NT / 64;
  const int lane = tid & 63, wave = tid >> 6;
  const int per_w = (ceil_div(n_docs, NWV) + 63) / 64 * 64;
  const int w_lo = min(n_docs, wave * per_w), w_hi = min(n_docs, w_lo + per_w);
  __shared__ int wsum[3][NWV], wbase[3][NWV], wtot[3];
  int n1 = 0, ns = 0, nl = 0;  // wave-uniform: cost-1 items of longer documents, short documents, long documents
  int lmax = 0;
  for (int g0 = w_lo; g0 < w_hi; g0 += 64) {
    const int k = g0 + lane;
    const bool in = k < w_hi;
    const int L = in ? cu[k + 1] - cu[k] : 0;
    lmax = max(lmax, L);
    const int m = ceil_div(L, 128);
    const bool small = L >= 1 && L <= SMALL_DOC;
    const bool one = in && !small && (KIND == 1 ? (m >= 1) : (m == 1));
    n1 += __popcll(__ballot(one));
    ns += __popcll(__ballot(small));
    nl += __popcll(__ballot(m >= 2));
    if (m >= 2) {
      if (KIND == 0) {
        const int n = ceil_div(L, 256);
        for (int bb = 0; bb + 1 < n; ++bb) atomicAdd(&hist[2 * bb + 2], 1);
        atomicAdd(&hist[m], 1);
      } else if (KIND == 1) {
        for (int c = 2; c <= m; ++c) atomicAdd(&hist[c], 1);
      } else {
        atomicAdd(&hist[m], n_items_of<KIND>(L, m));
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lmax = max(lmax, __shfl_xor(lmax, off, 64));
  if (lane == 0) {
    if (n1 + ns) atomicAdd(&hist[1], n1 + ns);
    if (KIND >= 2 && lmax) atomicMax(&longest, lmax);
    wsum[0][wave] = n1;
    wsum[1][wave] = ns;
    wsum[2][wave] = nl;
  }
  __syncthreads();
  if (tid < 3) {  // exclusive prefix over the waves, in document order
    int run = 0;
    for (int w = 0; w < NWV; ++w) {
      wbase[tid][w] = run;
      run += wsum[tid][w];
    }
    wtot[tid] = run;
  }
  __syncthreads();
  const int base1 = wbase[0][wave], bases = wbase[1][wave], basel = wbase[2][wave];
  const int tot1 = wtot[0], tots = wtot[1], totl = wtot[2];
  if (tid == 0) ctr[2] = tots;  // after the clearing above (the barriers order them)
  {
    int j = basel;
    for (int g0 = w_lo; g0 < w_hi; g0 += 64) {
      const int k = g0 + lane;
      const int m = k < w_hi ? ceil_div(cu[k + 1] - cu[k], 128) : 0;
      const uint64_t bl = __ballot(m >= 2);
      if (m >= 2) {
        const int pos = j + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bl >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bl, 0u));
        long_doc[pos] = k;
        long_m[pos] = m;
      }
      j += __popcll(bl);
    }
  }
  __syncthreads();

  // ---- phase B: before[c] = number of items with cost > c (suffix sums over the histogram)
  {
    const int per_c = ceil_div(max_cost, NT);
    // thread tid covers costs c in (max_cost - (tid+1)*per_c, max_cost - tid*per_c]
    const int chi = max_cost - tid * per_c, clo = max(chi - per_c, 0);
    int local = 0;
    for (int c = chi; c > clo; --c) local += hist[c];
    int total;
    int run = wg_exclusive_scan(local, scratch, &total);
    for (int c = chi; c > clo; --c) {
      before[c] = run;
      run += hist[c];
    }
    if (tid == 0) {
      list[0] = total;
      list[1] = KIND;
      list[2] = n_docs;
      const int64_t tokens = n_docs > 0 ? (int64_t)cu[n_docs] - cu[0] : 0;
      list[3] = (KIND >= 2 && tokens > 0 && (int64_t)longest * n_docs >= 4 * tokens) ? (int)(ctr - list) : 0;
    }
  }
  __syncthreads();

  int4* items = reinterpret_cast<int4*>(list + 4);
  // ---- phase C1: cost-1 items, placed by document order (short documents after the others)
  {
    const int b1 = before[1];
    const float rG = 1.0f / (float)G;
    int r = b1 + base1, rs = b1 + tot1 + bases;  // wave-uniform: next position of each run
    for (int g0 = w_lo; g0 < w_hi; g0 += 64) {
      const int k = g0 + lane;
      const bool in = k < w_hi;
      const int L = in ? cu[k + 1] - cu[k] : 0;
      const int m = ceil_div(L, 128);
      const bool small = L >= 1 && L <= SMALL_DOC;
      const bool one = in && !small && (KIND == 1 ? (m >= 1) : (m == 1));
      const uint64_t bs = __ballot(small), bo = __ballot(one);
      if (small || one) {
        const uint64_t bb = small ? bs : bo;
        const int below = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bb, 0u));
        const int pos = (small ? rs : r) + below;
        // serpentine tag: round = pos / G from a float estimate, corrected exactly
        int round = (int)((float)pos * rG);
        while (round > 0 && round * G > pos) --round;
        while ((round + 1) * G <= pos) ++round;
        const int w = pos - round * G;
        items[pos] = make_int4(k, KIND == 1 ? m - 1 : 0, 1, (round & 1) ? (G - 1 - w) : w);
      }
      r += __popcll(bo);
      rs += __popcll(bs);
    }
  }
  // ---- phase C2: items of cost >= 2, one thread per cost walking the long documents in order
  for (int c = 2 + tid; c <= max_cost; c += NT) {
    if (hist[c] == 0) continue;
    int r = before[c];
    for (int j = 0; j < totl; ++j) {
      const int m = long_m[j];
      if (has_cost<KIND>(m, c)) {
        if constexpr (KIND >= 2) {  // non-causal: all of the document's items, in block order
          const int k = long_doc[j];
          const int n = n_items_of<KIND>(cu[k + 1] - cu[k], m);
          for (int b = 0; b < n; ++b, ++r) items[r] = make_int4(k, b, c, serpentine(r, G));
        } else {
          const int blk = (KIND == 0) ? ((c == m) ? ceil_div(m, 2) - 1 : c / 2 - 1) : (m - c);
          items[r] = make_int4(long_doc[j], blk, c, serpentine(r, G));
          r++;
        }
      }
    }
  }
}

}  // namespace

size_t worklist_lds_bytes(int T) {
  const int max_cost = (T + 127) / 128 + 1;
  const int max_long = T / 129 + 2;
  return sizeof(int) * (2 * (max_cost + 2) + 2 * max_long + NT / 64 + 1);
}

hipError_t launch_worklist(const int32_t* cu, int n_docs, int T, int kind, int n_workers, int32_t* list,
                           int32_t* ctr, hipStream_t s) {
  const int max_cost = (T + 127) / 128 + 1;
  const int max_long = T / 129 + 2;
  const size_t lds = worklist_lds_bytes(T);
  auto go = [&](auto kern) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(1), dim3(NT), lds, s, cu, n_docs, max_cost, max_long, n_workers, list, ctr);
    return hipGetLastError();
  };
  switch (kind) {
    case 0: return go(worklist_kernel<0>);
    case 1: return go(worklist_kernel<1>);
    case 2: return go(worklist_kernel<2>);
    default: return go(worklist_kernel<3>);
  }
}

}  // namespace flamia
