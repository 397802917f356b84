// C ABI of libflamia (declared in include/flamia.h): argument checks and kernel launches.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "../../include/flamia.h"
#include "kernels.h"
#ifdef FLAMIA_DEBUG_DUMP
#include "../../include/flamia_debug.h"
#endif

using namespace flamia;

#ifdef FLAMIA_DEBUG_DUMP
namespace {
DebugDump g_dbg{};  // all-NULL: nothing dumped
}
extern "C" flamia_status flamia_debug_set_dump(const flamia_debug_dump* d) {
  if (!d) {
    g_dbg = DebugDump{};
    return FLAMIA_OK;
  }
  if (d->row_hi <= d->row_lo || d->key_hi <= d->key_lo || d->head_hi <= d->head_lo) return FLAMIA_ERR_SHAPE;
  g_dbg = DebugDump{d->row_lo, d->row_hi, d->key_lo, d->key_hi, d->head_lo, d->head_hi, d->fwd_s, d->fwd_m,
                    d->fwd_p, d->bwd_s, d->bwd_dp, d->bwd_p, d->bwd_ps, d->bwd_ds, d->bwd_dss, d->dq_part,
                    d->n_tiles, d->dq_s, d->dq_dp, d->dq_ds, d->dq_dss, d->fwd_ps};
  return FLAMIA_OK;
}
#endif

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// softmax_scale * log2(e), formed in double and rounded once; the forward and the backward
// use this same float, so their scores agree bit for bit.
float score_scale(float softmax_scale, int d) {
  const double ss = softmax_scale > 0.f ? (double)softmax_scale : 1.0 / sqrt((double)d);
  return (float)(ss * 1.4426950408889634074);
}
float resolved_scale(float softmax_scale, int d) {
  return softmax_scale > 0.f ? softmax_scale : (float)(1.0 / sqrt((double)d));
}

int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

}  // namespace

namespace {
// Backward workspace: a 256-byte header (status, chunk count), pi [Hq, T], the chunk layout
// tables, then the dShat store (per (block, query head): 8 KiB of codes, then 8 exponent bytes
// padded to a 128-byte line, so every block starts on a cache line).
constexpr size_t DS_BLOCK_BYTES = 128 * 64 + 128;
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
// (document, key tile) table entries: at most ceil(T / 128) + n_docs tiles.
int64_t n_tiles(int32_t n_docs, int32_t T) { return ((int64_t)T + 127) / 128 + n_docs; }
// entries of the per-chunk tables (a bound on the chunk count + 2)
int64_t n_chunk_entries(int32_t T) { return ((int64_t)T + 63) / 64 + 16; }
struct BwdLayout {
  size_t pi, tile_base, kv_chunk, kv_off, chunk_start, chunk_first, counters, store;  // byte offsets
};
BwdLayout bwd_layout(int32_t n_docs, int32_t T, int32_t Hq) {
  BwdLayout l{};
  size_t off = 256;
  l.pi = off;          off += align256((size_t)T * Hq * 2);
  l.tile_base = off;   off += align256(((size_t)n_docs + 1) * 4);
  l.kv_chunk = off;    off += align256((size_t)n_tiles(n_docs, T) * 4);
  l.kv_off = off;      off += align256((size_t)n_tiles(n_docs, T) * 8);
  l.chunk_start = off; off += align256((size_t)n_chunk_entries(T) * 4);
  l.chunk_first = off; off += align256((size_t)n_chunk_entries(T) * 8);
  l.counters = off;    off += align256((size_t)n_chunk_entries(T) * 64);  // 16 int32 per chunk
  l.store = off;
  return l;
}
// Stored blocks (per query head) of the largest single backward item: the query tiles of a
// T-token document.
int64_t max_item_blocks(int32_t T) { return std::max<int64_t>(1, ((int64_t)T + 63) / 64); }
// Stored blocks of a document of length L: one per (128-key tile kappa, 64-query tile qt >= 2 kappa)
// (non-causal: every 64-query tile), none when the document has a single key tile.
int64_t doc_blocks(int64_t L, bool non_causal) {
  const int64_t n_kt = (L + 127) / 128, n_qt = (L + 63) / 64;
  if (n_kt < 2) return 0;
  return non_causal ? n_kt * n_qt : n_kt * n_qt - n_kt * (n_kt - 1);
}
// An upper bound of the stored blocks of any documents of total length T: a document of length L
// in (128 m, 128 (m + 1)] stores at most (m + 1)(m + 2) < (L / 128)(L / 128 + 3) + 2 blocks, at
// most T / 129 documents store any, and sum L^2 <= T^2.
int64_t worst_blocks(int32_t T) {
  const int64_t t = T;
  return (t * t) / 16384 + 5 * t / 128 + 3;
}
// The same for non-causal attention, whose documents store every (query tile, key tile) pair:
// (m + 1)(2m + 2) < 2 (L / 128)(L / 128 + 3) + 2 blocks for L in (128 m, 128 (m + 1)].
int64_t worst_blocks_nc(int32_t T) {
  const int64_t t = T;
  return (t * t) / 8192 + 5 * t / 64 + 3;
}
// The same bounds for documents no longer than M tokens: sum L^2 <= M T.
int64_t worst_blocks_max(int32_t T, int32_t M, bool non_causal) {
  const int64_t t = T, m = std::min<int64_t>(M, T);
  return non_causal ? (m * t) / 8192 + 5 * t / 64 + 3 : (m * t) / 16384 + 5 * t / 128 + 3;
}
}  // namespace

extern "C" {

const char* flamia_status_str(flamia_status s) {
  switch (s) {
    case FLAMIA_OK: return "ok";
    case FLAMIA_ERR_NULL: return "null pointer";
    case FLAMIA_ERR_SHAPE: return "bad shape or stride";
    case FLAMIA_ERR_UNSUPPORTED: return "unsupported size";
    case FLAMIA_ERR_WORKSPACE: return "buffer too small";
    case FLAMIA_ERR_HIP: return "HIP error";
    case FLAMIA_ERR_SCRATCH: return "call too large for the static scratch";
  }
  return "unknown status";
}

int32_t flamia_num_workers(void) { return num_cus(); }

size_t flamia_worklist_bytes(int32_t n_docs, int32_t T, int32_t kind) {
  (void)kind;
  if (n_docs < 0 || T < 0) return 0;
  return worklist_ctr_offset(n_docs, T) + 4 * FWD_CTR_WORDS;
}

flamia_status flamia_build_worklist(const int32_t* cu_seqlens, int32_t n_docs, int32_t T, int32_t kind,
                                    int32_t n_workers, void* list, size_t list_bytes, void* stream) {
  if (!cu_seqlens || !list) return FLAMIA_ERR_NULL;
  if (n_docs < 0 || T < 0 || n_workers < 1 || kind < FLAMIA_LIST_FWD || kind > FLAMIA_LIST_BWD_NC)
    return FLAMIA_ERR_SHAPE;
  if (T > FLAMIA_MAX_T_WORKLIST) return FLAMIA_ERR_UNSUPPORTED;
  if (list_bytes < flamia_worklist_bytes(n_docs, T, kind)) return FLAMIA_ERR_WORKSPACE;
  if (!aligned(list, 16)) return FLAMIA_ERR_SHAPE;
  int32_t* l = static_cast<int32_t*>(list);
  hipError_t e = launch_worklist(cu_seqlens, n_docs, T, kind, n_workers, l,
                                 l + worklist_ctr_offset(n_docs, T) / 4, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FLAMIA_OK : FLAMIA_ERR_HIP;
}

flamia_status flamia_quantize(const flamia_qtensor* tensors, int32_t n_tensors, int32_t T, int32_t d,
                              const int32_t* cu_seqlens, int32_t n_docs, const void* o, int64_t o_stride_t,
                              int64_t o_stride_h, float* D, void* stream) {
  if (!tensors || !cu_seqlens) return FLAMIA_ERR_NULL;
  if (n_tensors < 1 || n_tensors > 3 || (o && n_tensors != 1)) return FLAMIA_ERR_SHAPE;
  if (T < 0 || n_docs < 0) return FLAMIA_ERR_SHAPE;
  if (T > FLAMIA_MAX_T) return FLAMIA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return FLAMIA_ERR_UNSUPPORTED;
  if (o && !D) return FLAMIA_ERR_NULL;
  if (o && tensors[0].hadamard) return FLAMIA_ERR_UNSUPPORTED;  // dO is never rotated
  QuantParams p{};
  p.n_tensors = n_tensors;
  p.T = T;
  p.cu = cu_seqlens;
  p.n_docs = n_docs;
  p.maxH = 0;
  for (int i = 0; i < n_tensors; ++i) {
    const flamia_qtensor& t = tensors[i];
    if (!t.x || !t.codes || !t.scales) return FLAMIA_ERR_NULL;
    if (t.H < 1) return FLAMIA_ERR_SHAPE;
    // 16-byte vector loads of 8 BF16 values
    if (!aligned(t.x, 16) || (t.stride_t % 8) || (t.stride_h % 8) || t.stride_t < 0 || t.stride_h < 0)
      return FLAMIA_ERR_SHAPE;
    if (!aligned(t.codes, 16)) return FLAMIA_ERR_SHAPE;
    if ((t.mx4_codes == nullptr) != (t.mx4_scales == nullptr)) return FLAMIA_ERR_NULL;
    if (t.mx4_codes && o) return FLAMIA_ERR_UNSUPPORTED;  // the 4-bit copy is for Q and K
    if (t.mx4_codes && !aligned(t.mx4_codes, 4)) return FLAMIA_ERR_SHAPE;
    p.t[i] = QTensorDev{static_cast<const uint16_t*>(t.x), t.stride_t, t.stride_h, t.H, t.codes, t.scales,
                        t.hadamard ? 1 : 0, t.per_token ? 1 : 0, t.mx4_codes, t.mx4_scales};
    if (t.H > p.maxH) p.maxH = t.H;
  }
  if (o) {
    if (!aligned(o, 16) || (o_stride_t % 8) || (o_stride_h % 8) || o_stride_t < 0 || o_stride_h < 0)
      return FLAMIA_ERR_SHAPE;
    p.o = static_cast<const uint16_t*>(o);
    p.ost = o_stride_t;
    p.osh = o_stride_h;
    p.D = D;
  }
  int64_t wgs = 0;
  for (int i = 0; i < n_tensors; ++i) {
    p.wg_base[i] = (int32_t)wgs;
    wgs += (int64_t)tensors[i].H * ((T + 127) / 128);
    if (wgs > 0x7FFFFFFF) return FLAMIA_ERR_UNSUPPORTED;  // grid size
  }
  p.wg_base[n_tensors] = (int32_t)wgs;
  hipError_t e = launch_quantize(p, d, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FLAMIA_OK : FLAMIA_ERR_HIP;
}

flamia_status flamia_fwd(const flamia_fwd_args* a, void* stream) {
  if (!a) return FLAMIA_ERR_NULL;
  if (!a->q || !a->k || !a->v || !a->sq || !a->sk || !a->sv || !a->cu_seqlens || !a->fwd_list || !a->o || !a->lse)
    return FLAMIA_ERR_NULL;
  if (a->T < 0 || a->Hq < 1 || a->Hkv < 1 || a->n_docs < 0) return FLAMIA_ERR_SHAPE;
  if (a->d != 64 && a->d != 128) return FLAMIA_ERR_UNSUPPORTED;
  if (a->Hq % a->Hkv) return FLAMIA_ERR_UNSUPPORTED;
  if (a->precise && a->non_causal) return FLAMIA_ERR_UNSUPPORTED;
  if (a->T > FLAMIA_MAX_T) return FLAMIA_ERR_UNSUPPORTED;
  if (!aligned(a->o, 8) || (a->o_stride_t % 4) || (a->o_stride_h % 4) || a->o_stride_t < 0 || a->o_stride_h < 0)
    return FLAMIA_ERR_SHAPE;
  if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->fwd_list, 16))
    return FLAMIA_ERR_SHAPE;
  const int n4 = (a->q4 != nullptr) + (a->sq4 != nullptr) + (a->k4 != nullptr) + (a->sk4 != nullptr);
  if (n4 != 0 && n4 != 4) return FLAMIA_ERR_NULL;
  if (n4 && a->precise) return FLAMIA_ERR_UNSUPPORTED;
  if (n4 && (!aligned(a->q4, 16) || !aligned(a->k4, 16) || !aligned(a->sq4, 4) || !aligned(a->sk4, 4)))
    return FLAMIA_ERR_SHAPE;
  const int grid = num_cus();
  if (grid <= 0) return FLAMIA_ERR_HIP;
  FwdParams p{};
  p.q4 = a->q4; p.sq4 = a->sq4; p.k4 = a->k4; p.sk4 = a->sk4;
  p.q = a->q; p.k = a->k; p.v = a->v; p.sq = a->sq; p.sk = a->sk; p.sv = a->sv;
  p.T = a->T; p.Hq = a->Hq; p.Hkv = a->Hkv;
  p.c = score_scale(a->softmax_scale, a->d);
  p.cu = a->cu_seqlens; p.n_docs = a->n_docs;
  p.list = static_cast<int32_t*>(a->fwd_list);
  p.o = static_cast<uint16_t*>(a->o); p.ost = a->o_stride_t; p.osh = a->o_stride_h;
  p.lse = a->lse;
  p.causal = a->non_causal ? 0 : 1;
  p.precise = a->precise ? 1 : 0;
  p.small = small_docs_pass(a->precise != 0, n4 != 0, a->Hq, a->Hkv);
#ifdef FLAMIA_DEBUG_DUMP
  p.dbg = g_dbg;
#endif
  hipError_t e = launch_fwd(p, a->d, grid, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FLAMIA_OK : FLAMIA_ERR_HIP;
}


size_t flamia_bwd_workspace_bytes(int32_t n_docs, int32_t T, int32_t Hq, int32_t d, size_t store_budget) {
  if (T < 0 || Hq < 1 || n_docs < 0 || (d != 64 && d != 128)) return 0;
  const int64_t lo = 2 * max_item_blocks(T);                      // the smallest store accepted
  const int64_t hi = worst_blocks_nc(T) + max_item_blocks(T);     // one chunk for any documents
  const int64_t want = (int64_t)(store_budget / ((size_t)Hq * DS_BLOCK_BYTES));
  const int64_t blocks = std::max(lo, std::min(want, hi));
  return bwd_layout(n_docs, T, Hq).store + (size_t)blocks * Hq * DS_BLOCK_BYTES;
}

size_t flamia_bwd_workspace_bytes_for(const int32_t* cu_seqlens_host, int32_t n_docs, int32_t T, int32_t Hq,
                                      int32_t d, int32_t non_causal) {
  if (T < 0 || Hq < 1 || n_docs < 0 || (n_docs > 0 && !cu_seqlens_host) || (d != 64 && d != 128)) return 0;
  int64_t blocks = 0;
  for (int32_t k = 0; k < n_docs; ++k) blocks += doc_blocks((int64_t)cu_seqlens_host[k + 1] - cu_seqlens_host[k], non_causal != 0);
  const int64_t store = std::max<int64_t>(blocks, max_item_blocks(T)) + max_item_blocks(T);
  return bwd_layout(n_docs, T, Hq).store + (size_t)store * Hq * DS_BLOCK_BYTES;
}

flamia_status flamia_bwd(const flamia_bwd_args* a, void* stream) {
  if (!a) return FLAMIA_ERR_NULL;
  if (!a->q || !a->k || !a->v || !a->dO || !a->sq || !a->sk || !a->sv || !a->sdO || !a->lse || !a->D ||
      !a->cu_seqlens || !a->fwd_list || !a->bwd_list || !a->dq || !a->dk || !a->dv || !a->workspace)
    return FLAMIA_ERR_NULL;
  if (a->T < 0 || a->Hq < 1 || a->Hkv < 1 || a->n_docs < 0) return FLAMIA_ERR_SHAPE;
  if (a->d != 64 && a->d != 128) return FLAMIA_ERR_UNSUPPORTED;
  if (a->Hq % a->Hkv) return FLAMIA_ERR_UNSUPPORTED;
  if (a->T > FLAMIA_MAX_T) return FLAMIA_ERR_UNSUPPORTED;
  if (a->non_causal && a->causal_dq_scale) return FLAMIA_ERR_UNSUPPORTED;
  if (a->non_causal && a->precise) return FLAMIA_ERR_UNSUPPORTED;  // the precision options are causal
  const int n4 = (a->q4 != nullptr) + (a->sq4 != nullptr) + (a->k4 != nullptr) + (a->sk4 != nullptr);
  if (n4 != 0 && n4 != 4) return FLAMIA_ERR_NULL;
  if (n4 && a->precise) return FLAMIA_ERR_UNSUPPORTED;
  if (n4 && (!aligned(a->q4, 16) || !aligned(a->k4, 16) || !aligned(a->sq4, 4) || !aligned(a->sk4, 4)))
    return FLAMIA_ERR_SHAPE;
  if (a->workspace_bytes < flamia_bwd_workspace_bytes(a->n_docs, a->T, a->Hq, a->d, 0)) return FLAMIA_ERR_WORKSPACE;
  const int64_t st[6] = {a->dq_stride_t, a->dq_stride_h, a->dk_stride_t, a->dk_stride_h, a->dv_stride_t, a->dv_stride_h};
  for (int i = 0; i < 6; ++i)
    if (st[i] < 0 || (st[i] % 4)) return FLAMIA_ERR_SHAPE;
  if (!aligned(a->dq, 8) || !aligned(a->dk, 8) || !aligned(a->dv, 8) || !aligned(a->workspace, 256))
    return FLAMIA_ERR_SHAPE;
  if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->dO, 16) ||
      !aligned(a->fwd_list, 16) || !aligned(a->bwd_list, 16))
    return FLAMIA_ERR_SHAPE;
  // the un-rotation moves 16-byte pieces of 8 values
  if (a->hadamard && (!aligned(a->dq, 16) || !aligned(a->dk, 16) || (a->dq_stride_t % 8) || (a->dq_stride_h % 8) ||
                      (a->dk_stride_t % 8) || (a->dk_stride_h % 8)))
    return FLAMIA_ERR_SHAPE;
  const int grid = num_cus();
  if (grid <= 0) return FLAMIA_ERR_HIP;
  BwdParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v; p.dO = a->dO;
  p.sq = a->sq; p.sk = a->sk; p.sv = a->sv; p.sdo = a->sdO;
  p.lse = a->lse; p.Dv = a->D;
  p.T = a->T; p.Hq = a->Hq; p.Hkv = a->Hkv;
  p.c = score_scale(a->softmax_scale, a->d);
  p.softmax_scale = resolved_scale(a->softmax_scale, a->d);
  p.cu = a->cu_seqlens; p.n_docs = a->n_docs;
  p.list = static_cast<const int32_t*>(a->bwd_list);
  p.fwd_list = static_cast<const int32_t*>(a->fwd_list);
  p.dq = static_cast<uint16_t*>(a->dq); p.dk = static_cast<uint16_t*>(a->dk); p.dv = static_cast<uint16_t*>(a->dv);
  p.dqst = a->dq_stride_t; p.dqsh = a->dq_stride_h;
  p.dkst = a->dk_stride_t; p.dksh = a->dk_stride_h;
  p.dvst = a->dv_stride_t; p.dvsh = a->dv_stride_h;
  uint8_t* ws = static_cast<uint8_t*>(a->workspace);
  const BwdLayout lay = bwd_layout(a->n_docs, a->T, a->Hq);
  p.status = reinterpret_cast<int32_t*>(ws);
  p.pi = reinterpret_cast<int16_t*>(ws + lay.pi);
  p.tile_base = reinterpret_cast<int32_t*>(ws + lay.tile_base);
  p.kv_chunk = reinterpret_cast<int32_t*>(ws + lay.kv_chunk);
  p.kv_off = reinterpret_cast<int64_t*>(ws + lay.kv_off);
  p.chunk_start = reinterpret_cast<int32_t*>(ws + lay.chunk_start);
  p.chunk_first = reinterpret_cast<int64_t*>(ws + lay.chunk_first);
  p.counters = reinterpret_cast<int32_t*>(ws + lay.counters);
  p.ds_store = ws + lay.store;
  // Chunks: the store holds cap blocks per query head; a chunk spans chunk_cap = cap - (largest
  // item) blocks of last-block positions, so it never overflows the store; the launches cover
  // the most chunks any documents of total length T (no longer than max_doc_len, when given)
  // could need (those past the laid-out count exit at once; a layout that needs more fails with
  // status 3 in the prologue).
  const int64_t cap = (int64_t)((a->workspace_bytes - lay.store) / DS_BLOCK_BYTES) / a->Hq;
  p.chunk_cap = cap - max_item_blocks(a->T);
  if (p.chunk_cap < max_item_blocks(a->T)) return FLAMIA_ERR_WORKSPACE;
  const int64_t worst = a->max_doc_len > 0 ? worst_blocks_max(a->T, a->max_doc_len, a->non_causal != 0)
                                           : (a->non_causal ? worst_blocks_nc(a->T) : worst_blocks(a->T));
  const int64_t max_chunks = (worst - 1) / p.chunk_cap + 1;
  if (max_chunks + 2 > n_chunk_entries(a->T)) return FLAMIA_ERR_WORKSPACE;
  p.max_chunks = (int32_t)max_chunks;
  p.n_tab = (int32_t)n_tiles(a->n_docs, a->T);
  p.pi_out = a->dq_exp_out;
  // the precision options take the causal prescale per token (maxima up to the row)
  p.causal = (a->causal_dq_scale || a->precise) ? 1 : 0;
  p.causal_mask = a->non_causal ? 0 : 1;
  p.precise = a->precise ? 1 : 0;
  p.q4 = a->q4; p.sq4 = a->sq4; p.k4 = a->k4; p.sk4 = a->sk4;
  p.small = small_docs_pass(a->precise != 0, n4 != 0, a->Hq, a->Hkv);
#ifdef FLAMIA_DEBUG_DUMP
  p.dbg = g_dbg;
#endif
  hipError_t e = launch_bwd(p, a->d, grid, static_cast<hipStream_t>(stream));
  if (e == hipSuccess && a->hadamard) {
    e = launch_unrotate(p.dq, a->dq_stride_t, a->dq_stride_h, a->T, a->Hq, a->d, static_cast<hipStream_t>(stream));
    if (e == hipSuccess)
      e = launch_unrotate(p.dk, a->dk_stride_t, a->dk_stride_h, a->T, a->Hkv, a->d, static_cast<hipStream_t>(stream));
  }
  return e == hipSuccess ? FLAMIA_OK : FLAMIA_ERR_HIP;
}

// ------------------------------------------------------------------------------------------
// Backward without allocation: the workspace is a file-scope device array.  In host code the
// array's name is only a stand-in: its device address, different on every GPU, is looked up
// once per device with hipGetSymbolAddress and cached; kernels receive that address.
static __device__ __align__(256) uint8_t scratch[FLAMIA_STATIC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::once_flag scratch_once[MAX_DEVICES];
void* scratch_ptr[MAX_DEVICES];
hipError_t scratch_err[MAX_DEVICES];
}  // namespace

flamia_status flamia_bwd_static(const flamia_bwd_args* a, void* stream) {
  if (!a) return FLAMIA_ERR_NULL;
  if (a->T < 0 || a->Hq < 1 || a->n_docs < 0) return FLAMIA_ERR_SHAPE;
  if (a->d != 64 && a->d != 128) return FLAMIA_ERR_UNSUPPORTED;
  const size_t need = flamia_bwd_workspace_bytes(a->n_docs, a->T, a->Hq, a->d, 0);
  if (need == 0) return FLAMIA_ERR_SHAPE;
  if (need > FLAMIA_STATIC_SCRATCH_BYTES) return FLAMIA_ERR_SCRATCH;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return FLAMIA_ERR_HIP;
  std::call_once(scratch_once[dev], [dev] {
    scratch_err[dev] = hipGetSymbolAddress(&scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (scratch_err[dev] != hipSuccess || !scratch_ptr[dev]) return FLAMIA_ERR_HIP;
  flamia_bwd_args b = *a;
  b.workspace = scratch_ptr[dev];
  b.workspace_bytes = FLAMIA_STATIC_SCRATCH_BYTES;
  return flamia_bwd(&b, stream);
}

}  // extern "C"
