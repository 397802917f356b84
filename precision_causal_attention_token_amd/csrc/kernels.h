// Internal launch interface between the C-ABI layer (flamia_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flamia {

#ifdef FLAMIA_DEBUG_DUMP
// Test builds only (the library variant the parity tests build with FLAMIA_DEBUG_DUMP): where the
// attention kernels copy the intermediates they compute.  Every array is [heads][rows][keys] over
// the window [head_lo, head_hi) x [row_lo, row_hi) x [key_lo, key_hi) (query heads, absolute rows
// and keys); only visited (row, key) pairs of one document are written; NULL arrays are skipped.
struct DebugDump {
  int32_t row_lo, row_hi, key_lo, key_hi, head_lo, head_hi;
  float* fwd_s;       // forward score accumulator after the causal mask (-inf where masked)
  float* fwd_m;       // running maximum (score units) the pair's probability was formed against
  uint8_t* fwd_p;     // E4M3 code of 2^8 p
  float* bwd_s;       // backward score accumulator after the mask
  float* bwd_dp;      // the D - dP accumulator
  uint8_t* bwd_p;     // Phat code and its block exponent byte
  uint8_t* bwd_ps;
  uint8_t* bwd_ds;    // dShat code and its block exponent byte
  uint8_t* bwd_dss;
  float* dq_part;     // [heads][rows][n_tiles][d]: each key tile's dQ partial times 2^pi, as converted to FP16
  int32_t n_tiles;
  float* dq_s;        // precision options' dQ pass: score accumulator after the mask
  float* dq_dp;       // dP - D as it formed it
  uint8_t* dq_ds;     // code of dS 2^e(K_j) and its (row, 32-key block) exponent byte
  uint8_t* dq_dss;
  uint8_t* fwd_ps;    // 4-bit scores: the probability code's 32-key group exponent byte
};
// Position of (query head, row) in the window's rows, or -1 outside it.
__device__ __forceinline__ int64_t dbg_row(const DebugDump& g, int h, int row) {
  if (h < g.head_lo || h >= g.head_hi || row < g.row_lo || row >= g.row_hi) return -1;
  return (int64_t)(h - g.head_lo) * (g.row_hi - g.row_lo) + (row - g.row_lo);
}
// Position of (query head, row, key) in the dump window, or -1 outside it.
__device__ __forceinline__ int64_t dbg_index(const DebugDump& g, int h, int row, int key) {
  if (h < g.head_lo || h >= g.head_hi || row < g.row_lo || row >= g.row_hi || key < g.key_lo || key >= g.key_hi)
    return -1;
  return ((int64_t)(h - g.head_lo) * (g.row_hi - g.row_lo) + (row - g.row_lo)) * (g.key_hi - g.key_lo) +
         (key - g.key_lo);
}
#endif

// int32 words of the forward's unit counters after a work list's items
constexpr int FWD_CTR_WORDS = 16;
// byte offset of those counters in a list buffer over n_docs documents of total length T
__host__ __device__ inline size_t worklist_ctr_offset(int n_docs, int T) {
  return 16 + 16 * ((size_t)((T + 127) / 128) + (size_t)n_docs);
}
// Documents of at most SMALL_DOC tokens: one token block each, so every product over one of them
// takes a single exponent per operand.  The work lists put their items last and count them in
// counter word 2; on the default 8-bit path the small-document pass takes them instead (its
// lanes form each row's products one after another, so longer documents stay on the tiles).
constexpr int SMALL_DOC = 8;
constexpr int SMALL_MAX_GROUP = 8;  // query heads per KV head the small-document pass takes
// Whether a call leaves the short documents to the small-document pass (forward and backward
// decide alike, so both passes form each score the same way): the default 8-bit path.
inline int small_docs_pass(bool precise, bool qk4, int Hq, int Hkv) {
  return (!precise && !qk4 && Hq / Hkv <= SMALL_MAX_GROUP) ? 1 : 0;
}
// Items an attention kernel walks: the whole list, or (skip_small) all but the closing items of
// the short documents.
__device__ __forceinline__ int list_walk_items(const int32_t* list, int T, int skip_small) {
  const int n = list[0];
  if (!skip_small) return n;
  return n - list[worklist_ctr_offset(list[2], T) / 4 + 2];
}

struct QTensorDev {
  const uint16_t* x;
  int64_t st, sh;   // element strides
  int32_t H;
  uint8_t* codes;
  uint8_t* scales;
  int32_t hadamard;  // rows rotated by H / sqrt(d) before quantisation
  int32_t per_token;  // one exponent per token (blocks of one token)
  uint8_t* codes4;    // optional 4-bit copy: E2M1 codes [T, H, d/2] (even channel in the low
  uint8_t* scales4;   // nibble) and one E8M0 byte per 32 channels of a token [H, T, d/32]
};

struct QuantParams {
  QTensorDev t[3];
  int32_t n_tensors;
  int32_t T, maxH;
  int32_t wg_base[4];  // first workgroup of each tensor's (window, head) units; [n_tensors]: total
  const int32_t* cu;
  int32_t n_docs;
  const uint16_t* o;  // dO pass only
  int64_t ost, osh;
  float* D;
};

struct FwdParams {
  const uint8_t *q, *k, *v, *sq, *sk, *sv;
  int32_t T, Hq, Hkv;
  float c;  // softmax_scale * log2(e), rounded once to float
  const int32_t* cu;
  int32_t n_docs;
  int32_t* list;  // written only at a dynamic list's unit counters
  uint16_t* o;
  int64_t ost, osh;
  float* lse;
  int32_t causal;  // 1: keys j <= i; 0: every key of the document
  int32_t precise;  // the precision options (per-token scales, V folded into P)
  // 4-bit scores (q4 != nullptr): E2M1 copies of Q and K [T, H, d/2] with exponents [H, T, d/32]
  const uint8_t *q4, *sq4, *k4, *sk4;
  int32_t small;  // 1: documents of at most SMALL_DOC tokens are left to the small-document pass
#ifdef FLAMIA_DEBUG_DUMP
  DebugDump dbg;
#endif
};

struct BwdParams {
  const uint8_t *q, *k, *v, *dO, *sq, *sk, *sv, *sdo;
  const float *lse, *Dv;
  int32_t T, Hq, Hkv;
  float c;              // softmax_scale * log2(e), identical to the forward's
  float softmax_scale;
  const int32_t* cu;
  int32_t n_docs;
  const int32_t* list;      // backward list (128-key tiles)
  const int32_t* fwd_list;  // forward list (256-query items), drives the dQ kernel
  uint16_t *dq, *dk, *dv;
  int64_t dqst, dqsh, dkst, dksh, dvst, dvsh;
  int32_t* status;          // workspace header: [0] status (0 once laid out, 3 when cu_seqlens do
                            // not fit the sizes the host gave), [1] key-tile chunks
  int16_t* pi;              // workspace: [Hq, T]
  int32_t* tile_base;       // workspace: first entry of each document in the key-tile tables, [n_docs + 1]
  int32_t* kv_chunk;        // workspace: chunk of each (document, key tile), [tiles]
  int64_t* kv_off;          // workspace: its first dShat block within the chunk's store, [tiles]
  int32_t* chunk_start;     // workspace: first backward-list item of each chunk, [tiles + 2]
  int32_t* counters;        // workspace: per chunk 16 counters, the next unit of the key-tile (0..7)
                            // and of the dQ pass (8..15), one per XCD partition (dynamic
                            // assignment), [16 (tiles + 2)], zeroed by the prologue
  int64_t* chunk_first;     // workspace: block prefix of each chunk's first item, [tiles + 2]
  uint8_t* ds_store;        // workspace: dShat blocks of the current chunk, per (block, query head)
                            // 8 KiB of codes and 8 exponent bytes, 8320 bytes apart
  int64_t chunk_cap;        // a chunk holds the items whose last block (per query head) falls in
                            // one span of chunk_cap blocks; with the largest item it fits the store
  int32_t max_chunks;       // chunk launches of the call (chunks past the laid-out count exit)
  int32_t n_tab;            // entries of the (document, key tile) tables
  int32_t chunk;            // the chunk a launch works on
  int16_t* pi_out;          // optional copy of pi
  int32_t causal;           // causal dQ prescale option
  int32_t causal_mask;      // 1: keys j <= i; 0: every key of the document
  int32_t precise;          // the precision options: per-token scales folded into P and dS, dQ
                            // recomputed query-stationary with row-wise dS exponents
  const uint8_t *q4, *sq4, *k4, *sk4;  // 4-bit scores: the forward's E2M1 copies (or nullptr)
  int32_t small;  // 1: documents of at most SMALL_DOC tokens are left to the small-document pass
#ifdef FLAMIA_DEBUG_DUMP
  DebugDump dbg;
#endif
};

hipError_t launch_quantize(const QuantParams& p, int d, hipStream_t s);
// In-place rotation of BF16 rows [T, H, d] (element strides) by H / sqrt(d): gradients of
// rotated operands back to the inputs' basis.
hipError_t launch_unrotate(uint16_t* x, int64_t st, int64_t sh, int T, int H, int d, hipStream_t s);
hipError_t launch_worklist(const int32_t* cu, int n_docs, int T, int kind, int n_workers, int32_t* list,
                           int32_t* ctr, hipStream_t s);
hipError_t launch_fwd(const FwdParams& p, int d, int grid, hipStream_t s);
hipError_t launch_bwd(const BwdParams& p, int d, int grid, hipStream_t s);
// The small-document pass (documents of 1 .. SMALL_DOC tokens, default 8-bit path): forward
// O / LSE and backward dQ / dK / dV of those documents' rows.  The backward's runs after the
// prologue (it reads pi).
hipError_t launch_small_fwd(const FwdParams& p, int d, hipStream_t s);
hipError_t launch_small_bwd(const BwdParams& p, int d, hipStream_t s);
// dQ under the precision options (query-stationary recomputation), after the key-tile pass.
hipError_t launch_dq_precise(const BwdParams& p, int d, int grid, hipStream_t s);

}  // namespace flamia
