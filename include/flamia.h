/*
 * flamia.h — C ABI of libflamia.so: causal, packed-document attention forward and backward
 * on token-block MXFP8 operands for AMD MI355X (gfx950).
 *
 * The method is the MXFP8 path of FLAMIA ("FLAMIA: FLAsh MIcroscaling Attention for Fast and
 * Causally Safe Training on Blackwell"), as described by the jaehun.me review (cited [J]
 * below, by section) and the agihunt.info summary ([A]).
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers; `stream` is a hipStream_t (NULL = default stream).
 *    Every call only enqueues work on `stream` and returns; nothing synchronises with the host.
 *  - The caller allocates and owns every buffer, including work lists and workspaces sized by
 *    the *_bytes queries.  The library allocates no device memory and keeps no mutable global
 *    state; buffers must stay alive until the enqueued work has completed.
 *  - Packed layout: documents are consecutive token ranges of one row of T tokens, described by
 *    `cu_seqlens` (int32, n_docs + 1 entries, non-decreasing, 0 <= cu_seqlens[0],
 *    cu_seqlens[n_docs] <= T; a document k is [cu_seqlens[k], cu_seqlens[k+1]); empty documents
 *    are allowed).  Tokens outside every document are "invalid rows": O = 0, LSE = +inf,
 *    dQ = dK = dV = 0, codes 0, scale byte 0, D = 0 ([J] §3.4 "Packed documents").
 *    cu_seqlens that violate these rules give undefined results (never checked on the device,
 *    which would need a host synchronisation).
 *  - Heads: Q and dO have Hq heads, K and V have Hkv heads, Hq % Hkv == 0; query head h reads
 *    KV head h / (Hq / Hkv) (grouped-query attention, [J] §3.4 "Backward pass").
 *  - Head dimension d is 64 or 128.  BF16 tensors are [T, H, d] with element strides
 *    (stride_t, stride_h) and d contiguous.  Quantised codes are u8 [T, H, d] contiguous (OCP
 *    E4M3FN); scale tables are u8 [H, T]: one E8M0 byte (exponent + 127) per token, equal for
 *    all tokens of a 32-token document block ([J] §3.1, §3.4 "dense scale table").
 *  - LSE is float32 [Hq, T] in log2 units: LSE_i = log2 sum_j 2^(t_ij) with
 *    t_ij = softmax_scale * log2(e) * S_ij.
 *  - Errors: argument checks run synchronously on the host and return a status; a failed
 *    kernel launch returns FLAMIA_ERR_HIP.  No exception crosses the ABI.
 */
#ifndef FLAMIA_H
#define FLAMIA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FLAMIA_OK = 0,
  FLAMIA_ERR_NULL = 1,        /* a required pointer is NULL */
  FLAMIA_ERR_SHAPE = 2,       /* negative or inconsistent sizes, bad strides */
  FLAMIA_ERR_UNSUPPORTED = 3, /* d not in {64, 128}, Hq % Hkv != 0, T or n_docs beyond limits */
  FLAMIA_ERR_WORKSPACE = 4,   /* a caller buffer is smaller than its *_bytes query */
  FLAMIA_ERR_HIP = 5,         /* a HIP call or kernel launch failed */
  FLAMIA_ERR_SCRATCH = 6      /* flamia_bwd_static: the call needs more than the static scratch */
} flamia_status;

/* Host.  Static string naming a status. */
const char* flamia_status_str(flamia_status s);

/* Largest T accepted by the work-list builder and the quantiser (tokens per call). */
#define FLAMIA_MAX_T (1 << 24)
/* Largest total T accepted by flamia_build_worklist (its single-workgroup sort keeps the
 * cost histogram and the list of multi-tile documents in LDS). */
#define FLAMIA_MAX_T_WORKLIST (1 << 20)

/* ------------------------------------------------------------------------------------------
 * Work lists ([J] §3.4 "Work scheduling"; [A]).
 *
 * FLAMIA_LIST_FWD: one item per 256 consecutive queries of a document (block b covers document
 *   offsets [256b, min(256b+256, L))); cost = number of 128-key tiles it visits,
 *   ceil(min(256(b+1), L) / 128).
 * FLAMIA_LIST_BWD: one item per 128-key tile kappa of a document; cost = number of 128-query
 *   tiles at or after it, ceil((L - 128 kappa) / 128).
 * FLAMIA_LIST_FWD_NC, FLAMIA_LIST_BWD_NC: the same items for non-causal attention, where every
 *   item of a document visits (serves) all of its ceil(L / 128) key (query) tiles: that is the
 *   cost of each of them, so a document's items stay together in block order.
 * Items are enumerated by (document, block) and stably sorted by descending cost, except that
 * among equal costs the items of documents of 1 .. 8 tokens (one item of cost 1 each) come after
 * the others: they close the list.  `worker` tags them in alternating (serpentine) order over
 * n_workers: for list index i, with
 * r = i / n_workers, worker = i % n_workers if r is even, else n_workers - 1 - i % n_workers.
 * The list is built on the GPU with no host synchronisation; build it once per micro-batch
 * and reuse it for every layer.
 *
 * Schedule ([J] §3.4 "Work scheduling"): a non-causal list whose longest document is at least
 * 4 times the average document length (over all n_docs documents, empty ones included:
 * longest * n_docs >= 4 * total length) is marked for dynamic assignment; the forward then hands
 * out its units from a counter instead of walking them in serpentine order.  Causal lists are not
 * marked: the forward walks them statically, and the backward takes its units dynamically for
 * every list.
 *
 * Buffer layout: int32 header[4] = {n_items, kind, n_docs, counters}, then n_items
 * flamia_work_item; after the room for the items (16 + 16 * (ceil(T / 128) + n_docs) bytes from
 * the start), 16 int32 unit counters of the forward, cleared by the build, except word 2, which
 * holds the number of documents of 1 .. 8 tokens (the items that close the list; on the default
 * 8-bit path with at most 8 query heads per KV head, flamia_fwd and flamia_bwd leave them to a
 * small-document pass and the tile kernels walk the others).  `counters` is 0 for a list walked
 * statically, else the counters' position in int32 words from the buffer's start (the list is
 * marked dynamic); every forward on a marked list leaves words 0 and 1 cleared, and forwards
 * sharing a marked list must not overlap in time.
 * ------------------------------------------------------------------------------------------ */
typedef struct {
  int32_t doc;    /* document index */
  int32_t blk;    /* 256-query block (FWD) or 128-key tile (BWD), counted from the document start */
  int32_t cost;   /* 128-key tiles visited (FWD) or 128-query tiles served (BWD) */
  int32_t worker; /* serpentine tag over n_workers */
} flamia_work_item;

typedef enum { FLAMIA_LIST_FWD = 0, FLAMIA_LIST_BWD = 1, FLAMIA_LIST_FWD_NC = 2, FLAMIA_LIST_BWD_NC = 3 } flamia_list_kind;

/* Host.  Bytes needed for a list over n_docs documents of total length T:
 * 16 + 16 * (ceil(T / 128) + n_docs) (header and an upper bound of the items) + 64 (counters). */
size_t flamia_worklist_bytes(int32_t n_docs, int32_t T, int32_t kind);

/* Enqueue the work-list build.  cu_seqlens: device int32 [n_docs + 1].  list: device buffer of
 * list_bytes >= flamia_worklist_bytes(n_docs, T, kind).  n_workers >= 1.
 * Errors: NULL pointers, n_docs < 0, T < 0 or T > FLAMIA_MAX_T_WORKLIST, bad kind,
 * n_workers < 1, small buffer. */
flamia_status flamia_build_worklist(const int32_t* cu_seqlens, int32_t n_docs, int32_t T, int32_t kind,
                                    int32_t n_workers, void* list, size_t list_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Token-block quantiser ([J] §3.1 MXFP8 path, §3.2 round-up exponents, §3.3 D, §3.4 fusion and
 * packed documents; [A]).
 *
 * For each tensor, document k, 32-token block b counted from the document start (the last
 * block may be shorter) and head h: amax = max |x| over the block's tokens and all d channels;
 * s = the smallest integer with amax <= 448 * 2^s (clamped to [-127, 127]; amax = 0 gives
 * -127); the byte s + 127 is written for every token of the block into scales[h][t]; codes are
 * the E4M3 round-to-nearest-even of x * 2^-s (never saturating).  Each input byte is read once
 * per call.  Up to three tensors (e.g. Q, K, V, with their own head counts) share one launch.
 *
 * dO pass: with `o` non-NULL, exactly one tensor (dO, H heads) is given, and D[h][t] =
 * sum_c deq(dO_{t,h,c}) * O_{t,h,c} is also written (float32 [H, T]); deq(x) = code * 2^s, the
 * same quantised dO that the backward's dP product reads ([J] §3.3).
 *
 * Hadamard rotation ([J] §3.4 "Hadamard rotation", "Quantization fusion"): with hadamard = 1 a
 * tensor's (token, head) rows are first multiplied by H / sqrt(d), H the Sylvester Hadamard
 * matrix, in FP32 with a fixed order: butterflies for strides 1, 2, ..., d/2 in turn, a pair
 * (a, b) at that distance (a the lower index) becoming (a + b, a - b), then the multiply by
 * RN32(1 / sqrt(d)); the block rule above then runs on those FP32 values.  Meant for Q and K
 * together (scores are unchanged in exact arithmetic); the backward then rotates dQ and dK back
 * (flamia_bwd_args.hadamard).  Not with the dO pass.
 *
 * Per-token scales ([J] §3.2, the precision options): with per_token = 1 every token of a
 * document is its own block, so its exponent and codes depend on that token alone (also for the
 * dO pass).
 *
 * 4-bit copy for the scores ([J] §3.1 "Mixed NVFP4/FP8 path", as MXFP4, the microscaling
 * analogue of the pages' NVFP4): with mx4_codes / mx4_scales given, the same pass also writes
 * E2M1 codes (values 0, 0.5, 1, 1.5, 2, 3, 4, 6; round to nearest even, the sign kept on zero)
 * with one round-up E8M0 exponent per 32 consecutive channels of one token (smallest s with
 * amax <= 6 2^s, amax over the FP32 values the 8-bit codes are taken from, rotated when
 * hadamard = 1).  It feeds only the score product (flamia_fwd_args.q4/k4 and the backward's
 * recomputation); each token's copy depends on that token alone.  Rows outside every document:
 * codes and exponent bytes 0.
 * ------------------------------------------------------------------------------------------ */
typedef struct {
  const void* x;              /* bf16 [T, H, d], element strides below, d contiguous */
  int64_t stride_t, stride_h; /* in elements */
  int32_t H;                  /* heads of this tensor */
  uint8_t* codes;             /* out: u8 [T, H, d] contiguous */
  uint8_t* scales;            /* out: u8 [H, T] */
  int32_t hadamard;           /* 1: rotate each row by H / sqrt(d) first (Q and K); 0: plain */
  int32_t per_token;          /* 1: one exponent per token (blocks of one token; the precision
                                 options, with flamia_fwd_args.precise / flamia_bwd_args.precise) */
  uint8_t* mx4_codes;         /* optional out (both or neither): the 4-bit copy for the score
                                 product, E2M1 codes u8 [T, H, d/2], two per byte, the even
                                 channel in the low nibble, 4-byte aligned */
  uint8_t* mx4_scales;        /* optional out: its exponents u8 [H, T, d/32] */
} flamia_qtensor;

/* Errors: NULL pointers, n_tensors not in [1, 3] (1 with `o`), H < 1, T < 0 or > FLAMIA_MAX_T,
 * d not in {64, 128}, n_docs < 0, D NULL when o is given, hadamard or a 4-bit copy with o
 * (UNSUPPORTED), only one of mx4_codes / mx4_scales (NULL). */
flamia_status flamia_quantize(const flamia_qtensor* tensors, int32_t n_tensors, int32_t T, int32_t d,
                              const int32_t* cu_seqlens, int32_t n_docs, const void* o, int64_t o_stride_t,
                              int64_t o_stride_h, float* D, void* stream);

/* ------------------------------------------------------------------------------------------
 * Forward ([J] §1.2, §3.1, §3.4; [A]).
 *
 * For each query row i of document k (offset r) and query head h (KV head g):
 *   t_ij = softmax_scale * log2(e) * 2^(e(Q_i) + e(K_j)) * sum_c q(Q_ic) q(K_jc)   (j <= i)
 * 128-key tiles counted from the document start are visited from the diagonal tile down to
 * tile 0, the running max m updated once per tile; per tile p_j = 2^(t_ij - m),
 * l = 2^(m_old - m) l + sum p_j, and the P operand is E4M3_RNE(2^8 p_j) with scale 2^-8.
 * O_i = BF16(acc / l) is written into the packed output; LSE_i = m + log2 l.
 * Work comes from a FLAMIA_LIST_FWD list built for the same cu_seqlens, n_docs and T; (item,
 * head) units are spread over a persistent grid in list order, statically (serpentine), or, for a
 * list marked dynamic, from the list's counter.  Invalid rows get O = 0 and LSE = +inf.
 * Non-causal attention (non_causal = 1; [J] §3.4 "Backward pass", §4.8): every key of the
 * row's document is visible; the key tiles are visited from the document's last one down to
 * tile 0.  Batched attention is the special case of documents of equal length.  Either list kind
 * gives the same results (the items are the same); FLAMIA_LIST_FWD_NC orders them by the
 * non-causal costs.
 * ------------------------------------------------------------------------------------------ */
typedef struct {
  const uint8_t *q, *k, *v;       /* codes: q [T, Hq, d]; k, v [T, Hkv, d] */
  const uint8_t *sq, *sk, *sv;    /* scale tables: sq [Hq, T]; sk, sv [Hkv, T] */
  int32_t T, Hq, Hkv, d;
  float softmax_scale;            /* <= 0 selects 1 / sqrt(d) */
  const int32_t* cu_seqlens;      /* [n_docs + 1] */
  int32_t n_docs;
  void* fwd_list;                 /* FLAMIA_LIST_FWD list for cu_seqlens (a list marked dynamic
                                     is written: its unit counters, cleared again by the call) */
  void* o;                        /* out: bf16 [T, Hq, d], element strides below */
  int64_t o_stride_t, o_stride_h;
  float* lse;                     /* out: float32 [Hq, T], log2 units */
  int32_t non_causal;             /* 0: causal (j <= i); 1: every key of the document */
  int32_t precise;                /* 1: the precision options ([J] §3.2): Q, K, V quantised with
                                     per_token = 1; V's exponent is folded into the probability
                                     operand, E4M3(2^(8 + e(V_j) - v_i) p_ij) with operand scale
                                     2^(v_i - 8), v_i the largest V exponent among the keys row i
                                     has visited so far (at least -119), and V enters P V with its
                                     bare codes, so no later token changes row i.  Causal only
                                     (non_causal = 1 is FLAMIA_ERR_UNSUPPORTED). */
  const uint8_t *q4, *sq4;        /* optional (all four or none): 4-bit scores ([J] §3.1 "Mixed
                                     NVFP4/FP8 path", §3.4 "Softmax throughput"): the score
                                     product takes these E2M1 copies from flamia_quantize (codes
                                     [T, H, d/2], 16-byte aligned; exponents [H, T, d/32],
                                     4-byte aligned) instead of q, k, and the P operand is
                                     quantised in the log domain: per row and tile, each 32-key
                                     group gets the round-up E8M0 exponent e of its largest p
                                     (taken from its largest score) and codes E4M3_RNE(p 2^-e)
                                     with operand scale 2^e; l sums the unrounded p.  Not with
                                     precise (FLAMIA_ERR_UNSUPPORTED). */
  const uint8_t *k4, *sk4;
} flamia_fwd_args;

/* Errors: NULL pointers, sizes, d, head ratio.  On the default 8-bit path (neither precise nor the
 * 4-bit scores) with at most 8 query heads per KV head, documents of 1 .. 8 tokens (the items that
 * close the work list) go through a small-document pass launched by this call; flamia_bwd decides
 * alike, so both passes form each score the same way. */
flamia_status flamia_fwd(const flamia_fwd_args* args, void* stream);

/* ------------------------------------------------------------------------------------------
 * Backward ([J] §1.2, §3.1, §3.2, §3.3, §3.4 "Backward pass"; [A]).
 *
 * Recomputes t_ij bit-identically to the forward (same codes, scales, matrix instruction and
 * score scale), P_ij = 2^(t_ij - LSE_i), dP_ij = deq(dO_i) . deq(V_j), dS_ij = P_ij (dP_ij - D_i).
 * The P and dS operands of the gradient products are E4M3 with one round-up E8M0 exponent per
 * 32x32 block (query block x key block, both counted from the document start):
 *   dV_j = sum_{h in group} sum_i deq(Phat_ij) deq(dO_i)
 *   dK_j = softmax_scale * sum_{h in group} sum_i deq(dShat_ij) deq(Q_i)
 *   dQ_i = BF16(softmax_scale * 2^-pi_i * acc16_i), acc16 the FP16 sum, over 128-key tiles in
 *          ascending order, of FP16(2^pi_i * sum_{j in tile} deq(dShat_ij) deq(K_j)).
 * The power-of-two prescale pi ([J] §3.2): with C_d = ceil(log2(2 d 448^3)),
 *   pi_i = clamp(15 - C_d - E_i, -64, 64), E_i = e(dO) + e(V) + e(K) with
 *   causal_dq_scale = 0: maxima over every token of the call (per query head);
 *   causal_dq_scale = 1: e(dO_i) of the row's own block and maxima of e(V), e(K) over the row's
 *                        document up to and including its own block, so no later token
 *                        changes the rounding of earlier rows.
 * Reduction of dQ: a document with a single 128-key tile has one contribution per row, which
 * the key-tile pass turns into dQ directly.  For longer documents the key-tile pass stores
 * the dShat codes and exponents of every visited (64-query tile, key tile, query head) in the
 * workspace's store, and a query-tile pass (driven by the forward work list) reads them back
 * in ascending key-tile order and keeps acc16 in registers.  When the store cannot hold every
 * block of the call, the backward list is cut into consecutive chunks that each fit (laid out
 * on the GPU from cu_seqlens, no host synchronisation); each chunk runs both passes, and rows
 * whose key tiles continue in a later chunk leave their FP16 sums in the dQ output rows until
 * then.  The backward list visits each document's key tiles in ascending order, so the sums
 * are the same whatever the chunking.  The order of every sum is fixed, so results are
 * bit-reproducible, and no workgroup waits for another.
 * Work comes from a FLAMIA_LIST_BWD list (key-tile pass; each (item, KV head) unit runs all
 * query heads of its group, so dK and dV are written once) and a FLAMIA_LIST_FWD list (dQ
 * pass), both built for the same cu_seqlens.  Both passes assign their units dynamically
 * ([J] §3.4 "Work scheduling"): a workgroup takes the next unit of the list from a counter in
 * the workspace (zeroed by the call itself) when it finishes one, so units run in list order
 * (descending cost) on whichever compute unit is free.
 * ------------------------------------------------------------------------------------------ */
typedef struct {
  const uint8_t *q, *k, *v, *dO;      /* codes (dO: [T, Hq, d], from the dO quantiser pass) */
  const uint8_t *sq, *sk, *sv, *sdO;  /* scale tables */
  const float *lse, *D;               /* forward LSE and the dO pass's D, float32 [Hq, T] */
  int32_t T, Hq, Hkv, d;
  float softmax_scale;                /* must equal the forward's (<= 0: 1 / sqrt(d)) */
  const int32_t* cu_seqlens;
  int32_t n_docs;
  const void* fwd_list;               /* FLAMIA_LIST_FWD list for cu_seqlens */
  const void* bwd_list;               /* FLAMIA_LIST_BWD list for cu_seqlens */
  void *dq, *dk, *dv;                 /* out: bf16; dq [T, Hq, d], dk, dv [T, Hkv, d] */
  int64_t dq_stride_t, dq_stride_h, dk_stride_t, dk_stride_h, dv_stride_t, dv_stride_h;
  void* workspace;                    /* at least flamia_bwd_workspace_bytes(n_docs, T, Hq, d, 0)
                                         bytes, 256-byte aligned, any contents; every byte beyond
                                         that enlarges the dShat store (fewer, larger chunks) */
  size_t workspace_bytes;
  int32_t causal_dq_scale;            /* 0: sequence-wide prescale (default); 1: causal */
  int16_t* dq_exp_out;                /* optional out: pi as int16 [Hq, T] (0 on invalid rows) */
  int32_t non_causal;                 /* as in the forward (must match it); the non-causal
                                         backward visits every (query tile, key tile) pair of a
                                         document and takes the sequence-wide prescale only
                                         (causal_dq_scale = 1 is FLAMIA_ERR_UNSUPPORTED) */
  int32_t hadamard;                   /* 1: Q and K were quantised with hadamard = 1; the
                                         gradients of the rotated operands, as BF16 rows, are
                                         rotated back in place (same FP32 arithmetic as the
                                         quantiser, BF16 round to nearest even), so dq and dk are
                                         the gradients of the unrotated inputs.  Needs dq, dk
                                         16-byte aligned and their strides multiples of 8. */
  int32_t precise;                    /* 1: the precision options ([J] §3.2), causal only
                                         (non_causal = 1 is FLAMIA_ERR_UNSUPPORTED): Q, K, V and
                                         dO quantised with per_token = 1, the forward run with
                                         precise = 1.  Each gradient product takes the operand it
                                         contracts over with bare codes and that operand's
                                         exponent moves into the quantised one before rounding:
                                           dV_j = sum_i Phat''_ij q(dO_i),  P'' = P 2^e(dO_i),
                                           dK_j = softmax_scale sum_i dShat''_ij q(Q_i),
                                                  dS'' = dS 2^e(Q_i)  (32 x 32 block exponents),
                                           dQ_i as above from dShat'_ij q(K_j), dS' = dS 2^e(K_j)
                                                  with one exponent per (row i, 32-key block);
                                         pi_i takes the maxima of e(V), e(K) up to row i itself
                                         (causal_dq_scale is implied).  No later token then
                                         changes an earlier row's dQ, nor (through shared
                                         exponents) an earlier key's dK, dV.  dQ comes from a
                                         query-stationary pass that recomputes S, dP and dS';
                                         nothing is stored, so the call runs as one chunk in
                                         any workspace the default accepts. */
  const uint8_t *q4, *sq4, *k4, *sk4; /* optional (all four or none, as given to the forward):
                                         the recomputed scores take these 4-bit copies, bit for
                                         bit the forward's; dK, dQ keep the 8-bit q, k.  Not with
                                         precise (FLAMIA_ERR_UNSUPPORTED). */
  int32_t max_doc_len;                /* optional (<= 0: not given): the length of the longest
                                         document, or any larger number.  The key-tile and dQ
                                         passes are launched once per chunk that the documents
                                         could need, counted without the lengths (no copy of
                                         cu_seqlens reaches the host): for any documents of total
                                         length T, or with this bound for documents no longer
                                         than max_doc_len (sum of L^2 <= max_doc_len * T), which
                                         is most often one chunk and saves the launches that
                                         would find nothing to do.  A call whose documents need
                                         more chunks than were launched (a bound below the longest
                                         document can cause it) sets status word 3 in the
                                         workspace, and its gradient passes do not run. */
} flamia_bwd_args;

/* Host.  Backward workspace for n_docs documents of total length T: a header, pi [Hq, T], the
 * chunk layout tables (n_docs + ceil(T / 128) entries) and a dShat store of about store_budget
 * bytes, clamped between twice the largest single key tile (ceil(T / 64) blocks of 8320 bytes
 * per query head: store_budget = 0 gives the smallest workspace the backward accepts) and what
 * one chunk of any documents of total length T needs.  Depends on the sizes only, never on the
 * document lengths, so sizing needs no copy of cu_seqlens on the host.  A smaller store runs the
 * backward in more chunks (more launches, the FP16 dQ sums carried between them).  Returns 0 on
 * bad arguments. */
size_t flamia_bwd_workspace_bytes(int32_t n_docs, int32_t T, int32_t Hq, int32_t d, size_t store_budget);

/* Host.  Workspace with which a backward over these documents runs as one chunk (the fastest):
 * the store holds every dShat block of the call (non_causal != 0: of the non-causal backward,
 * which stores every (query tile, key tile) pair).  For callers that already hold the document
 * lengths on the host (cu_seqlens_host: HOST int32 [n_docs + 1]; NULL only when n_docs == 0).
 * Returns 0 on bad arguments. */
size_t flamia_bwd_workspace_bytes_for(const int32_t* cu_seqlens_host, int32_t n_docs, int32_t T, int32_t Hq,
                                      int32_t d, int32_t non_causal);

/* Errors: NULL pointers, sizes, d, head ratio, a workspace smaller than
 * flamia_bwd_workspace_bytes(n_docs, T, Hq, d, 0) (FLAMIA_ERR_WORKSPACE).  The status word (first
 * int32 of the workspace) is 0 once the backward has run, 3 when the documents could not be laid
 * out in the launched chunks (inconsistent cu_seqlens, or max_doc_len below the longest
 * document); then the gradient passes do not run.  Documents of 1 .. 8 tokens take the
 * small-document pass under the same condition as in flamia_fwd. */
flamia_status flamia_bwd(const flamia_bwd_args* args, void* stream);

/* ------------------------------------------------------------------------------------------
 * Backward that allocates nothing, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The same as flamia_bwd, except that args->workspace and args->workspace_bytes are ignored: the
 * workspace is a static device array of FLAMIA_STATIC_SCRATCH_BYTES held by the library on every
 * GPU it runs on until the process ends (its address on the current device is looked up on the
 * first call there).  All of it becomes the backward's workspace, so calls whose smallest
 * workspace, flamia_bwd_workspace_bytes(n_docs, T, Hq, d, 0), exceeds it are rejected with
 * FLAMIA_ERR_SCRATCH (roughly T * Hq up to 2^17 at T = 16384, Hq = 8); larger calls need
 * flamia_bwd.  No hipMalloc, hipFree or allocating library call is made.  The array's contents
 * on entry do not matter (the backward writes everything it reads).  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be serialised by the caller.  Errors: as flamia_bwd, plus
 * FLAMIA_ERR_SCRATCH.
 * ------------------------------------------------------------------------------------------ */
#define FLAMIA_STATIC_SCRATCH_BYTES (64u << 20)
flamia_status flamia_bwd_static(const flamia_bwd_args* args, void* stream);

/* Host.  Number of compute units of the current device, the persistent grid used by
 * flamia_fwd / flamia_bwd (one workgroup per compute unit). */
int32_t flamia_num_workers(void);

#ifdef __cplusplus
}
#endif

#endif /* FLAMIA_H */
