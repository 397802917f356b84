/*
 * flamia_debug.h — test variant of libflamia: intermediate dumps of the attention kernels.
 *
 * Only the library built with FLAMIA_DEBUG_DUMP (the parity tests' variant) exports this entry
 * point; the product library does not.  The variant computes exactly what the product library
 * computes (its outputs are compared bit for bit in the tests) and in addition copies the
 * intermediates it forms into caller buffers, so that every E4M3 decision and every score can be
 * checked one by one: the forward and backward scores must be bit-identical and their masks the
 * same (the forward/backward consistency of "FLAMIA: FLAsh MIcroscaling Attention for Fast and
 * Causally Safe Training on Blackwell", jaehun.me review §3.3 and §4.6), and each probability and
 * dS code must be a correct rounding of the value the method defines (§3.1, §3.3).
 */
#ifndef FLAMIA_DEBUG_H
#define FLAMIA_DEBUG_H

#include <stdint.h>

#include "flamia.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Every array is DEVICE memory laid out [heads][rows][keys] over the window
 * [head_lo, head_hi) x [row_lo, row_hi) x [key_lo, key_hi): query heads, absolute packed rows and
 * keys.  Only pairs of one document that the kernel visits are written (the caller fills the
 * arrays beforehand, e.g. with NaN / 0xFF, to tell untouched entries apart).  NULL arrays are
 * skipped.  The buffers are owned by the caller and must stay alive until the calls that use them
 * have completed. */
typedef struct {
  int32_t row_lo, row_hi, key_lo, key_hi, head_lo, head_hi;
  float* fwd_s;     /* forward: score accumulator sum_c q(Q_ic) q(K_jc) 2^(e(Q_i)+e(K_j)), -inf where masked */
  float* fwd_m;     /* forward: running maximum m (score units) that the pair's probability used */
  uint8_t* fwd_p;   /* forward: E4M3 code of 2^8 2^(t_ij - m) */
  float* bwd_s;     /* backward: score accumulator, -inf where masked */
  float* bwd_dp;    /* backward: D_i - dP_ij as accumulated (precision options: times
                       2^(e(Q_i) - e(dO_i)), the key-tile pass's folded form) */
  uint8_t* bwd_p;   /* backward: Phat code (dV operand; precision options: of P 2^e(dO_i)) */
  uint8_t* bwd_ps;  /* backward: its 32x32 block exponent byte */
  uint8_t* bwd_ds;  /* backward: dShat code (dK, dQ operand; precision options: dK only, of
                       dS 2^e(Q_i)) */
  uint8_t* bwd_dss; /* backward: its 32x32 block exponent byte */
  float* dq_part;   /* backward: [heads][rows][n_tiles][d], the FP32 dQ partial of each 128-key tile
                       (counted from the document start) times 2^pi, the value converted to FP16 */
  int32_t n_tiles;  /* key tiles per row in dq_part */
  /* the precision options' query-stationary dQ pass: */
  float* dq_s;      /* its score accumulator, -inf where masked */
  float* dq_dp;     /* dP_ij - D_i as it formed it */
  uint8_t* dq_ds;   /* E4M3 code of dS_ij 2^e(K_j) (the dQ operand) */
  uint8_t* dq_dss;  /* its exponent byte, one per (row, 32-key block) */
  uint8_t* fwd_ps;  /* forward with 4-bit scores: exponent byte of the probability code's 32-key
                       group (the log-domain operand scale) */
} flamia_debug_dump;

/* Host.  Set the dump buffers used by every later flamia_fwd / flamia_bwd of this process (the
 * setting is process-wide, not per stream); NULL switches dumping off.  Errors: an empty or
 * inverted window. */
flamia_status flamia_debug_set_dump(const flamia_debug_dump* dump);

#ifdef __cplusplus
}
#endif

#endif /* FLAMIA_DEBUG_H */
