/*
 * cakv_diag.h -- measurement aid of libcakv.so (AMD Instinct MI355X, gfx950).
 *
 * Not an operation of the method: it measures the bf16 matrix-core rate the
 * chip sustains, the practical ceiling against which the forward kernel's
 * rate is read beside the nominal dense peak. The matrix cores' power draw
 * depends on the operand bits, and under the board's power limit the clock
 * settles lower for random operands than for zeros.
 *
 * Conventions as in cakv.h (device pointers owned by the caller, nothing
 * allocated, work enqueued on `stream`, status returned, message in
 * cakv_last_error()).
 */
#ifndef CAKV_DIAG_H
#define CAKV_DIAG_H

#include "cakv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Workgroups (4 waves each) of one cakv_diag_mfma_burn launch. */
#define CAKV_DIAG_MFMA_WG 2048

/*
 * One kernel in which every wave issues back-to-back v_mfma_f32_32x32x16_bf16
 * products: `iters` rounds of 16 products into 4 independent accumulators,
 * the A operand rotating through 8 register fragments and B through 4.
 * Operands are pseudo-random bf16 values in [-1, 1) (zero_operands == 0) or
 * zeros (zero_operands != 0). No memory is touched in the timed loop.
 * FLOPs per launch = CAKV_DIAG_MFMA_WG * 4 * iters * 16 * 32768; the caller
 * times the launch (events on `stream`).
 * sink: device pointer to at least one float; written only if the products
 *       add up to exactly 1234.5 (it keeps them from being optimised away).
 * Errors: CAKV_ERR_NULL (sink), CAKV_ERR_SHAPE (iters < 0 or > 2^31 - 1),
 *         CAKV_ERR_HIP. iters == 0 returns CAKV_OK and launches nothing.
 */
cakv_status cakv_diag_mfma_burn(int zero_operands, int64_t iters, float* sink, void* stream);

/*
 * Ordering check (a test aid, not an operation of the method). Every kernel
 * of the library maps its workgroup id to a unit of work (a query tile, a
 * key tile, a key-range part, a decode split) and no workgroup waits for
 * another, so every result must be the same whichever workgroup takes which
 * unit. This sets, for the whole process, a permutation that the launchers
 * apply to those logical ids from the next call on: order 0 (the default)
 * none, 1 a scrambled order, 2 the reversed order. Results must stay
 * bit-identical; order 1 and 2 give up the XCD-aware placement, so they are
 * for tests only. Not synchronised with calls in flight on other threads.
 * Errors: CAKV_ERR_RANGE for an order outside [0, 2].
 */
cakv_status cakv_diag_set_workgroup_order(int order);

#ifdef __cplusplus
}
#endif

#endif /* CAKV_DIAG_H */
