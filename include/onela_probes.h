/*
 * onela_probes.h - measurement probes used by bench.py (libonela_probes.so).
 *
 * Not part of the decode path. They measure, on the box at hand, what the
 * step kernel is compared against: the HBM rate of a plain device copy, the
 * bf16 matrix-core rate of a register-only MFMA loop, and the rate of the
 * shared-state projection P = S0 [k q] (OneLA review, evolve.pub, "Scope &
 * Claims": the state enters a step only through S0 k_t and S0 q_t) run on its
 * own, with the step kernel's tile shapes and split-bf16 S0, so that its
 * MFMA efficiency can be stated apart from the HBM-bound fused step.
 *
 * All pointers are device memory owned by the caller; every call is
 * asynchronous on hip_stream (NULL = the null stream) and returns 0, -1 for
 * bad arguments, or -5 when the launch fails. None allocates.
 */
#ifndef ONELA_PROBES_H
#define ONELA_PROBES_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[i] = src[i] for n16 16-byte elements (both 16-byte aligned). */
int32_t onela_probe_copy(const void* src, void* dst, size_t n16, void* hip_stream);

/* n_wg workgroups of 8 waves; every wave issues iters x 8 independent
 * 16x16x32 bf16 MFMAs on register operands (16384 flops each) and writes one
 * float per lane to out [n_wg * 512] so that nothing is dead code. */
int32_t onela_probe_mfma(float* out, int32_t n_wg, int32_t iters, void* hip_stream);

/* S0 float32 [n_pairs][128][128] -> planes bf16 [n_pairs][2][128*128]: the
 * hi plane (rne(S0)) then the lo plane (rne(S0 - hi)) of each pair, both in
 * MFMA A-fragment order: 16-byte fragment f = (w*4 + kk)*64 + lane holds
 * S0[16w + lane%16][32kk + 8(lane/16) + 0..7]. This is the form the step
 * kernel holds the shared state in; planes feeds onela_probe_projection.
 * Both pointers 16-byte aligned. */
int32_t onela_probe_planes(const float* S0, uint16_t* planes, int32_t n_pairs, void* hip_stream);

/* For every (request, head) pair p = r*H + h: colsum[p][i] = sum over beams b
 * of (S0_s k_b)[i] + (S0_s q_b)[i] with s the pair whose operands p reads,
 * computed as the step kernel computes its projection (S0 as bf16 hi + lo
 * A-fragments loaded from the planes, 16x16x32 MFMA tiles, k and q staged
 * through LDS 64 beams at a time). s = p when resident_pairs = 0; otherwise
 * s = p mod resident_pairs, so that the operands of only resident_pairs pairs
 * are read and stay in the L2 caches (the projection's matrix-core rate
 * without the memory's limit). planes: as written by onela_probe_planes,
 * [n_req*H] pairs; k, q: bf16 [n_req*W][H][128] (16-byte aligned); colsum:
 * float32 [n_req*H][128]. d_k = d_v = 128; W a multiple of 64;
 * 0 <= resident_pairs <= n_req*H. */
int32_t onela_probe_projection(const uint16_t* planes, const uint16_t* k, const uint16_t* q, int32_t n_req,
                               int32_t H, int32_t W, int32_t resident_pairs, float* colsum, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* ONELA_PROBES_H */
