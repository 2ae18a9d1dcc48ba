/*
 * nc_ops.h -- component entry points of the d20 forward/backward library.
 *
 * Each call runs one kernel family of the training step on caller-owned
 * device buffers, so that a component can be checked against its plain
 * definition and timed on its own.  The model-level calls in nc.h are built
 * from exactly these kernels.  Conventions as in nc.h: device pointers, the
 * caller owns every buffer, the work is enqueued on `hip_stream` (NULL = the
 * default stream), nothing is allocated, host checks run first and enqueue
 * nothing on failure.  dtype is an nc_dtype; "T" below means fp32 or bf16
 * storage accordingly.  `portable` = 1 selects the plain (non-MFMA) kernels.
 */
#ifndef NC_OPS_H
#define NC_OPS_H

#include <stddef.h>
#include <stdint.h>

#include "nc.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Matrix product C[m][n] = sum_k P[m][k] * Q[n][k]   (the linear layers,
 * y = x W^T, of the speedrun walkthrough's Transformer, section Pretraining).
 *   P    T [M][K] row-major, or [K][M] when p_trans = 1
 *   Q    T [N][K] row-major, or [K][N] when q_trans = 1
 *   C    fp32 [M][N] (out_f32 = 1, written with plain stores) or T [M][N]
 *        (out_f32 = 0, rounded to T)
 *   splits  split-K factor (out_f32 = 1 only): split i sums the 64-wide k
 *        blocks [i*nb/splits, (i+1)*nb/splits), nb = K/64; splits > 1 needs
 *        `part`, fp32 scratch of splits*M*N elements, reduced in a fixed
 *        order.
 * M, N multiples of 64; K a multiple of 64, splits <= K/64.  The
 * matrix-core kernel (portable = 0, bf16) stores a rounded C in 16-byte
 * pieces: with out_f32 = 0, C must be 16-byte aligned (N is a multiple of
 * 64, so every row then is), otherwise NC_ERR_UNSUPPORTED. */
int nc_op_matmul(int32_t dtype, int32_t p_trans, int32_t q_trans, int64_t M, int64_t N, int64_t K,
                 const void* P, const void* Q, void* C, int32_t out_f32, int32_t splits, float* part,
                 int32_t portable, void* hip_stream);

/* Batched matrix products with the linear-combination epilogue, the form
 * Muon's Newton-Schulz iteration runs in (section Pretraining, optimiser
 * paragraph): for b < batch,
 *   C_b[m][n] = alpha * sum_k P_b[m][k] Q_b[n][k] + gamma * aux_b[m][n]
 * (aux = NULL: C_b = the plain product, alpha and gamma unused), all in the
 * dtype T, accumulation fp32, one rounding at the store.
 *   P_b = P + b sP   T [M][K]
 *   Q_b = Q + b sQ   T [N][K], or [K][N] when q_trans = 1
 *   C_b = C + b sC, aux_b = aux + b sAux   T [M][N]   (aux may not alias C)
 * Strides in elements, >= 0 and multiples of 8 (NC_ERR_INVALID_ARG
 * otherwise).  M, N, K multiples of 64 (NC_ERR_SHAPE); the matrix-core path
 * (portable = 0, bf16) also needs M, N multiples of 128 and a 16-byte
 * aligned C, and returns NC_ERR_UNSUPPORTED otherwise.  fp32 always takes the portable kernel.
 * sym = 1 (M == N; Newton-Schulz's X X^T and c A A + b A): the caller
 * asserts every C_b is symmetric (Q_b = P_b, and aux_b symmetric); the
 * matrix-core kernel then computes the tiles on and above the diagonal and
 * copies the rest across it.  The portable kernel computes every tile.
 * batch <= 65535. */
int nc_op_matmul_batched(int32_t dtype, int32_t q_trans, int32_t batch, int64_t M, int64_t N, int64_t K,
                         const void* P, int64_t sP, const void* Q, int64_t sQ, void* C, int64_t sC,
                         const void* aux, int64_t sAux, float alpha, float gamma, int32_t sym, int32_t portable,
                         void* hip_stream);

/* Parameter-free RMSNorm (section Pretraining: no RMSNorm parameters):
 * y = x / sqrt(mean(x^2) + eps) per row; r = the per-row factor (fp32).
 *   x, y T [rows][d];  r fp32 [rows]. */
int nc_op_rmsnorm_fwd(int32_t dtype, int64_t rows, int32_t d, float eps, const void* x, void* y, float* r,
                      void* hip_stream);

/* Its reverse mode from the saved output: dx = r * (dy - y * mean(dy * y));
 * dx_io receives dx (accumulate = 0) or dx_io + dx (accumulate = 1). */
int nc_op_rmsnorm_bwd(int32_t dtype, int64_t rows, int32_t d, const void* y, const float* r, const void* dy,
                      void* dx_io, int32_t accumulate, void* hip_stream);

/* Matrix-core throughput probe (not part of the training step): `blocks`
 * workgroups of 4 waves each issue `iters` iterations of 8 independent
 * v_mfma_f32_32x32x16_bf16 on register operands, i.e.
 * blocks * 4 * iters * 8 * 32768 FLOP with no memory traffic, so its rate
 * is the bf16 matrix throughput the chip sustains under that load (the
 * clock it holds), a measured counterpart of the 2.5 PFLOP/s dense peak.
 *   sink  fp32 [blocks * 256], one value per thread (keeps the work live).
 * iters >= 1, 1 <= blocks <= 2^20. */
int nc_op_mfma_loop(int64_t iters, int32_t blocks, float* sink, void* hip_stream);

/* Properties of HIP device `device` (hipGetDeviceProperties): compute
 * units, peak shader clock and memory clock (kHz), memory bus width (bits)
 * -- the figures the spec peaks are derived from.  Host call: launches
 * nothing, enqueues nothing. */
int nc_op_device_info(int32_t device, int32_t* compute_units, int32_t* clock_khz, int32_t* mem_clock_khz,
                      int32_t* mem_bus_bits);

/* Rotary table tab[t][i] = (cos, sin)(t * base^(-2i/Q)), fp32 [T][Q/2][2],
 * computed in fp64 and rounded once. */
int nc_op_rope_table(int32_t T, int32_t Q, float base, float* tab, void* hip_stream);

/* Causal attention forward over token-major qkv.
 *   qkv  T [B*T][3*H*Q]: per token q | k | v (q, k already rotated)
 *   o    T [B*T][H*Q];  lse fp32 [B][H][T] (log-sum-exp of the scaled scores) */
int nc_op_attention_fwd(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t Q, const void* qkv, void* o,
                        float* lse, int32_t portable, void* hip_stream);

/* Causal attention backward.
 *   dout T [B*T][H*Q];  delta fp32 [B][H][T] scratch (rowsum(dO * O));
 *   dqkv T [B*T][3*H*Q] receives dq | dk | dv; when rope_tab (fp32
 *   [T][Q/2][2]) is non-NULL, dq and dk are rotated back by -angle. */
int nc_op_attention_bwd(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t Q, const void* qkv, const void* o,
                        const void* dout, const float* lse, float* delta, void* dqkv, const float* rope_tab,
                        int32_t portable, void* hip_stream);

/* The same backward with the softmax gradient stored instead of recomputed
 * (the path nc_backward takes): delta first, then the dK/dV kernel writes
 * dS^T = (P (dP - delta))^T in bf16 -- the causal part, as 64-key x
 * 32-query pieces -- into ds_scratch, and the dQ kernel forms dQ = dS K
 * from it without recomputing S and dP (Walkthrough, Pretraining: the
 * attention of the trained model; the gradient is the method's, only the
 * order of work differs).  bf16, Q = 128, T a multiple of 64 only, else
 * NC_ERR_UNSUPPORTED.  ds_scratch: nc_op_attention_ds_bytes(B, T, H) bytes
 * of device memory the caller owns; its contents on return are unspecified.
 * Other arguments, layouts and results as nc_op_attention_bwd. */
int nc_op_attention_bwd_ds(int32_t B, int32_t T, int32_t H, int32_t Q, const void* qkv, const void* o,
                           const void* dout, const float* lse, float* delta, void* dqkv, const float* rope_tab,
                           void* ds_scratch, void* hip_stream);
/* Bytes of the dS^T scratch for B x H heads of T tokens (NC_ERR_SHAPE for
 * non-positive sizes or T not a multiple of 64). */
int64_t nc_op_attention_ds_bytes(int32_t B, int32_t T, int32_t H);

/* Embedding gather x[n] = E[idx[n]] (T [V][d] -> T [n][d]), a bitwise row
 * copy.  An id outside [0, V) reads nothing: its row of x is all NaN. */
int nc_op_embed_fwd(int32_t dtype, int64_t n, int32_t d, int32_t V, const void* E, const int32_t* idx, void* x,
                    void* hip_stream);

/* Embedding gradient, the transpose of the gather: for every v in [0, V),
 * dE[v] = (accumulate ? dE[v] : 0) + sum of g[p] over the positions p with
 * idx[p] = v (fp32 dE [V][d]; g T [n][d]; positions with idx outside
 * [0, V) contribute nothing).  Deterministic: the (id, position) pairs are
 * sorted by id (stable radix sort) and each id's rows are summed in
 * increasing position, so repeated calls give identical bits.  scratch is
 * device memory of nc_op_embed_bwd_scratch_bytes(n, d) bytes owned by the
 * caller; d a multiple of 64, 0 < n < 2^31.  Returns NC_ERR_INVALID_ARG on
 * NULL pointers, NC_ERR_SHAPE on sizes outside these limits (the scratch
 * size query returns NC_ERR_SHAPE for them too). */
int64_t nc_op_embed_bwd_scratch_bytes(int64_t n, int32_t d);
int nc_op_embed_bwd(int32_t dtype, int64_t n, int32_t d, int32_t V, const void* g, const int32_t* idx, float* dE,
                    int32_t accumulate, void* scratch, void* hip_stream);

/* Fused unembedding + log-softmax + cross-entropy, forward only:
 * ce[n] = logsumexp_v(xf[n] . U[v]) - xf[n] . U[tgt[n]] (0 where tgt < 0,
 * NaN where tgt >= V),
 * lse[n] the log-sum-exp, without storing the logits.
 *   xf T [n][d], U T [V][d], tgt int32 [n], ce, lse fp32 [n]
 *   scratch: fp32 device scratch of nc_op_head_scratch_bytes(...) bytes */
int64_t nc_op_head_scratch_bytes(int32_t dtype, int64_t n, int32_t d, int32_t V, int32_t portable);
int nc_op_head_ce_fwd(int32_t dtype, int64_t n, int32_t d, int32_t V, const void* xf, const void* U,
                      const int32_t* tgt, float* ce, float* lse, void* scratch, int32_t portable,
                      void* hip_stream);

/* The first kernel of nc_op_head_ce_fwd alone: the unembedding product with
 * its log-sum-exp epilogue, writing per-tile (max, sum of exp) partials and
 * the target logits into `scratch` (same size and layout), without the
 * combine.  One kernel launch, for timing the dominant kernel of the step. */
int nc_op_head_gemm_lse(int32_t dtype, int64_t n, int32_t d, int32_t V, const void* xf, const void* U,
                        const int32_t* tgt, void* scratch, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* NC_OPS_H */
