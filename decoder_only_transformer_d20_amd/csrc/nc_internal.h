// Internal declarations shared by the host library and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace nc {

// ---------------------------------------------------------------------------
// storage types
// ---------------------------------------------------------------------------
struct bf16 {
  uint16_t x;
};

__host__ __device__ inline float to_f32(float v) { return v; }
__host__ __device__ inline float to_f32(bf16 v) {
  uint32_t u = (uint32_t)v.x << 16;
  float f;
  __builtin_memcpy(&f, &u, 4);
  return f;
}

template <typename T> __host__ __device__ inline T from_f32(float f);
template <> __host__ __device__ inline float from_f32<float>(float f) { return f; }
// round to nearest, ties to even; NaN stays a quiet NaN
template <> __host__ __device__ inline bf16 from_f32<bf16>(float f) {
  uint32_t u;
  __builtin_memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return bf16{(uint16_t)0x7fc0};
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16{(uint16_t)(u >> 16)};
}

// ---------------------------------------------------------------------------
// GEMM:  C[m][n] = sum_k P[m][k] * Q[n][k]       (m < M, n < N, k < K)
// P is stored [M][K] (p_trans = 0) or [K][M] (p_trans = 1); likewise Q is
// [N][K] or [K][N].  The epilogue decides what is written.
// ---------------------------------------------------------------------------
enum Epi {
  EPI_STORE = 0,     // C(T) = acc
  EPI_ROPE = 1,      // C(T) = acc, columns < rope_cols rotated in adjacent pairs
  EPI_RESID = 2,     // C(T) = aux(T) + acc            (aux may alias C)
  EPI_DRELU2 = 3,    // C(T) = acc * 2 sqrt(aux(T)), aux = relu(h)^2 (so the factor is 2 relu(h))
  EPI_F32 = 4,       // C(f32) = (beta ? C : 0) + acc; with splits > 1, partials
  EPI_LSE = 5,       // per-row (max, sum exp) of the N-tile -> lse_part; z[tgt] -> ztgt
  EPI_DZ = 6,        // C(T) = (exp(acc - lse[m]) - [n == tgt[m]]) * inv_nvalid
  EPI_RELU2 = 7,     // C(T) = relu(acc)^2
  EPI_AXPBY = 8,     // C(T) = ep_alpha * acc + ep_gamma * aux(T)   (aux may not alias C)
  EPI_LSEZ = 9,      // EPI_LSE, and C(T) = acc - (row max of the N-tile): the logits kept
                     // for the backward, relative to their tile's maximum (lse_part[.].x)
};

struct GemmDesc {
  int M, N, K;
  const void* P; int64_t ldp; int p_trans;
  const void* Q; int64_t ldq; int q_trans;
  int epi;
  void* C; int64_t ldc;
  const void* aux; int64_t ldaux;
  int beta;                 // EPI_F32: add to C
  int splits;               // EPI_F32: split-K count (partials + reduce when > 1); split i
                            // covers the 64-wide k blocks [i*nb/splits, (i+1)*nb/splits), nb = K/64
  float* part;              // EPI_F32 split-K partials [splits][M][N]
  // EPI_ROPE
  const float2* rope;       // [T][head_dim/2] (cos, sin)
  int rope_T, rope_cols, head_dim;
  // EPI_LSE / EPI_DZ
  const int32_t* tgt;       // [M]
  float2* lse_part;         // [M][lse_stride]
  int lse_stride;           // number of N-tiles
  float* ztgt;              // [M]
  const float* lse;         // [M]
  const float* row_scale;   // [M] factor of row m's dz: w_m / n_valid, 0 for an ignored target
  // EPI_AXPBY
  float ep_alpha, ep_gamma;
  // batched products (EPI_STORE / EPI_AXPBY, splits == 1): item b reads
  // P + b sP, Q + b sQ, aux + b sAux and writes C + b sC (elements);
  // batch 0 or 1 is a single product
  int batch;
  int64_t sP, sQ, sC, sAux;
  // sym = 1 (matrix-core kernel, M == N, square tiles, STORE / AXPBY): the
  // result is known to be symmetric (P Q^T with Q = P, or a linear
  // combination of such products); only the tiles on and above the
  // diagonal are computed and the rest is mirrored from them.  Other
  // kernels compute every tile.
  int sym;
};

// ---------------------------------------------------------------------------
// attention on token-major qkv: row (b*T + t) holds [q | k | v], each H*Q
// ---------------------------------------------------------------------------
struct AttnDesc {
  int B, T, H, Q;
  const void* qkv;          // [B*T][3*H*Q], q and k already rotated
  const void* o;            // [B*T][H*Q]
  void* o_out;
  float* lse;               // [B][H][T]
  const void* dout;         // [B*T][H*Q]
  float* delta;             // [B][H][T] rowsum(dO * O)
  void* dqkv;               // [B*T][3*H*Q]
  const float2* rope;       // inverse rotation of dq, dk on store; NULL = none
  // bf16 dS^T tiles (attn_ds_elems), written by the dK/dV kernel and read
  // by the dQ kernel; NULL = the dQ kernel recomputes S and dP instead
  void* ds;
};
// elements of the dS^T tile buffer for B x H heads of T tokens: per head,
// query block qb (128 queries) holds 2 (qb + 1) tiles of 64 keys x 128
// queries (the causal part, whole 64-key tiles)
inline int64_t attn_ds_elems(int64_t B, int64_t T, int64_t H) {
  const int64_t nq = (T + 127) / 128;
  return B * H * nq * (nq + 1) * 64 * 128;
}

// ---------------------------------------------------------------------------
// launchers (all enqueue on `s`; return hipError_t of the launch)
// ---------------------------------------------------------------------------
template <typename T> hipError_t gemm_portable(const GemmDesc& g, hipStream_t s);
hipError_t gemm_mfma_bf16(const GemmDesc& g, hipStream_t s);          // product + split-K reduce
hipError_t gemm_mfma_bf16_product(const GemmDesc& g, hipStream_t s);  // the product kernel alone
bool gemm_mfma_supported(const GemmDesc& g);
int gemm_mfma_tile_m(const GemmDesc& g);   // tile sizes the MFMA GEMM picks for a product
int gemm_mfma_tile_n(const GemmDesc& g);
hipError_t splitk_reduce(const float* part, int splits, int64_t n, float* out, int beta, hipStream_t s);
// blocks x 4 waves x iters x 8 products of 32x32x16 (bf16) on registers only
hipError_t mfma_loop(int64_t iters, int blocks, float* sink, hipStream_t s);

template <typename T> hipError_t attn_fwd_portable(const AttnDesc& a, hipStream_t s);
template <typename T> hipError_t attn_bwd_portable(const AttnDesc& a, hipStream_t s);
bool attn_mfma_supported(const AttnDesc& a);   // head dim 128, T % 64 == 0
hipError_t attn_fwd_mfma(const AttnDesc& a, hipStream_t s);
hipError_t attn_bwd_mfma(const AttnDesc& a, hipStream_t s);
template <typename T> hipError_t attn_delta(const AttnDesc& a, hipStream_t s);

// x[n] = E[idx[n]]; an id outside [0, V) gives a NaN row (no read)
template <typename T> hipError_t embed_fwd(const T* E, const int32_t* idx, T* x, int64_t n, int d, int V,
                                           hipStream_t s);
// dE [V][d] (accumulate ? += : =) per-id sums of g rows, deterministic (sort
// by id, ordered sums); scratch of embed_bwd_scratch_bytes(n, d) bytes
int64_t embed_bwd_scratch_bytes(int64_t n, int d);
template <typename T> hipError_t embed_bwd(const T* g, const int32_t* idx, float* dE, int64_t n, int d, int V,
                                           int accumulate, void* scratch, hipStream_t s);
template <typename T> hipError_t rmsnorm_fwd(const T* x, T* y, float* r, int64_t rows, int d, float eps, hipStream_t s);
template <typename T> hipError_t rmsnorm_bwd(const T* y, const float* r, const T* dy, T* dx_io, int64_t rows, int d,
                                            int accumulate, hipStream_t s);
hipError_t rope_table(float2* tab, int T, int Q, float base, hipStream_t s);
// rows t0 .. t0+T-1 of the same table (same fp64 angles)
hipError_t rope_table_at(float2* tab, int t0, int T, int Q, float base, hipStream_t s);
// ce = 0 for an ignored target, NaN for a target >= V
hipError_t ce_combine(const float2* part, int nblk, const float* ztgt, const int32_t* tgt,
                      float* lse, float* ce, int64_t rows, int V, hipStream_t s);
// dz [rows][V] = (softmax(z) - onehot(tgt)) * rs from z [rows][V] written by
// an EPI_LSEZ product (z relative to its tile's row max, the tile width
// tile_w and per-tile maxima from part [rows][nblk]); the target column is
// formed from the fp32 target logit ztgt
template <typename T>
hipError_t dz_from_logits(const T* z, T* dz, int64_t rows, int V, int tile_w, const float2* part, int nblk,
                          const float* ztgt, const int32_t* tgt, const float* lse, const float* rs, hipStream_t s);
hipError_t count_valid(const int32_t* tgt, int64_t n, float* inv_nvalid, hipStream_t s);
// out[i] = tgt[i] >= 0 ? *inv_nvalid * (w ? w[i] : 1) : 0 (NaN for tgt[i] >= V)
hipError_t row_scale(const int32_t* tgt, const float* w, const float* inv_nvalid, int64_t n, int V, float* out,
                     hipStream_t s);
// out = {sum over valid targets of w ce, that sum / n_valid}, fp64, fixed order
hipError_t weighted_loss(const float* ce, const int32_t* tgt, const float* w, int64_t n, double* out, hipStream_t s);
hipError_t loss_bpb(const float* ce, const int32_t* tgt, const int32_t* bytes, int64_t n, int V, double* out,
                    hipStream_t s);
hipError_t fill_f32(float* p, int64_t n, float v, hipStream_t s);
// out [cols][rows] = transpose of in [rows][cols]; rows, cols multiples of 8
hipError_t transpose_bf16(const bf16* in, int64_t rows, int64_t cols, bf16* out, hipStream_t s);
hipError_t copy_bytes(void* dst, const void* src, size_t n, hipStream_t s);

// ---------------------------------------------------------------------------
// KV-cache inference
// ---------------------------------------------------------------------------
constexpr int kMaxDecodeBatch = 16;   // sequences per decode step
// y[b][n] = epi(sum_k x[b][k] W[n][k]), b < nb: EPI_STORE, EPI_ROPE (pairs of
// columns < rope_cols rotated by the angles in rope[head_dim/2], one
// position), EPI_RESID (+ aux[b][n], aux may be y), EPI_RELU2, EPI_F32 (fp32 y)
struct GemvDesc {
  int nb, N, K;
  const void* W;            // [N][K]
  const void* x; int64_t ldx;
  void* y; int64_t ldy;
  const void* aux;
  const float2* rope; int rope_cols, head_dim;
  // EPI_ROPE on qkv: when kv_K is set, columns [d, 2d) also go to
  // kv_K[b][pos][:] and [2d, 3d) to kv_V[b][pos][:] (seq stride in elements)
  void* kv_K; void* kv_V; int64_t kv_seq_stride; int kv_d, kv_pos;
  // norm = 1: x is the raw residual stream and the product is taken of
  // RMSNorm(x) = x / sqrt(mean(x^2) + norm_eps), the row scale formed in the
  // same pass (EPI_ROPE, EPI_RELU2 and EPI_F32 only)
  int norm;
  float norm_eps;
};
template <typename T> hipError_t gemv(const GemvDesc& g, int epi, hipStream_t s);
// K, V [batch][max_len][d] of one layer: seq_stride = max_len * d
template <typename T> hipError_t kv_append(const T* qkv, int nb, int d, T* K, T* V, int64_t seq_stride, int pos,
                                           hipStream_t s);
template <typename T> hipError_t kv_prefill(const T* qkv, int len, int d, int nb, T* K, T* V, int64_t seq_stride,
                                            hipStream_t s);
struct AttnDecodeDesc {
  int H, Q, L, nchunks;     // L keys (positions 0 .. L-1) per sequence
  const void* qkv;          // [nb][3 H Q], q rotated
  const void* K; const void* V; int64_t seq_stride;
  float scale_log2;         // log2(e) / sqrt(Q)
  float* part;              // [nb][H][nchunks][2 + Q]
  void* o;                  // [nb][H Q]
};
int attn_decode_chunks(int L);
// next token per row of logits [n][V] (nc_sample)
hipError_t sample(const float* logits, int n, int V, float temperature, int top_k, const float* u, int32_t* out,
                  hipStream_t s);
// the same draw over many workgroups (nc_sample_parallel): scratch of
// sample_parallel_scratch_bytes(n, V) bytes, 256-byte aligned
int64_t sample_parallel_scratch_bytes(int n, int V);
hipError_t sample_parallel(const float* logits, int n, int V, float temperature, int top_k, const float* u,
                           int32_t* out, void* scratch, hipStream_t s);
template <typename T> hipError_t attn_decode(const AttnDecodeDesc& a, int nb, hipStream_t s);

// ---------------------------------------------------------------------------
// optimiser step
// ---------------------------------------------------------------------------
struct AdamwArgs {
  float grad_scale;         // multiplies g first
  float beta1, beta2;
  float decay;              // 1 - lr * weight_decay
  float lr;
  float inv_bc1, inv_bc2;   // 1 / (1 - beta^step)
  float eps;
};
// p, m, v fp32 [n] updated in place; out = p in the model dtype; n % 4 == 0
template <typename T> hipError_t adamw(int64_t n, float* p, const float* g, float* m, float* v, T* out,
                                       const AdamwArgs& a, hipStream_t s);
constexpr int kMuonMaxPartials = 1024;
int muon_partials(int64_t n);   // partial sums muon_momentum writes for n elements
// Each call covers `count` matrices of n = r * c elements, matrix j at
// element offset j * stride of g / buf / W / out, with its partial sums at
// partials + j * kMuonMaxPartials and its iteration operand at X + j * r * c.
// buf = mu buf + scale g;  partials[j][i] = sum of u^2 over block i's
// elements, u = scale g + mu buf (nesterov) or buf;  n % 4 == 0
hipError_t muon_momentum(int64_t n, int count, int64_t stride, const float* g, float* buf, float scale, float mu,
                         int nesterov, float* partials, hipStream_t s);
// X = u / (||u||_F + eps) as [r][c], or [c][r] when r > c;  r, c multiples of 64
template <typename T> hipError_t muon_normalise(int r, int c, int count, int64_t stride, const float* g,
                                                const float* buf, float scale, float mu, int nesterov,
                                                const float* partials, float eps, T* X, hipStream_t s);
// W [r][c] -= lr X (X [r][c], or [c][r] when r > c);  out = W in the model dtype
template <typename T> hipError_t muon_apply(int r, int c, int count, int64_t stride, const T* X, float lr, float* W,
                                            T* out, hipStream_t s);

}  // namespace nc
