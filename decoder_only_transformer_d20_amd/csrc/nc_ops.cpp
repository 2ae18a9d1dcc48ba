// Component entry points (include/nc_ops.h): argument checks and dispatch to
// the same launchers the model-level calls use.
#include "nc_ops.h"
#include "nc_internal.h"

using namespace nc;

namespace {

bool dtype_ok(int32_t dt) { return dt == NC_DTYPE_F32 || dt == NC_DTYPE_BF16; }
int status_of(hipError_t e) {
  if (e == hipSuccess) return NC_OK;
  if (e == hipErrorInvalidValue) return NC_ERR_SHAPE;
  if (e == hipErrorNotSupported) return NC_ERR_UNSUPPORTED;
  return NC_ERR_HIP;
}

// portable = 0 means the matrix-core kernel or nothing: a shape it cannot
// take is reported as unsupported rather than run elsewhere.
hipError_t dispatch_gemm(int32_t dtype, int32_t portable, const GemmDesc& g, hipStream_t s) {
  if (dtype == NC_DTYPE_F32) return gemm_portable<float>(g, s);
  if (portable) return gemm_portable<bf16>(g, s);
  if (!gemm_mfma_supported(g)) return hipErrorNotSupported;
  return gemm_mfma_bf16(g, s);
}

int head_tile(int32_t dtype, int64_t n, int32_t d, int32_t V, int32_t portable) {
  if (dtype == NC_DTYPE_F32 || portable) return 64;
  GemmDesc g{};
  g.M = (int)n; g.N = V; g.K = d; g.splits = 1; g.epi = EPI_LSE;
  return gemm_mfma_supported(g) ? gemm_mfma_tile_n(g) : 64;
}

}  // namespace

extern "C" {

int nc_op_matmul(int32_t dtype, int32_t p_trans, int32_t q_trans, int64_t M, int64_t N, int64_t K, const void* P,
                 const void* Q, void* C, int32_t out_f32, int32_t splits, float* part, int32_t portable,
                 void* hip_stream) {
  if (!dtype_ok(dtype) || !P || !Q || !C) return NC_ERR_INVALID_ARG;
  if (M <= 0 || N <= 0 || K <= 0 || M % 64 || N % 64 || M > (1 << 30) || N > (1 << 30) || K > (1 << 30))
    return NC_ERR_SHAPE;
  if (splits < 1 || (splits > 1 && (!out_f32 || !part))) return NC_ERR_INVALID_ARG;
  if (K % 64 || splits > K / 64) return NC_ERR_SHAPE;
  GemmDesc g{};
  g.M = (int)M; g.N = (int)N; g.K = (int)K;
  g.P = P; g.ldp = p_trans ? M : K; g.p_trans = p_trans ? 1 : 0;
  g.Q = Q; g.ldq = q_trans ? N : K; g.q_trans = q_trans ? 1 : 0;
  g.epi = out_f32 ? EPI_F32 : EPI_STORE;
  g.C = C; g.ldc = N; g.splits = splits; g.part = part;
  return status_of(dispatch_gemm(dtype, portable, g, (hipStream_t)hip_stream));
}

int nc_op_matmul_batched(int32_t dtype, int32_t q_trans, int32_t batch, int64_t M, int64_t N, int64_t K,
                         const void* P, int64_t sP, const void* Q, int64_t sQ, void* C, int64_t sC,
                         const void* aux, int64_t sAux, float alpha, float gamma, int32_t sym, int32_t portable,
                         void* hip_stream) {
  if (!dtype_ok(dtype) || !P || !Q || !C) return NC_ERR_INVALID_ARG;
  if (batch < 1 || batch > 65535 || (q_trans != 0 && q_trans != 1) || (sym != 0 && sym != 1))
    return NC_ERR_INVALID_ARG;
  if (sym && M != N) return NC_ERR_SHAPE;
  if (M <= 0 || N <= 0 || K <= 0 || M % 64 || N % 64 || K % 64 || M > (1 << 30) || N > (1 << 30) || K > (1 << 30))
    return NC_ERR_SHAPE;
  if (sP < 0 || sQ < 0 || sC < 0 || sAux < 0 || (sP | sQ | sC | sAux) % 8) return NC_ERR_INVALID_ARG;
  GemmDesc g{};
  g.M = (int)M; g.N = (int)N; g.K = (int)K;
  g.P = P; g.ldp = K; g.p_trans = 0;
  g.Q = Q; g.ldq = q_trans ? N : K; g.q_trans = q_trans;
  g.epi = aux ? EPI_AXPBY : EPI_STORE;
  g.C = C; g.ldc = N; g.splits = 1;
  g.aux = aux; g.ldaux = N; g.ep_alpha = alpha; g.ep_gamma = gamma;
  g.batch = batch; g.sP = sP; g.sQ = sQ; g.sC = sC; g.sAux = sAux; g.sym = sym;
  return status_of(dispatch_gemm(dtype, portable, g, (hipStream_t)hip_stream));
}

int nc_op_rmsnorm_fwd(int32_t dtype, int64_t rows, int32_t d, float eps, const void* x, void* y, float* r,
                      void* hip_stream) {
  if (!dtype_ok(dtype) || !x || !y || !r) return NC_ERR_INVALID_ARG;
  if (rows <= 0 || d <= 0 || d % 64) return NC_ERR_SHAPE;
  hipStream_t s = (hipStream_t)hip_stream;
  return status_of(dtype == NC_DTYPE_F32 ? rmsnorm_fwd<float>((const float*)x, (float*)y, r, rows, d, eps, s)
                                         : rmsnorm_fwd<bf16>((const bf16*)x, (bf16*)y, r, rows, d, eps, s));
}

int nc_op_rmsnorm_bwd(int32_t dtype, int64_t rows, int32_t d, const void* y, const float* r, const void* dy,
                      void* dx_io, int32_t accumulate, void* hip_stream) {
  if (!dtype_ok(dtype) || !y || !r || !dy || !dx_io) return NC_ERR_INVALID_ARG;
  if (rows <= 0 || d <= 0 || d % 64) return NC_ERR_SHAPE;
  hipStream_t s = (hipStream_t)hip_stream;
  return status_of(dtype == NC_DTYPE_F32
                       ? rmsnorm_bwd<float>((const float*)y, r, (const float*)dy, (float*)dx_io, rows, d,
                                            accumulate ? 1 : 0, s)
                       : rmsnorm_bwd<bf16>((const bf16*)y, r, (const bf16*)dy, (bf16*)dx_io, rows, d,
                                           accumulate ? 1 : 0, s));
}

int nc_op_device_info(int32_t device, int32_t* compute_units, int32_t* clock_khz, int32_t* mem_clock_khz,
                      int32_t* mem_bus_bits) {
  if (!compute_units || !clock_khz || !mem_clock_khz || !mem_bus_bits || device < 0) return NC_ERR_INVALID_ARG;
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, device) != hipSuccess) return NC_ERR_HIP;
  *compute_units = p.multiProcessorCount;
  *clock_khz = p.clockRate;
  *mem_clock_khz = p.memoryClockRate;
  *mem_bus_bits = p.memoryBusWidth;
  return NC_OK;
}

int nc_op_mfma_loop(int64_t iters, int32_t blocks, float* sink, void* hip_stream) {
  if (!sink) return NC_ERR_INVALID_ARG;
  if (iters < 1 || blocks < 1 || blocks > (1 << 20)) return NC_ERR_SHAPE;
  return status_of(mfma_loop(iters, blocks, sink, (hipStream_t)hip_stream));
}

int nc_op_rope_table(int32_t T, int32_t Q, float base, float* tab, void* hip_stream) {
  if (!tab) return NC_ERR_INVALID_ARG;
  if (T <= 0 || Q <= 0 || Q % 2) return NC_ERR_SHAPE;
  return status_of(rope_table((float2*)tab, T, Q, base, (hipStream_t)hip_stream));
}

int nc_op_attention_fwd(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t Q, const void* qkv, void* o,
                        float* lse, int32_t portable, void* hip_stream) {
  if (!dtype_ok(dtype) || !qkv || !o || !lse) return NC_ERR_INVALID_ARG;
  if (B <= 0 || T <= 0 || H <= 0 || Q <= 0 || T % 64 || Q % 64) return NC_ERR_SHAPE;
  AttnDesc a{};
  a.B = B; a.T = T; a.H = H; a.Q = Q; a.qkv = qkv; a.o_out = o; a.lse = lse;
  hipStream_t s = (hipStream_t)hip_stream;
  if (dtype == NC_DTYPE_F32) return status_of(attn_fwd_portable<float>(a, s));
  return status_of(portable ? attn_fwd_portable<bf16>(a, s) : attn_fwd_mfma(a, s));
}

int nc_op_attention_bwd(int32_t dtype, int32_t B, int32_t T, int32_t H, int32_t Q, const void* qkv, const void* o,
                        const void* dout, const float* lse, float* delta, void* dqkv, const float* rope_tab,
                        int32_t portable, void* hip_stream) {
  if (!dtype_ok(dtype) || !qkv || !o || !dout || !lse || !delta || !dqkv) return NC_ERR_INVALID_ARG;
  if (B <= 0 || T <= 0 || H <= 0 || Q <= 0 || T % 64 || Q % 64) return NC_ERR_SHAPE;
  AttnDesc a{};
  a.B = B; a.T = T; a.H = H; a.Q = Q;
  a.qkv = qkv; a.o = o; a.dout = dout; a.lse = (float*)lse; a.delta = delta; a.dqkv = dqkv;
  a.rope = (const float2*)rope_tab;
  hipStream_t s = (hipStream_t)hip_stream;
  if (dtype == NC_DTYPE_F32) return status_of(attn_bwd_portable<float>(a, s));
  return status_of(portable ? attn_bwd_portable<bf16>(a, s) : attn_bwd_mfma(a, s));
}

int nc_op_attention_bwd_ds(int32_t B, int32_t T, int32_t H, int32_t Q, const void* qkv, const void* o,
                           const void* dout, const float* lse, float* delta, void* dqkv, const float* rope_tab,
                           void* ds_scratch, void* hip_stream) {
  if (!qkv || !o || !dout || !lse || !delta || !dqkv || !ds_scratch) return NC_ERR_INVALID_ARG;
  if (B <= 0 || T <= 0 || H <= 0 || Q <= 0 || T % 64 || Q % 64) return NC_ERR_SHAPE;
  AttnDesc a{};
  a.B = B; a.T = T; a.H = H; a.Q = Q;
  a.qkv = qkv; a.o = o; a.dout = dout; a.lse = (float*)lse; a.delta = delta; a.dqkv = dqkv;
  a.rope = (const float2*)rope_tab;
  a.ds = ds_scratch;
  if (!attn_mfma_supported(a)) return NC_ERR_UNSUPPORTED;
  return status_of(attn_bwd_mfma(a, (hipStream_t)hip_stream));
}

int64_t nc_op_attention_ds_bytes(int32_t B, int32_t T, int32_t H) {
  if (B <= 0 || T <= 0 || H <= 0 || T % 64) return NC_ERR_SHAPE;
  return attn_ds_elems(B, T, H) * 2;
}

int nc_op_embed_fwd(int32_t dtype, int64_t n, int32_t d, int32_t V, const void* E, const int32_t* idx, void* x,
                    void* hip_stream) {
  if (!dtype_ok(dtype) || !E || !idx || !x) return NC_ERR_INVALID_ARG;
  if (n <= 0 || d <= 0 || d % 64 || V <= 0) return NC_ERR_SHAPE;
  hipStream_t s = (hipStream_t)hip_stream;
  return status_of(dtype == NC_DTYPE_F32 ? embed_fwd<float>((const float*)E, idx, (float*)x, n, d, V, s)
                                         : embed_fwd<bf16>((const bf16*)E, idx, (bf16*)x, n, d, V, s));
}

int64_t nc_op_embed_bwd_scratch_bytes(int64_t n, int32_t d) {
  if (n <= 0 || d <= 0 || d % 64 || n >= (1LL << 31)) return NC_ERR_SHAPE;
  return embed_bwd_scratch_bytes(n, d);
}

int nc_op_embed_bwd(int32_t dtype, int64_t n, int32_t d, int32_t V, const void* g, const int32_t* idx, float* dE,
                    int32_t accumulate, void* scratch, void* hip_stream) {
  if (!dtype_ok(dtype) || !g || !idx || !dE || !scratch) return NC_ERR_INVALID_ARG;
  if (n <= 0 || d <= 0 || d % 64 || V <= 0 || n >= (1LL << 31)) return NC_ERR_SHAPE;
  hipStream_t s = (hipStream_t)hip_stream;
  return status_of(dtype == NC_DTYPE_F32
                       ? embed_bwd<float>((const float*)g, idx, dE, n, d, V, accumulate, scratch, s)
                       : embed_bwd<bf16>((const bf16*)g, idx, dE, n, d, V, accumulate, scratch, s));
}

int64_t nc_op_head_scratch_bytes(int32_t dtype, int64_t n, int32_t d, int32_t V, int32_t portable) {
  if (!dtype_ok(dtype)) return NC_ERR_INVALID_ARG;
  if (n <= 0 || d <= 0 || V <= 0 || n % 64 || V % 64 || d % 64) return NC_ERR_SHAPE;
  const int64_t nblk = V / head_tile(dtype, n, d, V, portable);
  return n * nblk * 8 + n * 4;
}

int nc_op_head_ce_fwd(int32_t dtype, int64_t n, int32_t d, int32_t V, const void* xf, const void* U,
                      const int32_t* tgt, float* ce, float* lse, void* scratch, int32_t portable,
                      void* hip_stream) {
  if (!dtype_ok(dtype) || !xf || !U || !tgt || !ce || !lse || !scratch) return NC_ERR_INVALID_ARG;
  if (n <= 0 || d <= 0 || V <= 0 || n % 64 || V % 64 || d % 64 || n > (1 << 30)) return NC_ERR_SHAPE;
  const int nblk = V / head_tile(dtype, n, d, V, portable);
  GemmDesc g{};
  g.M = (int)n; g.N = V; g.K = d;
  g.P = xf; g.ldp = d; g.Q = U; g.ldq = d;
  g.epi = EPI_LSE; g.splits = 1;
  g.tgt = tgt;
  g.lse_part = (float2*)scratch;
  g.lse_stride = nblk;
  g.ztgt = (float*)((char*)scratch + n * nblk * 8);
  hipStream_t s = (hipStream_t)hip_stream;
  hipError_t e = dispatch_gemm(dtype, portable, g, s);
  if (e == hipSuccess) e = ce_combine(g.lse_part, nblk, g.ztgt, tgt, lse, ce, n, V, s);
  return status_of(e);
}

int nc_op_head_gemm_lse(int32_t dtype, int64_t n, int32_t d, int32_t V, const void* xf, const void* U,
                        const int32_t* tgt, void* scratch, void* hip_stream) {
  if (dtype != NC_DTYPE_BF16 || !xf || !U || !tgt || !scratch) return NC_ERR_INVALID_ARG;
  if (n <= 0 || d <= 0 || V <= 0 || n % 64 || V % 64 || d % 64 || n > (1 << 30)) return NC_ERR_SHAPE;
  const int nblk = V / head_tile(dtype, n, d, V, 0);
  GemmDesc g{};
  g.M = (int)n; g.N = V; g.K = d;
  g.P = xf; g.ldp = d; g.Q = U; g.ldq = d;
  g.epi = EPI_LSE; g.splits = 1;
  g.tgt = tgt;
  g.lse_part = (float2*)scratch;
  g.lse_stride = nblk;
  g.ztgt = (float*)((char*)scratch + n * nblk * 8);
  return status_of(dispatch_gemm(dtype, 0, g, (hipStream_t)hip_stream));
}

}  // extern "C"
