// Host side of the C ABI declared in include/nc.h and include/nc_ops.h:
// configuration checks, the flat parameter layout, the workspace plan and
// the order of kernel launches for the forward and backward passes.
//
// The step follows the nanochat speedrun walkthrough (lyylswood.com,
// sections Pretraining): pre-norm blocks of causal self-attention with
// rotary positions and a squared-ReLU MLP, parameter-free RMSNorm, untied
// embedding / unembedding, next-token cross-entropy and bits per byte.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "nc.h"
#include "nc_ops.h"
#include "nc_internal.h"

using namespace nc;

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool is_block(const nc_config& c) { return (c.flags & NC_FLAG_BLOCK_ONLY) != 0; }
bool is_bf16(const nc_config& c) { return c.dtype == NC_DTYPE_BF16; }
size_t esize(const nc_config& c) { return is_bf16(c) ? 2 : 4; }
bool portable(const nc_config& c) { return !is_bf16(c) || (c.flags & NC_FLAG_PORTABLE_KERNELS); }

int validate(const nc_config* c) {
  if (!c) return NC_ERR_INVALID_ARG;
  if (c->dtype != NC_DTYPE_F32 && c->dtype != NC_DTYPE_BF16) return NC_ERR_INVALID_ARG;
  if (c->flags & ~(NC_FLAG_BLOCK_ONLY | NC_FLAG_PORTABLE_KERNELS)) return NC_ERR_INVALID_ARG;
  if (c->n_layer <= 0 || c->d_model <= 0 || c->n_head <= 0 || c->head_dim <= 0 || c->d_ff <= 0 ||
      c->batch <= 0 || c->seq_len <= 0)
    return NC_ERR_SHAPE;
  if (c->n_head * c->head_dim != c->d_model) return NC_ERR_SHAPE;
  if (c->d_model % 64 || c->d_ff % 64 || c->seq_len % 64 || c->head_dim % 64) return NC_ERR_SHAPE;
  if (c->head_dim > 256) return NC_ERR_UNSUPPORTED;
  if (is_block(*c)) {
    if (c->n_layer != 1 || c->vocab != 0) return NC_ERR_SHAPE;
  } else {
    if (c->vocab <= 0 || c->vocab % 64) return NC_ERR_SHAPE;
  }
  if (!(c->rms_eps >= 0.f) || !(c->rope_base > 0.f)) return NC_ERR_INVALID_ARG;
  // one row of the residual stream must fit the RMSNorm kernel's registers
  if ((int64_t)c->d_model * (int64_t)esize(*c) > 64 * 8 * 16) return NC_ERR_UNSUPPORTED;
  return NC_OK;
}

int64_t layer_elems(const nc_config& c) {
  const int64_t d = c.d_model, F = c.d_ff;
  return 4 * d * d + 2 * F * d;
}

// The N-tile the GEMM dispatcher uses for an [M x N] output (the head's
// log-sum-exp partials have one entry per N-tile).
int tile_n(const nc_config& c, int M, int N) {
  if (portable(c)) return 64;
  GemmDesc g{};
  g.M = M; g.N = N; g.K = c.d_model; g.splits = 1; g.epi = EPI_LSE;
  return gemm_mfma_supported(g) ? gemm_mfma_tile_n(g) : 64;
}

// Split-K factor for the weight-gradient products (K = tokens).  Each split
// is a (tile, k-range) unit of the persistent grid; more splits fill the
// chip's 256 CUs in fuller waves but write and re-read more fp32 partials.
// The count minimises a simple model: compute time at 1 PFLOP/s scaled by
// the wave quantisation, plus the partials' round trip at 5 TB/s.
int choose_splits(const nc_config& c, int M, int N, int64_t K) {
  constexpr int kCUs = 256;
  int64_t tiles = (int64_t)(M / 64) * (N / 64);
  if (!portable(c)) {
    GemmDesc g{};
    g.M = M; g.N = N; g.K = (int)K; g.splits = 1; g.epi = EPI_F32; g.p_trans = 1; g.q_trans = 1;
    const int bm = gemm_mfma_tile_m(g), bn = gemm_mfma_tile_n(g);
    tiles = (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn);
  }
  const int64_t nb = K / 64;
  int best_s = 1;
  double best = 0.0;
  for (int s = 1; s <= 32 && s <= nb; ++s) {
    const double units = (double)tiles * s;
    const double waves = std::ceil(units / kCUs);
    const double t = 2.0 * M * N * (double)K / 1e15 * (waves * kCUs / units) + (s > 1 ? s * 8.0 * M * N / 5e12 : 0.0);
    if (s == 1 || t < best * (1.0 - 1e-9)) {
      best = t;
      best_s = s;
    }
  }
  return best_s;
}

struct Plan {
  size_t total = 0;
  size_t rope = 0, idx = 0, tgt = 0, x = 0, xf = 0, rf = 0, ce = 0, lse_head = 0, ztgt = 0, lse_part = 0, rowscale = 0;
  bool keep_logits = false;   // zkeep is laid out (the head's backward runs as one chunk)
  size_t scalars = 0, dz = 0, zkeep = 0, g = 0, gtmp = 0, big = 0, part = 0, delta = 0, wt = 0, embs = 0;
  size_t layer0 = 0, layer_stride = 0;
  size_t l_a = 0, l_r1 = 0, l_qkv = 0, l_o = 0, l_lse = 0, l_m = 0, l_r2 = 0, l_u = 0;
  int head_nblk = 0;
  int64_t head_chunk = 0;
};

Plan make_plan(const nc_config& c) {
  Plan p;
  const size_t es = esize(c);
  const int64_t N = (int64_t)c.batch * c.seq_len, d = c.d_model, F = c.d_ff, V = c.vocab;
  const int64_t BHT = (int64_t)c.batch * c.n_head * c.seq_len;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  p.rope = take((size_t)c.seq_len * (c.head_dim / 2) * 8);
  p.scalars = take(256);
  p.delta = take(BHT * 4);
  p.g = take(N * d * es);
  p.gtmp = take(N * d * es);
  p.big = take(N * std::max(F, 3 * d) * es);
  // bf16: transposed image of the weight an activation gradient multiplies by
  if (is_bf16(c)) p.wt = take(std::max({F * d, 3 * d * d, is_block(c) ? 0 : V * d}) * es);
  // split-K partials: the largest of the weight-gradient products
  size_t part = 0;
  auto need = [&](int M_, int N_, int64_t K_) {
    const int s = choose_splits(c, M_, N_, K_);
    if (s > 1) part = std::max(part, (size_t)s * M_ * N_ * 4);
  };
  need((int)(3 * d), (int)d, N);
  need((int)d, (int)d, N);
  need((int)F, (int)d, N);
  need((int)d, (int)F, N);
  if (!is_block(c)) {
    p.idx = take(N * 4);
    p.tgt = take(N * 4);
    p.rowscale = take(N * 4);
    p.x = take(N * d * es);
    p.xf = take(N * d * es);
    p.rf = take(N * 4);
    p.ce = take(N * 4);
    p.lse_head = take(N * 4);
    p.ztgt = take(N * 4);
    p.head_nblk = (int)(V / tile_n(c, (int)std::min<int64_t>(N, 1 << 30), (int)V));
    p.lse_part = take((size_t)N * p.head_nblk * 8);
    // token chunks for the head's backward: whole rows, up to 64k tokens
    // (the d20 batch in one piece: the products over the chunk then fill
    // whole waves of tiles; dz takes 2 bytes per token and vocabulary entry)
    const int64_t rows = std::max<int64_t>(1, std::min<int64_t>(c.batch, 65536 / c.seq_len));
    p.head_chunk = rows * c.seq_len;
    p.dz = take((size_t)p.head_chunk * V * es);
    // the forward's logits, kept for the backward when it is one chunk
    p.keep_logits = p.head_chunk >= N;
    if (p.keep_logits) p.zkeep = take((size_t)N * V * es);
    p.embs = take((size_t)embed_bwd_scratch_bytes(N, (int)d));
    need((int)V, (int)d, p.head_chunk);
  }
  p.part = take(part);
  // saved activations, one block of regions per layer
  size_t lo = 0;
  auto ltake = [&](size_t bytes) { size_t o = lo; lo += align_up(bytes); return o; };
  p.l_a = ltake(N * d * es);
  p.l_r1 = ltake(N * 4);
  p.l_qkv = ltake(N * 3 * d * es);
  p.l_o = ltake(N * d * es);
  p.l_lse = ltake(BHT * 4);
  p.l_m = ltake(N * d * es);
  p.l_r2 = ltake(N * 4);
  p.l_u = ltake(N * F * es);
  p.layer_stride = lo;
  p.layer0 = off;
  off += lo * c.n_layer;
  p.total = off;
  return p;
}

}  // namespace

struct nc_ctx {
  nc_config cfg;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  hipStream_t stream = nullptr;
  Plan plan;
  bool have_forward = false;
  bool have_block_forward = false;
  bool logits_kept = false;        // plan.zkeep holds the last forward's logits
  int64_t fallbacks = 0;           // bf16 launches that took a portable kernel (nc_fallback_count)
  void* static_scratch = nullptr;  // this device's nc_decode_static scratch
  std::string static_scratch_err;
  std::string err;
  // kernel timing (nc_trace_*)
  int trace_family = -1;
  std::vector<hipEvent_t> ev;      // start/end pairs, created on demand
  size_t n_rec = 0;
  double trace_flops = 0.0, trace_bytes = 0.0;

  template <typename T> T* at(size_t off) { return reinterpret_cast<T*>(ws + off); }
  char* layer(int l) { return ws + plan.layer0 + plan.layer_stride * (size_t)l; }
  ~nc_ctx() {
    for (hipEvent_t e : ev) hipEventDestroy(e);
  }
};

namespace {

int fail(nc_ctx* ctx, hipError_t e, const char* what) {
  ctx->err = std::string(what) + ": " + hipGetErrorString(e);
  return NC_ERR_HIP;
}
#define NC_TRY(expr, what)                      \
  do {                                          \
    hipError_t e_ = (expr);                     \
    if (e_ != hipSuccess) return fail(ctx, e_, what); \
  } while (0)

// ---- kernel timing -----------------------------------------------------------
constexpr size_t kMaxTrace = 65536;

int gemm_family(const GemmDesc& g) {
  const int key = g.p_trans * 2 + g.q_trans;
  switch (g.epi) {
    case EPI_ROPE: return key == 0 ? NC_TRACE_GEMM_QKV_ROPE : -1;
    case EPI_RESID: return key == 0 ? NC_TRACE_GEMM_RESIDUAL : -1;
    case EPI_RELU2: return key == 0 ? NC_TRACE_GEMM_RELU2 : -1;
    case EPI_STORE: return key <= 1 ? NC_TRACE_GEMM_DGRAD : -1;
    case EPI_LSE:
    case EPI_LSEZ: return key == 0 ? NC_TRACE_GEMM_HEAD_LSE : -1;
    case EPI_DZ: return key == 0 ? NC_TRACE_GEMM_HEAD_DZ : -1;
    case EPI_DRELU2: return key <= 1 ? NC_TRACE_GEMM_DGRAD_RELU2 : -1;
    case EPI_F32: return key == 3 ? NC_TRACE_GEMM_WGRAD : -1;
    default: return -1;
  }
}

// algorithmic HBM bytes of one product: operands read once, result written once
double gemm_bytes(const GemmDesc& g, size_t es) {
  const double M = g.M, N = g.N, K = g.K;
  double b = (M * K + N * K) * es;
  switch (g.epi) {
    case EPI_F32: b += M * N * 4.0 * (g.beta ? 2 : 1); break;
    case EPI_LSE: b += M * 4.0 * 2; break;                       // targets in, z[target] out
    case EPI_LSEZ: b += M * 4.0 * 2 + M * N * es; break;         // and the logits out
    case EPI_DZ: b += M * N * es + M * 8.0; break;
    case EPI_RESID:
    case EPI_DRELU2:
    case EPI_AXPBY: b += 2.0 * M * N * es; break;
    default: b += M * N * es; break;
  }
  return b;
}

// run `launch` bracketed by events when `family` is being traced
template <typename F>
hipError_t traced(nc_ctx* ctx, int family, double flops, double bytes, F&& launch) {
  if (family < 0 || family != ctx->trace_family || ctx->n_rec >= kMaxTrace) return launch();
  if (ctx->ev.size() < 2 * (ctx->n_rec + 1)) {
    for (int i = 0; i < 2; ++i) {
      hipEvent_t e;
      hipError_t r = hipEventCreate(&e);
      if (r != hipSuccess) return r;
      ctx->ev.push_back(e);
    }
  }
  hipError_t r = hipEventRecord(ctx->ev[2 * ctx->n_rec], ctx->stream);
  if (r != hipSuccess) return r;
  r = launch();
  if (r != hipSuccess) return r;
  r = hipEventRecord(ctx->ev[2 * ctx->n_rec + 1], ctx->stream);
  if (r != hipSuccess) return r;
  ctx->n_rec++;
  ctx->trace_flops += flops;
  ctx->trace_bytes += bytes;
  return hipSuccess;
}

// family < -1: the forward/backward family of the product's layout and epilogue
hipError_t run_gemm(nc_ctx* ctx, const GemmDesc& g, int family = -2) {
  if (!is_bf16(ctx->cfg)) return gemm_portable<float>(g, ctx->stream);
  if (portable(ctx->cfg)) return gemm_portable<bf16>(g, ctx->stream);
  if (!gemm_mfma_supported(g)) {
    ctx->fallbacks++;
    return gemm_portable<bf16>(g, ctx->stream);
  }
  double items = g.batch > 1 ? g.batch : 1;
  if (g.sym) {
    // the tiles on and above the diagonal are computed, the rest mirrored
    const double t = g.M / gemm_mfma_tile_m(g);
    items *= (t + 1) / (2 * t);
  }
  hipError_t e = traced(ctx, family < -1 ? gemm_family(g) : family, 2.0 * g.M * g.N * g.K * items,
                        gemm_bytes(g, 2) * items, [&] { return gemm_mfma_bf16_product(g, ctx->stream); });
  if (e == hipSuccess && g.epi == EPI_F32 && g.splits > 1)
    e = splitk_reduce(g.part, g.splits, (int64_t)g.M * g.N, (float*)g.C, g.beta, ctx->stream);
  return e;
}

GemmDesc gemm(int M, int N, int K, const void* P, int64_t ldp, int pt, const void* Q, int64_t ldq, int qt, int epi,
              void* C, int64_t ldc) {
  GemmDesc g{};
  g.M = M; g.N = N; g.K = K;
  g.P = P; g.ldp = ldp; g.p_trans = pt;
  g.Q = Q; g.ldq = ldq; g.q_trans = qt;
  g.epi = epi; g.C = C; g.ldc = ldc; g.splits = 1;
  return g;
}

// Activation gradient dX[M][cols] = dY[M][rows] W (W [rows][cols], the
// weight of a forward product y = x W^T).  In bf16 the weight is first
// transposed into the workspace, so the product reads both operands k-major;
// in fp32 the product reads W as a transposed operand.
template <typename T>
hipError_t dgrad_desc(nc_ctx* ctx, int M, const T* dY, int64_t ldy, const T* W, int rows, int cols, int epi, T* out,
                      int64_t ldo, GemmDesc* g) {
  if constexpr (sizeof(T) == 2) {
    T* wt = ctx->at<T>(ctx->plan.wt);
    hipError_t e = transpose_bf16((const bf16*)W, rows, cols, (bf16*)wt, ctx->stream);
    if (e != hipSuccess) return e;
    *g = gemm(M, cols, rows, dY, ldy, 0, wt, rows, 0, epi, out, ldo);
  } else {
    *g = gemm(M, cols, rows, dY, ldy, 0, W, cols, 1, epi, out, ldo);
  }
  return hipSuccess;
}

// weight gradient dW[M'][N'] (+)= sum over tokens P[tok][m'] Q[tok][n']
hipError_t weight_grad(nc_ctx* ctx, int Mw, int Nw, const void* P, int64_t ldp, const void* Q, int64_t ldq,
                       float* dW, int accumulate) {
  const int64_t N = (int64_t)ctx->cfg.batch * ctx->cfg.seq_len;
  GemmDesc g = gemm(Mw, Nw, (int)N, P, ldp, 1, Q, ldq, 1, EPI_F32, dW, Nw);
  g.beta = accumulate;
  g.splits = choose_splits(ctx->cfg, Mw, Nw, N);
  g.part = ctx->at<float>(ctx->plan.part);
  return run_gemm(ctx, g);
}

// causal score pairs of one step: B * H * T (T + 1) / 2
double attn_pairs(const AttnDesc& a) { return (double)a.B * a.H * (double)a.T * (a.T + 1) / 2.0; }

template <typename T> hipError_t attn_fwd(nc_ctx* ctx, const AttnDesc& a) {
  if (!portable(ctx->cfg) && attn_mfma_supported(a)) {
    // S = Q K^T and O = P V over the causal pairs; q,k,v read, o and lse written
    const double tok = (double)a.B * a.T, d = (double)a.H * a.Q;
    return traced(ctx, NC_TRACE_ATTN_FWD, 2 * 2.0 * attn_pairs(a) * a.Q, tok * (3 * d + d) * 2 + tok * a.H * 4,
                  [&] { return attn_fwd_mfma(a, ctx->stream); });
  }
  if (!portable(ctx->cfg)) ctx->fallbacks++;
  return attn_fwd_portable<T>(a, ctx->stream);
}
template <typename T> hipError_t attn_bwd(nc_ctx* ctx, const AttnDesc& a) {
  if (!portable(ctx->cfg) && attn_mfma_supported(a)) {
    // flash backward: recompute S, then dV, dP, dQ, dK (5 causal products);
    // q,k,v,o,dO read, dq,dk,dv written (with stored dS also its round trip,
    // which is the implementation's, not the method's)
    const double tok = (double)a.B * a.T, d = (double)a.H * a.Q;
    return traced(ctx, NC_TRACE_ATTN_BWD, 5 * 2.0 * attn_pairs(a) * a.Q, tok * (5 * d + 3 * d) * 2 + tok * a.H * 8,
                  [&] { return attn_bwd_mfma(a, ctx->stream); });
  }
  if (!portable(ctx->cfg)) ctx->fallbacks++;
  return attn_bwd_portable<T>(a, ctx->stream);
}

// one pre-norm block; x is the residual stream, updated in place
template <typename T>
int layer_forward(nc_ctx* ctx, int l, const T* w, T* x) {
  const nc_config& c = ctx->cfg;
  const Plan& p = ctx->plan;
  const int N = c.batch * c.seq_len, d = c.d_model, F = c.d_ff;
  const T* Wqkv = w;
  const T* Wo = w + 3LL * d * d;
  const T* W1 = w + 4LL * d * d;
  const T* W2 = W1 + (int64_t)F * d;
  char* L = ctx->layer(l);
  T* a = (T*)(L + p.l_a);
  float* r1 = (float*)(L + p.l_r1);
  T* qkv = (T*)(L + p.l_qkv);
  T* o = (T*)(L + p.l_o);
  float* lse = (float*)(L + p.l_lse);
  T* m = (T*)(L + p.l_m);
  float* r2 = (float*)(L + p.l_r2);
  T* u = (T*)(L + p.l_u);
  hipStream_t s = ctx->stream;

  NC_TRY(rmsnorm_fwd<T>(x, a, r1, N, d, c.rms_eps, s), "rmsnorm (attention input)");
  GemmDesc g = gemm(N, 3 * d, d, a, d, 0, Wqkv, d, 0, EPI_ROPE, qkv, 3 * d);
  g.rope = ctx->at<float2>(p.rope); g.rope_T = c.seq_len; g.rope_cols = 2 * d; g.head_dim = c.head_dim;
  NC_TRY(run_gemm(ctx, g), "qkv projection + rotary");
  AttnDesc ad{};
  ad.B = c.batch; ad.T = c.seq_len; ad.H = c.n_head; ad.Q = c.head_dim;
  ad.qkv = qkv; ad.o_out = o; ad.lse = lse;
  NC_TRY(attn_fwd<T>(ctx, ad), "attention forward");
  g = gemm(N, d, d, o, d, 0, Wo, d, 0, EPI_RESID, x, d);
  g.aux = x; g.ldaux = d;
  NC_TRY(run_gemm(ctx, g), "output projection + residual");
  NC_TRY(rmsnorm_fwd<T>(x, m, r2, N, d, c.rms_eps, s), "rmsnorm (MLP input)");
  // the saved MLP activation is u = relu(h)^2, h = m W1^T: the down
  // projection and dW2 consume u as is, and dh needs only 2 relu(h) = 2 sqrt(u)
  NC_TRY(run_gemm(ctx, gemm(N, F, d, m, d, 0, W1, d, 0, EPI_RELU2, u, F)), "MLP up projection + relu^2");
  g = gemm(N, d, F, u, F, 0, W2, F, 0, EPI_RESID, x, d);
  g.aux = x; g.ldaux = d;
  NC_TRY(run_gemm(ctx, g), "MLP down projection + residual");
  return NC_OK;
}

// reverse of layer_forward: g = dL/d(layer output) in, dL/d(layer input) out
template <typename T>
int layer_backward(nc_ctx* ctx, int l, const T* w, T* gr, float* dw, int accumulate) {
  const nc_config& c = ctx->cfg;
  const Plan& p = ctx->plan;
  const int N = c.batch * c.seq_len, d = c.d_model, F = c.d_ff;
  const T* Wqkv = w;
  const T* Wo = w + 3LL * d * d;
  const T* W1 = w + 4LL * d * d;
  const T* W2 = W1 + (int64_t)F * d;
  float* dWqkv = dw;
  float* dWo = dw + 3LL * d * d;
  float* dW1 = dw + 4LL * d * d;
  float* dW2 = dW1 + (int64_t)F * d;
  char* L = ctx->layer(l);
  T* a = (T*)(L + p.l_a);
  float* r1 = (float*)(L + p.l_r1);
  T* qkv = (T*)(L + p.l_qkv);
  T* o = (T*)(L + p.l_o);
  float* lse = (float*)(L + p.l_lse);
  T* m = (T*)(L + p.l_m);
  float* r2 = (float*)(L + p.l_r2);
  T* u = (T*)(L + p.l_u);
  T* tmp = ctx->at<T>(p.gtmp);
  T* big = ctx->at<T>(p.big);
  hipStream_t s = ctx->stream;

  // MLP: x2 = x1 + u W2^T, u = relu(h)^2, h = m W1^T
  NC_TRY(weight_grad(ctx, d, F, gr, d, u, F, dW2, accumulate), "dW2");
  GemmDesc g;
  NC_TRY(dgrad_desc<T>(ctx, N, gr, d, W2, d, F, EPI_DRELU2, big, F, &g), "transpose W2");
  g.aux = u; g.ldaux = F;
  NC_TRY(run_gemm(ctx, g), "dh = (g W2) * 2 relu(h)");
  NC_TRY(weight_grad(ctx, F, d, big, F, m, d, dW1, accumulate), "dW1");
  NC_TRY(dgrad_desc<T>(ctx, N, big, F, W1, F, d, EPI_STORE, tmp, d, &g), "transpose W1");
  NC_TRY(run_gemm(ctx, g), "dm = dh W1");
  NC_TRY(rmsnorm_bwd<T>(m, r2, tmp, gr, N, d, 1, s), "rmsnorm backward (MLP input)");
  // attention: x1 = x0 + o Wo^T
  NC_TRY(weight_grad(ctx, d, d, gr, d, o, d, dWo, accumulate), "dWo");
  NC_TRY(dgrad_desc<T>(ctx, N, gr, d, Wo, d, d, EPI_STORE, tmp, d, &g), "transpose Wo");
  NC_TRY(run_gemm(ctx, g), "do = g Wo");
  AttnDesc ad{};
  ad.B = c.batch; ad.T = c.seq_len; ad.H = c.n_head; ad.Q = c.head_dim;
  ad.qkv = qkv; ad.o = o; ad.lse = lse; ad.dout = tmp; ad.delta = ctx->at<float>(p.delta);
  ad.dqkv = big; ad.rope = ctx->at<float2>(p.rope);
  // S and dP are recomputed in the dQ kernel (ad.ds = null).  Storing dS
  // instead (nc_op_attention_bwd_ds, +1.4 GB of workspace at d20) measured
  // the same time: the dQ kernel saves what the dK/dV kernel's dS stores and
  // the separate delta pass cost.
  ad.ds = nullptr;
  NC_TRY(attn_bwd<T>(ctx, ad), "attention backward");
  NC_TRY(weight_grad(ctx, 3 * d, d, big, 3 * d, a, d, dWqkv, accumulate), "dWqkv");
  NC_TRY(dgrad_desc<T>(ctx, N, big, 3 * d, Wqkv, 3 * d, d, EPI_STORE, tmp, d, &g), "transpose Wqkv");
  NC_TRY(run_gemm(ctx, g), "da = dqkv Wqkv");
  NC_TRY(rmsnorm_bwd<T>(a, r1, tmp, gr, N, d, 1, s), "rmsnorm backward (attention input)");
  return NC_OK;
}

template <typename T>
int model_forward(nc_ctx* ctx, const T* params, const int32_t* idx, const int32_t* tgt, float* ce_out,
                  bool keep_logits = true) {
  ctx->logits_kept = false;
  const nc_config& c = ctx->cfg;
  const Plan& p = ctx->plan;
  const int N = c.batch * c.seq_len, d = c.d_model, V = c.vocab;
  hipStream_t s = ctx->stream;
  int32_t* widx = ctx->at<int32_t>(p.idx);
  int32_t* wtgt = ctx->at<int32_t>(p.tgt);
  NC_TRY(copy_bytes(widx, idx, (size_t)N * 4, s), "copy token ids");
  NC_TRY(copy_bytes(wtgt, tgt, (size_t)N * 4, s), "copy targets");
  NC_TRY(count_valid(wtgt, N, ctx->at<float>(p.scalars), s), "count valid targets");
  T* x = ctx->at<T>(p.x);
  NC_TRY(embed_fwd<T>(params, widx, x, N, d, V, s), "embedding gather");
  const T* w = params + (int64_t)V * d;
  for (int l = 0; l < c.n_layer; ++l) {
    int st = layer_forward<T>(ctx, l, w + (int64_t)l * layer_elems(c), x);
    if (st != NC_OK) return st;
  }
  T* xf = ctx->at<T>(p.xf);
  float* rf = ctx->at<float>(p.rf);
  NC_TRY(rmsnorm_fwd<T>(x, xf, rf, N, d, c.rms_eps, s), "final rmsnorm");
  const T* U = w + (int64_t)c.n_layer * layer_elems(c);
  // When the head's backward runs as one chunk, the product keeps the
  // logits (relative to their tile's row maximum) and the backward forms dz
  // from them instead of recomputing the product.
  const bool keep_z = keep_logits && p.keep_logits;
  GemmDesc g = gemm(N, V, d, xf, d, 0, U, d, 0, keep_z ? EPI_LSEZ : EPI_LSE, keep_z ? ctx->at<T>(p.zkeep) : nullptr,
                    keep_z ? V : 0);
  g.tgt = wtgt; g.lse_part = ctx->at<float2>(p.lse_part); g.lse_stride = p.head_nblk;
  g.ztgt = ctx->at<float>(p.ztgt);
  NC_TRY(run_gemm(ctx, g), "unembedding + log-sum-exp partials");
  ctx->logits_kept = keep_z;
  float* ce = ctx->at<float>(p.ce);
  NC_TRY(ce_combine(g.lse_part, p.head_nblk, g.ztgt, wtgt, ctx->at<float>(p.lse_head), ce, N, V, s), "cross-entropy");
  if (ce_out) NC_TRY(copy_bytes(ce_out, ce, (size_t)N * 4, s), "copy ce");
  return NC_OK;
}

template <typename T>
int model_backward(nc_ctx* ctx, const T* params, float* grads, int accumulate, const float* tok_w) {
  const nc_config& c = ctx->cfg;
  const Plan& p = ctx->plan;
  const int N = c.batch * c.seq_len, d = c.d_model, V = c.vocab;
  hipStream_t s = ctx->stream;
  const T* w = params + (int64_t)V * d;
  const T* U = w + (int64_t)c.n_layer * layer_elems(c);
  float* dE = grads;
  float* dw = grads + (int64_t)V * d;
  float* dU = dw + (int64_t)c.n_layer * layer_elems(c);
  T* xf = ctx->at<T>(p.xf);
  T* gr = ctx->at<T>(p.g);
  T* tmp = ctx->at<T>(p.gtmp);
  T* dz = ctx->at<T>(p.dz);
  const int32_t* wtgt = ctx->at<int32_t>(p.tgt);
  // head, one token chunk at a time: dz = (softmax(z) - onehot) w / n_valid
  // (w = 1 unless token weights are given), dxf = dz U, dU (+)= dz^T xf.
  // (U is transposed once, for every chunk.)
  float* rs = ctx->at<float>(p.rowscale);
  NC_TRY(row_scale(wtgt, tok_w, ctx->at<float>(p.scalars), N, V, rs, s), "dz row factors");
  GemmDesc gx;
  NC_TRY(dgrad_desc<T>(ctx, 0, dz, V, U, V, d, EPI_STORE, tmp, d, &gx), "transpose U");
  const bool kept_z = ctx->logits_kept;          // then the head runs as one chunk
  for (int64_t r0 = 0; r0 < N; r0 += p.head_chunk) {
    const int Mc = (int)std::min<int64_t>(p.head_chunk, N - r0);
    GemmDesc g;
    if (kept_z) {
      const double nz = (double)N * V;
      NC_TRY(traced(ctx, NC_TRACE_GEMM_HEAD_DZ, 4.0 * nz, 2.0 * nz * sizeof(T),
                    [&] {
                      return dz_from_logits<T>(ctx->at<T>(p.zkeep), dz, N, V, V / p.head_nblk,
                                               ctx->at<float2>(p.lse_part), p.head_nblk, ctx->at<float>(p.ztgt),
                                               wtgt, ctx->at<float>(p.lse_head), rs, s);
                    }),
             "dz from the kept logits");
    } else {
      g = gemm(Mc, V, d, xf + r0 * d, d, 0, U, d, 0, EPI_DZ, dz, V);
      g.tgt = wtgt + r0; g.lse = ctx->at<float>(p.lse_head) + r0; g.row_scale = rs + r0;
      NC_TRY(run_gemm(ctx, g), "recompute logits -> dz");
    }
    gx.M = Mc;
    gx.C = tmp + r0 * d;
    NC_TRY(run_gemm(ctx, gx), "dxf = dz U");
    g = gemm(V, d, Mc, dz, V, 1, xf + r0 * d, d, 1, EPI_F32, dU, d);
    g.beta = (accumulate || r0 > 0) ? 1 : 0;
    g.splits = choose_splits(c, V, d, Mc);
    g.part = ctx->at<float>(p.part);
    NC_TRY(run_gemm(ctx, g), "dU = dz^T xf");
  }
  NC_TRY(rmsnorm_bwd<T>(xf, ctx->at<float>(p.rf), tmp, gr, N, d, 0, s), "final rmsnorm backward");
  for (int l = c.n_layer - 1; l >= 0; --l) {
    int st = layer_backward<T>(ctx, l, w + (int64_t)l * layer_elems(c), gr, dw + (int64_t)l * layer_elems(c),
                               accumulate);
    if (st != NC_OK) return st;
  }
  NC_TRY(embed_bwd<T>(gr, ctx->at<int32_t>(p.idx), dE, N, d, V, accumulate, ctx->at<char>(p.embs), s),
         "embedding gradient");
  return NC_OK;
}

template <typename T>
int block_forward(nc_ctx* ctx, const T* w, const T* x, T* y) {
  const nc_config& c = ctx->cfg;
  const size_t bytes = (size_t)c.batch * c.seq_len * c.d_model * sizeof(T);
  NC_TRY(copy_bytes(y, x, bytes, ctx->stream), "copy block input");
  return layer_forward<T>(ctx, 0, w, y);
}

template <typename T>
int block_backward(nc_ctx* ctx, const T* w, const T* dy, T* dx, float* dparams, int accumulate) {
  const nc_config& c = ctx->cfg;
  const size_t bytes = (size_t)c.batch * c.seq_len * c.d_model * sizeof(T);
  NC_TRY(copy_bytes(dx, dy, bytes, ctx->stream), "copy upstream gradient");
  return layer_backward<T>(ctx, 0, w, dx, dparams, accumulate);
}

// ---- optimiser step ------------------------------------------------------------
struct OptimTensor {
  int tensor, layer;
  int64_t off, rows, cols;
};

std::vector<OptimTensor> optim_tensors(const nc_config& c) {
  std::vector<OptimTensor> v;
  const int64_t d = c.d_model, F = c.d_ff, V = c.vocab;
  const int64_t base = is_block(c) ? 0 : V * d;
  if (!is_block(c)) v.push_back({NC_T_E, -1, 0, V, d});
  const int64_t sizes[6][2] = {{d, d}, {d, d}, {d, d}, {d, d}, {F, d}, {d, F}};
  for (int l = 0; l < c.n_layer; ++l) {
    int64_t off = base + layer_elems(c) * l;
    for (int t = 0; t < 6; ++t) {
      v.push_back({NC_T_WQ + t, l, off, sizes[t][0], sizes[t][1]});
      off += sizes[t][0] * sizes[t][1];
    }
  }
  if (!is_block(c)) v.push_back({NC_T_U, -1, base + layer_elems(c) * c.n_layer, V, d});
  return v;
}

int64_t param_count_of(const nc_config& c) {
  return (is_block(c) ? 0 : 2 * (int64_t)c.vocab * c.d_model) + layer_elems(c) * c.n_layer;
}

// Muon's matrices as sets (one tensor of every layer: same shape, layer l
// at off0 + l * stride), and the sets grouped by their wide orientation
// [rw][cw] (rw <= cw): a group's Newton-Schulz products run as one batched
// launch over its matrices, set by set, layer by layer.
struct MuonSet {
  int tensor, r, c, count;
  int64_t off0, stride;
};
struct MuonGroup {
  int rw, cw, nb;
  std::vector<MuonSet> sets;
};

std::vector<MuonGroup> muon_groups(const nc_config& c) {
  const int64_t d = c.d_model, F = c.d_ff;
  const int64_t base = is_block(c) ? 0 : (int64_t)c.vocab * d;
  const int64_t sizes[6][2] = {{d, d}, {d, d}, {d, d}, {d, d}, {F, d}, {d, F}};
  std::vector<MuonGroup> gs;
  int64_t off = base;
  for (int t = 0; t < 6; ++t) {
    const MuonSet st{NC_T_WQ + t, (int)sizes[t][0], (int)sizes[t][1], c.n_layer, off, layer_elems(c)};
    off += sizes[t][0] * sizes[t][1];
    const int rw = std::min(st.r, st.c), cw = std::max(st.r, st.c);
    auto it = std::find_if(gs.begin(), gs.end(), [&](const MuonGroup& g) { return g.rw == rw && g.cw == cw; });
    if (it == gs.end()) gs.push_back({rw, cw, st.count, {st}});
    else { it->sets.push_back(st); it->nb += st.count; }
  }
  return gs;
}

// scratch: per-matrix partial sums | X (two, ping-pong) | A | B, each sized
// for the largest group and 256-aligned
struct OptimScratch {
  size_t partials = 0, x0 = 0, x1 = 0, a = 0, b = 0, total = 0;
};

OptimScratch optim_scratch(const nc_config& c) {
  int64_t max_x = 0, max_a = 0, max_nb = 0;
  for (const MuonGroup& g : muon_groups(c)) {
    const int64_t nb = g.nb;
    max_x = std::max(max_x, nb * g.rw * g.cw);
    max_a = std::max(max_a, nb * g.rw * g.rw);
    max_nb = std::max(max_nb, nb);
  }
  const size_t es = esize(c);
  OptimScratch o;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t r = off; off += align_up(bytes); return r; };
  o.partials = take(max_nb * kMuonMaxPartials * 4);
  o.x0 = take(max_x * es);
  o.x1 = take(max_x * es);
  o.a = take(max_a * es);
  o.b = take(max_a * es);
  o.total = off;
  return o;
}

bool hp_ok(const nc_optim_hparams* h) {
  auto fin = [](float x) { return std::isfinite(x); };
  if (!fin(h->grad_scale) || !fin(h->lr_embed) || !fin(h->lr_unembed) || !fin(h->lr_matrix) ||
      !fin(h->weight_decay) || !fin(h->ns_a) || !fin(h->ns_b) || !fin(h->ns_c))
    return false;
  if (!(h->beta1 >= 0.f && h->beta1 < 1.f) || !(h->beta2 >= 0.f && h->beta2 < 1.f)) return false;
  if (!(h->eps >= 0.f) || !fin(h->eps) || h->adam_step < 1) return false;
  if (!(h->momentum >= 0.f && h->momentum < 1.f)) return false;
  if (h->nesterov != 0 && h->nesterov != 1) return false;
  if (h->ns_steps < 0 || h->ns_steps > 100) return false;
  return true;
}

// AdamW on E or U: p, m at the tensor's parameter offset; v after the
// parameter-sized region (E's first, then U's)
template <typename T>
hipError_t optim_adamw(nc_ctx* ctx, const OptimTensor& t, float* master, T* params, const float* grads, float* state,
                       const nc_optim_hparams* h) {
  const nc_config& c = ctx->cfg;
  const int64_t n = t.rows * t.cols;
  const double lr = t.tensor == NC_T_E ? h->lr_embed : h->lr_unembed;
  AdamwArgs a;
  a.grad_scale = h->grad_scale;
  a.beta1 = h->beta1;
  a.beta2 = h->beta2;
  a.decay = (float)(1.0 - lr * h->weight_decay);
  a.lr = (float)lr;
  a.inv_bc1 = (float)(1.0 / (1.0 - std::pow((double)h->beta1, (double)h->adam_step)));
  a.inv_bc2 = (float)(1.0 / (1.0 - std::pow((double)h->beta2, (double)h->adam_step)));
  a.eps = h->eps;
  float* v = state + param_count_of(c) + (t.tensor == NC_T_E ? 0 : n);
  return traced(ctx, NC_TRACE_OPTIM_ADAMW, 0.0, 30.0 * (double)n, [&] {
    return adamw<T>(n, master + t.off, grads + t.off, state + t.off, v, params + t.off, a, ctx->stream);
  });
}

// Muon on one group of same-shaped matrices: the elementwise parts one
// launch per set (all layers), the Newton-Schulz products batched over the
// whole group
template <typename T>
hipError_t optim_muon(nc_ctx* ctx, const MuonGroup& grp, float* master, T* params, const float* grads, float* state,
                      char* scratch, const OptimScratch& sc, const nc_optim_hparams* h) {
  const int rw = grp.rw, cw = grp.cw, nb = grp.nb;
  const int64_t sx = (int64_t)rw * cw, sa = (int64_t)rw * rw;
  float* partials = reinterpret_cast<float*>(scratch + sc.partials);
  T* X = reinterpret_cast<T*>(scratch + sc.x0);
  T* Xn = reinterpret_cast<T*>(scratch + sc.x1);
  T* A = reinterpret_cast<T*>(scratch + sc.a);
  T* B = reinterpret_cast<T*>(scratch + sc.b);
  hipError_t e = hipSuccess;
  int first = 0;                       // the set's first matrix in the group
  for (const MuonSet& st : grp.sets) {
    float* part = partials + (size_t)first * kMuonMaxPartials;
    if (e == hipSuccess)
      e = muon_momentum((int64_t)st.r * st.c, st.count, st.stride, grads + st.off0, state + st.off0, h->grad_scale,
                        h->momentum, h->nesterov, part, ctx->stream);
    if (e == hipSuccess)
      e = muon_normalise<T>(st.r, st.c, st.count, st.stride, grads + st.off0, state + st.off0, h->grad_scale,
                            h->momentum, h->nesterov, part, 1e-7f, X + first * sx, ctx->stream);
    first += st.count;
  }
  for (int it = 0; it < h->ns_steps && e == hipSuccess; ++it) {
    // A = X X^T
    // (A and B are symmetric: the matrix-core kernel computes their upper
    // tiles and mirrors the rest)
    GemmDesc ga = gemm(rw, rw, cw, X, cw, 0, X, cw, 0, EPI_STORE, A, rw);
    ga.batch = nb; ga.sP = sx; ga.sQ = sx; ga.sC = sa; ga.sym = 1;
    e = run_gemm(ctx, ga, NC_TRACE_OPTIM_NS);
    // B = ns_c A A^T + ns_b A   (A is symmetric, so A A^T = A A)
    if (e == hipSuccess) {
      GemmDesc gb = gemm(rw, rw, rw, A, rw, 0, A, rw, 0, EPI_AXPBY, B, rw);
      gb.aux = A; gb.ldaux = rw; gb.ep_alpha = h->ns_c; gb.ep_gamma = h->ns_b;
      gb.batch = nb; gb.sP = sa; gb.sQ = sa; gb.sC = sa; gb.sAux = sa; gb.sym = 1;
      e = run_gemm(ctx, gb, NC_TRACE_OPTIM_NS);
    }
    // X' = B X + ns_a X
    if (e == hipSuccess) {
      GemmDesc gx = gemm(rw, cw, rw, B, rw, 0, X, cw, 1, EPI_AXPBY, Xn, cw);
      gx.aux = X; gx.ldaux = cw; gx.ep_alpha = 1.f; gx.ep_gamma = h->ns_a;
      gx.batch = nb; gx.sP = sa; gx.sQ = sx; gx.sC = sx; gx.sAux = sx;
      e = run_gemm(ctx, gx, NC_TRACE_OPTIM_NS);
    }
    std::swap(X, Xn);
  }
  first = 0;
  for (const MuonSet& st : grp.sets) {
    const float lr = (float)((double)h->lr_matrix * std::sqrt(std::max(1.0, (double)st.r / st.c)));
    if (e == hipSuccess)
      e = muon_apply<T>(st.r, st.c, st.count, st.stride, X + first * sx, lr, master + st.off0, params + st.off0,
                        ctx->stream);
    first += st.count;
  }
  return e;
}

template <typename T>
int optimizer_step(nc_ctx* ctx, float* master, T* params, const float* grads, float* state, char* scratch,
                   const nc_optim_hparams* h) {
  const OptimScratch sc = optim_scratch(ctx->cfg);
  for (const OptimTensor& t : optim_tensors(ctx->cfg))
    if (t.tensor == NC_T_E || t.tensor == NC_T_U)
      NC_TRY(optim_adamw<T>(ctx, t, master, params, grads, state, h), "AdamW");
  for (const MuonGroup& grp : muon_groups(ctx->cfg))
    NC_TRY(optim_muon<T>(ctx, grp, master, params, grads, state, scratch, sc, h), "Muon");
  return NC_OK;
}

// ---- KV-cache inference -------------------------------------------------------
// decode scratch: x, a, o [mb][d] | qkv [mb][3d] | u [mb][F] (model dtype) |
// r [mb] | rotary row [Q/2] | attention partials [mb][H][chunks][2+Q] (fp32)
struct DecodeScratch {
  size_t x = 0, a = 0, o = 0, qkv = 0, u = 0, r = 0, rope = 0, part = 0, total = 0;
};

DecodeScratch decode_scratch(const nc_config& c, int mb, int ml) {
  const size_t es = esize(c);
  const int64_t d = c.d_model, F = c.d_ff;
  DecodeScratch o;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t r = off; off += align_up(bytes); return r; };
  o.x = take(mb * d * es);
  o.a = take(mb * d * es);
  o.o = take(mb * d * es);
  o.qkv = take(mb * 3 * d * es);
  o.u = take(mb * F * es);
  o.r = take(mb * 4);
  o.rope = take(c.head_dim / 2 * 8);
  o.part = take((size_t)mb * c.n_head * attn_decode_chunks(ml) * (2 + c.head_dim) * 4);
  o.total = off;
  return o;
}

int kv_shape_ok(const nc_config& c, int mb, int ml) {
  if (is_block(c)) return NC_ERR_STATE;
  if (mb < 1 || mb > kMaxDecodeBatch || ml < 1 || ml > (1 << 24)) return NC_ERR_SHAPE;
  if (c.head_dim != 32 && c.head_dim != 64 && c.head_dim != 96 && c.head_dim != 128) return NC_ERR_UNSUPPORTED;
  return NC_OK;
}

template <typename T>
int prefill(nc_ctx* ctx, const T* params, const int32_t* idx, int len, int nseq, T* kv, int mb, int ml,
            float* logits) {
  const nc_config& c = ctx->cfg;
  const Plan& p = ctx->plan;
  const int d = c.d_model, V = c.vocab;
  // the whole forward over the (padded) prompt; its targets are the ids
  // themselves, since only the saved k, v and the final norm are used
  int st = model_forward<T>(ctx, params, idx, idx, nullptr, false);
  if (st != NC_OK) return st;
  ctx->have_forward = true;
  const int64_t sstride = (int64_t)ml * d, lstride = 2 * (int64_t)mb * sstride;
  for (int l = 0; l < c.n_layer; ++l) {
    const T* qkv = reinterpret_cast<const T*>(ctx->layer(l) + p.l_qkv);
    T* K = kv + l * lstride;
    NC_TRY(kv_prefill<T>(qkv, len, d, nseq, K, K + (int64_t)mb * sstride, sstride, ctx->stream), "kv prefill");
  }
  const T* U = params + (int64_t)V * d + (int64_t)c.n_layer * layer_elems(c);
  GemvDesc g{};
  g.nb = 1; g.N = V; g.K = d; g.W = U;
  g.x = ctx->at<T>(p.xf) + (int64_t)(len - 1) * d; g.ldx = d;
  g.y = logits; g.ldy = V;
  NC_TRY(gemv<T>(g, EPI_F32, ctx->stream), "prefill logits");
  return NC_OK;
}

// sc: the layout of `scratch` (any layout at least (nseq, pos + 1) large)
template <typename T>
int decode(nc_ctx* ctx, const T* params, const int32_t* tokens, int nseq, int pos, T* kv, int mb, int ml,
           char* scratch, const DecodeScratch& sc, float* logits) {
  const nc_config& c = ctx->cfg;
  const int d = c.d_model, F = c.d_ff, V = c.vocab, H = c.n_head, Q = c.head_dim;
  hipStream_t s = ctx->stream;
  T* x = reinterpret_cast<T*>(scratch + sc.x);
  T* a = reinterpret_cast<T*>(scratch + sc.a);
  float* r = reinterpret_cast<float*>(scratch + sc.r);
  T* o = reinterpret_cast<T*>(scratch + sc.o);
  T* qkv = reinterpret_cast<T*>(scratch + sc.qkv);
  T* u = reinterpret_cast<T*>(scratch + sc.u);
  float2* rope = reinterpret_cast<float2*>(scratch + sc.rope);
  float* part = reinterpret_cast<float*>(scratch + sc.part);
  NC_TRY(embed_fwd<T>(params, tokens, x, nseq, d, V, s), "decode embedding");
  NC_TRY(rope_table_at(rope, pos, 1, Q, c.rope_base, s), "decode rotary row");
  const int64_t sstride = (int64_t)ml * d, lstride = 2 * (int64_t)mb * sstride;
  const T* w = params + (int64_t)V * d;
  // RMSNorm of the residual stream before qkv, the MLP and the logits: for
  // one or two sequences formed inside those products (41 fewer launches,
  // 1.02 -> 0.96 ms per step at one sequence); for more, each product's
  // extra sum-of-squares reduction costs more than the launch it saves
  // (1.59 -> 1.87 ms at 16), so a separate kernel writes the normed rows.
  const bool fuse_norm = nseq <= 2;
  auto normed = [&](const T** in) -> hipError_t {
    *in = fuse_norm ? x : a;
    return fuse_norm ? hipSuccess : rmsnorm_fwd<T>(x, a, r, nseq, d, c.rms_eps, s);
  };
  // norm: the product is of RMSNorm(xin), formed in the same kernel
  auto gv = [&](const T* W, int N, int K, const T* xin, T* y, int64_t ldy, int epi, int norm) {
    GemvDesc g{};
    g.nb = nseq; g.N = N; g.K = K; g.W = W; g.x = xin; g.ldx = K; g.y = y; g.ldy = ldy; g.aux = y;
    g.rope = rope; g.rope_cols = 2 * d; g.head_dim = Q;
    g.norm = norm; g.norm_eps = c.rms_eps;
    return gemv<T>(g, epi, s);
  };
  for (int l = 0; l < c.n_layer; ++l) {
    const T* lw = w + (int64_t)l * layer_elems(c);
    const T* Wqkv = lw;
    const T* Wo = lw + 3 * (int64_t)d * d;
    const T* W1 = Wo + (int64_t)d * d;
    const T* W2 = W1 + (int64_t)F * d;
    T* K = kv + l * lstride;
    T* Vc = K + (int64_t)mb * sstride;
    {
      // q, k, v of RMSNorm(x) with rotary; k and v also appended to the
      // cache at pos
      const T* xa = nullptr;
      NC_TRY(normed(&xa), "decode rmsnorm (attention)");
      GemvDesc g{};
      g.nb = nseq; g.N = 3 * d; g.K = d; g.W = Wqkv; g.x = xa; g.ldx = d; g.y = qkv; g.ldy = 3 * d;
      g.rope = rope; g.rope_cols = 2 * d; g.head_dim = Q;
      g.kv_K = K; g.kv_V = Vc; g.kv_seq_stride = sstride; g.kv_d = d; g.kv_pos = pos;
      g.norm = fuse_norm; g.norm_eps = c.rms_eps;
      NC_TRY(gemv<T>(g, EPI_ROPE, s), "decode qkv + kv append");
    }
    AttnDecodeDesc ad{};
    ad.H = H; ad.Q = Q; ad.L = pos + 1; ad.nchunks = attn_decode_chunks(pos + 1);
    ad.qkv = qkv; ad.K = K; ad.V = Vc; ad.seq_stride = sstride;
    ad.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)Q));
    ad.part = part; ad.o = o;
    NC_TRY(attn_decode<T>(ad, nseq, s), "decode attention");
    NC_TRY(gv(Wo, d, d, o, x, d, EPI_RESID, 0), "decode attention output");
    const T* xm = nullptr;
    NC_TRY(normed(&xm), "decode rmsnorm (mlp)");
    NC_TRY(gv(W1, F, d, xm, u, F, EPI_RELU2, fuse_norm), "decode mlp up");
    NC_TRY(gv(W2, d, F, u, x, d, EPI_RESID, 0), "decode mlp down");
  }
  const T* xf = nullptr;
  NC_TRY(normed(&xf), "decode final rmsnorm");
  GemvDesc g{};
  g.nb = nseq; g.N = V; g.K = d; g.W = w + (int64_t)c.n_layer * layer_elems(c);
  g.x = xf; g.ldx = d; g.y = logits; g.ldy = V;
  g.norm = fuse_norm; g.norm_eps = c.rms_eps;
  NC_TRY(gemv<T>(g, EPI_F32, s), "decode logits");
  return NC_OK;
}

// ---- allocation-free decode (nc_decode_static) -------------------------------
// The scratch lives in a file-scope device array: every GPU the library runs
// on holds its own copy from the code object's load until the process ends.
// In host code the array's name is only a host-side stand-in, never a device
// address: host code uses the address hipGetSymbolAddress returns, looked up
// once per device (with that device current) and kept per device.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
static __device__ __align__(256) char nc_static_decode_scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices];

// the calling thread's current device's copy of the array
hipError_t static_scratch_address(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(nc_static_decode_scratch));
    if (e != hipSuccess) return e;
    g_static_ptr[dev] = p;
  }
  *out = g_static_ptr[dev];
  return hipSuccess;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

int64_t nc_param_count(const nc_config* cfg) {
  int st = validate(cfg);
  if (st != NC_OK) return st;
  const int64_t per = layer_elems(*cfg) * cfg->n_layer;
  return is_block(*cfg) ? per : per + 2LL * cfg->vocab * cfg->d_model;
}

int nc_param_offset(const nc_config* cfg, int32_t tensor, int32_t layer, int64_t* offset, int64_t* rows,
                    int64_t* cols) {
  int st = validate(cfg);
  if (st != NC_OK) return st;
  if (!offset || !rows || !cols) return NC_ERR_INVALID_ARG;
  const int64_t d = cfg->d_model, F = cfg->d_ff, V = cfg->vocab;
  const int64_t base = is_block(*cfg) ? 0 : V * d;
  if (tensor == NC_T_E || tensor == NC_T_U) {
    if (is_block(*cfg)) return NC_ERR_INVALID_ARG;
    *rows = V; *cols = d;
    *offset = tensor == NC_T_E ? 0 : base + layer_elems(*cfg) * cfg->n_layer;
    return NC_OK;
  }
  if (tensor < NC_T_WQ || tensor > NC_T_W2 || layer < 0 || layer >= cfg->n_layer) return NC_ERR_INVALID_ARG;
  int64_t off = base + layer_elems(*cfg) * layer;
  const int64_t sizes[6][2] = {{d, d}, {d, d}, {d, d}, {d, d}, {F, d}, {d, F}};
  for (int t = NC_T_WQ; t < tensor; ++t) off += sizes[t - NC_T_WQ][0] * sizes[t - NC_T_WQ][1];
  *offset = off;
  *rows = sizes[tensor - NC_T_WQ][0];
  *cols = sizes[tensor - NC_T_WQ][1];
  return NC_OK;
}

int64_t nc_workspace_bytes(const nc_config* cfg) {
  int st = validate(cfg);
  if (st != NC_OK) return st;
  return (int64_t)make_plan(*cfg).total;
}

const char* nc_status_string(int status) {
  switch (status) {
    case NC_OK: return "ok";
    case NC_ERR_INVALID_ARG: return "invalid argument";
    case NC_ERR_SHAPE: return "unsupported or inconsistent shape";
    case NC_ERR_WORKSPACE: return "workspace too small or misaligned";
    case NC_ERR_STATE: return "call out of order";
    case NC_ERR_HIP: return "HIP error";
    case NC_ERR_UNSUPPORTED: return "not supported";
    default: return "unknown status";
  }
}

int nc_init(const nc_config* cfg, void* workspace, size_t ws_bytes, void* hip_stream, nc_ctx** out) {
  if (!out) return NC_ERR_INVALID_ARG;
  *out = nullptr;
  int st = validate(cfg);
  if (st != NC_OK) return st;
  if (!workspace) return NC_ERR_INVALID_ARG;
  Plan plan = make_plan(*cfg);
  if (ws_bytes < plan.total || ((uintptr_t)workspace % kAlign) != 0) return NC_ERR_WORKSPACE;
  nc_ctx* ctx = new (std::nothrow) nc_ctx();
  if (!ctx) return NC_ERR_INVALID_ARG;
  ctx->cfg = *cfg;
  ctx->ws = (char*)workspace;
  ctx->ws_bytes = ws_bytes;
  ctx->stream = (hipStream_t)hip_stream;
  ctx->plan = plan;
  hipError_t e = rope_table(ctx->at<float2>(plan.rope), cfg->seq_len, cfg->head_dim, cfg->rope_base, ctx->stream);
  if (e != hipSuccess) {
    delete ctx;
    return NC_ERR_HIP;
  }
  // the device address of this device's static decode scratch; a failure
  // here only disables nc_decode_static on this context
  const hipError_t se = static_scratch_address(&ctx->static_scratch);
  if (se != hipSuccess) ctx->static_scratch_err = hipGetErrorString(se);
  *out = ctx;
  return NC_OK;
}

int nc_set_stream(nc_ctx* ctx, void* hip_stream) {
  if (!ctx) return NC_ERR_INVALID_ARG;
  ctx->stream = (hipStream_t)hip_stream;
  return NC_OK;
}

void nc_destroy(nc_ctx* ctx) { delete ctx; }

int nc_trace_enable(nc_ctx* ctx, int32_t family) {
  if (!ctx) return NC_ERR_INVALID_ARG;
  if (family < -1 || family >= NC_TRACE_COUNT) return NC_ERR_INVALID_ARG;
  ctx->trace_family = family;
  ctx->n_rec = 0;
  ctx->trace_flops = ctx->trace_bytes = 0.0;
  return NC_OK;
}

int nc_trace_read(nc_ctx* ctx, int64_t* launches, double* ms, double* flops, double* bytes) {
  if (!ctx) return NC_ERR_INVALID_ARG;
  double total = 0.0;
  for (size_t i = 0; i < ctx->n_rec; ++i) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(ctx->ev[2 * i + 1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, ctx->ev[2 * i], ctx->ev[2 * i + 1]);
    if (e != hipSuccess) return fail(ctx, e, "trace read");
    total += t;
  }
  if (launches) *launches = (int64_t)ctx->n_rec;
  if (ms) *ms = total;
  if (flops) *flops = ctx->trace_flops;
  if (bytes) *bytes = ctx->trace_bytes;
  return NC_OK;
}

const char* nc_last_error(const nc_ctx* ctx) { return ctx ? ctx->err.c_str() : "null context"; }

int nc_fallback_count(nc_ctx* ctx, int64_t* count, int32_t reset) {
  if (!ctx || !count || (reset != 0 && reset != 1)) return NC_ERR_INVALID_ARG;
  *count = ctx->fallbacks;
  if (reset) ctx->fallbacks = 0;
  return NC_OK;
}

int nc_forward(nc_ctx* ctx, const void* params, const int32_t* idx, const int32_t* targets, float* ce_out) {
  if (!ctx || !params || !idx || !targets) return NC_ERR_INVALID_ARG;
  if (is_block(ctx->cfg)) return NC_ERR_STATE;
  ctx->have_forward = false;
  int st = is_bf16(ctx->cfg) ? model_forward<bf16>(ctx, (const bf16*)params, idx, targets, ce_out)
                             : model_forward<float>(ctx, (const float*)params, idx, targets, ce_out);
  ctx->have_forward = st == NC_OK;
  return st;
}

int nc_forward_eval(nc_ctx* ctx, const void* params, const int32_t* idx, const int32_t* targets, float* ce_out) {
  if (!ctx || !params || !idx || !targets) return NC_ERR_INVALID_ARG;
  if (is_block(ctx->cfg)) return NC_ERR_STATE;
  ctx->have_forward = false;
  int st = is_bf16(ctx->cfg) ? model_forward<bf16>(ctx, (const bf16*)params, idx, targets, ce_out, false)
                             : model_forward<float>(ctx, (const float*)params, idx, targets, ce_out, false);
  ctx->have_forward = st == NC_OK;
  return st;
}

int nc_loss_bpb(nc_ctx* ctx, const int32_t* token_bytes, double* out) {
  if (!ctx || !token_bytes || !out) return NC_ERR_INVALID_ARG;
  if (!ctx->have_forward) return NC_ERR_STATE;
  const Plan& p = ctx->plan;
  const int64_t N = (int64_t)ctx->cfg.batch * ctx->cfg.seq_len;
  NC_TRY(loss_bpb(ctx->at<float>(p.ce), ctx->at<int32_t>(p.tgt), token_bytes, N, ctx->cfg.vocab, out, ctx->stream),
         "loss / bpb");
  return NC_OK;
}

int nc_backward(nc_ctx* ctx, const void* params, float* grads, int32_t accumulate) {
  if (!ctx || !params || !grads) return NC_ERR_INVALID_ARG;
  if (accumulate != 0 && accumulate != 1) return NC_ERR_INVALID_ARG;
  if (!ctx->have_forward) return NC_ERR_STATE;
  return is_bf16(ctx->cfg) ? model_backward<bf16>(ctx, (const bf16*)params, grads, accumulate, nullptr)
                           : model_backward<float>(ctx, (const float*)params, grads, accumulate, nullptr);
}

int nc_backward_weighted(nc_ctx* ctx, const void* params, float* grads, int32_t accumulate,
                         const float* token_weights) {
  if (!ctx || !params || !grads || !token_weights) return NC_ERR_INVALID_ARG;
  if (accumulate != 0 && accumulate != 1) return NC_ERR_INVALID_ARG;
  if (!ctx->have_forward) return NC_ERR_STATE;
  return is_bf16(ctx->cfg) ? model_backward<bf16>(ctx, (const bf16*)params, grads, accumulate, token_weights)
                           : model_backward<float>(ctx, (const float*)params, grads, accumulate, token_weights);
}

int nc_loss_weighted(nc_ctx* ctx, const float* token_weights, double* out) {
  if (!ctx || !token_weights || !out) return NC_ERR_INVALID_ARG;
  if (!ctx->have_forward) return NC_ERR_STATE;
  const Plan& p = ctx->plan;
  const int64_t N = (int64_t)ctx->cfg.batch * ctx->cfg.seq_len;
  NC_TRY(weighted_loss(ctx->at<float>(p.ce), ctx->at<int32_t>(p.tgt), token_weights, N, out, ctx->stream),
         "weighted loss");
  return NC_OK;
}

int nc_block_forward(nc_ctx* ctx, const void* block_params, const void* x, void* y) {
  if (!ctx || !block_params || !x || !y) return NC_ERR_INVALID_ARG;
  if (!is_block(ctx->cfg)) return NC_ERR_STATE;
  if (x == y) return NC_ERR_INVALID_ARG;
  ctx->have_block_forward = false;
  int st = is_bf16(ctx->cfg) ? block_forward<bf16>(ctx, (const bf16*)block_params, (const bf16*)x, (bf16*)y)
                             : block_forward<float>(ctx, (const float*)block_params, (const float*)x, (float*)y);
  ctx->have_block_forward = st == NC_OK;
  return st;
}

int nc_block_backward(nc_ctx* ctx, const void* block_params, const void* dy, void* dx, float* dparams,
                      int32_t accumulate) {
  if (!ctx || !block_params || !dy || !dx || !dparams) return NC_ERR_INVALID_ARG;
  if (accumulate != 0 && accumulate != 1) return NC_ERR_INVALID_ARG;
  if (!is_block(ctx->cfg) || !ctx->have_block_forward) return NC_ERR_STATE;
  if (dy == dx) return NC_ERR_INVALID_ARG;
  return is_bf16(ctx->cfg)
             ? block_backward<bf16>(ctx, (const bf16*)block_params, (const bf16*)dy, (bf16*)dx, dparams, accumulate)
             : block_backward<float>(ctx, (const float*)block_params, (const float*)dy, (float*)dx, dparams,
                                     accumulate);
}

int nc_optim_default(const nc_config* cfg, int64_t it, int64_t num_iters, int32_t n_micro, nc_optim_hparams* out) {
  int st = validate(cfg);
  if (st != NC_OK) return st;
  if (!out || it < 0 || num_iters <= 0 || it > num_iters || n_micro < 1) return NC_ERR_INVALID_ARG;
  // lrm: 1 until the last 20 % of the iterations, then linear to 0
  const double warmdown = 0.2, final_frac = 0.0;
  const double progress = (double)it / (double)num_iters;
  const double lrm = progress < 1.0 - warmdown ? 1.0 : final_frac + (1.0 - final_frac) * (1.0 - progress) / warmdown;
  const double width = std::pow((double)cfg->d_model / 768.0, -0.5);
  const double frac = std::min((double)it / 300.0, 1.0);
  out->grad_scale = (float)(1.0 / n_micro);
  out->lr_embed = (float)(0.2 * width * lrm);
  out->lr_unembed = (float)(0.004 * width * lrm);
  out->beta1 = 0.8f;
  out->beta2 = 0.95f;
  out->eps = 1e-10f;
  out->weight_decay = 0.f;
  out->adam_step = (int32_t)std::min<int64_t>(it + 1, INT32_MAX);
  out->lr_matrix = (float)(0.02 * lrm);
  out->momentum = (float)((1.0 - frac) * 0.85 + frac * 0.95);
  out->nesterov = 1;
  out->ns_steps = 5;
  out->ns_a = 3.4445f;
  out->ns_b = -4.7750f;
  out->ns_c = 2.0315f;
  return NC_OK;
}

int64_t nc_optim_state_bytes(const nc_config* cfg) {
  int st = validate(cfg);
  if (st != NC_OK) return st;
  const int64_t extra = is_block(*cfg) ? 0 : 2 * (int64_t)cfg->vocab * cfg->d_model;
  return (param_count_of(*cfg) + extra) * 4;
}

int64_t nc_optim_scratch_bytes(const nc_config* cfg) {
  int st = validate(cfg);
  if (st != NC_OK) return st;
  return (int64_t)optim_scratch(*cfg).total;
}

int nc_optimizer_step(nc_ctx* ctx, float* master, void* params, const float* grads, void* state, void* scratch,
                      const nc_optim_hparams* hp) {
  if (!ctx || !master || !params || !grads || !state || !scratch || !hp) return NC_ERR_INVALID_ARG;
  if (!hp_ok(hp)) return NC_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(scratch) & (kAlign - 1)) || (reinterpret_cast<uintptr_t>(state) & 15) ||
      (reinterpret_cast<uintptr_t>(master) & 15) || (reinterpret_cast<uintptr_t>(grads) & 15) ||
      (reinterpret_cast<uintptr_t>(params) & 7))
    return NC_ERR_INVALID_ARG;
  return is_bf16(ctx->cfg)
             ? optimizer_step<bf16>(ctx, master, (bf16*)params, grads, (float*)state, (char*)scratch, hp)
             : optimizer_step<float>(ctx, master, (float*)params, grads, (float*)state, (char*)scratch, hp);
}

int nc_sample(const float* logits, int32_t n, int32_t V, float temperature, int32_t top_k, const float* u,
              int32_t* out, void* hip_stream) {
  if (!logits || !u || !out) return NC_ERR_INVALID_ARG;
  if (!(temperature >= 0.f) || !std::isfinite(temperature) || top_k < 0) return NC_ERR_INVALID_ARG;
  if (n < 1 || V < 1 || V > 65536) return NC_ERR_SHAPE;
  return sample(logits, n, V, temperature, top_k, u, out, (hipStream_t)hip_stream) == hipSuccess ? NC_OK
                                                                                                   : NC_ERR_HIP;
}

int64_t nc_sample_scratch_bytes(int32_t n, int32_t V) {
  if (n < 1 || n > 65535 || V < 1 || V > 65536) return NC_ERR_SHAPE;
  return sample_parallel_scratch_bytes(n, V);
}

int nc_sample_parallel(const float* logits, int32_t n, int32_t V, float temperature, int32_t top_k, const float* u,
                       int32_t* out, void* scratch, void* hip_stream) {
  if (!logits || !u || !out || !scratch) return NC_ERR_INVALID_ARG;
  if (!(temperature >= 0.f) || !std::isfinite(temperature) || top_k < 0) return NC_ERR_INVALID_ARG;
  if (n < 1 || n > 65535 || V < 1 || V > 65536) return NC_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(scratch) % 256) return NC_ERR_WORKSPACE;
  return sample_parallel(logits, n, V, temperature, top_k, u, out, scratch, (hipStream_t)hip_stream) == hipSuccess
             ? NC_OK
             : NC_ERR_HIP;
}

int64_t nc_kv_cache_bytes(const nc_config* cfg, int32_t max_batch, int32_t max_len) {
  int st = validate(cfg);
  if (st != NC_OK) return st;
  st = kv_shape_ok(*cfg, max_batch, max_len);
  if (st != NC_OK) return st;
  return 2 * (int64_t)cfg->n_layer * max_batch * max_len * cfg->d_model * (int64_t)esize(*cfg);
}

int64_t nc_decode_scratch_bytes(const nc_config* cfg, int32_t max_batch, int32_t max_len) {
  int st = validate(cfg);
  if (st != NC_OK) return st;
  st = kv_shape_ok(*cfg, max_batch, max_len);
  if (st != NC_OK) return st;
  return (int64_t)decode_scratch(*cfg, max_batch, max_len).total;
}

int nc_prefill(nc_ctx* ctx, const void* params, const int32_t* idx, int32_t prompt_len, int32_t nseq,
               void* kv_cache, int32_t max_batch, int32_t max_len, float* logits) {
  if (!ctx || !params || !idx || !kv_cache || !logits) return NC_ERR_INVALID_ARG;
  int st = kv_shape_ok(ctx->cfg, max_batch, max_len);
  if (st != NC_OK) return st;
  if (ctx->cfg.batch != 1) return NC_ERR_SHAPE;
  if (prompt_len < 1 || prompt_len > ctx->cfg.seq_len || prompt_len > max_len) return NC_ERR_SHAPE;
  if (nseq < 1 || nseq > max_batch) return NC_ERR_SHAPE;
  ctx->have_forward = false;
  return is_bf16(ctx->cfg)
             ? prefill<bf16>(ctx, (const bf16*)params, idx, prompt_len, nseq, (bf16*)kv_cache, max_batch, max_len,
                             logits)
             : prefill<float>(ctx, (const float*)params, idx, prompt_len, nseq, (float*)kv_cache, max_batch, max_len,
                              logits);
}

int nc_decode(nc_ctx* ctx, const void* params, const int32_t* tokens, int32_t nseq, int32_t pos, void* kv_cache,
              int32_t max_batch, int32_t max_len, void* scratch, float* logits) {
  if (!ctx || !params || !tokens || !kv_cache || !scratch || !logits) return NC_ERR_INVALID_ARG;
  int st = kv_shape_ok(ctx->cfg, max_batch, max_len);
  if (st != NC_OK) return st;
  if (nseq < 1 || nseq > max_batch || pos < 0 || pos >= max_len) return NC_ERR_SHAPE;
  if (reinterpret_cast<uintptr_t>(scratch) & (kAlign - 1)) return NC_ERR_INVALID_ARG;
  const DecodeScratch sc = decode_scratch(ctx->cfg, max_batch, max_len);
  return is_bf16(ctx->cfg)
             ? decode<bf16>(ctx, (const bf16*)params, tokens, nseq, pos, (bf16*)kv_cache, max_batch, max_len,
                            (char*)scratch, sc, logits)
             : decode<float>(ctx, (const float*)params, tokens, nseq, pos, (float*)kv_cache, max_batch, max_len,
                             (char*)scratch, sc, logits);
}

int64_t nc_decode_static_max_bytes(void) { return (int64_t)kStaticScratchBytes; }

int nc_decode_static(nc_ctx* ctx, const void* params, const int32_t* tokens, int32_t nseq, int32_t pos,
                     void* kv_cache, int32_t max_batch, int32_t max_len, float* logits) {
  if (!ctx || !params || !tokens || !kv_cache || !logits) return NC_ERR_INVALID_ARG;
  int st = kv_shape_ok(ctx->cfg, max_batch, max_len);
  if (st != NC_OK) return st;
  if (nseq < 1 || nseq > max_batch || pos < 0 || pos >= max_len) return NC_ERR_SHAPE;
  // the scratch is laid out for this call's own size (nseq sequences,
  // pos + 1 cached positions), not for the cache's maximum
  const DecodeScratch sc = decode_scratch(ctx->cfg, nseq, pos + 1);
  if (sc.total > kStaticScratchBytes) {
    ctx->err = "nc_decode_static: this call needs " + std::to_string(sc.total) +
               " bytes of scratch, more than the static maximum of " + std::to_string(kStaticScratchBytes);
    return NC_ERR_WORKSPACE;
  }
  if (!ctx->static_scratch) {
    ctx->err = "nc_decode_static: the static scratch's device address is unknown: " + ctx->static_scratch_err;
    return NC_ERR_HIP;
  }
  char* scratch = (char*)ctx->static_scratch;
  return is_bf16(ctx->cfg)
             ? decode<bf16>(ctx, (const bf16*)params, tokens, nseq, pos, (bf16*)kv_cache, max_batch, max_len,
                            scratch, sc, logits)
             : decode<float>(ctx, (const float*)params, tokens, nseq, pos, (float*)kv_cache, max_batch, max_len,
                             scratch, sc, logits);
}

}  // extern "C"
