// KV-cache inference kernels (nanochat speedrun walkthrough, section
// Pretraining, the sampling paragraph: a custom Engine with a KV cache and
// the two phases prefill and decode).  Decode processes one new token for
// each of a few sequences: every weight is read once per token, so each
// product is a matrix-vector product bound by HBM, not by the matrix cores.
// Here it is a VALU kernel that streams weight rows with coalesced 16-byte
// loads from every CU, with the training step's epilogues (rotary, residual,
// relu^2) fused.  Attention over the cache splits each sequence's keys into
// chunks, one workgroup per (chunk, head, sequence), and a second pass
// combines the chunks' (max, sum, output).
#include "nc_internal.h"

namespace nc {
namespace {

constexpr int kWaveD = 64;
constexpr int kCols = 4;           // output columns per wave of the matrix-vector product

template <typename T> struct V16;   // 16 bytes of T as floats
template <> struct V16<float> {
  static constexpr int n = 4;
  __device__ static inline void load(const float* p, float (&o)[4]) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
};
template <> struct V16<bf16> {
  static constexpr int n = 8;
  __device__ static inline void unpack(const uint4 v, float (&o)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static inline void load(const bf16* p, float (&o)[8]) { unpack(*reinterpret_cast<const uint4*>(p), o); }
};
template <> struct V16<float>;
__device__ inline void unpack16(const uint4 v, float (&o)[4]) {
  o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y); o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
}
__device__ inline void unpack16(const uint4 v, float (&o)[8]) { V16<bf16>::unpack(v, o); }

// y[b][n] = epi(sum_k x[b][k] W[n][k]) for b < nb (<= kMaxDecodeBatch), W
// [N][K] row-major in T, x [nb][K].  Workgroup g owns columns 4g .. 4g+3;
// its 4 waves take interleaved 16-byte pieces of K (wave w, lane l: pieces
// 64w + l + 256i), so 256 coalesced pieces of each row are in flight per
// step.  Partial sums are combined by a butterfly within each wave and then
// across the waves in LDS, in a fixed order.
//
// NORM: the input rows are the residual stream x and the product is taken
// of RMSNorm(x); each wave also sums x^2 over its share of K (the same
// pieces it multiplies), and the finishing lane scales its output by
// r = 1 / sqrt(sum / K + eps) -- the norm is linear in x, so
// sum_k (r x_k) w_k = r sum_k x_k w_k.  Nothing is rounded to bf16 between
// the norm and the product.
template <typename T, int EPI, int S, bool NORM>
__global__ void __launch_bounds__(256) k_gemv(GemvDesc g) {
  // S waves share a group of kCols columns, splitting K (S = 4: one group per
  // workgroup, for products with long rows; S = 1: four groups per
  // workgroup, each wave its own, for the wide logits product and for rows
  // of up to 2048)
  constexpr int VE = V16<T>::n;
  __shared__ float red[4][kMaxDecodeBatch * kCols];
  __shared__ float red_sq[4][NORM ? kMaxDecodeBatch : 1];
  float sq[NORM ? kMaxDecodeBatch : 1];
#pragma unroll
  for (int b = 0; b < (NORM ? kMaxDecodeBatch : 1); ++b) sq[b] = 0.f;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = wave / S, sub = wave % S;
  const int64_t n0 = ((int64_t)blockIdx.x * (4 / S) + grp) * kCols;   // < N: the launch covers N exactly
  const T* W = (const T*)g.W;
  const T* x = (const T*)g.x;
  float acc[kMaxDecodeBatch][kCols];
#pragma unroll
  for (int b = 0; b < kMaxDecodeBatch; ++b)
#pragma unroll
    for (int c = 0; c < kCols; ++c) acc[b][c] = 0.f;
  for (int k = (sub * 64 + lane) * VE; k < g.K; k += S * 64 * VE) {
    // every load of the step is issued before any arithmetic: the weight
    // rows' pieces and each sequence's input piece, as raw 16-byte words
    uint4 wr[kCols], xr[kMaxDecodeBatch];
#pragma unroll
    for (int c = 0; c < kCols; ++c) wr[c] = *reinterpret_cast<const uint4*>(W + (n0 + c) * (int64_t)g.K + k);
#pragma unroll
    for (int b = 0; b < kMaxDecodeBatch; ++b)
      xr[b] = b < g.nb ? *reinterpret_cast<const uint4*>(x + (int64_t)b * g.ldx + k) : make_uint4(0, 0, 0, 0);
    float w[kCols][VE];
#pragma unroll
    for (int c = 0; c < kCols; ++c) unpack16(wr[c], w[c]);
#pragma unroll
    for (int b = 0; b < kMaxDecodeBatch; ++b) {
      if (b < g.nb) {
        float xv[VE];
        unpack16(xr[b], xv);
#pragma unroll
        for (int c = 0; c < kCols; ++c)
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[b][c] = fmaf(xv[e], w[c][e], acc[b][c]);
        if constexpr (NORM) {
#pragma unroll
          for (int e = 0; e < VE; ++e) sq[b] = fmaf(xv[e], xv[e], sq[b]);
        }
      }
    }
  }
  // reduce-scatter butterfly over the 64 (sequence, column) sums: at step
  // s a lane keeps the half of its values selected by lane bit s and adds
  // the partner's copy of that half, so after 6 steps (63 shuffles, not
  // 6 per value) lane l holds the wave's total of value l = b * kCols + c
  static_assert(kMaxDecodeBatch * kCols == 64, "one value per lane");
  if (g.nb <= 2) {
    // few values: a full butterfly per value is cheaper (6 shuffles each)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (b < g.nb) {
#pragma unroll
        for (int c = 0; c < kCols; ++c) {
          float t = acc[b][c];
          for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
          if (lane == 0) red[wave][b * kCols + c] = t;
        }
      }
    }
  } else {
  float vals[64];
#pragma unroll
  for (int b = 0; b < kMaxDecodeBatch; ++b)
#pragma unroll
    for (int c = 0; c < kCols; ++c) vals[b * kCols + c] = acc[b][c];
#pragma unroll
  for (int st = 5; st >= 0; --st) {
    const int half = 1 << st;
    const bool upper = (lane >> st) & 1;
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float send = upper ? vals[i] : vals[i + half];
      const float keep = upper ? vals[i + half] : vals[i];
      vals[i] = keep + __shfl_xor(send, half, 64);
    }
  }
  red[wave][lane] = vals[0];
  }
  if constexpr (NORM) {
    for (int b = 0; b < g.nb; ++b) {
      float t = sq[b];
      for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
      if (lane == 0) red_sq[wave][b] = t;
    }
  }
  auto total = [&](int t) {
    if constexpr (S == 4) return (red[0][t] + red[1][t]) + (red[2][t] + red[3][t]);
    else return red[wave][t];
  };
  __syncthreads();
  // lane b * kCols + c of the group's first wave finishes output (b, n0 + c)
  const int t = lane;
  if (sub != 0 || t >= g.nb * kCols) return;
  const int b = t / kCols, c = t % kCols;
  const int64_t n = n0 + c;
  float rs = 1.f;                                   // the row's RMSNorm scale
  if constexpr (NORM) {
    // S = 4: the group's waves split K; S = 1: the wave saw all of K
    const float ss = S == 4 ? (red_sq[0][b] + red_sq[1][b]) + (red_sq[2][b] + red_sq[3][b]) : red_sq[wave][b];
    rs = 1.f / __builtin_sqrtf(ss / (float)g.K + g.norm_eps);
  }
  float v = total(t) * rs;
  if constexpr (EPI == EPI_ROPE) {
    // adjacent pairs (2i, 2i+1) of the rotated columns, angles of one position
    if (n < g.rope_cols) {
      const int tp = t ^ 1;
      const float other = total(tp) * rs;
      const float2 cs = g.rope[(n % g.head_dim) >> 1];
      v = (c & 1) ? other * cs.y + v * cs.x : v * cs.x - other * cs.y;
    }
  }
  if constexpr (EPI == EPI_RESID) v += to_f32(((const T*)g.aux)[(int64_t)b * g.ldy + n]);
  if constexpr (EPI == EPI_RELU2) v = fmaxf(v, 0.f) * fmaxf(v, 0.f);
  if constexpr (EPI == EPI_F32) {
    ((float*)g.y)[(int64_t)b * g.ldy + n] = v;
  } else {
    const T out = from_f32<T>(v);
    ((T*)g.y)[(int64_t)b * g.ldy + n] = out;
    // the qkv product also appends k and v to the cache at position pos
    if constexpr (EPI == EPI_ROPE) {
      if (g.kv_K && n >= g.kv_d) {
        T* dst = n < 2 * g.kv_d ? (T*)g.kv_K + (n - g.kv_d) : (T*)g.kv_V + (n - 2 * g.kv_d);
        dst[(int64_t)b * g.kv_seq_stride + (int64_t)g.kv_pos * g.kv_d] = out;
      }
    }
  }
}

// copy k and v of the new token (columns d .. 3d of qkv [nb][3d]) into the
// cache at position pos: K[b][pos][:], V[b][pos][:]
template <typename T>
__global__ void __launch_bounds__(256) k_kv_append(const T* __restrict__ qkv, int nb, int d, T* __restrict__ K,
                                                     T* __restrict__ V, int64_t seq_stride, int pos) {
  const int b = blockIdx.y;
  for (int i = threadIdx.x + blockIdx.x * 256; i < d; i += 256 * gridDim.x) {
    K[(int64_t)b * seq_stride + (int64_t)pos * d + i] = qkv[(int64_t)b * 3 * d + d + i];
    V[(int64_t)b * seq_stride + (int64_t)pos * d + i] = qkv[(int64_t)b * 3 * d + 2 * d + i];
  }
}

// prefill: rows t < len of the forward's qkv [rows][3d] into sequences
// 0 .. nb-1 of the cache (the same prompt for every sequence)
template <typename T>
__global__ void __launch_bounds__(256) k_kv_prefill(const T* __restrict__ qkv, int len, int d, int nb,
                                                     T* __restrict__ K, T* __restrict__ V, int64_t seq_stride) {
  const int t = blockIdx.x, b = blockIdx.y;
  if (t >= len) return;
  for (int i = threadIdx.x; i < d; i += 256) {
    K[(int64_t)b * seq_stride + (int64_t)t * d + i] = qkv[(int64_t)t * 3 * d + d + i];
    V[(int64_t)b * seq_stride + (int64_t)t * d + i] = qkv[(int64_t)t * 3 * d + 2 * d + i];
  }
}

// Decode attention, pass 1: workgroup (chunk, h, b) scores keys
// [64 chunk, +64) of sequence b against q (head h), L keys in all, and
// writes the chunk's max m, sum l and unnormalised output o[Q] (fp32) to
// part[b][h][chunk] = {m, l, o[Q]}.  Four threads share a key's dot product
// (Q/4 dimensions each); for the values, wave w takes keys 16w .. 16w+15
// and lane l dimensions 2l, 2l+1, one coalesced row per key.
template <typename T, int Q>
__global__ void __launch_bounds__(256) k_attn_decode(AttnDecodeDesc a) {
  constexpr int kChunk = 64, QP = Q / 4;
  static_assert(Q % 32 == 0 && Q <= 128, "head dim");
  __shared__ float qs[Q];
  __shared__ float ps[kChunk];
  __shared__ float red[8];
  __shared__ float os[4][Q];
  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int d = a.H * Q;
  const T* q = (const T*)a.qkv + (int64_t)b * 3 * d + h * Q;
  if (tid < Q) qs[tid] = to_f32(q[tid]);
  __syncthreads();
  const int64_t base = (int64_t)b * a.seq_stride + h * Q;
  const int jl = tid >> 2, part = tid & 3;
  const int j = chunk * kChunk + jl;
  float s = 0.f;
  if (j < a.L) {
    const T* kr = (const T*)a.K + base + (int64_t)j * d + part * QP;
#pragma unroll
    for (int i = 0; i < QP; i += V16<T>::n) {
      float kv[V16<T>::n];
      V16<T>::load(kr + i, kv);
#pragma unroll
      for (int e = 0; e < V16<T>::n; ++e) s = fmaf(qs[part * QP + i + e], kv[e], s);
    }
  }
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  const float sc = j < a.L ? s * a.scale_log2 : -INFINITY;
  float mx = sc;
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float p = j < a.L ? __builtin_amdgcn_exp2f(sc - M) : 0.f;
  if (part == 0) ps[jl] = p;
  float l = part == 0 ? p : 0.f;
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
  __syncthreads();
  if (lane == 0) red[4 + wave] = l;
  float o0 = 0.f, o1 = 0.f;
  const int jn = min(kChunk, a.L - chunk * kChunk);
  if (2 * lane < Q) {
#pragma unroll 4
    for (int jj = wave * 16; jj < min(wave * 16 + 16, jn); ++jj) {
      const T* vr = (const T*)a.V + base + (int64_t)(chunk * kChunk + jj) * d + 2 * lane;
      const float pj = ps[jj];
      o0 = fmaf(pj, to_f32(vr[0]), o0);
      o1 = fmaf(pj, to_f32(vr[1]), o1);
    }
    os[wave][2 * lane] = o0;
    os[wave][2 * lane + 1] = o1;
  }
  __syncthreads();
  float* out = a.part + (((int64_t)b * a.H + h) * a.nchunks + chunk) * (2 + Q);
  if (tid == 0) {
    out[0] = M;
    out[1] = (red[4] + red[5]) + (red[6] + red[7]);
  }
  if (tid < Q) out[2 + tid] = (os[0][tid] + os[1][tid]) + (os[2][tid] + os[3][tid]);
}

// pass 2: combine the chunks of (h, b): o = sum_c 2^(m_c - M) o_c / sum_c 2^(m_c - M) l_c
template <typename T>
__global__ void __launch_bounds__(128) k_attn_decode_combine(AttnDecodeDesc a) {
  const int h = blockIdx.x, b = blockIdx.y, i = threadIdx.x;
  const int Q = a.Q;
  const float* part = a.part + ((int64_t)b * a.H + h) * a.nchunks * (2 + Q);
  float M = -INFINITY;
#pragma unroll 8
  for (int c = 0; c < a.nchunks; ++c) M = fmaxf(M, part[c * (2 + Q)]);
  float num = 0.f, den = 0.f;
#pragma unroll 8
  for (int c = 0; c < a.nchunks; ++c) {
    const float w = __builtin_amdgcn_exp2f(part[c * (2 + Q)] - M);
    den = fmaf(w, part[c * (2 + Q) + 1], den);
    if (i < Q) num = fmaf(w, part[c * (2 + Q) + 2 + i], num);
  }
  if (i < Q) ((T*)a.o)[(int64_t)b * a.H * Q + h * Q + i] = from_f32<T>(num / den);
}

// order-preserving map of a float to uint32 (larger float -> larger key)
__device__ inline uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Next token of row blockIdx.x of logits [n][V] (see nc_sample).  Every
// pass reads the row coalesced.  The max and the digit counts stride over
// the row; for the weights, wave w owns the contiguous ids [w S, (w+1) S)
// and lane l the ids w S + 64 j + l, so the inverse-CDF walk is a
// wave-wide scan, 64 ids per step.  Every sum runs in a fixed order.
__global__ void __launch_bounds__(1024) k_sample(const float* __restrict__ logits, int V, float temperature,
                                                  int top_k, const float* __restrict__ u, int32_t* __restrict__ out) {
  constexpr int NT = 1024, NW = NT / 64;
  __shared__ float smax[NW];
  __shared__ int sarg[NW];
  __shared__ int hist[NW][16];
  __shared__ double wsum[NW];
  __shared__ int wlast[NW];
  __shared__ int s_bin, s_k, s_found;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* z = logits + (int64_t)blockIdx.x * V;
  // 1. largest logit, first id on ties
  float mx = -INFINITY;
  int am = V;
#pragma unroll 8
  for (int i = tid; i < V; i += NT)
    if (z[i] > mx || am == V) { mx = z[i]; am = i; }
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(mx, o, 64);
    const int a2 = __shfl_xor(am, o, 64);
    if (a2 != V && (am == V || m2 > mx || (m2 == mx && a2 < am))) { mx = m2; am = a2; }
  }
  if (lane == 0) { smax[wave] = mx; sarg[wave] = am; }
  __syncthreads();
  float zmax = smax[0];
  int amax = sarg[0];
  for (int w = 1; w < NW; ++w)
    if (sarg[w] != V && (amax == V || smax[w] > zmax || (smax[w] == zmax && sarg[w] < amax))) {
      zmax = smax[w];
      amax = sarg[w];
    }
  if (temperature == 0.f) {
    if (tid == 0) out[blockIdx.x] = amax;
    return;
  }
  // 2. the k-th largest key, 4 bits per pass (ties at it are all kept);
  // per-thread counts as 8-bit fields of 4 registers (at most V/1024 <= 64
  // keys a thread, checked at launch), summed by a butterfly per wave and
  // over the waves in LDS
  uint32_t prefix = 0, mask = 0;
  const bool select = top_k > 0 && top_k < V;
  if (select) {
    if (tid == 0) s_k = top_k;
    for (int shift = 28; shift >= 0; shift -= 4) {
      uint32_t pk0 = 0, pk1 = 0, pk2 = 0, pk3 = 0;
#pragma unroll 8
      for (int i = tid; i < V; i += NT) {
        const uint32_t key = fkey(z[i]);
        if ((key & mask) != prefix) continue;
        const uint32_t dgt = (key >> shift) & 15u;
        const uint32_t inc = 1u << (8 * (dgt & 3u));
        const uint32_t q = dgt >> 2;
        pk0 += q == 0 ? inc : 0u;
        pk1 += q == 1 ? inc : 0u;
        pk2 += q == 2 ? inc : 0u;
        pk3 += q == 3 ? inc : 0u;
      }
#pragma unroll
      for (int dg = 0; dg < 16; ++dg) {
        const uint32_t word = dg < 4 ? pk0 : dg < 8 ? pk1 : dg < 12 ? pk2 : pk3;
        int c = (int)((word >> (8 * (dg & 3))) & 255u);
        for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
        if (lane == 0) hist[wave][dg] = c;
      }
      __syncthreads();
      if (tid == 0) {
        int cum = 0, k = s_k, b = 15;
        for (; b > 0; --b) {
          int hb = 0;
          for (int w = 0; w < NW; ++w) hb += hist[w][b];
          if (cum + hb >= k) break;
          cum += hb;
        }
        s_bin = b;
        s_k = k - cum;
      }
      __syncthreads();
      prefix |= (uint32_t)s_bin << shift;
      mask |= 15u << shift;
    }
  }
  const uint32_t thr = prefix;
  const float wscale = 1.4426950408889634f / temperature;
  auto weight = [&](int i) -> float {   // 0 outside the row and for ids not kept
    if (i >= V) return 0.f;
    const float zi = z[i];
    if (select && fkey(zi) < thr) return 0.f;
    return __builtin_amdgcn_exp2f((zi - zmax) * wscale);
  };
  // 3. wave w owns the ids [w S, (w+1) S), S a multiple of 64, and lane l
  // the block of 64 ids w S + 64 l .. +63 (S <= 4096 ids, one block per
  // lane).  Each lane sums its block (fp32 weights, fp64 sum, in id
  // order); a lane scan gives the blocks' running sums and the wave total.
  const int S = ((V + NW - 1) / NW + 63) / 64 * 64;
  const int w0 = wave * S, w1 = min(V, w0 + S);
  const int b0 = w0 + 64 * lane, b1 = min(w1, b0 + 64);
  double bsum = 0.0;
  int blast = -1;
#pragma unroll 8
  for (int i = b0; i < b1; ++i) {
    bsum += (double)weight(i);
    if (!select || fkey(z[i]) >= thr) blast = i;
  }
  double incl = bsum;
  for (int o = 1; o < 64; o <<= 1) {
    const double up = __shfl_up(incl, o, 64);
    if (lane >= o) incl += up;
  }
  int last = blast;
  for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
  if (lane == 63) wsum[wave] = incl;
  if (lane == 0) wlast[wave] = last;
  if (tid == 0) s_found = 0;
  __syncthreads();
  double total = 0.0, excl = 0.0;
  for (int w = 0; w < NW; ++w) {
    if (w == wave) excl = total;
    total += wsum[w];
  }
  const double target = (double)u[blockIdx.x] * total;
  // 4. the wave whose range holds the target picks the block that crosses
  // it, then scans that block's 64 ids
  if (excl <= target && target < excl + wsum[wave]) {
    const unsigned long long cross = __ballot(bsum > 0.0 && excl + incl > target);
    int pick = wlast[wave];    // if rounding leaves no crossing: the range's last kept id
    if (cross) {
      const int jb = __ffsll((long long)cross) - 1;          // the crossing block
      const double before = excl + __shfl(incl - bsum, jb, 64);
      const int i = w0 + 64 * jb + lane;
      const double wi = i < w1 ? (double)weight(i) : 0.0;
      double run = wi;
      for (int o = 1; o < 64; o <<= 1) {
        const double up = __shfl_up(run, o, 64);
        if (lane >= o) run += up;
      }
      const unsigned long long hit = __ballot(wi > 0.0 && before + run > target);
      pick = hit ? w0 + 64 * jb + __ffsll((long long)hit) - 1 : __shfl(blast, jb, 64);
    }
    if (lane == 0) {
      out[blockIdx.x] = pick;
      s_found = 1;
    }
  }
  __syncthreads();
  if (!s_found && tid == 0) {
    // rounding left no id past the target: the row's last kept id
    int l = -1;
    for (int w = 0; w < NW; ++w) l = max(l, wlast[w]);
    out[blockIdx.x] = l;
  }
}

// ---------------------------------------------------------------------------
// The same draw spread over many workgroups: each row is cut into blocks of
// 1024 ids (one workgroup each) for the heavy passes.
//   1. per block: max and first argmax; with top-k, the block's k largest
//      keys (ties cut arbitrarily: the row's k largest are among the union)
//   2. per row: the k-th largest of the candidates (the threshold), the
//      row's max and first argmax (temperature 0 ends here)
//   3. per block: sum of the kept weights (fp32 exponentials, fp64 sum),
//      the block's last kept id
//   4. per row: running sums of the blocks in id order pick the block that
//      crosses u * total, and a scan of its 1024 ids in id order the token
// ---------------------------------------------------------------------------
constexpr int kSBlock = 1024;      // ids per workgroup
constexpr int kSMaxK = 256;        // largest top_k of the parallel path

struct SampleScratch {
  float* bmax; int* barg; int* bcnt; uint32_t* cand;   // [n][G], [n][G], [n][G], [n][G][kSMaxK]
  uint32_t* thr; float* zmax;                           // [n], [n]
  double* bsum; int* blast;                             // [n][G], [n][G]
};
inline int64_t sample_scratch_layout(int n, int V, char* base, SampleScratch* ss) {
  const int64_t G = (V + kSBlock - 1) / kSBlock;
  int64_t off = 0, o[8];
  const int64_t bytes[8] = {n * G * 4, n * G * 4, n * G * 4, n * G * kSMaxK * 4, (int64_t)n * 4, (int64_t)n * 4,
                            n * G * 8, n * G * 4};
  for (int i = 0; i < 8; ++i) {
    o[i] = off;
    off += (bytes[i] + 255) / 256 * 256;
  }
  if (ss)
    *ss = SampleScratch{(float*)(base + o[0]), (int*)(base + o[1]), (int*)(base + o[2]), (uint32_t*)(base + o[3]),
                        (uint32_t*)(base + o[4]), (float*)(base + o[5]), (double*)(base + o[6]), (int*)(base + o[7])};
  return off;
}

// (value, id) of the larger logit, the smaller id on ties; id V = none
__device__ inline void amax_merge(float& m, int& a, float m2, int a2, int V) {
  if (a2 != V && (a == V || m2 > m || (m2 == m && a2 < a))) { m = m2; a = a2; }
}

// The k-th largest (k >= 1) of the keys held by a workgroup (slots j < jn
// of NK per thread, valid ones flagged; jn uniform), 4 bits per pass.  Each
// wave counts digits into its own 16 LDS counters (integer adds: the order
// does not matter); wave 0 adds the waves' counts (lane = digit) and picks
// the digit by a suffix scan.
template <int NT, int NK>
__device__ inline uint32_t block_kth_key(const uint32_t (&key)[NK], const bool (&ok)[NK], int jn, int k,
                                         int (*hist)[16], int* s_state) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t prefix = 0, mask = 0;
  for (int shift = 28; shift >= 0; shift -= 4) {
    if (lane < 16) hist[wave][lane] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NK; ++j)
      if (j < jn && ok[j] && (key[j] & mask) == prefix) atomicAdd(&hist[wave][(key[j] >> shift) & 15u], 1);
    __syncthreads();
    if (wave == 0) {
      int hb = 0;
      if (lane < 16)
        for (int w = 0; w < NW; ++w) hb += hist[w][lane];
      int suf = hb;                               // keys in digits >= lane
      for (int o = 1; o < 16; o <<= 1) {
        const int t = __shfl_down(suf, o, 64);
        if (lane + o < 16) suf += t;
      }
      const unsigned long long ge = __ballot(lane < 16 && suf >= k);
      const int b = ge ? 63 - __clzll((long long)ge) : 0;   // the largest digit whose suffix reaches k
      const int above = __shfl(suf - hb, b, 64);            // keys in the digits above it
      if (lane == 0) {
        s_state[0] = b;
        s_state[1] = k - above;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)s_state[0] << shift;
    mask |= 15u << shift;
    k = s_state[1];
    __syncthreads();                              // before the counts are rewritten
  }
  return prefix;
}

__global__ void __launch_bounds__(256) k_sample_blocks(const float* __restrict__ logits, int V, int G, int top_k,
                                                       SampleScratch ss) {
  __shared__ float smax[4];
  __shared__ int sarg[4];
  __shared__ int hist[4][16];
  __shared__ int s_state[2];
  __shared__ int s_slot;
  const int g = blockIdx.x, row = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* z = logits + (int64_t)row * V;
  const int base = g * kSBlock;
  uint32_t key[4];
  bool ok[4];
  float mx = -INFINITY;
  int am = V;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = base + tid + 256 * j;
    ok[j] = i < V;
    const float zi = ok[j] ? z[i] : -INFINITY;
    key[j] = fkey(zi);
    if (ok[j]) amax_merge(mx, am, zi, i, V);
  }
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(mx, o, 64);
    const int a2 = __shfl_xor(am, o, 64);
    amax_merge(mx, am, m2, a2, V);
  }
  if (lane == 0) { smax[wave] = mx; sarg[wave] = am; }
  __syncthreads();
  if (tid == 0) {
    float m = smax[0];
    int a = sarg[0];
    for (int w = 1; w < 4; ++w) amax_merge(m, a, smax[w], sarg[w], V);
    ss.bmax[(int64_t)row * G + g] = m;
    ss.barg[(int64_t)row * G + g] = a;
  }
  if (top_k <= 0) return;                                   // uniform: no candidates needed
  const int nvalid = min(kSBlock, V - base);
  const int kl = min(top_k, nvalid);
  const uint32_t t = block_kth_key<256, 4>(key, ok, 4, kl, hist, s_state);
  // candidates: every key above t, then copies of t up to kl
  if (tid == 0) s_slot = 0;
  __syncthreads();
  uint32_t* cand = ss.cand + ((int64_t)row * G + g) * kSMaxK;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (ok[j] && key[j] > t) cand[atomicAdd(&s_slot, 1)] = key[j];
  __syncthreads();
  for (int c = s_slot + tid; c < kl; c += 256) cand[c] = t;
  if (tid == 0) ss.bcnt[(int64_t)row * G + g] = kl;
}

__global__ void __launch_bounds__(1024) k_sample_threshold(int V, int G, float temperature, int top_k,
                                                           SampleScratch ss, int32_t* __restrict__ out) {
  constexpr int NK = (64 * kSMaxK) / 1024;                  // candidates per thread, at most
  __shared__ int hist[16][16];
  __shared__ int s_state[2];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  if (tid < 64) {
    // the row's max and first argmax from the blocks' (G <= 64: one lane each)
    float m = -INFINITY;
    int a = V;
    if (lane < G) {
      m = ss.bmax[(int64_t)row * G + lane];
      a = ss.barg[(int64_t)row * G + lane];
    }
    for (int o = 32; o > 0; o >>= 1) {
      const float m2 = __shfl_xor(m, o, 64);
      const int a2 = __shfl_xor(a, o, 64);
      amax_merge(m, a, m2, a2, V);
    }
    if (lane == 0) {
      ss.zmax[row] = m;
      if (temperature == 0.f) out[row] = a;
    }
  }
  if (temperature == 0.f) return;
  if (top_k <= 0) {
    if (tid == 0) ss.thr[row] = 0u;                         // every key passes
    return;
  }
  // every block but the last holds top_k candidates (top_k <= 256 < 1024
  // ids), the last bcnt[G - 1]: candidate e is slot e % top_k of block
  // e / top_k, e < C
  const int C = (G - 1) * top_k + ss.bcnt[(int64_t)row * G + G - 1];
  uint32_t key[NK];
  bool ok[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const int e = tid + 1024 * j;
    ok[j] = e < C;
    key[j] = ok[j] ? ss.cand[((int64_t)row * G + e / top_k) * kSMaxK + e % top_k] : 0u;
  }
  const uint32_t t = block_kth_key<1024, NK>(key, ok, (C + 1023) / 1024, top_k, hist, s_state);
  if (tid == 0) ss.thr[row] = t;
}

__global__ void __launch_bounds__(256) k_sample_sums(const float* __restrict__ logits, int V, int G, float temperature,
                                                     SampleScratch ss) {
  __shared__ double ssum[4];
  __shared__ int slast[4];
  const int g = blockIdx.x, row = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* z = logits + (int64_t)row * V;
  const uint32_t thr = ss.thr[row];
  const float zm = ss.zmax[row], wscale = 1.4426950408889634f / temperature;
  double sum = 0.0;
  int last = -1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = g * kSBlock + tid + 256 * j;
    if (i < V) {
      const float zi = z[i];
      if (fkey(zi) >= thr) {
        sum += (double)__builtin_amdgcn_exp2f((zi - zm) * wscale);
        last = i;
      }
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    sum += __shfl_xor(sum, o, 64);
    last = max(last, __shfl_xor(last, o, 64));
  }
  if (lane == 0) { ssum[wave] = sum; slast[wave] = last; }
  __syncthreads();
  if (tid == 0) {
    ss.bsum[(int64_t)row * G + g] = (ssum[0] + ssum[1]) + (ssum[2] + ssum[3]);
    ss.blast[(int64_t)row * G + g] = max(max(slast[0], slast[1]), max(slast[2], slast[3]));
  }
}

__global__ void __launch_bounds__(1024) k_sample_pick(const float* __restrict__ logits, int V, int G,
                                                      float temperature, const float* __restrict__ u,
                                                      SampleScratch ss, int32_t* __restrict__ out) {
  __shared__ double wtot[16];
  __shared__ int s_block, s_hit;
  __shared__ double s_before;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const double* bs = ss.bsum + (int64_t)row * G;
  const int* bl = ss.blast + (int64_t)row * G;
  if (wave == 0) {
    // running sums of the blocks in id order (G <= 64: one lane each)
    const double mine = lane < G ? bs[lane] : 0.0;
    double incl = mine;
    for (int o = 1; o < 64; o <<= 1) {
      const double up = __shfl_up(incl, o, 64);
      if (lane >= o) incl += up;
    }
    const double total = __shfl(incl, 63, 64);
    const double target = (double)u[row] * total;
    const unsigned long long cross = __ballot(lane < G && mine > 0.0 && incl > target);
    int last = lane < G ? bl[lane] : -1;
    for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
    if (lane == 0) {
      s_block = cross ? __ffsll((long long)cross) - 1 : -1;
      s_hit = last;                                         // no crossing (rounding): the row's last kept id
      s_before = target;
    }
    if (cross) {
      const int jb = __ffsll((long long)cross) - 1;
      const double before = __shfl(incl - mine, jb, 64);
      if (lane == 0) s_before = target - before;            // the target within the block
    }
  }
  __syncthreads();
  const int gb = s_block;
  if (gb < 0) {
    if (tid == 0) out[row] = s_hit;
    return;
  }
  // scan the crossing block's ids in id order: thread tid holds id gb * 1024 + tid
  const float* z = logits + (int64_t)row * V;
  const uint32_t thr = ss.thr[row];
  const float zm = ss.zmax[row], wscale = 1.4426950408889634f / temperature;
  const int i = gb * kSBlock + tid;
  double w = 0.0;
  if (i < V) {
    const float zi = z[i];
    if (fkey(zi) >= thr) w = (double)__builtin_amdgcn_exp2f((zi - zm) * wscale);
  }
  double incl = w;
  for (int o = 1; o < 64; o <<= 1) {
    const double up = __shfl_up(incl, o, 64);
    if (lane >= o) incl += up;
  }
  if (lane == 63) wtot[wave] = incl;
  if (tid == 0) s_hit = bl[gb];                             // rounding fallback: the block's last kept id
  __syncthreads();
  double before = 0.0;
  for (int v = 0; v < wave; ++v) before += wtot[v];
  const unsigned long long hit = __ballot(w > 0.0 && before + incl > s_before);
  __syncthreads();
  if (hit && lane == 0) atomicMin(&s_hit, gb * kSBlock + wave * 64 + __ffsll((long long)hit) - 1);
  __syncthreads();
  if (tid == 0) out[row] = s_hit;
}

}  // namespace

int64_t sample_parallel_scratch_bytes(int n, int V) { return sample_scratch_layout(n, V, nullptr, nullptr); }

hipError_t sample_parallel(const float* logits, int n, int V, float temperature, int top_k, const float* u,
                           int32_t* out, void* scratch, hipStream_t s) {
  if (n < 1 || n > 65535 || V < 1 || V > 64 * kSBlock || top_k < 0 || !(temperature >= 0.f))
    return hipErrorInvalidValue;
  if (top_k >= V) top_k = 0;                                // keeps every id
  if (top_k > kSMaxK) return sample(logits, n, V, temperature, top_k, u, out, s);
  SampleScratch ss;
  sample_scratch_layout(n, V, (char*)scratch, &ss);
  const int G = (V + kSBlock - 1) / kSBlock;
  k_sample_blocks<<<dim3(G, n), 256, 0, s>>>(logits, V, G, temperature == 0.f ? 0 : top_k, ss);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_sample_threshold<<<n, 1024, 0, s>>>(V, G, temperature, top_k, ss, out);
  e = hipGetLastError();
  if (e != hipSuccess || temperature == 0.f) return e;
  k_sample_sums<<<dim3(G, n), 256, 0, s>>>(logits, V, G, temperature, ss);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_sample_pick<<<n, 1024, 0, s>>>(logits, V, G, temperature, u, ss, out);
  return hipGetLastError();
}

hipError_t sample(const float* logits, int n, int V, float temperature, int top_k, const float* u, int32_t* out,
                  hipStream_t s) {
  // one 64-id block per lane of the 16 waves
  if (n < 1 || V < 1 || V > 65536 || top_k < 0 || !(temperature >= 0.f)) return hipErrorInvalidValue;
  k_sample<<<n, 1024, 0, s>>>(logits, V, temperature, top_k, u, out);
  return hipGetLastError();
}

template <typename T>
hipError_t gemv(const GemvDesc& g, int epi, hipStream_t s) {
  if (g.nb < 1 || g.nb > kMaxDecodeBatch || g.N % kCols || g.K % V16<T>::n || g.N <= 0 || g.K <= 0)
    return hipErrorInvalidValue;
  // A column group per wave (the input read by 4x fewer waves) for wide
  // products (the logits) and for short rows (K <= 2048: split over 4 waves
  // a 1280-long row leaves 96 of the 256 lanes idle; per wave it is 2.5
  // full steps; 0.955 -> 0.901 ms per d20 step at one sequence); 4 waves
  // per group, splitting K, for long rows (W2, K = 5120).
  const bool wide = (g.N >= 16384 || g.K <= 2048) && g.N % (4 * kCols) == 0;
  const unsigned blocks = wide ? (unsigned)(g.N / (4 * kCols)) : (unsigned)(g.N / kCols);
  if (g.norm && epi != EPI_ROPE && epi != EPI_RELU2 && epi != EPI_F32) return hipErrorInvalidValue;
#define NC_GEMV(E, N)                                                \
  if (wide) k_gemv<T, E, 1, N><<<blocks, 256, 0, s>>>(g);            \
  else k_gemv<T, E, 4, N><<<blocks, 256, 0, s>>>(g);                 \
  break;
  if (g.norm) {
    switch (epi) {
      case EPI_ROPE: NC_GEMV(EPI_ROPE, true)
      case EPI_RELU2: NC_GEMV(EPI_RELU2, true)
      default: NC_GEMV(EPI_F32, true)
    }
  } else {
    switch (epi) {
      case EPI_STORE: NC_GEMV(EPI_STORE, false)
      case EPI_ROPE: NC_GEMV(EPI_ROPE, false)
      case EPI_RESID: NC_GEMV(EPI_RESID, false)
      case EPI_RELU2: NC_GEMV(EPI_RELU2, false)
      case EPI_F32: NC_GEMV(EPI_F32, false)
      default: return hipErrorInvalidValue;
    }
  }
#undef NC_GEMV
  return hipGetLastError();
}

template <typename T>
hipError_t kv_append(const T* qkv, int nb, int d, T* K, T* V, int64_t seq_stride, int pos, hipStream_t s) {
  k_kv_append<T><<<dim3((d + 255) / 256, nb), 256, 0, s>>>(qkv, nb, d, K, V, seq_stride, pos);
  return hipGetLastError();
}

template <typename T>
hipError_t kv_prefill(const T* qkv, int len, int d, int nb, T* K, T* V, int64_t seq_stride, hipStream_t s) {
  k_kv_prefill<T><<<dim3(len, nb), 256, 0, s>>>(qkv, len, d, nb, K, V, seq_stride);
  return hipGetLastError();
}

int attn_decode_chunks(int L) { return (L + 63) / 64; }

template <typename T>
hipError_t attn_decode(const AttnDecodeDesc& a, int nb, hipStream_t s) {
  if (a.L < 1 || a.nchunks != attn_decode_chunks(a.L) || a.nchunks > 65535) return hipErrorInvalidValue;
  if (a.Q == 128) k_attn_decode<T, 128><<<dim3(a.nchunks, a.H, nb), 256, 0, s>>>(a);
  else if (a.Q == 64) k_attn_decode<T, 64><<<dim3(a.nchunks, a.H, nb), 256, 0, s>>>(a);
  else if (a.Q == 96) k_attn_decode<T, 96><<<dim3(a.nchunks, a.H, nb), 256, 0, s>>>(a);
  else if (a.Q == 32) k_attn_decode<T, 32><<<dim3(a.nchunks, a.H, nb), 256, 0, s>>>(a);
  else return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_attn_decode_combine<T><<<dim3(a.H, nb), 128, 0, s>>>(a);
  return hipGetLastError();
}

template hipError_t gemv<float>(const GemvDesc&, int, hipStream_t);
template hipError_t gemv<bf16>(const GemvDesc&, int, hipStream_t);
template hipError_t kv_append<float>(const float*, int, int, float*, float*, int64_t, int, hipStream_t);
template hipError_t kv_append<bf16>(const bf16*, int, int, bf16*, bf16*, int64_t, int, hipStream_t);
template hipError_t kv_prefill<float>(const float*, int, int, int, float*, float*, int64_t, hipStream_t);
template hipError_t kv_prefill<bf16>(const bf16*, int, int, int, bf16*, bf16*, int64_t, hipStream_t);
template hipError_t attn_decode<float>(const AttnDecodeDesc&, int, hipStream_t);
template hipError_t attn_decode<bf16>(const AttnDecodeDesc&, int, hipStream_t);

}  // namespace nc
