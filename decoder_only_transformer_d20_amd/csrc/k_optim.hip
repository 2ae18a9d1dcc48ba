// Optimiser-step kernels (nanochat speedrun walkthrough, section Pretraining,
// optimiser paragraph: Muon on the matrices, AdamW on the embedding and the
// unembedding).  AdamW is one fused elementwise pass.  Muon's elementwise
// parts are here: the momentum update with the sum of squares of the
// Nesterov direction, the normalise-and-cast into the iteration's operand,
// and the final apply.  Its Newton-Schulz products run on the GEMM kernels
// with the AXPBY epilogue.  All of it is HBM-bound.
#include "nc_internal.h"

namespace nc {
namespace {

constexpr int kThreads = 256;      // four waves (the block reductions assume it)
constexpr int kTile = 64;          // transposing tiles: 64 x 64 elements
static_assert(kThreads == 256, "block reductions");

__device__ inline float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ inline void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

template <typename T> __device__ inline void st4_t(T* p, float4 v);
template <> __device__ inline void st4_t<float>(float* p, float4 v) { st4(p, v); }
template <> __device__ inline void st4_t<bf16>(bf16* p, float4 v) {
  const uint32_t lo = (uint32_t)from_f32<bf16>(v.x).x | ((uint32_t)from_f32<bf16>(v.y).x << 16);
  const uint32_t hi = (uint32_t)from_f32<bf16>(v.z).x | ((uint32_t)from_f32<bf16>(v.w).x << 16);
  *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}

// AdamW on n elements (n % 4 == 0, 16-byte aligned): decoupled decay, then
// the bias-corrected moment ratio; the model-dtype copy of the result goes
// to out.
template <typename T>
__global__ void __launch_bounds__(kThreads) k_adamw(int64_t n4, float* __restrict__ p, const float* __restrict__ g,
                                                     float* __restrict__ m, float* __restrict__ v, T* __restrict__ out,
                                                     AdamwArgs a) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kThreads) {
    float4 pv = ld4(p + 4 * i), gv = ld4(g + 4 * i), mv = ld4(m + 4 * i), vv = ld4(v + 4 * i);
    float* pp = &pv.x;
    float* gp = &gv.x;
    float* mp = &mv.x;
    float* vp = &vv.x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gi = gp[e] * a.grad_scale;
      mp[e] = a.beta1 * mp[e] + (1.f - a.beta1) * gi;
      vp[e] = a.beta2 * vp[e] + (1.f - a.beta2) * gi * gi;
      pp[e] = pp[e] * a.decay - a.lr * (mp[e] * a.inv_bc1) / (__builtin_sqrtf(vp[e] * a.inv_bc2) + a.eps);
    }
    st4(p + 4 * i, pv);
    st4(m + 4 * i, mv);
    st4(v + 4 * i, vv);
    st4_t<T>(out + 4 * i, pv);
  }
}

// Muon momentum over n elements (n % 4 == 0) of each of gridDim.y matrices
// (matrix y at element offset y * stride): buf = mu buf + s g, and the
// direction u = s g + mu buf (Nesterov) or buf.  Each block writes the fp32
// sum of u^2 over its elements to partials[y][blockIdx.x] (a fixed tree, so
// repeated calls give identical bits).
__global__ void __launch_bounds__(kThreads) k_muon_momentum(int64_t n4, const float* __restrict__ g,
                                                             float* __restrict__ buf, float s, float mu, int nesterov,
                                                             float* __restrict__ partials, int64_t stride) {
  __shared__ float red[kThreads / 64];
  g += blockIdx.y * stride;
  buf += blockIdx.y * stride;
  partials += (int64_t)blockIdx.y * kMuonMaxPartials;
  float acc = 0.f;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += (int64_t)gridDim.x * kThreads) {
    float4 gv = ld4(g + 4 * i), bv = ld4(buf + 4 * i);
    float* gp = &gv.x;
    float* bp = &bv.x;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gi = gp[e] * s;
      bp[e] = mu * bp[e] + gi;
      const float u = nesterov ? gi + mu * bp[e] : bp[e];
      acc += u * u;
    }
    st4(buf + 4 * i, bv);
  }
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) t += red[w];
    partials[blockIdx.x] = t;
  }
}

// The iteration's starting point X = u / (||u||_F + eps) in the model dtype,
// u recomputed from g and the updated buf.  X is [r][c] as the matrix, or
// [c][r] when r > c (the wide orientation).  Every block sums the partials
// itself, in fp64, in index order.  One block per 64 x 64 tile
// (r, c multiples of 64) of matrix z (g, buf at z * stride, partials at
// z * kMuonMaxPartials, X at z * r * c); a transposed tile goes through LDS.
template <typename T>
__global__ void __launch_bounds__(kThreads) k_muon_normalise(int r, int c, const float* __restrict__ g,
                                                              const float* __restrict__ buf, float s, float mu,
                                                              int nesterov, const float* __restrict__ partials,
                                                              int nparts, float eps, T* __restrict__ X,
                                                              int64_t stride) {
  __shared__ float tile[kTile][kTile + 1];
  __shared__ double red[kThreads / 64];
  g += blockIdx.z * stride;
  buf += blockIdx.z * stride;
  partials += (int64_t)blockIdx.z * kMuonMaxPartials;
  X += (int64_t)blockIdx.z * r * c;
  // ||u||^2: thread t sums partials t, t + 256, ... in fp64, then a fixed
  // tree over the block -- the same order in every block
  double t = 0.0;
  for (int i = threadIdx.x; i < nparts; i += kThreads) t += (double)partials[i];
  for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = t;
  __syncthreads();
  const double total = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = (float)(1.0 / (sqrt(total) + (double)eps));
  const int r0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
  const int tc = (threadIdx.x & 15) * 4, tr = threadIdx.x >> 4;   // 16 x 4 columns, 16 rows per sweep
  const bool tall = r > c;
#pragma unroll
  for (int k = 0; k < kTile / 16; ++k) {
    const int64_t idx = (int64_t)(r0 + tr + 16 * k) * c + c0 + tc;
    float4 gv = ld4(g + idx), bv = ld4(buf + idx);
    float4 u;
    u.x = (nesterov ? gv.x * s + mu * bv.x : bv.x) * inv;
    u.y = (nesterov ? gv.y * s + mu * bv.y : bv.y) * inv;
    u.z = (nesterov ? gv.z * s + mu * bv.z : bv.z) * inv;
    u.w = (nesterov ? gv.w * s + mu * bv.w : bv.w) * inv;
    if (!tall) {
      st4_t<T>(X + idx, u);
    } else {
      tile[tr + 16 * k][tc] = u.x;
      tile[tr + 16 * k][tc + 1] = u.y;
      tile[tr + 16 * k][tc + 2] = u.z;
      tile[tr + 16 * k][tc + 3] = u.w;
    }
  }
  if (!tall) return;
  __syncthreads();
  // X [c][r]: row c0 + j holds column j of the tile
#pragma unroll
  for (int k = 0; k < kTile / 16; ++k) {
    const int j = tr + 16 * k;
    st4_t<T>(X + (int64_t)(c0 + j) * r + r0 + tc,
             make_float4(tile[tc][j], tile[tc + 1][j], tile[tc + 2][j], tile[tc + 3][j]));
  }
}

template <typename T> __device__ inline float4 ld4_t(const T* p);
template <> __device__ inline float4 ld4_t<float>(const float* p) { return ld4(p); }
template <> __device__ inline float4 ld4_t<bf16>(const bf16* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return make_float4(to_f32(bf16{(uint16_t)(w.x & 0xffff)}), to_f32(bf16{(uint16_t)(w.x >> 16)}),
                     to_f32(bf16{(uint16_t)(w.y & 0xffff)}), to_f32(bf16{(uint16_t)(w.y >> 16)}));
}

// W -= lr X (X as the matrix [r][c], or [c][r] when r > c); out = W in the
// model dtype.  One block per 64 x 64 tile of matrix z (W, out at
// z * stride, X at z * r * c).
template <typename T>
__global__ void __launch_bounds__(kThreads) k_muon_apply(int r, int c, const T* __restrict__ X, float lr,
                                                          float* __restrict__ W, T* __restrict__ out, int64_t stride) {
  __shared__ float tile[kTile][kTile + 1];
  X += (int64_t)blockIdx.z * r * c;
  W += blockIdx.z * stride;
  out += blockIdx.z * stride;
  const int r0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
  const int tc = (threadIdx.x & 15) * 4, tr = threadIdx.x >> 4;
  const bool tall = r > c;
  if (tall) {
    // X rows c0 .. c0+63 (columns of W), columns r0 .. r0+63
#pragma unroll
    for (int k = 0; k < kTile / 16; ++k) {
      const int j = tr + 16 * k;
      const float4 x = ld4_t<T>(X + (int64_t)(c0 + j) * r + r0 + tc);
      tile[tc][j] = x.x;
      tile[tc + 1][j] = x.y;
      tile[tc + 2][j] = x.z;
      tile[tc + 3][j] = x.w;
    }
    __syncthreads();
  }
#pragma unroll
  for (int k = 0; k < kTile / 16; ++k) {
    const int i = tr + 16 * k;
    const int64_t idx = (int64_t)(r0 + i) * c + c0 + tc;
    const float4 x = tall ? make_float4(tile[i][tc], tile[i][tc + 1], tile[i][tc + 2], tile[i][tc + 3])
                          : ld4_t<T>(X + idx);
    float4 w = ld4(W + idx);
    w.x -= lr * x.x;
    w.y -= lr * x.y;
    w.z -= lr * x.z;
    w.w -= lr * x.w;
    st4(W + idx, w);
    st4_t<T>(out + idx, w);
  }
}

int blocks_for(int64_t n4) {
  const int64_t b = (n4 + kThreads - 1) / kThreads;
  return (int)(b < kMuonMaxPartials ? (b < 1 ? 1 : b) : kMuonMaxPartials);
}

}  // namespace

template <typename T>
hipError_t adamw(int64_t n, float* p, const float* g, float* m, float* v, T* out, const AdamwArgs& a, hipStream_t s) {
  if (n <= 0 || n % 4) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  const int64_t blocks = (n4 + kThreads - 1) / kThreads;
  k_adamw<T><<<(int)(blocks < 8192 ? blocks : 8192), kThreads, 0, s>>>(n4, p, g, m, v, out, a);
  return hipGetLastError();
}

int muon_partials(int64_t n) { return blocks_for(n / 4); }

hipError_t muon_momentum(int64_t n, int count, int64_t stride, const float* g, float* buf, float scale, float mu,
                         int nesterov, float* partials, hipStream_t s) {
  if (n <= 0 || n % 4 || count < 1 || count > 65535) return hipErrorInvalidValue;
  k_muon_momentum<<<dim3(blocks_for(n / 4), count), kThreads, 0, s>>>(n / 4, g, buf, scale, mu, nesterov, partials,
                                                                      stride);
  return hipGetLastError();
}

template <typename T>
hipError_t muon_normalise(int r, int c, int count, int64_t stride, const float* g, const float* buf, float scale,
                          float mu, int nesterov, const float* partials, float eps, T* X, hipStream_t s) {
  if (r <= 0 || c <= 0 || r % kTile || c % kTile || count < 1 || count > 65535) return hipErrorInvalidValue;
  k_muon_normalise<T><<<dim3(c / kTile, r / kTile, count), kThreads, 0, s>>>(
      r, c, g, buf, scale, mu, nesterov, partials, muon_partials((int64_t)r * c), eps, X, stride);
  return hipGetLastError();
}

template <typename T>
hipError_t muon_apply(int r, int c, int count, int64_t stride, const T* X, float lr, float* W, T* out, hipStream_t s) {
  if (r <= 0 || c <= 0 || r % kTile || c % kTile || count < 1 || count > 65535) return hipErrorInvalidValue;
  k_muon_apply<T><<<dim3(c / kTile, r / kTile, count), kThreads, 0, s>>>(r, c, X, lr, W, out, stride);
  return hipGetLastError();
}

template hipError_t adamw<float>(int64_t, float*, const float*, float*, float*, float*, const AdamwArgs&, hipStream_t);
template hipError_t adamw<bf16>(int64_t, float*, const float*, float*, float*, bf16*, const AdamwArgs&, hipStream_t);
template hipError_t muon_normalise<float>(int, int, int, int64_t, const float*, const float*, float, float, int,
                                          const float*, float, float*, hipStream_t);
template hipError_t muon_normalise<bf16>(int, int, int, int64_t, const float*, const float*, float, float, int,
                                         const float*, float, bf16*, hipStream_t);
template hipError_t muon_apply<float>(int, int, int, int64_t, const float*, float, float*, float*, hipStream_t);
template hipError_t muon_apply<bf16>(int, int, int, int64_t, const bf16*, float, float*, bf16*, hipStream_t);

}  // namespace nc
