// Portable tiled GEMM (fp32 FMA, no matrix cores) with the full epilogue set.
//
// It serves the fp32 configuration, where products must stay fp32, and the
// bf16 cross-check mode.  Tile 64 x 64 x 16, 256 threads, 4 x 4 outputs per
// thread; operands are staged k-major in LDS as fp32 whatever their layout in
// memory, so the four operand layouts differ only in the global index math.
#include "nc_internal.h"

namespace nc {
namespace {

constexpr int BM = 64, BN = 64, BK = 16;

template <typename T>
__device__ inline float load_op(const T* p, int64_t ld, int trans, int64_t row, int64_t k) {
  return to_f32(trans ? p[k * ld + row] : p[row * ld + k]);
}

template <typename T>
__global__ void __launch_bounds__(256) k_gemm_portable(GemmDesc g) {
  __shared__ float Ps[BK][BM + 4];
  __shared__ float Qs[BK][BN + 4];
  __shared__ float Cs[BM][BN + 1];
  const T* P = (const T*)g.P;
  const T* Q = (const T*)g.Q;
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int64_t nb = g.K / 64;                   // split z: 64-wide k blocks [z nb/s, (z+1) nb/s)
  const int64_t kbeg = (int64_t)blockIdx.z * nb / g.splits * 64, kend = ((int64_t)blockIdx.z + 1) * nb / g.splits * 64;

  float acc[4][4] = {};
  for (int64_t k0 = kbeg; k0 < kend; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      int r, k;
      if (g.p_trans) { r = e % BM; k = e / BM; } else { r = e / BK; k = e % BK; }
      Ps[k][r] = load_op(P, g.ldp, g.p_trans, m0 + r, k0 + k);
      if (g.q_trans) { r = e % BN; k = e / BN; } else { r = e / BK; k = e % BK; }
      Qs[k][r] = load_op(Q, g.ldq, g.q_trans, n0 + r, k0 + k);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = Ps[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Qs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  if (g.epi == EPI_LSE || g.epi == EPI_LSEZ) {
    // per-row max and sum of exp over this 64-column tile, plus the target
    // logit; EPI_LSEZ also stores the logits relative to the row max
    __shared__ float rmax[BM];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) Cs[ty * 4 + i][tx * 4 + j] = acc[i][j];
    __syncthreads();
    if (tid < BM) {
      const int64_t m = m0 + tid;
      float mx = -INFINITY;
      for (int j = 0; j < BN; ++j) mx = fmaxf(mx, Cs[tid][j]);
      float s = 0.f;
      for (int j = 0; j < BN; ++j) s += expf(Cs[tid][j] - mx);
      g.lse_part[m * g.lse_stride + blockIdx.x] = make_float2(mx, s);
      const int t = g.tgt[m];
      if (t >= n0 && t < n0 + BN) g.ztgt[m] = Cs[tid][t - n0];
      rmax[tid] = mx;
    }
    if (g.epi == EPI_LSEZ) {
      __syncthreads();
      for (int e = tid; e < BM * BN; e += 256) {
        const int r = e / BN, cl = e % BN;
        ((T*)g.C)[(m0 + r) * g.ldc + n0 + cl] = from_f32<T>(Cs[r][cl] - rmax[r]);
      }
    }
    return;
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = acc[i][j];
    const int64_t n = n0 + tx * 4;
    switch (g.epi) {
      case EPI_ROPE:
        if (n < g.rope_cols) {
          const int half = g.head_dim / 2;
          const int t = (int)(m % g.rope_T);
#pragma unroll
          for (int j = 0; j < 4; j += 2) {
            const int pi = (int)((n + j) % g.head_dim) / 2;
            const float2 cs = g.rope[(int64_t)t * half + pi];
            const float x0 = v[j], x1 = v[j + 1];
            v[j] = x0 * cs.x - x1 * cs.y;
            v[j + 1] = x0 * cs.y + x1 * cs.x;
          }
        }
        break;
      case EPI_RESID: {
        const T* a = (const T*)g.aux + m * g.ldaux + n;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] += to_f32(a[j]);
        break;
      }
      case EPI_DRELU2: {
        const T* a = (const T*)g.aux + m * g.ldaux + n;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] *= 2.f * sqrtf(fmaxf(to_f32(a[j]), 0.f));
        break;
      }
      case EPI_AXPBY: {
        const T* a = (const T*)g.aux + m * g.ldaux + n;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = g.ep_alpha * v[j] + g.ep_gamma * to_f32(a[j]);
        break;
      }
      case EPI_RELU2:
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = fmaxf(v[j], 0.f) * fmaxf(v[j], 0.f);
        break;
      case EPI_DZ: {
        const int t = g.tgt[m];
        const float l = g.lse[m];
        const float sc = g.row_scale[m];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = (expf(v[j] - l) - ((n + j) == t ? 1.f : 0.f)) * sc;
        break;
      }
      default:
        break;
    }
    if (g.epi == EPI_F32) {
      if (g.splits > 1) {
        float* pp = g.part + (int64_t)blockIdx.z * g.M * g.N + m * g.N + n;
#pragma unroll
        for (int j = 0; j < 4; ++j) pp[j] = v[j];
      } else {
        float* c = (float*)g.C + m * g.ldc + n;
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = (g.beta ? c[j] : 0.f) + v[j];
      }
    } else {
      T* c = (T*)g.C + m * g.ldc + n;
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = from_f32<T>(v[j]);
    }
  }
}

}  // namespace

template <typename T>
hipError_t gemm_portable(const GemmDesc& g, hipStream_t s) {
  if (g.batch > 1) {
    // one launch per item of a batched product
    if (g.splits != 1 || (g.epi != EPI_STORE && g.epi != EPI_AXPBY)) return hipErrorInvalidValue;
    for (int b = 0; b < g.batch; ++b) {
      GemmDesc gi = g;
      gi.batch = 1;
      gi.P = (const T*)g.P + b * g.sP;
      gi.Q = (const T*)g.Q + b * g.sQ;
      gi.C = (T*)g.C + b * g.sC;
      gi.aux = g.aux ? (const T*)g.aux + b * g.sAux : nullptr;
      hipError_t e = gemm_portable<T>(gi, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  if (g.M % BM || g.N % BN || g.splits < 1 || g.K % 64 || g.splits > g.K / 64) return hipErrorInvalidValue;
  if (g.splits > 1 && g.epi != EPI_F32) return hipErrorInvalidValue;
  dim3 grid(g.N / BN, g.M / BM, g.splits);
  k_gemm_portable<T><<<grid, 256, 0, s>>>(g);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && g.epi == EPI_F32 && g.splits > 1) {
    if (g.ldc != g.N) return hipErrorInvalidValue;
    e = splitk_reduce(g.part, g.splits, (int64_t)g.M * g.N, (float*)g.C, g.beta, s);
  }
  return e;
}

template hipError_t gemm_portable<float>(const GemmDesc&, hipStream_t);
template hipError_t gemm_portable<bf16>(const GemmDesc&, hipStream_t);

}  // namespace nc
