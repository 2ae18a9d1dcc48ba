// Portable causal attention (no matrix cores): one 64-lane wave per query
// row (forward, dQ) or key row (dK, dV), online softmax over the causal
// prefix.  Serves the fp32 configuration and the bf16 cross-check mode.
//
// Layout: qkv token-major [B*T][3*H*Q] (q | k | v, q and k already rotated),
// o and dO token-major [B*T][H*Q], lse and delta [B][H][T] fp32.  A lane owns
// head elements [lane*E, lane*E + E) with E = Q / 64, so a rotary pair
// (2i, 2i+1) is in one lane when E >= 2 and in two neighbouring lanes
// when E == 1.
#include "nc_internal.h"

namespace nc {
namespace {

constexpr int kWave = 64;
constexpr int kMaxE = 4;   // head_dim <= 256

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

template <typename T>
__device__ inline void load_head(const T* p, int E, int lane, float* v) {
#pragma unroll
  for (int e = 0; e < kMaxE; ++e)
    if (e < E) v[e] = to_f32(p[lane * E + e]);
}

// inverse rotation (angle -phi) of the lane's elements of one head row
__device__ inline void rope_inverse(float* v, int E, int lane, const float2* tab_t) {
  if (E >= 2) {
#pragma unroll
    for (int e = 0; e < kMaxE; e += 2) {
      if (e < E) {
        const float2 cs = tab_t[(lane * E + e) / 2];
        const float x0 = v[e], x1 = v[e + 1];
        v[e] = x0 * cs.x + x1 * cs.y;
        v[e + 1] = -x0 * cs.y + x1 * cs.x;
      }
    }
  } else {
    const float other = __shfl_xor(v[0], 1, kWave);
    const float2 cs = tab_t[lane / 2];
    v[0] = (lane & 1) ? (-other * cs.y + v[0] * cs.x) : (v[0] * cs.x + other * cs.y);
  }
}

template <typename T>
__global__ void __launch_bounds__(256) k_attn_fwd(AttnDesc a) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int B = a.B, Tn = a.T, H = a.H, Q = a.Q, E = Q / kWave;
  if (w >= (int64_t)B * H * Tn) return;
  const int t = (int)(w % Tn);
  const int h = (int)((w / Tn) % H);
  const int64_t b = w / ((int64_t)Tn * H);
  const int64_t ld = 3LL * H * Q;
  const T* qkv = (const T*)a.qkv;
  const T* rowbase = qkv + b * Tn * ld;
  float q[kMaxE], acc[kMaxE] = {}, kv[kMaxE];
  load_head(rowbase + t * ld + h * Q, E, lane, q);
  const float scale = 1.0f / sqrtf((float)Q);
  float mx = -INFINITY, l = 0.f;
  for (int j = 0; j <= t; ++j) {
    load_head(rowbase + j * ld + (int64_t)H * Q + h * Q, E, lane, kv);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < kMaxE; ++e)
      if (e < E) s += q[e] * kv[e];
    s = wave_sum(s) * scale;
    const float mn = fmaxf(mx, s);
    const float corr = expf(mx - mn), p = expf(s - mn);
    l = l * corr + p;
    load_head(rowbase + j * ld + 2LL * H * Q + h * Q, E, lane, kv);
#pragma unroll
    for (int e = 0; e < kMaxE; ++e)
      if (e < E) acc[e] = acc[e] * corr + p * kv[e];
    mx = mn;
  }
  T* o = (T*)a.o_out + (b * Tn + t) * (int64_t)H * Q + h * Q;
#pragma unroll
  for (int e = 0; e < kMaxE; ++e)
    if (e < E) o[lane * E + e] = from_f32<T>(acc[e] / l);
  if (lane == 0) a.lse[(b * H + h) * Tn + t] = mx + logf(l);
}

// dQ for one query row: sum over keys j <= t of dS[t,j] k_j / sqrt(Q)
template <typename T>
__global__ void __launch_bounds__(256) k_attn_dq(AttnDesc a) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int B = a.B, Tn = a.T, H = a.H, Q = a.Q, E = Q / kWave;
  if (w >= (int64_t)B * H * Tn) return;
  const int t = (int)(w % Tn);
  const int h = (int)((w / Tn) % H);
  const int64_t b = w / ((int64_t)Tn * H);
  const int64_t ld = 3LL * H * Q, ldo = (int64_t)H * Q;
  const T* rowbase = (const T*)a.qkv + b * Tn * ld;
  float q[kMaxE], dO[kMaxE], kr[kMaxE], vr[kMaxE], dq[kMaxE] = {};
  load_head(rowbase + t * ld + h * Q, E, lane, q);
  load_head((const T*)a.dout + (b * Tn + t) * ldo + h * Q, E, lane, dO);
  const float scale = 1.0f / sqrtf((float)Q);
  const float lse = a.lse[(b * H + h) * Tn + t];
  const float D = a.delta[(b * H + h) * Tn + t];
  for (int j = 0; j <= t; ++j) {
    load_head(rowbase + j * ld + ldo + h * Q, E, lane, kr);
    load_head(rowbase + j * ld + 2 * ldo + h * Q, E, lane, vr);
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < kMaxE; ++e)
      if (e < E) { s += q[e] * kr[e]; dp += dO[e] * vr[e]; }
    s = wave_sum(s);
    dp = wave_sum(dp);
    const float p = expf(s * scale - lse);
    const float ds = p * (dp - D);
#pragma unroll
    for (int e = 0; e < kMaxE; ++e)
      if (e < E) dq[e] += ds * kr[e];
  }
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) dq[e] *= scale;
  if (a.rope) rope_inverse(dq, E, lane, a.rope + (int64_t)t * (Q / 2));
  T* out = (T*)a.dqkv + (b * Tn + t) * ld + h * Q;
#pragma unroll
  for (int e = 0; e < kMaxE; ++e)
    if (e < E) out[lane * E + e] = from_f32<T>(dq[e]);
}

// dK, dV for one key row j: sums over queries t >= j
template <typename T>
__global__ void __launch_bounds__(256) k_attn_dkdv(AttnDesc a) {
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int B = a.B, Tn = a.T, H = a.H, Q = a.Q, E = Q / kWave;
  if (w >= (int64_t)B * H * Tn) return;
  const int j = (int)(w % Tn);
  const int h = (int)((w / Tn) % H);
  const int64_t b = w / ((int64_t)Tn * H);
  const int64_t ld = 3LL * H * Q, ldo = (int64_t)H * Q;
  const T* rowbase = (const T*)a.qkv + b * Tn * ld;
  float kr[kMaxE], vr[kMaxE], q[kMaxE], dO[kMaxE], dk[kMaxE] = {}, dv[kMaxE] = {};
  load_head(rowbase + j * ld + ldo + h * Q, E, lane, kr);
  load_head(rowbase + j * ld + 2 * ldo + h * Q, E, lane, vr);
  const float scale = 1.0f / sqrtf((float)Q);
  for (int t = j; t < Tn; ++t) {
    load_head(rowbase + t * ld + h * Q, E, lane, q);
    load_head((const T*)a.dout + (b * Tn + t) * ldo + h * Q, E, lane, dO);
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < kMaxE; ++e)
      if (e < E) { s += q[e] * kr[e]; dp += dO[e] * vr[e]; }
    s = wave_sum(s);
    dp = wave_sum(dp);
    const float p = expf(s * scale - a.lse[(b * H + h) * Tn + t]);
    const float ds = p * (dp - a.delta[(b * H + h) * Tn + t]);
#pragma unroll
    for (int e = 0; e < kMaxE; ++e)
      if (e < E) { dv[e] += p * dO[e]; dk[e] += ds * q[e]; }
  }
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) dk[e] *= scale;
  if (a.rope) rope_inverse(dk, E, lane, a.rope + (int64_t)j * (Q / 2));
  T* out = (T*)a.dqkv + (b * Tn + j) * ld;
#pragma unroll
  for (int e = 0; e < kMaxE; ++e)
    if (e < E) {
      out[ldo + h * Q + lane * E + e] = from_f32<T>(dk[e]);
      out[2 * ldo + h * Q + lane * E + e] = from_f32<T>(dv[e]);
    }
}

inline unsigned nblocks(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

template <typename T>
hipError_t attn_fwd_portable(const AttnDesc& a, hipStream_t s) {
  if (a.Q % kWave || a.Q > kWave * kMaxE) return hipErrorInvalidValue;
  k_attn_fwd<T><<<nblocks((int64_t)a.B * a.H * a.T, 4), 256, 0, s>>>(a);
  return hipGetLastError();
}

template <typename T>
hipError_t attn_bwd_portable(const AttnDesc& a, hipStream_t s) {
  if (a.Q % kWave || a.Q > kWave * kMaxE) return hipErrorInvalidValue;
  hipError_t e = attn_delta<T>(a, s);
  if (e != hipSuccess) return e;
  const unsigned nb = nblocks((int64_t)a.B * a.H * a.T, 4);
  k_attn_dq<T><<<nb, 256, 0, s>>>(a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_attn_dkdv<T><<<nb, 256, 0, s>>>(a);
  return hipGetLastError();
}

template hipError_t attn_fwd_portable<float>(const AttnDesc&, hipStream_t);
template hipError_t attn_fwd_portable<bf16>(const AttnDesc&, hipStream_t);
template hipError_t attn_bwd_portable<float>(const AttnDesc&, hipStream_t);
template hipError_t attn_bwd_portable<bf16>(const AttnDesc&, hipStream_t);

}  // namespace nc
