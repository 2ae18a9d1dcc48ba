// Causal flash attention, forward and backward, on gfx950 matrix cores
// (bf16 operands, fp32 accumulation and softmax statistics), head dim 128.
//
// Forward: a workgroup (4 waves) owns 128 query rows of one (row, head), a
// wave 32 of them; it walks the 64-key tiles up to its diagonal with an
// online softmax.  Backward: delta = rowsum(dO * O) (attn_delta), then one
// kernel accumulates dQ over key tiles and one accumulates dK, dV over query
// tiles, both recomputing P from the saved log-sum-exp -- no atomics, so the
// result does not depend on scheduling.  dQ and dK leave through the
// inverse rotary rotation, so the caller receives gradients with respect to
// the pre-rotation q and k.
#include <type_traits>

#include "attn_mfma.h"

namespace nc {
using namespace attn;

namespace {

constexpr float kScaleLog2 = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)

// Block -> (tile, head, row).  Workgroups are dealt to the 8 XCDs
// round-robin; renumbering so each XCD takes a contiguous run of the
// (row, head) groups keeps the 16 tiles that share one head's K/V (or Q/dO)
// rows in one XCD's L2.
__device__ inline void tile_order(int ntile, int H, int B, int& tile, int& h, int& b) {
  const int total = ntile * H * B;
  int L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
  tile = L % ntile;
  h = (L / ntile) % H;
  b = L / (ntile * H);
}

// ===========================================================================
// forward
// ===========================================================================
__global__ void __launch_bounds__(256, 2) k_attn_fwd(AttnDesc a) {
  __shared__ __attribute__((aligned(16))) char smem[2][32768];   // per stage: K image | V image
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hh = lane >> 5;
  const int T = a.T, H = a.H, d = H * HD;
  int qt, h, b;
  tile_order(T / 128, H, a.B, qt, h, b);
  qt = T / 128 - 1 - qt;                                         // heaviest tiles first
  const int64_t ld = 3LL * d;
  const bf16* rows = (const bf16*)a.qkv + (int64_t)b * T * ld;
  const bf16* qb = rows + h * HD;
  const bf16* kb = rows + d + h * HD;
  const bf16* vb = rows + 2 * d + h * HD;
  const int q0 = qt * 128, i0 = q0 + wave * 32, my_i = i0 + (lane & 31);

  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(gload(qb + (int64_t)my_i * ld + 16 * s + 8 * hh));

  floatx16 o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) zero(o[t]);
  float m = -INFINITY, l = 0.f;
  TrOff tv;
  tv.init(lane);
  uint32_t offK[2];
#pragma unroll
  for (int js = 0; js < 2; ++js) offK[js] = offN(js * 32 + (lane & 31), hh);   // chunk 2 ks + hh: ^ 32 ks

  const int ntiles = (q0 + 128) / 64;
  u32x4 rk[4], rv[4];
  // next key tile into registers while this one is used; stored after
  auto gl = [&](int jt) {
    const int64_t j0 = (int64_t)jt * 64;
    load_nat64<256>(kb + j0 * ld, ld, tid, rk);
    load_nat64<256>(vb + j0 * ld, ld, tid, rv);
  };
  auto st = [&](int stage) {
    store_nat64<256>(smem[stage], tid, rk);
    store_nat64<256>(smem[stage] + 16384, tid, rv);
  };
  gl(0);
  st(0);
  __syncthreads();

  for (int jt = 0; jt < ntiles; ++jt) {
    const bool more = jt + 1 < ntiles;
    if (more) gl(jt + 1);
    const int j0 = jt * 64;
    const char* sK = smem[jt & 1];
    const char* sV = sK + 16384;
    if (j0 <= i0 + 31) {
      floatx16 s[2];
      zero(s[0]);
      zero(s[1]);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int js = 0; js < 2; ++js) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + (offK[js] ^ (32u * ks)));
          s[js] = mfma(kf, qf[ks], s[js]);
        }
      // running max over raw scores (the positive scale preserves order);
      // masked keys only on the diagonal tiles
      if (j0 + 63 > i0) {
#pragma unroll
        for (int js = 0; js < 2; ++js)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (j0 + js * 32 + 8 * (r >> 2) + 4 * hh + (r & 3) > my_i) s[js][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int js = 0; js < 2; ++js)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[js][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * kScaleLog2;
      // m is the reference (log2-scaled) the exponentials are taken
      // against.  It follows the running maximum lazily: only when some
      // row's maximum passes it by more than kLazy is it raised (and the
      // running sums rescaled), so p <= 2^kLazy -- harmless in fp32 sums
      // and bf16 operands -- and most tiles skip the rescale.
      constexpr float kLazy = 8.f;
      if (__any(mx > m + kLazy)) {
        const float mn = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        l *= alpha;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[t][r] *= alpha;
        m = mn;
      }
      float ls = 0.f;
#pragma unroll
      for (int js = 0; js < 2; ++js)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[js][r], kScaleLog2, -m));
          s[js][r] = p;
          ls += p;
        }
      l += ls;
#pragma unroll
      for (int sp = 0; sp < 4; ++sp) {
        const bf16x8 pf = pack8(s[sp >> 1], 8 * (sp & 1));
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x8 vf = frag_tr(sV, tv.l(t, sp), tv.h(t, sp));
          o[t] = mfma(vf, pf, o[t]);
        }
      }
    }
    if (more) st((jt + 1) & 1);
    __syncthreads();
  }

  l += __shfl_xor(l, 32, 64);
  const float inv = 1.f / l;
  bf16* out = (bf16*)a.o_out + ((int64_t)b * T + my_i) * d + h * HD + 4 * hh;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint2 w = make_uint2(pack2(o[t][4 * g] * inv, o[t][4 * g + 1] * inv),
                                 pack2(o[t][4 * g + 2] * inv, o[t][4 * g + 3] * inv));
      *reinterpret_cast<uint2*>(out + t * 32 + 8 * g) = w;
    }
  if (hh == 0) a.lse[((int64_t)b * H + h) * T + my_i] = (m + __log2f(l)) * kLn2;
}

// inverse rotation of 4 consecutive features (2 adjacent pairs) at pair index pi
__device__ inline void rope_inv4(float* v, const float2* tab_t, int pi) {
  const float4 cs = *reinterpret_cast<const float4*>(tab_t + pi);
  const float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
  v[0] = x0 * cs.x + x1 * cs.y;
  v[1] = -x0 * cs.y + x1 * cs.x;
  v[2] = x2 * cs.z + x3 * cs.w;
  v[3] = -x2 * cs.w + x3 * cs.z;
}

// store a wave's 32 rows x 128 features accumulator (lane = row, regs = features)
__device__ inline void store_rows(floatx16 (&acc)[4], float scale, bf16* dst_row, const float2* rope_t, int hh) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float v[4] = {acc[t][4 * g] * scale, acc[t][4 * g + 1] * scale, acc[t][4 * g + 2] * scale,
                    acc[t][4 * g + 3] * scale};
      const int f = t * 32 + 8 * g + 4 * hh;
      if (rope_t) rope_inv4(v, rope_t, f >> 1);
      *reinterpret_cast<uint2*>(dst_row + f) = make_uint2(pack2(v[0], v[1]), pack2(v[2], v[3]));
    }
}

// ===========================================================================
// backward: dQ (one wave = 32 query rows, walking key tiles up to the
// diagonal).  It also forms delta_i = sum_d dO[i,d] O[i,d] from the rows it
// holds and stores it for the dK kernel.  K and V tiles are double-buffered:
// the next tile's loads are in flight while this one is used.
// ===========================================================================
__global__ void __launch_bounds__(256, 2) k_attn_dq(AttnDesc a) {
  __shared__ __attribute__((aligned(16))) char smem[2][32768];   // per stage: K image | V image
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hh = lane >> 5;
  const int T = a.T, H = a.H, d = H * HD;
  int qt, h, b;
  tile_order(T / 128, H, a.B, qt, h, b);
  qt = T / 128 - 1 - qt;
  const int64_t ld = 3LL * d;
  const bf16* rows = (const bf16*)a.qkv + (int64_t)b * T * ld;
  const bf16* qb = rows + h * HD;
  const bf16* kb = rows + d + h * HD;
  const bf16* vb = rows + 2 * d + h * HD;
  const int q0 = qt * 128, i0 = q0 + wave * 32, my_i = i0 + (lane & 31);
  const int64_t tok = (int64_t)b * T + my_i;
  const bf16* dob = (const bf16*)a.dout + tok * d + h * HD;
  const bf16* ob = (const bf16*)a.o + tok * d + h * HD;

  const int ntiles = (q0 + 128) / 64;
  // one staging register set, used for the K then the V image of a tile
  u32x4 rg[4];
  auto gl = [&](const bf16* src, int jt) { load_nat64<256>(src + (int64_t)jt * 64 * ld, ld, tid, rg); };
  auto st = [&](char* img) { store_nat64<256>(img, tid, rg); };
  gl(kb, 0);

  bf16x8 qf[8], dof[8];
  float Dl = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    qf[s] = as_bf16x8(gload(qb + (int64_t)my_i * ld + 16 * s + 8 * hh));
    const u32x4 dw = gload(dob + 16 * s + 8 * hh), ow = gload(ob + 16 * s + 8 * hh);
    dof[s] = as_bf16x8(dw);
#pragma unroll
    for (int e = 0; e < 4; ++e) Dl += bf_lo(dw[e]) * bf_lo(ow[e]) + bf_hi(dw[e]) * bf_hi(ow[e]);
  }
  Dl += __shfl_xor(Dl, 32, 64);
  const int64_t sidx = ((int64_t)b * H + h) * T + my_i;
  if (hh == 0) a.delta[sidx] = Dl;
  const float lse2 = a.lse[sidx] * kLog2e;

  floatx16 dq[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) zero(dq[t]);
  TrOff tk;
  tk.init(lane);
  uint32_t offR[2];
#pragma unroll
  for (int js = 0; js < 2; ++js) offR[js] = offN(js * 32 + (lane & 31), hh);   // chunk 2 ks + hh: ^ 32 ks

  st(smem[0]);
  gl(vb, 0);
  st(smem[0] + 16384);
  __syncthreads();
  // The next tile is staged in two halves, each loaded before and written
  // after half of this tile's work: K(jt+1) around keys 0-31, V(jt+1)
  // around keys 32-63.
  for (int jt = 0; jt < ntiles; ++jt) {
    const bool more = jt + 1 < ntiles;
    char* nx = smem[(jt + 1) & 1];
    if (more) gl(kb, jt + 1);
    const int j0 = jt * 64;
    const char* sK = smem[jt & 1];
    const char* sV = sK + 16384;
#pragma unroll
    for (int js = 0; js < 2; ++js) {
      if (js == 1 && more) {
        st(nx);
        gl(vb, jt + 1);
      }
      const int jh = j0 + js * 32;
      if (jh > i0 + 31) continue;                 // all 32 keys above the diagonal
      floatx16 s, dp;
      zero(s);
      zero(dp);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + (offR[js] ^ (32u * ks)));
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(sV + (offR[js] ^ (32u * ks)));
        s = mfma(kf, qf[ks], s);
        dp = mfma(vf, dof[ks], dp);
      }
      const bool diag = jh + 31 > i0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(s[r] * kScaleLog2 - lse2);
        if (diag && jh + 8 * (r >> 2) + 4 * hh + (r & 3) > my_i) p = 0.f;
        s[r] = p * (dp[r] - Dl);                   // dS
      }
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        const bf16x8 df = pack8(s, 8 * gp);
        const uint32_t sp = js * 2 + gp;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bf16x8 kf = frag_tr(sK, tk.l(t, sp), tk.h(t, sp));
          dq[t] = mfma(kf, df, dq[t]);
        }
      }
    }
    if (more) st(nx + 16384);
    __syncthreads();
  }
  bf16* dst = (bf16*)a.dqkv + tok * ld + h * HD;
  store_rows(dq, 0.08838834764831845f, dst, a.rope ? a.rope + (int64_t)my_i * (HD / 2) : nullptr, hh);
}

// ===========================================================================
// backward: dK and dV.  A block owns 128 keys and has 8 waves in 4 pairs;
// the two waves of pair w (w and w + 4, on the same SIMD) own keys
// jb + 32w .. +31 and walk the 32-query halves of the query tiles from the
// diagonal, splitting the work:
//   wave w     (P role): S = Q K^T, P = exp(S - lse) -> LDS, dV += P^T dO
//   wave w + 4 (D role): dP = dO V^T; one half later, with that half's P
//                        from LDS, dS = P (dP - delta), dK += dS^T Q
// The D role lags one half so that, between two barriers, the two waves'
// work is independent and interleaves on their SIMD; each issues 32 MFMAs
// per half and P's exponentials are formed once.  Q and dO tiles (with
// their log-sum-exp and delta values) are double-buffered: the next tile's
// loads are in flight during this one, and a stage is rewritten only after
// the lagging role's last use of it.
// ===========================================================================
__global__ void __launch_bounds__(512, 1) k_attn_dkdv(AttnDesc a) {
  constexpr int SST = 32768 + 512;               // per stage: Q image | dO image | lse2[64] | delta[64]
  constexpr int PX = 4096;                       // one pair's P for one half: [4][64 lanes][4 floats]
  __shared__ __attribute__((aligned(16))) char smem[2 * SST + 8 * PX];
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave & 3;
  const bool roleP = wave < 4;
  const int T = a.T, H = a.H, d = H * HD;
  int kt, h, b;
  tile_order(T / 128, H, a.B, kt, h, b);                         // low key tiles do the most work
  const int64_t ld = 3LL * d;
  const bf16* rows = (const bf16*)a.qkv + (int64_t)b * T * ld;
  const bf16* qb = rows + h * HD;
  const bf16* kb = rows + d + h * HD;
  const bf16* vb = rows + 2 * d + h * HD;
  const bf16* dob = (const bf16*)a.dout + (int64_t)b * T * d + h * HD;
  const int jb = kt * 128, jw = jb + pair * 32, my_j = jw + (lane & 31);
  const float* lse_bh = a.lse + ((int64_t)b * H + h) * T;
  const float* del_bh = a.delta + ((int64_t)b * H + h) * T;

  u32x4 rq[2], ro[2];
  float rs = 0.f;                                // lse (threads 0-63) or delta (64-127) of one query
  // (lse is scaled to base 2 when stored, not when loaded: a use right
  // after the load would wait for every load in flight)
  auto gl = [&](int qt) {
    const int64_t i0 = (int64_t)qt * 64;
    load_nat64<512>(qb + i0 * ld, ld, tid, rq);
    load_nat64<512>(dob + i0 * d, d, tid, ro);
    if (tid < 64) rs = lse_bh[i0 + tid];
    else if (tid < 128) rs = del_bh[i0 + tid - 64];
  };
  auto st = [&](char* base) {
    store_nat64<512>(base, tid, rq);
    store_nat64<512>(base + 16384, tid, ro);
    if (tid < 128) reinterpret_cast<float*>(base + 32768)[tid] = tid < 64 ? rs * kLog2e : rs;
  };
  const int qt0 = jb / 64, nq = T / 64;
  gl(qt0);

  // key-side operand: K rows (P role) or V rows (D role) of the pair's keys
  bf16x8 kv[8];
  {
    const bf16* src = (roleP ? kb : vb) + (int64_t)my_j * ld + 8 * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s) kv[s] = as_bf16x8(gload(src + 16 * s));
    // Wait for these rows here, once: otherwise the loop's first products
    // wait on the load counter, which by then also counts the next tile's
    // loads, and every tile would sit out their latency.
#pragma unroll
    for (int s = 0; s < 8; ++s) asm volatile("" : "+v"(kv[s]));
  }
  floatx16 acc[4];                               // dV (P role) or dK (D role)
#pragma unroll
  for (int t = 0; t < 4; ++t) zero(acc[t]);
  TrOff tt;
  tt.init(lane);
  uint32_t offR[2];
#pragma unroll
  for (int is = 0; is < 2; ++is) offR[is] = offN(is * 32 + (lane & 31), hh);   // chunk 2 ks + hh: ^ 32 ks
  float* pxb = reinterpret_cast<float*>(smem + 2 * SST) + pair * 2 * (PX / 4);

  // phase 2 of a half: acc += X^T x with X^T read transposed from img (Q^T
  // for dK, dO^T for dV) at the half's slot pairs
  auto accumulate = [&](floatx16& x, const char* img, int is) {
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      const uint32_t sp = is * 2 + gp;
      const bf16x8 bfr = pack8(x, 8 * gp);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = mfma(frag_tr(img, tt.l(t, sp), tt.h(t, sp)), bfr, acc[t]);
    }
  };
  // D role, lagging half: dS = P (dP - delta), dK += dS^T Q
  floatx16 dpp;                                  // dP of the pending half
  zero(dpp);
  bool pend = false;                             // a half waits for its dS / dK
  const char* pQ = smem;                         // that half's stage
  int pis = 0, pk = 0;
  auto finish_d = [&]() {
    const float* px = pxb + (pk & 1) * (PX / 4);
    const float* sD = reinterpret_cast<const float*>(pQ + 32768) + 64;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int il = pis * 32 + 8 * g + 4 * hh;
      const float4 Dv = *reinterpret_cast<const float4*>(sD + il);
      const float4 P = *reinterpret_cast<const float4*>(px + (g * 64 + lane) * 4);
      dpp[4 * g + 0] = P.x * (dpp[4 * g + 0] - Dv.x);
      dpp[4 * g + 1] = P.y * (dpp[4 * g + 1] - Dv.y);
      dpp[4 * g + 2] = P.z * (dpp[4 * g + 2] - Dv.z);
      dpp[4 * g + 3] = P.w * (dpp[4 * g + 3] - Dv.w);
    }
    accumulate(dpp, pQ, pis);
  };

  st(smem);
  __syncthreads();
  // One loop per role (the roles branch on a wave-uniform value; both
  // loops pass the same barriers).
  auto run = [&](auto role) {
    constexpr bool kP = decltype(role)::value;
    int k = 0;                                   // half counter: P of half k goes to buffer k & 1
    for (int qt = qt0; qt < nq; ++qt) {
      const bool more = qt + 1 < nq;
      if (more) gl(qt + 1);
      const int i0 = qt * 64;
      const char* sQ = smem + ((qt - qt0) & 1) * SST;
      const char* sO = sQ + 16384;
      const float* sL = reinterpret_cast<const float*>(sQ + 32768);
#pragma unroll
      for (int is = 0; is < 2; ++is, ++k) {
        const int ih = i0 + is * 32;
        const bool live = ih + 31 >= jw;          // some query of the half sees the pair's keys
        const bool diag = ih < jw + 31;
        if constexpr (!kP) {
          if (pend) finish_d();
        }
        // lane = key j, register r = query ih + 8(r/4) + 4hh + r%4
        floatx16 x;
        zero(x);
        if (live) {
          const char* img = kP ? sQ : sO;
#pragma unroll
          for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 fa = *reinterpret_cast<const bf16x8*>(img + (offR[is] ^ (32u * ks)));
            x = mfma(fa, kv[ks], x);
          }
        }
        if constexpr (kP) {
          if (live) {
            float* px = pxb + (k & 1) * (PX / 4);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int il = is * 32 + 8 * g + 4 * hh;
              const float4 L = *reinterpret_cast<const float4*>(sL + il);
              const float Ls[4] = {L.x, L.y, L.z, L.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * g + e;
                float p = __builtin_amdgcn_exp2f(x[r] * kScaleLog2 - Ls[e]);
                if (diag && i0 + il + e < my_j) p = 0.f;
                x[r] = p;
              }
              *reinterpret_cast<float4*>(px + (g * 64 + lane) * 4) =
                  make_float4(x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]);
            }
            accumulate(x, sO, is);                // dV += P^T dO
          }
        } else {
          dpp = x;
          pend = live;
          pQ = sQ;
          pis = is;
          pk = k;
        }
        // P of this half visible to the D role from here on; with is = 1,
        // the staged next tile is written first (its stage last served the
        // previous tile, whose pending half the D role finished above)
        if (is == 1 && more) st(smem + ((qt + 1 - qt0) & 1) * SST);
        __syncthreads();
      }
    }
  };
  if (roleP) run(std::true_type{});
  else run(std::false_type{});
  if (!roleP && pend) finish_d();
  bf16* dst = (bf16*)a.dqkv + ((int64_t)b * T + my_j) * ld + h * HD;
  if (roleP) store_rows(acc, 1.f, dst + 2 * d, nullptr, hh);
  else store_rows(acc, 0.08838834764831845f, dst + d, a.rope ? a.rope + (int64_t)my_j * (HD / 2) : nullptr, hh);
}

}  // namespace

bool attn_mfma_supported(const AttnDesc& a) { return a.Q == HD && a.T % 128 == 0 && a.T > 0; }

hipError_t attn_fwd_mfma(const AttnDesc& a, hipStream_t s) {
  if (!attn_mfma_supported(a)) return hipErrorNotSupported;
  k_attn_fwd<<<dim3(a.T / 128, a.H, a.B), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t attn_bwd_mfma(const AttnDesc& a, hipStream_t s) {
  if (!attn_mfma_supported(a)) return hipErrorNotSupported;
  const dim3 grid(a.T / 128, a.H, a.B);
  k_attn_dq<<<grid, 256, 0, s>>>(a);             // also writes delta
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_attn_dkdv<<<grid, 512, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace nc
