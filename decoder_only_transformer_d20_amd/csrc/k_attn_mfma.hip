// Causal flash attention, forward and backward, on gfx950 matrix cores
// (bf16 operands, fp32 accumulation and softmax statistics), head dim 128,
// T a multiple of 64.
//
// Forward: a workgroup (4 waves) owns 128 query rows of one (row, head), a
// wave 32 of them; it walks the 64-key tiles up to its diagonal with an
// online softmax, issuing the next tile's score products while it forms
// the current tile's exponentials.  Backward: one kernel accumulates dQ
// over key tiles (and forms delta = rowsum(dO * O)), one accumulates dK, dV
// over query tiles; both recompute P from the saved log-sum-exp -- no
// atomics, so the result does not depend on scheduling.  dQ and dK leave
// through the inverse rotary rotation, so the caller receives gradients with
// respect to the pre-rotation q and k.  Every tile reaches LDS by direct
// global-to-LDS copies into a ring of slots: the forward's and dQ's K/V
// tiles as buffer loads (TileCopy: a scalar tile offset on offsets computed
// once), the others as global_load_lds_dwordx4.
#include <type_traits>

#include "attn_mfma.h"

namespace nc {
using namespace attn;

namespace {

constexpr float kScaleLog2 = kLog2e * 0.08838834764831845f;   // log2(e) / sqrt(128)

// Block -> (tile, head, row); tile 0 is the heaviest of a (row, head) group
// (the most key or query tiles to walk).  Workgroups are dealt to the 8 XCDs
// round-robin; renumbering so each XCD takes a contiguous run of the
// (row, head) groups keeps the tiles that share one head's K/V (or Q/dO)
// rows in one XCD's L2.  Within an XCD's run, windows of kOrderWindow groups
// are dispatched heaviest tile first across the window (all its groups'
// tile 0, then their tile 1, ...): a window holds about as many blocks as
// the XCD runs at once, so the groups in flight are the same as group by
// group, but the light tiles come last and fill the slots the heavy ones
// leave, instead of one group's heavy tile starting last and running alone.
constexpr int kOrderWindow = 4;
__device__ inline void tile_order(int ntile, int H, int B, int& tile, int& h, int& b) {
  const int total = ntile * H * B;
  const int L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  int grp;
  if ((H * B) % 8 == 0) {
    const int per = H * B / 8;                   // groups per XCD
    const int x = L & 7, j = L >> 3;
    const int wi = j / (kOrderWindow * ntile);
    const int g0 = wi * kOrderWindow;
    const int gw = min(kOrderWindow, per - g0);  // groups in this window
    const int r = j - wi * kOrderWindow * ntile;
    tile = r / gw;
    grp = x * per + g0 + r % gw;
  } else {
    const int Lr = (total & 7) == 0 ? (L & 7) * (total >> 3) + (L >> 3) : L;
    tile = Lr % ntile;
    grp = Lr / ntile;
  }
  h = grp % H;
  b = grp / H;
}

// ===========================================================================
// forward, software-pipelined: while a wave forms the softmax weights of key
// tile j it already issues the score products of tile j + 1, so its matrix
// core has independent work during the exponentials; the lazy maximum check
// of tile j + 1 runs after tile j's value products.  LDS holds K tiles in a
// ring of two (K[j+1] is read while K[j+2] is staged) and V tiles in a ring
// of two (V[j] is read while V[j+1] is staged).
// ===========================================================================
// kHalf: the one 64-query block that T % 128 == 64 leaves at the end of
// each row, launched separately (waves 2, 3 have no queries), so the
// full-block kernel carries none of its guards.
template <bool kHalf>
__global__ void __launch_bounds__(256, 2) k_attn_fwd(AttnDesc a) {
  // separate arrays, so the compiler can tell the copies into one slot from
  // the reads of another
  __shared__ __attribute__((aligned(16))) char sK0[16384], sK1[16384], sV0[16384], sV1[16384];
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, H = a.H, d = H * HD;
  int qt, h, b;
  if (kHalf) {
    qt = T / 128;
    h = blockIdx.y;
    b = blockIdx.z;
  } else {
    tile_order(T / 128, H, a.B, qt, h, b);
    qt = T / 128 - 1 - qt;                                       // heaviest tiles first
  }
  const int64_t ld = 3LL * d;
  const bf16* rows = (const bf16*)a.qkv + (int64_t)b * T * ld;
  const bf16* qb = rows + h * HD;
  const bf16* kb = rows + d + h * HD;
  const bf16* vb = rows + 2 * d + h * HD;
  const int q0 = qt * 128, i0 = q0 + wave * 32;
  // in the half block, waves 2, 3 have no queries: they run on a valid row
  // and store nothing
  const bool active = !kHalf || i0 < T;
  const int my_i = active ? i0 + (lane & 31) : T - 1;
  const int ntk = T / 64;                                        // key tiles that exist
  const int ntiles = (q0 + 128) / 64;                            // the block's (even; ntk + 1 for a half block)
  const int last = (i0 + 31) / 64;                               // this wave's diagonal tile

  // the bytes of one head's K (or V) column block: rows 0 .. T-1, 128 wide
  const int64_t span = (int64_t)(T - 1) * ld * 2 + HD * 2;
  TileCopy<4> ck, cv;
  ck.init(kb, span, ld, wave, lane);
  cv.init(vb, span, ld, wave, lane);
  auto dmaK = [&](int jt, char* img) { ck.copy(jt * 64, ld, img, wave); };
  auto dmaV = [&](int jt, char* img) { cv.copy(jt * 64, ld, img, wave); };
  // (copies past the last key tile re-copy that tile into a slot nobody
  // reads: clamped indices keep the loop free of branches)
  dmaK(0, sK0);
  dmaV(0, sV0);
  dmaK(kHalf ? min(1, ntk - 1) : 1, sK1);

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
  auto kfrag = [&](const char* sK, int js, int ks) {
    return *reinterpret_cast<const bf16x8*>(sK + (offK[js] ^ (32u * ks)));
  };

  // keys after the query on the diagonal tile
  auto mask = [&](int jt, floatx16 (&s)[2]) {
#pragma unroll
    for (int js = 0; js < 2; ++js)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (jt * 64 + js * 32 + 8 * (r >> 2) + 4 * hh + (r & 3) > my_i) s[js][r] = -INFINITY;
  };
  // m is the reference (log2-scaled) the exponentials are taken against.
  // It follows the running maximum lazily: only when some row's maximum
  // passes it by more than kLazy is it raised (and the running sums
  // rescaled), so p <= 2^kLazy -- harmless in fp32 sums and bf16 operands
  // -- and most tiles skip the rescale.
  auto raise_max = [&](const floatx16 (&s)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int js = 0; js < 2; ++js)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[js][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * kScaleLog2;
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
  };
  // weights e = 4 ks .. 4 ks + 3 of the 32 in s (in place), added to ls
  auto weights4 = [&](floatx16 (&s)[2], int ks, float& ls) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * ks + e;
      const float p = __builtin_amdgcn_exp2f(fmaf(s[r >> 4][r & 15], kScaleLog2, -m));
      s[r >> 4][r & 15] = p;
      ls += p;
    }
  };
  auto values = [&](const char* sV, floatx16 (&s)[2]) {
#pragma unroll
    for (int sp = 0; sp < 4; ++sp) {
      const bf16x8 pf = pack8(s[sp >> 1], 8 * (sp & 1));
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] = mfma(frag_tr(sV, tv.l(t, sp), tv.h(t, sp)), pf, o[t]);
    }
  };

  // q rows first: the score products below would otherwise wait on the
  // memory counter behind the tile copies
#pragma unroll
  for (int s = 0; s < 8; ++s) asm volatile("" : "+v"(qf[s]));
  vm_wait();
  __syncthreads();
  floatx16 sa[2], sb[2];
  zero(sa[0]);
  zero(sa[1]);
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
#pragma unroll
    for (int js = 0; js < 2; ++js) sa[js] = mfma(kfrag(sK0, js, ks), qf[ks], sa[js]);
  if (last == 0) mask(0, sa);
  raise_max(sa);
  __syncthreads();                                               // K slot 0 is rewritten below

  // Key tile jt of parity P: s_cur holds its scores (masked where needed,
  // m covering their maximum).  Reads K slot 1 - P (tile jt + 1) and V slot
  // P (tile jt); the copies of K[jt + 2] into K slot P and V[jt + 1] into V
  // slot 1 - P (both last read before the previous barrier) are issued
  // before and waited for after.
  auto slots = [&](auto par, char*& kNext, char*& kFree, char*& vCur, char*& vFree) {
    constexpr int P = decltype(par)::value;
    kNext = P ? sK0 : sK1;
    kFree = P ? sK1 : sK0;
    vCur = P ? sV1 : sV0;
    vFree = P ? sV0 : sV1;
  };
  // a tile before the wave's diagonal one: tile jt + 1's score products
  // interleave with tile jt's exponentials
  auto tile_mid = [&](int jt, const char* kNext, const char* vCur, floatx16 (&s_cur)[2], floatx16 (&s_nxt)[2]) {
    zero(s_nxt[0]);
    zero(s_nxt[1]);
    float ls = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int js = 0; js < 2; ++js) s_nxt[js] = mfma(kfrag(kNext, js, ks), qf[ks], s_nxt[js]);
      weights4(s_cur, ks, ls);
    }
    l += ls;
    values(vCur, s_cur);
    if (jt + 1 == last) mask(jt + 1, s_nxt);
    raise_max(s_nxt);
  };
  // the wave's diagonal tile
  auto tile_last = [&](const char* vCur, floatx16 (&s_cur)[2]) {
    float ls = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) weights4(s_cur, ks, ls);
    l += ls;
    values(vCur, s_cur);
  };
  char *kNext, *kFree, *vCur, *vFree;
  // every wave's diagonal tile is ntiles - 2 (waves 0, 1) or ntiles - 1
  // (waves 2, 3): the tiles before ntiles - 2 take the same path in every
  // wave (ntiles - 2 is even, so the loop runs in pairs of slot parities)
  // (a wave without queries runs the loop on its clamped row and discards
  // the result)
  for (int jt = 0; jt < ntiles - 2; jt += 2) {
    slots(std::false_type{}, kNext, kFree, vCur, vFree);
    dmaK(jt + 2, kFree);
    dmaV(jt + 1, vFree);
    tile_mid(jt, kNext, vCur, sa, sb);
    vm_wait();
    __syncthreads();
    slots(std::true_type{}, kNext, kFree, vCur, vFree);
    dmaK(kHalf ? min(jt + 3, ntk - 1) : jt + 3, kFree);
    dmaV(jt + 2, vFree);
    tile_mid(jt + 1, kNext, vCur, sb, sa);
    vm_wait();
    __syncthreads();
  }
  {
    const int jt = ntiles - 2;
    slots(std::false_type{}, kNext, kFree, vCur, vFree);
    dmaV(kHalf ? min(jt + 1, ntk - 1) : jt + 1, vFree);
    if (jt < last) tile_mid(jt, kNext, vCur, sa, sb);
    else tile_last(vCur, sa);
    vm_wait();
    __syncthreads();
    slots(std::true_type{}, kNext, kFree, vCur, vFree);
    if (jt + 1 == last) tile_last(vCur, sb);
  }

  l += __shfl_xor(l, 32, 64);
  const float inv = 1.f / l;
  // (a wave without queries stores nothing: its lanes are switched off
  // for the stores rather than returned early, which keeps the register
  // allocation of the loop above as it is without that wave)
  bf16* out = (bf16*)a.o_out + ((int64_t)b * T + my_i) * d + h * HD + 4 * hh;
  if (active) {
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
}

// (instantiated explicitly: without it the host stub of one of the
// launched instantiations was left undefined in the library)
template __global__ void k_attn_fwd<false>(AttnDesc);
template __global__ void k_attn_fwd<true>(AttnDesc);

// store a wave's 32 rows x 128 features accumulator (lane = row, regs =
// features), rotated back by the row's rotary angles when `rot` (wave-
// uniform).  Every rotary factor is requested before the first store: the
// memory counter is in order, so a factor loaded after a store would wait
// for that store as well.
__device__ inline void store_rows(floatx16 (&acc)[4], float scale, bf16* dst_row, const float2* rope_t, int hh,
                                  bool rot) {
  float4 cs[16];
  if (rot) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        cs[4 * t + g] = *reinterpret_cast<const float4*>(rope_t + ((t * 32 + 8 * g + 4 * hh) >> 1));
  }
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float v[4] = {acc[t][4 * g] * scale, acc[t][4 * g + 1] * scale, acc[t][4 * g + 2] * scale,
                    acc[t][4 * g + 3] * scale};
      const int f = t * 32 + 8 * g + 4 * hh;
      if (rot) {
        const float4 c = cs[4 * t + g];
        const float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
        v[0] = x0 * c.x + x1 * c.y;
        v[1] = -x0 * c.y + x1 * c.x;
        v[2] = x2 * c.z + x3 * c.w;
        v[3] = -x2 * c.w + x3 * c.z;
      }
      *reinterpret_cast<uint2*>(dst_row + f) = make_uint2(pack2(v[0], v[1]), pack2(v[2], v[3]));
    }
}

// ===========================================================================
// backward: dQ, restructured so the softmax-gradient arithmetic overlaps
// matrix-core work.  Per 64-key tile a wave forms S and dP of both 32-key
// halves, then dS of the first half while the second half's products run,
// then dS of the second half beside the first half's dQ products.  K and V
// tiles are copied straight into a 2-slot LDS ring (TileCopy); the
// tile on the wave's diagonal is peeled off the loop so the loop body has
// no masking.  Also forms delta_i = sum_d dO[i,d] O[i,d] for the dK/dV
// kernel, as k_attn_dq does.
// ===========================================================================
__global__ void __launch_bounds__(256, 2) k_attn_dq(AttnDesc a) {
  __shared__ __attribute__((aligned(16))) char sK0[16384], sV0[16384], sK1[16384], sV1[16384];
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, H = a.H, d = H * HD;
  int qt, h, b;
  const int ntq = (T + 127) / 128;
  tile_order(ntq, H, a.B, qt, h, b);
  qt = ntq - 1 - qt;
  const int64_t ld = 3LL * d;
  const bf16* rows = (const bf16*)a.qkv + (int64_t)b * T * ld;
  const bf16* qb = rows + h * HD;
  const bf16* kb = rows + d + h * HD;
  const bf16* vb = rows + 2 * d + h * HD;
  const int q0 = qt * 128, i0 = q0 + wave * 32;
  // with T % 128 == 64 the last block's waves 2, 3 have no queries: they
  // load a valid row, compute nothing and store nothing
  const bool active = i0 < T;
  const int my_i = active ? i0 + (lane & 31) : T - 1;
  const int64_t tok = (int64_t)b * T + my_i;
  const bf16* dob = (const bf16*)a.dout + tok * d + h * HD;
  const bf16* ob = (const bf16*)a.o + tok * d + h * HD;
  const int ntk = T / 64;                                        // key tiles that exist
  const int ntiles = (q0 + 128) / 64;                            // the block's (even; ntk + 1 for a half block)
  const int last = (i0 + 31) / 64;                               // the wave's diagonal tile

  const int64_t span = (int64_t)(T - 1) * ld * 2 + HD * 2;
  TileCopy<4> ck, cv;
  ck.init(kb, span, ld, wave, lane);
  cv.init(vb, span, ld, wave, lane);
  auto dma = [&](int jt, char* sK, char* sV) {
    ck.copy(jt * 64, ld, sK, wave);
    cv.copy(jt * 64, ld, sV, wave);
  };
  dma(0, sK0, sV0);

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
  if (active && hh == 0) a.delta[sidx] = Dl;
  const float lse2 = a.lse[sidx] * kLog2e;

  floatx16 dq[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) zero(dq[t]);
  TrOff tk;
  tk.init(lane);
  uint32_t offR[2];
#pragma unroll
  for (int js = 0; js < 2; ++js) offR[js] = offN(js * 32 + (lane & 31), hh);   // chunk 2 ks + hh: ^ 32 ks

  // S = K Q^T and dP = V dO^T of keys js * 32 .. +31 of the tile
  auto products = [&](const char* sK, const char* sV, int js, floatx16& s, floatx16& dp) {
    zero(s);
    zero(dp);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      s = mfma(*reinterpret_cast<const bf16x8*>(sK + (offR[js] ^ (32u * ks))), qf[ks], s);
      dp = mfma(*reinterpret_cast<const bf16x8*>(sV + (offR[js] ^ (32u * ks))), dof[ks], dp);
    }
  };
  // dS = P (dP - delta), P = exp(S / sqrt(Q) - lse), for elements r0 .. r0+n-1
  auto grad = [&](floatx16& s, const floatx16& dp, int r0, int n) {
#pragma unroll
    for (int r = r0; r < r0 + n; ++r) {
      const float p = __builtin_amdgcn_exp2f(s[r] * kScaleLog2 - lse2);
      s[r] = p * (dp[r] - Dl);
    }
  };
  auto mask = [&](int jh, floatx16& s) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (jh + 8 * (r >> 2) + 4 * hh + (r & 3) > my_i) s[r] = -INFINITY;
  };
  // dQ += dS K over keys js * 32 .. +31 (K^T read transposed), 2 MFMAs per
  // key group gp; `during(gp)` runs beside them
  auto dq_acc = [&](const char* sK, int js, const floatx16& ds, auto during) {
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      const bf16x8 df = pack8(ds, 8 * gp);
      const uint32_t sp = js * 2 + gp;
#pragma unroll
      for (int t = 0; t < 4; ++t) dq[t] = mfma(frag_tr(sK, tk.l(t, sp), tk.h(t, sp)), df, dq[t]);
      during(gp);
    }
  };

  // a tile wholly below the wave's diagonal
  auto tile_full = [&](const char* sK, const char* sV) {
    floatx16 s0, p0, s1, p1;
    products(sK, sV, 0, s0, p0);
    // second half's products beside the first half's dS
    zero(s1);
    zero(p1);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      s1 = mfma(*reinterpret_cast<const bf16x8*>(sK + (offR[1] ^ (32u * ks))), qf[ks], s1);
      p1 = mfma(*reinterpret_cast<const bf16x8*>(sV + (offR[1] ^ (32u * ks))), dof[ks], p1);
      grad(s0, p0, 2 * ks, 2);
    }
    dq_acc(sK, 0, s0, [&](int gp) { grad(s1, p1, 8 * gp, 8); });
    dq_acc(sK, 1, s1, [&](int) {});
  };
  // the wave's diagonal tile: keys jd .. jd+31 cross it (jd = i0 or i0 - 32)
  auto tile_diag = [&](const char* sK, const char* sV, int jt) {
    const bool odd = (wave & 1) != 0;                            // first half wholly below
    floatx16 s0, p0;
    products(sK, sV, 0, s0, p0);
    if (odd) {
      floatx16 s1, p1;
      products(sK, sV, 1, s1, p1);
      grad(s0, p0, 0, 16);
      mask(jt * 64 + 32, s1);
      grad(s1, p1, 0, 16);
      dq_acc(sK, 0, s0, [&](int) {});
      dq_acc(sK, 1, s1, [&](int) {});
    } else {
      mask(jt * 64, s0);
      grad(s0, p0, 0, 16);
      dq_acc(sK, 0, s0, [&](int) {});
    }
  };

#pragma unroll
  for (int s = 0; s < 8; ++s) {
    asm volatile("" : "+v"(qf[s]));
    asm volatile("" : "+v"(dof[s]));
  }
  vm_wait();
  __syncthreads();
  // every wave's diagonal tile is ntiles - 2 (waves 0, 1) or ntiles - 1
  // (waves 2, 3); the tiles before take the same path in every wave
  // (a wave without queries runs the loop on its clamped row and discards
  // the result; copies past the last key tile re-copy that tile)
  for (int jt = 0; jt < ntiles - 2; jt += 2) {
    dma(jt + 1, sK1, sV1);
    tile_full(sK0, sV0);
    vm_wait();
    __syncthreads();
    dma(jt + 2, sK0, sV0);
    tile_full(sK1, sV1);
    vm_wait();
    __syncthreads();
  }
  {
    const int jt = ntiles - 2;
    dma(min(jt + 1, ntk - 1), sK1, sV1);
    if (active) {
      if (jt < last) tile_full(sK0, sV0);
      else tile_diag(sK0, sV0, jt);
    }
    vm_wait();
    __syncthreads();
    if (active && jt + 1 == last) tile_diag(sK1, sV1, jt + 1);
  }
  if (!active) return;
  bf16* dst = (bf16*)a.dqkv + tok * ld + h * HD;
  store_rows(dq, 0.08838834764831845f, dst, a.rope + (int64_t)my_i * (HD / 2), hh, a.rope != nullptr);
}

// ===========================================================================
// backward: dK and dV, one wave per 32 keys doing all four products, two
// blocks per CU.  A block owns 128 keys (4 waves) and walks the 32-query
// tiles from its first key on.  Each wave keeps its keys' K rows in
// registers (the B operand of S = Q K^T); the block's V rows sit in LDS
// (the B operand of dP = dO V^T); Q, dO, lse and delta of the current query
// tile are copied into a 2-slot LDS ring.  Per tile a wave forms S and dP,
// P = exp(S - lse) and dS = P (dP - delta), and accumulates dV += P^T dO and
// dK += dS^T Q (dO^T, Q^T read transposed).  No exchange between waves: the
// only barrier is the ring swap, and with two blocks per CU the two waves
// on a SIMD come from different blocks.  No atomics: each wave sums its
// keys' gradients over the query tiles in order.
// ===========================================================================
// kDS: also store dS^T, the tile's 32 keys x 32 queries, into the dS^T
// tile buffer the stored-dS dQ kernel reads.  Tile (head, query block qb,
// 64-key tile kt) holds four 4 KB pieces, one per 32-query tile, each
// [64 keys][32 queries] bf16 (64-byte rows, so two key rows fill a 128-byte
// line and a wave's two stores write whole lines).  Lane (key, hh) writes
// its two packed groups gp (the dK product's B operands) as 16-byte chunks
// at query columns 16 gp + 8 hh .. +7: the columns hold the queries in the
// products' slot order (within each 16: 0-3, 8-11, 4-7, 12-15).
constexpr int kDkdvKeys = 128;
template <bool kDS>
__global__ void __launch_bounds__(256, 2) k_attn_dkdv(AttnDesc a) {
  constexpr int SST = 16384 + 256;               // per slot: Q image | dO image | lse[32] | delta[32]
  __shared__ __attribute__((aligned(16))) char sV[kDkdvKeys * 256];
  __shared__ __attribute__((aligned(16))) char st0[SST], st1[SST];
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, H = a.H, d = H * HD;
  int kt, h, b;
  tile_order((T + kDkdvKeys - 1) / kDkdvKeys, H, a.B, kt, h, b);
  const int64_t ld = 3LL * d;
  const bf16* rows = (const bf16*)a.qkv + (int64_t)b * T * ld;
  const bf16* qb = rows + h * HD;
  const bf16* kb = rows + d + h * HD;
  const bf16* vb = rows + 2 * d + h * HD;
  const bf16* dob = (const bf16*)a.dout + (int64_t)b * T * d + h * HD;
  const float* lse_bh = a.lse + ((int64_t)b * H + h) * T;
  const float* del_bh = a.delta + ((int64_t)b * H + h) * T;
  const int jb = kt * kDkdvKeys, jw = jb + 32 * wave;
  const int nqb = (T + 127) / 128;
  // this lane's row (key) of its 64-key tile in query block 0; query block
  // qb's tiles start qb (qb + 1) tiles further
  bf16* ds_w = kDS ? (bf16*)a.ds + (((int64_t)b * H + h) * nqb * (nqb + 1) + (jw >> 6)) * (64 * HD) +
                         ((jw & 63) + (lane & 31)) * 32 + 8 * hh
                   : nullptr;
  // with T % 128 == 64 the last block's waves 2, 3 have no keys: they load a
  // valid K row, skip every tile (all its queries precede T <= jw) and store
  // nothing
  const bool keys = jw < T;
  const int my_j = keys ? jw + (lane & 31) : T - 1;

  // this wave's V rows into the block's image (rows 32 wave ..)
  if (keys) {
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const int row = 32 * wave + i + (lane >> 4);
      const int chunk = (lane & 15) ^ (int)swz(row);
      __builtin_amdgcn_global_load_lds((gbl_vptr)(vb + (int64_t)(jb + row) * ld + chunk * 8),
                                       (lds_vptr)(sV + (32 * wave + i) * 256), 16, 0, 0);
    }
  }
  // one 32-query tile (Q, dO rows and their lse, delta) into a ring slot
  auto dma = [&](int qt, char* st) __attribute__((always_inline)) {
    const int64_t i0 = (int64_t)qt * 32;
    dma_rows<4>(qb + i0 * ld, ld, st, 32, wave, lane);
    dma_rows<4>(dob + i0 * d, d, st + 8192, 32, wave, lane);
    if (lane < 32) {
      if (wave == 0)
        __builtin_amdgcn_global_load_lds((gbl_vptr)(lse_bh + i0 + lane), (lds_vptr)(st + 16384), 4, 0, 0);
      else if (wave == 1)
        __builtin_amdgcn_global_load_lds((gbl_vptr)(del_bh + i0 + lane), (lds_vptr)(st + 16384 + 128), 4, 0, 0);
    }
  };
  const int qt0 = jb / 32, nq = T / 32;
  dma(qt0, st0);

  bf16x8 kf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) kf[s] = as_bf16x8(gload(kb + (int64_t)my_j * ld + 16 * s + 8 * hh));
#pragma unroll
  for (int s = 0; s < 8; ++s) asm volatile("" : "+v"(kf[s]));

  floatx16 accV[4], accK[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    zero(accV[t]);
    zero(accK[t]);
  }
  TrOff tt;
  tt.init(lane);
  const uint32_t offR = offN(lane & 31, hh);                     // chunk 2 ks + hh: ^ 32 ks
  const uint32_t offV = offN(32 * wave + (lane & 31), hh);

  // acc += X^T x over the tile's 32 queries, X^T read transposed from img
  auto accumulate = [&](floatx16 (&acc)[4], const floatx16& x, const char* img) __attribute__((always_inline)) {
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      const bf16x8 bfr = pack8(x, 8 * gp);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = mfma(frag_tr(img, tt.l(t, gp), tt.h(t, gp)), bfr, acc[t]);
    }
  };
  // one 32-query tile in slot st (lane = key, register r = query
  // i0 + 8 (r / 4) + 4 hh + r % 4)
  auto tile = [&](const char* st, int qt) __attribute__((always_inline)) {
    const int i0 = qt * 32;
    bf16* dst_ds = kDS ? ds_w + ((i0 >> 7) * ((i0 >> 7) + 1)) * (64 * HD) + (i0 & 127) * 64 : nullptr;
    // with kDS the tile's dS is stored even where every query precedes the
    // keys (zeros), so every tile leaves exactly two stores behind its copy
    bf16x8 d0 = {}, d1 = {};
    if (i0 >= jw) {                              // else every query of the tile precedes the keys
      const char* sQ = st;
      const char* sO = st + 8192;
      const float* sL = reinterpret_cast<const float*>(st + 16384);
      floatx16 x, y;
      zero(x);
      zero(y);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        x = mfma(*reinterpret_cast<const bf16x8*>(sQ + (offR ^ (32u * ks))), kf[ks], x);
        y = mfma(*reinterpret_cast<const bf16x8*>(sO + (offR ^ (32u * ks))),
                 *reinterpret_cast<const bf16x8*>(sV + (offV ^ (32u * ks))), y);
      }
      if (i0 == jw) {                            // the tile on the diagonal
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (i0 + 8 * (r >> 2) + 4 * hh + (r & 3) < my_j) x[r] = -INFINITY;
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 L = *reinterpret_cast<const float4*>(sL + 8 * g + 4 * hh);
        x[4 * g + 0] = __builtin_amdgcn_exp2f(fmaf(x[4 * g + 0], kScaleLog2, -L.x * kLog2e));
        x[4 * g + 1] = __builtin_amdgcn_exp2f(fmaf(x[4 * g + 1], kScaleLog2, -L.y * kLog2e));
        x[4 * g + 2] = __builtin_amdgcn_exp2f(fmaf(x[4 * g + 2], kScaleLog2, -L.z * kLog2e));
        x[4 * g + 3] = __builtin_amdgcn_exp2f(fmaf(x[4 * g + 3], kScaleLog2, -L.w * kLog2e));
      }
      accumulate(accV, x, sO);                   // dV += P^T dO
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 D = *reinterpret_cast<const float4*>(sL + 32 + 8 * g + 4 * hh);
        y[4 * g + 0] = x[4 * g + 0] * (y[4 * g + 0] - D.x);
        y[4 * g + 1] = x[4 * g + 1] * (y[4 * g + 1] - D.y);
        y[4 * g + 2] = x[4 * g + 2] * (y[4 * g + 2] - D.z);
        y[4 * g + 3] = x[4 * g + 3] * (y[4 * g + 3] - D.w);
      }
      if constexpr (kDS) {
        d0 = pack8(y, 0);
        d1 = pack8(y, 8);
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) accK[t4] = mfma(frag_tr(sQ, tt.l(t4, 0), tt.h(t4, 0)), d0, accK[t4]);
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) accK[t4] = mfma(frag_tr(sQ, tt.l(t4, 1), tt.h(t4, 1)), d1, accK[t4]);
      } else {
        accumulate(accK, y, sQ);                 // dK += dS^T Q
      }
    }
    if constexpr (kDS) {
      // streamed out, read back once by the dQ kernel: non-temporal
      __builtin_nontemporal_store(d0, reinterpret_cast<bf16x8*>(dst_ds));
      __builtin_nontemporal_store(d1, reinterpret_cast<bf16x8*>(dst_ds + 16));
    }
  };
  vm_wait();
  __syncthreads();
  // two tiles per trip, so each ring slot is a fixed array (nq - qt0 is even).
  // With kDS every tile leaves its two dS stores in flight: they were
  // issued after the ring copy (the compiler barrier keeps that order, and
  // the memory counter completes in issue order), so waiting until at most
  // 2 operations remain waits for the copy alone.
  // The barrier is then LDS-only: __syncthreads() would also wait for the
  // stores (no wave of the block reads them; the dQ kernel does, after
  // this kernel).
  auto sync_copy = [&]() __attribute__((always_inline)) {
    if constexpr (kDS) {
      vm_wait_but2();
      lds_barrier();
    } else {
      vm_wait();
      __syncthreads();
    }
  };
  for (int qt = qt0; qt < nq; qt += 2) {
    dma(qt + 1, st1);
    asm volatile("" ::: "memory");
    tile(st0, qt);
    sync_copy();
    if (qt + 2 < nq) dma(qt + 2, st0);
    asm volatile("" ::: "memory");
    tile(st1, qt + 1);
    sync_copy();
  }
  if (!keys) return;
  bf16* dst = (bf16*)a.dqkv + ((int64_t)b * T + my_j) * ld + h * HD;
  store_rows(accV, 1.f, dst + 2 * d, nullptr, hh, false);
  store_rows(accK, 0.08838834764831845f, dst + d, a.rope + (int64_t)my_j * (HD / 2), hh, a.rope != nullptr);
}

// ===========================================================================
// backward with stored dS: delta first (the dK/dV kernel needs it before
// any dQ work), then dK/dV storing dS^T, then dQ = dS K from those tiles.
// ===========================================================================
// delta[b][h][t] = sum_e dO[b,t,h,e] O[b,t,h,e]: 8 lanes per (token, head),
// 16 features each, fp32 sums combined across the 8 lanes.
__global__ void __launch_bounds__(256) k_attn_delta_rows(AttnDesc a) {
  const int64_t n = (int64_t)a.B * a.T * a.H;
  const int64_t pr = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);    // token * H + head
  const int e = threadIdx.x & 7;
  const int64_t p = pr < n ? pr : n - 1;
  const int64_t off = p * HD + 16 * e;                                  // [B*T][H][128] rows
  const u32x4* dv = reinterpret_cast<const u32x4*>((const bf16*)a.dout + off);
  const u32x4* ov = reinterpret_cast<const u32x4*>((const bf16*)a.o + off);
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const u32x4 dw = dv[c], ow = ov[c];
#pragma unroll
    for (int k = 0; k < 4; ++k) acc += bf_lo(dw[k]) * bf_lo(ow[k]) + bf_hi(dw[k]) * bf_hi(ow[k]);
  }
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  acc += __shfl_xor(acc, 4, 64);
  if (e == 0 && pr < n) {
    const int64_t tok = p / a.H, b = tok / a.T, t = tok % a.T;
    const int h = (int)(p % a.H);
    a.delta[(b * a.H + h) * a.T + t] = acc;
  }
}

// dQ = dS K / sqrt(128) from the stored dS^T tiles.  A block owns 128
// queries (a wave 32) and walks the 64-key tiles up to its diagonal; each
// tile's K rows and dS^T image are copied into a 2-slot LDS ring.  A wave
// multiplies only the 32-key halves that begin at or before its first
// query (the dK/dV kernel wrote exactly those, with zeros where the causal
// mask applies), so no masking is needed here.  Both operands come from
// transposing reads: K^T (features x keys) as A, dS^T's column block of
// the wave's queries (keys x queries) as B, keys in the same slot order on
// both sides.  The result's lane n holds the query the column n of the
// image stands for: i0 + n with bits 2 and 3 swapped.
__global__ void __launch_bounds__(256, 2) k_attn_dq_ds(AttnDesc a) {
  __shared__ __attribute__((aligned(16))) char sK0[16384], sD0[16384], sK1[16384], sD1[16384];
  const int tid = threadIdx.x, lane = tid & 63, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int T = a.T, H = a.H, d = H * HD;
  int qt, h, b;
  const int ntq = (T + 127) / 128;
  tile_order(ntq, H, a.B, qt, h, b);
  qt = ntq - 1 - qt;
  const int64_t ld = 3LL * d;
  const bf16* kb = (const bf16*)a.qkv + (int64_t)b * T * ld + d + h * HD;
  const bf16* dsq = (const bf16*)a.ds + (((int64_t)b * H + h) * ntq * (ntq + 1) + (int64_t)qt * (qt + 1)) * (64 * HD);
  const int q0 = qt * 128, i0 = q0 + wave * 32;
  const bool active = i0 < T;
  const int c = lane & 31;
  const int my_i = i0 + ((c & ~12) | ((c & 4) << 1) | ((c & 8) >> 1));
  const int ntk = T / 64;                                        // key tiles that exist
  const int ntiles = (q0 + 128) / 64;                            // the block's (even; ntk + 1 for a half block)

  // the dS^T tile into a natural [64 keys][128 queries] image: chunk c of
  // key row r comes from the 32-query piece c / 4, chunk c % 4 of its row
  auto dma = [&](int jt, char* sK, char* sD) __attribute__((always_inline)) {
    dma_nat64(kb + (int64_t)min(jt, ntk - 1) * 64 * ld, ld, sK, wave, lane);
    const bf16* t = dsq + (int64_t)jt * (64 * HD);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * wave + 4 * i + (lane >> 4);
      const int c = (lane & 15) ^ (int)swz(row);
      __builtin_amdgcn_global_load_lds((gbl_vptr)(t + (c >> 2) * (64 * 32) + row * 32 + (c & 3) * 8),
                                       (lds_vptr)(sD + (16 * wave + 4 * i) * 256), 16, 0, 0);
    }
  };
  dma(0, sK0, sD0);

  floatx16 dq[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) zero(dq[t]);
  TrOff tk;
  tk.init(lane);
  // keys js * 32 .. +31 of the tile
  auto half = [&](const char* sK, const char* sD, int js) __attribute__((always_inline)) {
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      const int sp = 2 * js + gp;
      const bf16x8 df = frag_tr(sD, tk.l(wave, sp), tk.h(wave, sp));
#pragma unroll
      for (int t = 0; t < 4; ++t) dq[t] = mfma(frag_tr(sK, tk.l(t, sp), tk.h(t, sp)), df, dq[t]);
    }
  };
  // tile jt: both halves when the second begins at or before i0, else the first
  auto tile = [&](const char* sK, const char* sD, int jt) __attribute__((always_inline)) {
    const int jh = jt * 64;
    if (!active || jh > i0) return;
    half(sK, sD, 0);
    if (jh + 32 <= i0) half(sK, sD, 1);
  };

  vm_wait();
  __syncthreads();
  for (int jt = 0; jt < ntiles; jt += 2) {
    dma(jt + 1, sK1, sD1);
    tile(sK0, sD0, jt);
    vm_wait();
    __syncthreads();
    if (jt + 2 < ntiles) dma(jt + 2, sK0, sD0);
    tile(sK1, sD1, jt + 1);
    vm_wait();
    __syncthreads();
  }
  if (!active) return;
  bf16* dst = (bf16*)a.dqkv + ((int64_t)b * T + my_i) * ld + h * HD;
  store_rows(dq, 0.08838834764831845f, dst, a.rope + (int64_t)my_i * (HD / 2), hh, a.rope != nullptr);
}

}  // namespace

// T a multiple of 64: the forward and dQ kernels take 128-query blocks and
// the dK/dV kernel 128-key blocks, so when T % 128 == 64 the last block's
// waves past T sit idle (no loads, no stores).
// The tile copies address one batch row's qkv block through a buffer
// resource (32-bit size and offsets): T * 3 H Q * 2 bytes must stay below
// 2^31.
bool attn_mfma_supported(const AttnDesc& a) {
  return a.Q == HD && a.T % 64 == 0 && a.T > 0 && (int64_t)a.T * 3 * a.H * HD * 2 < (int64_t(1) << 31);
}

hipError_t attn_fwd_mfma(const AttnDesc& a, hipStream_t s) {
  if (!attn_mfma_supported(a)) return hipErrorNotSupported;
  if (a.T >= 128) {
    k_attn_fwd<false><<<dim3(a.T / 128, a.H, a.B), 256, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.T % 128) k_attn_fwd<true><<<dim3(1, a.H, a.B), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t attn_bwd_mfma(const AttnDesc& a, hipStream_t s) {
  if (!attn_mfma_supported(a)) return hipErrorNotSupported;
  const dim3 gq((a.T + 127) / 128, a.H, a.B), gk((a.T + kDkdvKeys - 1) / kDkdvKeys, a.H, a.B);
  hipError_t e;
  if (a.ds) {
    const int64_t pairs = (int64_t)a.B * a.T * a.H;
    k_attn_delta_rows<<<(unsigned)((pairs + 31) / 32), 256, 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_attn_dkdv<true><<<gk, 256, 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    k_attn_dq_ds<<<gq, 256, 0, s>>>(a);
    return hipGetLastError();
  }
  k_attn_dq<<<gq, 256, 0, s>>>(a);   // also writes delta
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_attn_dkdv<false><<<gk, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace nc
