// bf16 matrix-core GEMM for gfx950 (CDNA4), shared by the per-tile-size
// translation units.
//
//   C[m][n] = sum_k P[m][k] * Q[n][k]
//
// Block: 512 threads (8 waves, 2 along m x 4 along n), tile BM x BN x 64,
// fp32 accumulation in v_mfma_f32_32x32x16_bf16.  Q (the n side) is the
// instruction's A operand and P (the m side) its B operand, so a lane's
// sixteen accumulators hold one row m and runs of four consecutive columns
// n: every epilogue works on contiguous 8-byte (bf16) / 16-byte (fp32)
// pieces of a row, and row-wise reductions (log-sum-exp) stay in a lane.
//
// Both operand tiles live in LDS as [row][64 k] bf16 (128 B per row), the
// 16-byte chunk c of row r stored at chunk slot c ^ ((r >> 1) & 7) (see
// lds_off): fragment reads and row writes are free of bank conflicts.
// Operands stored k-major ([rows][K]) are copied in 16-byte pieces;
// operands stored row-major in k ([K][rows], the backward pass's transposed
// products) are read as 8 x 8 blocks and transposed in registers before the
// LDS write, so every layout reaches the same LDS image.  Two LDS stages
// and one register stage: the global loads of tile k+2 are in flight while
// tile k is multiplied and tile k+1 is written; one barrier per tile.
#pragma once

#include "nc_internal.h"

namespace nc {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BK = 64;
constexpr float kLog2e = 1.4426950408889634f;

// LDS swizzle: chunk c of row r at chunk slot c ^ ((r >> 1) & 7).  gfx950's
// LDS serves 16 lanes x 16 B (64 banks) per cycle; a fragment read takes 16
// consecutive rows at one chunk, rows r and r+1 differ in bank half (128 B
// rows) and the 8 even (odd) rows in slot, so the 16 reads are distinct.
__device__ inline uint32_t lds_off(int row, int chunk) {
  return (uint32_t)row * 128u + ((uint32_t)(chunk ^ ((row >> 1) & 7)) << 4);
}

__device__ inline float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// two fp32 -> packed bf16, round to nearest even: one v_cvt_pk_bf16_f32
__device__ inline uint32_t pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 8 x 8 bf16 transpose: in[kk] holds 8 consecutive rows' elements at one k;
// out[e] holds row e's 8 consecutive k values.
__device__ inline void transpose8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a = in[2 * p][e >> 1], b = in[2 * p + 1][e >> 1];
      out[e][p] = (e & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
  }
}

typedef const u32x4 __attribute__((address_space(1)))* gptr;

template <bool B, typename T>
__device__ inline T& pick(T& a, T& b) {
  if constexpr (B) return a;
  else return b;
}

// Per-thread plan for one operand tile (R rows x 64 k), loaded by 256
// threads into `reg` (8 x 16 B) and written to LDS.
//  k-major operand ([rows][K]): thread tl takes chunk tl & 7 of rows
//    (tl >> 3) + 32 i, i < R/32 -- 8 lanes read one 128-byte row segment.
//  transposed operand ([K][rows]): thread tl < R takes the 8 x 8 block at
//    k rows (tl & 7)*8 .. +7 and tile rows (tl >> 3)*8 .. +7.
template <int R, bool TRANS>
struct Plan {
  gptr ptr;          // this thread's first 16-byte piece of the current tile
  int64_t step;      // elements between the thread's successive pieces
  int64_t kstep;     // elements to advance by one 64-k tile
  uint32_t lds[8];   // byte offsets in the operand's LDS image
  bool active;

  __device__ inline void init(const bf16* base, int64_t ld, int64_t row0, int64_t k0, int tl) {
    if (!TRANS) {
      const int r = tl >> 3, c = tl & 7;
      ptr = (gptr)(base + (row0 + r) * ld + k0 + c * 8);
      step = 32 * ld;
      kstep = BK;
#pragma unroll
      for (int i = 0; i < 8; ++i) lds[i] = i < R / 32 ? lds_off(r + 32 * i, c) : 0;
      active = true;
    } else {
      const int kc = tl & 7, mg = tl >> 3;
      ptr = (gptr)(base + (k0 + kc * 8) * ld + row0 + mg * 8);
      step = ld;
      kstep = (int64_t)BK * ld;
#pragma unroll
      for (int e = 0; e < 8; ++e) lds[e] = lds_off(mg * 8 + e, kc);
      active = tl < R;
    }
  }
  static constexpr bool kAllActive = !TRANS || R >= 256;   // 256 loaders cover the tile
  __device__ inline void load(u32x4 (&reg)[8]) const {
    if (!TRANS) {
#pragma unroll
      for (int i = 0; i < R / 32; ++i) reg[i] = ptr[(i * step) >> 3];
    } else if (kAllActive || active) {
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) reg[kk] = ptr[(kk * step) >> 3];
    }
  }
  __device__ inline void store(const u32x4 (&reg)[8], char* lds_base) const {
    if (!TRANS) {
#pragma unroll
      for (int i = 0; i < R / 32; ++i) *reinterpret_cast<u32x4*>(lds_base + lds[i]) = reg[i];
    } else if (kAllActive || active) {
      u32x4 t[8];
      transpose8(reg, t);
#pragma unroll
      for (int e = 0; e < 8; ++e) *reinterpret_cast<u32x4*>(lds_base + lds[e]) = t[e];
    }
  }
  __device__ inline void advance_if(bool more) { ptr += more ? (kstep >> 3) : 0; }
};

// NW = 8: waves in a 2 x 4 grid, wave tile (BM/2) x (BN/4), waves 0-3 stage
//         P and waves 4-7 stage Q (two waves per SIMD).  The library uses this.
// NW = 4: waves in a 2 x 2 grid, wave tile (BM/2) x (BN/2) -- half the LDS
//         fragment reads per FLOP; every thread stages both operands; the
//         accumulators live in AGPRs (one wave per SIMD).  Measured 10-15%
//         slower on the d20 shapes, so it is not instantiated.
template <int NW, int BM, int BN, bool PT, bool QT, int EPI>
__global__ void __launch_bounds__(NW * 64, 1) k_gemm_mfma(GemmDesc g) {
  static_assert(BM % 64 == 0 && BN % 128 == 0 && (NW == 4 || NW == 8), "tile");
  constexpr int WGN = NW / 2;                    // waves along n
  constexpr int WTM = BM / 2, WTN = BN / WGN;    // wave tile
  constexpr int FM = WTM / 32, FN = WTN / 32;    // 32x32 fragments per wave
  constexpr int STAGE = (BM + BN) * 128;         // bytes per LDS stage
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // Block -> (split, m-tile, n-tile).  Workgroups are dealt to the 8 XCDs
  // round-robin, so the flat index is renumbered to give each XCD a
  // contiguous run of logical tiles (splits outermost: with 8 splits an XCD
  // owns one K range).  Within a split, tiles are rastered in groups of
  // kGroupM m-tiles, m fastest: the ~32 blocks an XCD runs at once cover
  // about 8 m-tiles x 4 n-tiles, so each P panel and each Q panel (weights)
  // is reused from that XCD's L2 instead of refetched per tile.
  constexpr int kGroupM = 8;
  const int ntn = g.N / BN, ntm = g.M / BM;
  const int ntiles = ntn * ntm, total = ntiles * g.splits;
  int L = blockIdx.x;
  if ((total & 7) == 0) L = (L & 7) * (total >> 3) + (L >> 3);
  const int split = L / ntiles;
  const int t = L - split * ntiles;
  const int first_m = (t / (kGroupM * ntn)) * kGroupM;
  const int gm = min(kGroupM, ntm - first_m);
  const int tg = t - first_m * ntn;
  const int tm = first_m + tg % gm, tn = tg / gm;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;

  const int kper = g.K / g.splits;
  const int64_t kbeg = (int64_t)split * kper;
  const int nk = kper / BK;

  // NW = 8: waves 0-3 stage P tiles, waves 4-7 stage Q tiles (a wave-uniform
  // split).  NW = 4: every thread stages its share of both.  When both
  // operands have the same layout and tile height, a thread's single plan is
  // set up for whichever operand it stages, so the main loop has no branch.
  constexpr bool kUnified = NW == 8 && PT == QT && BM == BN;
  const bool loadsP = NW == 4 || tid < 256;
  const bool loadsQ = NW == 4 || tid >= 256;
  Plan<BM, PT> pp;
  Plan<BN, QT> pq;
  uint32_t my_lds = 0;
  if constexpr (kUnified) {
    if (loadsP) pp.init((const bf16*)g.P, g.ldp, m0, kbeg, tid & 255);
    else pp.init((const bf16*)g.Q, g.ldq, n0, kbeg, tid & 255);
    my_lds = loadsP ? 0u : (uint32_t)BM * 128u;
  } else {
    if (loadsP) pp.init((const bf16*)g.P, g.ldp, m0, kbeg, tid & 255);
    if (loadsQ) pq.init((const bf16*)g.Q, g.ldq, n0, kbeg, tid & 255);
  }
  u32x4 reg[8], regq[8];
  u32x4(&rq)[8] = pick<NW == 4>(regq, reg);   // NW = 8: a thread stages one operand only
  auto stage_load = [&]() {
    if constexpr (kUnified) {
      pp.load(reg);
    } else {
      if (loadsP) pp.load(reg);
      if (loadsQ) pq.load(rq);
    }
  };
  auto stage_store = [&](char* base) {
    if constexpr (kUnified) {
      pp.store(reg, base + my_lds);
    } else {
      if (loadsP) pp.store(reg, base);
      if (loadsQ) pq.store(rq, base + BM * 128);
    }
  };
  auto stage_advance = [&](bool more) {
    if constexpr (kUnified) {
      pp.advance_if(more);
    } else {
      if (loadsP) pp.advance_if(more);
      if (loadsQ) pq.advance_if(more);
    }
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Pipeline (stage s of LDS holds tile t with s = t & 1):
  //   iteration t:  write tile t+1 (staged in registers) to stage (t+1)&1,
  //                 issue the global loads of tile t+2,
  //                 k16 steps 0-2 of tile t (fragments read one step ahead),
  //                 barrier,
  //                 read tile t+1's step-0 fragments, then step 3 of tile t --
  //   so the MFMAs of step 3 cover the first LDS reads after the barrier.
  // The write of tile t+1 reuses the stage tile t-1 occupied; its last reads
  // were issued before the previous barrier, which waits for them.
  // Tiles past the last are never fetched: the staged tile index is clamped
  // to nk-1 (the pointer stops advancing), so the final iterations restage
  // the last tile into the idle stage instead of branching around the copy.
  stage_load();                 // tile 0
  stage_store(smem);
  stage_advance(nk > 1);
  stage_load();                 // tile min(1, nk-1)
  __syncthreads();

  const int frow = lane & 31, fchunk = lane >> 5;
  uint32_t offQ[FN], offP[FM];
#pragma unroll
  for (int j = 0; j < FN; ++j) offQ[j] = BM * 128 + lds_off(wn * WTN + j * 32 + frow, fchunk);
#pragma unroll
  for (int i = 0; i < FM; ++i) offP[i] = lds_off(wm * WTM + i * 32 + frow, fchunk);
  // chunk 2s + fchunk sits at slot (2s + fchunk) ^ f(row) = (fchunk ^ f(row)) ^ 2s:
  // the k16 step s moves the byte offset by an xor of 32*s

  bf16x8 a[2][FN], bb[2][FM];
  auto read_frags = [&](const char* st, int s, int buf) {
#pragma unroll
    for (int j = 0; j < FN; ++j) a[buf][j] = *reinterpret_cast<const bf16x8*>(st + (offQ[j] ^ (32u * s)));
#pragma unroll
    for (int i = 0; i < FM; ++i) bb[buf][i] = *reinterpret_cast<const bf16x8*>(st + (offP[i] ^ (32u * s)));
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[buf][j], bb[buf][i], acc[i][j], 0, 0, 0);
  };
  read_frags(smem, 0, 0);

  for (int kt = 0; kt < nk; ++kt) {
    const char* st = smem + (kt & 1) * STAGE;
    char* nx = smem + ((kt + 1) & 1) * STAGE;
    stage_store(nx);              // tile min(kt+1, nk-1)
    stage_advance(kt + 2 < nk);
    stage_load();                 // tile min(kt+2, nk-1)
#pragma unroll
    for (int s = 0; s < BK / 16 - 1; ++s) {
      read_frags(st, s + 1, (s + 1) & 1);
      mfmas(s & 1);
      // Interleave so every memory instruction issues between MFMAs: in
      // step 0 the staged tile's LDS writes and the next global loads, in
      // every step the fragment reads of the following step.
      constexpr int nm = FM * FN, nr = FM + FN, ns = kUnified ? BM / 32 : 0;
      if (s == 0 && kUnified) {
#pragma unroll
        for (int q = 0; q < nm; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // MFMA
          if (q < ns) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);       // DS write
          if (q < ns) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);       // global load
          if (q < nr) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);       // DS read
        }
      } else {
#pragma unroll
        for (int q = 0; q < nm; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (q < nr) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    }
    __syncthreads();
    read_frags(nx, 0, 0);         // next tile's step 0 (a harmless reread after the last)
    mfmas((BK / 16 - 1) & 1);
#pragma unroll
    for (int q = 0; q < FM * FN; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (q < FM + FN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  }
  __syncthreads();

  // ------------------------------------------------------------------ epilogue
  // lane holds row m = m0 + wm*WTM + i*32 + (lane&31) and, for register
  // group q (4 regs), columns n = n0 + wn*WTN + j*32 + 8q + 4*(lane>>5) + 0..3
  const int64_t nw = n0 + wn * WTN + 4 * (lane >> 5);

  if constexpr (EPI == EPI_LSE) {
    float2* red = reinterpret_cast<float2*>(smem);      // [4 wn][BM]
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int ml = wm * WTM + i * 32 + (lane & 31);
      const int64_t m = m0 + ml;
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[i][j][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      float s = 0.f;
      const float mxs = mx * kLog2e;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += __builtin_amdgcn_exp2f(acc[i][j][r] * kLog2e - mxs);
      s += __shfl_xor(s, 32, 64);
      if (lane < 32) red[wn * BM + ml] = make_float2(mx, s);
      // the target's logit, from whichever lane holds it
      const int t = g.tgt[m];
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (t == nw + j * 32 + 8 * (r >> 2) + (r & 3)) g.ztgt[m] = acc[i][j][r];
    }
    __syncthreads();
    if (tid < BM) {
      float2 p[WGN];
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < WGN; ++w) {
        p[w] = red[w * BM + tid];
        M = fmaxf(M, p[w].x);
      }
      float S = 0.f;
#pragma unroll
      for (int w = 0; w < WGN; ++w) S += p[w].y * __builtin_amdgcn_exp2f((p[w].x - M) * kLog2e);
      g.lse_part[(m0 + tid) * g.lse_stride + tn] = make_float2(M, S);
    }
    return;
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t m = m0 + wm * WTM + i * 32 + (lane & 31);
      float dz_l = 0.f, dz_s = 0.f;
      int dz_t = -1;
      int rope_t = 0;
      if constexpr (EPI == EPI_DZ) {
        dz_t = g.tgt[m];
        dz_l = g.lse[m] * kLog2e;
        dz_s = dz_t >= 0 ? *g.inv_nvalid : 0.f;
      }
      if constexpr (EPI == EPI_ROPE) rope_t = (int)(m % g.rope_T);
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t n = nw + j * 32 + 8 * q;
          float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          if constexpr (EPI == EPI_F32) {
            if (g.splits > 1) {
              float* dst = g.part + (int64_t)split * g.M * g.N + m * g.N + n;
              *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
              float* dst = (float*)g.C + m * g.ldc + n;
              float4 o = make_float4(v[0], v[1], v[2], v[3]);
              if (g.beta) {
                const float4 c = *reinterpret_cast<const float4*>(dst);
                o.x += c.x; o.y += c.y; o.z += c.z; o.w += c.w;
              }
              *reinterpret_cast<float4*>(dst) = o;
            }
            continue;
          }
          if constexpr (EPI == EPI_ROPE) {
            if (n < g.rope_cols) {
              const int pi = (int)(n % g.head_dim) >> 1;
              const float4 cs = *reinterpret_cast<const float4*>(g.rope + (int64_t)rope_t * (g.head_dim >> 1) + pi);
              const float x0 = v[0], x1 = v[1], x2 = v[2], x3 = v[3];
              v[0] = x0 * cs.x - x1 * cs.y;
              v[1] = x0 * cs.y + x1 * cs.x;
              v[2] = x2 * cs.z - x3 * cs.w;
              v[3] = x2 * cs.w + x3 * cs.z;
            }
          }
          if constexpr (EPI == EPI_RESID || EPI == EPI_DRELU2) {
            const uint2 a = *reinterpret_cast<const uint2*>((const bf16*)g.aux + m * g.ldaux + n);
            const float a0 = bf_lo(a.x), a1 = bf_hi(a.x), a2 = bf_lo(a.y), a3 = bf_hi(a.y);
            if constexpr (EPI == EPI_RESID) {
              v[0] += a0; v[1] += a1; v[2] += a2; v[3] += a3;
            } else {
              // aux = relu(h)^2, so 2 relu(h) = 2 sqrt(aux)
              v[0] *= 2.f * __builtin_sqrtf(fmaxf(a0, 0.f));
              v[1] *= 2.f * __builtin_sqrtf(fmaxf(a1, 0.f));
              v[2] *= 2.f * __builtin_sqrtf(fmaxf(a2, 0.f));
              v[3] *= 2.f * __builtin_sqrtf(fmaxf(a3, 0.f));
            }
          }
          if constexpr (EPI == EPI_RELU2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = fmaxf(v[e], 0.f) * fmaxf(v[e], 0.f);
          }
          if constexpr (EPI == EPI_DZ) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = (__builtin_amdgcn_exp2f(v[e] * kLog2e - dz_l) - ((n + e) == dz_t ? 1.f : 0.f)) * dz_s;
          }
          *reinterpret_cast<uint2*>((bf16*)g.C + m * g.ldc + n) = make_uint2(pack2(v[0], v[1]), pack2(v[2], v[3]));
        }
    }
  }
}

template <int NW, int BM, int BN, bool PT, bool QT, int EPI>
hipError_t launch(const GemmDesc& g, hipStream_t s) {
  dim3 grid((g.M / BM) * (g.N / BN) * g.splits);
  k_gemm_mfma<NW, BM, BN, PT, QT, EPI><<<grid, NW * 64, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace mfma
}  // namespace nc

// Operand-layout / epilogue combinations the library uses.
//   forward:  qkv (ROPE), o Wo^T + x and u W2^T + x (RESID),
//             u = relu(m W1^T)^2 (RELU2), head (LSE), head recompute (DZ)
//   backward: weight gradients (both operands transposed, fp32 partials),
//             activation gradients (Q transposed: STORE, DRELU2)
//   tests:    every layout with fp32 and bf16 stores
#define NC_MFMA_COMBOS(X)     \
  X(0, 0, EPI_STORE)          \
  X(0, 0, EPI_ROPE)           \
  X(0, 0, EPI_RESID)          \
  X(0, 0, EPI_RELU2)          \
  X(0, 0, EPI_LSE)            \
  X(0, 0, EPI_DZ)             \
  X(0, 0, EPI_F32)            \
  X(0, 1, EPI_STORE)          \
  X(0, 1, EPI_DRELU2)         \
  X(0, 1, EPI_F32)            \
  X(1, 0, EPI_STORE)          \
  X(1, 0, EPI_F32)            \
  X(1, 1, EPI_STORE)          \
  X(1, 1, EPI_F32)

namespace nc {
namespace mfma {
inline bool combo_supported(const GemmDesc& g) {
#define NC_X(PT, QT, EPI) \
  if (g.p_trans == PT && g.q_trans == QT && g.epi == EPI) return true;
  NC_MFMA_COMBOS(NC_X)
#undef NC_X
  return false;
}

template <int NW, int BM, int BN>
hipError_t dispatch(const GemmDesc& g, hipStream_t s) {
#define NC_X(PT, QT, EPI) \
  if (g.p_trans == PT && g.q_trans == QT && g.epi == EPI) return launch<NW, BM, BN, PT, QT, EPI>(g, s);
  NC_MFMA_COMBOS(NC_X)
#undef NC_X
  return hipErrorInvalidValue;
}

hipError_t gemm_256x256(const GemmDesc& g, hipStream_t s);
hipError_t gemm_256x128(const GemmDesc& g, hipStream_t s);
hipError_t gemm_128x128(const GemmDesc& g, hipStream_t s);
}  // namespace mfma
}  // namespace nc
