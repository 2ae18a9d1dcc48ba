// bf16 matrix-core GEMM for gfx950 (CDNA4), shared by the per-tile-size
// translation units.
//
//   C[m][n] = sum_k P[m][k] * Q[n][k]
//
// Block: 512 threads (8 waves, 2 along m x 4 along n), tile BM x BN x 64,
// fp32 accumulation in v_mfma_f32_32x32x16_bf16.  Q (the n side) is the
// instruction's A operand and P (the m side) its B operand, so a lane's
// sixteen accumulators hold one row m and runs of four consecutive columns
// n, so row-wise reductions (log-sum-exp) stay in a lane.  Other epilogues
// pass the accumulators through LDS and finish them in row order, so aux
// reads and output writes are contiguous runs of a row.
//
// An operand stored k-major ([rows][K]) lives in LDS as [row][64 k] bf16
// (128 B per row), the 16-byte chunk c of row r at chunk slot
// c ^ ((r >> 1) & 7) (see lds_off); a fragment is one ds_read_b128 per lane.
// An operand stored the other way ([K][rows], the weight gradients' token
// contractions) is copied unchanged, as [64 k][R rows] (2R bytes per k row,
// chunk c of k row k at slot c ^ 4 (k & 3)), and its fragments are read with
// gfx950's transposing LDS read (ds_read_b64_tr_b16): within each group of
// 16 lanes, lane i receives element i & 3 of the 8-byte pieces that lanes
// 4e + (i >> 2), e < 4, address -- so when those 16 lanes address four k
// rows x four 4-element column pieces, every lane gets four consecutive k
// of one row, which is the operand layout of the MFMA.  No layout needs
// VALU transposes.  Global loads and LDS writes are row segments of 16-byte
// chunks in either layout, and every fragment read and row write is free of
// bank conflicts.  Two LDS stages and one register stage: the global loads
// of k-tile t+2 are in flight while k-tile t is multiplied and k-tile t+1 is
// written; one barrier per k-tile.  The grid is persistent (one block per
// CU, each looping over output tiles).
#pragma once

#include <algorithm>
#include <type_traits>

#include "nc_internal.h"

namespace nc {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

typedef const u32x4 __attribute__((address_space(1)))* gptr;

// Per-thread plan for one operand tile (R rows x 64 k), loaded by 256
// threads into `reg` (R/32 x 16 B) and written to LDS.
//  k-major operand ([rows][K]): thread tl takes chunk tl & 7 of rows
//    (tl >> 3) + 32 i, i < R/32 -- 8 lanes read one 128-byte row segment.
//    Row r + 32 i has the swizzle of row r, so its LDS offset is that of
//    row r plus 4096 i.
//  [K][rows] operand: thread tl takes chunk tl % (R/8) of k rows
//    tl / (R/8) + (2048/R) i, i < R/32 -- R/8 lanes read one 2R-byte row;
//    the k rows of a thread agree mod 4, so their LDS offsets also step by
//    (2048/R) * 2R = 4096 bytes.
// Both layouts therefore load and store the same way; only the mapping
// set up here differs.  The state is layout-independent, so the two wave
// roles of a block share one set of registers.
struct Plan {
  gptr ptr;          // this thread's first 16-byte piece of the current tile
  int64_t step;      // elements between the thread's successive pieces
  int64_t kstep;     // elements to advance by one 64-k tile
  uint32_t lds0;     // byte offset of the first piece in the operand's LDS image

  template <int R, bool TRANS>
  __device__ inline void init(const bf16* base, int64_t ld, int64_t row0, int64_t k0, int tl) {
    if (!TRANS) {
      const int r = tl >> 3, c = tl & 7;
      ptr = (gptr)(base + (row0 + r) * ld + k0 + c * 8);
      step = 32 * ld;
      kstep = BK;
      lds0 = lds_off(r, c);
    } else {
      constexpr int CPR = R / 8;                 // 16-byte chunks per k row
      const int c = tl % CPR, kr = tl / CPR;
      ptr = (gptr)(base + (k0 + kr) * ld + row0 + c * 8);
      step = (int64_t)(256 / CPR) * ld;
      kstep = (int64_t)BK * ld;
      lds0 = (uint32_t)kr * (2u * R) + ((uint32_t)(c ^ (4 * (kr & 3))) << 4);
    }
  }
  template <int R>
  __device__ inline void load(u32x4 (&reg)[8]) const {
#pragma unroll
    for (int i = 0; i < R / 32; ++i) reg[i] = ptr[(i * step) >> 3];
  }
  template <int R>
  __device__ inline void store(const u32x4 (&reg)[8], char* lds_base) const {
#pragma unroll
    for (int i = 0; i < R / 32; ++i) *reinterpret_cast<u32x4*>(lds_base + lds0 + 4096u * i) = reg[i];
  }
  __device__ inline void advance_if(bool more) { ptr += more ? (kstep >> 3) : 0; }
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
// One MFMA operand fragment from a [64 k][R rows] image: the lane's byte
// offset `off` (k rows 16 s + 8 (l >> 5) + ((l & 15) >> 2), see frag_tr_off)
// gives k 0-3 of its row, the same offset plus 4 k rows gives k 4-7.
template <int R>
__device__ inline bf16x8 frag_tr(const char* p) {
  typedef __attribute__((address_space(3))) v4i16* lptr;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr)(p));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lptr)(p + 8 * R));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// Lane l's offset for the fragment of rows row0 .. row0+31 at k16 step 0 in a
// [64 k][R rows] image.  Lane groups of 16 (g = l >> 4) cover rows
// row0 + 16 (g & 1) .. +15 at k half g >> 1; in a group, lane j addresses
// k row (j >> 2) of the four and the 4-element piece j & 3 of the rows --
// k rows that agree mod 4 share the swizzle 4 (j >> 2).
template <int R>
__device__ inline uint32_t frag_tr_off(int row0, int l) {
  const int j = l & 15, g = l >> 4;
  const int k = 8 * (g >> 1) + (j >> 2);
  const int m = row0 + 16 * (g & 1) + 4 * (j & 3);
  return (uint32_t)k * (2u * R) + ((uint32_t)((m >> 3) ^ (4 * (j >> 2))) << 4) + 8u * ((m >> 2) & 1);
}

// One output tile of the persistent grid: split, n-tile, k-tiles, origin,
// and the element offsets of its batch item's operands and result.
struct GemmTile {
  int split, tm, tn, nk;     // a shifted last tile (RAG) stores from row tm * BM,
  int64_t m0, n0, kbeg;      // column tn * BN on (> m0 / n0); tm is set only there
  int64_t pofs, qofs, cofs, aofs;
};

// The coordinates are the same in every lane, but forming them takes
// divisions the compiler runs on the vector unit; moved to scalar registers
// explicitly, they stop occupying 18 VGPRs through the main loop.
__device__ inline int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ inline int64_t uni(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ inline GemmTile uniform(GemmTile c) {
  c.split = uni(c.split); c.tm = uni(c.tm); c.tn = uni(c.tn); c.nk = uni(c.nk);
  c.m0 = uni(c.m0); c.n0 = uni(c.n0); c.kbeg = uni(c.kbeg);
  c.pofs = uni(c.pofs); c.qofs = uni(c.qofs); c.cofs = uni(c.cofs); c.aofs = uni(c.aofs);
  return c;
}

// Logical tile -> (split, m-tile, n-tile).  Workgroups are dealt to the 8
// XCDs round-robin (and a full grid's G is a multiple of 8, so a block stays
// on one XCD), so block slots are renumbered to give each XCD a contiguous
// run of logical tiles (splits outermost, so an XCD works through few K
// ranges).  Within a split, tiles are rastered in groups of kGroupM m-tiles,
// m fastest: the ~32 blocks an XCD runs at once cover about 8 m-tiles x 4
// n-tiles, so each P panel and each Q panel (weights) is reused from that
// XCD's L2 instead of refetched per tile.  Split i covers the k-tiles
// [i nkt/splits, (i+1) nkt/splits).  Batch items are outermost of all.
// A dimension that is not a multiple of the tile (a multiple of 128, at
// least 2 tiles) ends in a tile shifted back to end at the matrix edge: it
// computes the outputs it shares with its neighbour again and stores only
// its own (from tm * BM / tn * BN on), so every output is written by one
// tile.
template <int BM, int BN>
struct TileMap {
  static constexpr int kGroupM = 8, kNarrow = 8;
  int ntn, ntm, ntiles, total, nkt, G, chunk, splits, sym;
  int64_t sP, sQ, sC, sAux;
  __device__ inline TileMap(const GemmDesc& g) {
    ntn = (g.N + BN - 1) / BN;
    ntm = (g.M + BM - 1) / BM;
    sym = g.sym;
    ntiles = sym ? ntm * (ntm + 1) / 2 : ntn * ntm;   // sym: the tiles with tn >= tm
    splits = g.splits;
    total = ntiles * splits * (g.batch > 1 ? g.batch : 1);
    sP = g.sP; sQ = g.sQ; sC = g.sC; sAux = g.sAux;
    nkt = g.K / BK;
    G = (int)gridDim.x;
    chunk = (total + 7) >> 3;
  }
  // block slot v (block b takes v = b, b + G, ...) -> logical tile, or -1
  // once the slot's XCD range [x*chunk, (x+1)*chunk) is exhausted
  __device__ inline int logical(int v) const {
    if (G & 7) return v < total ? v : -1;
    const int x = v & 7, j = v >> 3;
    const int L = x * chunk + j;
    return (j < chunk && L < total) ? L : -1;
  }
  template <bool RAG>
  __device__ inline GemmTile coords(int L, const GemmDesc& g) const {
    GemmTile c;
    const int outer = L / ntiles;
    const int b = outer / splits;
    c.split = outer - b * splits;
    c.pofs = b * sP; c.qofs = b * sQ; c.cofs = b * sC; c.aofs = b * sAux;
    const int t = L - outer * ntiles;
    if (sym) {
      // row tm of the upper triangle holds ntm - tm tiles
      int tm = 0, rem = t;
      while (rem >= ntm - tm) {
        rem -= ntm - tm;
        ++tm;
      }
      if constexpr (RAG) c.tm = tm;
      c.tn = tm + rem;
      c.m0 = (int64_t)tm * BM;
      c.n0 = (int64_t)c.tn * BN;
      c.nk = nkt;
      c.kbeg = 0;
      return c;
    }
    const int first_m = (t / (kGroupM * ntn)) * kGroupM;
    const int gm = min(kGroupM, ntm - first_m);
    const int tg = t - first_m * ntn;
    // narrow products (few n-tiles): n fastest, so the blocks an XCD runs
    // at once cover whole rows of tiles and each P panel is fetched once;
    // wide ones: m fastest, so each Q panel serves gm blocks
    const bool nfast = ntn <= kNarrow;
    c.tn = nfast ? tg % ntn : tg / gm;
    const int tmi = first_m + (nfast ? tg / ntn : tg % gm);
    if constexpr (RAG) {
      c.tm = tmi;
      c.m0 = (int64_t)min(tmi * BM, g.M - BM);
      c.n0 = (int64_t)min(c.tn * BN, g.N - BN);
    } else {
      c.m0 = (int64_t)tmi * BM;
      c.n0 = (int64_t)c.tn * BN;
    }
    const int kt0 = (int)((int64_t)c.split * nkt / splits);
    c.nk = (int)((int64_t)(c.split + 1) * nkt / splits) - kt0;
    c.kbeg = (int64_t)kt0 * BK;
    return c;
  }
};

// Finish and store four consecutive outputs (row m, columns n .. n+3) of a
// row-order epilogue: x holds the fp32 products; y, cs, dz_t, dz_l, dz_s
// are the row's prefetched inputs (aux pair, rotary factors, target, lse
// and the dz row factor).
template <int EPI>
__device__ inline void epi_store4(const GemmDesc& g, const GemmTile& c, int64_t m, int64_t n, float (&x)[4],
                                  uint2 y, float4 cs, bool rot, int dz_t, float dz_l, float dz_s) {
  if constexpr (EPI == EPI_F32) {
    if (g.splits > 1) {
      float* dst = g.part + (int64_t)c.split * g.M * g.N + m * g.N + n;
      *reinterpret_cast<float4*>(dst) = make_float4(x[0], x[1], x[2], x[3]);
    } else {
      float* dst = (float*)g.C + m * g.ldc + n;
      float4 o = make_float4(x[0], x[1], x[2], x[3]);
      if (g.beta) {
        const float4 q = *reinterpret_cast<const float4*>(dst);
        o.x += q.x; o.y += q.y; o.z += q.z; o.w += q.w;
      }
      *reinterpret_cast<float4*>(dst) = o;
    }
    return;
  }
  if constexpr (EPI == EPI_ROPE) {
    // (rot ? rotated : as is), without a branch
    const float c0 = rot ? cs.x : 1.f, s0 = rot ? cs.y : 0.f;
    const float c1 = rot ? cs.z : 1.f, s1 = rot ? cs.w : 0.f;
    const float x0 = x[0], x1 = x[1], x2 = x[2], x3 = x[3];
    x[0] = x0 * c0 - x1 * s0;
    x[1] = x0 * s0 + x1 * c0;
    x[2] = x2 * c1 - x3 * s1;
    x[3] = x2 * s1 + x3 * c1;
  }
  if constexpr (EPI == EPI_RESID || EPI == EPI_DRELU2 || EPI == EPI_AXPBY) {
    const float a0 = bf_lo(y.x), a1 = bf_hi(y.x), a2 = bf_lo(y.y), a3 = bf_hi(y.y);
    if constexpr (EPI == EPI_RESID) {
      x[0] += a0; x[1] += a1; x[2] += a2; x[3] += a3;
    } else if constexpr (EPI == EPI_AXPBY) {
      x[0] = g.ep_alpha * x[0] + g.ep_gamma * a0;
      x[1] = g.ep_alpha * x[1] + g.ep_gamma * a1;
      x[2] = g.ep_alpha * x[2] + g.ep_gamma * a2;
      x[3] = g.ep_alpha * x[3] + g.ep_gamma * a3;
    } else {
      // aux = relu(h)^2, so 2 relu(h) = 2 sqrt(aux)
      x[0] *= 2.f * __builtin_sqrtf(fmaxf(a0, 0.f));
      x[1] *= 2.f * __builtin_sqrtf(fmaxf(a1, 0.f));
      x[2] *= 2.f * __builtin_sqrtf(fmaxf(a2, 0.f));
      x[3] *= 2.f * __builtin_sqrtf(fmaxf(a3, 0.f));
    }
  }
  if constexpr (EPI == EPI_RELU2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = fmaxf(x[e], 0.f) * fmaxf(x[e], 0.f);
  }
  if constexpr (EPI == EPI_DZ) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      x[e] = (__builtin_amdgcn_exp2f(x[e] * kLog2e - dz_l) - ((n + e) == dz_t ? 1.f : 0.f)) * dz_s;
  }
  if constexpr (EPI == EPI_LSEZ) {
    // logits relative to the tile's row maximum (dz_l): entries with a
    // non-negligible probability sit close to it, where bf16 is finest
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] -= dz_l;
  }
  // Non-temporal stores keep the streamed-out product from displacing the
  // operand panels in the caches: on the 65,536 x 5,120 x 1,280 product,
  // 3 % with a plain epilogue and 1.6 % with an aux tile read beside the
  // store (warmed-up, interleaved repetitions).  The linear combination
  // keeps the plain store: its small outputs are the next product's
  // operands.
  u32x2 w;
  w.x = pack2(x[0], x[1]);
  w.y = pack2(x[2], x[3]);
  u32x2* dst = reinterpret_cast<u32x2*>((bf16*)g.C + c.cofs + m * g.ldc + n);
  if constexpr (EPI == EPI_AXPBY) *dst = w;
  else __builtin_nontemporal_store(w, dst);
}

// Per-row (max, sum exp) of a tile's logits from the WGN column groups
// (red [WGN][BM], written by the waves), combined by the first BM threads.
template <int WGN, int BM>
__device__ inline void lse_combine(const GemmDesc& g, const GemmTile& c, const float2* red, int etid,
                                   float* row_max) {
  if (etid < BM) {
    float2 p[WGN];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WGN; ++w) {
      p[w] = red[w * BM + etid];
      M = fmaxf(M, p[w].x);
    }
    float S = 0.f;
#pragma unroll
    for (int w = 0; w < WGN; ++w) S += p[w].y * __builtin_amdgcn_exp2f((p[w].x - M) * kLog2e);
    g.lse_part[(c.m0 + etid) * g.lse_stride + c.tn] = make_float2(M, S);
    if (row_max) row_max[etid] = M;
  }
}

// Waves in a 2 x 4 grid, wave tile (BM/2) x (BN/4); waves 0-3 stage P and
// waves 4-7 stage Q (two waves per SIMD).
//
// Persistent: the grid holds as many blocks as fit on the device at once and
// block b takes the logical tiles b, b + G, b + 2G, ... (G = grid size).
// While a tile's epilogue runs, the first k-tile of the block's next tile is
// already on its way into registers, so tile boundaries cost neither a
// block launch nor an exposed load latency.
//
// RAG: M or N is not a multiple of the tile; a separate instantiation, so
// the exact-fit kernels carry none of the shifted tile's bookkeeping.
template <int NW, int BM, int BN, bool PT, bool QT, int EPI, bool RAG>
__global__ void __launch_bounds__(NW * 64, 1) k_gemm_mfma(GemmDesc g) {
  static_assert(BM % 64 == 0 && BN % 128 == 0 && NW == 8, "tile");
  constexpr int WGN = NW / 2;                    // waves along n
  constexpr int WTM = BM / 2, WTN = BN / WGN;    // wave tile
  constexpr int FM = WTM / 32, FN = WTN / 32;    // 32x32 fragments per wave
  constexpr int STAGE = (BM + BN) * 128;         // bytes per LDS stage
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  __shared__ float zrow_max[EPI == EPI_LSEZ ? BM : 1];      // the tile's row maxima (EPI_LSEZ)

  const int tid = threadIdx.x;
  // the wave index as a scalar: wave-role branches are uniform
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  const TileMap<BM, BN> tm(g);
  typedef GemmTile Tile;

  // Waves 0-3 stage P tiles, waves 4-7 Q tiles (a wave-uniform split), with
  // one plan per thread.  Staging code depends only on the tile height, so
  // with BM = BN it is the same for both roles and the main loop has no
  // branch.
  constexpr bool kUnified = BM == BN;
  const bool loadsP = wave < 4;
  const int tl = tid & 255;
  Plan pl;
  const uint32_t my_lds = loadsP ? 0u : (uint32_t)BM * 128u;
  auto plan_init = [&](const Tile& c) {
    if (loadsP) pl.init<BM, PT>((const bf16*)g.P + c.pofs, g.ldp, c.m0, c.kbeg, tl);
    else pl.init<BN, QT>((const bf16*)g.Q + c.qofs, g.ldq, c.n0, c.kbeg, tl);
  };
  u32x4 reg[8];
  auto stage_load = [&]() {
    if constexpr (BM == BN) {
      pl.load<BM>(reg);
    } else {
      if (loadsP) pl.load<BM>(reg);
      else pl.load<BN>(reg);
    }
  };
  auto stage_store = [&](char* base) {
    if constexpr (BM == BN) {
      pl.store<BM>(reg, base + my_lds);
    } else {
      if (loadsP) pl.store<BM>(reg, base);
      else pl.store<BN>(reg, base + BM * 128);
    }
  };
  auto stage_advance = [&](bool more) { pl.advance_if(more); };

  const int frow = lane & 31, fchunk = lane >> 5;
  uint32_t offQ[FN], offP[FM];
#pragma unroll
  for (int j = 0; j < FN; ++j)
    offQ[j] = BM * 128 + (QT ? frag_tr_off<BN>(wn * WTN + j * 32, lane) : lds_off(wn * WTN + j * 32 + frow, fchunk));
#pragma unroll
  for (int i = 0; i < FM; ++i)
    offP[i] = PT ? frag_tr_off<BM>(wm * WTM + i * 32, lane) : lds_off(wm * WTM + i * 32 + frow, fchunk);
  // k-major image: chunk 2s + fchunk sits at slot (2s + fchunk) ^ f(row) =
  // (fchunk ^ f(row)) ^ 2s, so the k16 step s moves the byte offset by an
  // xor of 32*s; [64 k][R] image: step s is 16 k rows further, 32R bytes
  auto frag = [&](const char* st, uint32_t off, int s, auto trans, auto rows) -> bf16x8 {
    if constexpr (decltype(trans)::value) return frag_tr<decltype(rows)::value>(st + off + 32u * decltype(rows)::value * s);
    else return *reinterpret_cast<const bf16x8*>(st + (off ^ (32u * s)));
  };

  floatx16 acc[FM][FN];
  bf16x8 a[2][FN], bb[2][FM];
  auto read_frags = [&](const char* st, int s, int buf) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
      a[buf][j] = frag(st, offQ[j], s, std::integral_constant<bool, QT>{}, std::integral_constant<int, BN>{});
#pragma unroll
    for (int i = 0; i < FM; ++i)
      bb[buf][i] = frag(st, offP[i], s, std::integral_constant<bool, PT>{}, std::integral_constant<int, BM>{});
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[buf][j], bb[buf][i], acc[i][j], 0, 0, 0);
  };

  // Interleave so every memory instruction issues between MFMAs: in the
  // last step before the barrier the staged k-tile's LDS writes and the next
  // global loads, then the fragment reads of the following step; in the
  // other steps the fragment reads, spread evenly.
  // In the staging step the next step's fragment reads can go to the LDS
  // queue ahead of the k-tile's writes (kReadsFirst), so they are not
  // waited for behind the writes at the barrier: 1-4 % faster per product
  // family.  The rotary, log-sum-exp and dz epilogues keep the reads after
  // the writes: with their extra live state the other order spills.
  constexpr bool kReadsFirst = EPI == EPI_STORE || EPI == EPI_RESID || EPI == EPI_DRELU2 || EPI == EPI_RELU2 ||
                               (EPI == EPI_F32 && PT == QT);
  constexpr int kMfma = FM * FN;
  constexpr int kReads = FM * (PT ? 2 : 1) + FN * (QT ? 2 : 1);   // LDS read instructions per step
  constexpr int kStage = BM / 32;                                 // LDS writes / global loads per k-tile
  static_assert(kReads <= 3 * kMfma, "interleave");
  // reads placed after the q-th MFMA, kPer at a time: as early as possible
  // (the next step's operands have the longest to land), or, in a staging
  // step, after the LDS writes, as late as possible
  constexpr int kPer = (kReads + kMfma - 1) / kMfma;
  auto reads_early = [&](int q) { return std::min(kPer, std::max(0, kReads - kPer * q)); };
  auto reads_late = [&](int q) { return reads_early(kMfma - 1 - q); };
  auto interleave_reads = [&]() {
#pragma unroll
    for (int q = 0; q < kMfma; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      const int r = reads_early(q);
      if (r >= 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (r >= 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (r >= 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  int v = blockIdx.x;
  if (tm.logical(v) < 0) return;                 // no tile for this block (uniform)
  Tile cur = uniform(tm.template coords<RAG>(tm.logical(v), g));
  plan_init(cur);
  stage_load();                 // k-tile 0 of the first tile
  stage_store(smem);

  for (;;) {
    const int nk = cur.nk;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Pipeline (stage s of LDS holds k-tile t with s = t & 1):
    //   iteration t:  k16 steps 0-2 of k-tile t (fragments read one step
    //                 ahead), with, during step 2, k-tile t+1 (staged in
    //                 registers) written to stage (t+1)&1 and the global
    //                 loads of k-tile t+2 issued;
    //                 barrier;
    //                 read k-tile t+1's step-0 fragments, then step 3 of
    //                 k-tile t -- its MFMAs cover the first LDS reads after
    //                 the barrier.
    // The write of k-tile t+1 reuses the stage k-tile t-1 occupied; its
    // last reads were issued before the previous barrier, which waits for
    // them.  A k-tile's loads have a whole iteration to arrive, and the
    // first one's latency hides behind the previous tile's epilogue.
    // K-tiles past the last are never fetched: the staged index is clamped
    // to nk-1 (the pointer stops advancing), so the final iterations restage
    // the last k-tile into the idle stage instead of branching around it.
    stage_advance(nk > 1);
    stage_load();               // k-tile min(1, nk-1)
    __syncthreads();
    read_frags(smem, 0, 0);

    for (int kt = 0; kt < nk; ++kt) {
      const char* st = smem + (kt & 1) * STAGE;
      char* nx = smem + ((kt + 1) & 1) * STAGE;
#pragma unroll
      for (int s = 0; s < BK / 16 - 1; ++s) {
        if (s == BK / 16 - 2 && !kReadsFirst) {
          // before the next fragment reads, so the staging registers are
          // free again by the time those land
          stage_store(nx);      // k-tile min(kt+1, nk-1)
          stage_advance(kt + 2 < nk);
          stage_load();         // k-tile min(kt+2, nk-1)
        }
        read_frags(st, s + 1, (s + 1) & 1);
        if (s == BK / 16 - 2 && kReadsFirst) {
          stage_store(nx);
          stage_advance(kt + 2 < nk);
          stage_load();
        }
        mfmas(s & 1);
        // Interleave so every memory instruction issues between MFMAs: in
        // the last step before the barrier the staged k-tile's LDS writes
        // and the next global loads, then the fragment reads of the
        // following step; in the other steps the fragment reads.
        if (s == BK / 16 - 2 && kUnified) {
#pragma unroll
          for (int q = 0; q < kMfma; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // MFMA
            if constexpr (kReadsFirst) {
              const int r = reads_early(q);
              if (r >= 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
              if (r >= 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
              if (r >= 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if (q < kStage) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);   // DS write
            if (q < kStage) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load
            if constexpr (!kReadsFirst) {
              const int r = reads_late(q);
              if (r >= 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // DS read
              if (r >= 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
              if (r >= 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
          }
        } else {
          interleave_reads();
        }
      }
      __syncthreads();
      read_frags(nx, 0, 0);       // next k-tile's step 0 (a harmless reread after the last)
      mfmas((BK / 16 - 1) & 1);
      interleave_reads();
    }
    __syncthreads();

    // The block's next tile: its first k-tile's loads are issued once the
    // accumulators have gone to LDS, and overlap the rest of the epilogue.
    const int vn = v + tm.G;
    const int Ln = tm.logical(vn);
    const bool more = Ln >= 0;
    const Tile c = cur;
    auto prefetch_next = [&]() {
      if (more) {
        cur = uniform(tm.template coords<RAG>(Ln, g));
        plan_init(cur);
        stage_load();
      }
    };
    v = vn;
    // The thread index, opaque to the compiler once per tile: without this
    // the epilogue's per-thread addresses are hoisted out of the tile loop
    // and held (or spilled) through the main loop.
    int etid = tid;
    asm volatile("" : "+v"(etid));
    const int elane = etid & 63;

    // ---------------------------------------------------------------- epilogue
    // lane holds row m = m0 + wm*WTM + i*32 + (lane&31) and, for register
    // group q (4 regs), columns n = n0 + wn*WTN + j*32 + 8q + 4*(lane>>5) + 0..3
    if constexpr (EPI == EPI_LSE || EPI == EPI_LSEZ) {
      const int64_t nw = c.n0 + wn * WTN + 4 * (elane >> 5);
      float2* red = reinterpret_cast<float2*>(smem);      // [4 wn][BM]
      // the rows' targets, all requested before the reductions: their
      // latency is exposed once per tile and overlaps the exponentials
      int tg[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) tg[i] = g.tgt[c.m0 + wm * WTM + i * 32 + (elane & 31)];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int ml = wm * WTM + i * 32 + (elane & 31);
        const int64_t m = c.m0 + ml;
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
        if (elane < 32) red[wn * BM + ml] = make_float2(mx, s);
        // the target's logit, from whichever lane holds it
        const int t = tg[i];
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (t == nw + j * 32 + 8 * (r >> 2) + (r & 3)) g.ztgt[m] = acc[i][j][r];
      }
      __syncthreads();
      if constexpr (EPI == EPI_LSE) {
        prefetch_next();
        lse_combine<WGN, BM>(g, c, red, etid, nullptr);
      } else {
        // the logits themselves follow through the row-order store below,
        // once the maxima are in LDS and the partials read
        lse_combine<WGN, BM>(g, c, red, etid, zrow_max);
        __syncthreads();
      }
    }
    // Outputs staged in LDS as bf16 ([rows][BN], 512-byte rows of 32
    // 16-byte chunks, chunk ch of row r at slot ch ^ (r & 31)), then stored
    // in 16-byte row-contiguous pieces.  The whole tile goes through LDS at
    // once, written by all waves; the kept logits go in two halves (waves
    // with wm = h write half h), which measured faster for that epilogue
    // only.
    //  * plain, relu^2, kept logits: the op needs no input beyond the tile
    //    (the kept logits its row maxima, already in LDS), so it is applied
    //    to the accumulators where they are; one rounding of the same fp32
    //    value as a row-order pass would give.
    //  * residual, 2 sqrt(u), rotary: the product is rounded to bf16 as it
    //    is staged and the op is applied to that in the row-order pass,
    //    where its inputs (the aux row pieces, the rotary factors of the
    //    row's position) are contiguous: half the LDS traffic and one pass
    //    instead of two, for a second rounding of the result.  Their inputs
    //    are requested before the staging writes, so their latency overlaps
    //    the LDS round trip.
    constexpr bool kOpPass = EPI == EPI_RESID || EPI == EPI_DRELU2 || EPI == EPI_ROPE;
    constexpr bool kBf16Stage =
        (EPI == EPI_STORE || EPI == EPI_RELU2 || EPI == EPI_LSEZ || kOpPass) && BN == 256 && WTM == 128;
    if constexpr (kBf16Stage) {
      constexpr int NPASS = EPI == EPI_LSEZ ? 2 : 1;
      constexpr int RP = BM / NPASS;                   // rows per pass
      constexpr int CH = BN / 8;                       // 16-byte bf16 chunks per row
      constexpr int PER = RP * CH / (NW * 64);         // chunks per thread and pass
      constexpr int RSTEP = NW * 64 / CH;              // rows between a thread's chunks
      static_assert(RP * BN * 2 <= 2 * STAGE && (RP * CH) % (NW * 64) == 0 && RP % WTM == 0, "epilogue staging");
      static_assert(!kOpPass || NPASS == 1, "op pass");
      char* eb = smem;
      // a shifted last tile stores from row tm BM and column tn BN on (0 or
      // 128 past the tile's origin): whole row blocks and chunks drop out
      const int row_skip = RAG ? c.tm * BM - (int)c.m0 : 0;
      const int col_from = RAG ? c.tn * BN - (int)c.n0 : 0;
      // a thread's chunks share one column run (ch_t) and are RSTEP rows apart
      const int ch_t = etid % CH, r_t = etid / CH;
      // residual / 2 sqrt(u): the thread's aux pieces, all requested now
      u32x4 pa[kOpPass && EPI != EPI_ROPE ? PER : 1];
      if constexpr (EPI == EPI_RESID || EPI == EPI_DRELU2) {
        const bf16* ax = (const bf16*)g.aux + c.aofs + (c.m0 + r_t) * g.ldaux + c.n0 + ch_t * 8;
#pragma unroll
        for (int k = 0; k < PER; ++k) pa[k] = *reinterpret_cast<const u32x4*>(ax + (int64_t)k * RSTEP * g.ldaux);
      }
      // rotary: the (cos, sin) of the chunk's four pairs at each row's
      // position, requested WR rows ahead (the first WR now)
      constexpr int WR = EPI == EPI_ROPE ? 4 : 1;
      float4 pc[WR][2];
      const int n_t = (int)c.n0 + 8 * ch_t;
      const bool rot = EPI == EPI_ROPE && n_t < g.rope_cols;
      const float2* rp = nullptr;
      uint32_t t0 = 0;
      if constexpr (EPI == EPI_ROPE) {
        rp = g.rope + ((n_t % g.head_dim) >> 1);
        t0 = (uint32_t)((c.m0 + r_t) % g.rope_T);
      }
      auto fetch_rope = [&](int k) {
        if constexpr (EPI == EPI_ROPE) {
          if (rot) {
            const uint32_t t = (t0 + (uint32_t)(k * RSTEP)) % (uint32_t)g.rope_T;
            const float4* f = reinterpret_cast<const float4*>(rp + t * (uint32_t)(g.head_dim >> 1));
            pc[k % WR][0] = f[0];
            pc[k % WR][1] = f[1];
          }
        }
      };
#pragma unroll
      for (int k = 0; k < WR; ++k) fetch_rope(k);
#pragma unroll
      for (int h = 0; h < NPASS; ++h) {
        if (NPASS == 1 || wm == h) {
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const int r = (NPASS == 1 ? wm * WTM : 0) + i * 32 + (elane & 31);   // row within the pass
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int col = wn * WTN + j * 32 + 8 * q + 4 * (elane >> 5);
                float x[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                if constexpr (EPI == EPI_RELU2) {
#pragma unroll
                  for (int e = 0; e < 4; ++e) x[e] = fmaxf(x[e], 0.f) * fmaxf(x[e], 0.f);
                }
                if constexpr (EPI == EPI_LSEZ) {
                  // the kept logits, relative to the tile's row maximum
                  const float zm = zrow_max[h * RP + r];
#pragma unroll
                  for (int e = 0; e < 4; ++e) x[e] -= zm;
                }
                u32x2 w;
                w.x = pack2(x[0], x[1]);
                w.y = pack2(x[2], x[3]);
                *reinterpret_cast<u32x2*>(eb + r * 512 + (((col >> 3) ^ (r & 31)) << 4) + 8 * ((col >> 2) & 1)) = w;
              }
          }
        }
        __syncthreads();
        if (h == NPASS - 1) prefetch_next();
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          const int r = r_t + k * RSTEP;
          u32x4 v = *reinterpret_cast<const u32x4*>(eb + r * 512 + ((ch_t ^ (r & 31)) << 4));
          if constexpr (EPI == EPI_RESID || EPI == EPI_DRELU2) {
            const u32x4 y = pa[k];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float lo = bf_lo(v[e]), hi = bf_hi(v[e]);
              if constexpr (EPI == EPI_RESID) {
                lo += bf_lo(y[e]);
                hi += bf_hi(y[e]);
              } else {
                // aux = relu(h)^2, so 2 relu(h) = 2 sqrt(aux)
                lo *= 2.f * __builtin_sqrtf(fmaxf(bf_lo(y[e]), 0.f));
                hi *= 2.f * __builtin_sqrtf(fmaxf(bf_hi(y[e]), 0.f));
              }
              v[e] = pack2(lo, hi);
            }
          }
          if constexpr (EPI == EPI_ROPE) {
            if (rot) {
              const float4 f0 = pc[k % WR][0], f1 = pc[k % WR][1];
              const float cs[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float x0 = bf_lo(v[e]), x1 = bf_hi(v[e]);
                const float co = cs[2 * e], si = cs[2 * e + 1];
                v[e] = pack2(x0 * co - x1 * si, x0 * si + x1 * co);
              }
            }
            if (k + WR < PER) fetch_rope(k + WR);
          }
          if (!RAG || (h * RP + r >= row_skip && ch_t * 8 >= col_from)) {
            bf16* dst = (bf16*)g.C + c.cofs + (c.m0 + h * RP + r) * g.ldc + c.n0 + ch_t * 8;
            // the 2 sqrt(u) gradient keeps plain stores (its aux input
            // streams in beside the output; measured slower non-temporal)
            if constexpr (EPI == EPI_DRELU2) *reinterpret_cast<u32x4*>(dst) = v;
            else __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
          }
        }
        if (h + 1 < NPASS) __syncthreads();
      }
    }
    if constexpr (EPI != EPI_LSE && !kBf16Stage) {
      // Two passes, one per half of the tile's rows (the waves with wm = h
      // own rows h*WTM ..): those waves write their fp32 accumulators to
      // LDS as [WTM][BN] (16-byte chunk cc of row r at slot cc ^ (r & 15), so
      // the 16 rows of a write and the 16 chunks of a read are
      // conflict-free), then all threads read the half back a row segment
      // at a time and finish it -- aux reads and stores cover contiguous
      // runs of a row instead of 8 bytes in each of 32 rows.
      constexpr int CPR = BN / 4;                      // 16-byte fp32 chunks per row
      constexpr int RPS = NW * 64 / CPR;               // rows per sweep of the block
      static_assert(WTM * BN * 4 <= 2 * STAGE && CPR >= 16 && (NW * 64) % CPR == 0, "epilogue staging");
      float* ep = reinterpret_cast<float*>(smem);
      const int cc = etid % CPR, r0 = etid / CPR;
      const int64_t n = c.n0 + 4 * cc;
      constexpr int NR = WTM / RPS;                    // rows per thread and pass
      int pi = 0;
      if constexpr (EPI == EPI_ROPE) pi = (int)(n % g.head_dim) >> 1;
      const bool rot = EPI == EPI_ROPE && n < g.rope_cols;
      const bool tile_rot = EPI == EPI_ROPE && c.n0 < g.rope_cols;   // uniform over the block
      // a shifted last tile stores from row tm BM, column tn BN on: the
      // shift is 0 or 128 (dimensions are multiples of 128), so whole passes
      // (WTM = 128 rows) and whole column runs of a thread drop out
      const int row_skip = RAG ? c.tm * BM - (int)c.m0 : 0;
      const bool col_keep = !RAG || 4 * cc >= c.tn * BN - (int)c.n0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool keep = !RAG || (col_keep && h * WTM >= row_skip);
        // The pass's global inputs (aux rows, rotary factors, per-row loss
        // terms) are requested W rows ahead of their use, the first W
        // before the LDS round trip, which hides their latency.
        constexpr int W = (EPI == EPI_ROPE || EPI == EPI_DZ) ? (NR >= 16 ? NR / 4 : NR) : (NR >= 8 ? NR / 2 : NR);
        uint2 pa[W];
        float4 pc[W];
        int pt[W];
        float pl[W], ps[W];
        // rotary: position of the pass's first row in its sequence (rows
        // index tokens; the table is read for every column, in bounds, and
        // used where rot holds)
        uint32_t tpos = 0;
        if constexpr (EPI == EPI_ROPE) tpos = (uint32_t)((c.m0 + h * WTM + r0) % g.rope_T);
        auto fetch = [&](int k) {
          const int64_t m = c.m0 + h * WTM + r0 + k * RPS;
          if constexpr (EPI == EPI_RESID || EPI == EPI_DRELU2 || EPI == EPI_AXPBY)
            pa[k % W] = *reinterpret_cast<const uint2*>((const bf16*)g.aux + c.aofs + m * g.ldaux + n);
          if constexpr (EPI == EPI_ROPE) {
            // a tile with no rotated column (v) reads no rotary factors
            if (tile_rot) {
              const uint32_t t = (tpos + (uint32_t)(k * RPS)) % (uint32_t)g.rope_T;
              pc[k % W] = *reinterpret_cast<const float4*>(g.rope + t * (uint32_t)(g.head_dim >> 1) + pi);
            } else {
              pc[k % W] = make_float4(1.f, 0.f, 1.f, 0.f);
            }
          }
          if constexpr (EPI == EPI_DZ) {
            pt[k % W] = g.tgt[m];
            pl[k % W] = g.lse[m];
            ps[k % W] = g.row_scale[m];
          }
        };
#pragma unroll
        for (int k = 0; k < W; ++k) fetch(k);
        if (wm == h) {
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const int r = i * 32 + (elane & 31);
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int ch = (wn * WTN + j * 32 + 8 * q) / 4 + (elane >> 5);
                *reinterpret_cast<float4*>(ep + r * BN + ((ch ^ (r & 15)) << 2)) =
                    make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
              }
          }
        }
        __syncthreads();
        if (h == 1) prefetch_next();
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          const int r = r0 + k * RPS;
          const int64_t m = c.m0 + h * WTM + r;
          const float4 f = *reinterpret_cast<const float4*>(ep + r * BN + ((cc ^ (r & 15)) << 2));
          float x[4] = {f.x, f.y, f.z, f.w};
          const uint2 y = pa[k % W];
          const float4 cs = pc[k % W];
          int dz_t = 0;
          float dz_l = 0.f, dz_s = 0.f;
          if constexpr (EPI == EPI_DZ) {
            dz_t = pt[k % W];
            dz_l = pl[k % W] * kLog2e;
            dz_s = ps[k % W];
          }
          if constexpr (EPI == EPI_LSEZ) dz_l = zrow_max[h * WTM + r];
          if (k + W < NR) fetch(k + W);
          if (keep) epi_store4<EPI>(g, c, m, n, x, y, cs, rot, dz_t, dz_l, dz_s);
        }
        if (h == 0) __syncthreads();
      }
    }
    if (!more) break;
    __syncthreads();            // epilogue LDS traffic done before k-tile 0 is written
    // The next tile's k-tile 0, staged here rather than at the top of the
    // loop: its loads were issued before the epilogue's stores, and in
    // straight-line code the wait for them leaves those stores in flight
    // (at the loop head, merged with the first tile's path, it would wait
    // for the stores as well).
    stage_store(smem);
  }
}

// Blocks of a kernel that fit on the device at once, times the device's CU
// count, rounded up to a multiple of 8 (one share per XCD); cached per
// instantiation (`cached`) and device.
template <typename Kernel>
int resident_blocks(Kernel kern, int threads, int (&cached)[16]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = 0;
  if (!cached[dev]) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0) != hipSuccess || per_cu < 1)
      per_cu = 1;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
    cached[dev] = ((per_cu * cus) + 7) / 8 * 8;
  }
  return cached[dev];
}

template <int NW, int BM, int BN, bool PT, bool QT, int EPI, bool RAG>
hipError_t launch(const GemmDesc& g, hipStream_t s) {
  static int cached[16] = {0};
  const int ntiles = g.sym ? (g.M / BM) * (g.M / BM + 1) / 2 : ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
  const int total = ntiles * g.splits * (g.batch > 1 ? g.batch : 1);
  dim3 grid(std::min(total, resident_blocks(k_gemm_mfma<NW, BM, BN, PT, QT, EPI, RAG>, NW * 64, cached)));
  k_gemm_mfma<NW, BM, BN, PT, QT, EPI, RAG><<<grid, NW * 64, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace mfma
}  // namespace nc

// Operand-layout / epilogue combinations the library uses.
//   forward:  qkv (ROPE), o Wo^T + x and u W2^T + x (RESID),
//             u = relu(m W1^T)^2 (RELU2), head (LSE), head recompute (DZ)
//   backward: weight gradients (both operands transposed, fp32 partials),
//             activation gradients against transposed weight images
//             (both k-major: STORE, DRELU2)
//   tests:    every layout with fp32 and bf16 stores
// Combinations that also run with M or N a multiple of 128 but not of a
// 256 tile (a shifted last tile): the products of a model whose widths are
// odd multiples of 128 -- qkv + rotary, the residual products, activation
// gradients and weight gradients.
#define NC_MFMA_RAGGED_COMBOS(X) \
  X(0, 0, EPI_STORE)             \
  X(0, 0, EPI_ROPE)              \
  X(0, 0, EPI_RESID)             \
  X(1, 1, EPI_F32)

#define NC_MFMA_COMBOS(X)     \
  X(0, 0, EPI_STORE)          \
  X(0, 0, EPI_ROPE)           \
  X(0, 0, EPI_RESID)          \
  X(0, 0, EPI_RELU2)          \
  X(0, 0, EPI_DRELU2)         \
  X(0, 0, EPI_LSE)            \
  X(0, 0, EPI_LSEZ)           \
  X(0, 0, EPI_DZ)             \
  X(0, 0, EPI_F32)            \
  X(0, 0, EPI_AXPBY)          \
  X(0, 1, EPI_STORE)          \
  X(0, 1, EPI_AXPBY)          \
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

inline bool ragged_combo(const GemmDesc& g) {
#define NC_X(PT, QT, EPI) \
  if (g.p_trans == PT && g.q_trans == QT && g.epi == EPI) return true;
  NC_MFMA_RAGGED_COMBOS(NC_X)
#undef NC_X
  return false;
}

template <int NW, int BM, int BN>
hipError_t dispatch(const GemmDesc& g, hipStream_t s) {
  if (g.M % BM || g.N % BN) {
    if constexpr (BM == 256) {
      if (g.sym || g.M < BM || g.N < BN) return hipErrorInvalidValue;
#define NC_X(PT, QT, EPI) \
  if (g.p_trans == PT && g.q_trans == QT && g.epi == EPI) return launch<NW, BM, BN, PT, QT, EPI, true>(g, s);
      NC_MFMA_RAGGED_COMBOS(NC_X)
#undef NC_X
    }
    return hipErrorInvalidValue;
  }
#define NC_X(PT, QT, EPI) \
  if (g.p_trans == PT && g.q_trans == QT && g.epi == EPI) return launch<NW, BM, BN, PT, QT, EPI, false>(g, s);
  NC_MFMA_COMBOS(NC_X)
#undef NC_X
  return hipErrorInvalidValue;
}

hipError_t gemm_256x256(const GemmDesc& g, hipStream_t s);
hipError_t gemm_256x128(const GemmDesc& g, hipStream_t s);
hipError_t gemm_128x128(const GemmDesc& g, hipStream_t s);
}  // namespace mfma
}  // namespace nc
