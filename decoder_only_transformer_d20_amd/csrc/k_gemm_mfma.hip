// bf16 MFMA GEMM: shape checks and tile selection (kernels in gemm_mfma.h).
#include "gemm_mfma.h"

namespace nc {

namespace {
// Products that may end in a tile shifted back to the matrix edge (the
// layouts and epilogues listed in NC_MFMA_RAGGED_COMBOS): each output is
// finished on its own, so the shifted tile recomputes the outputs it shares
// with its neighbour and does not store them.
bool ragged_ok(const GemmDesc& g) { return !g.sym && mfma::ragged_combo(g); }
// 256 along a dimension that is a multiple of 256 or, for those products,
// at least 1024 and a multiple of 128: the last tile then overlaps by 128,
// at most 1/8 of that dimension's work recomputed, which costs less than
// the narrower tiles' lower matrix-core rate.
int pick_tile(int D, bool ragged) { return (D % 256 == 0 || (ragged && D >= 1024)) ? 256 : 128; }
}  // namespace

int gemm_mfma_tile_m(const GemmDesc& g) { return pick_tile(g.M, ragged_ok(g)); }
int gemm_mfma_tile_n(const GemmDesc& g) {
  // a 256-row tile pairs with 256 or 128 columns; 128-row tiles with 128
  if (gemm_mfma_tile_m(g) != 256) return 128;
  return pick_tile(g.N, ragged_ok(g));
}

bool gemm_mfma_supported(const GemmDesc& g) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0 || g.M % 128 || g.N % 128 || g.splits < 1) return false;
  if (g.K % mfma::BK || g.splits > g.K / mfma::BK) return false;
  if (g.splits > 1 && g.epi != EPI_F32) return false;
  if (g.batch > 1 && (g.splits != 1 || (g.epi != EPI_STORE && g.epi != EPI_AXPBY))) return false;
  if ((int64_t)(g.M / 128) * (g.N / 128) * g.splits * (g.batch > 1 ? g.batch : 1) > (1 << 30)) return false;
  if (g.sym && (g.M != g.N || gemm_mfma_tile_m(g) != gemm_mfma_tile_n(g) || g.splits != 1 ||
                g.batch > 65535 ||
                (g.epi != EPI_STORE && g.epi != EPI_AXPBY)))
    return false;
  if (g.epi == EPI_ROPE && (g.head_dim % 4 || g.rope_cols % 4)) return false;
  // 16-byte output stores (the bf16 stores of the plain and relu^2 outputs)
  if (g.epi != EPI_F32 && g.epi != EPI_LSE && (g.ldc % 8 || (uintptr_t)g.C % 16)) return false;
  // 16-byte reads of the residual / relu(h)^2 rows and of the rotary factors
  if ((g.epi == EPI_RESID || g.epi == EPI_DRELU2) && (g.ldaux % 8 || (uintptr_t)g.aux % 16)) return false;
  if (g.epi == EPI_ROPE && (uintptr_t)g.rope % 16) return false;
  return mfma::combo_supported(g);
}

namespace {
// C[i][j] = C[j][i] wherever the tile row of i lies below the tile row of j
// (tiles of `tile` rows): the lower tiles of a symmetric product whose upper
// tiles were computed.  A workgroup moves one 64 x 64 block through LDS:
// 16-byte row pieces in and out (8 per row, two per thread), the transpose
// done in LDS.  Only the nlow strictly-lower blocks of an item are
// launched: blockIdx.x enumerates them row by row.
__global__ void __launch_bounds__(256) k_mirror_lower(unsigned short* C, int n, int64_t ldc, int64_t sC, int tile) {
  __shared__ unsigned short blk[64][64 + 2];
  const int per = tile / 64;                          // 64-blocks per tile side
  int bi = per, rem = blockIdx.x;                     // rows of blocks below the first tile row
  while (rem >= (bi / per) * per) {                   // block row bi holds (tile row of bi) * per lower blocks
    rem -= (bi / per) * per;
    ++bi;
  }
  const int bj = rem;
  unsigned short* c = C + (int64_t)blockIdx.y * sC;
  const int t = threadIdx.x;
  // source block (rows bj, columns bi): row r, 16-byte piece q
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = (t >> 3) + 32 * h, q = t & 7;
    const uint4 v = *reinterpret_cast<const uint4*>(c + (int64_t)(bj * 64 + r) * ldc + bi * 64 + 8 * q);
    const unsigned short* e = reinterpret_cast<const unsigned short*>(&v);
#pragma unroll
    for (int k = 0; k < 8; ++k) blk[r][8 * q + k] = e[k];
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = (t >> 3) + 32 * h, q = t & 7;      // destination row r = source column
    uint4 v;
    unsigned short* e = reinterpret_cast<unsigned short*>(&v);
#pragma unroll
    for (int k = 0; k < 8; ++k) e[k] = blk[8 * q + k][r];
    *reinterpret_cast<uint4*>(c + (int64_t)(bi * 64 + r) * ldc + bj * 64 + 8 * q) = v;
  }
}
}  // namespace

hipError_t gemm_mfma_bf16_product(const GemmDesc& g, hipStream_t s) {
  if (!gemm_mfma_supported(g)) return hipErrorInvalidValue;
  const int bm = gemm_mfma_tile_m(g), bn = gemm_mfma_tile_n(g);
  hipError_t e;
  if (bm == 256 && bn == 256) e = mfma::gemm_256x256(g, s);
  else if (bm == 256) e = mfma::gemm_256x128(g, s);
  else e = mfma::gemm_128x128(g, s);
  if (e != hipSuccess || !g.sym) return e;
  // strictly-lower 64-blocks of one item: tile rows 1 .. T-1, row tr holding
  // tr * per blocks in each of its per block rows
  const int per = bm / 64, T = g.M / bm;
  const int nlow = per * per * T * (T - 1) / 2;
  if (nlow == 0) return hipSuccess;
  if (g.ldc % 8 || g.sC % 8) return hipErrorInvalidValue;
  k_mirror_lower<<<dim3(nlow, g.batch > 1 ? g.batch : 1), 256, 0, s>>>((unsigned short*)g.C, g.M, g.ldc, g.sC, bm);
  return hipGetLastError();
}


hipError_t gemm_mfma_bf16(const GemmDesc& g, hipStream_t s) {
  hipError_t e = gemm_mfma_bf16_product(g, s);
  if (e == hipSuccess && g.epi == EPI_F32 && g.splits > 1) {
    if (g.ldc != g.N) return hipErrorInvalidValue;
    e = splitk_reduce(g.part, g.splits, (int64_t)g.M * g.N, (float*)g.C, g.beta, s);
  }
  return e;
}

namespace {
// Matrix-core throughput probe: every wave issues `iters` iterations of eight
// independent v_mfma_f32_32x32x16_bf16 on register operands -- no memory
// traffic, no dependence between the iterations' products beyond each
// accumulator's own chain -- so the rate it reaches is what the matrix
// cores sustain at the clock the chip holds under that load.  Each thread
// writes the sum of its accumulators to sink, which keeps the work live.
__global__ void __launch_bounds__(256) k_mfma_loop(int64_t iters, float* sink) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float floatx16 __attribute__((ext_vector_type(16)));
  const int tid = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)((float)((tid + e) & 31) * 0.001f);
    b[e] = (__bf16)((float)((tid ^ e) & 31) * 0.001f);
  }
  floatx16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = floatx16{};
  for (int64_t i = 0; i < iters; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  sink[(int64_t)blockIdx.x * 256 + tid] = s;
}
}  // namespace

hipError_t mfma_loop(int64_t iters, int blocks, float* sink, hipStream_t s) {
  k_mfma_loop<<<blocks, 256, 0, s>>>(iters, sink);
  return hipGetLastError();
}

}  // namespace nc
