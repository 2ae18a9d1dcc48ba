// bf16 MFMA GEMM: shape checks and tile selection (kernels in gemm_mfma.h).
#include "gemm_mfma.h"

namespace nc {

int gemm_mfma_tile_m(int M, int /*N*/) { return M % 256 == 0 ? 256 : 128; }
int gemm_mfma_tile_n(int M, int N) {
  // a 256-row tile pairs with 256 or 128 columns; 128-row tiles with 128
  if (M % 256 != 0) return 128;
  return N % 256 == 0 ? 256 : 128;
}

bool gemm_mfma_supported(const GemmDesc& g) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0 || g.M % 128 || g.N % 128 || g.splits < 1) return false;
  if (g.K % mfma::BK || g.splits > g.K / mfma::BK) return false;
  if (g.splits > 1 && g.epi != EPI_F32) return false;
  if (g.epi == EPI_ROPE && (g.head_dim % 4 || g.rope_cols % 4)) return false;
  return mfma::combo_supported(g);
}

hipError_t gemm_mfma_bf16_product(const GemmDesc& g, hipStream_t s) {
  if (!gemm_mfma_supported(g)) return hipErrorInvalidValue;
  const int bm = gemm_mfma_tile_m(g.M, g.N), bn = gemm_mfma_tile_n(g.M, g.N);
  if (bm == 256 && bn == 256) return mfma::gemm_256x256(g, s);
  if (bm == 256) return mfma::gemm_256x128(g, s);
  return mfma::gemm_128x128(g, s);
}

hipError_t gemm_mfma_bf16(const GemmDesc& g, hipStream_t s) {
  hipError_t e = gemm_mfma_bf16_product(g, s);
  if (e == hipSuccess && g.epi == EPI_F32 && g.splits > 1) {
    if (g.ldc != g.N) return hipErrorInvalidValue;
    e = splitk_reduce(g.part, g.splits, (int64_t)g.M * g.N, (float*)g.C, g.beta, s);
  }
  return e;
}

}  // namespace nc
