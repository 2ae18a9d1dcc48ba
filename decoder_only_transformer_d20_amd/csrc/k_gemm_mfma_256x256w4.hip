// bf16 MFMA GEMM instantiations for 256 x 256 tiles, 4 waves of 128 x 128.
#include "gemm_mfma.h"

namespace nc {
namespace mfma {
hipError_t gemm_256x256_w4(const GemmDesc& g, hipStream_t s) { return dispatch<4, 256, 256>(g, s); }
}  // namespace mfma
}  // namespace nc
