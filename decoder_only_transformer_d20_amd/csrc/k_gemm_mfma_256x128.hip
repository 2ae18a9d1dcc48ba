// bf16 MFMA GEMM instantiations for 256 x 128 tiles.
#include "gemm_mfma.h"

namespace nc {
namespace mfma {
hipError_t gemm_256x128(const GemmDesc& g, hipStream_t s) { return dispatch<8, 256, 128>(g, s); }
}  // namespace mfma
}  // namespace nc
