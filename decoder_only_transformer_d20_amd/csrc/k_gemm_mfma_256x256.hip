// bf16 MFMA GEMM instantiations for 256 x 256 tiles.
#include "gemm_mfma.h"

namespace nc {
namespace mfma {
hipError_t gemm_256x256(const GemmDesc& g, hipStream_t s) { return dispatch<8, 256, 256>(g, s); }
}  // namespace mfma
}  // namespace nc
