// bf16 MFMA GEMM instantiations for 128 x 128 tiles.
#include "gemm_mfma.h"

namespace nc {
namespace mfma {
hipError_t gemm_128x128(const GemmDesc& g, hipStream_t s) { return dispatch<8, 128, 128>(g, s); }
}  // namespace mfma
}  // namespace nc
