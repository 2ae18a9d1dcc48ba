// bf16 MFMA flash attention for gfx950 (placeholder: routes to the portable kernels).
#include "nc_internal.h"

namespace nc {
hipError_t attn_fwd_mfma(const AttnDesc& a, hipStream_t s) { return attn_fwd_portable<bf16>(a, s); }
hipError_t attn_bwd_mfma(const AttnDesc& a, hipStream_t s) { return attn_bwd_portable<bf16>(a, s); }
}  // namespace nc
