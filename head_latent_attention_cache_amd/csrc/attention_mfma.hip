// Latent attention on bf16 MFMA (placeholder until the tiled kernel lands).
#include "launch.hpp"

namespace mla {
bool attn_mfma_supported(const Dims&) { return false; }
size_t attn_mfma_workspace(const Dims&, const Geo&, int, int) { return 0; }
hipError_t launch_attn_mfma(const AttnArgs&, void*, size_t, hipStream_t) { return hipErrorNotSupported; }
}  // namespace mla
