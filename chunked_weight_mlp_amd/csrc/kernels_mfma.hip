// MFMA kernels (gfx950): placeholder until the bf16 MFMA path lands; every
// bf16 layer runs on the generic kernels meanwhile.
#include "internal.h"

namespace ipttt {

bool mfma_supported(int, int) { return false; }
hipError_t mf_gateup(const Slab &, const __bf16 *, const Weights &, const WsPtrs &, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t mf_proj(const Slab &, const Weights &, const WsPtrs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t mf_update_scan(const Slab &, const WsPtrs &, float *, hipStream_t) { return hipErrorNotSupported; }
hipError_t mf_update_one(const Slab &, int, const WsPtrs &, float *, hipStream_t) { return hipErrorNotSupported; }
hipError_t mf_apply(const Slab &, int, int, const WsPtrs &, float *, hipStream_t) { return hipErrorNotSupported; }

}  // namespace ipttt
