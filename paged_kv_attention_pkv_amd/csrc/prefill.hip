// prefill.hip -- causal paged prefill (bf16, MFMA).  Not built yet: the entry
// point reports "unsupported" until the kernel lands.
#include "internal.hpp"

namespace pkv {

size_t prefill_workspace(const PoolGeom &, int, int, int, int, int) { return 0; }

hipError_t launch_prefill(const PoolGeom &, const PrefillArgs &, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace pkv
