// Chunked-prefill attention (placeholder until the matrix-core kernel lands).
#include "kivi_device.h"
#include "kivi_internal.h"

namespace kivi {

int launch_prefill(const CacheView&, int, int, const void*, const int32_t*, int, const int32_t*,
                   const int32_t*, int, const int32_t*, int, float, int, void*, void*) {
    return (int)hipErrorNotSupported;
}

}  // namespace kivi
