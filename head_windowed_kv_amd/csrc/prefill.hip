// Chunked-prefill windowed causal attention (placeholder until the MFMA
// kernel lands): reports UNSUPPORTED for every configuration.
#include <hip/hip_runtime.h>

#include "hwkv_internal.h"

namespace hwkv {

bool prefill_supported(hwkv_dtype, int, int) { return false; }

hwkv_status launch_prefill(const hwkv_layout&, int, const PrefillArgs&, hipStream_t) {
    return fail(HWKV_ERR_UNSUPPORTED, "prefill kernel not built");
}

}  // namespace hwkv
