// Host-only stand-ins for the kernel launchers of the library, so that the
// host half (layout.cpp, api.cpp) can be built with g++ and the address and
// undefined-behaviour sanitizers.  Every launcher only counts its calls;
// nothing touches device memory.
#include "hwkv_internal.h"

namespace hwkv {

int g_launches = 0;

// a fake, suitably aligned device address for the static scratch
hwkv_status static_scratch(hipStream_t, void** ptr) {
    *ptr = reinterpret_cast<void*>(uintptr_t(7) << 30);
    return HWKV_OK;
}

bool append_supported(const hwkv_layout&) { return true; }
bool decode_supported(const hwkv_layout&, int) { return true; }
bool prefill_supported(const hwkv_layout&, int) { return true; }

hwkv_status launch_append(const hwkv_layout&, const AppendArgs&, hipStream_t) {
    g_launches++;
    return HWKV_OK;
}
hwkv_status launch_decode_split(const hwkv_layout&, int, const DecodeSplitArgs&, hipStream_t) {
    g_launches++;
    return HWKV_OK;
}
hwkv_status launch_decode_merge(const hwkv_layout&, int, const DecodeMergeArgs&, hipStream_t) {
    g_launches++;
    return HWKV_OK;
}
hwkv_status launch_prefill(const hwkv_layout&, int, const PrefillArgs&, hipStream_t) {
    g_launches++;
    return HWKV_OK;
}
hwkv_status launch_decode_step(const hwkv_layout&, int, const DecodeSplitArgs&, hipStream_t) {
    g_launches++;
    return HWKV_OK;
}
hwkv_status launch_decode_split_append(const hwkv_layout&, int, const DecodeSplitArgs&,
                                       hipStream_t) {
    g_launches++;
    return HWKV_OK;
}

}  // namespace hwkv
