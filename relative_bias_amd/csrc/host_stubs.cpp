// Host-only stand-ins for the kernel launchers and the scratch lookup,
// linked into the sanitizer build of the C-ABI host layer
// (librpa_hostsan.so, built by relative_bias_amd/build_hostsan.py).  That
// build runs the argument checks, the split planner and the workspace
// arithmetic of rpa_api.cpp under AddressSanitizer and
// UndefinedBehaviorSanitizer on a machine without a GPU, where no call may
// reach a launch: every stand-in reports that no device is present.
#include "rpa_internal.h"

namespace rpa {

hipError_t launch_attention(const AttnParams &, int, int64_t, bool, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_combine(const CombineParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_slot_mapping(const SlotParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_kv_write(const KvWriteParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_kv_write_fp8(const KvWriteParams &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_balanced_decode(const AttnParams &, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t scratch_device_ptr(void **) { return hipErrorNoDevice; }

}  // namespace rpa
