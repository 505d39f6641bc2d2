// Kernel launchers for the host-only sanitizer build of pa_api.cpp: that
// build checks the host side of the C ABI (argument validation, workspace
// planning, metadata checks) under AddressSanitizer and UBSan on a machine
// without a GPU, so no kernel is compiled and every launch reports an error.
#include "pa_internal.h"

namespace pa {

hipError_t launch_kv_write(const KvWriteArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_decode(const DecodeArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prefill_f32(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prefill_bf16(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
