// Host-only stand-ins for the GPU side of libattn: with these, the C ABI's
// host code (argument checks, plans, error reporting) builds and runs under
// AddressSanitizer and UndefinedBehaviorSanitizer on a machine without a GPU.
// Every launcher accepts its arguments and launches nothing; the three HIP
// runtime calls the host code makes are answered here too, so the HIP
// runtime library is not loaded.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace attn {
int g_launches = 0;
hipError_t launch_fwd_prefill(const FwdArgs&, Elt, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_fwd_row(const FwdArgs&, Elt, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_fwd_f32(const FwdArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode(const DecodeArgs&, Elt, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_qkv_proj(const QkvArgs&, Elt, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_masked_softmax(const SoftmaxArgs&, Elt, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_sinusoidal_pe(float*, int, int, int, hipEvent_t, hipEvent_t, hipStream_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t decode_scratch(void** ptr) {
    *ptr = reinterpret_cast<void*>(0x7e0000000000ull);   // a device address stand-in, never dereferenced
    return hipSuccess;
}
}  // namespace attn

extern "C" {
const char* hipGetErrorString(hipError_t) { return "host stand-in"; }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) { return hipErrorInvalidValue; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
}
