// read_stream.hip -- the bench's read-only HBM reference (libattn_probe.so).
//
// Not part of the attention path: bench.py times it on the box that runs the
// decode, over as many bytes as one decode call reads, so the decode rate can
// be read against what a plain read achieves on that same machine (the timing
// practice of the depthwise-convolution page, section 4.1; coalesced 16-byte
// loads: "CUDA first principles" page, section 3.2).
//
// The grid sweeps the buffer in passes: thread t of the grid reads 16-byte
// chunk t + k*threads (k = 0..15) of each pass, all 16 loads in flight
// together, non-temporal like the decode's own K/V loads. Each thread folds
// what it read into one word and stores it, so no load is dead.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kInFlight = 16;
constexpr int kThreads = 512;
constexpr int kGrid = 256;   // one workgroup per CU
constexpr int kNonTemporal = 2;

__global__ __launch_bounds__(kThreads) void read_stream_kernel(const u32x4_t* __restrict__ p, long long n16,
                                                               unsigned* __restrict__ out) {
    // offsets stay below 2^31 bytes (checked on the host); loads past n16 are
    // clamped to chunk 0, which exists
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, 0x7fffffff, 0x00020000);
    const long long nt = (long long)gridDim.x * blockDim.x;
    const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    unsigned x = 0;
    for (long long base = 0; base < n16; base += nt * kInFlight) {
        u32x4_t v[kInFlight];
#pragma unroll
        for (int k = 0; k < kInFlight; ++k) {
            const long long i = base + gid + k * nt;
            v[k] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)((i < n16 ? i : 0) * 16), 0, kNonTemporal);
        }
        __builtin_amdgcn_sched_barrier(0);   // all loads of the pass issued before the first use
#pragma unroll
        for (int k = 0; k < kInFlight; ++k) {
            const unsigned a = v[k][0], b = v[k][3];   // scalar copies of vector elements
            x ^= a ^ b;
        }
    }
    out[gid] = x;
}

}  // namespace

// Reads `bytes` (a multiple of 16, below 2 GiB) at device pointer p, 16-byte
// aligned; out: device uint32[256 * 512]. ev_start / ev_stop (either may be
// NULL) are recorded on the kernel itself. Returns the hipError_t value.
extern "C" int attn_probe_read_stream(const void* p, long long bytes, unsigned* out, void* stream, void* ev_start,
                                      void* ev_stop) {
    if (!p || !out || bytes <= 0 || (bytes & 15) || bytes > 0x7fffffffLL || (reinterpret_cast<uintptr_t>(p) & 15))
        return (int)hipErrorInvalidValue;
    hipExtLaunchKernelGGL(read_stream_kernel, dim3(kGrid), dim3(kThreads), 0, (hipStream_t)stream,
                          (hipEvent_t)ev_start, (hipEvent_t)ev_stop, 0, (const u32x4_t*)p, bytes / 16, out);
    return (int)hipGetLastError();
}
