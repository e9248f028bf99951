// pe.hip -- sinusoidal position encoding table.
//
// pe[s][2i] = sin(pos * w_i), pe[s][2i+1] = cos(pos * w_i), pos = pos0 + s,
// w_i = 10000^(-2i/d_model) ("Week-4 CUDA notes" page, section 2.3).
//
// The page computes the table in fp32, with the frequencies precomputed
// once and each element one multiply and one sin or cos. Here a workgroup
// covers kPeRows positions and kPeThreads frequency pairs (a 2-D grid, so
// the chip holds many waves to hide the fp64 and sincos latency): each
// thread takes one pair i, computes w_i once (fp64) and reuses it for those
// rows; the angle pos * w_i is formed
// and reduced modulo 2*pi in fp64 (Cody and Waite's two-part constant), so
// that fp32 sin/cos of the reduced angle stay accurate to a few ulp at any
// position (an fp32 product pos * w_i alone would lose about 2^-24 * pos
// radians). Each (sin, cos) pair is one 8-byte store; a wave writes 512
// contiguous bytes of a row.
#include <hip/hip_runtime.h>

#include "../launch.h"
#include "../plan.h"

namespace attn {
namespace {

constexpr double kTwoPiHi = 6.283185307179586;          // 2*pi rounded to double
constexpr double kTwoPiLo = 2.4492935982947064e-16;     // 2*pi - kTwoPiHi
constexpr double kInvTwoPi = 0.15915494309189535;       // 1/(2*pi)
constexpr double kLog2Base = 13.287712379549449;        // log2(10000)

typedef float f32x2_t __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(kPeThreads) void sinusoidal_pe_kernel(float* __restrict__ pe, int S, int d_model,
                                                                   int pos0) {
    const int half = d_model / 2;
    const int s0 = blockIdx.x * kPeRows;
    const int i = blockIdx.y * kPeThreads + threadIdx.x;   // frequency pair
    if (i >= half) return;
    const double w = exp2(-((double)(2 * i) / (double)d_model) * kLog2Base);
#pragma unroll
    for (int r = 0; r < kPeRows; ++r) {
        const int s = s0 + r;
        if (s >= S) break;
        const double angle = (double)(pos0 + s) * w;
        const double k = rint(angle * kInvTwoPi);
        const double red = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, angle));   // in [-pi, pi] up to rounding
        float sn, cs;
        sincosf((float)red, &sn, &cs);
        const f32x2_t pair = {sn, cs};
        *(f32x2_t*)(pe + (size_t)s * d_model + 2 * i) = pair;
    }
}

}  // namespace

hipError_t launch_sinusoidal_pe(float* pe, int S, int d_model, int pos0, hipEvent_t ev_start, hipEvent_t ev_stop,
                                hipStream_t stream) {
    const unsigned rows = (unsigned)((S + kPeRows - 1) / kPeRows);
    const unsigned chunks = (unsigned)((d_model / 2 + kPeThreads - 1) / kPeThreads);
    hipExtLaunchKernelGGL(sinusoidal_pe_kernel, dim3(rows, chunks), dim3(kPeThreads), 0, stream, ev_start, ev_stop, 0,
                          pe, S, d_model, pos0);
    return hipGetLastError();
}

}  // namespace attn
