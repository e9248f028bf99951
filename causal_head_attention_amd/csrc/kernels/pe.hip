// pe.hip -- sinusoidal position encoding table.
//
// pe[s][2i] = sin(pos * w_i), pe[s][2i+1] = cos(pos * w_i), pos = pos0 + s,
// w_i = 10000^(-2i/d_model) ("Week-4 CUDA notes" page, section 2.3).
//
// The page computes the table in fp32, with the frequencies precomputed
// once and each element one multiply and one sin or cos. Here a workgroup
// covers kPeRows positions and 2 * kPeThreads frequency pairs: each thread
// takes two adjacent pairs, computes their w_i once (fp64) and reuses them
// for those rows, and writes both pairs of a row with one 16-byte store
// when the row layout allows it. The angle pos * w_i is formed and reduced
// modulo pi/2 in fp64 (Cody and Waite's two-part constant), which keeps the
// quadrant; sin and cos of the reduced angle r, |r| <= pi/4, come from their
// Taylor series (through r^11 and r^12, whose remainders are below 1e-11)
// in fp32 by Horner's rule, and the quadrant swaps and negates them. The
// result is accurate to a few fp32 ulp at any position (an fp32 product
// pos * w_i alone would lose about 2^-24 * pos radians).
#include <hip/hip_runtime.h>

#include "../launch.h"
#include "../plan.h"

namespace attn {
namespace {

constexpr double kHalfPiHi = 1.5707963267948966;       // pi/2 rounded to double
constexpr double kHalfPiLo = 6.123233995736766e-17;    // pi/2 - kHalfPiHi
constexpr double kTwoOverPi = 0.6366197723675814;      // 2/pi
constexpr double kLog2Base = 13.287712379549449;       // log2(10000)

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// sin and cos of a non-negative angle (fp64), rounded to fp32
__device__ __forceinline__ void sincos_of(double angle, float& sn, float& cs) {
    const double k = rint(angle * kTwoOverPi);
    const double red = fma(-k, kHalfPiLo, fma(-k, kHalfPiHi, angle));   // in [-pi/4, pi/4] up to rounding
    const int q = (int)k & 3;                                          // angle = r + q * pi/2 (mod 2 pi)
    const float r = (float)red, r2 = r * r;
    // sin r = r + r^3 (-1/3! + r^2 (1/5! + r^2 (-1/7! + r^2 (1/9! - r^2/11!))))
    float ps = -1.0f / 39916800.0f;
    ps = __builtin_fmaf(ps, r2, 1.0f / 362880.0f);
    ps = __builtin_fmaf(ps, r2, -1.0f / 5040.0f);
    ps = __builtin_fmaf(ps, r2, 1.0f / 120.0f);
    ps = __builtin_fmaf(ps, r2, -1.0f / 6.0f);
    const float s = __builtin_fmaf(r * r2, ps, r);
    // cos r = 1 + r^2 (-1/2! + r^2 (1/4! + ... + r^2/12!))
    float pc = 1.0f / 479001600.0f;
    pc = __builtin_fmaf(pc, r2, -1.0f / 3628800.0f);
    pc = __builtin_fmaf(pc, r2, 1.0f / 40320.0f);
    pc = __builtin_fmaf(pc, r2, -1.0f / 720.0f);
    pc = __builtin_fmaf(pc, r2, 1.0f / 24.0f);
    pc = __builtin_fmaf(pc, r2, -0.5f);
    const float c = __builtin_fmaf(r2, pc, 1.0f);
    // sin(r + q pi/2), cos(r + q pi/2): q = 1 gives (cos r, -sin r), q = 2
    // (-sin r, -cos r), q = 3 (-cos r, sin r)
    const float a = (q & 1) ? c : s, b = (q & 1) ? s : c;
    sn = (q & 2) ? -a : a;
    cs = ((q + 1) & 2) ? -b : b;
}

// VEC: rows start 16-byte aligned (d_model % 4 == 0 and pe 16-byte aligned),
// so a thread's two pairs are one 16-byte store
template <bool VEC>
__global__ __launch_bounds__(kPeThreads) void sinusoidal_pe_kernel(float* __restrict__ pe, int S, int d_model,
                                                                   int pos0) {
    const int half = d_model / 2;
    const int s0 = blockIdx.x * kPeRows;
    const int i0 = (blockIdx.y * kPeThreads + threadIdx.x) * 2;   // first of this thread's two pairs
    if (i0 >= half) return;
    const bool two = i0 + 1 < half;
    const double w0 = exp2(-((double)(2 * i0) / (double)d_model) * kLog2Base);
    const double w1 = exp2(-((double)(2 * i0 + 2) / (double)d_model) * kLog2Base);
#pragma unroll
    for (int r = 0; r < kPeRows; ++r) {
        const int s = s0 + r;
        if (s >= S) break;
        const double pos = (double)(pos0 + s);
        float sn0, cs0, sn1, cs1;
        sincos_of(pos * w0, sn0, cs0);
        sincos_of(pos * w1, sn1, cs1);
        float* const row = pe + (size_t)s * d_model + 2 * i0;
        if constexpr (VEC) {
            *(f32x4_t*)row = (f32x4_t){sn0, cs0, sn1, cs1};
        } else {
            *(f32x2_t*)row = (f32x2_t){sn0, cs0};
            if (two) *(f32x2_t*)(row + 2) = (f32x2_t){sn1, cs1};
        }
    }
}

}  // namespace

hipError_t launch_sinusoidal_pe(float* pe, int S, int d_model, int pos0, hipEvent_t ev_start, hipEvent_t ev_stop,
                                hipStream_t stream) {
    const unsigned rows = (unsigned)((S + kPeRows - 1) / kPeRows);
    const unsigned chunks = (unsigned)pe_grid_chunks(d_model);
    if (d_model % 4 == 0 && (reinterpret_cast<uintptr_t>(pe) & 15u) == 0)
        hipExtLaunchKernelGGL(sinusoidal_pe_kernel<true>, dim3(rows, chunks), dim3(kPeThreads), 0, stream, ev_start,
                              ev_stop, 0, pe, S, d_model, pos0);
    else
        hipExtLaunchKernelGGL(sinusoidal_pe_kernel<false>, dim3(rows, chunks), dim3(kPeThreads), 0, stream, ev_start,
                              ev_stop, 0, pe, S, d_model, pos0);
    return hipGetLastError();
}

}  // namespace attn
