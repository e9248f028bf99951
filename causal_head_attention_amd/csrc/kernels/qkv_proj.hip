// qkv_proj.hip -- the Q, K and V projections as one GEMM on gfx950 matrix cores.
//
// C[M, 3N] = X[M, E] . W[3N, E]^T in fp32 (N = H*D), written as three
// [M, N] = [B, S, H, D] tensors: columns [0, N) of C are Q, [N, 2N) K and
// [2N, 3N) V. The weights are stored output-major (row c*N + n holds the E
// weights of output column n of Q, K or V), so both operands of every MFMA
// are contiguous along the contraction.
//
// Method: Q = X W_Q, K = X W_K, V = X W_V ("Hand-written Masked Multi-Head
// Attention CUDA kernel" page, section 2) computed as one concatenated GEMM
// ("Week-4 CUDA notes" page, section 2.1); shared-memory tiling of both
// operands, 128-bit loads, double buffering ("Week-4 CUDA notes" page,
// sections 1.2-1.3).
//
// One workgroup (8 waves, 2 per SIMD) owns a 256 x 384 tile of C and walks E
// in steps of 32: both operand tiles go HBM -> registers -> LDS (rows padded
// to 80 bytes, so the lanes that read one MFMA fragment spread over the
// banks), double-buffered in LDS, one barrier per step. Two register sets
// carry the loads, so each K slice is requested two steps before it is
// stored (its L2 / Infinity Cache latency is about one step). Wave (wm, wn)
// of the 2 x 4 grid computes a 128 x 96 sub-tile as 4 x 3 blocks of
// v_mfma_f32_32x32x16_{bf16,f16}: per k-step 7 fragment reads feed 12 MFMAs.
// The 2,048 x 12,288 projection of a 4,096-wide model is 8 x 32 = 256 tiles,
// one workgroup per CU. Workgroup ids are remapped so each XCD gets a
// contiguous range of logical tiles, M-tile fastest: the workgroups that
// share a W tile run on one XCD at the same time and find it in its L2.
#include <hip/hip_runtime.h>

#include "../launch.h"
#include "../plan.h"

namespace attn {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
struct GemmMma;
template <>
struct GemmMma<__bf16> {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    __device__ static f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct GemmMma<_Float16> {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    __device__ static f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

constexpr int kRowBytes = kGemmBK * 2 + 16;            // one padded LDS row (32 elements + 16 B)
constexpr int kRowChunks = kGemmBK * 2 / 16;           // 16-byte chunks of a row
constexpr int kABytes = kGemmBM * kRowBytes;
constexpr int kBBytes = kGemmBN * kRowBytes;
constexpr int kStageBytes = kABytes + kBBytes;
constexpr int kAChunks = kGemmBM * kRowChunks / kGemmThreads;   // 16-byte loads per thread
constexpr int kBChunks = kGemmBN * kRowChunks / kGemmThreads;
constexpr int kWaveM = kGemmBM / kGemmWavesM, kWaveN = kGemmBN / kGemmWavesN;   // outputs of one wave
constexpr int kMB = kWaveM / 32, kNB = kWaveN / 32;                           // its 32 x 32 blocks
static_assert(kMB * 32 == kWaveM && kNB * 32 == kWaveN, "waves own whole 32 x 32 blocks");
static_assert(kAChunks * kGemmThreads * 16 == kGemmBM * kGemmBK * 2, "A tile splits evenly");
static_assert(kBChunks * kGemmThreads * 16 == kGemmBN * kGemmBK * 2, "B tile splits evenly");
static_assert(2 * kStageBytes <= 160 * 1024, "two stages fit in LDS");

template <typename T>
__global__ __launch_bounds__(kGemmThreads) void qkv_proj_kernel(const uint16_t* __restrict__ X,
                                                                const uint16_t* __restrict__ W, T* __restrict__ Qo,
                                                                T* __restrict__ Ko, T* __restrict__ Vo, int M, int E,
                                                                int N) {
    typedef typename GemmMma<T>::v8 v8;
    __shared__ __attribute__((aligned(16))) char lds[2 * kStageBytes];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const int wm = wave % kGemmWavesM, wn = wave / kGemmWavesM;

    const int tiles_m = (M + kGemmBM - 1) / kGemmBM;
    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int mt = item % tiles_m, nt = item / tiles_m;
    const int m0 = mt * kGemmBM, n0 = nt * kGemmBN;
    const int NN = 3 * N;

    // Descriptors over this tile's rows: rows past M (or past 3N) read as 0.
    const int rows_a = min(kGemmBM, M - m0), rows_b = min(kGemmBN, NN - n0);
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void*)(X + (size_t)m0 * E), (short)0, rows_a * E * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)(W + (size_t)n0 * E), (short)0, rows_b * E * 2, 0x00020000);

    // thread t stages 16-byte chunks c = t + 512 i: row c / 4, chunk c % 4;
    // two register sets, so a K slice is loaded two steps before it is stored
    struct Regs {
        u32x4_t a[kAChunks], b[kBChunks];
    };
    Regs r0, r1;
    auto gload = [&](Regs& r, int k0) {
#pragma unroll
        for (int i = 0; i < kAChunks; ++i) {
            const int c = tid + kGemmThreads * i;
            r.a[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, (c / kRowChunks) * E * 2 + k0 * 2 + (c % kRowChunks) * 16,
                                                      0, 0);
        }
#pragma unroll
        for (int i = 0; i < kBChunks; ++i) {
            const int c = tid + kGemmThreads * i;
            r.b[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, (c / kRowChunks) * E * 2 + k0 * 2 + (c % kRowChunks) * 16,
                                                      0, 0);
        }
    };
    auto lstore = [&](const Regs& r, int st) {
        char* a = lds + st * kStageBytes;
        char* b = a + kABytes;
#pragma unroll
        for (int i = 0; i < kAChunks; ++i) {
            const int c = tid + kGemmThreads * i;
            *(u32x4_t*)(a + (c / kRowChunks) * kRowBytes + (c % kRowChunks) * 16) = r.a[i];
        }
#pragma unroll
        for (int i = 0; i < kBChunks; ++i) {
            const int c = tid + kGemmThreads * i;
            *(u32x4_t*)(b + (c / kRowChunks) * kRowBytes + (c % kRowChunks) * 16) = r.b[i];
        }
    };

    f32x16_t acc[kMB][kNB];
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.f;

    // A fragment: lane holds row l32 of a 32-row block, elements 8g..8g+7 of
    // the 16-wide k-step; B fragment likewise for a row of W (a column of C)
    const int a_lane = (wm * kWaveM + l32) * kRowBytes + g * 16;
    const int b_lane = (wn * kWaveN + l32) * kRowBytes + g * 16;

    const int nk = E / kGemmBK;
    auto slice = [&](int i) { return (i < nk ? i : nk - 1) * kGemmBK; };   // past the end: reload the last
    auto compute = [&](int st) {
        const char* a = lds + st * kStageBytes + a_lane;
        const char* b = lds + st * kStageBytes + kABytes + b_lane;
#pragma unroll
        for (int ks = 0; ks < kGemmBK / 16; ++ks) {
            v8 af[kMB], bf[kNB];
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb) af[mb] = *(const v8*)(a + mb * 32 * kRowBytes + ks * 32);
#pragma unroll
            for (int nb = 0; nb < kNB; ++nb) bf[nb] = *(const v8*)(b + nb * 32 * kRowBytes + ks * 32);
#pragma unroll
            for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
                for (int nb = 0; nb < kNB; ++nb) acc[mb][nb] = GemmMma<T>::mfma(af[mb], bf[nb], acc[mb][nb]);
        }
    };
    gload(r0, slice(0));
    gload(r1, slice(1));
    lstore(r0, 0);
    __syncthreads();
    // steps s (stage 0) and s+1 (stage 1): slice s+2 goes into r0 while stage 0
    // is read, slice s+1 (in r1 since the previous pair) lands in stage 1;
    // stores past the last step write a stage no one reads again
    for (int s = 0; s < nk; s += 2) {
        gload(r0, slice(s + 2));
        compute(0);
        lstore(r1, 1);
        __syncthreads();
        if (s + 1 < nk) {
            gload(r1, slice(s + 3));
            compute(1);
            lstore(r0, 0);
            __syncthreads();
        }
    }

    // Epilogue. Lane holds column l32 of each 32 x 32 block and rows
    // 8*(r/4) + 4*g + r%4 (register r); a block's 32 columns lie in one of
    // Q, K, V because N is a multiple of 32. Rows past M fall outside the
    // output descriptor and are dropped.
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
        const int cb = n0 + wn * kWaveN + nb * 32;   // first column of the block in C
        if (cb >= NN) continue;
        const int which = cb / N;
        T* out = which == 0 ? Qo : (which == 1 ? Ko : Vo);
        const int col = cb - which * N + l32;
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(out + (size_t)m0 * N), (short)0, rows_a * N * 2, 0x00020000);
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * kWaveM + mb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                const T x = (T)acc[mb][nb][r];
                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x), ro,
                                                      (row * N + col) * 2, 0, 0);
            }
    }
}

template <typename T>
hipError_t launch_t(const QkvArgs& a, hipStream_t stream) {
    const int tiles_m = (a.M + kGemmBM - 1) / kGemmBM;
    const int tiles_n = (3 * a.N + kGemmBN - 1) / kGemmBN;
    hipExtLaunchKernelGGL(qkv_proj_kernel<T>, dim3((unsigned)(tiles_m * tiles_n)), dim3(kGemmThreads), 0, stream,
                          a.ev_start, a.ev_stop, 0, (const uint16_t*)a.x, (const uint16_t*)a.w, (T*)a.q, (T*)a.k,
                          (T*)a.v, a.M, a.E, a.N);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_proj(const QkvArgs& a, Elt t, hipStream_t stream) {
    switch (t) {
        case Elt::BF16: return launch_t<__bf16>(a, stream);
        case Elt::F16: return launch_t<_Float16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
