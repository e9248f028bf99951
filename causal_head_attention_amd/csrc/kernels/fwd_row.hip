// fwd_row.hip -- one wave per query row: the per-query mapping.
//
// The independent cross-check path: under ATTN_ALGO=row every forward entry
// point (all three storage types, key mask and KV-cache forms) runs here
// instead of the matrix-core kernels, so tests can compare two kernels that
// share no tiling. Each iteration takes
// 64 keys: lane j computes the score of key j0+j (one K row, read in
// 16-byte pieces), the wave reduces max and sum with cross-lane shuffles, and the
// lanes switch to owning head dims to accumulate p_j * V[j0+j, :] with
// coalesced V-row loads.
//
// Method: per-query block mapping ("Hand-written Masked Multi-Head
// Attention CUDA kernel" page, section 2.1); Q row in registers, dot
// products, warp-level max then exp and sum, never writing scores out
// (same page, section 2.2; shuffle reduction instead of shared memory and
// barriers: section 4.1); online softmax with running max and sum and the
// -inf mask ("Week-4 CUDA notes" page, section 2.2); fp32 accumulation
// (MMHA page, section 3.3); a padded key's score set to -inf (Week-4 notes
// page, section 2.2).
#include <hip/hip_runtime.h>

#include "../launch.h"
#include "../plan.h"

namespace attn {
namespace {

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }
template <typename T>
__device__ __forceinline__ T from_f32(float x) { return (T)x; }

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Element e of a 16-byte piece, widened to fp32 (the word is copied out
// first: bit-casting a vector-element lvalue reads element 0 with this
// compiler).
template <typename T>
__device__ __forceinline__ float elem_of(const u32x4_t& w, int e);
template <>
__device__ __forceinline__ float elem_of<float>(const u32x4_t& w, int e) {
    const unsigned u = w[e];
    return __builtin_bit_cast(float, u);
}
template <>
__device__ __forceinline__ float elem_of<__bf16>(const u32x4_t& w, int e) {
    const unsigned u = w[e >> 1];
    return __builtin_bit_cast(float, (u >> (16 * (e & 1))) << 16);
}
template <>
__device__ __forceinline__ float elem_of<_Float16>(const u32x4_t& w, int e) {
    const unsigned u = w[e >> 1];
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(u >> (16 * (e & 1))));
}

constexpr int kRowVBatch = 16;   // V-row loads in flight together in the P.V phase

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

template <typename T, int D>
__global__ __launch_bounds__(kRowThreads) void fwd_row_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                              const T* __restrict__ V, T* __restrict__ O,
                                                              int H, int S_q, int S_cap, int causal, float c,
                                                              const int32_t* __restrict__ kv_lens,
                                                              float* __restrict__ lse,
                                                              const uint8_t* __restrict__ key_mask) {
    constexpr int DPL = (D + 63) / 64;   // head dims per lane in the P.V phase
    __shared__ float qs[D];
    const int lane = threadIdx.x;
    // flat grid over (b, h, i), i fastest
    const int i = (int)(blockIdx.x % (unsigned)S_q);
    const int bh = (int)(blockIdx.x / (unsigned)S_q);
    const int h = bh % H, b = bh / H;
    const size_t qoff = ((size_t)((size_t)b * S_q + i) * H + h) * D;
    for (int d = lane; d < D; d += 64) qs[d] = to_f32(Q[qoff + d]);
    __syncthreads();

    // valid keys of this batch entry; rows of K and V are S_cap apart per entry
    const int S_kv = kv_lens ? min(max(kv_lens[b], 0), S_cap) : S_cap;
    const int n_keys = causal ? max(0, min(S_kv, i + 1 + (S_kv - S_q))) : S_kv;
    float m_run = -INFINITY, l_run = 0.f;
    float acc[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[e] = 0.f;

    for (int j0 = 0; j0 < n_keys; j0 += 64) {
        const int j = j0 + lane;
        float s = -INFINITY;
        // key j is hidden when the key-padding mask says so ([B, S_cap] bytes)
        if (j < n_keys && (!key_mask || key_mask[(size_t)b * S_cap + j] != 0)) {
            // the lane's K row in 16-byte pieces (rows are 16-byte aligned): one
            // load instruction then covers 64 rows once, not once per head dim
            const u32x4_t* krow = (const u32x4_t*)(K + ((size_t)((size_t)b * S_cap + j) * H + h) * D);
            constexpr int E = 16 / (int)sizeof(T);   // elements per piece
            float dot = 0.f;
#pragma unroll 4
            for (int pc = 0; pc < D / E; ++pc) {
                const u32x4_t w = krow[pc];
#pragma unroll
                for (int e = 0; e < E; ++e) dot = __builtin_fmaf(qs[E * pc + e], elem_of<T>(w, e), dot);
            }
            s = dot * c;
        }
        const float m_new = fmaxf(m_run, wave_max(s));
        // m_new is -inf only while every key so far is hidden by the mask
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        const float pj = __builtin_amdgcn_exp2f(s - m_use);
        l_run = l_run * alpha + wave_sum(pj);
        m_run = m_new;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] *= alpha;
        const int nj = min(64, n_keys - j0);
        if (nj == 64) {
            // a full chunk: V rows in batches of 16 loads in flight, then their
            // FMAs (same key order as the loop below)
#pragma unroll 1
            for (int jb = 0; jb < 64; jb += kRowVBatch) {
                float vv[kRowVBatch][DPL];
#pragma unroll
                for (int u = 0; u < kRowVBatch; ++u) {
                    const T* vrow = V + ((size_t)((size_t)b * S_cap + j0 + jb + u) * H + h) * D;
#pragma unroll
                    for (int e = 0; e < DPL; ++e) {
                        const int d = lane + 64 * e;
                        vv[u][e] = d < D ? to_f32(vrow[d]) : 0.f;
                    }
                }
#pragma unroll
                for (int u = 0; u < kRowVBatch; ++u) {
                    const float p = __shfl(pj, jb + u);
                    // a weight of exactly 0 (a hidden key) adds nothing, also
                    // when that key's padding slot holds a NaN
#pragma unroll
                    for (int e = 0; e < DPL; ++e) acc[e] = __builtin_fmaf(p, p != 0.f ? vv[u][e] : 0.f, acc[e]);
                }
            }
        } else {
            for (int jj = 0; jj < nj; ++jj) {
                const float p = __shfl(pj, jj);
                const T* vrow = V + ((size_t)((size_t)b * S_cap + j0 + jj) * H + h) * D;
#pragma unroll
                for (int e = 0; e < DPL; ++e) {
                    const int d = lane + 64 * e;
                    if (d < D) acc[e] = __builtin_fmaf(p, p != 0.f ? to_f32(vrow[d]) : 0.f, acc[e]);
                }
            }
        }
    }
    // a row that sees no key (a KV-cache entry shorter than the chunk) is 0
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
        const int d = lane + 64 * e;
        if (d < D) O[qoff + d] = from_f32<T>(acc[e] * inv);
    }
    // log of the softmax denominator, natural units: ln 2 * (m + log2 l)
    if (lse && lane == 0)
        lse[((size_t)b * H + h) * S_q + i] = l_run > 0.f ? (m_run + __builtin_log2f(l_run)) * 0.69314718055994531f
                                                         : -INFINITY;
}

template <typename T, int D>
hipError_t launch_row(const FwdArgs& a, hipStream_t stream) {
    const unsigned grid = (unsigned)((long long)a.B * a.H * a.S_q);
    hipExtLaunchKernelGGL((fwd_row_kernel<T, D>), dim3(grid), dim3(kRowThreads), 0, stream, a.ev_start, a.ev_stop,
                          0, (const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.o, a.H, a.S_q, a.S_kv, a.causal,
                          a.scale_log2, a.kv_lens, a.lse, a.key_mask);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_row_t(const FwdArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 32: return launch_row<T, 32>(a, stream);
        case 64: return launch_row<T, 64>(a, stream);
        case 128: return launch_row<T, 128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_fwd_row(const FwdArgs& a, Elt t, hipStream_t stream) {
    switch (t) {
        case Elt::F32: return launch_row_t<float>(a, stream);
        case Elt::BF16: return launch_row_t<__bf16>(a, stream);
        case Elt::F16: return launch_row_t<_Float16>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace attn
