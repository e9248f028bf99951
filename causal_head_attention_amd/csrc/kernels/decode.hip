// decode.hip -- single-query attention against a KV cache, split along the keys.
//
// Split kernel: workgroup (split, h, b) takes keys [256*split, 256*split+256)
// of sequence b (clipped to its length; workgroups past the length exit at
// once). Each of its 4 waves streams 64 keys: a key's head vector is one
// contiguous row, read by D*sizeof(T)/16 lanes with 16-byte loads, so a wave
// load instruction covers several keys and every load of the wave is issued
// before the first score is needed. Scores are reduced across the lanes of a
// key with shuffles, the wave's softmax state (max, sum, D accumulators) is
// merged across waves in LDS, and the workgroup writes one partial state.
// Combine kernel: per (b, h), rescale each split's partial state to the
// common maximum, add, divide by the common sum. Splits are merged in a
// fixed order, so results do not change from run to run.
//
// Method: per-query (GEMV-shaped) mapping, dot products and softmax fused
// with the score row kept on chip ("Hand-written Masked Multi-Head
// Attention CUDA kernel" page, sections 2.1 and 2.2); online softmax and
// the need for one common normaliser when a row is spread over several
// blocks ("Week-4 CUDA notes" page, section 2.2); partial reductions in
// the wave, final reduction per block (MMHA page, section 1); grouping
// work of irregular length instead of letting it diverge ("CUDA first
// principles" page, section 4.4).
#include <hip/hip_runtime.h>

#include "../launch.h"
#include "../plan.h"

namespace attn {
namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

template <typename T>
struct Elem;
template <>
struct Elem<float> {
    static constexpr int PER16 = 4;
    __device__ static float get(const u32x4_t& x, int e) {
        // copy the element out first: bit-casting the vector-element lvalue
        // itself reinterprets element 0 with this compiler
        const unsigned u = x[e];
        return __builtin_bit_cast(float, u);
    }
};
template <>
struct Elem<__bf16> {
    static constexpr int PER16 = 8;
    __device__ static float get(const u32x4_t& x, int e) {
        const unsigned u = (x[e >> 1] >> (16 * (e & 1))) << 16;
        return __builtin_bit_cast(float, u);
    }
};

__device__ __forceinline__ int clamp_len(int n, int S_cap) { return n < 0 ? 0 : (n > S_cap ? S_cap : n); }

template <typename T, int D>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_kernel(const T* __restrict__ q,
                                                                      const T* __restrict__ kc,
                                                                      const T* __restrict__ vc,
                                                                      const int32_t* __restrict__ seqlens,
                                                                      float* __restrict__ ws, int H, int S_cap,
                                                                      int n_split_max, float c) {
    constexpr int E = Elem<T>::PER16;                // elements per 16-byte chunk
    constexpr int LPK = D / E;                       // lanes per key
    constexpr int KPI = 64 / LPK;                    // keys per wave load instruction
    constexpr int NIT = kDecodeKeysPerWave / KPI;    // load instructions per wave
    constexpr int NB = NIT < 16 ? NIT : 16;          // loads in flight per batch
    static_assert(NIT % NB == 0, "batching");

    __shared__ float sm[kDecodeWaves], sl[kDecodeWaves];
    __shared__ float sacc[kDecodeWaves][D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int split = (int)(blockIdx.x % (unsigned)n_split_max);
    const int bh = (int)(blockIdx.x / (unsigned)n_split_max);
    const int h = bh % H, b = bh / H;
    const int len = clamp_len(seqlens[b], S_cap);
    if (split * kDecodeChunk >= len) return;   // uniform for the whole workgroup

    const int kend = min(len, (split + 1) * kDecodeChunk);
    const int kstart = split * kDecodeChunk + wave * kDecodeKeysPerWave;
    const int sub = lane % LPK, kl = lane / LPK;

    float qv[E];
    {
        const u32x4_t x = *(const u32x4_t*)(q + ((size_t)b * H + h) * D + E * sub);
#pragma unroll
        for (int e = 0; e < E; ++e) qv[e] = Elem<T>::get(x, e) * c;
    }

    float m_run = -INFINITY, l_run = 0.f, acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.f;

#pragma unroll
    for (int bt = 0; bt < NIT / NB; ++bt) {
        u32x4_t kr[NB], vr[NB];
        const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int it = 0; it < NB; ++it) {
            const int key = kstart + (bt * NB + it) * KPI + kl;
            kr[it] = zero;
            vr[it] = zero;
            if (key < kend) {
                const size_t off = ((size_t)((size_t)b * S_cap + key) * H + h) * D + E * sub;
                kr[it] = *(const u32x4_t*)(kc + off);
                vr[it] = *(const u32x4_t*)(vc + off);
            }
        }
        float s[NB];
#pragma unroll
        for (int it = 0; it < NB; ++it) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) d = __builtin_fmaf(qv[e], Elem<T>::get(kr[it], e), d);
#pragma unroll
            for (int m = LPK / 2; m >= 1; m >>= 1) d += __shfl_xor(d, m);
            const int key = kstart + (bt * NB + it) * KPI + kl;
            s[it] = key < kend ? d : -INFINITY;
        }
        float mx = s[0];
#pragma unroll
        for (int it = 1; it < NB; ++it) mx = fmaxf(mx, s[it]);
#pragma unroll
        for (int m = LPK; m < 64; m <<= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float ls = 0.f, part[E];
#pragma unroll
        for (int e = 0; e < E; ++e) part[e] = 0.f;
#pragma unroll
        for (int it = 0; it < NB; ++it) {
            const float p = __builtin_amdgcn_exp2f(s[it] - m_use);
            ls += p;
#pragma unroll
            for (int e = 0; e < E; ++e) part[e] = __builtin_fmaf(p, Elem<T>::get(vr[it], e), part[e]);
        }
        l_run = l_run * alpha + ls;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = acc[e] * alpha + part[e];
        m_run = m_new;
    }
    // sum over the key groups of the wave (lanes with equal `sub`)
#pragma unroll
    for (int m = LPK; m < 64; m <<= 1) {
        l_run += __shfl_xor(l_run, m);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += __shfl_xor(acc[e], m);
    }
    if (lane == 0) {
        sm[wave] = m_run;
        sl[wave] = l_run;
    }
    if (kl == 0) {
#pragma unroll
        for (int e = 0; e < E; ++e) sacc[wave][E * sub + e] = acc[e];
    }
    __syncthreads();

    float* rec = ws + ((size_t)bh * n_split_max + split) * (D + 2);
    float M = sm[0];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, sm[w]);   // finite: wave 0 has a valid key
    float wt[kDecodeWaves];
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) wt[w] = __builtin_amdgcn_exp2f(sm[w] - M);
    for (int d = tid; d < D; d += kDecodeThreads) {
        float a = 0.f;
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w) a = __builtin_fmaf(wt[w], sacc[w][d], a);
        rec[2 + d] = a;
    }
    if (tid == 0) {
        float L = 0.f;
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w) L = __builtin_fmaf(wt[w], sl[w], L);
        rec[0] = M;
        rec[1] = L;
    }
}

template <typename T, int D>
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* __restrict__ ws,
                                                             const int32_t* __restrict__ seqlens,
                                                             T* __restrict__ o, int H, int S_cap, int n_split_max) {
    const int bh = blockIdx.x;
    const int b = bh / H;
    const int d = threadIdx.x;
    if (d >= D) return;
    const int len = clamp_len(seqlens[b], S_cap);
    T* out = o + (size_t)bh * D;   // [B, 1, H, D]: (b, h) row is bh
    if (len == 0) {
        out[d] = (T)0.f;
        return;
    }
    const int ns = (len + kDecodeChunk - 1) / kDecodeChunk;
    const float* rec = ws + (size_t)bh * n_split_max * (D + 2);
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, rec[(size_t)s * (D + 2)]);
    float L = 0.f, a = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float* r = rec + (size_t)s * (D + 2);
        const float w = __builtin_amdgcn_exp2f(r[0] - M);
        L = __builtin_fmaf(w, r[1], L);
        a = __builtin_fmaf(w, r[2 + d], a);
    }
    out[d] = (T)(a / L);
}

template <typename T, int D>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
    const int nsm = decode_n_split_max(a.S_cap);
    const unsigned grid1 = (unsigned)((long long)nsm * a.H * a.B);
    hipExtLaunchKernelGGL((decode_split_kernel<T, D>), dim3(grid1), dim3(kDecodeThreads), 0, stream, a.ev_start,
                          nullptr, 0, (const T*)a.q, (const T*)a.kcache, (const T*)a.vcache, a.seqlens, a.workspace,
                          a.H, a.S_cap, nsm, a.scale_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipExtLaunchKernelGGL((decode_combine_kernel<T, D>), dim3((unsigned)(a.H * a.B)), dim3(128), 0, stream, nullptr,
                          a.ev_stop, 0, (const float*)a.workspace, a.seqlens, (T*)a.o, a.H, a.S_cap, nsm);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 32: return launch<T, 32>(a, stream);
        case 64: return launch<T, 64>(a, stream);
        case 128: return launch<T, 128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, bool dtype_is_bf16, hipStream_t stream) {
    return dtype_is_bf16 ? launch_t<__bf16>(a, stream) : launch_t<float>(a, stream);
}

}  // namespace attn
