// decode.hip -- single-query attention against a KV cache, split along the keys.
//
// Split kernel: workgroup (split, b) takes keys [64*split, 64*split+64) of
// sequence b (clipped to its length; workgroups past the length exit at
// once) for ALL heads. The cache is [B, S_cap, H, D], so one token's H head
// rows are one contiguous span: each wave owns a group of heads whose rows
// for one token are read by one 16-byte-per-lane load instruction, and the
// eight waves of the workgroup together sweep whole token rows. A head's
// D elements sit in one group of D*sizeof(T)/16 lanes ("a row"), so the dot
// product reduces with DPP inside the row and the head's softmax state (max,
// sum, D accumulators) lives in that row; one partial state per (b, h,
// split) goes to the workspace.
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
// principles" page, section 4.4); contiguous, coalesced loads ("CUDA first
// principles" page, section 3.2).
#include <hip/hip_runtime.h>

#include "../launch.h"
#include "../plan.h"

namespace attn {
namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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

constexpr int kNonTemporal = 2;   // buffer-load cache policy: nt

__device__ __forceinline__ int clamp_len(int n, int S_cap) { return n < 0 ? 0 : (n > S_cap ? S_cap : n); }

// DPP lane moves inside 16-lane rows (gfx9 encodings).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadSwap1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kRowMirror = 0x140;      // lane i <-> 15-i within 16

// Sum over groups of N consecutive lanes (N = 4, 8, 16 or 32); every lane of
// the group gets the total.
template <int N>
__device__ __forceinline__ float row_sum(float x) {
    x += dpp<kQuadSwap1>(x);
    x += dpp<kQuadSwap2>(x);
    if constexpr (N >= 8) x += dpp<kRowHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kRowMirror>(x);
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    return x;
}

template <typename T, int D>
struct DecCfg {
    static constexpr int E = Elem<T>::PER16;     // elements per 16-byte chunk
    static constexpr int LPH = D / E;            // lanes per head row
    static constexpr int HPI = 64 / LPH;         // heads per wave load instruction
};

// Descriptor over sequence b's cache rows ([S_cap, H, D] slice); reads past
// the slice return zeros.
template <typename T, int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t seq_rsrc(const T* base, int b, int S_cap, int H) {
    const T* p = base + (size_t)b * S_cap * H * D;
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, S_cap * H * D * (int)sizeof(T), 0x00020000);
}

template <typename T, int D>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_kernel(const T* __restrict__ q,
                                                                      const T* __restrict__ kc,
                                                                      const T* __restrict__ vc,
                                                                      const int32_t* __restrict__ seqlens,
                                                                      float* __restrict__ ws, int H, int S_cap,
                                                                      int n_split_max, float c) {
    using C = DecCfg<T, D>;
    constexpr int E = C::E, LPH = C::LPH, HPI = C::HPI;
    constexpr bool kBf16 = sizeof(T) == 2;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int split = (int)(blockIdx.x % (unsigned)n_split_max);
    const int b = (int)(blockIdx.x / (unsigned)n_split_max);
    const int len = clamp_len(seqlens[b], S_cap);
    const int k0 = split * kDecodeChunk;
    if (k0 >= len) return;   // uniform for the whole workgroup
    const int k1 = min(len, k0 + kDecodeChunk);
    const int sub = lane % LPH, hl = lane / LPH;
    const __amdgpu_buffer_rsrc_t rk = seq_rsrc<T, D>(kc, b, S_cap, H);
    const __amdgpu_buffer_rsrc_t rv = seq_rsrc<T, D>(vc, b, S_cap, H);
    const int key_bytes = H * D * (int)sizeof(T);
    const int n_groups = (H + HPI - 1) / HPI;

    for (int grp = wave; grp < n_groups; grp += kDecodeWaves) {
        const int h = grp * HPI + hl;
        const bool h_ok = h < H;
        const int lane_off = ((h_ok ? h : 0) * D + E * sub) * (int)sizeof(T);

        // this row's query chunk; bf16 stays packed (exact) for v_dot2 and the
        // scale is applied to the reduced score
        const u32x4_t qx = *(const u32x4_t*)(q + ((size_t)b * H + (h_ok ? h : 0)) * D + E * sub);
        float qf[E];
        if constexpr (!kBf16) {
#pragma unroll
            for (int e = 0; e < E; ++e) qf[e] = Elem<T>::get(qx, e);
        }

        float m_run = -INFINITY, l_run = 0.f, acc[E];
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = 0.f;

        for (int kb = k0; kb < k1; kb += kDecodeBatch) {
            u32x4_t kr[kDecodeBatch], vr[kDecodeBatch];
#pragma unroll
            for (int it = 0; it < kDecodeBatch; ++it) {
                const int off = lane_off + (kb + it) * key_bytes;
                // read-once stream: non-temporal, so the loads do not allocate
                // in the caches (and do not evict whatever is resident there)
                kr[it] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, kNonTemporal);
                vr[it] = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kNonTemporal);
            }
            float s[kDecodeBatch];
#pragma unroll
            for (int it = 0; it < kDecodeBatch; ++it) {
                float d = 0.f;
                if constexpr (kBf16) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        // scalar copies first (bit-casting a vector-element lvalue
                        // reads element 0 with this compiler)
                        const unsigned kw = kr[it][w], qw = qx[w];
                        d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, kw),
                                                            __builtin_bit_cast(bf16x2_t, qw), d, false);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) d = __builtin_fmaf(qf[e], Elem<T>::get(kr[it], e), d);
                }
                d = row_sum<LPH>(d) * c;
                s[it] = (kb + it < k1) ? d : -INFINITY;
            }
            // slots past the length may hold anything (even NaN): their
            // probability is 0, and their values must not reach the sums
            if (kb + kDecodeBatch > k1) {
                const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int it = 0; it < kDecodeBatch; ++it)
                    if (kb + it >= k1) vr[it] = zero;
            }
            float mx = s[0];
#pragma unroll
            for (int it = 1; it < kDecodeBatch; ++it) mx = fmaxf(mx, s[it]);
            const float m_new = fmaxf(m_run, mx);   // finite: key kb < k1 is valid
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] *= alpha;
            m_run = m_new;
            if constexpr (kBf16) {
                // pairs of keys: P rounded to bf16, V pairs packed per head dim,
                // one v_dot2 per (pair, dim); the sum adds the same rounded P
#pragma unroll
                for (int it = 0; it < kDecodeBatch; it += 2) {
                    const bf16x2_t pp = {(__bf16)__builtin_amdgcn_exp2f(s[it] - m_new),
                                         (__bf16)__builtin_amdgcn_exp2f(s[it + 1] - m_new)};
                    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
                    l_run = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l_run, false);
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const unsigned va = (vr[it][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                        const unsigned vb = (vr[it + 1][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                        acc[e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, va | (vb << 16)), pp,
                                                                 acc[e], false);
                    }
                }
            } else {
#pragma unroll
                for (int it = 0; it < kDecodeBatch; ++it) {
                    const float p = __builtin_amdgcn_exp2f(s[it] - m_new);
                    l_run += p;
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(p, Elem<T>::get(vr[it], e), acc[e]);
                }
            }
        }
        // one partial record per (b, h, split): [max, sum, D accumulators]
        if (h_ok) {
            float* rec = ws + (((size_t)b * H + h) * n_split_max + split) * (D + 2);
            if (sub == 0) {
                rec[0] = m_run;
                rec[1] = l_run;
            }
#pragma unroll
            for (int e = 0; e < E; ++e) rec[2 + E * sub + e] = acc[e];
        }
    }
}

// Combine: one workgroup per (b, h). The split maxima are read in parallel
// (one split per thread) and reduced; each split's weight exp2(m_s - M) goes
// to LDS with the common sum. Then thread (part, d) adds the weighted
// accumulators of head dim d for the splits s = part, part + P, ... with all
// of its loads issued before the first add, and the P parts are summed in
// LDS. Fixed order throughout, so the result is deterministic.
template <typename T, int D>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(const float* __restrict__ ws,
                                                                         const int32_t* __restrict__ seqlens,
                                                                         T* __restrict__ o, int H, int S_cap,
                                                                         int n_split_max) {
    constexpr int P = kCombineThreads / D;        // split parts
    constexpr int PER = 16;                       // loads in flight per thread per round
    __shared__ float w_s[kDecodeMaxSplits];
    __shared__ float red[kCombineThreads / 64];
    __shared__ float part_acc[P][D];
    const int bh = blockIdx.x;
    const int b = bh / H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int len = clamp_len(seqlens[b], S_cap);
    T* out = o + (size_t)bh * D;   // [B, 1, H, D]: the (b, h) row is bh
    if (len == 0) {
        for (int d = tid; d < D; d += kCombineThreads) out[d] = (T)0.f;
        return;
    }
    const int ns = (len + kDecodeChunk - 1) / kDecodeChunk;
    const float* rec = ws + (size_t)bh * n_split_max * (D + 2);
    // common maximum
    float m = -INFINITY;
    for (int s = tid; s < ns; s += kCombineThreads) m = fmaxf(m, rec[(size_t)s * (D + 2)]);
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) m = fmaxf(m, __shfl_xor(m, x));
    if (lane == 0) red[wave] = m;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int w = 1; w < kCombineThreads / 64; ++w) M = fmaxf(M, red[w]);
    __syncthreads();
    // per-split weights and the common sum
    float L = 0.f;
    for (int s = tid; s < ns; s += kCombineThreads) {
        const float w = __builtin_amdgcn_exp2f(rec[(size_t)s * (D + 2)] - M);
        w_s[s] = w;
        L = __builtin_fmaf(w, rec[(size_t)s * (D + 2) + 1], L);
    }
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) L += __shfl_xor(L, x);
    if (lane == 0) red[wave] = L;
    __syncthreads();
    float Lt = 0.f;
#pragma unroll
    for (int w = 0; w < kCombineThreads / 64; ++w) Lt += red[w];
    // weighted accumulators: thread (part, d)
    const int d = tid % D, part = tid / D;
    float a = 0.f;
    for (int s0 = part; s0 < ns; s0 += P * PER) {
        float x[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int s = s0 + j * P;
            x[j] = s < ns ? rec[(size_t)s * (D + 2) + 2 + d] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int s = s0 + j * P;
            if (s < ns) a = __builtin_fmaf(w_s[s], x[j], a);
        }
    }
    part_acc[part][d] = a;
    __syncthreads();
    if (tid < D) {
        float t = 0.f;
#pragma unroll
        for (int q = 0; q < P; ++q) t += part_acc[q][tid];
        out[tid] = (T)(t / Lt);
    }
}

template <typename T, int D>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
    const int nsm = decode_n_split_max(a.S_cap);
    const unsigned grid1 = (unsigned)((long long)nsm * a.B);
    hipExtLaunchKernelGGL((decode_split_kernel<T, D>), dim3(grid1), dim3(kDecodeThreads), 0, stream, a.ev_start,
                          nullptr, 0, (const T*)a.q, (const T*)a.kcache, (const T*)a.vcache, a.seqlens, a.workspace,
                          a.H, a.S_cap, nsm, a.scale_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipExtLaunchKernelGGL((decode_combine_kernel<T, D>), dim3((unsigned)(a.H * a.B)), dim3(kCombineThreads), 0,
                          stream, nullptr, a.ev_stop, 0, (const float*)a.workspace, a.seqlens, (T*)a.o, a.H,
                          a.S_cap, nsm);
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
