// decode.hip -- single-query attention against a KV cache, split along the keys.
//
// Split kernel: the valid keys of all sequences, laid end to end, form one
// token space; workgroup w of kDecodeSplitWGs (one per CU) streams an equal
// share of it, for ALL heads, one segment per sequence its share touches.
// The cache is [B, S_cap, H, D], so one token's H head rows are one
// contiguous span: each wave owns a group of heads whose rows for one token
// are read by one 16-byte-per-lane load instruction, and the eight waves of
// the workgroup together sweep whole token rows. A head's D elements sit in
// one group of D*sizeof(T)/16 lanes ("a row"), so the dot product reduces
// with DPP inside the row and the head's softmax state (max, sum, D
// accumulators) lives in that row; each (segment, h) leaves one partial
// record in the workspace. Equal shares keep every CU streaming until the
// end (a fixed number of keys per workgroup left a partly idle second wave
// of workgroups and many that only found their sequence already ended).
// Combine kernel: per (b, h), rescale each segment's partial state to the
// common maximum, add, divide by the common sum, in one pass over the
// records. Segments are merged in a fixed order, so results do not change
// from run to run.
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
// 16-bit types: elements stay packed in pairs for v_dot2 (exact products,
// fp32 accumulation).
template <>
struct Elem<__bf16> {
    static constexpr int PER16 = 8;
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
    __device__ static float get(const u32x4_t& x, int e) {
        const unsigned u = (x[e >> 1] >> (16 * (e & 1))) << 16;
        return __builtin_bit_cast(float, u);
    }
    __device__ static float dot2(v2 a, v2 b, float c) { return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false); }
};
template <>
struct Elem<_Float16> {
    static constexpr int PER16 = 8;
    typedef _Float16 v2 __attribute__((ext_vector_type(2)));
    __device__ static float get(const u32x4_t& x, int e) {
        const unsigned short u = (unsigned short)(x[e >> 1] >> (16 * (e & 1)));
        return (float)__builtin_bit_cast(_Float16, u);
    }
    __device__ static float dot2(v2 a, v2 b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }
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

// Sum over the workgroup; every thread gets it. `red` holds one slot per wave.
template <int NT = kDecodeThreads>
__device__ __forceinline__ long long block_sum(long long x, long long* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    __syncthreads();   // earlier readers of red are done
    if (lane == 0) red[wave] = x;
    __syncthreads();
    long long t = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) t += red[w];
    return t;
}

// Record index of segment (w, b), workgroup w's part of sequence b: w + b.
// It is unique. Workgroup ranges and sequences both tile the token space in
// order; if workgroup w+k (k >= 1) reached into sequence b-k, its range
// would start before sequence b-k+1 does, hence before sequence b, while
// workgroup w's range, which ends where w+1's begins, reaches into b.
__device__ __forceinline__ int record_of(int w, int b) { return w + b; }

template <typename T, int D>
__global__ __launch_bounds__(kDecodeThreads) void decode_split_kernel(const T* __restrict__ q,
                                                                      const T* __restrict__ kc,
                                                                      const T* __restrict__ vc,
                                                                      const int32_t* __restrict__ seqlens,
                                                                      float* __restrict__ ws, int B, int H, int S_cap,
                                                                      float c) {
    using C = DecCfg<T, D>;
    constexpr int E = C::E, LPH = C::LPH, HPI = C::HPI;
    constexpr bool k16 = sizeof(T) == 2;   // bf16 or fp16: packed v_dot2 paths
    __shared__ long long red[kDecodeThreads / 64];
    __shared__ long long incl_s[kDecodeScanLds];   // inclusive prefix sums of the lengths

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int w = blockIdx.x, G = gridDim.x;
    const bool scan_in_lds = B <= kDecodeScanLds;

    // (1) prefix sums of the clamped lengths (the token space), one read of seqlens
    long long run = 0;
    for (int base = 0; base < B; base += kDecodeThreads) {
        const int bb = base + tid;
        const long long len = bb < B ? clamp_len(seqlens[bb], S_cap) : 0;
        long long incl = len;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const long long y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        __syncthreads();
        if (lane == 63) red[wave] = incl;
        __syncthreads();
        long long wpre = 0, ctot = 0;
#pragma unroll
        for (int x = 0; x < kDecodeThreads / 64; ++x) {
            ctot += red[x];
            if (x < wave) wpre += red[x];
        }
        if (scan_in_lds && bb < B) incl_s[bb] = incl + wpre + run;
        run += ctot;
    }
    const long long Ttot = run;
    if (Ttot == 0) return;   // uniform
    const long long Ct = (Ttot + G - 1) / G;
    const long long lo = (long long)w * Ct;
    const long long hi = lo + Ct < Ttot ? lo + Ct : Ttot;
    if (lo >= hi) return;   // uniform

    // (2) first sequence reaching into [lo, hi): the number of sequences
    // that end at or before lo, and where it starts
    int b_first;
    long long P;
    if (scan_in_lds) {
        __syncthreads();
        int n = 0, span = B;   // binary search: incl_s is non-decreasing
        while (span > 0) {
            const int half = span >> 1;
            if (incl_s[n + half] <= lo) {
                n += half + 1;
                span -= half + 1;
            } else {
                span = half;
            }
        }
        b_first = n;
        P = n > 0 ? incl_s[n - 1] : 0;
    } else {
        long long n_before = 0, t_before = 0;
        run = 0;
        for (int base = 0; base < B; base += kDecodeThreads) {
            const int bb = base + tid;
            const long long len = bb < B ? clamp_len(seqlens[bb], S_cap) : 0;
            long long incl = len;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const long long y = __shfl_up(incl, o);
                if (lane >= o) incl += y;
            }
            __syncthreads();
            if (lane == 63) red[wave] = incl;
            __syncthreads();
            long long wpre = 0, ctot = 0;
#pragma unroll
            for (int x = 0; x < kDecodeThreads / 64; ++x) {
                ctot += red[x];
                if (x < wave) wpre += red[x];
            }
            if (bb < B && incl + wpre + run <= lo) {
                n_before += 1;
                t_before += len;
            }
            run += ctot;
        }
        b_first = (int)block_sum<kDecodeThreads>(n_before, red);
        P = block_sum<kDecodeThreads>(t_before, red);
    }

    // (3) one segment per sequence the range touches
    const int sub = lane % LPH, hl = lane / LPH;
    const int key_bytes = H * D * (int)sizeof(T);
    const int n_groups = (H + HPI - 1) / HPI;
    for (int b = b_first; b < B && P < hi; ++b) {
        const int len = scan_in_lds ? (int)(incl_s[b] - P) : clamp_len(seqlens[b], S_cap);
        if (len > 0) {
            const int k0 = (int)((lo > P ? lo : P) - P);
            const int k1 = (int)((hi < P + len ? hi : P + len) - P);
            const int rec_id = record_of(w, b);
            // descriptors over sequence b's rows that end at key k1: loads
            // past it return zeros without touching memory
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(kc + (size_t)b * S_cap * H * D), (short)0, k1 * key_bytes, 0x00020000);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(vc + (size_t)b * S_cap * H * D), (short)0, k1 * key_bytes, 0x00020000);
            for (int grp = wave; grp < n_groups; grp += kDecodeWaves) {
                const int h = grp * HPI + hl;
                const bool h_ok = h < H;
                const int lane_off = ((h_ok ? h : 0) * D + E * sub) * (int)sizeof(T);

                // this row's query chunk; 16-bit types stay packed (exact) for v_dot2
                // and the scale is applied to the reduced score
                const u32x4_t qx = *(const u32x4_t*)(q + ((size_t)b * H + (h_ok ? h : 0)) * D + E * sub);
                float qf[E];
                if constexpr (!k16) {
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
                        if constexpr (k16) {
#pragma unroll
                            for (int w = 0; w < 4; ++w) {
                                // scalar copies first (bit-casting a vector-element lvalue
                                // reads element 0 with this compiler)
                                const unsigned kw = kr[it][w], qw = qx[w];
                                d = Elem<T>::dot2(__builtin_bit_cast(typename Elem<T>::v2, kw),
                                                  __builtin_bit_cast(typename Elem<T>::v2, qw), d);
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
                    if constexpr (k16) {
                        // pairs of keys: P rounded to the storage type, V pairs packed per head dim,
                        // one v_dot2 per (pair, dim); the sum adds the same rounded P
#pragma unroll
                        for (int it = 0; it < kDecodeBatch; it += 2) {
                            typedef typename Elem<T>::v2 v2;
                            const v2 pp = {(T)__builtin_amdgcn_exp2f(s[it] - m_new),
                                           (T)__builtin_amdgcn_exp2f(s[it + 1] - m_new)};
                            const v2 ones = {(T)1.0f, (T)1.0f};
                            l_run = Elem<T>::dot2(pp, ones, l_run);
#pragma unroll
                            for (int e = 0; e < E; ++e) {
                                const unsigned va = (vr[it][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                                const unsigned vb = (vr[it + 1][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                                acc[e] = Elem<T>::dot2(__builtin_bit_cast(v2, va | (vb << 16)), pp, acc[e]);
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
                // one partial record per (segment, h): [max, sum, D accumulators]
                if (h_ok) {
                    float* rec = ws + ((size_t)rec_id * H + h) * (D + 2);
                    if (sub == 0) {
                        rec[0] = m_run;
                        rec[1] = l_run;
                    }
#pragma unroll
                    for (int e = 0; e < E; ++e) rec[2 + E * sub + e] = acc[e];
                }
            }
        }
        P += len;
    }
}

// Combine: one workgroup per (b, h). Sequence b's segments belong to split
// workgroups w0..w1; thread (part, d) merges head dim d of the segments
// s = part, part + NP, ... online (running maximum), with all of its loads
// issued before the first use, and the NP parts are merged in LDS. Fixed
// order throughout, so the result is deterministic.
template <typename T, int D>
__global__ __launch_bounds__(kCombineThreads) void decode_combine_kernel(const float* __restrict__ ws,
                                                                         const int32_t* __restrict__ seqlens,
                                                                         T* __restrict__ o, int B, int H, int S_cap,
                                                                         int G) {
    constexpr int NP = kCombineThreads / D;       // parts
    constexpr int PER = 16;                       // segments in flight per thread per round
    __shared__ float part_m[NP], part_l[NP];
    __shared__ float part_acc[NP][D];
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63;
    T* out = o + (size_t)bh * D;   // [B, 1, H, D]: the (b, h) row is bh
    // token-space geometry (total, start of sequence b, its length): every
    // wave sums the lengths itself, so no barrier precedes the record loads
    long long all = 0, before = 0, mine = 0;
    for (int bb = lane; bb < B; bb += 64) {
        const long long l = clamp_len(seqlens[bb], S_cap);
        all += l;
        if (bb < b) before += l;
        if (bb == b) mine = l;
    }
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) {
        all += __shfl_xor(all, x);
        before += __shfl_xor(before, x);
        mine += __shfl_xor(mine, x);
    }
    const long long Ttot = all, Pb = before;
    const int len = (int)mine;
    if (len == 0) {   // uniform; a sequence with no keys gives a zero row
        for (int d = tid; d < D; d += kCombineThreads) out[d] = (T)0.f;
        return;
    }
    const long long Ct = (Ttot + G - 1) / G;
    const int w0 = (int)(Pb / Ct), w1 = (int)((Pb + len - 1) / Ct);
    const int ns = w1 - w0 + 1;
    const size_t stride = (size_t)H * (D + 2);   // between consecutive records
    const float* rec = ws + ((size_t)record_of(w0, b) * H + h) * (D + 2);

    const int d = tid % D, part = tid / D;
    float M = -INFINITY, L = 0.f, A = 0.f;
    for (int s0 = part; s0 < ns; s0 += NP * PER) {
        float mm[PER], ll[PER], xx[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int s = s0 + j * NP;
            const bool ok = s < ns;
            mm[j] = ok ? rec[(size_t)s * stride] : -INFINITY;
            ll[j] = ok ? rec[(size_t)s * stride + 1] : 0.f;
            xx[j] = ok ? rec[(size_t)s * stride + 2 + d] : 0.f;
        }
        float mn = M;
#pragma unroll
        for (int j = 0; j < PER; ++j) mn = fmaxf(mn, mm[j]);   // finite: segment s0 exists
        const float a = __builtin_amdgcn_exp2f(M - mn);        // 0 while M is -inf
        L *= a;
        A *= a;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const float wj = __builtin_amdgcn_exp2f(mm[j] - mn);   // 0 for absent segments
            L = __builtin_fmaf(wj, ll[j], L);
            A = __builtin_fmaf(wj, xx[j], A);
        }
        M = mn;
    }
    if (d == 0) {
        part_m[part] = M;
        part_l[part] = L;
    }
    part_acc[part][d] = A;
    __syncthreads();
    if (tid < D) {
        float Mt = part_m[0];
#pragma unroll
        for (int p = 1; p < NP; ++p) Mt = fmaxf(Mt, part_m[p]);
        float Lt = 0.f, t = 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const float wp = __builtin_amdgcn_exp2f(part_m[p] - Mt);   // 0 for a part with no segment
            Lt = __builtin_fmaf(wp, part_l[p], Lt);
            t = __builtin_fmaf(wp, part_acc[p][tid], t);
        }
        out[tid] = (T)(t / Lt);
    }
}

template <typename T, int D>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
    hipExtLaunchKernelGGL((decode_split_kernel<T, D>), dim3(kDecodeSplitWGs), dim3(kDecodeThreads), 0, stream,
                          a.ev_start, nullptr, 0, (const T*)a.q, (const T*)a.kcache, (const T*)a.vcache, a.seqlens,
                          a.workspace, a.B, a.H, a.S_cap, a.scale_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipExtLaunchKernelGGL((decode_combine_kernel<T, D>), dim3((unsigned)(a.H * a.B)), dim3(kCombineThreads), 0,
                          stream, nullptr, a.ev_stop, 0, (const float*)a.workspace, a.seqlens, (T*)a.o, a.B, a.H,
                          a.S_cap, kDecodeSplitWGs);
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

hipError_t launch_decode(const DecodeArgs& a, Elt t, hipStream_t stream) {
    switch (t) {
        case Elt::F32: return launch_t<float>(a, stream);
        case Elt::BF16: return launch_t<__bf16>(a, stream);
        case Elt::F16: return launch_t<_Float16>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace attn
