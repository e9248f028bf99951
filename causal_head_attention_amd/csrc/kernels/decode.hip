// decode.hip -- single-query attention against a KV cache, split along the keys.
//
// One kernel. The valid keys of all sequences, laid end to end, form one
// token space; workgroup w of kDecodeSplitWGs (one per CU) streams one
// contiguous share of it (the shares are sized to the XCD the workgroup
// runs on), for ALL heads, one segment per sequence its share touches.
// The cache is [B, S_cap, H, D], so one token's H head rows are one
// contiguous span: each wave owns a group of heads whose rows for one token
// are read by one 16-byte-per-lane load instruction, and the eight waves of
// the workgroup together sweep whole token rows. A head's D elements sit in
// one group of D*sizeof(T)/16 lanes ("a row"), so the dot product reduces
// with DPP inside the row and the head's softmax state (max, sum, D
// accumulators) lives in that row. Shares of the whole token space keep
// every CU streaming until the end (a fixed number of keys per workgroup left a partly idle
// second wave of workgroups and many that only found their sequence
// already ended).
// A segment that holds a whole sequence divides by its sum and writes the
// output. Any other segment leaves one partial record per head; the wave
// that finds all segments of its sequence done (flags, below) rescales each
// record to the common maximum, adds, and divides by the common sum, in
// segment order, so results do not change from run to run. The merge runs
// on the CUs that just finished streaming, without a second launch.
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

#include <mutex>

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

// Values every lane of a wave holds alike but the compiler cannot prove so
// (they come out of LDS): taken from lane 0 into scalar registers, so that
// buffer descriptors built from them need no per-lane loop.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

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
__device__ __forceinline__ int block_sum(int x, int* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    __syncthreads();   // earlier readers of red are done
    if (lane == 0) red[wave] = x;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) t += red[w];
    return t;
}

// Record index of segment (w, b), workgroup w's part of sequence b: w + b.
// It is unique. Workgroup ranges and sequences both tile the token space in
// order; if workgroup w+k (k >= 1) reached into sequence b-k, its range
// would start before sequence b-k+1 does, hence before sequence b, while
// workgroup w's range, which ends where w+1's begins, reaches into b.
__device__ __forceinline__ int record_of(int w, int b) { return w + b; }

// The lane's E fp32 outputs converted to the storage type (round to
// nearest even) and packed for one 16-byte store.
template <typename T, int E>
__device__ __forceinline__ u32x4_t pack_row(const float (&x)[E]) {
    u32x4_t r;
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = __builtin_bit_cast(unsigned, x[e]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const unsigned lo = __builtin_bit_cast(unsigned short, (T)x[2 * i]);
            const unsigned hi = __builtin_bit_cast(unsigned short, (T)x[2 * i + 1]);
            r[i] = lo | (hi << 16);
        }
    }
    return r;
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Cache-policy bits of buffer loads and stores on this chip: sc1 makes an
// access coherent at device scope (stores write through the per-XCD L2,
// loads do not take a line another XCD's L2 may have made stale), the same
// encoding the compiler gives device-scope atomic loads and stores.
constexpr int kDeviceScope = 16;

// Partial records move between workgroups that may sit on different XCDs.
// They are written and read with device-scope accesses, so the hand-off
// needs no cache write-back or invalidation (which would be one whole-L2
// operation per wave), only a wait for the writer's stores to complete.
__device__ __forceinline__ void store_record(__amdgpu_buffer_rsrc_t r, int off, f32x4_t x) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x), r, off, 0, kDeviceScope);
}
__device__ __forceinline__ f32x4_t load_record(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kDeviceScope));
}

// Partial merge of sequence b's records for one head over the segments
// first, first + step, ... below ns, in that order: rescale each segment's
// state to the running maximum and add. This lane owns dims E*sub ..
// E*sub+E-1 of head h. Segment s is record w0 + s + b.
template <typename T, int D>
__device__ __forceinline__ void merge_part(const float* __restrict__ ws, int b, int h, int sub, int H, int w0,
                                           int first, int step, int ns, float& M, float& L,
                                           float (&A)[DecCfg<T, D>::E]) {
    constexpr int E = DecCfg<T, D>::E, RF = decode_record_floats(D), PER = kDecodeMergeBatch;
    const int stride = H * RF * 4;   // bytes between consecutive records
    // records w0+b .. w0+b+ns-1, head h; offsets fit 32 bits (checked on the host)
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(ws + (size_t)record_of(w0, b) * H * RF), (short)0, ns * stride, 0x00020000);
    const int base = h * RF * 4;
    for (int s0 = first; s0 < ns; s0 += PER * step) {
        f32x4_t ml[PER], xx[PER][E / 4];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int s = s0 + j * step < ns ? s0 + j * step : s0;   // in range; unused past ns
            const int off = base + s * stride;
            ml[j] = load_record(rr, off);
#pragma unroll
            for (int v = 0; v < E / 4; ++v) xx[j][v] = load_record(rr, off + 4 * (4 + E * sub + 4 * v));
        }
        __builtin_amdgcn_sched_barrier(0);   // every load of the batch in flight first
        float mn = M;
#pragma unroll
        for (int j = 0; j < PER; ++j) mn = fmaxf(mn, ml[j][0]);   // finite: segment s0 exists
        const float a = __builtin_amdgcn_exp2f(M - mn);           // 0 while M is -inf
        L *= a;
#pragma unroll
        for (int e = 0; e < E; ++e) A[e] *= a;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const float wj = s0 + j * step < ns ? __builtin_amdgcn_exp2f(ml[j][0] - mn) : 0.f;
            L = __builtin_fmaf(wj, ml[j][1], L);
#pragma unroll
            for (int e = 0; e < E; ++e) A[e] = __builtin_fmaf(wj, xx[j][e / 4][e % 4], A[e]);
        }
        M = mn;
    }
}

// Workgroups 0 .. kDecodeSplitWGs-1 stream (one per CU): (1) prefix sums
// of the clamped lengths and the zero rows of empty sequences, (2) the
// workgroup's token range and the first sequence in it, (3) per segment and
// head group the streamed dot products and online softmax; a segment that
// holds a whole sequence writes the output rows, any other one writes its
// partial records and (4) raises its flags. The workgroups after them merge:
// each takes (sequence, head group) pairs cut into several segments, its
// waves split the segments, wait for their flags, merge them, and the
// workgroup combines the waves' partial states in LDS.
//
// Hand-off: a segment's wave sets its flag for (segment, head group) to this
// call's tag once its records are complete (device-scope stores, then a wait
// for their completion); the merging wave waits until its segments' flags
// carry the tag, merges, and resets them to zero, so every flag is zero again
// when the kernel ends (a replay with the same tag finds zeros; stale garbage
// matches a tag with odds 2^-64). Streaming workgroups never wait, and
// merging ones wait only for streaming ones, which have lower indices:
// workgroups start in index order, so each one waited for is already running
// or done. The wait is bounded all the same (kDecodeSpinLimit polls); if it
// ever ran out, the rows would be NaN.
template <typename T, int D>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(const T* __restrict__ q, const T* __restrict__ kc,
                                                                const T* __restrict__ vc,
                                                                const int32_t* __restrict__ seqlens,
                                                                T* __restrict__ o, float* __restrict__ ws,
                                                                unsigned long long* __restrict__ flags, int B, int H,
                                                                int S_cap, float c, unsigned long long tag) {
    using C = DecCfg<T, D>;
    constexpr int E = C::E, LPH = C::LPH, HPI = C::HPI, RF = decode_record_floats(D);
    constexpr bool k16 = sizeof(T) == 2;   // bf16 or fp16: packed v_dot2 paths
    __shared__ int red[kDecodeWaves];
    __shared__ int incl_s[kDecodeScanLds];   // inclusive prefix sums of the lengths
    __shared__ int batches_s[kDecodeWaves];  // load batches each wave has started

    const int tid = threadIdx.x, lane = tid & 63, wave = uni(tid >> 6);
    const int w = blockIdx.x;
    const bool scan_in_lds = B <= kDecodeScanLds;

    // (1) prefix sums of the clamped lengths (the token space), one read of seqlens
    int run = 0;
    for (int base = 0; base < B; base += kDecodeThreads) {
        const int bb = base + tid;
        const int len = bb < B ? clamp_len(seqlens[bb], S_cap) : 0;
        int incl = len;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        __syncthreads();
        if (lane == 63) red[wave] = incl;
        __syncthreads();
        int wpre = 0, ctot = 0;
#pragma unroll
        for (int x = 0; x < kDecodeWaves; ++x) {
            ctot += red[x];
            if (x < wave) wpre += red[x];
        }
        if (scan_in_lds && bb < B) incl_s[bb] = incl + wpre + run;
        run += ctot;
    }
    const int Ttot = uni(run);
    __syncthreads();   // incl_s complete
    constexpr int G = kDecodeSplitWGs;   // streaming workgroups
    const int n_groups = (H + HPI - 1) / HPI;
    const int sub = lane % LPH, hl = lane / LPH;

    if (w >= G) {   // uniform: a merging workgroup
        if (Ttot == 0) return;
        __shared__ float part_acc[kDecodeWaves][64 * E];
        __shared__ float part_ml[kDecodeWaves][64][2];
        __shared__ int part_ok[kDecodeWaves];
        const int m = w - G, GM = gridDim.x - G;
        for (int p = m; p < B * n_groups; p += GM) {
            const int b = p / n_groups, grp = p % n_groups;
            int Pb;
            int len;
            if (scan_in_lds) {
                Pb = b > 0 ? incl_s[b - 1] : 0;
                len = (int)(incl_s[b] - Pb);
            } else {
                int t = 0;
                for (int bb = tid; bb < b; bb += kDecodeThreads) t += clamp_len(seqlens[bb], S_cap);
                Pb = block_sum(t, red);
                len = clamp_len(seqlens[b], S_cap);
            }
            Pb = uni(Pb);
            len = uni(len);
            if (len == 0) continue;   // uniform
            const int w0 = decode_range_of(Pb, Ttot), ns = decode_range_of(Pb + len - 1, Ttot) - w0 + 1;
            if (ns == 1) continue;   // uniform: one workgroup held it whole
            // this wave's segments: wave, wave + kDecodeWaves, ...
            bool ready = false;
            for (int spin = 0; spin < kDecodeSpinLimit && !ready; ++spin) {
                bool all = true;
                for (int s0 = wave; s0 < ns; s0 += 64 * kDecodeWaves) {
                    const int s = s0 + kDecodeWaves * lane;
                    const unsigned long long f = __hip_atomic_load(
                        &flags[(size_t)record_of(w0 + (s < ns ? s : s0), b) * H + grp], __ATOMIC_RELAXED,
                        __HIP_MEMORY_SCOPE_AGENT);
                    all = __all(s >= ns || f == tag) && all;
                }
                ready = all;
                if (!ready) __builtin_amdgcn_s_sleep(8);
            }
            const int h = grp * HPI + hl;
            float M = -INFINITY, L = 0.f, A[E];
#pragma unroll
            for (int e = 0; e < E; ++e) A[e] = 0.f;
            if (ready) merge_part<T, D>(ws, b, h < H ? h : 0, sub, H, w0, wave, kDecodeWaves, ns, M, L, A);
            part_ml[wave][lane][0] = M;
            part_ml[wave][lane][1] = L;
#pragma unroll
            for (int e = 0; e < E; ++e) part_acc[wave][lane * E + e] = A[e];
            if (lane == 0) part_ok[wave] = ready;
            __syncthreads();
            if (wave == 0 && h < H) {
                // the waves' partial states, in wave order
                bool ok = true;
                float Mt = -INFINITY;
#pragma unroll
                for (int v = 0; v < kDecodeWaves; ++v) {
                    ok = ok && part_ok[v];
                    Mt = fmaxf(Mt, part_ml[v][lane][0]);   // finite: wave 0 has segment 0
                }
                float Lt = 0.f, out[E];
#pragma unroll
                for (int e = 0; e < E; ++e) out[e] = 0.f;
#pragma unroll
                for (int v = 0; v < kDecodeWaves; ++v) {
                    const float wv = __builtin_amdgcn_exp2f(part_ml[v][lane][0] - Mt);   // 0 for a wave with none
                    Lt = __builtin_fmaf(wv, part_ml[v][lane][1], Lt);
#pragma unroll
                    for (int e = 0; e < E; ++e) out[e] = __builtin_fmaf(wv, part_acc[v][lane * E + e], out[e]);
                }
#pragma unroll
                for (int e = 0; e < E; ++e) out[e] = ok ? out[e] / Lt : __builtin_nanf("");
                *(u32x4_t*)(o + ((size_t)b * H + h) * D + E * sub) = pack_row<T, E>(out);
            }
            for (int s = wave + kDecodeWaves * lane; s < ns; s += 64 * kDecodeWaves)
                __hip_atomic_store(&flags[(size_t)record_of(w0 + s, b) * H + grp], 0ull, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();   // the partial-state LDS is reused by the next pair
        }
        return;
    }

    // a sequence with no keys gives a zero row; workgroup w writes those of
    // sequences w, w + G, ...
    const int n16 = H * D * (int)sizeof(T) / 16;   // 16-byte chunks per sequence's output
    for (int b = w; b < B; b += G) {
        const int len =
            scan_in_lds ? incl_s[b] - (b > 0 ? incl_s[b - 1] : 0) : clamp_len(seqlens[b], S_cap);
        if (len == 0) {   // uniform
            const u32x4_t zero = {0u, 0u, 0u, 0u};
            u32x4_t* out = (u32x4_t*)(o + (size_t)b * H * D);
            for (int i = tid; i < n16; i += kDecodeThreads) out[i] = zero;
        }
    }
    if (Ttot == 0) return;   // uniform
    const int lo = decode_range_start(w, Ttot);
    const int hi = decode_range_start(w + 1, Ttot);
    if (lo >= hi) return;   // uniform

    // (2) first sequence reaching into [lo, hi): the number of sequences
    // that end at or before lo, and where it starts
    int b_first;
    int P;
    if (scan_in_lds) {
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
        int n_before = 0, t_before = 0;
        run = 0;
        for (int base = 0; base < B; base += kDecodeThreads) {
            const int bb = base + tid;
            const int len = bb < B ? clamp_len(seqlens[bb], S_cap) : 0;
            int incl = len;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(incl, o);
                if (lane >= o) incl += y;
            }
            __syncthreads();
            if (lane == 63) red[wave] = incl;
            __syncthreads();
            int wpre = 0, ctot = 0;
#pragma unroll
            for (int x = 0; x < kDecodeWaves; ++x) {
                ctot += red[x];
                if (x < wave) wpre += red[x];
            }
            if (bb < B && incl + wpre + run <= lo) {
                n_before += 1;
                t_before += len;
            }
            run += ctot;
        }
        b_first = (int)block_sum(n_before, red);
        P = block_sum(t_before, red);
    }
    b_first = uni(b_first);
    P = uni(P);

    // (3) one segment per sequence the range touches; each wave streams the
    // keys of its head groups in batches of NB, all loads of a batch in flight
    // together.
    constexpr int NB = kDecodeBatch;
    const int key_bytes = H * D * (int)sizeof(T);
    const int P0 = P;   // where sequence b_first starts
    int last_b = b_first;
    // Waves w and w ^ 4 share a SIMD and stream the same keys for different
    // heads. Issue arbitration favours the older wave: left alone, waves 0-3
    // finished their keys well before waves 4-7, which then streamed on with
    // half the loads in flight per SIMD. So before each batch a wave compares
    // its batch count with its partner's (a relaxed read; a stale value only
    // delays the correction) and, while behind, takes the highest priority.
    static_assert(kDecodeWaves == 8, "waves w and w ^ 4 share a SIMD");
    if (lane == 0) __hip_atomic_store(&batches_s[wave], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __syncthreads();
    int batches = 0;
    for (int b = b_first; b < B && P < hi; ++b) {
        const int len = uni(scan_in_lds ? incl_s[b] - P : clamp_len(seqlens[b], S_cap));
        if (len > 0) {
            last_b = b;
            const int k0 = (lo > P ? lo : P) - P;
            const int k1 = (hi < P + len ? hi : P + len) - P;
            const bool whole = k0 == 0 && k1 == len;   // uniform
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
                for (int kb = k0; kb < k1; kb += NB) {
                    const int partner = uni(
                        __hip_atomic_load(&batches_s[wave ^ 4], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
                    if (batches < partner) __builtin_amdgcn_s_setprio(3);
                    else if (batches > partner) __builtin_amdgcn_s_setprio(0);
                    ++batches;
                    if (lane == 0)
                        __hip_atomic_store(&batches_s[wave], batches, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    u32x4_t kr[NB], vr[NB];
                    // read-once stream: non-temporal, so the loads do not allocate in
                    // the caches (and do not evict whatever is resident there); K
                    // first, so the scores can start while V is still arriving
#pragma unroll
                    for (int it = 0; it < NB; ++it)
                        kr[it] = __builtin_amdgcn_raw_buffer_load_b128(rk, lane_off + (kb + it) * key_bytes, 0,
                                                                       kNonTemporal);
#pragma unroll
                    for (int it = 0; it < NB; ++it)
                        vr[it] = __builtin_amdgcn_raw_buffer_load_b128(rv, lane_off + (kb + it) * key_bytes, 0,
                                                                       kNonTemporal);
                    // keep all 2*NB loads ahead of their first use: left alone, the
                    // scheduler sinks loads toward their uses to save registers and
                    // the batch degenerates to one or two loads in flight
                    __builtin_amdgcn_sched_barrier(0);
                    float s[NB];
#pragma unroll
                    for (int it = 0; it < NB; ++it) {
                        float d = 0.f;
                        if constexpr (k16) {
#pragma unroll
                            for (int x = 0; x < 4; ++x) {
                                // scalar copies first (bit-casting a vector-element lvalue
                                // reads element 0 with this compiler)
                                const unsigned kw = kr[it][x], qw = qx[x];
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
                    // keys past k1 read as zeros (descriptor bound): their
                    // probability is 0 and their V rows add nothing
                    float mx = s[0];
#pragma unroll
                    for (int it = 1; it < NB; ++it) mx = fmaxf(mx, s[it]);
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
                        for (int it = 0; it < NB; it += 2) {
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
                        for (int it = 0; it < NB; ++it) {
                            const float p = __builtin_amdgcn_exp2f(s[it] - m_new);
                            l_run += p;
#pragma unroll
                            for (int e = 0; e < E; ++e) acc[e] = __builtin_fmaf(p, Elem<T>::get(vr[it], e), acc[e]);
                        }
                    }
                }
                if (h_ok) {
                    if (whole) {
                        // the whole sequence in one segment: its output row, with
                        // the merge's arithmetic for one record (acc / l)
                        float out[E];
#pragma unroll
                        for (int e = 0; e < E; ++e) out[e] = acc[e] / l_run;
                        *(u32x4_t*)(o + ((size_t)b * H + h) * D + E * sub) = pack_row<T, E>(out);
                    } else {
                        // one partial record per (segment, h): [max, sum, 0, 0, D accumulators]
                        const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
                            (void*)(ws + (size_t)record_of(w, b) * H * RF), (short)0, H * RF * 4, 0x00020000);
                        const int off = h * RF * 4;
                        if (sub == 0) store_record(rw, off, f32x4_t{m_run, l_run, 0.f, 0.f});
#pragma unroll
                        for (int v = 0; v < E / 4; ++v)
                            store_record(rw, off + 4 * (4 + E * sub + 4 * v),
                                         f32x4_t{acc[4 * v], acc[4 * v + 1], acc[4 * v + 2], acc[4 * v + 3]});
                    }
                }
            }
        }
        P += len;
    }
    __builtin_amdgcn_s_setprio(0);

    // (4) flags. Only the first and the last segment of the range can be
    // part of a longer sequence: the first when that sequence starts before
    // lo, the last when it runs past hi.
    const bool first_cut = P0 < lo;   // sequence b_first starts before the range
    const bool last_cut = P > hi;     // sequence last_b runs past it
    if (!first_cut && !last_cut) return;   // uniform: every segment was whole
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's records are complete
    if (lane == 0) {
        for (int grp = wave; grp < n_groups; grp += kDecodeWaves) {
            if (first_cut)
                __hip_atomic_store(&flags[(size_t)record_of(w, b_first) * H + grp], tag, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            if (last_cut && !(last_b == b_first && first_cut))
                __hip_atomic_store(&flags[(size_t)record_of(w, last_b) * H + grp], tag, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <typename T, int D>
hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
    char* ws = (char*)a.workspace;
    unsigned long long* flags = (unsigned long long*)(ws + decode_records_bytes(a.B, a.H, a.D));
    // merging workgroups: one per (sequence, head group) pair, at most kDecodeMergeWGs
    const long long pairs = (long long)a.B * ((a.H + DecCfg<T, D>::HPI - 1) / DecCfg<T, D>::HPI);
    const unsigned grid = kDecodeSplitWGs + (unsigned)(pairs < kDecodeMergeWGs ? pairs : kDecodeMergeWGs);
    if (a.ev_start || a.ev_stop)   // timed: events on the kernel itself
        hipExtLaunchKernelGGL((decode_kernel<T, D>), dim3(grid), dim3(kDecodeThreads), 0, stream,
                              a.ev_start, a.ev_stop, 0, (const T*)a.q, (const T*)a.kcache, (const T*)a.vcache,
                              a.seqlens, (T*)a.o, (float*)ws, flags, a.B, a.H, a.S_cap, a.scale_log2, a.tag);
    else   // the plain launch, which stream capture records
        hipLaunchKernelGGL((decode_kernel<T, D>), dim3(grid), dim3(kDecodeThreads), 0, stream,
                           (const T*)a.q, (const T*)a.kcache, (const T*)a.vcache, a.seqlens, (T*)a.o, (float*)ws,
                           flags, a.B, a.H, a.S_cap, a.scale_log2, a.tag);
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

// The allocation-free decode's workspace: a file-scope device array, one copy
// per GPU the library runs on, held until the process ends. It starts zeroed
// (the flags' idle state) and every call leaves its flags zero again. In host
// code the array's name is not a device address: the address comes from
// hipGetSymbolAddress, taken once per device with that device current.
namespace {
__device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // per device, set once under the mutex
}  // namespace

hipError_t decode_scratch(void** ptr) {
    *ptr = nullptr;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace attn
