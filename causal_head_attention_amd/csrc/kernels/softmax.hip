// softmax.hip -- standalone row softmax of a score matrix under the causal rule.
//
// p[i][j] = exp(scale*s[i][j] - m_i) / sum_j' exp(scale*s[i][j'] - m_i) over
// the keys row i may see (j <= i + S_kv - S_q when causal), 0 elsewhere.
//
// A generic softmax reads, exponentiates and normalises every entry of a
// causal score matrix although the upper triangle is masked ("Hand-written
// Masked Multi-Head Attention CUDA kernel" page, section 1); here the masked
// entries are not read or exponentiated, only written as 0 (the -inf mask of
// the "Week-4 CUDA notes" page, section 2.2, taken to its end; at most the
// rest of the 16-byte chunk holding a row's last visible score is fetched,
// and never used). One wave owns one row: lane t holds 16-byte chunks t,
// t + 64, ... of the visible part in registers, the row maximum and the sum
// of exponentials are reduced with cross-lane shuffles (no LDS, no barrier),
// and the whole row is written back in 16-byte stores, the all-zero chunks
// before the loads complete. The score matrix is read once and the
// probabilities written once: the kernel is bound by HBM (a plain streaming
// kernel with the same one-to-two read/write mix is the practical ceiling).
#include <hip/hip_runtime.h>

#include "../launch.h"
#include "../plan.h"

namespace attn {
namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kNonTemporal = 2;   // buffer-load cache policy: nt

template <typename T>
struct Chunk;   // 16 bytes of T <-> floats
template <>
struct Chunk<float> {
    static constexpr int E = 4;
    __device__ static void unpack(const u32x4_t& c, float (&x)[E]) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const unsigned u = c[e];
            x[e] = __builtin_bit_cast(float, u);
        }
    }
    __device__ static u32x4_t pack(const float (&x)[E]) {
        u32x4_t c;
#pragma unroll
        for (int e = 0; e < E; ++e) c[e] = __builtin_bit_cast(unsigned, x[e]);
        return c;
    }
};
template <typename H16>
struct Chunk16 {
    static constexpr int E = 8;
    __device__ static void unpack(const u32x4_t& c, float (&x)[E]) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const unsigned w = c[e >> 1];
            x[e] = (float)__builtin_bit_cast(H16, (unsigned short)(w >> (16 * (e & 1))));
        }
    }
    __device__ static u32x4_t pack(const float (&x)[E]) {
        u32x4_t c;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const unsigned lo = __builtin_bit_cast(unsigned short, (H16)x[2 * k]);
            const unsigned hi = __builtin_bit_cast(unsigned short, (H16)x[2 * k + 1]);
            c[k] = lo | (hi << 16);
        }
        return c;
    }
};
template <>
struct Chunk<__bf16> : Chunk16<__bf16> {};
template <>
struct Chunk<_Float16> : Chunk16<_Float16> {};

template <typename T, int NC>   // NC: 16-byte chunks per lane (row <= 64 * NC chunks)
__global__ __launch_bounds__(kSmThreads) void masked_softmax_kernel(const T* s, T* p, long long rows, int S_q,
                                                                    int S_kv, float scale_log2, int causal) {
    using C = Chunk<T>;
    constexpr int E = C::E;
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * kSmRowsPerBlock + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int i = (int)(row % S_q);
    int n = causal ? i + (S_kv - S_q) + 1 : S_kv;   // visible keys 0 .. n-1
    n = n < 0 ? 0 : (n > S_kv ? S_kv : n);
    // descriptors over this row; the input one ends at the end of the chunk
    // that holds the last visible key, so masked scores past that chunk are
    // never fetched (a 16-byte load that crosses a descriptor's end comes
    // back zero-filled, so the end must not split a chunk; the few masked
    // entries of the last chunk are replaced by -inf below)
    const int in_bytes = (n * (int)sizeof(T) + 15) & ~15;   // <= the row: a whole number of chunks
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(s + (size_t)row * S_kv), (short)0, in_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p + (size_t)row * S_kv), (short)0, S_kv * (int)sizeof(T), 0x00020000);
    const int n_chunks = S_kv / E;   // the row is a whole number of chunks (host-checked)

    // chunks past the last visible key hold zeros only: store them first,
    // so these writes overlap the loads below
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < NC; ++k) {
        const int c = lane + 64 * k;
        if (c >= n_chunks) break;
        if (c * E >= n) __builtin_amdgcn_raw_buffer_store_b128(zero, rp, c * 16, 0, 0);
    }

    // the scores are read once: non-temporal loads (cache policy nt) keep
    // them from displacing the probabilities being written in L2
    float x[NC][E];
    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
        const int c = lane + 64 * k;
        u32x4_t raw = {0u, 0u, 0u, 0u};
        if (c * E < n) raw = __builtin_amdgcn_raw_buffer_load_b128(rs, c * 16, 0, kNonTemporal);
        C::unpack(raw, x[k]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            // scores in base-2 units; masked and absent keys at -inf
            x[k][e] = (c * E + e < n) ? x[k][e] * scale_log2 : -INFINITY;
            m = fmaxf(m, x[k][e]);
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float mu = (m == -INFINITY) ? 0.f : m;   // a row with no visible key stays 0
    float l = 0.f;
#pragma unroll
    for (int k = 0; k < NC; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e) {
            x[k][e] = __builtin_amdgcn_exp2f(x[k][e] - mu);   // exactly 0 where masked
            l += x[k][e];
        }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
    const float inv = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
        const int c = lane + 64 * k;
        if (c >= n_chunks) break;
        if (c * E >= n) continue;   // stored as zeros above
#pragma unroll
        for (int e = 0; e < E; ++e) x[k][e] *= inv;
        __builtin_amdgcn_raw_buffer_store_b128(C::pack(x[k]), rp, c * 16, 0, 0);
    }
}

template <typename T, int NC>
hipError_t launch_nc(const SoftmaxArgs& a, hipStream_t stream) {
    const long long rows = (long long)a.B * a.H * a.S_q;
    const unsigned grid = (unsigned)((rows + kSmRowsPerBlock - 1) / kSmRowsPerBlock);
    hipExtLaunchKernelGGL((masked_softmax_kernel<T, NC>), dim3(grid), dim3(kSmThreads), 0, stream, a.ev_start,
                          a.ev_stop, 0, (const T*)a.s, (T*)a.p, rows, a.S_q, a.S_kv, a.scale_log2, a.causal);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const SoftmaxArgs& a, hipStream_t stream) {
    const long long row_bytes = (long long)a.S_kv * (long long)sizeof(T);
    if (row_bytes <= 64LL * 16 * kSmChunksSmall) return launch_nc<T, kSmChunksSmall>(a, stream);
    return launch_nc<T, kSmChunksMax>(a, stream);
}

}  // namespace

hipError_t launch_masked_softmax(const SoftmaxArgs& a, Elt t, hipStream_t stream) {
    switch (t) {
        case Elt::F32: return launch_t<float>(a, stream);
        case Elt::BF16: return launch_t<__bf16>(a, stream);
        case Elt::F16: return launch_t<_Float16>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace attn
