// fwd_f32.hip -- fp32 attention forward on the fp32 matrix cores of gfx950.
//
// O = softmax(scale * Q K^T + M) V for fp32 Q, K, V, O, both contractions on
// v_mfma_f32_32x32x2_f32 (fp32 products, fp32 accumulation: full single
// precision, no reduced-precision inputs). Definition: "Hand-written Masked
// Multi-Head Attention CUDA kernel" page, section 2 (scores, causal mask,
// softmax, weighted sum of V); online softmax with running max and sum and
// the -inf mask: "Week-4 CUDA notes" page, section 2.2; fp32 accumulation:
// MMHA page, section 3.3.
//
// One workgroup owns 32 queries of one (b, h). Its 8 waves (2 per SIMD) take
// the block's 32-key tiles round-robin, each keeping its own running max,
// running sum and O^T accumulator for the 32 queries; the eight partial
// states are merged through LDS at the end (the common-normaliser merge of
// the Week-4 page, section 2.2). Per tile a wave computes
//   S^T (32 keys x 32 queries) = K . Q^T     D/2 MFMAs, k = 2 head dims each
//   O^T (D x 32 queries)      += V^T . P^T   16 * D/32 MFMAs, k = 2 keys each
// Lane l owns query l % 32 and, of each 32-row output block, rows
// 8*(r/4) + 4*(l/32) + r%4 (register r). The contraction order is free as
// long as both operands follow it:
//   * over head dims, k-step 4m+e gives lane half g the dim 8m + 4g + e, so
//     a lane's K row and Q row come in 16-byte loads (dims 8m+4g .. +3)
//     straight from global memory into MFMA operands, no LDS;
//   * over keys, k-step j gives lane half g the key 8*(j/4) + 4g + j%4 --
//     exactly the key of register j of the S^T accumulator, so P is used in
//     place (never rounded, never moved) and V^T's operand is one 4-byte
//     load: lanes 0-31 read 32 consecutive dims of one V row.
// All global reads go through buffer descriptors that end at the valid rows,
// so rows past S_q or past the entry's S_kv read as 0 (and their scores are
// masked to -inf).
#include <hip/hip_runtime.h>

#include "../launch.h"
#include "../plan.h"

namespace attn {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Descriptor over rows [0, rows) of one head of a [B, S, H, D] fp32 tensor
// whose entry b starts at row b * S_rows (byte offsets row * H * D * 4 + 4d).
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const float* base, int b, int h, int S_rows, int rows,
                                                           int H) {
    const float* p = base + ((size_t)b * S_rows * H + h) * D;
    const int bytes = rows > 0 ? ((rows - 1) * H * D + D) * 4 : 0;
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, bytes, 0x00020000);
}

template <int D, bool KMASK>
__global__ __launch_bounds__(kF32Threads) void fwd_f32_kernel(const float* __restrict__ Q,
                                                             const float* __restrict__ K,
                                                             const float* __restrict__ V, float* __restrict__ O,
                                                             int H, int S_q, int S_cap, int causal, float c,
                                                             int n_qblk, const int32_t* __restrict__ kv_lens,
                                                             float* __restrict__ lse,
                                                             const uint8_t* __restrict__ key_mask) {
    constexpr int NF4 = D / 8;   // 16-byte pieces of a lane's K or Q row (dims 8m + 4g .. +3)
    constexpr int DB = D / 32;   // 32-row blocks of O^T
    constexpr int W = kF32Threads / 64;
    // merge slots: per wave and lane, m, l and the DB*16 accumulator registers,
    // at an odd stride so that lanes writing one register, and the threads of
    // the final pass reading consecutive dims, fall in distinct banks
    constexpr int SL = 2 + DB * 16 + 1;
    __shared__ __attribute__((aligned(16))) float xs[W * 64 * SL];
    __shared__ float wts[kF32Q][W];   // per query: each wave's merge weight, already divided by the sum

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;

    // (b, h, 32-query block); the blocks of one head are contiguous per XCD,
    // so they find its K and V rows in one L2
    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int qb = item % n_qblk, bh = item / n_qblk;
    const int h = bh % H, b = bh / H;
    const int S_kv = kv_lens ? min(max(kv_lens[b], 0), S_cap) : S_cap;
    const int off = S_kv - S_q;   // bottom-right alignment of the causal rule
    const int q0 = qb * kF32Q;
    const int qi = q0 + l32;      // this lane's query
    // keys [0, lane_end) are visible to this lane's query; [0, kend) to some
    // query of the block
    const int lane_end = qi >= S_q ? 0 : (causal ? min(S_kv, max(0, qi + 1 + off)) : S_kv);
    const int q_last = min(q0 + kF32Q - 1, S_q - 1);
    const int kend = causal ? min(S_kv, max(0, q_last + 1 + off)) : S_kv;
    const int ntiles = (kend + kF32N - 1) / kF32N;

    const __amdgpu_buffer_rsrc_t rq = head_rsrc<D>(Q, b, h, S_q, S_q, H);
    const __amdgpu_buffer_rsrc_t rk = head_rsrc<D>(K, b, h, S_cap, S_kv, H);
    const __amdgpu_buffer_rsrc_t rv = head_rsrc<D>(V, b, h, S_cap, S_kv, H);
    const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(KMASK ? key_mask + (size_t)b * S_cap : key_mask), (short)0, KMASK ? S_kv : 0, 0x00020000);
    const int row_bytes = H * D * 4;

    // Q^T operand: this lane's query row, dims 8m + 4g .. +3 for k-steps 4m .. 4m+3
    f32x4_t qf[NF4];
#pragma unroll
    for (int m = 0; m < NF4; ++m)
        qf[m] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                rq, qi * row_bytes + (8 * m + 4 * g) * 4, 0, 0));

    f32x16_t acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
    float m_run = -INFINITY;   // running max of score * c for query qi
    float l_run = 0.f;         // this lane's share of the running sum (its 16 keys per tile)

    // one tile's operands: the K rows (dims as in qf), the V^T operands of
    // the 16 key steps of each O^T block, and the key-mask bytes
    struct TileOps {
        f32x4_t k[NF4];
        float v[DB][16];
        unsigned mb[16];
    };
    auto load_tile = [&](int t, TileOps& x) {
        const int k0 = t * kF32N;
#pragma unroll
        for (int m = 0; m < NF4; ++m)
            x.k[m] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rk, (k0 + l32) * row_bytes + (8 * m + 4 * g) * 4, 0, 0));
        // V^T operand of key step j of block db: key k0 + 8*(j/4) + 4g + j%4, dim 32*db + l32
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int key = k0 + 8 * (j >> 2) + 4 * g + (j & 3);
                x.v[db][j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                           rv, key * row_bytes + (32 * db + l32) * 4, 0, 0));
            }
        if constexpr (KMASK) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                x.mb[r] = __builtin_amdgcn_raw_buffer_load_b8(rm, k0 + 8 * (r >> 2) + 4 * g + (r & 3), 0, 0);
        }
    };
    // where the registers hold two tiles (D = 32; D = 64 without the mask
    // bytes) the next tile's operands load while this one computes
    constexpr bool kPrefetch = D <= 32 || (D <= 64 && !KMASK);
    TileOps cur, nxt;
    if (wave < ntiles) load_tile(wave, cur);   // in flight with the Q loads

    for (int t = wave; t < ntiles; t += W) {
        const int k0 = t * kF32N;
        if constexpr (kPrefetch) {
            if (t + W < ntiles) load_tile(t + W, nxt);
        } else {
            if (t != wave) load_tile(t, cur);
        }
        const f32x4_t (&kf)[NF4] = cur.k;
        const unsigned (&mb)[16] = cur.mb;
        f32x16_t s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int m = 0; m < NF4; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float kv = kf[m][e], qv = qf[m][e];
                s = mfma_f32(kv, qv, s);
            }

        // scores in base-2 units; hidden keys at -inf
        float x[16];
        float mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + 8 * (r >> 2) + 4 * g + (r & 3);
            bool hide = key >= lane_end;
            if constexpr (KMASK) hide = hide || mb[r] == 0u;
            const float sr = s[r];
            x[r] = hide ? -INFINITY : sr * c;
            mt = fmaxf(mt, x[r]);
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));   // the other 16 keys of the query sit in lane l ^ 32
        const float m_new = fmaxf(m_run, mt);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            x[r] = __builtin_amdgcn_exp2f(x[r] - m_use);   // exactly 0 where hidden
            ls += x[r];
        }
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;

        // O^T += V^T . P^T; k-step j: key k0 + 8*(j/4) + 4g + j%4, dim 32*db + l32
        // (the key of mask byte j: a hidden key's V is replaced by 0, so
        // whatever its padding slot holds never reaches the sum)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                float vj = cur.v[db][j];
                if constexpr (KMASK) vj = mb[j] == 0u ? 0.f : vj;
                acc[db] = mfma_f32(vj, x[j], acc[db]);
            }
        if constexpr (kPrefetch) cur = nxt;
    }

    // ---- merge the eight waves' states
    float* slot = xs + (wave * 64 + lane) * SL;
    slot[0] = m_run;
    slot[1] = l_run;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) slot[2 + db * 16 + r] = acc[db][r];
    __syncthreads();

    // per query: the common maximum M, the waves' weights 2^(m_w - M) / L
    // with L the total sum, and the log-sum-exp
    if (tid < kF32Q) {
        const int qq = tid;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, xs[(w * 64 + qq) * SL]);
        const float mu = M == -INFINITY ? 0.f : M;
        float a[W], L = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float* sw = xs + w * 64 * SL;
            a[w] = __builtin_amdgcn_exp2f(sw[qq * SL] - mu);   // 0 for a wave that saw no key
            L += a[w] * (sw[qq * SL + 1] + sw[(qq + 32) * SL + 1]);
        }
        // a row that sees no key (a KV-cache entry shorter than the chunk) is 0
        const float inv = L > 0.f ? 1.0f / L : 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) wts[qq][w] = a[w] * inv;
        // log of the softmax denominator, natural units: ln 2 * (M + log2 L)
        if (lse && q0 + qq < S_q)
            lse[((size_t)b * H + h) * S_q + q0 + qq] =
                L > 0.f ? (M + __builtin_log2f(L)) * 0.69314718055994531f : -INFINITY;
    }
    __syncthreads();

    // output (query qq, dim d): lane qq + 32 * ((d % 32) / 4 % 2), register
    // 4 * ((d % 32) / 8) + d % 4 of block d / 32; consecutive threads take
    // consecutive dims so the stores coalesce
    for (int idx = tid; idx < kF32Q * D; idx += kF32Threads) {
        const int qq = idx / D, d = idx % D;
        if (q0 + qq >= S_q) break;   // idx grows with qq: every later index is past S_q too
        const int dd = d & 31;
        const int ln = qq + 32 * ((dd >> 2) & 1);
        const int reg = (d >> 5) * 16 + 4 * (dd >> 3) + (dd & 3);
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) o = __builtin_fmaf(wts[qq][w], xs[(w * 64 + ln) * SL + 2 + reg], o);
        O[((size_t)((size_t)b * S_q + q0 + qq) * H + h) * D + d] = o;
    }
}

template <int D, bool KMASK>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
    const int n_qblk = (a.S_q + kF32Q - 1) / kF32Q;
    const unsigned grid = (unsigned)((long long)a.B * a.H * n_qblk);
    hipExtLaunchKernelGGL((fwd_f32_kernel<D, KMASK>), dim3(grid), dim3(kF32Threads), 0, stream, a.ev_start,
                          a.ev_stop, 0, (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.H,
                          a.S_q, a.S_kv, a.causal, a.scale_log2, n_qblk, a.kv_lens, a.lse, a.key_mask);
    return hipGetLastError();
}

template <bool KMASK>
hipError_t launch_m(const FwdArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 32: return launch_d<32, KMASK>(a, stream);
        case 64: return launch_d<64, KMASK>(a, stream);
        case 128: return launch_d<128, KMASK>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
    return a.key_mask ? launch_m<true>(a, stream) : launch_m<false>(a, stream);
}

}  // namespace attn
