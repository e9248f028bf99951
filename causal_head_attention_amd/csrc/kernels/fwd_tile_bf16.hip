// fwd_tile_bf16.hip -- fused causal attention forward on gfx950 matrix cores.
//
// One workgroup (8 waves) owns one (b, h, block of 128 queries); with the
// causal mask it owns two blocks, r and n-1-r, run one after the other so
// every workgroup walks the same number of KV tiles. For each 64-key tile:
//
//   K tile  : HBM -> registers -> LDS  (row-major, 16-byte chunks XOR-swizzled)
//   V tile  : HBM -> registers -> transposed in registers -> LDS as V^T
//   S^T     = K . Q^T            v_mfma_f32_32x32x16_bf16, fp32 accumulate
//   mask    : only on tiles that cross the diagonal or the ragged key end
//   softmax : online (running max, running sum) in fp32, base-2 exponent
//   O^T    += V^T . P^T          v_mfma_f32_32x32x16_bf16, P rounded to bf16
//
// and the next tile's HBM loads are in flight while the current one is
// computed (double-buffered LDS, one barrier per tile). The score matrix
// never leaves registers.
//
// Method: fused QK^T + mask + softmax + P.V with the score row kept on chip
// and K tiles staged in shared memory ("Hand-written Masked Multi-Head
// Attention CUDA kernel" page, sections 2.1-2.2 and 3); the online softmax
// recurrence m' = max(m, x), l' = l*exp(m-m') + exp(x-m') and the -inf
// mask ("Week-4 CUDA notes" page, section 2.2); skipping the masked half of
// the score matrix instead of computing it (MMHA page, section 1) and
// per-thread key bounds instead of per-element branches (MMHA page,
// section 2.3); fp32 arithmetic on half-width storage (MMHA page,
// section 3.3); prefetching the next K tile (MMHA page, section 4.2).
//
// Why S^T and O^T rather than S and O. In the 32x32 MFMA result a lane
// holds one COLUMN n = lane%32 and 16 rows m = 8*(r/4) + 4*(lane/32) + r%4
// (register r). Computing S^T = K Q^T puts one query per lane (the column)
// and its keys in registers, so the row max and row sum need only one
// exchange between lanes l and l^32, and the probabilities already sit where
// the B operand of O^T = V^T P^T wants them (B lane l holds column n =
// lane%32 and 8 consecutive K-indices). O^T keeps one query per lane too, so
// the rescale by exp(m_old - m_new) is a per-lane scalar.
//
// Key order inside a 32-key block. The A-operand row a lane loads for S^T is
// key swap_bits23(lane%32); with that permutation register r of half g holds
// key 16*(r/8) + 8*g + (r%8), so registers 8s..8s+7 are 8 consecutive keys:
// exactly one 16-byte V^T chunk for the P.V step. (The contraction index
// order inside an MFMA only has to agree between A and B, which it does by
// construction: both sides use chunk 2*ks + g of head_dim, and keys
// 16*s + 8*g .. +7 for P.V.)
#include <hip/hip_runtime.h>

#include "../launch.h"
#include "../plan.h"

namespace attn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int swap_bits23(int x) {
    return (x & ~0xC) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Byte offset of 16-byte chunk `ch` of K-tile row `row` (D/8 chunks per row).
// The XOR makes the 32 lanes that read one chunk column (rows
// swap_bits23(lane)) hit 32 different chunk positions.
template <int D>
__device__ __forceinline__ int k_lds_off(int row, int ch) {
    constexpr int KCH = D / 8;
    return row * (D * 2) + 16 * (ch ^ (swap_bits23(row & 31) % KCH));
}

// Byte offset of element (d, key) of the V^T tile (64 keys = 8 chunks per row).
__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }
__device__ __forceinline__ int vt_lds_off(int d, int key) {
    return d * 128 + 16 * ((key >> 3) ^ vt_swz(d)) + 2 * (key & 7);
}

__device__ __forceinline__ unsigned half_of(u32x4_t x, int e) {
    // bf16 element e (0..7) of a 16-byte vector
    return (x[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
}

template <int D>
struct TileCfg {
    static constexpr int KCH = D / 8;            // 16-byte chunks per K row
    static constexpr int KS = D / 16;            // MFMA k-steps for S^T
    static constexpr int DB = D / 32;            // 32-row blocks of O^T
    static constexpr int KR = D / 32;            // keys per V-transposer thread
    static constexpr int NPRE = D / 32;          // 16-byte prefetch registers per thread
    static constexpr int K_BYTES = kTileN * D * 2;
    static constexpr int STAGE = 2 * K_BYTES;    // K tile + V^T tile
    static constexpr int LDS = tile_lds_bytes(D);
};

// Issue the HBM loads of KV tile `tile0` into registers.
// Waves 0-3 load K (row-major 16-byte chunks), waves 4-7 load V (KR keys x
// 8 head dims each, to be transposed).
template <int D>
__device__ __forceinline__ void load_tile(u32x4_t (&pre)[TileCfg<D>::NPRE], const __bf16* __restrict__ K,
                                          const __bf16* __restrict__ V, int b, int h, int H, int S_kv,
                                          int tile0, int tid) {
    using C = TileCfg<D>;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    if (tid < 256) {
#pragma unroll
        for (int it = 0; it < C::NPRE; ++it) {
            const int ci = tid + 256 * it;
            const int row = ci / C::KCH, ch = ci % C::KCH;
            const int key = tile0 + row;
            pre[it] = zero;
            if (key < S_kv)
                pre[it] = *(const u32x4_t*)(K + ((size_t)((size_t)b * S_kv + key) * H + h) * D + 8 * ch);
        }
    } else {
        const int u = tid - 256;
        const int c8 = u % (D / 8), kq = u / (D / 8);
#pragma unroll
        for (int kk = 0; kk < C::KR; ++kk) {
            const int key = tile0 + kq * C::KR + kk;
            pre[kk] = zero;
            if (key < S_kv)
                pre[kk] = *(const u32x4_t*)(V + ((size_t)((size_t)b * S_kv + key) * H + h) * D + 8 * c8);
        }
    }
}

// Write the prefetched registers of one tile into LDS stage `stage`.
template <int D>
__device__ __forceinline__ void store_tile(const u32x4_t (&pre)[TileCfg<D>::NPRE], char* stage, int tid) {
    using C = TileCfg<D>;
    if (tid < 256) {
#pragma unroll
        for (int it = 0; it < C::NPRE; ++it) {
            const int ci = tid + 256 * it;
            const int row = ci / C::KCH, ch = ci % C::KCH;
            *(u32x4_t*)(stage + k_lds_off<D>(row, ch)) = pre[it];
        }
    } else {
        char* vt = stage + C::K_BYTES;
        const int u = tid - 256;
        const int c8 = u % (D / 8), kq = u / (D / 8);
        const int key0 = kq * C::KR;
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
            const int d = 8 * c8 + dd;
            char* dst = vt + vt_lds_off(d, key0);
            if constexpr (C::KR == 4) {
                u32x2_t w;
                w[0] = half_of(pre[0], dd) | (half_of(pre[1], dd) << 16);
                w[1] = half_of(pre[2], dd) | (half_of(pre[3], dd) << 16);
                *(u32x2_t*)dst = w;
            } else if constexpr (C::KR == 2) {
                *(unsigned*)dst = half_of(pre[0], dd) | (half_of(pre[1], dd) << 16);
            } else {
                *(unsigned short*)dst = (unsigned short)half_of(pre[0], dd);
            }
        }
    }
}

template <int D>
__global__ __launch_bounds__(kTileThreads) void fwd_tile_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, int B, int H, int S_q, int S_kv, int causal, float c /* scale*log2e */,
    int n_qblk, int items_per_bh, int paired) {
    using C = TileCfg<D>;
    __shared__ __attribute__((aligned(16))) char lds[C::LDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int wq = wave & 3;     // query sub-block of this wave
    const int half = wave >> 2;  // key half of every tile
    const int off = S_kv - S_q;  // absolute position of query i is i + off

    const int item = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = item / items_per_bh;
    const int p = item % items_per_bh;
    const int b = bh / H, h = bh % H;
    const int qb_first = n_qblk - 1 - p;
    const int nphase = (paired && p != qb_first) ? 2 : 1;

    for (int phase = 0; phase < nphase; ++phase) {
        const int qb = phase == 0 ? qb_first : p;
        const int nt = tiles_for_block(qb, S_q, S_kv, causal);
        const int q0 = qb * kTileM + 32 * wq;      // first query of this wave
        const int qi = q0 + l32;                   // this lane's query
        const bool wave_has_rows = q0 < S_q;
        const int q_last = (q0 + 31 < S_q ? q0 + 31 : S_q - 1);
        const int key_last = causal ? q_last + off : S_kv - 1;   // last key any row of the wave sees
        const int lane_key_limit = causal ? qi + off : S_kv - 1; // last key this lane sees

        // Q^T fragments (B operand): lane holds query qi, head dims 16*ks + 8*g .. +7.
        bf16x8_t qf[C::KS];
        {
            const bool ok = qi < S_q;
            const __bf16* qrow = Q + ((size_t)((size_t)b * S_q + (ok ? qi : 0)) * H + h) * D;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                u32x4_t x = {0u, 0u, 0u, 0u};
                if (ok) x = *(const u32x4_t*)(qrow + 16 * ks + 8 * g);
                qf[ks] = __builtin_bit_cast(bf16x8_t, x);
            }
        }

        f32x16_t acc[C::DB];
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
        float m_run = -INFINITY;   // running max of (score * c) for query qi
        float l_run = 0.f;         // this lane's share of the running sum

        u32x4_t pre[C::NPRE];
        load_tile<D>(pre, K, V, b, h, H, S_kv, 0, tid);
        store_tile<D>(pre, lds, tid);
        __syncthreads();

        for (int t = 0; t < nt; ++t) {
            const bool more = t + 1 < nt;
            if (more) load_tile<D>(pre, K, V, b, h, H, S_kv, (t + 1) * kTileN, tid);

            const char* stage = lds + (t & 1) * C::STAGE;
            const int kb_local = 32 * half;
            const int kbase = t * kTileN + kb_local;   // first key of this wave's half tile
            if (wave_has_rows && kbase <= key_last && kbase < S_kv) {
                // ---- S^T = K . Q^T over this wave's 32 keys x 32 queries
                f32x16_t s;
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] = 0.f;
                const char* krow = stage + (kb_local + swap_bits23(l32)) * (D * 2);
#pragma unroll
                for (int ks = 0; ks < C::KS; ++ks) {
                    const bf16x8_t a = *(const bf16x8_t*)(krow + 16 * ((2 * ks + g) ^ (l32 % C::KCH)));
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
                }
                // ---- mask: only where the tile crosses the diagonal or the key end
                const bool need_mask = (causal && kbase + 31 > q0 + off) || (kbase + 32 > S_kv);
                if (need_mask) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kbase + 16 * (r >> 3) + 8 * g + (r & 7);
                        if (key > lane_key_limit || key >= S_kv) s[r] = -INFINITY;
                    }
                }
                // ---- online softmax (base 2: exp(x*scale) = 2^(x*scale*log2 e))
                float mx = s[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float m_new = fmaxf(m_run, mx * c);
                const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
                float pr[16];
                float rs = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m_use));
                    rs += pr[r];
                }
                l_run = l_run * alpha + rs;
                m_run = m_new;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
                bf16x8_t pb[2];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                    for (int i = 0; i < 8; ++i) pb[s2][i] = (__bf16)pr[8 * s2 + i];
                // ---- O^T += V^T . P^T
                const char* vt = stage + C::K_BYTES;
#pragma unroll
                for (int db = 0; db < C::DB; ++db) {
                    const int d = 32 * db + l32;
                    const char* vrow = vt + d * 128;
                    const int sw = vt_swz(d);
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        const bf16x8_t a = *(const bf16x8_t*)(vrow + 16 * ((4 * half + 2 * s2 + g) ^ sw));
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[s2], acc[db], 0, 0, 0);
                    }
                }
            }
            if (more) store_tile<D>(pre, lds + ((t + 1) & 1) * C::STAGE, tid);
            __syncthreads();
        }

        // ---- merge the two key halves (waves wq and wq+4) through LDS
        float* xf = (float*)lds;
        float* slot = xf + wq * (64 * (C::DB * 16 + 2));
        if (half == 1) {
            slot[lane] = m_run;
            slot[64 + lane] = l_run;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) slot[128 + (db * 16 + r) * 64 + lane] = acc[db][r];
        }
        __syncthreads();
        if (half == 0 && wave_has_rows) {
            const float m1 = slot[lane];
            const float l1 = slot[64 + lane];
            const float m = fmaxf(m_run, m1);
            const float mu = (m == -INFINITY) ? 0.f : m;
            const float a0 = __builtin_amdgcn_exp2f(m_run - mu);
            const float a1 = __builtin_amdgcn_exp2f(m1 - mu);
            float l = a0 * l_run + a1 * l1;
            l += __shfl_xor(l, 32);
            const float inv = 1.0f / l;
            if (qi < S_q) {
                __bf16* orow = O + ((size_t)((size_t)b * S_q + qi) * H + h) * D;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        __bf16 ob[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 4 * j + e;
                            const float x1 = slot[128 + (db * 16 + r) * 64 + lane];
                            ob[e] = (__bf16)((a0 * acc[db][r] + a1 * x1) * inv);
                        }
                        // lane holds head dims 32*db + 8*j + 4*g .. +3 of its query
                        *(u32x2_t*)(orow + 32 * db + 8 * j + 4 * g) = __builtin_bit_cast(u32x2_t, ob);
                    }
            }
        }
        __syncthreads();
    }
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
    const TileGrid tg = tile_grid(a.B, a.H, a.S_q, a.causal);
    hipLaunchKernelGGL(fwd_tile_bf16_kernel<D>, dim3((unsigned)tg.n_items), dim3(kTileThreads), 0, stream,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o, a.B, a.H,
                       a.S_q, a.S_kv, a.causal, a.scale_log2, tg.n_qblk, tg.items_per_bh, tg.paired);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_tile_bf16(const FwdArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 32: return launch_d<32>(a, stream);
        case 64: return launch_d<64>(a, stream);
        case 128: return launch_d<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
