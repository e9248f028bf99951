// fwd_tile.hip -- fused causal attention forward on gfx950 matrix cores
// (bf16 or fp16 storage, fp32 arithmetic).
//
// One workgroup (8 waves) owns two blocks of 128 queries of one (b, h), r
// and n-1-r, run one after the other: with the causal mask every workgroup
// then walks the same number of KV tiles, and without it each pays the fixed
// costs of a block once for two (with per-entry cache lengths, one block per
// workgroup). Per 64-key tile:
//
//   K tile  : HBM -> registers -> LDS  (row-major, rows padded by 16 bytes)
//   V tile  : HBM -> registers -> LDS (key rows, as loaded); the P.V
//             operands V^T come from transposing LDS reads (ds_read_b64_tr_b16)
//   S^T     = K . Q^T            v_mfma_f32_32x32x16_bf16, fp32 accumulate
//   mask    : on tiles that cross the diagonal or the ragged key end, and
//             on every tile when a key-padding mask is given
//   softmax : online (running max, running sum) in fp32, base-2 exponent
//   O^T    += V^T . P^T          v_mfma_f32_32x32x16_bf16 (or _f16), P rounded
//                                to the storage type
//
// A block walks its KV tiles from the diagonal down to tile 0 (the online
// softmax does not depend on the order). The workgroups of one head then
// reach a given tile at different times, the one with the shortest block
// first, so only one of them waits for its first fetch from HBM.
//
// Software pipeline, one barrier per tile: in iteration t a wave issues
// P(t-1) V(t-1) and the scores of tile t+1 on the matrix cores while it runs
// the softmax of tile t on the vector ALUs; no MFMA of an iteration waits
// for that iteration's vector work. K tiles are staged two tiles ahead, V
// tiles are loaded in the iteration before the one that reads them
// (double-buffered LDS for each), so HBM/L2 latency overlaps a whole
// iteration. Loads go through per-head
// buffer descriptors: rows past the end read as zeros, with no branches.
// The score matrix never leaves registers.
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

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// The 16-bit storage types and their matrix-core / dot-product forms.
template <typename T>
struct Mma;
template <>
struct Mma<__bf16> {
    typedef __bf16 v8 __attribute__((ext_vector_type(8)));
    typedef __bf16 v2 __attribute__((ext_vector_type(2)));
    __device__ static f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static float dot2(v2 a, v2 b, float c) { return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false); }
};
template <>
struct Mma<_Float16> {
    typedef _Float16 v8 __attribute__((ext_vector_type(8)));
    typedef _Float16 v2 __attribute__((ext_vector_type(2)));
    __device__ static f32x16_t mfma(v8 a, v8 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ static float dot2(v2 a, v2 b, float c) { return __builtin_amdgcn_fdot2(a, b, c, false); }
};

__device__ __forceinline__ int swap_bits23(int x) {
    return (x & ~0xC) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// LDS layout of one stage (padded rows instead of XOR swizzles, so every
// MFMA operand read is a base register plus an immediate offset):
//   K tile : 64 rows of D bf16, row stride 2*D + 16 bytes. Key r of the tile
//            sits in LDS row (r & ~31) | swap_bits23(r & 31), so the lane that
//            reads LDS row 32*half + lane%32 gets key swap_bits23(lane%32)
//            and 8 (or 16) consecutive lanes read 8 (16) consecutive rows:
//            with the 16-byte pad those fall in distinct banks.
//   V tile : 64 key rows of D bf16 in key order, as loaded, row stride
//            tile_vrow_bytes(D). The P.V operands (V^T) come from the
//            transposing LDS read ds_read_b64_tr_b16: in each 16-lane group,
//            lane j addresses 4 head dims of key row j/4, and the read hands
//            lane j one head dim for those 4 keys. The stride puts the 4 rows
//            of a half-wave's read in distinct 64-byte bank windows.
template <int D>
struct TileCfg {
    static constexpr int KCH = D / 8;            // 16-byte chunks per K row
    static constexpr int KS = D / 16;            // MFMA k-steps for S^T
    static constexpr int DB = D / 32;            // 32-row blocks of O^T
    static constexpr int NPRE = D / 32;          // 16-byte prefetch registers per thread
    static constexpr int KROW = 2 * D + 16;
    static constexpr int VROW = tile_vrow_bytes(D);
    static constexpr int K_BYTES = kTileN * KROW;
    static constexpr int V_BYTES = kTileN * VROW;
    static constexpr int LDS = tile_lds_bytes(D);
    static_assert(2 * (K_BYTES + V_BYTES) <= LDS, "stages fit");
};

// Buffer resource for the rows of one (b, h) head inside a [B, S, H, D]
// tensor: base at (b, 0, h, 0), valid bytes up to the end of row S-1. A load
// whose offset lies past the last row returns zeros and a store there is
// dropped, so ragged tails need neither branches nor clamped addresses.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const uint16_t* base, int b, int h, int S, int H) {
    const uint16_t* p = base + ((size_t)b * S * H + h) * D;
    const int bytes = ((S - 1) * H + 1) * D * 2;
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, bytes, 0x00020000);
}

// Byte offset of 16-byte chunk `ch` of token `tok` in a head's rows.
template <int D>
__device__ __forceinline__ int tok_off(int tok, int ch, int H) {
    return (tok * H * D + 8 * ch) * 2;
}

// Descriptor for the rows of one KV tile: the head's descriptor moved to the
// tile's first token, its range shortened to match (zero once past the end).
// All operands are wave-uniform, so this is scalar work; the per-lane offsets
// then stay loop-invariant.
// The K and V rows of batch entry b are S_cap rows apart (the cache
// capacity); only the first S valid ones are in range.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* base, int b, int h, int S_cap, int S, int H,
                                                            int tile0) {
    const uint16_t* p = base + ((size_t)b * S_cap * H + h) * D + (size_t)tile0 * H * D;
    const int bytes = ((S - 1) * H + 1) * D * 2 - tile0 * H * D * 2;
    return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, bytes > 0 ? bytes : 0, 0x00020000);
}

// Loader roles: waves 0-3 stage K tiles, waves 4-7 stage V tiles, each 16
// bytes of a key row per lane and load (D/8 lanes per row).
template <int D>
__device__ __forceinline__ void load_k(u32x4_t (&pre)[TileCfg<D>::NPRE], __amdgpu_buffer_rsrc_t rt, int H,
                                       int tid) {
    using C = TileCfg<D>;
#pragma unroll
    for (int it = 0; it < C::NPRE; ++it) {
        const int ci = tid + 256 * it;
        const int row = ci / C::KCH, ch = ci % C::KCH;
        pre[it] = __builtin_amdgcn_raw_buffer_load_b128(rt, tok_off<D>(row, ch, H), 0, 0);
    }
}

template <int D>
__device__ __forceinline__ void load_v(u32x4_t (&pre)[TileCfg<D>::NPRE], __amdgpu_buffer_rsrc_t rt, int H,
                                       int tid) {
    using C = TileCfg<D>;
#pragma unroll
    for (int it = 0; it < C::NPRE; ++it) {
        const int ci = (tid - 256) + 256 * it;
        const int row = ci / C::KCH, ch = ci % C::KCH;
        pre[it] = __builtin_amdgcn_raw_buffer_load_b128(rt, tok_off<D>(row, ch, H), 0, 0);
    }
}

template <int D>
__device__ __forceinline__ void store_k(const u32x4_t (&pre)[TileCfg<D>::NPRE], char* kst, int tid) {
    using C = TileCfg<D>;
#pragma unroll
    for (int it = 0; it < C::NPRE; ++it) {
        const int ci = tid + 256 * it;
        const int row = ci / C::KCH, ch = ci % C::KCH;
        const int lrow = (row & ~31) | swap_bits23(row & 31);
        *(u32x4_t*)(kst + lrow * C::KROW + 16 * ch) = pre[it];
    }
}

template <int D>
__device__ __forceinline__ void store_v(const u32x4_t (&pre)[TileCfg<D>::NPRE], char* vst, int tid) {
    using C = TileCfg<D>;
#pragma unroll
    for (int it = 0; it < C::NPRE; ++it) {
        const int ci = (tid - 256) + 256 * it;
        const int row = ci / C::KCH, ch = ci % C::KCH;
        *(u32x4_t*)(vst + row * C::VROW + 16 * ch) = pre[it];
    }
}

// S^T (32 keys of this wave's half tile x 32 queries) = K . Q^T; `krow` is
// this lane's K row (chunk g) in the stage.
template <typename T, int D>
__device__ __forceinline__ f32x16_t qk_tile(const char* krow, const typename Mma<T>::v8 (&qf)[TileCfg<D>::KS]) {
    using C = TileCfg<D>;
    f32x16_t s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
        const typename Mma<T>::v8 a = *(const typename Mma<T>::v8*)(krow + 32 * ks);
        s = Mma<T>::mfma(a, qf[ks], s);
    }
    return s;
}

// Workgroup barrier that only orders LDS traffic: unlike __syncthreads it
// does not wait for this wave's global loads and stores, so loads issued for
// the next block and the output stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The value lane l^32 holds (v_permlane32_swap: the two half-waves trade
// registers, no LDS round trip).
__device__ __forceinline__ float partner_lane(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto pr = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    // lanes 0-31 find the upper half's value in the second result, lanes 32-63 in the first
    const unsigned lo = pr[0], hi = pr[1];
    return __builtin_bit_cast(float, (__lane_id() < 32) ? hi : lo);
}

// Entries whose lengths are ranked in LDS (2 ints each); above this the
// longest-first order is skipped.
// (The ranking is O(B) per thread, a few hundred cycles at the limit.)
constexpr int kMaxRankedEntries = 256;
static_assert(2 * kMaxRankedEntries * sizeof(int) <= tile_lds_bytes(32), "rank table fits in LDS");

// Work placement for the KV-cache form. Logical unit u = rank * H + h (rank
// 0 = the longest entry) has items_per_bh items p. Hardware workgroup x runs
// on XCD x % 8 and workgroups start roughly in x order, so: consecutive
// groups of 8 units take consecutive blocks of 8*G workgroups (G =
// items_per_bh), and the G items of one unit sit 8 apart -- the same XCD,
// sharing its L2 for that head's K and V. A final group of m < 8 units is
// packed the same way with stride m. A bijection on [0, n).
__device__ __forceinline__ void kv_order(int x, int n, int G, int& u, int& p) {
    const int group = x / (8 * G);
    const int within = x % (8 * G);
    const int full_units = (n / G) / 8 * 8;   // units in complete groups of 8
    const int m = (group * 8 < full_units) ? 8 : (n / G - full_units);
    p = within / m;
    u = group * 8 + within % m;
}

// Row maxima are only re-based when they grow by more than 2^kLazy: until
// then probabilities are taken against a stale maximum (at most 2^kLazy,
// far from fp32/bf16 overflow) and the accumulators are left alone. The
// final O = acc / l is the same quantity either way.
constexpr float kLazy = 8.0f;

// KMASK: a key-padding mask is given (a separate instantiation, so the
// unmasked kernel carries none of its registers or branches).
template <typename T, int D, bool KMASK>
__global__ __launch_bounds__(kTileThreads) void fwd_tile_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    T* __restrict__ O, int B, int H, int S_q, int S_cap, int causal, float c /* scale*log2e */,
    int n_qblk, int items_per_bh, int paired, const int32_t* __restrict__ kv_lens, float* __restrict__ lse,
    const uint8_t* __restrict__ key_mask) {
    typedef typename Mma<T>::v8 v8;
    typedef typename Mma<T>::v2 v2;
    const v2 kOnes2 = {(T)1.0f, (T)1.0f};
    using C = TileCfg<D>;
    __shared__ __attribute__((aligned(16))) char lds[C::LDS];
    // an MFMA A operand of V^T: two transposing reads, keys +0..3 and +4..7
    auto vt_operand = [](const char* p) {
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p + 4 * C::VROW));
        const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
        const u32x4_t w = {l2[0], l2[1], h2[0], h2[1]};
        return __builtin_bit_cast(v8, w);
    };
    // stages: K0 K1 V0 V1, then four key-mask stages (tile of step u in u % 4)
    auto kst = [&](int i) { return lds + i * C::K_BYTES; };
    auto vst = [&](int i) { return lds + 2 * C::K_BYTES + i * C::V_BYTES; };
    auto mst = [&](int u) { return lds + tile_stage_bytes(D) + (u & 3) * kTileN; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int wq = wave & 3;     // query sub-block of this wave
    const int half = wave >> 2;  // key half of every tile
    const bool k_loader = tid < 256;
    // per-lane operand offsets inside a stage (the k-steps / blocks are immediates)
    const int k_lane = (32 * half + l32) * C::KROW + 16 * g;
    // transposing V^T reads: lane j of 16-lane group grp addresses head dims
    // 16*(grp&1) + 4*(j&3) .. +3 of key row j/4 (+ 8*(grp>>1), + 32*half), so
    // lane (l32, g) gets head dim l32 of a 32-dim block for keys 8g..8g+3 of
    // a 16-key step (and 8g+4..8g+7 from the read 4 rows on): the key order of
    // its P registers
    const int v_lane = (32 * half + 8 * (lane >> 5) + ((lane & 15) >> 2)) * C::VROW + 32 * ((lane >> 4) & 1) +
                       8 * (lane & 3);

    int bh, p;
    if (KMASK && !kv_lens) {
        // key padding: entries differ in the tiles they visit; kv_order spreads
        // the heads of every entry over all XCDs, so no XCD is left with the
        // longest entry alone
        kv_order(blockIdx.x, gridDim.x, items_per_bh, bh, p);
    } else if (!kv_lens) {
        const int item = xcd_remap(blockIdx.x, gridDim.x);
        bh = item / items_per_bh;
        p = item % items_per_bh;
    } else {
        // KV-cache entries differ in length: run the longest first. Every
        // workgroup ranks the entries by length (in LDS) and takes the
        // (b, h) of its rank; see kv_order for the XCD placement.
        kv_order(blockIdx.x, gridDim.x, items_per_bh, bh, p);
        if (B <= kMaxRankedEntries) {
            int* lens = (int*)lds;
            int* perm = lens + kMaxRankedEntries;
            for (int e = tid; e < B; e += kTileThreads) lens[e] = min(max(kv_lens[e], 0), S_cap);
            __syncthreads();
            for (int e = tid; e < B; e += kTileThreads) {
                int rank = 0;
                for (int f = 0; f < B; ++f) rank += (lens[f] > lens[e]) || (lens[f] == lens[e] && f < e);
                perm[rank] = e;
            }
            __syncthreads();
            bh = perm[bh / H] * H + bh % H;
            __syncthreads();   // the table's LDS is reused by the first stage stores
        }
    }
    const int b = bh / H, h = bh % H;
    // valid keys of this batch entry (all S_cap rows unless lengths are given)
    const int S_kv = kv_lens ? min(max(kv_lens[b], 0), S_cap) : S_cap;
    const int off = S_kv - S_q;  // absolute position of query i is i + off (may be < 0)
    const int qb_first = n_qblk - 1 - p;
    const int nphase = (paired && p != qb_first) ? 2 : 1;

    const __amdgpu_buffer_rsrc_t rq = head_rsrc<D>(Q, b, h, S_q, H);
    const __amdgpu_buffer_rsrc_t ro = head_rsrc<D>((const uint16_t*)O, b, h, S_q, H);

    // The loads that open a query block: its Q^T fragments (B operand: lane
    // holds query qi, head dims 16*ks + 8*g .. +7) and tile 0 of K and V.
    // They are issued before the previous block's merge, so their latency
    // overlaps it.
    v8 qf[C::KS];
    u32x4_t pre[C::NPRE];
    // Key-padding mask: the first kTileN K-loader threads carry one byte of
    // it per key of the tile they stage (bytes past S_kv read as 0: hidden).
    const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(key_mask ? key_mask + (size_t)b * S_cap : key_mask), (short)0, key_mask ? S_kv : 0, 0x00020000);
    const bool m_loader = KMASK && tid < kTileN;
    unsigned mpre = 0;
    auto load_mask = [&](int tile0) {
        if (m_loader) mpre = __builtin_amdgcn_raw_buffer_load_b8(rm, tile0 + tid, 0, 0);
    };
    auto store_mask = [&](int u) {
        if (m_loader) mst(u)[tid] = (char)mpre;
    };
    // With a key-padding mask, keys before the entry's first visible key and
    // after its last one are skipped tile by tile: [vis_lo, vis_hi) bounds
    // the visible keys (empty when none is visible).
    int vis_lo = 0, vis_hi = S_kv;
    if constexpr (KMASK) {
        int* sv = (int*)mst(0);   // the mask stages are free until the prologue
        if (tid == 0) {
            sv[0] = S_kv;
            sv[1] = 0;
        }
        __syncthreads();
        int lo_t = S_kv, hi_t = 0;
        const uint8_t* row = key_mask + (size_t)b * S_cap;
        for (int j = tid; j < S_kv; j += kTileThreads)
            if (row[j] != 0) {
                lo_t = min(lo_t, j);
                hi_t = j + 1;
            }
#pragma unroll
        for (int x = 32; x >= 1; x >>= 1) {
            lo_t = min(lo_t, __shfl_xor(lo_t, x));
            hi_t = max(hi_t, __shfl_xor(hi_t, x));
        }
        if (lane == 0) {
            atomicMin(&sv[0], lo_t);
            atomicMax(&sv[1], hi_t);
        }
        __syncthreads();
        vis_lo = sv[0];
        vis_hi = sv[1];
        __syncthreads();   // before the stages are written
    }
    // KV tiles [lo, hi) block qb visits (walked from hi-1 down to lo)
    auto block_tiles = [&](int qb, int& lo, int& hi) {
        hi = tiles_for_block(qb, S_q, S_kv, causal);
        lo = 0;
        if constexpr (KMASK) {
            hi = min(hi, (vis_hi + kTileN - 1) / kTileN);
            lo = min(vis_lo / kTileN, hi);
        }
    };
    auto issue_block = [&](int qb) {
        const int qi = qb * kTileM + 32 * wq + l32;
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks)
            qf[ks] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rq, tok_off<D>(qi, 2 * ks + g, H), 0, 0));
        int lo, hi;
        block_tiles(qb, lo, hi);
        const int first = (hi - 1) * kTileN;   // tiles run backwards
        if (hi > lo) {
            if (k_loader) load_k<D>(pre, tile_rsrc<D>(K, b, h, S_cap, S_kv, H, first), H, tid);
            else load_v<D>(pre, tile_rsrc<D>(V, b, h, S_cap, S_kv, H, first), H, tid);
            load_mask(first);
        }
    };
    issue_block(qb_first);

    for (int phase = 0; phase < nphase; ++phase) {
        const int qb = phase == 0 ? qb_first : p;
        int tile_lo, tile_hi;
        block_tiles(qb, tile_lo, tile_hi);
        const int nt = tile_hi - tile_lo;          // steps (tiles visited)
        const int q0 = qb * kTileM + 32 * wq;      // first query of this wave
        const int qi = q0 + l32;                   // this lane's query
        const bool wave_has_rows = q0 < S_q;
        const int q_last = (q0 + 31 < S_q ? q0 + 31 : S_q - 1);
        const int key_last = causal ? q_last + off : S_kv - 1;   // last key any row of the wave sees
        const int lane_key_limit = causal ? qi + off : S_kv - 1; // last key this lane sees

        f32x16_t acc[C::DB];
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
        float m_ref = -INFINITY;   // reference maximum of (score * c) for query qi
        float l_run = 0.f;         // this lane's share of the running sum

        // Prologue: tile 0 (K and V) staged; S(0) computed while K(1) lands.
        if (k_loader) {
            store_k<D>(pre, kst(0), tid);
            store_mask(0);
        } else {
            store_v<D>(pre, vst(0), tid);
            // the stage a first-step P.V (with P = 0) reads: finite zeros
            const u32x4_t z = {0u, 0u, 0u, 0u};
            for (int i = tid - 256; i < C::V_BYTES / 16; i += 256) *(u32x4_t*)(vst(1) + 16 * i) = z;
        }
        __syncthreads();
        // step u works on KV tile nt-1-u: the diagonal tile first
        auto tile_of = [&](int u) { return tile_hi - 1 - u; };
        if (k_loader && nt > 1) {
            load_k<D>(pre, tile_rsrc<D>(K, b, h, S_cap, S_kv, H, tile_of(1) * kTileN), H, tid);
            load_mask(tile_of(1) * kTileN);
        }
        // unconditional: every path into the loop has then waited for the Q
        // loads, so the loop body never waits on them (or on the prefetch)
        f32x16_t sa = qk_tile<T, D>(kst(0) + k_lane, qf), sb;
        if (k_loader && nt > 1) {
            store_k<D>(pre, kst(1), tid);
            store_mask(1);
        }
        __syncthreads();

        // One tile: s_c holds S(t); S(t+1) goes to s_n. P(t-1) waits in
        // pb_prev and its P.V product runs in step t, so no MFMA of a step
        // depends on that step's vector work. V(t) is loaded in step t and
        // staged at its end; P.V(t-1) reads the stage written one step ago.
        v8 pb_prev[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int i = 0; i < 8; ++i) pb_prev[s2][i] = (T)0.f;
        // a re-base decided in step t scales the accumulator at the start of
        // step t+1, once P.V(t-1) is in and before P.V(t) is added
        bool rescale_due = false;
        float alpha_due = 1.f;
        auto apply_rescale = [&]() {
            if (rescale_due) {
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[db][r] *= alpha_due;
                rescale_due = false;
            }
        };
        auto step = [&](int t, f32x16_t& s_c, f32x16_t& s_n) {
            // (a) HBM loads: K two tiles ahead; V of this tile (V(0) came with
            // the block's opening loads)
            const bool ld_k = k_loader && t + 2 < nt;
            const bool ld_v = !k_loader && t >= 1;
            if (ld_k) {
                load_k<D>(pre, tile_rsrc<D>(K, b, h, S_cap, S_kv, H, tile_of(t + 2) * kTileN), H, tid);
                load_mask(tile_of(t + 2) * kTileN);
            }
            if (ld_v) load_v<D>(pre, tile_rsrc<D>(V, b, h, S_cap, S_kv, H, tile_of(t) * kTileN), H, tid);

            const int kbase = tile_of(t) * kTileN + 32 * half;   // first key of this wave's half tile
            const bool work = wave_has_rows && kbase <= key_last && kbase < S_kv;
            // a wave skips the tiles whose keys all lie past its last query (the
            // first ones in this order, so no P.V is pending there); the first
            // tile it does see still needs its scores from here
            if (!work && t + 1 < nt && wave_has_rows && kbase - kTileN <= key_last && kbase - kTileN < S_kv)
                s_n = qk_tile<T, D>(kst((t + 1) & 1) + k_lane, qf);
            if (work) {
                apply_rescale();
                // (b) mask: where the tile crosses the diagonal or the key end,
                // and everywhere when keys are hidden by the key-padding mask
                // (this lane's keys are bytes 32*half + 16*(r/8) + 8*g + r%8 of
                // the tile's mask stage)
                if constexpr (KMASK) {
                    const char* mrow = mst(t) + 32 * half + 8 * g;
                    const u32x2_t m0 = *(const u32x2_t*)mrow;
                    const u32x2_t m1 = *(const u32x2_t*)(mrow + 16);
                    const unsigned w4[4] = {m0[0], m0[1], m1[0], m1[1]};
                    // fast path: a tile off the diagonal and the key end whose
                    // mask bytes are all nonzero for every lane of the wave hides
                    // nothing (a word has a zero byte iff (w - 0x01010101) & ~w &
                    // 0x80808080 is nonzero; bytes past S_kv read as 0)
                    const bool tile_edge = (causal && kbase + 31 > q0 + off) || (kbase + 32 > S_kv);
                    unsigned zb = 0u;
#pragma unroll
                    for (int x = 0; x < 4; ++x) zb |= (w4[x] - 0x01010101u) & ~w4[x] & 0x80808080u;
                    const bool any_hidden = __builtin_amdgcn_ballot_w64(zb != 0u) != 0;
                    if (tile_edge || any_hidden) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = kbase + 16 * (r >> 3) + 8 * g + (r & 7);
                            const unsigned byte = (w4[r >> 2] >> (8 * (r & 3))) & 0xFFu;
                            // branch-free: one compare chain and a select per register
                            const bool hide = (key > lane_key_limit) | (key >= S_kv) | (byte == 0u);
                            s_c[r] = hide ? -INFINITY : s_c[r];
                        }
                    }
                } else {
                    if ((causal && kbase + 31 > q0 + off) || (kbase + 32 > S_kv)) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int key = kbase + 16 * (r >> 3) + 8 * g + (r & 7);
                            if (key > lane_key_limit || key >= S_kv) s_c[r] = -INFINITY;
                        }
                    }
                }
                float mx = s_c[0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s_c[r]);
                // (c) row max (one exchange with the partner lane l^32), lazy re-base
                mx = fmaxf(mx, partner_lane(mx)) * c;   // row max over both half-waves
                const bool rebase = __builtin_amdgcn_ballot_w64(mx > m_ref + kLazy) != 0;
                // re-base: the sum now; the accumulator after P.V(t-1) is in
                const float m_new = rebase ? fmaxf(m_ref, mx) : m_ref;
                const float alpha = (m_new == -INFINITY || !rebase) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
                l_run *= alpha;
                m_ref = m_new;
                const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
                // (d) O^T += V^T . P(t-1)^T, then S(t+1), both on the matrix
                // cores while the vector ALUs form P(t)
                const char* vt = vst((t + 1) & 1) + v_lane;
                v8 va[C::DB][2];
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) va[db][s2] = vt_operand(vt + 64 * db + 16 * s2 * C::VROW);
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        acc[db] = Mma<T>::mfma(va[db][s2], pb_prev[s2], acc[db]);
                s_n = qk_tile<T, D>(kst((t + 1) & 1) + k_lane, qf);
                // P is rounded to the storage type for the P.V product; the row sum adds up
                // the same rounded values, so the weights that multiply V are
                // exactly normalised (a near one-hot row returns its V row)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        pb_prev[s2][i] = (T)__builtin_amdgcn_exp2f(__builtin_fmaf(s_c[8 * s2 + i], c, -m_use));
#pragma unroll
                    // row sum of the rounded values: one v_dot2 (x 1.0) per pair
                    for (int i = 0; i < 4; ++i) {
                        const v2 pair = {pb_prev[s2][2 * i], pb_prev[s2][2 * i + 1]};
                        l_run = Mma<T>::dot2(pair, kOnes2, l_run);
                    }
                }
                // schedule: the V^T operand reads, the P.V MFMAs each followed by
                // a slice of the softmax VALU work, then the K operand reads and
                // the S(t+1) MFMAs, likewise interleaved
                __builtin_amdgcn_sched_group_barrier(0x100, 4 * C::DB, 0);
#pragma unroll
                for (int i = 0; i < 2 * C::DB; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, C::KS, 0);
#pragma unroll
                for (int i = 0; i < C::KS; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                }
                rescale_due = rebase;
                alpha_due = alpha;
            }
            // (f) land the loaded tiles in stages whose last reader ran one
            // iteration ago
            if (ld_k) {
                store_k<D>(pre, kst(t & 1), tid);
                store_mask(t + 2);   // stage (t+2)%4 was last read in step t-2
            }
            if (ld_v) store_v<D>(pre, vst(t & 1), tid);
            __syncthreads();
        };
        for (int t = 0; t < nt; t += 2) {
            step(t, sa, sb);
            if (t + 1 < nt) step(t + 1, sb, sa);
        }
        // the last P.V: V(nt-1) was staged at the end of the last step
        apply_rescale();
        {
            const char* vt = vst((nt - 1) & 1) + v_lane;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    acc[db] = Mma<T>::mfma(vt_operand(vt + 64 * db + 16 * s2 * C::VROW), pb_prev[s2], acc[db]);
        }
        lds_barrier();   // every wave's reads of the stages are done before the merge reuses them

        // the next block's opening loads run under this block's merge
        if (phase + 1 < nphase) issue_block(p);

        // ---- merge the two key halves (waves wq and wq+4) through LDS
        float* xf = (float*)lds;
        float* slot = xf + wq * (64 * (C::DB * 16 + 2));
        if (half == 1) {
            slot[lane] = m_ref;
            slot[64 + lane] = l_run;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) slot[128 + (db * 16 + r) * 64 + lane] = acc[db][r];
        }
        lds_barrier();
        if (half == 0 && wave_has_rows) {
            const float m1 = slot[lane];
            const float l1 = slot[64 + lane];
            const float m = fmaxf(m_ref, m1);
            const float mu = (m == -INFINITY) ? 0.f : m;
            const float a0 = __builtin_amdgcn_exp2f(m_ref - mu);
            const float a1 = __builtin_amdgcn_exp2f(m1 - mu);
            float l = a0 * l_run + a1 * l1;
            l += partner_lane(l);
            // a row that sees no key (a KV-cache entry shorter than the chunk) is 0
            const float inv = l > 0.f ? 1.0f / l : 0.f;
            // log of the softmax denominator in natural units: ln 2 * (m + log2 l)
            if (lse && g == 0 && qi < S_q)
                lse[((size_t)b * H + h) * S_q + qi] = l > 0.f ? (mu + __builtin_log2f(l)) * 0.69314718055994531f
                                                            : -INFINITY;
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    T ob[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int r = 4 * j + e;
                        const float x1 = slot[128 + (db * 16 + r) * 64 + lane];
                        ob[e] = (T)((a0 * acc[db][r] + a1 * x1) * inv);
                    }
                    // lane holds head dims 32*db + 8*j + 4*g .. +3 of its query;
                    // rows past S_q fall outside the descriptor and are dropped
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, ob), ro,
                                                          (qi * H * D + 32 * db + 8 * j + 4 * g) * 2, 0, 0);
                }
        }
        lds_barrier();
    }
}

template <typename T, int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
    const TileGrid tg = tile_grid(a.B, a.H, a.S_q, a.causal, a.kv_lens != nullptr);
    if (a.key_mask)
        hipExtLaunchKernelGGL((fwd_tile_kernel<T, D, true>), dim3((unsigned)tg.n_items), dim3(kTileThreads), 0,
                              stream, a.ev_start, a.ev_stop, 0, (const uint16_t*)a.q, (const uint16_t*)a.k,
                              (const uint16_t*)a.v, (T*)a.o, a.B, a.H, a.S_q, a.S_kv, a.causal, a.scale_log2,
                              tg.n_qblk, tg.items_per_bh, tg.paired, a.kv_lens, a.lse, a.key_mask);
    else
        hipExtLaunchKernelGGL((fwd_tile_kernel<T, D, false>), dim3((unsigned)tg.n_items), dim3(kTileThreads), 0,
                              stream, a.ev_start, a.ev_stop, 0, (const uint16_t*)a.q, (const uint16_t*)a.k,
                              (const uint16_t*)a.v, (T*)a.o, a.B, a.H, a.S_q, a.S_kv, a.causal, a.scale_log2,
                              tg.n_qblk, tg.items_per_bh, tg.paired, a.kv_lens, a.lse, nullptr);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 32: return launch_d<T, 32>(a, stream);
        case 64: return launch_d<T, 64>(a, stream);
        case 128: return launch_d<T, 128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_fwd_tile(const FwdArgs& a, Elt t, hipStream_t stream) {
    switch (t) {
        case Elt::BF16: return launch_t<__bf16>(a, stream);
        case Elt::F16: return launch_t<_Float16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn
