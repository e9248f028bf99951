// fwd_prefill.hip -- fused causal attention forward on gfx950 matrix cores
// (bf16 or fp16 storage, fp32 arithmetic): the attn_fwd and attn_fwd_kvcache
// path.
//
// Work item: one workgroup of 8 waves. With the causal rule (or without it)
// an item is two 128-query blocks of one (b, h), r and n-1-r (the smaller
// one first), so every item walks the same number of 64-key tiles; with
// per-entry cache lengths it is one block. Wave w holds queries 32*(w%4) .. +31 of the block and key half
// w/4 of every tile; the two halves merge at the end of the block.
//
// The blocks of an item form ONE stream of key tiles, each block's tiles
// walked from tile 0 (or the first visible one) up to its diagonal: the
// items of one head, which run on one XCD, start on the same tiles, so
// those come from HBM once and from L2 for the rest (walking down from
// each block's own diagonal, every item started on tiles of its own, and
// the opening read all of them from HBM at once). K and V tiles go from HBM
// straight into a ring of three LDS stages through the LDS path of the
// buffer loads (no staging registers, no LDS store instructions), issued two
// steps before their use; a step ends with one wait for the previous step's
// loads and one barrier. The second block's Q and first tiles arrive during
// the first block's last steps, so a block change costs only the merge.
//
// Step u of a block, tile t_u (the u-th from the bottom), key half of a wave:
//   matrix cores : O^T += V^T(t_{u-1}) . P(t_{u-1})^T   (one step late)
//                  S^T(t_{u+1}) = K(t_{u+1}) . Q^T       (one step early)
//   vector ALUs  : row max of S(t_u) with a lazy re-base, P(t_u) =
//                  2^(S*c - m) rounded to the storage type, row sums of the
//                  rounded P
// so no MFMA of a step waits for that step's vector work. The steps whose
// tile crosses the diagonal or the ragged key end (the last one or two of a
// block) run a separate masked copy of the step; the remaining loop has no
// branch but the rare re-base.
//
// Method: fused QK^T + mask + softmax + P.V with the score row kept on chip
// and K tiles staged in shared memory ("Hand-written Masked Multi-Head
// Attention CUDA kernel" page, sections 2.1-2.2 and 3); the online softmax
// recurrence m' = max(m, x), l' = l*exp(m-m') + exp(x-m') and the -inf
// mask ("Week-4 CUDA notes" page, section 2.2); skipping the masked half of
// the score matrix instead of computing it (MMHA page, section 1) and
// per-thread key bounds instead of per-element branches (MMHA page,
// section 2.3); fp32 arithmetic on half-width storage (MMHA page,
// section 3.3); loading the next K tiles while the current one computes
// (MMHA page, section 4.2).
//
// Operand layouts. In the 32x32 MFMA result a lane holds one COLUMN n =
// lane%32 and 16 rows m = 8*(r/4) + 4*(lane/32) + r%4 (register r).
// Computing S^T = K Q^T puts one query per lane (the column) and its keys in
// registers: the row max and sum need one exchange between lanes l and
// l^32, and the probabilities already sit where the B operand of
// O^T = V^T P^T wants them. The A-operand row a lane reads for S^T is key
// swap_bits23(lane%32) of its half, so register r of half g holds key
// 16*(r/8) + 8*g + (r%8): registers 8s..8s+7 are 8 consecutive keys, one
// B-operand chunk of the P.V step. V^T operands come from the transposing
// LDS read ds_read_b64_tr_b16 of V rows stored as loaded.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "../launch.h"
#include "../plan.h"

namespace attn {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
// (This compiler reads element 0 for __builtin_bit_cast applied to an
// element of an ext_vector_type value; vector elements are copied to a
// scalar, or kept in float vectors, before any bit cast.)

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

// LDS layout (offsets in bytes):
//   V ring : 3 stages of 64 key rows of 2*D bytes, as loaded. The 16-byte
//            chunk c of row r sits at chunk position c ^ (vswz(r) << 2), so
//            the 4 rows one half-wave's transposing read touches fall in
//            distinct 64-byte bank windows.
//   K ring : 3 stages of 64 rows of 2*D + 16 bytes (16-byte pad). Key k of
//            the tile sits in row (k & ~31) | swap_bits23(k & 31); 8 (16)
//            consecutive lanes then read 8 (16) consecutive padded rows,
//            which fall in distinct banks. Every operand read is a base
//            register plus an immediate.
//   merge  : the two key halves' partial accumulators, exchanged one block
//            per half and round, and their (m, l); with D = 32, the
//            key-half-1 waves' one block and (m, l).
//   masks  : (with a key-padding mask) 4 stages of 256 bytes: the tile's
//            mask bytes as loaded from a 4-byte aligned address, so the byte
//            of key k sits at msh + k (msh: the mask row's address mod 4);
//            then one bit per key tile of the entry: the tile holds a key
//            the mask hides.
template <int D>
struct Cfg {
    static constexpr int KS = D / 16;      // MFMA k-steps of S^T
    static constexpr int DB = D / 32;      // 32-row blocks of O^T
    static constexpr int KCH = D / 8;      // 16-byte chunks of a key row
    static constexpr int KROW = prefill_krow_bytes(D);
    static constexpr int VROW = 2 * D;
    static constexpr int K_STAGE = prefill_k_stage_bytes(D);
    static constexpr int V_STAGE = prefill_v_stage_bytes(D);
    static constexpr int K_LOADS = K_STAGE / 1024;   // one-kilobyte wave loads per stage
    static constexpr int V_LOADS = V_STAGE / 1024;
    static constexpr int K_SLOTS = (K_LOADS + kTileWaves - 1) / kTileWaves;
    static constexpr int V_SLOTS = (V_LOADS + kTileWaves - 1) / kTileWaves;
    static constexpr int V_RING = 0;
    static constexpr int K_RING = kPrefillStages * V_STAGE;
    static constexpr int MERGE = K_RING + kPrefillStages * K_STAGE;
    static constexpr int MDB = prefill_merge_db(D);
    static constexpr int MREC = prefill_merge_rec_floats(D);
    static constexpr int ROUNDS = DB / MDB;
    static constexpr int LDS = prefill_lds_bytes(D);
    // (masked instantiation only) the key-mask stages, then the tile bits
    static constexpr int MASKS = LDS;
    static constexpr int TBITS = MASKS + kPrefillMaskStages * kPrefillMaskStageBytes;
    static constexpr int ROWS_PER_256 = 256 / VROW;   // V rows sharing one 256-byte bank span
    static_assert(K_STAGE % 1024 == 0 && V_STAGE % 1024 == 0, "stages are whole wave loads");
    static_assert(MERGE + 4 * 64 * MREC * 4 <= LDS, "layout fits");
    static_assert(DB % MDB == 0, "whole merge rounds");
};

// Swizzle key of V row r: which of the row's 64-byte windows chunk 0 moves to.
template <int D>
__device__ __forceinline__ int vswz(int r) {
    return (r / Cfg<D>::ROWS_PER_256) & (Cfg<D>::DB - 1);
}

// The rows of one (b, h) head from token tok0 on, inside a [B, S_cap, H, D]
// tensor of which the first S_valid tokens of entry b are in range: a load
// past the last valid row returns zeros, a store there is dropped.
struct HeadRows {
    const char* p;
    unsigned bytes;
};
template <int D>
__device__ __forceinline__ HeadRows head_rows(const void* base, int b, int h, int S_cap, int S_valid, int H,
                                              int tok0) {
    const char* p = (const char*)base + (((size_t)b * S_cap * H + h) * D + (size_t)tok0 * H * D) * 2;
    const long long bytes = ((long long)(S_valid - 1) * H + 1) * D * 2 - (long long)tok0 * H * D * 2;
    return {p, (unsigned)(bytes > 0 ? bytes : 0)};
}
// As a buffer resource for the load/store builtins.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(HeadRows r) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)r.p, (short)0, (int)r.bytes, 0x00020000);
}

// 16 bytes per lane from global memory (descriptor d, byte offset voff)
// straight into LDS at lds_addr + 16*lane; M0 carries the LDS address (one
// wait state after writing it) and is restored. Written out rather than
// through the builtin, which makes the compiler wait for every such load
// before any later LDS read; here each stage is published explicitly (a
// vmcnt wait, then a barrier) two steps before it is read.
__device__ __forceinline__ void lds_dma16(u32x4_t dv, unsigned voff, unsigned lds_addr_v) {
    // the descriptor and the LDS address are wave-uniform; say so, so they
    // stay in scalar registers whatever the surrounding code
    const u32x4_t d = {(unsigned)__builtin_amdgcn_readfirstlane(dv[0]), (unsigned)__builtin_amdgcn_readfirstlane(dv[1]),
                       (unsigned)__builtin_amdgcn_readfirstlane(dv[2]), (unsigned)__builtin_amdgcn_readfirstlane(dv[3])};
    const unsigned lds_addr = (unsigned)__builtin_amdgcn_readfirstlane(lds_addr_v);
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_addr), "v"(voff), "s"(d)
        : "memory");
}

// 4 bytes per lane from global memory into LDS at lds_addr + 4*lane (the
// dword form of the same path); out of range: 0.
__device__ __forceinline__ void lds_dma4(u32x4_t dv, unsigned voff, unsigned lds_addr_v) {
    const u32x4_t d = {(unsigned)__builtin_amdgcn_readfirstlane(dv[0]), (unsigned)__builtin_amdgcn_readfirstlane(dv[1]),
                       (unsigned)__builtin_amdgcn_readfirstlane(dv[2]), (unsigned)__builtin_amdgcn_readfirstlane(dv[3])};
    const unsigned lds_addr = (unsigned)__builtin_amdgcn_readfirstlane(lds_addr_v);
    unsigned saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
        "buffer_load_dword %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds_addr), "v"(voff), "s"(d)
        : "memory");
}

// Wait until at most n of this wave's memory loads are in flight and its LDS
// reads are done, then meet the workgroup.
__device__ __forceinline__ void wait_vm_barrier(int n) {
    switch (n) {
        case 0: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(1) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(3) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        case 5: asm volatile("s_waitcnt vmcnt(5) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        case 6: asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        case 7: asm volatile("s_waitcnt vmcnt(7) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        case 8: asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        case 9: asm volatile("s_waitcnt vmcnt(9) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        case 10: asm volatile("s_waitcnt vmcnt(10) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        case 11: asm volatile("s_waitcnt vmcnt(11) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        case 12: asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        case 13: asm volatile("s_waitcnt vmcnt(13) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        case 14: asm volatile("s_waitcnt vmcnt(14) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        case 15: asm volatile("s_waitcnt vmcnt(15) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        case 16: asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    }
}

// Workgroup barrier that only orders LDS traffic.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The value lane l^32 holds (v_permlane32_swap: the two half-waves trade
// registers, no LDS round trip).
__device__ __forceinline__ float partner_lane(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto pr = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned lo = pr[0], hi = pr[1];
    return __builtin_bit_cast(float, (__lane_id() < 32) ? hi : lo);
}

// Entries, or (entry, block) classes, ranked in LDS (2 ints each); above
// this the classes fall back to entries, and the entries to launch order.
constexpr int kMaxRankedEntries = 256;
static_assert(2 * kMaxRankedEntries * sizeof(int) <= prefill_lds_bytes(32), "rank table fits in LDS");

// Work placement for per-entry lengths. Logical unit u = rank * H + h (rank
// 0 = the longest entry) has G items p. Hardware workgroup x runs on XCD
// x % 8 and workgroups start roughly in x order, so consecutive groups of 8
// units take consecutive blocks of 8*G workgroups and the G items of one unit
// sit 8 apart -- the same XCD, sharing its L2 for that head's K and V. A final
// group of m < 8 units is packed the same way with stride m. A bijection on
// [0, n).
__device__ __forceinline__ void kv_order(int x, int n, int G, int& u, int& p) {
    const int group = x / (8 * G);
    const int within = x % (8 * G);
    const int full_units = (n / G) / 8 * 8;
    const int m = (group * 8 < full_units) ? 8 : (n / G - full_units);
    p = within / m;
    u = group * 8 + within % m;
}

// Row maxima are only re-based when they grow by more than 2^kLazy: until
// then probabilities are taken against a stale maximum (at most 2^kLazy,
// far from fp32/bf16 overflow) and the accumulators are left alone. The
// final O = acc / l is the same quantity either way.
constexpr float kLazy = 8.0f;

template <bool B>
using Flag = std::integral_constant<bool, B>;

// The wave that loads the key-mask bytes: the last one, which has the
// fewest K and V loads for every head dim.
constexpr int kMaskWave = kTileWaves - 1;

// KMASK: a key-padding mask is given (attn_fwd_mask; a separate
// instantiation, so the unmasked kernel carries none of its work). Its
// per-step mask work runs only for entries whose mask hides a key before the
// last visible one; the others are a shorter key length.
template <typename T, int D, bool KMASK>
__global__ __launch_bounds__(kTileThreads) void prefill_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    T* __restrict__ O, int B, int H, int S_q, int S_cap, int causal, float c /* scale*log2e */, int n_qblk,
    int items_per_bh, int paired, const int32_t* __restrict__ kv_lens, float* __restrict__ lse,
    unsigned long long* __restrict__ clk, const uint8_t* __restrict__ key_mask) {
    typedef typename Mma<T>::v8 v8;
    typedef typename Mma<T>::v2 v2;
    using C = Cfg<D>;
    const v2 kOnes2 = {(T)1.0f, (T)1.0f};
    __shared__ __attribute__((aligned(1024))) char lds[KMASK ? prefill_lds_bytes_kmask(D) : C::LDS];
    const unsigned lds_u = (unsigned)(size_t)(lds_void_t*)lds;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int wq = wave & 3;     // query sub-block of this wave
    const int half = wave >> 2;  // key half of every tile
    const int HD2 = H * D * 2;   // bytes between consecutive tokens of a head
    // optional clock probe: workgroup 0 records the shader-clock counter and
    // the 100 MHz real-time counter when it starts and when it ends
    if (clk && blockIdx.x == 0 && tid == 0) {
        clk[0] = __builtin_amdgcn_s_memtime();
        clk[1] = __builtin_amdgcn_s_memrealtime();
    }

    // ---- work item
    int bh, p;
    if (KMASK) {
        // entries differ in the tiles their masks leave visible; kv_order
        // spreads the heads of every entry over all XCDs, so no XCD is left
        // with the longest entries alone
        kv_order(blockIdx.x, gridDim.x, items_per_bh, bh, p);
    } else if (!kv_lens) {
        const int item = xcd_remap(blockIdx.x, gridDim.x);
        bh = item / items_per_bh;
        p = item % items_per_bh;
    } else {
        // entries differ in length, and the blocks of an entry in the tiles
        // they walk: the (entry, block) classes run costliest first, ranked
        // in LDS by their tile counts. Workgroups are dispatched in launch
        // order, so a workgroup waits for the one before it to be placed:
        // with costs that only fall, a CU that frees up finds the next item
        // ready. The H heads of a class are consecutive workgroups, so head h
        // of every class runs on XCD h % 8 (H a multiple of 8) and shares that
        // head's K and V in one L2.
        const int G = items_per_bh;
        if (B * G <= kMaxRankedEntries && (long long)B * H * G == (long long)gridDim.x) {
            int* cost = (int*)lds;
            int* perm = cost + kMaxRankedEntries;
            for (int c = tid; c < B * G; c += kTileThreads) {
                const int len = min(max(kv_lens[c / G], 0), S_cap);
                cost[c] = tiles_for_block(n_qblk - 1 - c % G, S_q, len, causal);
            }
            __syncthreads();
            for (int c = tid; c < B * G; c += kTileThreads) {
                int rank = 0;
                for (int f = 0; f < B * G; ++f) rank += (cost[f] > cost[c]) || (cost[f] == cost[c] && f < c);
                perm[rank] = c;
            }
            __syncthreads();
            const int cls = perm[blockIdx.x / H];
            bh = (cls / G) * H + blockIdx.x % H;
            p = cls % G;
            __syncthreads();   // the table's LDS is reused by the first stages
        } else {
            // many entries: the longest entries first, their heads spread
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
                __syncthreads();   // the table's LDS is reused by the first stages
            }
        }
    }
    const int b = bh / H, h = bh % H;
    const int S_kv = kv_lens ? min(max(kv_lens[b], 0), S_cap) : S_cap;   // valid keys of this entry
    const int off = S_kv - S_q;   // absolute position of query i is i + off (may be < 0)
    const int qb_big = n_qblk - 1 - p;   // the item's only block when unpaired
    const int nblk = (paired && p != qb_big) ? 2 : 1;
    // the smaller block first: every item of a head then starts on tile 0,
    // and the larger blocks walk up behind one another (at most 14 tiles
    // apart at S = 2048), so they still find their tiles in L2 (with the
    // larger block first, the items that reached their smaller block last
    // re-read its low tiles from HBM)
    const int qbs[2] = {nblk == 2 ? p : qb_big, qb_big};
    // the entry's row of the key mask, and its address mod 4
    const uint8_t* const mrow = KMASK ? key_mask + (size_t)b * S_cap : nullptr;
    const int msh = (int)((unsigned long long)mrow & 3u);

    // With a key mask, the tiles before the entry's first visible key and
    // after its last one are skipped: [vis_lo, vis_hi) bounds the visible
    // keys (empty when none is). The row is read in 16-byte pieces through a
    // descriptor rounded out to 16-byte boundaries (a piece never reaches a
    // page the row does not touch); bytes outside the row are ignored.
    // The same pass marks the tiles that hold a hidden key; only their steps
    // apply the mask to the scores.
    int vis_lo = 0, vis_hi = S_kv;
    int first_hidden = S_kv;   // the row's first hidden key (S_kv: none)
    if constexpr (KMASK) {
        unsigned* tbits = (unsigned*)(lds + C::TBITS);
        for (int i = tid; i < kPrefillMaskTileBits / 32; i += kTileThreads) tbits[i] = 0u;
        __syncthreads();
        const unsigned long long ra = (unsigned long long)mrow;
        const int sh = (int)(ra & 15u);
        const int n_ch = (sh + S_kv + 15) >> 4;
        const __amdgpu_buffer_rsrc_t dm =
            __builtin_amdgcn_make_buffer_rsrc((void*)(mrow - sh), (short)0, n_ch * 16, 0x00020000);
        int lo_t = S_kv, hi_t = 0, hid_t = S_kv;
        for (int ch = tid; ch < n_ch; ch += kTileThreads) {
            const u32x4_t w =
                __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(dm, 16u * (unsigned)ch, 0, 0));
            const int k0 = 16 * ch - sh;   // row index of the piece's first byte
            int hid_first = S_kv, hid_last = -1;   // hidden keys of the piece
#pragma unroll
            for (int x = 0; x < 16; ++x) {
                const int k = k0 + x;
                if (k >= 0 && k < S_kv) {
                    if (((w[x >> 2] >> (8 * (x & 3))) & 0xFFu) != 0u) {
                        lo_t = min(lo_t, k);
                        hi_t = k + 1;
                    } else {
                        hid_first = min(hid_first, k);
                        hid_last = k;
                    }
                }
            }
            hid_t = min(hid_t, hid_first);
            // a piece spans at most two tiles
            if (hid_last >= 0) {
                const int t0 = hid_first / kTileN, t1 = hid_last / kTileN;
                if (t0 < kPrefillMaskTileBits) atomicOr(&tbits[t0 >> 5], 1u << (t0 & 31));
                if (t1 != t0 && t1 < kPrefillMaskTileBits) atomicOr(&tbits[t1 >> 5], 1u << (t1 & 31));
            }
        }
#pragma unroll
        for (int x = 32; x >= 1; x >>= 1) {
            lo_t = min(lo_t, __shfl_xor(lo_t, x));
            hi_t = max(hi_t, __shfl_xor(hi_t, x));
            hid_t = min(hid_t, __shfl_xor(hid_t, x));
        }
        // across the waves through the merge region (first used at the
        // first block's end)
        int* sv = (int*)(lds + C::MERGE);
        if (lane == 0) {
            sv[3 * wave] = lo_t;
            sv[3 * wave + 1] = hi_t;
            sv[3 * wave + 2] = hid_t;
        }
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kTileWaves; ++w) {
            lo_t = min(lo_t, sv[3 * w]);
            hi_t = max(hi_t, sv[3 * w + 1]);
            hid_t = min(hid_t, sv[3 * w + 2]);
        }
        vis_lo = __builtin_amdgcn_readfirstlane(lo_t);
        vis_hi = __builtin_amdgcn_readfirstlane(hi_t);
        first_hidden = __builtin_amdgcn_readfirstlane(hid_t);
    }
    // A mask that hides no key before the entry's last visible one (right
    // padding, or no padding) is a shorter key length: such entries run the
    // unmasked steps with the keys ending at vis_hi, and the mask bytes are
    // not read again. The causal offset stays that of the padded length.
    const bool mask_is_length = !KMASK || first_hidden >= vis_hi;
    const int kend = KMASK && mask_is_length ? vis_hi : S_kv;   // keys at and past kend are never seen

    // tiles [lo, hi) of each block (walked from lo up), and how many of the
    // top ones cross the diagonal or the key end
    int hi_[2] = {0, 0}, lo_[2] = {0, 0}, nedge_[2] = {0, 0};
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
        if (ph < nblk) {
            const int qb = qbs[ph];
            int hi = tiles_for_block(qb, S_q, S_kv, causal);
            int full = kend / kTileN;   // tiles wholly inside the valid keys
            if (causal) {
                const int lim = qb * kTileM + off + 1;   // keys the block's first query sees
                full = min(full, lim > 0 ? lim / kTileN : 0);
            }
            if constexpr (KMASK) {
                hi = min(hi, (vis_hi + kTileN - 1) / kTileN);
                lo_[ph] = min(vis_lo / kTileN, hi);
            }
            hi_[ph] = hi;
            nedge_[ph] = hi - min(max(full, 0), hi);
        }
    }
    const int nt0 = hi_[0] - lo_[0];
    const int N = nt0 + hi_[1] - lo_[1];   // tiles in the item's stream
    auto stream_tile = [&](int j) __attribute__((always_inline)) {
        if constexpr (KMASK) return j < nt0 ? lo_[0] + j : lo_[1] + (j - nt0);
        return j < nt0 ? j : j - nt0;
    };

    // ---- per-lane load offsets (loop-invariant; the tile moves the descriptor)
    unsigned k_voff[C::K_SLOTS], v_voff[C::V_SLOTS];
    int nk_w = 0, nv_w = 0;   // this wave's loads per K / V tile
#pragma unroll
    for (int s = 0; s < C::K_SLOTS; ++s) {
        const int i = wave + kTileWaves * s;
        const int P = 64 * i + lane;            // 16-byte position in the stage
        const int R = P / (C::KCH + 1), col = P % (C::KCH + 1);
        const int key = (R & ~31) | swap_bits23(R & 31);
        k_voff[s] = col < C::KCH ? (unsigned)(key * HD2 + 16 * col) : 0x80000000u;   // pad: out of range
        nk_w += i < C::K_LOADS;
    }
#pragma unroll
    for (int s = 0; s < C::V_SLOTS; ++s) {
        const int i = wave + kTileWaves * s;
        const int P = 64 * i + lane;
        const int r = P / C::KCH, pc = P % C::KCH;
        const int chunk = pc ^ (vswz<D>(r) << 2);
        v_voff[s] = (unsigned)(r * HD2 + 16 * chunk);
        nv_w += i < C::V_LOADS;
    }
    // K and V rows of this (b, h): the head's first row, its valid bytes, and
    // the bytes of one tile of rows (all below 2^31, checked on the host)
    const size_t head_off = ((size_t)b * S_cap * H + h) * D * 2;
    const char* k_head = (const char*)K + head_off;
    const char* v_head = (const char*)V + head_off;
    const int head_bytes = ((kend - 1) * H + 1) * D * 2;
    const int tile_bytes = kTileN * HD2;

    // The rest of the kernel, instantiated with the per-step key-mask work
    // (KM) and without it.
    auto body = [&](auto km_) __attribute__((always_inline)) {
        constexpr bool KM = decltype(km_)::value;
        // descriptor of the rows of stream tile j; past the end of the stream its
        // range is 0, so the loads read nothing and land zeros in a stage that no
        // later step reads (every step then issues the same loads)
        auto tile_desc = [&](const char* head, int j) __attribute__((always_inline)) {
            const bool in = j < N;
            const int t = in ? stream_tile(j) : 0;
            const unsigned long long a = (unsigned long long)(head + (size_t)t * tile_bytes);
            const int rem = head_bytes - t * tile_bytes;
            const unsigned range = (in && rem > 0) ? (unsigned)rem : 0u;
            return (u32x4_t){(unsigned)a, (unsigned)(a >> 32) & 0xFFFFu, range, 0x00020000u};
        };
        // with a key mask, the mask bytes of stream tile j go with its K rows
        // into mask stage j % 4: one wave loads 256 bytes from the 4-byte
        // boundary at or below the tile's first byte (the range is rounded up to
        // 4 bytes, so no load reaches a page the row does not touch)
        auto issue_k = [&](int j) __attribute__((always_inline)) {
            const u32x4_t d = tile_desc(k_head, j);
            const unsigned base = lds_u + C::K_RING + (unsigned)(j % kPrefillStages) * C::K_STAGE + 1024u * wave;
#pragma unroll
            for (int s = 0; s < C::K_SLOTS; ++s) {
                if (s < C::K_LOADS / kTileWaves || wave < C::K_LOADS % kTileWaves)
                    lds_dma16(d, k_voff[s], base + 1024u * kTileWaves * s);
            }
            if constexpr (KM) {
                if (wave == kMaskWave) {
                    const bool in = j < N;
                    const int t = in ? stream_tile(j) : 0;
                    const unsigned long long a = (unsigned long long)(mrow - msh + (size_t)t * kTileN);
                    const int rem = msh + S_kv - t * kTileN;   // bytes from a to the row's end
                    const u32x4_t dm = {(unsigned)a, (unsigned)(a >> 32) & 0xFFFFu,
                                        (in && rem > 0) ? (unsigned)(rem + 3) & ~3u : 0u, 0x00020000u};
                    lds_dma4(dm, 4u * (unsigned)lane, lds_u + C::MASKS + (unsigned)(j & 3) * kPrefillMaskStageBytes);
                }
            }
        };
        // whether stream tile j holds a key the mask hides (wave-uniform): the
        // LDS word of its bit, and the bit's position (32: a tile past the
        // bits, taken as holding one)
        auto tile_word = [&](int j, int& bit) __attribute__((always_inline)) {
            const int t = j < N ? stream_tile(j) : 0;
            bit = t < kPrefillMaskTileBits ? (t & 31) : 32;
            return *(const unsigned*)(lds + C::TBITS + 4 * ((t < kPrefillMaskTileBits ? t : 0) >> 5));
        };
        auto tile_hides = [&](unsigned w, int bit) __attribute__((always_inline)) {
            return bit >= 32 ? 1 : (int)(((unsigned)__builtin_amdgcn_readfirstlane(w) >> bit) & 1u);
        };
        // the mask bytes of the V rows this lane loads for stream tile j (read
        // from LDS ahead of issue_v, so the read's latency is hidden)
        auto v_mask_words = [&](int j, unsigned (&mw)[C::V_SLOTS]) __attribute__((always_inline)) {
#pragma unroll
            for (int s = 0; s < C::V_SLOTS; ++s) {
                const int r = (64 * (wave + kTileWaves * s) + lane) / C::KCH;   // key row of the tile
                // (a lane with no load in this slot reads a byte it ignores)
                mw[s] = *(const unsigned char*)(lds + C::MASKS + (j & 3) * kPrefillMaskStageBytes + msh + (r & (kTileN - 1)));
            }
        };
        // V rows of hidden keys get an out-of-range offset and land as zeros, so
        // whatever a padding slot holds never reaches P.V
        auto issue_v = [&](int j, const unsigned (&mw)[C::V_SLOTS]) __attribute__((always_inline)) {
            const u32x4_t d = tile_desc(v_head, j);
            const unsigned base = lds_u + C::V_RING + (unsigned)(j % kPrefillStages) * C::V_STAGE + 1024u * wave;
#pragma unroll
            for (int s = 0; s < C::V_SLOTS; ++s) {
                if (s < C::V_LOADS / kTileWaves || wave < C::V_LOADS % kTileWaves) {
                    unsigned vo = v_voff[s];
                    if constexpr (KM) vo = (mw[s] & 0xFFu) != 0u ? vo : 0x80000000u;
                    lds_dma16(d, vo, base + 1024u * kTileWaves * s);
                }
            }
        };
        const int nld = nk_w + nv_w + (KM && wave == kMaskWave ? 1 : 0);   // this wave's loads per step

        // ---- per-lane operand offsets inside a stage
        const int k_lane = C::K_RING + (32 * half + l32) * C::KROW + 16 * g;
        int v_lane[C::DB];
        {
            // lane j of 16-lane group grp addresses head dims 16*(grp&1) + 4*(j&3)
            // .. +3 of key row j/4 (+ 8*(grp>>1), + 32*half): lane (l32, g) gets
            // head dim l32 of a 32-dim block for keys 8g..8g+3 of a 16-key step
            // (and 8g+4..8g+7 from the read 4 rows on), the key order of its P
            const int row0 = 32 * half + 8 * g + ((lane & 15) >> 2);
            const int sw = vswz<D>(row0);
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
                v_lane[db] = C::V_RING + row0 * C::VROW + 64 * (db ^ sw) + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
        }
        auto vt_operand = [&](int addr) __attribute__((always_inline)) {
            const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds + addr));
            const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds + addr + 4 * C::VROW));
            const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
            const u32x4_t w = {l2[0], l2[1], h2[0], h2[1]};
            return __builtin_bit_cast(v8, w);
        };

        // Q^T fragments of a block (B operand: lane holds query qi, head dims
        // 16*ks + 8*g .. +7); rows past S_q read as zeros
        v8 qf[C::KS];
        auto issue_q = [&](int qb) __attribute__((always_inline)) {
            const __amdgpu_buffer_rsrc_t dq = rsrc_of(head_rows<D>(Q, b, h, S_q, S_q, H, 0));
            const int qi = qb * kTileM + 32 * wq + l32;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks)
                qf[ks] = __builtin_bit_cast(
                    v8, __builtin_amdgcn_raw_buffer_load_b128(dq, (unsigned)(qi * HD2 + 16 * (2 * ks + g)), 0, 0));
        };
        // S^T (32 keys of this wave's half tile x 32 queries) = K . Q^T from the
        // K stage holding stream tile j
        auto qk_tile = [&](int j) __attribute__((always_inline)) {
            const char* kp = lds + k_lane + (j % kPrefillStages) * C::K_STAGE;
            f32x16_t s;
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) s = Mma<T>::mfma(*(const v8*)(kp + 32 * ks), qf[ks], s);
            return s;
        };

        const __amdgpu_buffer_rsrc_t d_o = rsrc_of(head_rows<D>(O, b, h, S_q, S_q, H, 0));

        // the V stage the first step's P.V (with P = 0) reads: finite zeros
        for (int i = tid; i < C::V_STAGE / 16; i += kTileThreads)
            *(u32x4_t*)(lds + C::V_RING + (kPrefillStages - 1) * C::V_STAGE + 16 * i) = (u32x4_t){0u, 0u, 0u, 0u};

        // ---- opening loads: Q of the first block, K of stream tiles 0..2, V of 0
        int hides_cur = 0;   // (key mask) the current step's tile holds a hidden key
        if constexpr (KM) {
            int bit;
            const unsigned w = tile_word(0, bit);
            hides_cur = tile_hides(w, bit);
        }
        unsigned vmw[C::V_SLOTS];
#pragma unroll
        for (int s = 0; s < C::V_SLOTS; ++s) vmw[s] = 1u;
        issue_q(qbs[0]);
        issue_k(0);
        issue_k(1);
        if constexpr (KM) {
            // V(0) needs tile 0's mask bytes in LDS first
            wait_vm_barrier(0);
            v_mask_words(0, vmw);
            issue_v(0, vmw);
            issue_k(2);
        } else {
            issue_v(0, vmw);
            issue_k(2);
            // K(0) and K(1) must be in before the first scores and the first step
            wait_vm_barrier(nld);
        }

        int j0 = 0;   // stream index of the block's first tile
        for (int ph = 0; ph < nblk; ++ph) {
            const int qb = qbs[ph];
            const int lo = lo_[ph];
            const int nt = hi_[ph] - lo;   // the block's steps
            const int n_edge = nedge_[ph];
            const int q0 = qb * kTileM + 32 * wq;    // first query of this wave
            const int qi = q0 + l32;                 // this lane's query
            const int lane_key_limit = causal ? qi + off : kend - 1;   // last key this lane sees
            const bool next_block = ph + 1 < nblk;

            if (nt == 0) {
                // no key is visible to any query of the block: zero rows
                if (half == 0) {
                    const T zero = (T)0.f;
                    const T z4[4] = {zero, zero, zero, zero};
#pragma unroll
                    for (int db = 0; db < C::DB; ++db)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, z4), d_o,
                                                                  (unsigned)(qi * HD2 + (32 * db + 8 * jj + 4 * g) * 2), 0, 0);
                    if (lse && g == 0 && qi < S_q) lse[((size_t)b * H + h) * S_q + qi] = -INFINITY;
                }
                if (next_block) {
                    issue_q(qbs[ph + 1]);
                    // the next block's first K tiles were issued with the opening loads
                    wait_vm_barrier(0);
                }
                continue;
            }

            f32x16_t acc[C::DB];
#pragma unroll
            for (int db = 0; db < C::DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
            float m_ref = -INFINITY;   // reference maximum of (score * c) for query qi
            float l_run = 0.f;         // this lane's share of the running sum
            v8 pb_prev[2];             // P of the previous step (B operands of P.V)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int i = 0; i < 8; ++i) pb_prev[s2][i] = (T)0.f;
            bool rescale_due = false;  // a re-base decided in the last step, applied to acc in this one
            float alpha_due = 1.f;

            auto apply_rescale = [&]() __attribute__((always_inline)) {
                if (rescale_due) {
#pragma unroll
                    for (int db = 0; db < C::DB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha_due;
                    rescale_due = false;
                }
            };

            // scores of the block's first tile (its K stage was published by the
            // previous step's barrier or by the opening wait); the first step's K
            // load lands in that stage, so every wave must be past the read
            f32x16_t sa = qk_tile(j0), sb;
            lds_barrier();

            // One step: s_c holds S(u); S(u+1) goes to s_n. Every wave computes
            // every tile of the block, also one whose keys all lie past its
            // queries: the step takes as long as its busiest SIMD, and in every
            // step of a block some SIMD has two waves with visible keys.
            auto step = [&](auto mfma_first_f, auto last_f, int u, f32x16_t& s_c, f32x16_t& s_n) __attribute__((always_inline)) {
                constexpr bool LAST = decltype(last_f)::value;   // no next tile in this block
                const int j = j0 + u;
                // the next block's Q: no MFMA of a block's last step reads Q, so
                // its loads go out a step before the merge (the step's barrier
                // lets them run on)
                if constexpr (LAST) {
                    if (next_block) issue_q(qbs[ph + 1]);
                }
                // this step's operand addresses: K of tile u+1, V of tile u-1
                const char* kp = lds + k_lane + ((j + 1) % kPrefillStages) * C::K_STAGE;
                int vaddr[C::DB];
                {
                    const int vs = ((j + kPrefillStages - 1) % kPrefillStages) * C::V_STAGE;
#pragma unroll
                    for (int db = 0; db < C::DB; ++db) vaddr[db] = v_lane[db] + vs;
                }
                // (b) the diagonal and the key end: -inf past this lane's last key
                const int kbase = (lo + u) * kTileN + 32 * half;   // first key of this wave's half tile
                // (key mask) the next tile's flag and V rows' mask bytes, read now
                // and used at the end of the step
                unsigned hw_next = 0u;
                int hbit_next = 0;
                if constexpr (KM) {
                    hw_next = tile_word(j + 1, hbit_next);
                    v_mask_words(j + 1, vmw);
                }
                if (KM && hides_cur) {
                    // a tile with hidden keys: -inf for them too, by a select, so
                    // a NaN score of a padding slot is dropped (this lane's keys
                    // are 32*half + 16*(r/8) + 8*g + r%8: two runs of 8 bytes,
                    // each read as 12 aligned bytes and shifted by msh)
                    const char* mp = lds + C::MASKS + (j & 3) * kPrefillMaskStageBytes + 32 * half + 8 * g;
                    const u32x2_t m0 = *(const u32x2_t*)mp, m1 = *(const u32x2_t*)(mp + 16);
                    const unsigned e0 = *(const unsigned*)(mp + 8), e1 = *(const unsigned*)(mp + 24);
                    const unsigned x0 = m0[0], x1 = m0[1], y0 = m1[0], y1 = m1[1];
                    const unsigned mb[4] = {__builtin_amdgcn_alignbyte(x1, x0, msh), __builtin_amdgcn_alignbyte(e0, x1, msh),
                                            __builtin_amdgcn_alignbyte(y1, y0, msh), __builtin_amdgcn_alignbyte(e1, y1, msh)};
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kbase + 16 * (r >> 3) + 8 * g + (r & 7);
                        const bool hide = (key > lane_key_limit) | (key >= kend) | (((mb[r >> 2] >> (8 * (r & 3))) & 0xFFu) == 0u);
                        s_c[r] = hide ? -INFINITY : s_c[r];
                    }
                } else if (u >= nt - n_edge && ((causal && kbase + 31 > q0 + off) || (kbase + 32 > kend))) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kbase + 16 * (r >> 3) + 8 * g + (r & 7);
                        if (key > lane_key_limit || key >= kend) s_c[r] = -INFINITY;
                    }
                }
                apply_rescale();
                // (c) the step's matrix-core and vector work. The MFMAs (P.V of
                // the previous tile, scores of the next) do not depend on this
                // step's softmax, so the two waves of a SIMD (key halves 0 and 1)
                // take them in opposite orders: one issues its MFMAs while the
                // other works through its softmax, then they swap.
                auto core = [&](auto mfma_first_f) __attribute__((always_inline)) {
                    constexpr bool MFMA_FIRST = decltype(mfma_first_f)::value;
                    v8 va[C::DB][2];
#pragma unroll
                    for (int db = 0; db < C::DB; ++db)
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2) va[db][s2] = vt_operand(vaddr[db] + 16 * s2 * C::VROW);
                    v8 ka[C::KS];
                    if constexpr (!LAST) {
#pragma unroll
                        for (int ks = 0; ks < C::KS; ++ks) ka[ks] = *(const v8*)(kp + 32 * ks);
                    }
                    // row max (one exchange with the partner lane l^32), lazy
                    // re-base. IEEE maximum: a NaN score gives a NaN maximum (and
                    // no re-base) rather than being skipped, and on gfx950 it is
                    // one three-input instruction per two scores, with no quieting
                    // of the matrix cores' results first
                    float mx = s_c[0];
#pragma unroll
                    for (int r = 1; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, s_c[r]);
                    mx = __builtin_elementwise_maximum(mx, partner_lane(mx)) * c;
                    const bool rebase = __builtin_amdgcn_ballot_w64(mx > m_ref + kLazy) != 0;
                    const float m_new = rebase ? fmaxf(m_ref, mx) : m_ref;
                    const float alpha =
                        (m_new == -INFINITY || !rebase) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
                    l_run *= alpha;
                    m_ref = m_new;
                    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
                    // O^T += V^T . P(u-1)^T (P = 0 in a block's first step); S(u+1)
#pragma unroll
                    for (int db = 0; db < C::DB; ++db)
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2) acc[db] = Mma<T>::mfma(va[db][s2], pb_prev[s2], acc[db]);
                    if constexpr (!LAST) {
                        f32x16_t sn;
#pragma unroll
                        for (int r = 0; r < 16; ++r) sn[r] = 0.f;
#pragma unroll
                        for (int ks = 0; ks < C::KS; ++ks) sn = Mma<T>::mfma(ka[ks], qf[ks], sn);
                        s_n = sn;
                    }
                    // P(u) rounded to the storage type; the row sum adds up the
                    // same rounded values, so the weights that multiply V are
                    // exactly normalised
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            pb_prev[s2][i] = (T)__builtin_amdgcn_exp2f(__builtin_fmaf(s_c[8 * s2 + i], c, -m_use));
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const v2 pair = {pb_prev[s2][2 * i], pb_prev[s2][2 * i + 1]};
                            l_run = Mma<T>::dot2(pair, kOnes2, l_run);
                        }
                    }
                    constexpr int NMF = 2 * C::DB + (LAST ? 0 : C::KS);   // MFMAs of the step
                    __builtin_amdgcn_sched_group_barrier(0x100, 4 * C::DB + (LAST ? 0 : C::KS), 0);   // operand reads
                    if constexpr (MFMA_FIRST) {
                        __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 256, 0);
                    } else {
                        __builtin_amdgcn_sched_group_barrier(0x002, 256, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, NMF, 0);
                    }
                    rescale_due = rebase;
                    alpha_due = alpha;
                };
                core(mfma_first_f);
                // (d) loads for later steps, issued once this step's MFMAs are
                // queued: K two steps ahead, V of the next tile
                issue_k(j + 3);
                issue_v(j + 1, vmw);
                if constexpr (KM) hides_cur = tile_hides(hw_next, hbit_next);
                // (e) this wave's loads of the previous step have landed; publish
                wait_vm_barrier(LAST && next_block ? nld + C::KS : nld);
            };

            // two steps per iteration, so S(u) and S(u+1) swap registers without
            // copies; then the last step. The key halves run separate copies of
            // the sequence (their steps differ only in the order of their work).
            auto run_steps = [&](auto mf) __attribute__((always_inline)) {
                int u = 0;
                for (; u + 2 < nt; u += 2) {
                    step(mf, Flag<false>(), u, sa, sb);
                    step(mf, Flag<false>(), u + 1, sb, sa);
                }
                if (u + 1 < nt) {
                    step(mf, Flag<false>(), u, sa, sb);
                    ++u;
                    sa = sb;
                }
                step(mf, Flag<true>(), u, sa, sb);
            };
            if (half == 0) run_steps(Flag<true>());
            else run_steps(Flag<false>());
            // the last P.V: V of the last tile was published by the last barrier
            apply_rescale();
            {
                const int vs = ((j0 + nt - 1) % kPrefillStages) * C::V_STAGE;
#pragma unroll
                for (int db = 0; db < C::DB; ++db)
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2)
                        acc[db] = Mma<T>::mfma(vt_operand(v_lane[db] + vs + 16 * s2 * C::VROW), pb_prev[s2], acc[db]);
            }

            // ---- merge the two key halves (waves wq and wq+4) through LDS.
            // With an even number of accumulator blocks both halves finalize:
            // in round rd half 0 writes O block rd and half 1 block DB/2 + rd,
            // each sending its partner the other one. Both compute the same
            // weights from the two (m, l) and the same fma(a0, x0, a1 * x1) with
            // x0 from half 0 and x1 from half 1, so which half finalizes a block
            // does not change its bits. (One 32-row block, D = 32: half 1 sends,
            // half 0 finalizes.)
            if constexpr (C::DB % 2 == 0) {
                constexpr int HB = C::DB / 2;
                // [half][wq][q4][lane] float4 parts of a block, then [half][wq][lane] (m, l)
                f32x4_t* const xs = (f32x4_t*)(lds + C::MERGE);
                f32x2_t* const mls = (f32x2_t*)(lds + C::MERGE + 2 * 4 * 4 * 64 * 16);
                static_assert(2 * 4 * 4 * 64 * 16 + 2 * 4 * 64 * 8 <= 4 * 64 * C::MREC * 4, "merge region fits");
                const int mine = half * 4 + wq, theirs = (1 - half) * 4 + wq;
                auto merge = [&](auto hf) __attribute__((always_inline)) {
                    constexpr int HF = decltype(hf)::value ? 1 : 0;   // this wave's key half
                    float a0 = 1.f, a1 = 0.f, inv = 0.f;
#pragma unroll
                    for (int rd = 0; rd < HB; ++rd) {
                        const int send = (1 - HF) * HB + rd, fin = HF * HB + rd;
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4)
                            xs[(mine * 4 + q4) * 64 + lane] = (f32x4_t){acc[send][4 * q4], acc[send][4 * q4 + 1],
                                                                        acc[send][4 * q4 + 2], acc[send][4 * q4 + 3]};
                        if (rd == 0) mls[mine * 64 + lane] = (f32x2_t){m_ref, l_run};
                        lds_barrier();
                        if (rd == 0) {
                            const f32x2_t ml = mls[theirs * 64 + lane];
                            const float m0 = HF == 0 ? m_ref : ml[0], l0 = HF == 0 ? l_run : ml[1];
                            const float m1 = HF == 0 ? ml[0] : m_ref, l1 = HF == 0 ? ml[1] : l_run;
                            const float m = fmaxf(m0, m1);
                            const float mu = (m == -INFINITY) ? 0.f : m;
                            a0 = __builtin_amdgcn_exp2f(m0 - mu);
                            a1 = __builtin_amdgcn_exp2f(m1 - mu);
                            float l = __builtin_fmaf(a0, l0, a1 * l1);
                            l += partner_lane(l);
                            inv = l > 0.f ? 1.0f / l : 0.f;
                            if (HF == 0 && lse && g == 0 && qi < S_q)
                                lse[((size_t)b * H + h) * S_q + qi] =
                                    l > 0.f ? (mu + __builtin_log2f(l)) * 0.69314718055994531f : -INFINITY;
                        }
                        f32x4_t part[4];
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) part[q4] = xs[(theirs * 4 + q4) * 64 + lane];
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            T ob[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float x0 = HF == 0 ? acc[fin][4 * q4 + e] : part[q4][e];
                                const float x1 = HF == 0 ? part[q4][e] : acc[fin][4 * q4 + e];
                                ob[e] = (T)(__builtin_fmaf(a0, x0, a1 * x1) * inv);
                            }
                            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, ob), d_o,
                                                                  (unsigned)(qi * HD2 + (32 * fin + 8 * q4 + 4 * g) * 2), 0, 0);
                        }
                        if (rd + 1 < HB) lds_barrier();   // the parts are rewritten by the next round
                    }
                };
                if (half == 0) merge(Flag<false>());
                else merge(Flag<true>());
            } else {
                // ---- merge the two key halves (waves wq and wq+4) through LDS, in
                // rounds of MDB accumulator blocks; half 0 writes the block's rows
                float* rec = (float*)(lds + C::MERGE) + (wq * 64 + lane) * C::MREC;
                float a0 = 1.f, a1 = 0.f, inv = 0.f;
#pragma unroll
                for (int rd = 0; rd < C::ROUNDS; ++rd) {
                    if (half == 1) {
#pragma unroll
                        for (int x = 0; x < C::MDB; ++x)
#pragma unroll
                            for (int q4 = 0; q4 < 4; ++q4) {
                                const f32x4_t w = {acc[rd * C::MDB + x][4 * q4], acc[rd * C::MDB + x][4 * q4 + 1],
                                                   acc[rd * C::MDB + x][4 * q4 + 2], acc[rd * C::MDB + x][4 * q4 + 3]};
                                *(f32x4_t*)(rec + 16 * x + 4 * q4) = w;
                            }
                        if (rd == 0) *(f32x2_t*)(rec + 16 * C::MDB) = (f32x2_t){m_ref, l_run};
                    }
                    lds_barrier();
                    if (half == 0) {
                        if (rd == 0) {
                            const f32x2_t ml = *(const f32x2_t*)(rec + 16 * C::MDB);
                            const float m1 = ml[0];
                            const float l1 = ml[1];
                            const float m = fmaxf(m_ref, m1);
                            const float mu = (m == -INFINITY) ? 0.f : m;
                            a0 = __builtin_amdgcn_exp2f(m_ref - mu);
                            a1 = __builtin_amdgcn_exp2f(m1 - mu);
                            // (both weighted sums are written as one explicit fma, so
                            // every instantiation rounds them the same way)
                            float l = __builtin_fmaf(a0, l_run, a1 * l1);
                            l += partner_lane(l);
                            // a row that sees no key (a cache entry shorter than the chunk) is 0
                            inv = l > 0.f ? 1.0f / l : 0.f;
                            // log of the softmax denominator in natural units: ln 2 * (m + log2 l)
                            if (lse && g == 0 && qi < S_q)
                                lse[((size_t)b * H + h) * S_q + qi] =
                                    l > 0.f ? (mu + __builtin_log2f(l)) * 0.69314718055994531f : -INFINITY;
                        }
                        f32x4_t part[C::MDB][4];
#pragma unroll
                        for (int x = 0; x < C::MDB; ++x)
#pragma unroll
                            for (int q4 = 0; q4 < 4; ++q4) part[x][q4] = *(const f32x4_t*)(rec + 16 * x + 4 * q4);
#pragma unroll
                        for (int x = 0; x < C::MDB; ++x) {
                            const int db = rd * C::MDB + x;
#pragma unroll
                            for (int q4 = 0; q4 < 4; ++q4) {
                                T ob[4];
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    ob[e] = (T)(__builtin_fmaf(a0, acc[db][4 * q4 + e], a1 * part[x][q4][e]) * inv);
                                // lane holds head dims 32*db + 8*q4 + 4*g .. +3 of its
                                // query; rows past S_q fall outside the descriptor
                                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, ob), d_o,
                                                                      (unsigned)(qi * HD2 + (32 * db + 8 * q4 + 4 * g) * 2), 0, 0);
                            }
                        }
                    }
                    if (rd + 1 < C::ROUNDS) lds_barrier();   // the record is rewritten by the next round
                }
            }
            j0 += nt;
        }
    };
    if constexpr (KMASK) {
        if (mask_is_length) body(Flag<false>());
        else body(Flag<true>());
    } else {
        body(Flag<false>());
    }
    if (clk && blockIdx.x == 0 && tid == 0) {
        clk[2] = __builtin_amdgcn_s_memtime();
        clk[3] = __builtin_amdgcn_s_memrealtime();
    }
}

template <typename T, int D, bool KMASK>
hipError_t launch_m(const FwdArgs& a, hipStream_t stream) {
    const TileGrid tg = tile_grid(a.B, a.H, a.S_q, a.causal, a.kv_lens != nullptr);
    hipExtLaunchKernelGGL((prefill_kernel<T, D, KMASK>), dim3((unsigned)tg.n_items), dim3(kTileThreads), 0, stream,
                          a.ev_start, a.ev_stop, 0, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                          (T*)a.o, a.B, a.H, a.S_q, a.S_kv, a.causal, a.scale_log2, tg.n_qblk, tg.items_per_bh,
                          tg.paired, a.kv_lens, a.lse, a.clock_probe, a.key_mask);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
    // the mask comes without per-entry lengths (attn_fwd_mask)
    if (a.key_mask) return a.kv_lens ? hipErrorInvalidValue : launch_m<T, D, true>(a, stream);
    return launch_m<T, D, false>(a, stream);
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

hipError_t launch_fwd_prefill(const FwdArgs& a, Elt t, hipStream_t stream) {
    switch (t) {
        case Elt::BF16: return launch_t<__bf16>(a, stream);
        case Elt::F16: return launch_t<_Float16>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace attn

