// plan.h -- launch geometry shared by the host planner and the kernels.
//
// Everything here is a pure function of the problem sizes, so the host can
// compute (and the CPU tests can check) exactly what a kernel will do.
#pragma once

#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define ATTN_HD __host__ __device__
#else
#define ATTN_HD
#endif

namespace attn {

// ---------------------------------------------------------------------------
// MFMA prefill kernel (bf16 or fp16 storage): work items and tiles.
//   A work item is one (b, h, query block of BM rows); with the causal mask,
//   query blocks r and n-1-r share one workgroup so every workgroup visits
//   the same number of KV tiles (the causal triangle folded in half).
//   Eight waves, two per SIMD: wave w covers queries 32*(w%4) .. +31 of the
//   block and the key half w/4 of every 64-key tile.
// ---------------------------------------------------------------------------
constexpr int kTileM = 128;     // queries per block
constexpr int kTileN = 64;      // keys per KV tile
constexpr int kTileWaves = 8;
constexpr int kTileThreads = kTileWaves * 64;

constexpr int kNumXcd = 8;      // MI355X: 8 XCDs, workgroups dealt round-robin

// Hardware workgroup x (of n) runs on XCD x % 8. Return a logical id such
// that each XCD receives a contiguous range of logical ids (so neighbouring
// work items -- the blocks of one head -- share that XCD's L2).
ATTN_HD inline int xcd_remap(int x, int n) {
    if (n <= kNumXcd) return x;
    const int per = (n + kNumXcd - 1) / kNumXcd;   // ids on the "tall" XCDs
    int tall = n % kNumXcd;
    if (tall == 0) tall = kNumXcd;
    const int xcd = x % kNumXcd;
    const int local = x / kNumXcd;
    if (xcd < tall) return xcd * per + local;
    return tall * per + (xcd - tall) * (per - 1) + local;
}

// Prefill kernel (attn_fwd, attn_fwd_kvcache, attn_fwd_mask; fwd_prefill.hip):
// items, waves and tiles as above, with K and V tiles loaded straight into a
// ring of kPrefillStages LDS stages. K rows are padded by 16 bytes; V rows are
// unpadded (their 16-byte chunks swizzled instead). The key-half merge goes
// through its own region of 4 * 64 * prefill_merge_rec_floats(D) floats:
// with D >= 64 each half sends its partner one 32-row block of the
// accumulator per round (2 * 4 waves * 64 lanes * 16 floats) plus (m, l);
// with D = 32 one record of 16 + 4 floats per lane of the key-half-1 waves.
constexpr int kPrefillStages = 3;
ATTN_HD constexpr int prefill_krow_bytes(int D) { return 2 * D + 16; }
ATTN_HD constexpr int prefill_k_stage_bytes(int D) { return kTileN * (2 * D + 16); }
ATTN_HD constexpr int prefill_v_stage_bytes(int D) { return kTileN * 2 * D; }
ATTN_HD constexpr int prefill_merge_db(int D) { return D / 32 < 2 ? D / 32 : 2; }
ATTN_HD constexpr int prefill_merge_rec_floats(int D) { return 16 * prefill_merge_db(D) + 4; }
ATTN_HD constexpr int prefill_lds_bytes(int D) {
    return kPrefillStages * (prefill_k_stage_bytes(D) + prefill_v_stage_bytes(D)) +
           4 * 64 * prefill_merge_rec_floats(D) * 4;
}

// With a key-padding mask (attn_fwd_mask) the prefill kernel adds four
// key-mask stages of 256 bytes (64 lanes x 4 bytes, of which a tile's 64
// mask bytes and up to 3 bytes of alignment are used) and one bit per key
// tile of the entry, set where the tile holds a hidden key, for the first
// kPrefillMaskTileBits tiles (later tiles count as holding one).
constexpr int kPrefillMaskStages = 4;
constexpr int kPrefillMaskStageBytes = 4 * kTileN;
constexpr int kPrefillMaskTileBits = 16384;
ATTN_HD constexpr int prefill_lds_bytes_kmask(int D) {
    return prefill_lds_bytes(D) + kPrefillMaskStages * kPrefillMaskStageBytes + kPrefillMaskTileBits / 8;
}

// Number of KV tiles query block qb must visit.
ATTN_HD inline int tiles_for_block(int qb, int S_q, int S_kv, int causal) {
    const int n_all = (S_kv + kTileN - 1) / kTileN;
    if (!causal) return n_all;
    int last_q = (qb + 1) * kTileM - 1;
    if (last_q > S_q - 1) last_q = S_q - 1;
    const int last_key = last_q + (S_kv - S_q);
    if (last_key < 0) return 0;   // no query of the block sees any key (S_kv < S_q)
    const int n = last_key / kTileN + 1;
    return n < n_all ? n : n_all;
}

struct TileGrid {
    int n_qblk;         // query blocks per (b, h)
    int items_per_bh;   // work items per (b, h)
    int paired;         // 1: item p runs blocks n-1-p then p
    long long n_items;  // total workgroups
};

// Pairing evens out the causal triangle of a square (or nearly square)
// problem, where query block j sees about j+1 key tiles. Without the causal
// rule every block sees the same tiles; pairing then halves the number of
// workgroups, so each one pays the fixed costs of a block (the opening loads,
// a key-mask scan) once for two blocks and loads its second block under the
// first one's merge. With per-entry cache lengths the chunk is usually short
// against the cache, every block of an entry sees nearly the same number of
// tiles, and pairing only doubles the longest workgroup; such launches run
// one block per workgroup.
ATTN_HD inline TileGrid tile_grid(int B, int H, int S_q, int causal, bool kv_lengths = false) {
    (void)causal;
    TileGrid g;
    g.n_qblk = (S_q + kTileM - 1) / kTileM;
    g.paired = kv_lengths ? 0 : 1;
    g.items_per_bh = g.paired ? (g.n_qblk + 1) / 2 : g.n_qblk;
    g.n_items = (long long)B * H * g.items_per_bh;
    return g;
}

// ---------------------------------------------------------------------------
// Row kernel (the ATTN_ALGO=row cross-check path, any storage type): one
// wave per query.
// ---------------------------------------------------------------------------
constexpr int kRowThreads = 64;

// ---------------------------------------------------------------------------
// fp32 MFMA kernel: one workgroup per (b, h, block of kF32Q queries); its
// eight waves take the block's kF32N-key tiles round-robin.
// ---------------------------------------------------------------------------
constexpr int kF32Q = 32;
constexpr int kF32N = 32;
constexpr int kF32Threads = 512;

// ---------------------------------------------------------------------------
// Split-KV decode, one kernel.
//   The valid keys of all sequences, laid end to end, form one token space
//   of T = sum of the lengths. Workgroup w (of kDecodeSplitWGs) takes one
//   contiguous range of it (decode_range_start below), in order, and a
//   range that crosses a sequence boundary is processed as one segment per
//   sequence. Each
//   workgroup covers ALL heads of its keys: each wave owns a group of heads,
//   each load instruction reads one token's rows of those heads (contiguous
//   bytes). A segment that holds a whole sequence writes its output rows
//   directly; any other segment (w, b) leaves one partial record per head at
//   record index w + b (unique: see decode.hip) and raises one flag per head
//   group. Merging workgroups, launched after the streaming ones, take the
//   (sequence, head group) pairs cut into several segments and merge their
//   records once the segments' flags are raised.
// ---------------------------------------------------------------------------
constexpr int kDecodeWaves = 8;
constexpr int kDecodeSplitWGs = 256;      // one per CU of the chip
constexpr int kDecodeBatch = 8;           // keys whose loads are in flight together
constexpr int kDecodeThreads = kDecodeWaves * 64;
constexpr int kDecodeScanLds = 1024;      // length prefix sums kept in LDS up to this many sequences
constexpr int kDecodeMergeWGs = 256;      // merging workgroups at most (one per (sequence, head group) pair)
constexpr int kDecodeMergeBatch = 8;      // records whose loads are in flight together in a merge
constexpr int kDecodeSpinLimit = 1 << 22;  // polls of the segments' flags before a merge gives up (seconds)

// The streaming workgroups' ranges. Workgroups are dealt to the XCDs
// round-robin, so workgroup w runs on XCD w % 8, and on MI355X the odd XCDs
// stream about 8% slower than the even ones (a plain read in the decode's
// pattern shows it, and it stays with the XCD when every workgroup's range
// is moved to its neighbour). So each pair of workgroups (2p, 2p+1) shares
// a span of decode_pair_span(T) tokens unequally: the even one takes
// kDecodeEvenPermille / 1000 of it, rounded up, the odd one the rest. With
// T <= kDecodeSplitWGs tokens, workgroup w takes token w alone.
// The ranges tile [0, T) in workgroup order, and the empty ones come last
// (the spans are then at least 3 tokens, of which each side takes one or
// more): every workgroup between the first and the last of a sequence holds
// some of its keys, as the merge assumes.
constexpr int kDecodeEvenPermille = 530;
ATTN_HD inline int decode_pair_span(int T) {
    return (int)(((long long)T + kDecodeSplitWGs / 2 - 1) / (kDecodeSplitWGs / 2));
}
ATTN_HD inline int decode_even_part(int span) {   // for span >= 3: in [1, span - 1]
    return (int)(((long long)span * kDecodeEvenPermille + 999) / 1000);
}
// First token of workgroup w's range, for 0 <= w <= kDecodeSplitWGs (w =
// kDecodeSplitWGs gives T, the end of the last range).
ATTN_HD inline int decode_range_start(int w, int T) {
    if (T <= kDecodeSplitWGs) return w < T ? w : T;
    const int span = decode_pair_span(T);
    const long long s = (long long)(w >> 1) * span + ((w & 1) ? decode_even_part(span) : 0);
    return s < T ? (int)s : T;
}
// The workgroup whose range holds token t, for 0 <= t < T.
ATTN_HD inline int decode_range_of(int t, int T) {
    if (T <= kDecodeSplitWGs) return t;
    const int span = decode_pair_span(T);
    const int p = t / span;
    return 2 * p + (t - p * span >= decode_even_part(span) ? 1 : 0);
}

// Partial records: segment (w, b) uses index w + b, so at most
// kDecodeSplitWGs + B - 1 of them.
ATTN_HD inline long long decode_records(int B) {
    return (long long)kDecodeSplitWGs + B - 1;
}

// One partial record per (record, h): max, sum, two pad floats, then D
// accumulators, so the accumulators start 16-byte aligned.
ATTN_HD constexpr int decode_record_floats(int D) { return D + 4; }

// Workspace: the records, then one 64-bit flag per (record, h) (a head group
// uses the slot of its group index, and there are never more groups than
// heads). It does not depend on the cache capacity.
ATTN_HD inline size_t decode_records_bytes(int B, int H, int D) {
    return (size_t)decode_records(B) * (size_t)H * (size_t)decode_record_floats(D) * sizeof(float);
}
ATTN_HD inline size_t decode_workspace_bytes(int B, int H, int /*S_cap*/, int D) {
    return decode_records_bytes(B, H, D) + (size_t)decode_records(B) * (size_t)H * sizeof(unsigned long long);
}

// The allocation-free decode's fixed workspace (one per GPU): at most this
// many bytes of records and flags, e.g. B <= 722 sequences at H = 32, D = 128.
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;

// ---------------------------------------------------------------------------
// Q/K/V projection GEMM: 256 x 384 tiles of C = X W^T, 32-wide K steps,
// eight waves in a 2 x 4 grid (128 x 96 outputs each).
// ---------------------------------------------------------------------------
constexpr int kGemmBM = 256;
constexpr int kGemmBN = 384;
constexpr int kGemmBK = 32;
constexpr int kGemmWavesM = 2;
constexpr int kGemmWavesN = 4;
constexpr int kGemmThreads = kGemmWavesM * kGemmWavesN * 64;

// Sinusoidal position encoding: 256 threads, two frequency pairs each, and 4
// positions per workgroup (a 4096 x 4096 table is 1,024 x 4 workgroups; 8 or
// 16 positions per workgroup measured slower).
constexpr int kPeThreads = 256;
constexpr int kPeRows = 4;
ATTN_HD inline long long pe_grid_chunks(int d_model) {
    return ((long long)d_model / 2 + 2 * kPeThreads - 1) / (2 * kPeThreads);
}

// Masked softmax: one wave per row, kSmRowsPerBlock rows per workgroup. A
// lane holds up to kSmChunksMax 16-byte chunks of its row in registers, so a
// row is at most 64 * 16 * kSmChunksMax bytes (4096 fp32 or 8192 16-bit
// scores); rows of at most 64 * 16 * kSmChunksSmall bytes use a variant with
// fewer registers and more waves in flight.
constexpr int kSmRowsPerBlock = 4;
constexpr int kSmThreads = kSmRowsPerBlock * 64;
constexpr int kSmChunksSmall = 4;
constexpr int kSmChunksMax = 16;
constexpr long long kSmMaxRowBytes = 64LL * 16 * kSmChunksMax;

ATTN_HD inline long long qkv_grid(int M, int N) {
    return (long long)((M + kGemmBM - 1) / kGemmBM) * ((3LL * N + kGemmBN - 1) / kGemmBN);
}

}  // namespace attn
