/*
 * attn.h -- C ABI of the gfx950 (MI355X) causal multi-head attention library
 * (libattn.so).
 *
 * Operation. For every batch b and head h:
 *
 *     O = softmax(Q K^T / sqrt(D) + M) V
 *
 * with M the causal mask (0 where key j is visible to query i, -inf
 * elsewhere). This is the masked multi-head attention of the "Hand-written
 * Masked Multi-Head Attention CUDA kernel" page, section 2 (the page's
 * "O = AV^T" is read as O = A.V), computed the fused way that page's
 * section 2.2 and the "Week-4 CUDA notes" page, section 2.2 describe: the
 * score matrix never reaches device memory and the softmax is the one-pass
 * online form (running max and running sum).
 *
 * Conventions shared by every entry point
 *  - Tensors are dense, row-major [B, S, H, D] (batch, position, head,
 *    head_dim): MMHA page, section 2.1. Every pointer is a DEVICE pointer
 *    that stays owned by the caller; the library allocates no device memory
 *    and keeps no state besides a per-thread stream and error message.
 *  - Calls are asynchronous: they enqueue kernels on the calling thread's
 *    stream (attn_set_stream; default: the null stream) and return. A fault
 *    inside a kernel surfaces at the caller's next synchronisation.
 *  - Every entry point returns an attn_status_t. Arguments are validated on
 *    the host before any HIP call; a rejected call touches no memory and
 *    launches nothing. attn_last_error() then holds a readable reason.
 *    No C++ exception crosses this boundary and nothing aborts the process.
 *  - Data pointers must be 16-byte aligned (the kernels move 128-bit
 *    vectors: "Week-4 CUDA notes" page, section 1.2), the output must not
 *    overlap any input, and a pointer may be NULL only when its tensor has
 *    no elements.
 *  - Causal visibility (MMHA page, section 2.2: key j visible iff j <= i)
 *    with S_q <= S_kv places the S_q queries at the END of the key sequence:
 *    query i is at absolute position i + (S_kv - S_q) and sees keys
 *    j <= i + S_kv - S_q. With S_q == S_kv this is exactly j <= i.
 *  - Debug check: with the environment variable ATTN_CHECK=1, attn_decode
 *    and attn_fwd_kvcache first copy their device-side lengths to the host
 *    (a synchronous copy on the calling thread's stream, so not for code
 *    under graph capture) and reject with ATTN_ERR_INVALID_ARG any length
 *    below 0 or above the cache capacity, values the kernels would otherwise
 *    clamp. The check runs after the other argument checks, before the launch.
 *  - Arithmetic: scores, softmax and accumulation in fp32 whatever the
 *    storage type (MMHA page, section 3.3); the scale 1/sqrt(D) is an fp32
 *    value. bf16 results are rounded to nearest even.
 *  - Memory a call does not use -- cache rows past a length, padded tails,
 *    the K and V rows of keys a key mask hides -- never reaches a result and
 *    may hold anything, NaN and infinities included. Non-finite values in
 *    the data a call does use are not screened: they propagate into the
 *    affected output rows as IEEE arithmetic has it (a NaN score or value
 *    gives a NaN row).
 */
#ifndef ATTN_GFX950_H
#define ATTN_GFX950_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of q, k, v and o (and the caches). Arithmetic is fp32 in
 * every case; with ATTN_BF16 and ATTN_F16 the probabilities enter the P.V
 * product rounded to the same 16-bit type. ATTN_F16 is the half-precision
 * storage of the MMHA page, section 3.3. */
typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1, ATTN_F16 = 2 } attn_dtype_t;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARG = 1, /* bad size, pointer, alignment, aliasing or flag  */
    ATTN_ERR_UNSUPPORTED = 2, /* valid request outside what is built (D, dtype)  */
    ATTN_ERR_WORKSPACE = 3,   /* decode workspace missing or too small           */
    ATTN_ERR_HIP = 4          /* the HIP runtime reported an error at launch     */
} attn_status_t;

/*
 * attn_fwd -- fused masked multi-head attention forward (prefill).
 * Definition: MMHA page, section 2; fusion of QK^T, mask, softmax and P.V
 * in one kernel: MMHA page, sections 2.2 and 3, and "Week-4 CUDA notes"
 * page, section 2.2 (online softmax).
 *
 *   q : [B, S_q,  H, D]   k, v : [B, S_kv, H, D]   o : [B, S_q, H, D]
 *   All four have element type `dtype` (ATTN_F32, ATTN_BF16 or ATTN_F16).
 *   D must be 32, 64 or 128 (else ATTN_ERR_UNSUPPORTED).
 *   causal: 1 applies the mask above (requires S_q <= S_kv), 0 lets every
 *   query see all S_kv keys. Any other value is ATTN_ERR_INVALID_ARG.
 *   B, H or S_q equal to 0 is a valid empty call (nothing is launched);
 *   S_kv == 0 with a non-empty output is ATTN_ERR_INVALID_ARG (no keys to
 *   attend to). Negative sizes are ATTN_ERR_INVALID_ARG.
 *   o may not overlap q, k or v; q, k and v may alias each other.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int S_q,
             int S_kv, int D, int causal, int dtype);

/*
 * attn_fwd_kvcache -- attn_fwd for a chunk of new queries against a KV cache
 * with per-sequence lengths (chunked prefill), optionally returning the
 * log-sum-exp of each query row. Definition: the masked attention of the
 * MMHA page, section 2, applied per batch entry to the cache rows that are
 * valid for it; positions follow the bottom-right rule above with S_kv taken
 * per entry. The log-sum-exp is the log of the softmax denominator (the
 * running-sum state of the "Week-4 CUDA notes" page, section 2.2), which lets
 * partial results over disjoint key sets be merged later.
 *
 *   q, o        : [B, S_q, H, D]   the new queries (their keys and values are
 *                 expected to be in the cache already, at the end of each
 *                 entry's valid rows)
 *   kcache, vcache : [B, S_cap, H, D]
 *   seqlens_kv  : DEVICE int32[B] or NULL. Entry b's valid rows are
 *                 0 .. len_b-1, len_b = seqlens_kv[b] clamped to [0, S_cap]
 *                 (NULL: len_b = S_cap). Query i of entry b sits at position
 *                 len_b - S_q + i; causal=1 lets it see keys j <= that
 *                 position, causal=0 all len_b keys. A query that sees no key
 *                 (len_b < S_q, or len_b == 0) gets an all-zero output row and
 *                 a log-sum-exp of -inf. Rows at or past len_b are never read.
 *   lse         : DEVICE float [B, H, S_q] or NULL: ln(sum_j exp(q.k_j/sqrt(D)))
 *                 over the keys the query sees.
 *   dtype, D    : as attn_fwd (ATTN_F32, ATTN_BF16 or ATTN_F16; D in {32, 64, 128}).
 *   B, H or S_q equal to 0 is a valid empty call; S_cap must then be >= 0,
 *   otherwise >= 1. o may not overlap any other argument, nor lse any input.
 * With seqlens_kv = NULL and S_q <= S_cap this is attn_fwd (S_kv = S_cap)
 * plus the log-sum-exp, and o is bit-identical to attn_fwd's.
 */
int attn_fwd_kvcache(const void* q, const void* kcache, const void* vcache, const int32_t* seqlens_kv,
                     void* o, float* lse, int B, int H, int S_q, int S_cap, int D, int causal, int dtype);

/*
 * attn_fwd_mask -- attn_fwd with a key-padding mask, optionally returning
 * the log-sum-exp of each query row. A hidden key's score is -inf, so its
 * weight is exactly 0 ("Week-4 CUDA notes" page, section 2.2, for padded
 * positions); the mask combines with the causal rule of attn_fwd.
 *
 *   q, k, v, o, B, H, S_q, S_kv, D, causal, dtype : as attn_fwd
 *   key_mask : DEVICE uint8 [B, S_kv] or NULL; key_mask[b*S_kv + j] == 0
 *              hides key j of entry b from every query of that entry (any
 *              other value: visible). NULL hides nothing. No alignment is
 *              required.
 *   lse      : DEVICE float [B, H, S_q] or NULL, as attn_fwd_kvcache.
 * A query row left with no visible key gets an all-zero output row and a
 * log-sum-exp of -inf. Hidden keys' K and V rows never reach the result
 * (their scores are replaced by -inf by selection, and their V rows are
 * loaded as zeros or skipped), so padding slots may hold anything, NaN
 * included. o may not overlap any other argument, nor lse any input.
 */
int attn_fwd_mask(const void* q, const void* k, const void* v, const uint8_t* key_mask, void* o,
                  float* lse, int B, int H, int S_q, int S_kv, int D, int causal, int dtype);

/*
 * attn_decode_workspace_bytes -- device workspace attn_decode needs for
 * these sizes: (256 + B - 1) * H partial records of D + 4 floats (max, sum,
 * two pad floats, D accumulators), then (256 + B - 1) * H 64-bit flags. It
 * does not depend on S_cap. Returns 0 for invalid or empty sizes. The size
 * and the planning split follow the host-side shape checks of the
 * depthwise-convolution page, section 6.2.
 */
size_t attn_decode_workspace_bytes(int B, int H, int S_cap, int D);

/*
 * attn_decode -- single-query (GEMV-shaped) masked attention against a KV
 * cache: the per-query mapping of the MMHA page, section 2.1, with the
 * keys split across workgroups and the partial softmax states merged
 * afterwards (rows spanning several blocks need one common normaliser:
 * "Week-4 CUDA notes" page, section 2.2). The valid keys of all sequences,
 * laid end to end, are cut into 256 equal ranges, one workgroup each, so
 * the work is balanced whatever the length mix. One kernel launch: a
 * sequence cut into several ranges is merged by extra workgroups of the
 * same launch once the ranges' flags in the workspace are raised.
 *
 *   q, o            : [B, 1, H, D]
 *   kcache, vcache  : [B, S_cap, H, D]
 *   seqlens         : DEVICE int32[B]; query b attends cache slots
 *                     0 .. seqlens[b]-1 (it is the last position, so the
 *                     causal mask admits all of them). It is read on the
 *                     device only: a value <= 0 produces an all-zero output
 *                     row and a value > S_cap is treated as S_cap. Slots at
 *                     or beyond the length are never read, so they may
 *                     hold anything, NaN included.
 *   workspace       : DEVICE buffer of at least
 *                     attn_decode_workspace_bytes(B, H, S_cap, D) bytes,
 *                     16-byte aligned; any contents on entry are fine (each
 *                     call marks its flags with its own 64-bit value, and a
 *                     stale word matches it with odds 2^-64). Every flag a
 *                     call raises is zero again when it ends, so a captured
 *                     launch replayed from a graph is also correct. Calls
 *                     that share a workspace must be ordered on one stream:
 *                     overlapping calls on one workspace race.
 *   dtype           : ATTN_F32, ATTN_BF16 or ATTN_F16 for q, caches and o.
 *   D must be 32, 64 or 128. B == 0 or H == 0 is a valid empty call;
 *   S_cap must be >= 1 and B * S_cap below 2^31. o may not overlap any
 *   other argument.
 * A too-small or NULL workspace returns ATTN_ERR_WORKSPACE.
 */
int attn_decode(const void* q, const void* kcache, const void* vcache, const int32_t* seqlens,
                void* o, int B, int H, int S_cap, int D, int dtype, void* workspace,
                size_t workspace_bytes);

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same kernel and results, with no workspace argument.
 * Its workspace is the library's own fixed array in device memory, 16 MiB per
 * GPU (kDecodeScratchBytes), looked up once per device and kept until the
 * process ends; the call allocates nothing. Sizes whose workspace
 * (attn_decode_workspace_bytes) exceeds it return ATTN_ERR_WORKSPACE (about
 * B <= 722 sequences at H = 32, D = 128). Every call on a GPU shares that
 * GPU's array: calls that overlap on one GPU (two streams, two threads) race
 * and must be ordered by the caller. Arguments and errors otherwise as
 * attn_decode (the ATTN_CHECK length copy is not made here).
 */
int attn_decode_noalloc(const void* q, const void* kcache, const void* vcache, const int32_t* seqlens,
                        void* o, int B, int H, int S_cap, int D, int dtype);

/*
 * attn_qkv_proj -- the Q, K and V projections of the input rows as one GEMM
 * over the stacked weights: Q = X W_Q, K = X W_K, V = X W_V (MMHA page,
 * section 2), concatenated into a single GEMM ("Week-4 CUDA notes" page,
 * section 2.1). fp32 accumulation, outputs rounded to the storage type.
 *
 *   x       : [M, E]       input rows (M = B*S tokens), DEVICE
 *   w       : [3*H*D, E]   stacked weights, output-major (the layout of a
 *                          linear layer's weight): row c*H*D + n holds the E
 *                          weights of output column n of Q (c = 0), K (1) or
 *                          V (2), so q[m][n] = sum_e x[m][e] * w[n][e], DEVICE
 *   q, k, v : [M, H*D] each = [B, S, H, D], the inputs of attn_fwd, DEVICE
 *   dtype   : ATTN_BF16 or ATTN_F16 for all five (else ATTN_ERR_UNSUPPORTED).
 *   E must be a multiple of 32 and H*D of 32 (else ATTN_ERR_UNSUPPORTED).
 *   M == 0 is a valid empty call. Pointers 16-byte aligned; no output may
 *   overlap an input or another output.
 */
int attn_qkv_proj(const void* x, const void* w, void* q, void* k, void* v, int M, int E, int H, int D,
                  int dtype);

/*
 * attn_masked_softmax -- row softmax of a materialised score matrix under
 * the causal rule, the stage the MMHA page's section 1 describes on its
 * own, with the masked positions at -inf ("Week-4 CUDA notes" page,
 * section 2.2):
 *
 *     p[i][j] = exp(scale*s[i][j] - m_i) / sum_j' exp(scale*s[i][j'] - m_i)
 *
 * over the keys j that row i sees (m_i their maximum) and 0 elsewhere.
 *
 *   s, p   : DEVICE [B, H, S_q, S_kv], row-major, of the storage type dtype
 *            (ATTN_F32, ATTN_BF16 or ATTN_F16); p may be s itself (in place)
 *            but may not overlap it otherwise
 *   scale  : finite fp32 factor applied to every score (1/sqrt(D) for
 *            attention scores)
 *   causal : 1: row i sees keys j <= i + S_kv - S_q (the bottom-right rule of
 *            the other entry points; with S_q > S_kv the first S_q - S_kv rows
 *            see no key), 0: every row sees all S_kv keys
 * A row with no visible key is all zeros. Masked scores are never used, so
 * they may hold anything (NaN included); beyond the 16-byte chunk that holds
 * a row's last visible score they are not even read. Arithmetic is fp32; p is rounded to
 * the storage type. A row must be a whole number of 16-byte chunks and at
 * most 16 KiB (S_kv a multiple of 4 and <= 4096 for fp32, a multiple of 8
 * and <= 8192 for 16-bit types), else ATTN_ERR_UNSUPPORTED. An empty tensor
 * is a valid empty call.
 */
int attn_masked_softmax(const void* s, void* p, int B, int H, int S_q, int S_kv, float scale, int causal,
                        int dtype);

/*
 * attn_sinusoidal_pe -- the sinusoidal position encoding table ("Week-4 CUDA
 * notes" page, section 2.3): pe[s][2i] = sin(pos / 10000^(2i/d_model)),
 * pe[s][2i+1] = cos(pos / 10000^(2i/d_model)), pos = pos0 + s.
 *
 *   pe      : DEVICE float [S, d_model], 8-byte aligned (fp32, as the page
 *             requires: fp16 cannot hold the small frequencies)
 *   d_model : even, >= 2 (else ATTN_ERR_INVALID_ARG)
 *   pos0    : first position (>= 0); the last, pos0 + S - 1, must be <= 2^31 - 1
 *   S <= 67,108,860 and d_model <= 33,553,920 (the launch grid), else
 *   ATTN_ERR_UNSUPPORTED
 * The angle is formed and reduced modulo 2*pi in fp64, so every element is
 * within a few fp32 ulp of the exact value at any position. S == 0 is a
 * valid empty call.
 */
int attn_sinusoidal_pe(float* pe, int S, int d_model, int pos0);

/*
 * attn_set_stream -- set the HIP stream (a hipStream_t passed as void*) that
 * later calls from THIS thread enqueue on; NULL selects the null stream.
 * attn_get_stream returns the current thread's stream. The host side of a
 * launch (arguments prepared, kernel enqueued, no copies on the path) is the
 * host launch function of the depthwise-convolution page, section 3.2, with
 * the data kept on the device as the "CUDA first principles" page, section
 * 2.1 asks.
 */
int attn_set_stream(void* hip_stream);
void* attn_get_stream(void);

/*
 * attn_set_timing_events -- arm two HIP events (hipEvent_t passed as void*,
 * created by the caller, either may be NULL) for the NEXT attn_fwd or
 * attn_decode call on this thread: `start` is recorded when that call's first
 * kernel starts executing and `stop` when its last kernel finishes, so
 * hipEventElapsedTime(start, stop) is the call's device time without the
 * queueing gaps around it. The events are used once; the next call (whatever
 * its status) disarms them. Measurement plumbing, not part of the operation.
 */
int attn_set_timing_events(void* start, void* stop);

/*
 * attn_set_clock_probe -- arm a DEVICE buffer of four uint64 (8-byte
 * aligned; NULL disarms) for the NEXT call on this thread. If that call is
 * an attn_fwd, attn_fwd_kvcache or attn_fwd_mask that runs the 16-bit
 * prefill kernel, that kernel's workgroup 0 writes the shader-clock counter
 * (s_memtime) and the 100 MHz real-time counter (s_memrealtime) when it
 * starts, then both again when it ends; the ratio of the differences
 * times 100 MHz is the shader clock over that workgroup's run. Any other
 * call leaves the buffer untouched. The probe is used once, like the timing
 * events. Measurement plumbing, not part of the operation; it follows the
 * timing practice of the depthwise-convolution page, section 4.1.
 */
int attn_set_clock_probe(void* device_buf);

/* Reason for the last non-OK status returned on this thread ("" if none):
 * a rejected shape or argument (the host-side checks of the
 * depthwise-convolution page, section 6.2) or the runtime's message for a
 * launch error read right after the launch (that page, section 3.2).
 * The pointer stays valid until the next call into the library on this thread. */
const char* attn_last_error(void);

/* Static name of a status code ("ATTN_OK", ...), for the messages above. */
const char* attn_status_string(int status);

/*
 * Launch-plan introspection (host only, no HIP call): how attn_fwd would
 * split the work. Lets the tiling and causal load-balance rules be tested
 * without a GPU. Returns the same status attn_fwd would return for these
 * sizes (pointer checks excluded).
 *   kernel      : 0 none (empty call), 1 MFMA tile kernel (bf16 or fp16), 2 row kernel
 *                 (ATTN_ALGO=row), 3 fp32 MFMA kernel (fp32)
 *   block_m     : queries per work item phase (tile kernels), 1 (row kernel)
 *   block_n     : keys per KV tile
 *   paired      : 1 when each work item runs query block r and n-1-r
 *   grid        : workgroups launched
 *   threads     : threads per workgroup
 *   lds_bytes   : LDS per workgroup
 *   max_tiles   : largest number of KV tiles one work item visits
 *   min_tiles   : smallest number of KV tiles one work item visits
 */
typedef struct {
    int kernel;
    int block_m;
    int block_n;
    int paired;
    int grid;
    int threads;
    int lds_bytes;
    int max_tiles;
    int min_tiles;
} attn_fwd_plan_t;

int attn_fwd_plan(int B, int H, int S_q, int S_kv, int D, int causal, int dtype,
                  attn_fwd_plan_t* plan);

/*
 * Decode plan: split workgroups (each streams one contiguous share of the
 * sequences' valid keys), the partial records the workspace holds per head
 * (one per workgroup-sequence segment), threads per workgroup, and the
 * workspace size. Host only.
 */
typedef struct {
    int split_workgroups;
    int records;
    int threads;
    size_t workspace_bytes;
} attn_decode_plan_t;

int attn_decode_plan(int B, int H, int S_cap, int D, int dtype, attn_decode_plan_t* plan);

/*
 * Workgroup-id remap used by the prefill, fp32 and projection kernels:
 * hardware workgroup x of n runs on XCD x % 8; the remap gives each XCD a
 * contiguous range of logical work items so the items of one head share
 * that XCD's L2. A bijection on [0, n). Exposed so the host tests can check
 * it.
 */
int attn_xcd_remap(int x, int n);

/*
 * The decode's split of a token space of T valid keys (all sequences laid
 * end to end) over its split workgroups: attn_decode_range_start(w, T) is
 * the first token of workgroup w's range (0 <= w <= split_workgroups; w =
 * split_workgroups gives T), attn_decode_range_of(t, T) the workgroup whose
 * range holds token t (0 <= t < T). Workgroup w runs on XCD w % 8, and each
 * pair (2p, 2p+1) shares its span unequally, the even one taking 53%, since
 * MI355X's odd XCDs stream about 8% slower. Both return -1 for arguments
 * out of range. Exposed so the host tests can check them.
 */
int attn_decode_range_start(int w, int T);
int attn_decode_range_of(int t, int T);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_GFX950_H */
