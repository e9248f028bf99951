// attn_api.cpp -- the C ABI of libattn.so: validation, planning, dispatch.
//
// Every argument is checked here on the host before any HIP call, so a
// rejected call has no side effect and the checks can be exercised without a
// GPU. Launch errors are read back with hipGetLastError right after each
// launch (the host-launch practice of the depthwise-convolution page,
// section 3.2); configuration mistakes are caught before they become
// "invalid configuration" launches ("CUDA first principles" page,
// section 4.1). An environment switch picks the implementation, as the
// depthwise-convolution page's section 6.2 suggests for bisecting:
//   ATTN_ALGO=auto (default) | tile | row
// (auto and tile: the MFMA kernels -- the 16-bit prefill kernel or the fp32
// kernel; row: the per-query row kernel for every storage type)
// and ATTN_CHECK=1 turns on a debug check of the device-side lengths (a
// synchronous copy to the host before the launch).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/attn.h"
#include "launch.h"
#include "plan.h"

namespace {

thread_local hipStream_t t_stream = nullptr;
thread_local std::string t_error;
thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;   // for the next call only
thread_local unsigned long long* t_clock_probe = nullptr;             // for the next call only

// Take (and clear) the timing events armed for this call.
void take_events(hipEvent_t& start, hipEvent_t& stop) {
    start = t_ev_start;
    stop = t_ev_stop;
    t_ev_start = t_ev_stop = nullptr;
}

// Take (and clear) the clock probe armed for this call.
unsigned long long* take_clock_probe() {
    unsigned long long* p = t_clock_probe;
    t_clock_probe = nullptr;
    return p;
}

int fail(int status, const std::string& msg) {
    t_error = msg;
    return status;
}

int ok() {
    t_error.clear();
    return ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte size of a dense tensor, or -1 when it does not fit in 2^62.
long long tensor_bytes(long long a, long long b, long long c, long long d, long long elem) {
    const long long lim = (long long)1 << 62;
    long long n = elem;
    for (long long x : {a, b, c, d}) {
        if (x < 0) return -1;
        if (x != 0 && n > lim / x) return -1;
        n *= x;
    }
    return n;
}

bool overlap(const void* a, long long na, const void* b, long long nb) {
    if (!a || !b || na <= 0 || nb <= 0) return false;
    const uintptr_t x0 = reinterpret_cast<uintptr_t>(a), y0 = reinterpret_cast<uintptr_t>(b);
    return x0 < y0 + (uintptr_t)nb && y0 < x0 + (uintptr_t)na;
}

int elem_size(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }

bool dtype_built(int dtype) { return dtype == ATTN_F32 || dtype == ATTN_BF16 || dtype == ATTN_F16; }

attn::Elt elt_of(int dtype) {
    return dtype == ATTN_BF16 ? attn::Elt::BF16 : (dtype == ATTN_F16 ? attn::Elt::F16 : attn::Elt::F32);
}

enum Algo { kAuto, kTile, kRow };

Algo algo_from_env() {
    const char* s = std::getenv("ATTN_ALGO");
    if (!s || !*s || !std::strcmp(s, "auto")) return kAuto;
    if (!std::strcmp(s, "tile")) return kTile;
    if (!std::strcmp(s, "row")) return kRow;
    return kAuto;
}

// ATTN_CHECK=1: the device-side lengths are copied to the host (synchronising
// with this thread's stream) and any value the kernels would clamp -- below 0
// or above the cache capacity -- is rejected before the launch.
bool check_lengths_on() {
    const char* s = std::getenv("ATTN_CHECK");
    return s && !std::strcmp(s, "1");
}

int check_lengths(const char* fn, const int32_t* lens, int B, int cap) {
    std::vector<int32_t> h((size_t)B);
    hipError_t e = hipMemcpyAsync(h.data(), lens, (size_t)B * sizeof(int32_t), hipMemcpyDeviceToHost, t_stream);
    if (e == hipSuccess) e = hipStreamSynchronize(t_stream);
    if (e != hipSuccess)
        return fail(ATTN_ERR_HIP, std::string(fn) + ": ATTN_CHECK could not read the lengths: " + hipGetErrorString(e));
    for (int i = 0; i < B; ++i)
        if (h[(size_t)i] < 0 || h[(size_t)i] > cap)
            return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": ATTN_CHECK: length[" + std::to_string(i) +
                                                  "] = " + std::to_string(h[(size_t)i]) + " lies outside [0, " +
                                                  std::to_string(cap) + "]");
    return ATTN_OK;
}

// Checks shared by attn_fwd, attn_fwd_kvcache, attn_fwd_mask and
// attn_fwd_plan (sizes and flags only). With kvcache, S_kv is the cache capacity and the per-entry
// lengths may be shorter than S_q (rows that see no key come out as 0).
int check_fwd_sizes(int B, int H, int S_q, int S_kv, int D, int causal, int dtype, bool kvcache = false,
                    const char* fn = "attn_fwd") {
    if (B < 0 || H < 0 || S_q < 0 || S_kv < 0)
        return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": negative size (B=" + std::to_string(B) + " H=" +
                                              std::to_string(H) + " S_q=" + std::to_string(S_q) +
                                              " S_kv=" + std::to_string(S_kv) + ")");
    if (D <= 0) return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": head dim D must be positive");
    if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": causal must be 0 or 1");
    if (!dtype_built(dtype))
        return fail(ATTN_ERR_UNSUPPORTED, std::string(fn) + ": dtype " + std::to_string(dtype) +
                                              " not built (ATTN_F32=0, ATTN_BF16=1, ATTN_F16=2)");
    if (D != 32 && D != 64 && D != 128)
        return fail(ATTN_ERR_UNSUPPORTED, std::string(fn) + ": head dim D=" + std::to_string(D) +
                                              " not built (32, 64 or 128)");
    if (B == 0 || H == 0 || S_q == 0) return ATTN_OK;   // an empty call (no product formed before the checks below)
    if (S_kv == 0)
        return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + (kvcache ? ": S_cap == 0 leaves no cache rows"
                                                                     : ": S_kv == 0 leaves the softmax without keys"));
    if (!kvcache && causal && S_q > S_kv)
        return fail(ATTN_ERR_INVALID_ARG, std::string(fn) +
                                              ": causal needs S_q <= S_kv (queries are the last S_q positions)");
    const int es = elem_size(dtype);
    if (tensor_bytes(B, S_q, H, D, es) < 0 || tensor_bytes(B, S_kv, H, D, es) < 0)
        return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": tensor size overflows");
    if ((long long)B * H * S_q > 0x7fffffffLL || (long long)B * H * ((S_q + 127) / 128) > 0x7fffffffLL)
        return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": B*H*S_q exceeds the launch grid");
    // the kernels address one head's rows with 32-bit byte offsets
    const long long S_max = (S_q > S_kv ? S_q : S_kv) + 128;
    if (S_max * H * D * es > 0x7fffffffLL)
        return fail(ATTN_ERR_UNSUPPORTED, std::string(fn) + ": one batch entry spans more than 2 GiB "
                                                            "((S + 128) * H * D * elem_size); split the batch");
    return ATTN_OK;
}

// attn_fwd, attn_fwd_kvcache and attn_fwd_mask: pointer checks and dispatch.
int run_fwd(const char* fn, const void* q, const void* k, const void* v, const int32_t* kv_lens,
            const uint8_t* key_mask, void* o, float* lse, int B, int H, int S_q, int S_kv, int D, int causal,
            int dtype, bool kvcache) {
    hipEvent_t ev_start, ev_stop;
    take_events(ev_start, ev_stop);
    unsigned long long* const clk = take_clock_probe();
    const int st = check_fwd_sizes(B, H, S_q, S_kv, D, causal, dtype, kvcache, fn);
    if (st != ATTN_OK) return st;
    if ((long long)B * H * S_q == 0) return ok();
    const int es = elem_size(dtype);
    const long long nq = tensor_bytes(B, S_q, H, D, es), nkv = tensor_bytes(B, S_kv, H, D, es);
    const long long nlse = lse ? (long long)B * H * S_q * 4 : 0, nlen = kv_lens ? (long long)B * 4 : 0;
    const long long nmask = key_mask ? (long long)B * S_kv : 0;
    if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": NULL tensor pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": tensor pointers must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(kv_lens) & 3u))
        return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": lse and seqlens_kv must be 4-byte aligned");
    if (overlap(o, nq, q, nq) || overlap(o, nq, k, nkv) || overlap(o, nq, v, nkv) || overlap(o, nq, kv_lens, nlen) ||
        overlap(o, nq, lse, nlse) || overlap(o, nq, key_mask, nmask))
        return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": output overlaps another argument");
    if (overlap(lse, nlse, q, nq) || overlap(lse, nlse, k, nkv) || overlap(lse, nlse, v, nkv) ||
        overlap(lse, nlse, kv_lens, nlen) || overlap(lse, nlse, key_mask, nmask))
        return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": lse overlaps an input");
    if (kv_lens && check_lengths_on()) {
        const int cs = check_lengths(fn, kv_lens, B, S_kv);
        if (cs != ATTN_OK) return cs;
    }

    attn::FwdArgs a{q, k, v, o, B, H, S_q, S_kv, D, causal,
                    (float)(1.0f / std::sqrt((float)D)) * 1.4426950408889634f, ev_start, ev_stop, kv_lens, lse,
                    key_mask};
    a.clock_probe = clk;
    const Algo algo = algo_from_env();
    hipError_t e;
    if (algo == kRow)
        e = attn::launch_fwd_row(a, elt_of(dtype), t_stream);
    else if (dtype == ATTN_F32)
        e = attn::launch_fwd_f32(a, t_stream);
    else
        e = attn::launch_fwd_prefill(a, elt_of(dtype), t_stream);
    if (e != hipSuccess)
        return fail(ATTN_ERR_HIP, std::string(fn) + ": launch failed: " + hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int attn_set_stream(void* hip_stream) {
    t_stream = static_cast<hipStream_t>(hip_stream);
    return ok();
}

void* attn_get_stream(void) { return static_cast<void*>(t_stream); }

int attn_set_timing_events(void* start, void* stop) {
    t_ev_start = static_cast<hipEvent_t>(start);
    t_ev_stop = static_cast<hipEvent_t>(stop);
    return ok();
}

int attn_set_clock_probe(void* device_buf) {
    if (device_buf && (reinterpret_cast<uintptr_t>(device_buf) & 7u) != 0)
        return fail(ATTN_ERR_INVALID_ARG, "attn_set_clock_probe: buffer must be 8-byte aligned");
    t_clock_probe = static_cast<unsigned long long*>(device_buf);
    return ok();
}

const char* attn_last_error(void) { return t_error.c_str(); }

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ATTN_OK";
        case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG";
        case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
        case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE";
        case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
        default: return "ATTN_UNKNOWN_STATUS";
    }
}

int attn_xcd_remap(int x, int n) {
    if (n <= 0 || x < 0 || x >= n) return -1;
    return attn::xcd_remap(x, n);
}

int attn_decode_range_start(int w, int T) {
    if (T < 0 || w < 0 || w > attn::kDecodeSplitWGs) return -1;
    return attn::decode_range_start(w, T);
}

int attn_decode_range_of(int t, int T) {
    if (T <= 0 || t < 0 || t >= T) return -1;
    return attn::decode_range_of(t, T);
}

int attn_fwd_plan(int B, int H, int S_q, int S_kv, int D, int causal, int dtype, attn_fwd_plan_t* plan) {
    if (!plan) return fail(ATTN_ERR_INVALID_ARG, "attn_fwd_plan: plan is NULL");
    std::memset(plan, 0, sizeof(*plan));
    const int st = check_fwd_sizes(B, H, S_q, S_kv, D, causal, dtype);
    if (st != ATTN_OK) return st;
    if ((long long)B * H * S_q == 0) return ok();
    const Algo algo = algo_from_env();
    if (algo != kRow && dtype == ATTN_F32) {
        const int n_qblk = (S_q + attn::kF32Q - 1) / attn::kF32Q;
        plan->kernel = 3;
        plan->block_m = attn::kF32Q;
        plan->block_n = attn::kF32N;
        plan->paired = 0;
        plan->grid = (int)((long long)B * H * n_qblk);
        plan->threads = attn::kF32Threads;
        plan->lds_bytes = ((attn::kF32Threads / 64) * 64 * (2 + D / 2 + 1) + attn::kF32Q * (attn::kF32Threads / 64)) * 4;
        int mx = 0, mn = 1 << 30;
        for (int qb = 0; qb < n_qblk; ++qb) {
            const int q_last = std::min(qb * attn::kF32Q + attn::kF32Q - 1, S_q - 1);
            const int kend = causal ? std::min(S_kv, std::max(0, q_last + 1 + S_kv - S_q)) : S_kv;
            const int n = (kend + attn::kF32N - 1) / attn::kF32N;
            mx = n > mx ? n : mx;
            mn = n < mn ? n : mn;
        }
        plan->max_tiles = mx;
        plan->min_tiles = mn;
        return ok();
    }
    const bool tile = dtype != ATTN_F32 && algo != kRow;
    if (tile) {
        const attn::TileGrid g = attn::tile_grid(B, H, S_q, causal);
        plan->kernel = 1;
        plan->block_m = attn::kTileM;
        plan->block_n = attn::kTileN;
        plan->paired = g.paired;
        plan->grid = (int)g.n_items;
        plan->threads = attn::kTileThreads;
        plan->lds_bytes = attn::prefill_lds_bytes(D);   // attn_fwd runs the prefill kernel
        int mx = 0, mn = 1 << 30;
        for (int p = 0; p < g.items_per_bh; ++p) {
            const int qa = g.n_qblk - 1 - p;
            int n = attn::tiles_for_block(qa, S_q, S_kv, causal);
            if (g.paired && p != qa) n += attn::tiles_for_block(p, S_q, S_kv, causal);
            mx = n > mx ? n : mx;
            mn = n < mn ? n : mn;
        }
        plan->max_tiles = mx;
        plan->min_tiles = mn;
    } else {
        plan->kernel = 2;
        plan->block_m = 1;
        plan->block_n = 64;
        plan->grid = B * H * S_q;
        plan->threads = attn::kRowThreads;
        plan->lds_bytes = D * 4;
        plan->max_tiles = (S_kv + 63) / 64;
        plan->min_tiles = causal ? (S_kv - S_q + 1 + 63) / 64 : (S_kv + 63) / 64;
    }
    return ok();
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int S_q, int S_kv, int D,
             int causal, int dtype) {
    return run_fwd("attn_fwd", q, k, v, nullptr, nullptr, o, nullptr, B, H, S_q, S_kv, D, causal, dtype, false);
}

int attn_fwd_mask(const void* q, const void* k, const void* v, const uint8_t* key_mask, void* o, float* lse, int B,
                  int H, int S_q, int S_kv, int D, int causal, int dtype) {
    return run_fwd("attn_fwd_mask", q, k, v, nullptr, key_mask, o, lse, B, H, S_q, S_kv, D, causal, dtype, false);
}

int attn_fwd_kvcache(const void* q, const void* kcache, const void* vcache, const int32_t* seqlens_kv, void* o,
                     float* lse, int B, int H, int S_q, int S_cap, int D, int causal, int dtype) {
    return run_fwd("attn_fwd_kvcache", q, kcache, vcache, seqlens_kv, nullptr, o, lse, B, H, S_q, S_cap, D, causal,
                   dtype, true);
}

// Per-call flag value for the decode kernel: a process-wide call counter
// passed through the SplitMix64 finaliser (Steele, Lea and Flood, 2014), so
// consecutive calls get unrelated 64-bit values; never zero, the value a
// consumed flag is reset to.
static unsigned long long next_decode_tag() {
    static std::atomic<unsigned long long> calls{0};
    unsigned long long z = calls.fetch_add(1, std::memory_order_relaxed) + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z ? z : 1ull;
}

size_t attn_decode_workspace_bytes(int B, int H, int S_cap, int D) {
    if (B <= 0 || H <= 0 || S_cap <= 0 || (D != 32 && D != 64 && D != 128)) return 0;
    if (attn::decode_records(B) * H > 0x7fffffffLL) return 0;   // beyond what attn_decode_plan accepts
    return attn::decode_workspace_bytes(B, H, S_cap, D);
}

int attn_decode_plan(int B, int H, int S_cap, int D, int dtype, attn_decode_plan_t* plan) {
    if (!plan) return fail(ATTN_ERR_INVALID_ARG, "attn_decode_plan: plan is NULL");
    std::memset(plan, 0, sizeof(*plan));
    if (B < 0 || H < 0 || S_cap <= 0 || D <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "attn_decode: sizes must be B, H >= 0 and S_cap, D >= 1");
    if (!dtype_built(dtype))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode: dtype " + std::to_string(dtype) + " not built");
    if (D != 32 && D != 64 && D != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode: head dim D=" + std::to_string(D) + " not built");
    // key offsets inside one sequence are 32-bit (a load batch may reach
    // kDecodeBatch keys past the last valid one)
    const long long seq_bytes = tensor_bytes(1, (long long)S_cap + attn::kDecodeBatch, H, D, elem_size(dtype));
    if (seq_bytes < 0 || seq_bytes > 0x7fffffffLL)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode: one sequence's cache spans more than 2 GiB");
    if (tensor_bytes(B, S_cap, H, D, elem_size(dtype)) < 0 || attn::decode_records(B) * H > 0x7fffffffLL)
        return fail(ATTN_ERR_INVALID_ARG, "attn_decode: sizes overflow");
    // the kernel counts the valid keys of all sequences, laid end to end, in 32 bits
    if ((long long)B * S_cap > 0x7fffffffLL)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode: B * S_cap = " + std::to_string((long long)B * S_cap) +
                                              " keys in all, beyond 32-bit token counts");
    // a merge addresses up to kDecodeSplitWGs consecutive records with 32-bit offsets
    if ((long long)attn::kDecodeSplitWGs * H * attn::decode_record_floats(D) * 4 > 0x7fffffffLL)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode: H=" + std::to_string(H) + " heads beyond the merge's 32-bit offsets");
    plan->split_workgroups = attn::kDecodeSplitWGs;
    plan->records = (int)attn::decode_records(B);
    plan->threads = attn::kDecodeThreads;
    plan->workspace_bytes = attn_decode_workspace_bytes(B, H, S_cap, D);
    return ok();
}

namespace {

// attn_decode and attn_decode_noalloc: validation and launch. A NULL
// workspace with noalloc set means this GPU's fixed scratch array.
int run_decode(const char* fn, const void* q, const void* kcache, const void* vcache, const int32_t* seqlens,
               void* o, int B, int H, int S_cap, int D, int dtype, void* workspace, size_t workspace_bytes,
               bool noalloc) {
    hipEvent_t ev_start, ev_stop;
    take_events(ev_start, ev_stop);
    take_clock_probe();   // armed for an attn_fwd call only
    attn_decode_plan_t plan;
    const int st = attn_decode_plan(B, H, S_cap, D, dtype, &plan);
    if (st != ATTN_OK) return st;
    if ((long long)B * H == 0) return ok();
    const int es = elem_size(dtype);
    const long long nq = tensor_bytes(B, 1, H, D, es), nkv = tensor_bytes(B, S_cap, H, D, es);
    const long long nsl = (long long)B * 4;
    if (!q || !kcache || !vcache || !seqlens || !o)
        return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": NULL tensor pointer");
    if (!aligned16(q) || !aligned16(kcache) || !aligned16(vcache) || !aligned16(o))
        return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": tensor pointers must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(seqlens) & 3u) != 0)
        return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": seqlens must be 4-byte aligned");
    if (noalloc) {
        if (plan.workspace_bytes > attn::kDecodeScratchBytes)
            return fail(ATTN_ERR_WORKSPACE, std::string(fn) + ": these sizes need " +
                                                std::to_string(plan.workspace_bytes) +
                                                " bytes of workspace, beyond the fixed " +
                                                std::to_string(attn::kDecodeScratchBytes) + "-byte scratch");
        const hipError_t se = attn::decode_scratch(&workspace);
        if (se != hipSuccess)
            return fail(ATTN_ERR_HIP, std::string(fn) + ": scratch lookup failed: " + hipGetErrorString(se));
        workspace_bytes = attn::kDecodeScratchBytes;
    }
    if (!workspace || workspace_bytes < plan.workspace_bytes)
        return fail(ATTN_ERR_WORKSPACE, std::string(fn) + ": workspace needs " + std::to_string(plan.workspace_bytes) +
                                            " bytes, got " + std::to_string(workspace_bytes));
    if (!aligned16(workspace)) return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": workspace must be 16-byte aligned");
    const long long nws = (long long)plan.workspace_bytes;
    if (overlap(o, nq, q, nq) || overlap(o, nq, kcache, nkv) || overlap(o, nq, vcache, nkv) ||
        overlap(o, nq, seqlens, nsl) || overlap(o, nq, workspace, nws))
        return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": output overlaps another argument");
    if (overlap(workspace, nws, q, nq) || overlap(workspace, nws, kcache, nkv) ||
        overlap(workspace, nws, vcache, nkv) || overlap(workspace, nws, seqlens, nsl))
        return fail(ATTN_ERR_INVALID_ARG, std::string(fn) + ": workspace overlaps an input");
    if (!noalloc && check_lengths_on()) {   // (a host copy of the lengths)
        const int cs = check_lengths(fn, seqlens, B, S_cap);
        if (cs != ATTN_OK) return cs;
    }

    attn::DecodeArgs a{q, kcache, vcache, seqlens, o, B, H, S_cap, D,
                       (float)(1.0f / std::sqrt((float)D)) * 1.4426950408889634f, workspace, ev_start,
                       ev_stop, next_decode_tag()};
    const hipError_t e = attn::launch_decode(a, elt_of(dtype), t_stream);
    if (e != hipSuccess)
        return fail(ATTN_ERR_HIP, std::string(std::string(fn) + ": launch failed: ") + hipGetErrorString(e));
    return ok();
}

}  // namespace

int attn_decode(const void* q, const void* kcache, const void* vcache, const int32_t* seqlens, void* o, int B,
                int H, int S_cap, int D, int dtype, void* workspace, size_t workspace_bytes) {
    return run_decode("attn_decode", q, kcache, vcache, seqlens, o, B, H, S_cap, D, dtype, workspace,
                      workspace_bytes, false);
}

int attn_decode_noalloc(const void* q, const void* kcache, const void* vcache, const int32_t* seqlens, void* o,
                        int B, int H, int S_cap, int D, int dtype) {
    return run_decode("attn_decode_noalloc", q, kcache, vcache, seqlens, o, B, H, S_cap, D, dtype, nullptr, 0,
                      true);
}

int attn_sinusoidal_pe(float* pe, int S, int d_model, int pos0) {
    hipEvent_t ev_start, ev_stop;
    take_events(ev_start, ev_stop);
    take_clock_probe();   // armed for an attn_fwd call only
    if (S < 0 || d_model <= 0 || pos0 < 0)
        return fail(ATTN_ERR_INVALID_ARG, "attn_sinusoidal_pe: sizes must be S >= 0, d_model >= 1, pos0 >= 0");
    if (d_model & 1)
        return fail(ATTN_ERR_INVALID_ARG, "attn_sinusoidal_pe: d_model must be even (sine and cosine pairs)");
    if ((long long)pos0 + S - 1 > 0x7fffffffLL)   // the last position, pos0 + S - 1, is an int
        return fail(ATTN_ERR_INVALID_ARG, "attn_sinusoidal_pe: positions pos0 + S exceed 2^31 - 1");
    if (tensor_bytes(S, d_model, 1, 1, 4) < 0)
        return fail(ATTN_ERR_INVALID_ARG, "attn_sinusoidal_pe: size overflows");
    // launch grid: (S / kPeRows) x pe_grid_chunks(d_model) workgroups of kPeThreads
    if ((long long)(S + attn::kPeRows - 1) / attn::kPeRows * attn::kPeThreads > 0xffffffffLL)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_sinusoidal_pe: S exceeds the launch grid");
    if (attn::pe_grid_chunks(d_model) > 65535)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_sinusoidal_pe: d_model exceeds the launch grid");
    if (S == 0) return ok();
    if (!pe) return fail(ATTN_ERR_INVALID_ARG, "attn_sinusoidal_pe: NULL output pointer");
    if ((reinterpret_cast<uintptr_t>(pe) & 7u) != 0)
        return fail(ATTN_ERR_INVALID_ARG, "attn_sinusoidal_pe: output must be 8-byte aligned");
    const hipError_t e = attn::launch_sinusoidal_pe(pe, S, d_model, pos0, ev_start, ev_stop, t_stream);
    if (e != hipSuccess)
        return fail(ATTN_ERR_HIP, std::string("attn_sinusoidal_pe: launch failed: ") + hipGetErrorString(e));
    return ok();
}

int attn_masked_softmax(const void* s, void* p, int B, int H, int S_q, int S_kv, float scale, int causal,
                        int dtype) {
    hipEvent_t ev_start, ev_stop;
    take_events(ev_start, ev_stop);
    take_clock_probe();   // armed for an attn_fwd call only
    if (B < 0 || H < 0 || S_q < 0 || S_kv < 0)
        return fail(ATTN_ERR_INVALID_ARG, "attn_masked_softmax: negative size");
    if (causal != 0 && causal != 1) return fail(ATTN_ERR_INVALID_ARG, "attn_masked_softmax: causal must be 0 or 1");
    if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "attn_masked_softmax: scale must be finite");
    if (!dtype_built(dtype))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_masked_softmax: dtype " + std::to_string(dtype) +
                                              " not built (ATTN_F32=0, ATTN_BF16=1, ATTN_F16=2)");
    const int es = elem_size(dtype);
    const long long row_bytes = (long long)S_kv * es;
    if (row_bytes > attn::kSmMaxRowBytes)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_masked_softmax: a row of S_kv=" + std::to_string(S_kv) +
                                              " scores exceeds " + std::to_string(attn::kSmMaxRowBytes) + " bytes");
    if (row_bytes % 16 != 0)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_masked_softmax: a row must be a whole number of 16-byte chunks "
                                          "(S_kv a multiple of 4 for fp32, of 8 for 16-bit types)");
    const long long n = tensor_bytes(B, H, S_q, S_kv, es);
    if (n < 0) return fail(ATTN_ERR_INVALID_ARG, "attn_masked_softmax: tensor size overflows");
    const long long rows = (long long)B * H * S_q;
    if ((rows + attn::kSmRowsPerBlock - 1) / attn::kSmRowsPerBlock * attn::kSmThreads > 0xffffffffLL)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_masked_softmax: B*H*S_q rows exceed the launch grid");
    if (n == 0) return ok();
    if (!s || !p) return fail(ATTN_ERR_INVALID_ARG, "attn_masked_softmax: NULL tensor pointer");
    if (!aligned16(s) || !aligned16(p))
        return fail(ATTN_ERR_INVALID_ARG, "attn_masked_softmax: tensor pointers must be 16-byte aligned");
    if (s != p && overlap(s, n, p, n))
        return fail(ATTN_ERR_INVALID_ARG, "attn_masked_softmax: p overlaps s without being s itself");
    attn::SoftmaxArgs a{s, p, B, H, S_q, S_kv, causal, (float)((double)scale * 1.4426950408889634), ev_start, ev_stop};
    const hipError_t e = attn::launch_masked_softmax(a, elt_of(dtype), t_stream);
    if (e != hipSuccess)
        return fail(ATTN_ERR_HIP, std::string("attn_masked_softmax: launch failed: ") + hipGetErrorString(e));
    return ok();
}

int attn_qkv_proj(const void* x, const void* w, void* q, void* k, void* v, int M, int E, int H, int D, int dtype) {
    hipEvent_t ev_start, ev_stop;
    take_events(ev_start, ev_stop);
    take_clock_probe();   // armed for an attn_fwd call only
    if (M < 0 || E <= 0 || H <= 0 || D <= 0)
        return fail(ATTN_ERR_INVALID_ARG, "attn_qkv_proj: sizes must be M >= 0 and E, H, D >= 1");
    if (dtype != ATTN_BF16 && dtype != ATTN_F16)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_qkv_proj: dtype " + std::to_string(dtype) +
                                              " not built (ATTN_BF16 or ATTN_F16)");
    if (E % attn::kGemmBK != 0)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_qkv_proj: E must be a multiple of " + std::to_string(attn::kGemmBK));
    const long long N = (long long)H * D;
    if (N % 32 != 0) return fail(ATTN_ERR_UNSUPPORTED, "attn_qkv_proj: H*D must be a multiple of 32");
    // per-tile descriptors span 256 rows of X or of an output, 384 rows of W
    if ((long long)attn::kGemmBM * E * 2 > 0x7fffffffLL || (long long)attn::kGemmBN * E * 2 > 0x7fffffffLL ||
        (long long)attn::kGemmBM * N * 2 > 0x7fffffffLL || 3 * N > 0x7fffffffLL)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_qkv_proj: E or H*D too large for 32-bit tile offsets");
    if (tensor_bytes(M, E, 1, 1, 2) < 0 || tensor_bytes(3, N, E, 1, 2) < 0 || tensor_bytes(M, N, 1, 1, 2) < 0 ||
        attn::qkv_grid(M, (int)N) > 0x7fffffffLL)
        return fail(ATTN_ERR_INVALID_ARG, "attn_qkv_proj: sizes overflow");
    if (M == 0) return ok();
    if (!x || !w || !q || !k || !v) return fail(ATTN_ERR_INVALID_ARG, "attn_qkv_proj: NULL tensor pointer");
    if (!aligned16(x) || !aligned16(w) || !aligned16(q) || !aligned16(k) || !aligned16(v))
        return fail(ATTN_ERR_INVALID_ARG, "attn_qkv_proj: tensor pointers must be 16-byte aligned");
    const long long nx = (long long)M * E * 2, nw = 3 * N * E * 2, no = (long long)M * N * 2;
    const void* outs[3] = {q, k, v};
    for (int i = 0; i < 3; ++i) {
        if (overlap(outs[i], no, x, nx) || overlap(outs[i], no, w, nw))
            return fail(ATTN_ERR_INVALID_ARG, "attn_qkv_proj: an output overlaps an input");
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], no, outs[j], no))
                return fail(ATTN_ERR_INVALID_ARG, "attn_qkv_proj: outputs overlap each other");
    }
    attn::QkvArgs a{x, w, q, k, v, M, E, (int)N, ev_start, ev_stop};
    const hipError_t e = attn::launch_qkv_proj(a, elt_of(dtype), t_stream);
    if (e != hipSuccess)
        return fail(ATTN_ERR_HIP, std::string("attn_qkv_proj: launch failed: ") + hipGetErrorString(e));
    return ok();
}

}  // extern "C"
