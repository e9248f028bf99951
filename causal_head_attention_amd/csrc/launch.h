// launch.h -- internal launchers (host functions defined next to their kernels).
// Arguments reaching these have already been validated by the C ABI layer.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace attn {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int B, H, S_q, S_kv, D;
    int causal;
    float scale_log2;   // (1/sqrt(D)) * log2(e), fp32
    hipEvent_t ev_start;   // optional: recorded when the first kernel starts
    hipEvent_t ev_stop;    // optional: recorded when the last kernel ends
    // KV-cache form: k and v hold S_kv rows per batch entry (the cache
    // capacity), of which kv_lens[b] (device, clamped to [0, S_kv]) are valid;
    // nullptr means all S_kv rows are valid.
    const int32_t* kv_lens;
    float* lse;   // optional [B, H, S_q] natural-log sum of exp(scaled scores)
    // optional device uint8 [B, S_kv]: 0 hides key j of entry b from all
    // its queries (key padding); nullptr means no key is hidden
    const uint8_t* key_mask;
    // optional device uint64[4]: the prefill kernel's workgroup 0 writes the
    // shader-clock and real-time counters at its start and at its end
    unsigned long long* clock_probe;
};

// Storage type of q, k, v and o (arithmetic is fp32 throughout).
enum class Elt { F32, BF16, F16 };

struct DecodeArgs {
    const void* q;
    const void* kcache;
    const void* vcache;
    const int32_t* seqlens;
    void* o;
    int B, H, S_cap, D;
    float scale_log2;
    void* workspace;   // decode_workspace_bytes(B, H, S_cap, D) bytes
    hipEvent_t ev_start;   // optional: recorded when the kernel starts
    hipEvent_t ev_stop;    // optional: recorded when the kernel ends
    // nonzero value that marks this call's flags in the workspace; flags
    // left by earlier calls are zero, and garbage matches it with odds 2^-64
    unsigned long long tag;
};

struct QkvArgs {
    const void* x;   // [M, E]
    const void* w;   // [3N, E], output-major
    void* q;         // [M, N] each
    void* k;
    void* v;
    int M, E, N;
    hipEvent_t ev_start;
    hipEvent_t ev_stop;
};

struct SoftmaxArgs {
    const void* s;   // [B, H, S_q, S_kv] scores
    void* p;         // same shape; may be s itself
    int B, H, S_q, S_kv;
    int causal;
    float scale_log2;   // scale * log2(e), fp32
    hipEvent_t ev_start;
    hipEvent_t ev_stop;
};

// MFMA prefill kernel for 16-bit storage (BF16 or F16), with or without a
// key mask; D in {32, 64, 128}.
hipError_t launch_fwd_prefill(const FwdArgs& a, Elt t, hipStream_t stream);
// Row kernel: one wave per query row, any storage type.
hipError_t launch_fwd_row(const FwdArgs& a, Elt t, hipStream_t stream);
// fp32 kernel on the fp32 matrix cores; D in {32, 64, 128}.
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
// Split-KV decode (one kernel: streaming workgroups, then merging workgroups), any storage type.
hipError_t launch_decode(const DecodeArgs& a, Elt t, hipStream_t stream);
// Device address of this GPU's fixed decode workspace (kDecodeScratchBytes),
// looked up once per device; no allocation.
hipError_t decode_scratch(void** ptr);
// Q/K/V projection GEMM, 16-bit storage.
hipError_t launch_qkv_proj(const QkvArgs& a, Elt t, hipStream_t stream);
// Row softmax of scale * s under the causal rule, any storage type.
hipError_t launch_masked_softmax(const SoftmaxArgs& a, Elt t, hipStream_t stream);
// Sinusoidal position encoding table, fp32 [S, d_model].
hipError_t launch_sinusoidal_pe(float* pe, int S, int d_model, int pos0, hipEvent_t ev_start, hipEvent_t ev_stop,
                                hipStream_t stream);

}  // namespace attn
