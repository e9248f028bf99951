"""Benchmark: causal attention prefill TFLOPS and decode KV-read GB/s on one MI355X.

One step is one pass of the whole path over resident synthetic inputs:
  1. attn_fwd   on bf16 B=1, H=32, S=2048, D=128, causal  (prefill)
  2. attn_decode on bf16 B=16, H=32, D=128, KV capacity 4096, lengths U[1,4096]
Each call is timed by two hipEvents that the library attaches to its first
and last kernel dispatch (attn_set_timing_events -> hipExtLaunchKernelGGL on
torch's current stream), so the interval is the kernels' device time, and a
512 MiB fill runs before each call so neither finds its inputs in L2 or the
256 MB Infinity Cache.

`value` is the prefill rate: algorithmic causal FLOP (4*B*H*D per visible
query-key pair) / mean prefill kernel time. The decode rate (K and V bytes
of the valid tokens plus q and o / mean decode time) is reported beside it.
The CPU baseline is the fp64 oracle on the full prefill workload, timed on
the host cores (test infrastructure, not part of the product path).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--warm]
Only one GPU is supported; --gpus > 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import subprocess
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_MFMA_PEAK_TFLOPS = 2516.6   # MI355X dense bf16: 256 CU x 4096 FLOP/clk x 2.4 GHz
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
FP32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense fp32 matrix (the same figure as the fp32 vector peak)
FLUSH_BYTES = 512 << 20
CSRC = os.path.join(ROOT, "causal_head_attention_amd", "csrc")
PREFILL_SRC = os.path.join(CSRC, "kernels", "fwd_prefill.hip")
DECODE_SRC = os.path.join(CSRC, "kernels", "decode.hip")
# the local headers every kernel source includes: their constants set tile
# sizes, LDS layouts and the decode split, hence the kernels' traffic
KERNEL_HEADERS = [os.path.join(CSRC, "plan.h"), os.path.join(CSRC, "launch.h")]
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
NOMINAL_CLOCK_GHZ = 2.4          # the clock the MI355X peaks are quoted at


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _hipcc_version() -> str:
    import subprocess
    from causal_head_attention_amd import build as B
    try:
        return subprocess.run([B.hipcc(), "--version"], capture_output=True, text=True).stdout
    except (OSError, RuntimeError):
        return "unknown"


def code_text(path: str) -> bytes:
    """A C/C++ source without its comments and with runs of whitespace folded,
    so that edits to comments and layout leave a fingerprint unchanged."""
    import re
    text = open(path, encoding="utf-8").read()
    # string and character literals are kept whole; comments go
    pat = re.compile(r'"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|//[^\n]*|/\*.*?\*/', re.S)
    text = pat.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", text)
    return " ".join(text.split()).encode()


def build_sha256(path: str, headers=None) -> str:
    """Fingerprint of a kernel as built: its code (source and the local headers
    it includes, plan.h and launch.h, comments left out), the device flags it
    is compiled with (include paths left out, as they differ per machine) and
    the compiler's version banner."""
    from causal_head_attention_amd import build as B
    name = os.path.basename(path)
    flags = [f for f in B.COMMON if f != "-I" and not os.path.isabs(f)]
    flags += B.DEVICE_FLAGS + B.PER_SOURCE_FLAGS.get(name, [])
    h = hashlib.sha256(code_text(path))
    for hdr in (KERNEL_HEADERS if headers is None else headers):
        h.update(code_text(hdr))
    h.update(" ".join(flags).encode())
    h.update(_hipcc_version().encode())
    return h.hexdigest()


def measured_traffic(kernel: str, src: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    if they were taken on a different build of the kernel (source or flags)."""
    try:
        doc = json.load(open(TRAFFIC_JSON))
        ent = doc[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if ent.get("build_sha256") != build_sha256(src):
        return None
    return ent.get("bytes_per_launch")


class HipEvents:
    """hipEvent_t handles from the HIP runtime torch has already loaded."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            h = self.ct.c_void_p()
            if self.rt.hipEventCreate(self.ct.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(h.value)
        return out

    def ms(self, a, b) -> float:
        v = self.ct.c_float()
        if self.rt.hipEventElapsedTime(self.ct.byref(v), self.ct.c_void_p(a), self.ct.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return v.value

    def destroy(self, hs):
        for h in hs:
            self.rt.hipEventDestroy(self.ct.c_void_p(h))


def traffic_from_counters(fetch_csv: str, write_csv: str, copy_mib: int = 256) -> dict:
    """Turn two rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch) of `bench.py --copy-calibration MIB` into HBM bytes per launch.

    Each counter is scaled by what it reads for the calibration copy (the
    largest `__amd_rocclr_copyBuffer` dispatch: copy_mib MiB read and written).
    The result is keyed by the SHA-256 of the kernel sources it was taken on."""
    import csv

    prefill_grid = str(256 * 512)   # workgroups x threads of the S=2048 prefill launch

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            if "prefill_kernel" in name and r["Grid_Size"] != prefill_grid:
                name += " [kvcache]"   # the KV-cache launch of the same kernel
            vals.setdefault(name, []).append(float(r["Counter_Value"]))
        return vals

    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    f_scale = copy_kib / max(fetch["__amd_rocclr_copyBuffer"])
    w_scale = copy_kib / max(write["__amd_rocclr_copyBuffer"])

    def mean_of(vals, key):
        xs = [v for name, v in vals.items() if key in name and "[kvcache]" not in name]
        assert len(xs) == 1, f"{key}: {len(xs)} kernels match"
        return statistics.fmean(xs[0])

    out = {"note": (f"HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each "
                    f"scaled by what the counter reads for a {copy_mib} MiB device copy: FETCH_SIZE x {f_scale:.5f}, "
                    f"WRITE_SIZE x {w_scale:.5f}.")}
    prefill = {"fetch_kib": mean_of(fetch, "prefill_kernelIDF16bLi128"),
               "write_kib": mean_of(write, "prefill_kernelIDF16bLi128")}
    dec = {"fetch_kib": mean_of(fetch, "decode_kernelIDF16bLi128"),
           "write_kib": mean_of(write, "decode_kernelIDF16bLi128")}
    pb = round((prefill["fetch_kib"] * f_scale + prefill["write_kib"] * w_scale) * 1024)
    db = round((dec["fetch_kib"] * f_scale + dec["write_kib"] * w_scale) * 1024)
    out["prefill"] = {"bytes_per_launch": pb, "algorithmic_bytes": 4 * 2048 * 32 * 128 * 2,
                      "counters_kib": prefill, "build_sha256": build_sha256(PREFILL_SRC)}
    out["decode"] = {"bytes_per_launch": db, "counters_kib": dec, "build_sha256": build_sha256(DECODE_SRC),
                     "note": "one call = one kernel (streaming and merging workgroups)"}
    out["scales"] = {"fetch": f_scale, "write": w_scale}
    return out


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), for the baseline record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main() -> int:
    if len(sys.argv) >= 2 and sys.argv[1] == "--traffic-from":
        # bench.py --traffic-from FETCH_CSV WRITE_CSV [OUT]: write profiles/traffic.json (or OUT)
        doc = traffic_from_counters(sys.argv[2], sys.argv[3])
        json.dump(doc, open(sys.argv[4] if len(sys.argv) > 4 else TRAFFIC_JSON, "w"), indent=1)
        print(json.dumps(doc, indent=1))
        return 0
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm", action="store_true", help="also time 20 back-to-back calls without the flush")
    ap.add_argument("--skip-extras", action="store_true",
                    help="leave out the KV-cache, fp16, key-padding and Q/K/V projection measurements")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run one device copy of MIB MiB (reference for HBM counters)")
    ap.add_argument("--perf-log", default=None, metavar="PATH",
                    help="append one JSON line per measured leg (workload, kernel, revision, median/p95, "
                         "rate, fraction of roofline, parity) to PATH")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the kernels run per GPU and the multi-GPU sharding is a design note, not built.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import causal_head_attention_amd as attn
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    pc = workloads.BF16_S2048
    dc = workloads.BF16_DECODE

    log("generating inputs")
    q_h, k_h, v_h = workloads.make_prefill(pc)
    seqlens_h, qd_h, kc_h, vc_h = workloads.make_decode(dc)
    q, k, v = (t.to(dev) for t in (q_h, k_h, v_h))
    o = torch.empty_like(q)
    seqlens, qd, kc, vc = (t.to(dev) for t in (seqlens_h, qd_h, kc_h, vc_h))
    od = torch.empty_like(qd)
    ws = torch.empty(attn.attn_decode_workspace_bytes(dc.B, dc.H, dc.S_cap, dc.D), dtype=torch.uint8,
                     device=dev)
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    flops = pc.flops()
    dec_bytes = workloads.decode_kv_bytes(seqlens_h.tolist(), dc.H, dc.D, 2, dc.S_cap)

    hev = HipEvents()
    # one clock-probe row per timed step: the prefill kernel's workgroup 0
    # writes (shader clock, 100 MHz real time) at its start and at its end
    clk = torch.zeros(args.steps, 4, dtype=torch.int64, device=dev)

    def step(evs, probe=None):
        # events are attached to the kernels themselves (hipExtLaunchKernelGGL),
        # so each interval is the call's device time on its own stream
        flush.zero_()
        attn.attn_set_timing_events(evs[0], evs[1])
        attn.attn_set_clock_probe(probe)
        attn.attn_fwd(q, k, v, o, causal=True)
        flush.zero_()
        attn.attn_set_timing_events(evs[2], evs[3])
        attn.attn_decode(qd, kc, vc, seqlens, od, ws)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        evs = hev.create(4)
        step(evs)
        torch.cuda.synchronize()
        hev.destroy(evs)

    log(f"timing {args.steps} steps")
    events = [hev.create(4) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, evs in enumerate(events):
        step(evs, clk[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = [hev.ms(e[0], e[1]) for e in events]
    dec_ms = [hev.ms(e[2], e[3]) for e in events]
    for e in events:
        hev.destroy(e)
    c = clk.cpu().numpy()
    clock_ghz = [(c[i, 2] - c[i, 0]) / (c[i, 3] - c[i, 1]) * 0.1 for i in range(args.steps) if c[i, 3] > c[i, 1]]

    # the read-only reference: a plain non-temporal read of as many bytes as
    # one decode call reads, on this same GPU, cold like the decode
    log("read-only stream reference")
    import ctypes
    probe_lib = ctypes.CDLL(os.path.join(ROOT, "causal_head_attention_amd", "libattn_probe.so"))
    rs = probe_lib.attn_probe_read_stream
    rs.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_void_p]
    rs.restype = ctypes.c_int
    rs_bytes = dec_bytes // 16 * 16
    rs_buf = torch.ones(rs_bytes, dtype=torch.uint8, device=dev)
    rs_out = torch.empty(256 * 512, dtype=torch.int32, device=dev)
    rs_stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    rs_ms = []
    for i in range(23):
        e = hev.create(2)
        flush.zero_()
        if rs(rs_buf.data_ptr(), rs_bytes, rs_out.data_ptr(), rs_stream, e[0], e[1]) != 0:
            raise RuntimeError("attn_probe_read_stream failed")
        torch.cuda.synchronize()
        if i >= 3:
            rs_ms.append(hev.ms(e[0], e[1]))
        hev.destroy(e)
    del rs_buf, rs_out

    # warm-cache figures (no flush), for context only
    warm_f, warm_d = [], []
    if args.warm:
        for _ in range(20):
            e = hev.create(4)
            attn.attn_set_timing_events(e[0], e[1])
            attn.attn_fwd(q, k, v, o, causal=True)
            attn.attn_set_timing_events(e[2], e[3])
            attn.attn_decode(qd, kc, vc, seqlens, od, ws)
            torch.cuda.synchronize()
            warm_f.append(hev.ms(e[0], e[1]))
            warm_d.append(hev.ms(e[2], e[3]))
            hev.destroy(e)

    # KV-cache prefill (chunk of 512 queries per sequence against caches of
    # per-sequence length): the same tile kernel behind attn_fwd_kvcache,
    # timed cold like the step, outside the step's headline figure
    def cold_ms(call, n=20):
        """Device time of `call` (events on its kernels), 512 MiB fill before each."""
        for _ in range(3):
            call()
        torch.cuda.synchronize()
        out = []
        for _ in range(n):
            e = hev.create(2)
            flush.zero_()
            attn.attn_set_timing_events(e[0], e[1])
            call()
            torch.cuda.synchronize()
            out.append(hev.ms(e[0], e[1]))
            hev.destroy(e)
        return out

    def mfma_leg(ms, flop, workload):
        med = statistics.median(ms)
        tf = flop / (med * 1e-3) / 1e12
        return {"value": round(tf, 2), "unit": "TFLOPS", "workload": workload,
                "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                             "flop_per_launch": flop, "median_launch_us": round(med * 1e3, 2),
                             "mean_launch_us": round(statistics.fmean(ms) * 1e3, 2)}}

    kv = f16 = kp = qp = pe_leg = sm_leg = f32 = nc = s4k = None
    if not args.skip_extras:
        kc_cfg = workloads.BF16_KVCACHE
        log("KV-cache prefill: generating inputs")
        sl_kv_h, q_kv_h, kc_kv_h, vc_kv_h = workloads.make_kvcache_prefill(kc_cfg)
        sl_kv, q_kv, kc_kv, vc_kv = (t.to(dev) for t in (sl_kv_h, q_kv_h, kc_kv_h, vc_kv_h))
        o_kv = torch.empty_like(q_kv)
        lse_kv = torch.empty((kc_cfg.B, kc_cfg.H, kc_cfg.S_q), dtype=torch.float32, device=dev)
        kv_flops = kc_cfg.flops(sl_kv_h.tolist())

        def kv_call():
            attn.attn_fwd_kvcache(q_kv, kc_kv, vc_kv, sl_kv, o_kv, causal=True)

        kv = mfma_leg(cold_ms(kv_call), kv_flops,
                      f"bf16 causal chunk of {kc_cfg.S_q} queries x {kc_cfg.B} sequences, H={kc_cfg.H} "
                      f"D={kc_cfg.D}, cache capacity {kc_cfg.S_cap}, lengths {sl_kv_h.tolist()} (seed "
                      f"{kc_cfg.seed}); cold, 20 calls")
        del kc_kv, vc_kv

        # the bf16_s2048 shape with fp16 storage (v_mfma_f32_32x32x16_f16;
        # the dense fp16 peak equals the bf16 one)
        fc = workloads.FP16_S2048
        log("fp16 prefill")
        q16, k16, v16 = (t.to(dev) for t in workloads.make_prefill(fc))
        o16 = torch.empty_like(q16)
        f16 = mfma_leg(cold_ms(lambda: attn.attn_fwd(q16, k16, v16, o16, causal=True)), fc.flops(),
                       f"fp16 causal prefill B={fc.B} H={fc.H} S={fc.S_q} D={fc.D} (seed {fc.seed}); "
                       f"cold, 20 calls")
        del q16, k16, v16, o16

        # key-padding forward: right-padded entries, no causal rule; FLOP over
        # the visible (query, key) pairs only
        pc_k = workloads.BF16_KEYPAD
        log("key-padding prefill")
        lens_k, mask_k, qk_h, kk_h, vk_h = workloads.make_keypad_prefill(pc_k)
        qk, kk, vk, mk = (t.to(dev) for t in (qk_h, kk_h, vk_h, mask_k))
        ok = torch.empty_like(qk)
        kp = mfma_leg(cold_ms(lambda: attn.attn_fwd_mask(qk, kk, vk, mk, ok, causal=False)),
                      pc_k.flops(lens_k.tolist()),
                      f"bf16 key-padding forward B={pc_k.B} H={pc_k.H} S={pc_k.S} D={pc_k.D}, no causal rule, "
                      f"key lengths {lens_k.tolist()} (seed {pc_k.seed}); cold, 20 calls")
        del qk, kk, vk, mk, ok

        # the Q/K/V projection of the bf16_s2048 layer as one GEMM
        qc = workloads.BF16_QKV
        log("Q/K/V projection")
        xq_h, wq_h = workloads.make_qkv_proj(qc)
        xq, wq = xq_h.to(dev), wq_h.to(dev)
        outs = [torch.empty(qc.B, qc.S, qc.H, qc.D, dtype=qc.dtype, device=dev) for _ in range(3)]
        qp = mfma_leg(cold_ms(lambda: attn.qkv_proj(xq, wq, qc.H, qc.D, *outs)), qc.flops(),
                      f"bf16 Q/K/V projection M={qc.B * qc.S} E={qc.E} N=3x{qc.H * qc.D} (seed {qc.seed}); "
                      f"cold, 20 calls")
        del xq, wq, outs

        # the sinusoidal position-encoding table (fp32, HBM-bound: one write)
        log("position encoding table")
        pe_t = torch.empty(workloads.PE_S, workloads.PE_D, dtype=torch.float32, device=dev)
        pe_ms = cold_ms(lambda: attn.sinusoidal_pe(workloads.PE_S, workloads.PE_D, 0, out=pe_t))
        pe_mean = statistics.median(pe_ms)
        pe_bytes = workloads.PE_S * workloads.PE_D * 4
        pe_gbs = pe_bytes / (pe_mean * 1e-3) / 1e9
        pe_leg = {"value": round(pe_gbs, 1), "unit": "GB/s",
                  "workload": f"fp32 sinusoidal position table S={workloads.PE_S} d_model={workloads.PE_D}; "
                              f"cold, 20 calls",
                  "roofline": {"bound": "hbm", "achieved": round(pe_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(pe_gbs / HBM_PEAK_GBS, 4), "bytes_per_call": pe_bytes,
                               "median_launch_us": round(pe_mean * 1e3, 2)}}
        del pe_t

        # the standalone masked softmax over the bf16_s2048 layer's score
        # matrix (HBM-bound: visible scores read once, all of P written once)
        sc = workloads.BF16_SOFTMAX
        log("masked softmax")
        s_sm = workloads.make_scores(sc).to(dev)
        p_sm = torch.empty_like(s_sm)
        sm_ms = cold_ms(lambda: attn.masked_softmax(s_sm, sc.scale, sc.causal, out=p_sm))
        sm_mean = statistics.median(sm_ms)
        sm_bytes = sc.algorithmic_bytes()
        sm_gbs = sm_bytes / (sm_mean * 1e-3) / 1e9
        sm_leg = {"value": round(sm_gbs, 1), "unit": "GB/s",
                  "workload": f"bf16 causal score matrix [{sc.B}, {sc.H}, {sc.S_q}, {sc.S_kv}] ~ N(0, 128), "
                              f"scale 1/sqrt(128) (seed {sc.seed}); cold, 20 calls",
                  "roofline": {"bound": "hbm", "achieved": round(sm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                               "frac": round(sm_gbs / HBM_PEAK_GBS, 4), "bytes_per_call": sm_bytes,
                               "median_launch_us": round(sm_mean * 1e3, 2)}}
        del s_sm, p_sm

        # the bf16_s2048 data without the causal rule: every query block walks
        # all 32 key tiles (two blocks per workgroup)
        log("non-causal prefill")
        ncf = workloads.visible_pairs(pc.S_q, pc.S_kv, False) * 4 * pc.B * pc.H * pc.D
        onc = torch.empty_like(q)
        nc = mfma_leg(cold_ms(lambda: attn.attn_fwd(q, k, v, onc, causal=False)), ncf,
                      f"bf16 non-causal prefill B={pc.B} H={pc.H} S={pc.S_q} D={pc.D} (the bf16_s2048 data, "
                      f"seed {pc.seed}); cold, 20 calls")
        del onc

        # bf16 causal S=4096 with Q, K ~ N(0, 4^2): logits up to about +-100,
        # the softmax-stability workload at twice the sequence length
        c4k = workloads.BF16_S4096
        log("S=4096 prefill")
        q4, k4, v4 = (t.to(dev) for t in workloads.make_prefill(c4k))
        o4 = torch.empty_like(q4)
        s4k = mfma_leg(cold_ms(lambda: attn.attn_fwd(q4, k4, v4, o4, causal=True)), c4k.flops(),
                       f"bf16 causal prefill B={c4k.B} H={c4k.H} S={c4k.S_q} D={c4k.D}, Q and K ~ N(0, 4^2) "
                       f"(seed {c4k.seed}); cold, 20 calls")
        del q4, k4, v4, o4

        # the fp32 configuration (fp32 MFMA kernel), against the dense fp32
        # matrix peak
        c32 = workloads.FP32_SMALL
        log("fp32 prefill")
        q32, k32, v32 = (t.to(dev) for t in workloads.make_prefill(c32))
        o32 = torch.empty_like(q32)
        f32_ms = cold_ms(lambda: attn.attn_fwd(q32, k32, v32, o32, causal=True))
        f32_mean = statistics.median(f32_ms)
        f32_tf = c32.flops() / (f32_mean * 1e-3) / 1e12
        f32 = {"value": round(f32_tf, 3), "unit": "TFLOPS",
               "workload": f"fp32 causal prefill B={c32.B} H={c32.H} S={c32.S_q} D={c32.D} (seed {c32.seed}), "
                           f"v_mfma_f32_32x32x2_f32 for both products; cold, 20 calls",
               "roofline": {"bound": "mfma", "achieved": round(f32_tf, 3), "peak": FP32_MFMA_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(f32_tf / FP32_MFMA_PEAK_TFLOPS, 4),
                            "kernel": "fwd_f32_kernel<64>",
                            "flop_per_launch": c32.flops(), "median_launch_us": round(f32_mean * 1e3, 2)}}
        del q32, k32, v32, o32

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n} bytes read, {n} bytes written")

    # headline rates from the median call (the mean is reported beside it)
    fwd_med = statistics.median(fwd_ms)
    dec_med = statistics.median(dec_ms)
    tflops = flops / (fwd_med * 1e-3) / 1e12
    dec_gbs = dec_bytes / (dec_med * 1e-3) / 1e9
    clk_ghz = statistics.median(clock_ghz) if clock_ghz else None
    rs_gbs = rs_bytes / (statistics.median(rs_ms) * 1e-3) / 1e9

    # quick parity sample on the benchmarked outputs
    o_h = o.float().cpu().double().numpy()
    od_h = od.float().cpu().double().numpy()

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        import oracle
        log("CPU baseline: fp64 oracle on the full prefill workload, repeated for >= 10 s")
        passes, cpu_s = 0, 0.0
        while passes < 30 and (cpu_s < 10.0 or passes == 0):
            t = time.perf_counter()
            ref = oracle.attn_fwd(q_h, k_h, v_h, True)
            cpu_s += time.perf_counter() - t
            passes += 1
        cpu = {"value": passes * flops / cpu_s / 1e12, "unit": "TFLOPS", "cores": oracle.num_threads(),
               "kind": "oracle", "cpu_model": cpu_model(),
               "sample": f"full prefill workload (B=1 H=32 S=2048 D=128 causal), {passes} fp64 passes in "
                         f"{cpu_s:.2f} s; rate uses the same algorithmic FLOP count as the GPU figure"}
        err = np.abs(o_h - ref)
        parity = {"prefill_max_abs": float(err.max()),
                  "prefill_rel_l2": float(np.linalg.norm(o_h - ref) / np.linalg.norm(ref))}
        ref_d = np.zeros_like(od_h)
        for b in range(dc.B):
            n = int(seqlens_h[b])
            ref_d[b:b + 1] = oracle.attn_decode(qd_h[b:b + 1], kc_h[b:b + 1, :n], vc_h[b:b + 1, :n],
                                                np.array([n], dtype=np.int32))
        parity["decode_max_abs"] = float(np.abs(od_h - ref_d).max())

    line = {
        "metric": "causal attn fwd TFLOPS (bf16 S=2048 H=32 D=128); decode KV-read GB/s",
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(fwd_med + dec_med, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bf16 causal prefill B=1 H=32 S=2048 D=128 + bf16 decode B=16 H=32 D=128 "
                               "S_cap=4096 lengths U[1,4096] (seeds 1003, 1005)",
                   "cache": "cold (512 MiB fill before each call)",
                   "decode_tokens": int(sum(int(x) for x in seqlens_h))},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("prefill", PREFILL_SRC),
                     "kernel": "prefill_kernel<bf16,128>", "flop_per_launch": flops,
                     "rate_from": "median launch",
                     "median_launch_us": round(fwd_med * 1e3, 2),
                     "mean_launch_us": round(statistics.fmean(fwd_ms) * 1e3, 2),
                     "p95_launch_us": round(float(np.percentile(fwd_ms, 95)) * 1e3, 2),
                     "clock_ghz": round(clk_ghz, 3) if clk_ghz else None,
                     "clock_adjusted_frac": (round(tflops / (BF16_MFMA_PEAK_TFLOPS * clk_ghz / NOMINAL_CLOCK_GHZ), 4)
                                             if clk_ghz else None),
                     "clock_note": "shader clock over workgroup 0's run (s_memtime against the 100 MHz "
                                   "s_memrealtime), median over the timed calls; clock_adjusted_frac divides "
                                   f"by the peak scaled to that clock from {NOMINAL_CLOCK_GHZ} GHz"},
        "decode": {"value": round(dec_gbs, 1), "unit": "GB/s",
                   "roofline": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS,
                                "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                                "traffic": measured_traffic("decode", DECODE_SRC),
                                "bytes_per_call": dec_bytes,
                                "rate_from": "median call",
                                "median_call_us": round(dec_med * 1e3, 2),
                                "mean_call_us": round(statistics.fmean(dec_ms) * 1e3, 2),
                                "p95_call_us": round(float(np.percentile(dec_ms, 95)) * 1e3, 2),
                                "note": "one call = one kernel: 256 streaming workgroups and the merging "
                                        "workgroups after them"},
                   "read_stream_reference": {
                       "gbs": round(rs_gbs, 1), "frac_of_peak": round(rs_gbs / HBM_PEAK_GBS, 4),
                       "decode_over_reference": round(dec_gbs / rs_gbs, 4),
                       "bytes": rs_bytes, "median_us": round(statistics.median(rs_ms) * 1e3, 2),
                       "what": "libattn_probe.so read_stream_kernel: a plain non-temporal 16-byte-per-lane read "
                               "of the same number of bytes on this GPU, 256x512 threads, 16 loads in flight, "
                               "cold like the decode, median of 20"}},
        "warm_cache": ({"prefill_tflops": round(flops / (statistics.median(warm_f) * 1e-3) / 1e12, 2),
                        "decode_gbs": round(dec_bytes / (statistics.median(warm_d) * 1e-3) / 1e9, 1)}
                       if warm_f else None),
        "timing": "hipEvents attached to the first/last kernel dispatch of each call (start->end of the "
                  "kernels, no queueing gaps); 512 MiB fill before every call",
        "wall_ms_per_step_incl_flush": round(wall / args.steps * 1e3, 4),
        "kvcache_prefill": kv,
        "fp16_prefill": f16,
        "keypad_prefill": kp,
        "qkv_proj": qp,
        "position_encoding": pe_leg,
        "masked_softmax": sm_leg,
        "fp32_prefill": f32,
        "noncausal_prefill": nc,
        "s4096_prefill": s4k,
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(line), flush=True)
    if args.perf_log:
        append_perf_log(args.perf_log, line)
    return 0


def _git_rev():
    """The source revision: ATTN_GIT_REV if set (a copy of the tree without
    its history), else `git rev-parse HEAD`, else None."""
    rev = os.environ.get("ATTN_GIT_REV")
    if rev:
        return rev
    try:
        r = subprocess.run(["git", "rev-parse", "HEAD"], capture_output=True, text=True, cwd=ROOT, timeout=10)
        return (r.stdout.strip() or None) if r.returncode == 0 else None
    except (OSError, subprocess.SubprocessError):
        return None


def perf_log_records(line: dict) -> list:
    """One record per measured leg of a bench line: the per-version table of
    timings (P50 and P95, rate, fraction of the roofline) keyed by workload,
    kernel and source revision, so runs of different revisions line up."""
    common = {"rev": _git_rev(), "utc": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime()),
              "build": {"prefill": build_sha256(PREFILL_SRC)[:16], "decode": build_sha256(DECODE_SRC)[:16]},
              "algo": os.environ.get("ATTN_ALGO", "auto")}
    cpu = line.get("cpu_baseline") or {}
    parity = line.get("parity") or {}
    roof = line["roofline"]
    recs = [dict(common, leg="prefill", workload=line["config"]["workload"].split(" + ")[0],
                 kernel=roof["kernel"], value=line["value"], unit=line["unit"], frac=roof["frac"],
                 median_us=roof["median_launch_us"], p95_us=roof["p95_launch_us"],
                 clock_ghz=roof.get("clock_ghz"), max_abs=parity.get("prefill_max_abs"),
                 rel_l2=parity.get("prefill_rel_l2"),
                 oracle_tflops=cpu.get("value"), host_cores=cpu.get("cores"))]
    dr = line["decode"]["roofline"]
    recs.append(dict(common, leg="decode", workload=line["config"]["workload"].split(" + ")[-1],
                     kernel="decode_kernel<bf16,128>", value=line["decode"]["value"], unit="GB/s",
                     frac=dr["frac"], median_us=dr["median_call_us"], p95_us=dr["p95_call_us"],
                     max_abs=parity.get("decode_max_abs")))
    for key, leg in line.items():
        if isinstance(leg, dict) and "roofline" in leg and key != "decode" and "workload" in leg:
            r = leg["roofline"]
            recs.append(dict(common, leg=key, workload=leg["workload"], kernel=r.get("kernel"),
                             value=leg["value"], unit=leg["unit"], frac=r.get("frac"),
                             median_us=r.get("median_launch_us"), p95_us=r.get("p95_launch_us")))
    return recs


def append_perf_log(path: str, line: dict) -> None:
    with open(path, "a") as f:
        for rec in perf_log_records(line):
            f.write(json.dumps(rec) + "\n")


if __name__ == "__main__":
    sys.exit(main())
