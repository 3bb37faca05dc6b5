"""Benchmark of the microscaling-FP4 attention forward on one MI355X.

One step = the whole hot path on one batch of seeded synthetic input already
resident in HBM: quantize Q, K and V (mxattn_quantize) and run the attention
forward (mxattn_fwd, bf16 output).  Prints ONE JSON line:

  value      = counted FLOP / step time, in TOPS (4 B H N^2 d for non-causal runs;
               causal and packed-document runs count the visible half,
               4 H d sum L(L+1)/2)
  roofline   = the forward kernel against the dense FP4 MFMA peak (10.1 PFLOP/s),
               its duration measured with HIP events around each launch
  cpu_baseline = the CPU oracle timed on a bounded sample of the same workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TOPS (4·B·H·N²·d/t) at N=32K, d=128; % of FP4 MFMA peak"
FP4_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4 MFMA
FP4_MEASURED_TFLOPS = 8200.0  # the same MFMA measured back to back on one MI355X
# HBM bytes per forward launch from rocprofv3 FETCH_SIZE/WRITE_SIZE runs, scaled by a
# plain-copy calibration; read from the committed profile summaries, which record the
# SHA-256 of the kernel source they were taken on (None when absent or stale)
TRAFFIC_FILES = {"c3": "profiles/fwd_pp_kernel_c3_video_dit_32k_traffic.txt",
                 "c4": "profiles/fwd_pp_kernel_c4_gqa_causal_32k_traffic.txt",
                 "c5": "profiles/fwd_pp_kernel_c5_varlen_causal_64k_traffic.txt",
                 "c2": "profiles/fwd_pp_kernel_c2_mha_4k_traffic.txt"}
# the forward kernel's source: the kernel file and the headers it includes
KERNEL_SOURCES = ["microscaling_fp4_attention_amd/csrc/fwd.hip", "microscaling_fp4_attention_amd/csrc/device_util.h",
                  "microscaling_fp4_attention_amd/csrc/formats.h", "microscaling_fp4_attention_amd/csrc/kernels.h"]
# the same for the split-key decode at 128K keys (V tile-major), its main kernel
# decode at 128K keys, role VT: the MXFP4 route's profile and the QK4PV8 route's
DECODE_TRAFFIC_FILES = {False: "profiles/decode_kernel_gqa_128k.txt", True: "profiles/decode_qk4pv8_gqa_128k.txt"}
DECODE_SOURCES = ["microscaling_fp4_attention_amd/csrc/decode.hip"] + KERNEL_SOURCES[1:]


def _code_only(text):
    """C/C++ source without its comments, trailing blanks and empty lines (string and
    character literals kept as written)"""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":  # a literal: copy through its closing quote
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (ln.rstrip() for ln in "".join(out).split("\n"))
    return "\n".join(ln for ln in lines if ln)


def kernel_source_sha256(sources=None):
    """SHA-256 over a kernel's source files (the forward's by default), in list order,
    taken over their code only: an edit of comments or blank lines keeps the hash, so a
    profile stays tied to the code it measured"""
    import hashlib
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()


def profiled_traffic(cfg):
    return read_traffic(TRAFFIC_FILES.get(cfg, ""), KERNEL_SOURCES)


def read_traffic(rel, sources):
    path = os.path.join(ROOT, rel)
    if not rel or not os.path.isfile(path):
        return None
    fields = {}
    for line in open(path):
        if "=" in line:
            k, v = line.split("=", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_sha256(sources):
        return None  # the kernel changed since the counters were taken
    v = fields.get("traffic_bytes_per_launch")
    return int(v) if v is not None else None


BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0

# workload -> (Q/K format, V format, P mode, P format, description)
CONFIGS = {
    "c1": ("c1_single_head", "mxfp4", "mxfp4", "two_level", "nvfp4",
           "B1 H1 N1024 d128 non-causal, K with per-channel mean; MXFP4 Q/K/V, two-level P (E4M3/16)"),
    "c2": ("c2_mha_4k", "mxfp4", "mxfp4", "two_level", "nvfp4",
           "B2 H16 N4096 d128 non-causal, K mean + 0.1% x20 outliers; MXFP4 Q/K/V, two-level P (E4M3/16)"),
    "c3": ("c3_video_dit_32k", "mxfp4_uos", "mxfp4_uos", "pnq", "mxfp4_uos",
           "B1 H24 N32768 d128 non-causal, rank-16 peaked Q/K; MXFP4 UOS (Qmax 7.25) Q/K/V/P, PNQ"),
    "c4": ("c4_gqa_causal_32k", "nvfp4", "fp8v", "fp8", None,
           "B1 Hq32 Hkv8 N32768 d128 causal, K mean; QK4PV8: NVFP4 Q/K, FP8 P (scale 448) and V"),
    "c5": ("c5_varlen_causal_64k", "mxfp4", "mxfp4", "two_level", "nvfp4",
           "packed 65536 tokens (log-uniform 512..16384), H16 d128 block-diagonal causal, K outliers; "
           "MXFP4 Q/K/V, two-level P (E4M3/16)"),
    # the two-level forward at N = 32K, d = 128 on the video-DiT inputs, in both readings
    # of the level-2 block format: E4M3 per 16 keys (PV on the bf16 MFMA after exact
    # dequantization) and E8M0 per 32 keys (PV on the FP4 MFMA)
    "two_level_e4m3": ("c3_video_dit_32k", "mxfp4", "mxfp4", "two_level", "nvfp4",
                       "B1 H24 N32768 d128 non-causal, rank-16 peaked Q/K; MXFP4 Q/K/V, two-level P "
                       "(level-2 E4M3 per 16 keys)"),
    "two_level_e8m0": ("c3_video_dit_32k", "mxfp4", "mxfp4", "two_level", "mxfp4",
                       "B1 H24 N32768 d128 non-causal, rank-16 peaked Q/K; MXFP4 Q/K/V, two-level P "
                       "(level-2 E8M0 per 32 keys, OCP rule)"),
}


def route_peak(qf, vf, pm, pf):
    """MFMA types of the forward's two products and their combined dense peak (TFLOP/s):
    MXFP4 Q/K run on the FP4 MFMA, NVFP4 Q/K on f16 after exact dequantization (bf16 in
    the single-buffer kernel of the routes with an E4M3-scaled V, at the same peak); PV runs
    on FP8 for FP8 P, on FP4 for E8M0-scaled P with an MXFP4 V, on f16 for other P with an
    MXFP4 V (V's channels shifted into f16 range; under causally safe V the two diagonal
    key tiles of each query tile take bf16 products, at the same peak), on bf16 otherwise"""
    qk = ("fp4", FP4_PEAK_TFLOPS) if qf.startswith("mxfp4") else ("f16", BF16_PEAK_TFLOPS)
    if pm == "fp8":
        pv = ("fp8", FP8_PEAK_TFLOPS)
    elif pf is not None and pf.startswith("mxfp4") and vf.startswith("mxfp4"):
        pv = ("fp4", FP4_PEAK_TFLOPS)
    else:
        pv = ("f16" if vf.startswith("mxfp4") else "bf16", BF16_PEAK_TFLOPS)
    return f"QK {qk[0]}, PV {pv[0]}", 1.0 / (0.5 / qk[1] + 0.5 / pv[1])


def counted_flop(B, H, N, d, causal, doc_off):
    if doc_off is not None:
        L = np.diff(np.asarray(doc_off, np.int64))
        pairs = float(np.sum(L * (L + 1) // 2)) if causal else float(np.sum(L * L))
        return 4.0 * H * d * pairs
    if causal:
        return 4.0 * B * H * d * (N * (N + 1) / 2)
    return 4.0 * B * H * N * N * d


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads() -> int:
    """the host cores this process may use, at most 16 (one GPU's share of its host)"""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(wl, x, qf, vf, pm, pf, causal, doc_off, budget_s=10.0, exp_mode="exact"):
    """The oracle (plain C, one call per head or per block of query rows) on the host's
    cores: ctypes releases the GIL, so a thread pool runs the calls side by side.
    Quantization runs on the full Q, K and V; attention on query rows sampled from every
    query head (first and last rows, then evenly spaced ones) until the time budget is
    spent; the full forward's time is extrapolated from the per-row time."""
    import oracle
    import synth
    from concurrent.futures import ThreadPoolExecutor
    from tests.helpers import PM_ORACLE
    oracle.build(force=False)
    B, Hq, Hkv, N = wl["B"], wl["Hq"], wl["Hkv"], wl["N"]
    nthr = cpu_threads()
    pool = ThreadPoolExecutor(max_workers=nthr)

    def quant_qk_head(arr):
        c, sc = oracle.quantize_rows(arr, qf)
        return oracle.dequant_rows(c, sc, qf)

    def quant_v_head(arr):
        c, sc = oracle.quantize_cols(arr, vf, doc_off)
        return oracle.dequant_cols(c, sc, vf, doc_off)

    # quantization of the full tensors, one head per call (bf16 -> f32 widening untimed)
    qs = [synth.bf16_to_f32(x["q"][b, h]) for b in range(B) for h in range(Hq)]
    ks = [synth.bf16_to_f32(x["k"][b, h]) for b in range(B) for h in range(Hkv)]
    vs = [synth.bf16_to_f32(x["v"][b, h]) for b in range(B) for h in range(Hkv)]
    t0 = time.perf_counter()
    qd = list(pool.map(quant_qk_head, qs))
    kd = list(pool.map(quant_qk_head, ks))
    vd = list(pool.map(quant_v_head, vs))
    t_quant = time.perf_counter() - t0
    del qs, ks, vs

    def visible(i):
        if doc_off is not None:
            kidx = np.searchsorted(doc_off, i, side="right") - 1
            s0 = int(doc_off[kidx])
            return (i - s0 + 1) if causal else int(doc_off[kidx + 1]) - s0
        return (i + 1) if causal else N

    def rows_task(task):
        bh, rows = task
        b, h = divmod(bh, Hq)
        hk = h * Hkv // Hq
        oracle.attention(qd[bh][None, None], kd[b * Hkv + hk][None, None], vd[b * Hkv + hk][None, None],
                         PM_ORACLE[pm], pf, causal=causal, doc_off=doc_off, rows=rows, exp_mode=exp_mode)
        return sum(4.0 * 128 * visible(int(i)) for i in rows)

    # rows of every head in rounds: the first and last rows, then evenly spaced ones
    order = np.unique(np.concatenate([[0, N - 1], np.linspace(0, N - 1, num=min(N, 4096)).astype(np.int64)]))
    rng = np.random.default_rng(0)
    order = np.concatenate([order[[0, -1]], rng.permutation(order[1:-1])])
    # rows per head per round: calls of 4 rows, at least two per thread
    per = 4 * max(1, -(-2 * nthr // (B * Hq)))
    flop, nrows, t_att, r0 = 0.0, 0, 0.0, 0
    while t_att < budget_s and r0 < len(order):
        rows = np.sort(order[r0:r0 + per]).astype(np.int64)
        tasks = [(bh, rows[c:c + 4]) for bh in range(B * Hq) for c in range(0, len(rows), 4)]
        t0 = time.perf_counter()
        flop += sum(pool.map(rows_task, tasks))
        t_att += time.perf_counter() - t0
        nrows += len(rows) * B * Hq
        r0 += per
    pool.shutdown()
    total_rows = B * Hq * N
    t_full = t_quant + t_att / nrows * total_rows
    return {"value": flop / t_att / 1e12, "unit": "TOPS", "cores": nthr, "kind": "oracle",
            "cpu_model": cpu_model(),
            "quantize_s_full": round(t_quant, 3),
            "forward_s_extrapolated": round(t_full, 1),
            "sample": f"quantization of the full Q, K and V ({t_quant:.2f} s), then attention of {nrows} query "
                      f"rows ({nrows // (B * Hq)} per head, every head; {t_att:.1f} s) on {nthr} threads; value = "
                      f"counted FLOP of those rows / their wall time; the whole forward extrapolated from the "
                      f"per-row time: {t_full:.0f} s"}


def bench_decode(args, torch, mx):
    """Split-key decode step: quantize the new tokens' Q, then mxattn_decode over the cached,
    already quantized history.  Inputs are seeded normal bf16 drawn on the device."""
    B, Hq, Hkv, R, N = 4, 32, 8, 1, args.decode
    q4p8 = args.decode_route == "qk4pv8"  # NVFP4 Q/K, FP8 P and V
    qkf, vf = ("nvfp4", "fp8v") if q4p8 else ("mxfp4", "mxfp4")
    layout = args.decode_layout
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    q = torch.randn((B, Hq, R, 128), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((B, Hkv, N, 128), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((B, Hkv, N, 128), generator=g, device=dev).to(torch.bfloat16)
    K = mx.quantize(k, mx.ROLE_QK, qkf)
    V = mx.quantize(v, mx.ROLE_VT if layout == "vt" else mx.ROLE_V, vf)
    del k, v
    params = mx.fwd_params("fp8", None, causal=True, out_fp32=False) if q4p8 else \
        mx.fwd_params("two_level", "mxfp4", causal=True, out_fp32=False)
    out = torch.empty((B, Hq, R, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mx.decode_workspace_bytes(B, Hq, R, N), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    ev = []

    def step(record):
        Q = mx.quantize(q, mx.ROLE_QK, qkf)
        if record:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        mx.decode(Q, K, V, params, out=out, workspace=ws)
        if record:
            e1.record(stream)
            ev.append((e0, e1))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(args.steps):
        step(True)
    g1.record(stream)
    torch.cuda.synchronize()
    t_step = g0.elapsed_time(g1) / 1e3 / args.steps
    t_dec = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    hist = K.codes.numel() + K.scales.numel() + V.codes.numel() + V.scales.numel()  # history bytes read once
    gbs = hist / t_dec / 1e9
    route = "NVFP4 Q/K, FP8 P (E4M3 448 P~) and V" if q4p8 else "MXFP4 K/V/Q, two-level P"
    res = {"metric": "decode: quantized KV history read per second (GB/s), split-key "
                     + ("QK4PV8 decode" if q4p8 else "MXFP4 decode"),
           "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(t_step * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "nvfp4+fp8" if q4p8 else "mxfp4", "data": "synthetic (seeded normal bf16 drawn on the device)",
           "config": {"workload": f"decode: B{B} Hq{Hq} Hkv{Hkv} R{R} history {N} keys, {route}, "
                                  f"splits of 256 keys, V {'tile-major (role VT)' if layout == 'vt' else 'role V'}",
                      "history_bytes": hist},
           "t_decode_ms": round(t_dec * 1e3, 4),
           "tokens_per_s": round(B * R / t_step, 1),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": 8000.0, "unit": "GB/s",
                        "frac": round(gbs / 8000.0, 4),
                        "traffic": read_traffic(DECODE_TRAFFIC_FILES[q4p8], DECODE_SOURCES)
                        if (N, layout) == (131072, "vt") else None,
                        "kernel": "split-key decode (mxattn_decode)"}}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c3", choices=sorted(CONFIGS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--preproc", default="none", choices=["none", "smoothk", "center", "hadamard", "center+hadamard"],
                    help="outlier pre-processing of Q and K inside the step: smooth-K (K mean), sequence centering "
                         "with the compensation bias, and/or the normalized Hadamard rotation")
    ap.add_argument("--causal-safe", action="store_true",
                    help="causally safe V scales: quantize the per-key form of V in the step and use it on the "
                         "two key tiles of each 256-row query tile the causal boundary runs through (causal "
                         "workloads with a 4-bit V)")
    ap.add_argument("--exp", default="exact", choices=["exact", "mitchell", "schraudolph"],
                    help="exponential of P~: exact (hardware exp), or the bit-level Mitchell-P / Schraudolph "
                         "approximations for inference (ping-pong kernel routes)")
    ap.add_argument("--decode", type=int, default=0, metavar="N",
                    help="time the split-key decode instead: 4 requests, GQA 32:8, one new token each over an "
                         "N-key MXFP4 history (HBM-bound; reports the history bytes read per second)")
    ap.add_argument("--decode-layout", default="vt", choices=["vt", "v"],
                    help="layout of the decode's quantized V history: tile-major (role VT, the decode's own) or "
                         "role V (the prefill's)")
    ap.add_argument("--decode-route", default="mxfp4", choices=["mxfp4", "qk4pv8"],
                    help="operand route of the decode: MXFP4 Q/K/V with two-level P, or NVFP4 Q/K with FP8 P and V")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the attention forward is a single-GPU kernel here "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import microscaling_fp4_attention_amd as mx

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return

    if args.decode:
        bench_decode(args, torch, mx)
        return

    name, qf, vf, pm, pf, desc = CONFIGS[args.config]
    if args.causal_safe and (vf == "fp8v" or args.config in ("c1", "c2", "c3")):
        print("--causal-safe applies to the causal workloads with a 4-bit V (c5); an FP8 V is made safe by its "
              "round-up exponents", file=sys.stderr)
        sys.exit(2)
    log = (lambda *a: None) if args.quiet else (lambda *a: print(*a, file=sys.stderr, flush=True))
    t0 = time.time()
    x = synth.workload(name)
    log(f"[bench] inputs for {name} generated in {time.time() - t0:.1f} s")
    B, Hq, Hkv, N = x["B"], x["Hq"], x["Hkv"], x["N"]
    causal, doc_off = x["causal"], x["doc_off"]
    dev = torch.device("cuda:0")

    def to_dev(a):
        return torch.from_numpy(a.astype(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    cu = None if doc_off is None else torch.from_numpy(doc_off.astype(np.int32)).to(dev)
    params = mx.fwd_params(pm, pf, causal=causal, out_fp32=False, exp_mode=args.exp)
    center = args.preproc.startswith("center")
    smoothk = args.preproc == "smoothk"
    had = args.preproc.endswith("hadamard")
    ws, nd = None, 0
    if doc_off is not None:
        ws = mx.fwd_plan(doc_off, N, causal)
        nd = len(doc_off) - 1
    out = torch.empty((B, Hq, N, 128), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    ev = []

    def step(record):
        p = params
        if record:
            es = torch.cuda.Event(enable_timing=True)
            es.record(stream)
        if args.preproc == "none":
            Q = mx.quantize(q, mx.ROLE_QK, qf)
            K = mx.quantize(k, mx.ROLE_QK, qf)
        else:
            qm = mx.channel_mean(q, cu) if center else None
            km = mx.channel_mean(k, cu) if (center or smoothk) else None
            Q = mx.quantize(q, mx.ROLE_QK, qf, cu_seqlens=cu, mean=qm, hadamard=had)
            K = mx.quantize(k, mx.ROLE_QK, qf, cu_seqlens=cu, mean=km, hadamard=had)
            if center:
                p = mx.fwd_params(pm, pf, causal=causal, out_fp32=False, score_bias=mx.center_comp(qm, k, km, cu),
                                  exp_mode=args.exp)
        V = mx.quantize(v, mx.ROLE_V, vf, cu_seqlens=cu)
        if args.causal_safe:
            Vk = mx.quantize(v, mx.ROLE_VKEY, vf, cu_seqlens=cu)
            p = mx.fwd_params(pm, pf, causal=causal, out_fp32=False, score_bias=getattr(p, "_score_bias_ref", None),
                              vkey=Vk, exp_mode=args.exp)
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        mx.fwd(Q, K, V, p, out=out, workspace=ws, ndocs=nd)
        if record:
            e1.record(stream)
            ev.append((es, e0, e1))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for _ in range(args.steps):
        step(True)
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    t_step = g0.elapsed_time(g1) / 1e3 / args.steps
    Qx, Kx, Vx = mx.quantize(q, mx.ROLE_QK, qf), mx.quantize(k, mx.ROLE_QK, qf), mx.quantize(v, mx.ROLE_V, vf, cu_seqlens=cu)
    quant_bytes = 2 * (q.numel() + k.numel() + v.numel()) + sum(t.codes.numel() + t.scales.numel() for t in (Qx, Kx, Vx))
    del Qx, Kx, Vx
    fwd_ms = np.array([a.elapsed_time(b) for _, a, b in ev])
    quant_ms = np.array([a.elapsed_time(b) for a, b, _ in ev])
    t_fwd = float(np.mean(fwd_ms)) / 1e3
    # the quantize pass's bandwidth against a plain device copy (read + write) of 1 GiB,
    # four times the 256 MB Infinity Cache, timed after the steps on the same stream
    src = torch.empty(1 << 29, dtype=torch.int16, device=q.device)
    cp = torch.empty_like(src)
    cp.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(3):
        cp.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 3 * 2 * 2 * src.numel() / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, cp
    log(f"[bench] step {t_step * 1e3:.3f} ms (wall {wall / args.steps * 1e3:.3f} ms), fwd {t_fwd * 1e3:.3f} ms")

    flop = counted_flop(B, Hq, N, 128, causal, doc_off)
    route, rpeak = route_peak(qf, vf, pm, pf)
    tops = flop / t_step / 1e12
    fwd_tflops = flop / t_fwd / 1e12
    peak = FP4_PEAK_TFLOPS
    res = {
        "metric": METRIC,
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4" if qf.startswith("mxfp4") else "nvfp4+fp8" if pm == "fp8" else "nvfp4",
        "data": "synthetic (seeded SplitMix64/Box-Muller bf16 tensors of the workload's shape and structure)",
        "config": {"workload": f"{name}: {desc}", "B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "d": 128,
                   "causal": bool(causal), "ndocs": nd, "preproc": args.preproc,
                   "causal_safe_v": bool(args.causal_safe), "exp": args.exp, "counted_flop": flop},
        "pct_fp4_peak": round(100.0 * tops / FP4_PEAK_TFLOPS, 2),
        "t_fwd_ms": round(t_fwd * 1e3, 4),
        "t_quant_ms": round((t_step - t_fwd) * 1e3, 4),  # quantization and any pre-processing
        "t_fwd_median_ms": round(float(np.median(fwd_ms)), 4),
        "t_fwd_min_ms": round(float(np.min(fwd_ms)), 4),
        "t_quant_median_ms": round(float(np.median(quant_ms)), 4),
        # the quantize pass reads bf16 Q, K, V and writes their codes and scales
        "quant_gbs": round(quant_bytes / (float(np.median(quant_ms)) * 1e-3) / 1e9, 1) if args.preproc == "none" else None,
        "copy_gbs": round(copy_gbs, 1),  # torch copy_ of 1 GiB, read + write
        "roofline": {"bound": "mfma", "achieved": round(fwd_tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(fwd_tflops / peak, 4),
                     "traffic": profiled_traffic(args.config)
                     if args.preproc == "none" and not args.causal_safe and args.exp == "exact" else None,
                     "kernel": "attention forward (mxattn_fwd)",
                     # the operand route's own dense MFMA peak: QK and PV are half the FLOP each
                     "route_peak": round(rpeak, 1), "route_frac": round(fwd_tflops / rpeak, 4),
                     "route": route,
                     # the FP4 MFMA's rate measured on this chip with back-to-back 32x32x64
                     # MFMAs in every wave (8.2 PFLOP/s), beside the 10.1 PFLOP/s spec
                     "measured_fp4_peak": FP4_MEASURED_TFLOPS,
                     "measured_fp4_frac": round(fwd_tflops / FP4_MEASURED_TFLOPS, 4)},
        # the second ceiling: one exponential per visible score element (4 d = 512 counted
        # FLOP each), per nominal clock (2.4 GHz) per CU (256); 100% of the FP4 MFMA peak
        # would need 10.1e15 / 512 / (2.4e9 * 256) = 32.1 per clock per CU
        "softmax": {"exps_per_clk_per_cu": round(flop / 512.0 / t_fwd / (2.4e9 * 256), 2),
                    "at_fp4_peak": round(FP4_PEAK_TFLOPS * 1e12 / 512.0 / (2.4e9 * 256), 2)},
    }
    if not args.no_cpu:
        log("[bench] timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(x, x, qf, vf, pm, pf, causal, doc_off, exp_mode=args.exp)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
