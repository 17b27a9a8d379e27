#!/usr/bin/env python3
"""Benchmark of the GDN recurrence library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one gdn_forward call of the chunked causal form (64-token chunks, bf16
MFMA) with the fp32 state carried in and out, over the batched d=128 workload:
B=2 (guidance pair), H=32, T=32760 (21 latent frames x 30x52 tokens),
d_k=d_v=128, bf16 q/k/v/out, fp32 beta/decay/state, decay a = exp(-softplus(N(2,1))).
Inputs are seeded synthetic data (see gated_deltanet_recurrence_gdn_amd/inputs.py),
resident in HBM before timing starts.

Prints ONE JSON line: throughput in token*heads/s, the dominant kernel's HBM
roofline (algorithmic bytes / average kernel time from HIP events on the launch
stream), its MFMA utilisation, the float64 CPU oracle timed on a bounded sample of
the same inputs, and secondary measurements of the other forms (sequential scan,
5-call streaming, bidirectional).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_MFMA_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
FP32_VALU_PEAK_TFS = 157.3   # MI355X fp32 vector (published; counts packed FP32)
FP32_VALU_NOPACK_TFS = 78.6  # the same without packed FP32, which this build does not emit
CHUNK_KERNEL = "tm_kernel + chunk_kernel"  # the two launches of one chunked gdn_forward
PROFILES = os.path.join(ROOT, "profiles")


def algorithmic_bytes(B, T, H, dk, dv, es=2, es_out=None):
    """q, k, v read in the input dtype (es bytes) and out written (es_out bytes, es by
    default), beta and decay read in fp32, the fp32 state read once and written once."""
    es_out = es if es_out is None else es_out
    return B * T * H * ((2 * dk + dv) * es + dv * es_out + 8) + 2 * B * H * dk * dv * 4


def chunk_flops(B, T, H, dk, dv, C=64):
    """Dense-tile flop count of the chunked form per token*head:
    6 dk dv (K S^T, Q S^T and the state update) + 2C(3dk + 2dv) (K K^T, Q K^T, T R, P N
    and the chunk-local products) + C^2/3 (the triangular inverse)."""
    return B * T * H * (6 * dk * dv + 2 * C * (3 * dk + 2 * dv) + C * C / 3.0)


def scan_flops(B, T, H, dk, dv):
    """Two dot products and one rank-1 update per state row: 6 dk dv per token*head."""
    return B * T * H * 6 * dk * dv


def load_profile(name, source="gdn_chunk.hip"):
    """A committed rocprofv3 --pmc summary (profiles/<name>.json), if it was taken on the
    current kernel code (comments and whitespace aside); else None."""
    p = os.path.join(PROFILES, f"{name}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    from gated_deltanet_recurrence_gdn_amd.srchash import code_hash
    if t.get("kernel_code_sha256_16") != code_hash(source):
        return None
    return t


def load_traffic(workload):
    """HBM bytes per launch of the chunked kernel from the committed --pmc summary."""
    return load_profile(f"chunk_kernel_{workload}_traffic")


def provenance(torch, x):
    """What the numbers were measured on: input hash, software versions, host CPUs."""
    from gated_deltanet_recurrence_gdn_amd import inputs
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"inputs_sha256": inputs.sha256(x), "torch": torch.__version__, "hip": torch.version.hip,
            "gpu": torch.cuda.get_device_name(0), "host_cpus": os.cpu_count(), "host_cpus_usable": usable,
            "host_cpu_model": model}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=40,
                    help="untimed steps; the clock settles over the first ~30 launches of this kernel")
    ap.add_argument("--cpu-sample-tokens", type=int, default=0,
                    help="tokens per head of the oracle's CPU sample (prefix of the same inputs); "
                         "0 = every token of the workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-forms", action="store_true", help="skip the secondary forms")
    ap.add_argument("--form", choices=["chunked", "scan"], default="chunked",
                    help="the timed step: the chunked form (the benchmark) or, for profiling the scan "
                         "kernel with rocprofv3, the sequential scan on the same inputs")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run one plain 512 MiB device-to-device copy (a known-size "
                         "reference dispatch for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU; --gpus {args.gpus} is not supported "
              "(the per-head recurrence shards over (b, h) with no exchange, but no "
              "multi-GPU path is built)", file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_deltanet_recurrence_gdn_amd import inputs
    from gated_deltanet_recurrence_gdn_amd import binding as gb

    w = inputs.WORKLOADS["batched_bf16_d128"]
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    t0 = time.time()
    x = inputs.make_workload(w)
    gen_s = time.time() - t0
    d = {k_: v_.cuda() for k_, v_ in x.items()}
    s_in = torch.zeros((B, H, dv, dk), dtype=torch.float32, device="cuda")
    s_out = torch.empty_like(s_in)
    out = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device="cuda")
    g = gb.GDN(B, H, dk, dv, "bf16", max_T=T)
    stream = gb.current_stream()

    chunk_len = 64 if args.form == "chunked" else 1

    def step():
        st = gb.gdn_forward(g.h, d["q"], d["k"], d["v"], d["beta"], d["decay"], s_in, s_out, out, T, chunk_len,
                            stream)
        if st != gb.GDN_OK:
            raise gb.GDNError(st, gb.gdn_last_error(g.h))

    # The secondary forms are measured first (each after its own untimed calls), so the
    # headline's warm-up and timed steps follow seconds of GPU work.
    forms = None if args.no_forms else measure_forms(torch, gb, inputs, d, g, x)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = ev0.elapsed_time(ev1) / args.steps  # one gdn_forward (its two kernel launches) per step
    ms_per_step = wall * 1000.0 / args.steps
    th = B * H * T
    value = th / (ms_per_step / 1000.0)

    abytes = algorithmic_bytes(B, T, H, dk, dv)
    achieved = abytes / (kern_ms / 1000.0) / 1e9
    flops = chunk_flops(B, T, H, dk, dv)
    mfma_tfs = flops / (kern_ms / 1000.0) / 1e12
    traffic = load_traffic(w.name)
    mfma_ctr = load_profile(f"chunk_kernel_{w.name}_mfma")

    result = {
        "metric": "GDN tokens*heads/sec at d=128 (chunked causal form) + achieved HBM GB/s and MFMA % of peak",
        "value": value,
        "unit": "token*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; inputs.py recipe)",
        "config": {"workload": w.name, "B": B, "H": H, "T": T, "d_k": dk, "d_v": dv, "chunk_len": chunk_len,
                   "form": ("chunked causal" if chunk_len == 64 else "sequential scan (profiling run)") +
                           ", fp32 state in/out", "decay": "exp(-softplus(N(2,1)))"},
        "roofline": {
            "bound": "hbm",
            "kernel": CHUNK_KERNEL,
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": (traffic["bytes_per_launch"] if traffic else None),
            "algorithmic_bytes_per_launch": abytes,
            "kernel_ms": kern_ms,
        },
        "mfma": {"achieved": mfma_tfs, "peak": BF16_MFMA_PEAK_TFS, "unit": "TFLOP/s",
                 "frac": mfma_tfs / BF16_MFMA_PEAK_TFS, "flops_per_launch": flops,
                 "basis": "analytic dense-tile flop count over the measured time",
                 # rocprofv3: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x 1024 SIMDs), per kernel
                 "measured_busy": (mfma_ctr["mfma_busy"] if mfma_ctr else None)},
        "provenance": provenance(torch, x),
    }

    if args.calib_copy:
        src = torch.empty(256 * 1024 * 1024, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = src.numel() * src.element_size()
        del src, dst

    if forms is not None:
        result["forms"] = forms
    g.close()

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(x, args.cpu_sample_tokens)
    result["input_gen_s"] = round(gen_s, 2)
    print(json.dumps(result), flush=True)


def warm_up(torch, fn, calls, min_ms=100.0):
    """Untimed calls: at least `calls` of them and at least `min_ms` of wall time.  The
    GPU clock drops while the host generates a form's inputs and needs tens of
    milliseconds of load to come back, which a fixed count of short calls may not give."""
    t0 = time.perf_counter()
    n = 0
    while n < calls or (time.perf_counter() - t0) * 1e3 < min_ms:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def timed(torch, fn, reps, warm=10):
    """Average ms of `reps` back-to-back calls after the warm-up."""
    warm_up(torch, fn, warm)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def per_call(torch, fn, reps, warm=10, flush=None):
    """Median and min ms of single calls, each bracketed by its own HIP events on the
    current stream; `flush` (if given) runs before each call, outside the events."""
    warm_up(torch, fn, warm)
    ts = []
    for _ in range(reps):
        if flush is not None:
            flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts.sort()
    return {"median_ms": ts[len(ts) // 2], "min_ms": ts[0], "runs": reps}


def measure_forms(torch, gb, inputs, d, g, x):
    forms = {}
    B, T, H, dk = d["q"].shape
    dv = d["v"].shape[-1]
    stream = gb.current_stream()
    out = torch.empty((B, T, H, dv), dtype=torch.bfloat16, device="cuda")

    # Sequential scan form on the same inputs.
    def scan():
        assert gb.gdn_forward(g.h, d["q"], d["k"], d["v"], d["beta"], d["decay"], None, None, out, T, 1,
                              stream) == 0
    ms = timed(torch, scan, 3, warm=2)
    fl = scan_flops(B, T, H, dk, dv)
    tfs = fl / (ms / 1e3) / 1e12
    scan_traffic = load_profile("scan_kernel_batched_bf16_d128_traffic", "gdn_scan.hip")
    forms["scan_batched_bf16_d128"] = {
        "ms": ms, "token_heads_per_s": B * H * T / (ms / 1e3), "bound": "alu",
        "achieved_tflops": tfs, "peak_tflops": FP32_VALU_PEAK_TFS, "frac": tfs / FP32_VALU_PEAK_TFS,
        "peak_tflops_without_packed_fp32": FP32_VALU_NOPACK_TFS, "frac_without_packed_fp32": tfs / FP32_VALU_NOPACK_TFS,
        "hbm_gbs_algorithmic": algorithmic_bytes(B, T, H, dk, dv) / (ms / 1e3) / 1e9,
        # rocprofv3 FETCH_SIZE + WRITE_SIZE of scan_kernel (scaled by a plain copy), over this time
        "hbm_gbs_measured": (scan_traffic["bytes_per_launch"] / (ms / 1e3) / 1e9 if scan_traffic else None)}

    # 5-call streaming (state carried) vs one call over the same 23400 tokens.
    w = inputs.WORKLOADS["streaming_bf16_d128"]
    xs = {k_: v_.cuda() for k_, v_ in inputs.make_workload(w).items()}
    gs = gb.GDN(w.B, w.H, w.dk, w.dv, "bf16", max_T=w.T)
    n = w.T // w.calls
    parts = [{k_: v_[:, i * n:(i + 1) * n].contiguous() for k_, v_ in xs.items()} for i in range(w.calls)]
    state = torch.zeros((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device="cuda")
    outs = [torch.empty((w.B, n, w.H, w.dv), dtype=torch.bfloat16, device="cuda") for _ in range(w.calls)]
    out1 = torch.empty((w.B, w.T, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
    per_call_ms = []
    for i in range(w.calls):
        pi = parts[i]
        per_call_ms.append(timed(torch, lambda: gb.gdn_forward(gs.h, pi["q"], pi["k"], pi["v"], pi["beta"],
                                                            pi["decay"], state, state, outs[i], n, 64, stream), 5))
    one = timed(torch, lambda: gb.gdn_forward(gs.h, xs["q"], xs["k"], xs["v"], xs["beta"], xs["decay"], None,
                                              state, out1, w.T, 64, stream), 5)
    # Cold: a 512 MiB device write before each call evicts L2 and the 256 MB MALL.
    flush_buf = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device="cuda")
    flush = lambda: flush_buf.fill_(1)
    cold = [per_call(torch, lambda: gb.gdn_forward(gs.h, parts[i]["q"], parts[i]["k"], parts[i]["v"],
                                                   parts[i]["beta"], parts[i]["decay"], state, state, outs[i], n,
                                                   64, stream), 10, warm=2, flush=flush)["median_ms"]
            for i in range(w.calls)]
    forms["streaming_bf16_d128"] = {"per_call_ms": per_call_ms, "sum_ms": sum(per_call_ms), "one_shot_ms": one,
                                    "cold_per_call_median_ms": cold, "cold_sum_ms": sum(cold),
                                    "token_heads_per_s": w.B * w.H * w.T / (sum(per_call_ms) / 1e3)}
    gs.close()
    # The same calls on a GDN_FLAG_SEGMENTS handle (token segments run concurrently).
    gss = gb.GDN(w.B, w.H, w.dk, w.dv, "bf16", max_T=n, segments=True)
    state.zero_()
    seg_ms = [timed(torch, lambda: gb.gdn_forward(gss.h, parts[i]["q"], parts[i]["k"], parts[i]["v"],
                                                  parts[i]["beta"], parts[i]["decay"], state, state, outs[i], n,
                                                  64, stream), 5) for i in range(w.calls)]
    seg_cold = [per_call(torch, lambda: gb.gdn_forward(gss.h, parts[i]["q"], parts[i]["k"], parts[i]["v"],
                                                       parts[i]["beta"], parts[i]["decay"], state, state, outs[i],
                                                       n, 64, stream), 10, warm=2, flush=flush)["median_ms"]
                for i in range(w.calls)]
    forms["streaming_bf16_d128"]["segmented"] = {"per_call_ms": seg_ms, "sum_ms": sum(seg_ms),
                                                 "cold_per_call_median_ms": seg_cold, "cold_sum_ms": sum(seg_cold)}
    gss.close()
    del xs, parts

    # 3 frames at d = 64 (B=1, H=16, T=4680), warm and cold.
    w1 = inputs.WORKLOADS["causal_bf16_d64"]
    x1 = {k_: v_.cuda() for k_, v_ in inputs.make_workload(w1).items()}
    g1 = gb.GDN(w1.B, w1.H, w1.dk, w1.dv, "bf16", max_T=w1.T)
    o1 = torch.empty((w1.B, w1.T, w1.H, w1.dv), dtype=torch.bfloat16, device="cuda")
    f1 = lambda: gb.gdn_forward(g1.h, x1["q"], x1["k"], x1["v"], x1["beta"], x1["decay"], None, None, o1, w1.T,
                                64, stream)
    warm1 = per_call(torch, f1, 20)
    cold1 = per_call(torch, f1, 10, warm=2, flush=flush)
    th1 = w1.B * w1.H * w1.T
    forms["causal_bf16_d64"] = {"warm": warm1, "cold": cold1,
                                "token_heads_per_s_warm": th1 / (warm1["median_ms"] / 1e3),
                                "token_heads_per_s_cold": th1 / (cold1["median_ms"] / 1e3)}
    g1.close()
    g1s = gb.GDN(w1.B, w1.H, w1.dk, w1.dv, "bf16", max_T=w1.T, segments=True)
    f1s = lambda: gb.gdn_forward(g1s.h, x1["q"], x1["k"], x1["v"], x1["beta"], x1["decay"], None, None, o1, w1.T,
                                 64, stream)
    warm1s = per_call(torch, f1s, 20)
    cold1s = per_call(torch, f1s, 10, warm=2, flush=flush)
    forms["causal_bf16_d64"]["segmented"] = {"warm": warm1s, "cold": cold1s,
                                             "token_heads_per_s_warm": th1 / (warm1s["median_ms"] / 1e3)}
    g1s.close()
    del x1, o1, flush_buf

    # Bidirectional form, 21 frames.
    wb = inputs.WORKLOADS["bidi_bf16_d128"]
    xb = {k_: v_.cuda() for k_, v_ in inputs.make_workload(wb).items()}
    gbd = gb.GDN(wb.B, wb.H, wb.dk, wb.dv, "bf16", max_T=wb.T, bidi=True)
    ob = torch.empty((wb.B, wb.T, wb.H, wb.dv), dtype=torch.bfloat16, device="cuda")
    ms = timed(torch, lambda: gb.gdn_forward_bidi(gbd.h, xb["q"], xb["k"], xb["v"], xb["beta"], xb["decay"],
                                                  ob, wb.T, 64, stream), 5)
    forms["bidi_bf16_d128"] = {"ms": ms, "token_heads_per_s": wb.B * wb.H * wb.T / (ms / 1e3),
                               "design": "both directions concurrently; each sweep's first half in two launches and its second half in one, all but the first quarter's inverses formed on a side stream beside them; the first half's outputs kept as bf16 rows, which the second half's launch adds before writing out once"}
    gbd.close()
    del xb, ob

    # Fused input prologue on the bench shape: q, k, v read in place from a packed
    # [B, T, 2 H d_k + H d_v] bf16 projection, gate logits, normalisation and
    # activations inside the kernels.
    a_mean = inputs.WORKLOADS["batched_bf16_d128"].a_mean
    xp = inputs.make_packed_inputs(B, T, H, dk, dv, "bf16", seed=0, a_mean=a_mean)
    qkv = xp["qkv_buf"].cuda()
    bl, dl = xp["beta_logit"].cuda(), xp["decay_logit"].cuda()
    del xp
    gp = gb.GDN(B, H, dk, dv, "bf16", max_T=T)
    ts, bs = qkv.stride(1), qkv.stride(0)
    ms = timed(torch, lambda: gb.gdn_forward_packed(gp.h, qkv, ts, bs, bl, dl, None, None, out, T, 64, stream), 20)
    forms["packed_prologue_batched_bf16_d128"] = {
        "ms": ms, "token_heads_per_s": B * H * T / (ms / 1e3),
        "design": "strided reads of the packed rows; inverse k norms formed in the inverse pass and folded "
                  "into the per-token decay factors, inverse q norms in the output waves from the Q operands they "
                  "hold (v_dot2, two lane swaps, v_rsq); sigmoid / exp(-softplus) of the logits in the inverse pass"}
    gp.close()
    del qkv, bl, dl

    # FP8 (E4M3) q, k, v on the bench shape, out in bf16.
    x8 = {k_: v_.cuda() for k_, v_ in inputs.make_inputs(B, T, H, dk, dv, "fp8", seed=0, a_mean=a_mean).items()}
    g8 = gb.GDN(B, H, dk, dv, "fp8", max_T=T)
    ms = timed(torch, lambda: gb.gdn_forward(g8.h, x8["q"], x8["k"], x8["v"], x8["beta"], x8["decay"], None, None,
                                             out, T, 64, stream), 20)
    ab8 = algorithmic_bytes(B, T, H, dk, dv, es=1, es_out=2)
    forms["fp8_batched_d128"] = {
        "ms": ms, "token_heads_per_s": B * H * T / (ms / 1e3), "algorithmic_bytes": ab8,
        "hbm_gbs": ab8 / (ms / 1e3) / 1e9,
        "design": "E4M3 rows widened exactly to bf16 by the loaders (v_cvt_scalef32_pk_bf16_fp8); bf16 MFMA"}
    g8.close()
    return forms


def cpu_baseline(x, tokens):
    import oracle
    Ts = x["q"].shape[1] if tokens <= 0 else min(tokens, x["q"].shape[1])
    sample = {k_: v_[:, :Ts].contiguous() for k_, v_ in x.items()}
    B, _, H, _ = sample["q"].shape
    t0 = time.perf_counter()
    oracle.forward(**sample)
    dt = time.perf_counter() - t0
    th = B * H * Ts
    return {"value": th / dt, "unit": "token*heads/s", "cores": oracle.num_threads(), "kind": "oracle",
            "seconds": dt,
            "sample": f"float64 sequential oracle on the first {Ts} tokens of every head of the same "
                      f"inputs (B={B}, H={H}): {th} token*heads, including the bf16->f64 widening"}


if __name__ == "__main__":
    main()
