"""Benchmark of the chunkwise Kronecker delta rule forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload train_step]

A step is one kron_delta_fwd call over the whole workload (all B*H heads,
all T tokens): decay products, Gram tiles, forward substitution, readout and
state propagation all run inside that one kernel.  Inputs are seeded
synthetic draws (see delta_rule_recurrent_chunk_amd/synthetic.py) that are
resident in HBM before the timed region starts.  Prints one JSON line.

The roofline entry prices the kernel's algorithmic HBM bytes per launch
(q, k, v, f, beta, c read once, o and S_T written once) against the MI355X
HBM3E peak of 8 TB/s, using the average launch duration measured with HIP
events on the stream the kernel runs on.  The cpu_baseline entry times the
fp64 oracle on the host cores on a bounded sample of the same inputs.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "Kron-delta chunked fwd tokens/s (H=16,d=128) and % MFMA/HBM roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kd_fwd16_train_step_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "delta_rule_recurrent_chunk_amd", "csrc", n)
                  for n in ("kd_fwd.hip", "kd_fwd16.hip", "kd_device.h")]
COPY_ELEMS = 1 << 28     # calibration copy: 2^28 fp32 = 1 GiB read and 1 GiB written


def kernel_source_hash():
    """sha256 over the forward kernel's sources, to tell whether stored counter
    figures still describe the kernel that runs."""
    import hashlib
    hsh = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as fh:
            hsh.update(fh.read())
    return hsh.hexdigest()[:16]


def stored_traffic():
    """HBM bytes per launch from the committed counter summary, or None when the
    summary is missing or was taken on other kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                key, _, val = line.partition(":")
                vals[key.strip()] = val.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_bytes(w, esize, with_S0=False):
    """HBM bytes one forward launch must move: every input once, every output once."""
    ntok = w.B * w.T * w.H
    b = 4 * ntok * w.dk * esize          # q, k, v, f
    b += 2 * ntok * 4                    # beta, c (fp32)
    b += ntok * w.dv * esize             # o
    b += w.B * w.H * w.dv * w.dk * 4     # S_T (fp32)
    if with_S0:
        b += w.B * w.H * w.dv * w.dk * 4
    return b


def algorithmic_bytes_fwd_bwd(w, esize):
    """HBM bytes of one forward + backward step: the forward's inputs and o; the
    backward's inputs (q, k, v, f, beta, c, dO) and outputs (dq, dk, dv, df,
    dbeta, dc, dS0).  Checkpoints are the implementation's, not counted."""
    ntok = w.B * w.T * w.H
    fwd = algorithmic_bytes(w, esize) - w.B * w.H * w.dv * w.dk * 4   # no S_T in this step
    bwd = 5 * ntok * w.dk * esize + 2 * ntok * 4 + 4 * ntok * w.dk * esize + 2 * ntok * 4
    bwd += w.B * w.H * w.dv * w.dk * 4
    return fwd + bwd


def algorithmic_bytes_decode(w, esize):
    """HBM bytes of one decode call: the carried fp32 state read and written
    once, every token input once, o once."""
    ntok = w.B * w.T * w.H
    return 2 * w.B * w.H * w.dv * w.dk * 4 + 4 * ntok * w.dk * esize + 2 * ntok * 4 + ntok * w.dv * esize


def algorithmic_bytes_gdn2(w, esize):
    """HBM bytes of one Gated Delta Rule-2 forward launch: q, k, alpha, b (dk)
    and v, w (dv) once, o once, S_T (fp32) once."""
    ntok = w.B * w.T * w.H
    return ntok * (4 * w.dk + 2 * w.dv) * esize + ntok * w.dv * esize + w.B * w.H * w.dk * w.dv * 4


def algorithmic_bytes_mixer(w, esize):
    """HBM bytes of one mixer forward from the projections: q, k, f
    projections (dk) and v projection, output-gate logits g (dv) once, the
    beta and c logits (fp32) once, y once, S_T (fp32) once; the per-head
    parameters (conv taps, a_log, norm weights) are under 0.1% and not
    counted.  The rule's inputs and read-out between the steps are the
    implementation's, not counted."""
    ntok = w.B * w.T * w.H
    return (ntok * (3 * w.dk + 2 * w.dv) * esize + 2 * ntok * 4 + ntok * w.dv * esize
            + w.B * w.H * w.dv * w.dk * 4)


def mfma_flops_gdn2(w):
    """MFMA flops of one Gated Delta Rule-2 launch as issued, per (b, h, chunk)
    of C = 64 at d = 128: Grams 2 x 10 tiles x 2*16*16*d; Ebar S0 and Qbar S0
    2 x 2*C*d*d; the blocked solve 10 block products x 3 (hi/lo) x 2*16*16*d;
    readout 2*C*C*d; update 3 (hi/lo) x 2*C*d*d."""
    C = 64
    d = w.dk
    nch = (w.T + C - 1) // C
    per = (2 * 10 * 2 * 16 * 16 * d + 2 * 2 * C * d * d + 10 * 3 * 2 * 16 * 16 * d
           + 2 * C * C * d + 3 * 2 * C * d * d)
    return w.B * w.H * nch * per


def mfma_flops(w):
    """MFMA flops of one launch as issued (full 16x16 tiles, including the
    masked-out upper Gram tiles' partners): per (b, h, chunk) of C = 64 with
    d = dk = dv: Grams 3 x 10 tiles x 2*16*16*d, state reads 2 x 2*C*d*d,
    intra readout 2*C*C*d, state update 2*C*d*d."""
    C = 64
    d = w.dk
    nch = (w.T + C - 1) // C
    per = 3 * 10 * 2 * 16 * 16 * d + 2 * 2 * C * d * d + 2 * C * C * d + 2 * C * d * d
    return w.B * w.H * nch * per


def cpu_model():
    """The host CPU's model name and logical CPU count, from /proc/cpuinfo."""
    name, n = "unknown", 0
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    name = line.partition(":")[2].strip()
                    n += 1
    except OSError:
        pass
    return {"model": name, "logical_cpus": n, "affinity": len(os.sched_getaffinity(0))}


def cpu_baseline(x_np, w, budget_s=10.0, max_passes=64, one_core_s=5.0):
    """The fp64 oracle, unmodified, on the host cores: whole sequences of the
    same seeded workload, repeated in passes until about budget_s of wall time
    has been spent (the last pass may stop early); then the same on one thread
    for about one_core_s."""
    import oracle
    res = _cpu_leg(x_np, w, budget_s, max_passes)
    threads = oracle.num_threads()
    try:
        oracle.set_num_threads(1)
        one = _cpu_leg(x_np, w, one_core_s, max_passes)
    finally:
        oracle.set_num_threads(threads)
    res["one_core"] = {"value": one["value"], "unit": "tokens/s", "cores": one["cores"], "sample": one["sample"]}
    res["cpu"] = cpu_model()
    return res


def _cpu_leg(x_np, w, budget_s, max_passes):
    import oracle
    threads = oracle.num_threads()
    done_tok = 0
    t0 = time.perf_counter()
    nseq = 0
    for _ in range(max_passes):
        for b in range(w.B):
            sl = slice(b, b + 1)
            if w.mixer:
                from oracle import mixer as mx
                q, k, v, f, beta, c = mx.mixer_pre(x_np["q_raw"][sl], x_np["k_raw"][sl], x_np["v_raw"][sl],
                                                   x_np["f_raw"][sl], x_np["beta_raw"][sl], x_np["c_raw"][sl],
                                                   x_np["conv_q"], x_np["conv_k"], x_np["conv_v"],
                                                   x_np["a_log"])
                o, _, _ = oracle.fwd(q, k, v, f, beta, c, None)
                mx.rms_norm_gate(o, x_np["g"][sl], x_np["norm_w"], 1e-5)
                nseq += 1
                done_tok += w.T
                if time.perf_counter() - t0 > budget_s:
                    break
                continue
            if w.gdn2:
                oracle.gdn2_fwd(x_np["q"][sl], x_np["k"][sl], x_np["v"][sl], x_np["alpha"][sl],
                                x_np["b"][sl], x_np["w"][sl], None)
                nseq += 1
                done_tok += w.T
                if time.perf_counter() - t0 > budget_s:
                    break
                continue
            oracle.fwd(x_np["q"][sl], x_np["k"][sl], x_np["v"][sl], x_np["f"][sl],
                       x_np["beta"][sl], x_np["c"][sl],
                       x_np["S0"][sl] if x_np.get("S0") is not None else None)
            if w.backward:
                oracle.bwd(x_np["q"][sl], x_np["k"][sl], x_np["v"][sl], x_np["f"][sl],
                           x_np["beta"][sl], x_np["c"][sl], None, x_np["dO"][sl])
            nseq += 1
            done_tok += w.T
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done_tok / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": "fp64 oracle %s on %d sequences (passes over the %d sequences of the "
                      "workload; T=%d, H=%d, d=%d), same seeded inputs, %.1f s wall"
                      % ("mixer forward (pre-processing, rule, gated RMSNorm)" if w.mixer else
                         "Gated Delta Rule-2 forward" if w.gdn2 else
                         "forward + backward" if w.backward else "forward", nseq, w.B, w.T, w.H,
                         w.dk, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="train_step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the launches timed after evicting the caches with a 1 GiB write")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain elementwise copy kernel (1 GiB read, 1 GiB written; "
                         "the reference for the HBM byte counters) three times and exit")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        src = torch.empty(COPY_ELEMS, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)   # one elementwise kernel per call
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": COPY_ELEMS * 4,
                          "copy_bytes_written_per_launch": COPY_ELEMS * 4}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the Kronecker delta rule path here runs on a "
              "single MI355X (heads would shard across GPUs with no exchange); use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import delta_rule_recurrent_chunk_amd as kd
    from delta_rule_recurrent_chunk_amd import synthetic as sy

    w = sy.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    x = sy.rounded(sy.draw_workload(w), w.dtype)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    per_token = ("q", "k", "v", "f", "alpha", "b", "w", "q_raw", "k_raw", "v_raw", "f_raw", "g")
    names = (("q_raw", "k_raw", "v_raw", "f_raw", "beta_raw", "c_raw", "g", "conv_q", "conv_k", "conv_v",
              "a_log", "norm_w") if w.mixer else
             ("q", "k", "v", "alpha", "b", "w") if w.gdn2 else ("q", "k", "v", "f", "beta", "c"))
    t = {n: torch.tensor(x[n], dtype=tdt if n in per_token else torch.float32, device=dev) for n in names}
    esize = 2 if w.dtype == "bf16" else 4
    # the forward takes the few-heads form (preparation workers beside the
    # per-head passes) when the library asks for a workspace for it
    few_heads = (not (w.mixer or w.gdn2 or w.decode or w.backward) and
                 kd.workspace_bytes(w.B, w.T, w.H, w.dk, 1 if w.dtype == "bf16" else 0, with_backward=False) > 0)

    if w.mixer:      # a step is one mixer forward from the projections
        desc = kd.KdDesc(w.B, w.T, w.H, w.dk, w.dv, 1 if w.dtype == "bf16" else 0)
        import ctypes
        mws = torch.empty(max(int(kd.lib().kron_delta_workspace_bytes(ctypes.byref(desc), kd.KD_WS_MIXER)), 16),
                          dtype=torch.uint8, device=dev)

        def step():
            return kd.mixer_fwd(t["q_raw"], t["k_raw"], t["v_raw"], t["f_raw"], t["beta_raw"], t["c_raw"], t["g"],
                                t["conv_q"], t["conv_k"], t["conv_v"], t["a_log"], t["norm_w"], None,
                                norm_eps=1e-5, workspace=mws)
    elif w.gdn2:     # a step is one Gated Delta Rule-2 forward
        def step():
            return kd.gdn2_fwd(t["q"], t["k"], t["v"], t["alpha"], t["b"], t["w"], None)
    elif w.decode:   # a step is one decode call, the state updated in place
        t["S"] = torch.tensor(x["S0"], dtype=torch.float32, device=dev)

        def step():
            return kd.decode(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], t["S"])
    elif w.backward:   # a step is the forward plus the gate-aware backward
        t["dO"] = torch.tensor(x["dO"], dtype=tdt, device=dev)
        ws = torch.empty(max(kd.workspace_bytes(w.B, w.T, w.H, w.dk, 1 if w.dtype == "bf16" else 0,
                                                 with_backward=True), 16),
                         dtype=torch.uint8, device=dev)

        def step():   # training forward (o plus the backward's records), then the backward
            kd.fwd_train(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], None, workspace=ws)
            return kd.bwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], None, t["dO"],
                          workspace=ws, saved=True)
    else:
        def step():
            return kd.fwd(t["q"], t["k"], t["v"], t["f"], t["beta"], t["c"], None)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)   # the stream the binding launches on
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):   # back to back; one event between consecutive steps
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    kernel_ms = evs[0].elapsed_time(evs[-1]) / args.steps     # avg launch duration (events)
    ms_per_step = wall * 1e3 / args.steps

    tokens = w.B * w.T
    value = tokens / (ms_per_step * 1e-3)
    abytes = (algorithmic_bytes_mixer(w, esize) if w.mixer else
              algorithmic_bytes_gdn2(w, esize) if w.gdn2 else
              algorithmic_bytes_decode(w, esize) if w.decode else
              algorithmic_bytes_fwd_bwd(w, esize) if w.backward else algorithmic_bytes(w, esize))
    achieved = abytes / (kernel_ms * 1e-3) / 1e9
    flops = mfma_flops_gdn2(w) if w.gdn2 else mfma_flops(w)
    peak_tf = BF16_MFMA_PEAK_TFLOPS if w.dtype == "bf16" else 157.3
    traffic = stored_traffic() if args.workload == "train_step" else None

    out = {
        "metric": ("KronLSTM mixer fwd (pre + rule + gated RMSNorm) tokens/s (H=16,d=128) and % HBM roofline"
                   if w.mixer else
                   "Gated Delta Rule-2 chunked fwd tokens/s (H=16,d=128) and % HBM roofline"
                   if w.gdn2 else
                   "Kron-delta decode tokens/s (H=16,d=128) and % HBM roofline" if w.decode else
                   "Kron-delta chunked fwd+bwd tokens/s (H=16,d=128) and % HBM roofline"
                   if w.backward else METRIC),
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": ("synthetic (seeded: N(0,1) q/k/v projections, beta/c/output-gate logits; f logits "
                 "N(%g,1), a_log U(-1,1); conv taps N(0,1/%d); norm weights 1+0.1N(0,1))"
                 % (w.mu, sy.MIXER_CONV_SIZE)) if w.mixer else
                ("synthetic (seeded: L2-normalised N(0,1) q,k,v; alpha=exp(-exp(U(-1,1)) "
                 "softplus(-N(%g,1))); b,w=sigmoid(N(0,1)) per channel)" % w.mu) if w.gdn2 else
                "synthetic (seeded: L2-normalised N(0,1) q,k,v; f=sigmoid(N(%g,1))^exp(U(-1,1)); "
                "beta,c=sigmoid(N(0,1)))" % w.mu,
        "config": {"workload": ("%s: KronLSTM mixer forward from the projections (causal depthwise "
                                "conv K=%d, SiLU, L2 norm, gates; the Kronecker delta rule, chunk 64; "
                                "gated per-head RMSNorm), B=%d T=%d H=%d dk=dv=%d, %s projections, "
                                "fp32 gate logits and state, S0=0"
                                % (w.name, sy.MIXER_CONV_SIZE, w.B, w.T, w.H, w.dk, w.dtype))
                               if w.mixer else
                               ("%s: Gated Delta Rule-2 (decoupled erase and write) chunked "
                                "forward, B=%d T=%d H=%d dk=dv=%d, chunk 64, %s q/k/v/alpha/b/w, "
                                "fp32 state, S0=0" % (w.name, w.B, w.T, w.H, w.dk, w.dtype))
                               if w.gdn2 else
                               ("%s: Kronecker delta rule decode (token by token on the carried "
                                "state, updated in place), B=%d T=%d H=%d dk=dv=%d, %s q/k/v/f, "
                                "fp32 beta/c/state, S ~ N(0, 0.1^2)"
                                % (w.name, w.B, w.T, w.H, w.dk, w.dtype)) if w.decode else
                               ("%s: Kronecker delta rule chunked %s, B=%d T=%d H=%d "
                                "dk=dv=%d, chunk 64, %s q/k/v/f, fp32 beta/c/state, S0=0"
                                % (w.name, "forward + gate-aware backward" if w.backward else "forward",
                                   w.B, w.T, w.H, w.dk, w.dtype)),
                   "B": w.B, "T": w.T, "H": w.H, "d": w.dk, "tokens_per_step": tokens},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "kd_mixer_conv_kernel + kd_fwd16_kernel<false, true>"
                     if w.mixer else
                     "kd_gdn2_kernel" if w.gdn2 else
                     "kd_decode_kernel<bf16,128>" if w.decode else
                     "kd_fwd16_kernel(ckpt) + kd_bwd_clear_kernel + kd_bwd_fused_kernel" if w.backward else
                     "kd_fwd16_split_clear_kernel + kd_fwd16_split_fused_kernel" if few_heads else
                     "kd_fwd16_kernel<false, false>",
                     "kernel_ms": kernel_ms,
                     "launch_ms": {"mean": kernel_ms, "median": float(np.median(per_launch)),
                                   "p10": float(np.percentile(per_launch, 10)),
                                   "p90": float(np.percentile(per_launch, 90))},
                     "algorithmic_bytes_per_launch": abytes,
                     },
    }
    if w.mixer:   # the three steps timed on their own (events, 10 launches each)
        q, k, v, f, beta, c = kd.mixer_pre(t["q_raw"], t["k_raw"], t["v_raw"], t["f_raw"], t["beta_raw"],
                                           t["c_raw"], t["conv_q"], t["conv_k"], t["conv_v"], t["a_log"])
        o, _ = kd.fwd(q, k, v, f, beta, c, None)
        parts = {"pre": lambda: kd.mixer_pre(t["q_raw"], t["k_raw"], t["v_raw"], t["f_raw"], t["beta_raw"],
                                             t["c_raw"], t["conv_q"], t["conv_k"], t["conv_v"], t["a_log"]),
                 "rule": lambda: kd.fwd(q, k, v, f, beta, c, None),
                 "post": lambda: kd.mixer_post(o, t["g"], t["norm_w"], norm_eps=1e-5)}
        part_bytes = {"pre": w.B * w.T * w.H * (4 * w.dk * esize * 2 + 4 * 4),
                      "rule": algorithmic_bytes(w, esize),
                      "post": w.B * w.T * w.H * w.dv * esize * 3}
        out["steps"] = {}
        for name, fn in parts.items():
            fn()
            torch.cuda.synchronize()
            a_ = torch.cuda.Event(enable_timing=True)
            b_ = torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            for _ in range(10):
                fn()
            b_.record(stream)
            torch.cuda.synchronize()
            ms = a_.elapsed_time(b_) / 10
            out["steps"][name] = {"ms": ms, "hbm_frac": part_bytes[name] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if not w.backward and not w.decode and not w.mixer:
        out["roofline"]["mfma_tflops"] = flops / (kernel_ms * 1e-3) / 1e12
        out["roofline"]["mfma_frac"] = flops / (kernel_ms * 1e-3) / 1e12 / peak_tf
    if not args.no_cold:
        big = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        times = []
        for i in range(min(args.steps, 10)):
            big.fill_(i & 255)
            a = torch.cuda.Event(enable_timing=True)
            b_ = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b_.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b_))
        cold_ms = float(np.median(times))
        out["cold_cache"] = {"kernel_ms": cold_ms, "tokens_per_s": tokens / (cold_ms * 1e-3),
                             "hbm_frac": abytes / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                             "how": "median of %d launches, each after a 1 GiB fill that evicts "
                                    "the L2 and the last-level cache" % len(times)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
