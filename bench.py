#!/usr/bin/env python3
"""Benchmark libkda on one MI355X and print one JSON line.

One timed step is one kda_chunk_fwd call over the 64K-token prefill workload
(B=2, H=32, T=65536, d_k=d_v=128, bf16 q/k/v, fp32 alpha/beta/state, bf16 o:
1,540 algorithmic bytes per token-head), with inputs resident in HBM.  The same
run times the other workloads and calls and reports each under its own key:
the same prefill with an fp32 o, the 4K-token and 1M-token prefills, state
snapshots, the fused gate, a packed batch, the split prefill, batched decode
and speculative decode.

The GPU legs keep host copies of sampled heads' inputs and outputs; the last
leg, the CPU baseline, runs the fp64 oracle on all of them.  Its time on the
64K prefill sample, on this host's cores, is `cpu_baseline` (a one-thread rate
is reported beside it); its comparisons are the parity fields
(max|GPU - oracle| / RMS(oracle) per head, worst head).

Kernel times are the median of per-launch HIP events recorded on the stream the
kernels run on; `ms_per_step` is the wall time of the K timed steps / K.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs a,b,...]
                       [--no-cpu-baseline] [--copy-probe]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "KDA prefill tokens/s @T=64K,H=32,d=128 (%MFMA peak); decode state GB/s (%HBM)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 (fp16 is the same rate)
TOL_REL = 2e-2
RUN_CHUNK = 32                 # tokens per chunk the bf16 d_k=128 prefill kernel runs
LEGS = ("prefill", "prefill4k", "prefill1m", "snapshots", "gated", "varlen", "split", "decode", "spec")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def prefill_bytes(B, T, H, dk, dv, o_bytes, a_bytes=4):
    """Algorithmic bytes of one prefill call: per token-head the bf16 q/k/v reads,
    the alpha (a_bytes per channel) and beta reads and the o write; per chain one
    S0 read and one S_T write.  Returns (total, per token-head)."""
    per_th = 2 * (2 * dk + dv) + a_bytes * dk + 4 + o_bytes * dv
    return B * T * H * per_th + 2 * 4 * dk * dv * B * H, per_th


def prefill_flops_per_th(dk, dv, chunk):
    """FLOPs per token-head of the chunk form at chunk size `chunk`: the state
    products 6 d_k d_v, the triangular intra-chunk products C (3 d_k + 2 d_v) and
    the triangular solve C^2 / 3."""
    return 6 * dk * dv + chunk * (3 * dk + 2 * dv) + chunk * chunk / 3.0


def source_hash():
    h = hashlib.sha256()
    for f in sorted((ROOT / "gated_delta_rule_07_amd" / "csrc").glob("*")):
        h.update(f.read_bytes())
    return h.hexdigest()[:16]


def _profile_entry(fname, key):
    """An entry of a committed counter summary, if it was taken on the current
    kernel sources; else None."""
    f = ROOT / "profiles" / fname
    if not f.exists():
        return None
    try:
        d = json.loads(f.read_text())
    except ValueError:
        return None
    ent = d.get(key)
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent


def measured_traffic(key):
    ent = _profile_entry("traffic.json", key)
    return None if ent is None else ent.get("bytes_per_launch")


def event_ms(fn, n, torch):
    """Launch fn() n times on the current stream.  Returns (wall ms of all n,
    per-launch durations in ms from HIP events recorded around each launch on
    that stream)."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    return wall_ms, [s.elapsed_time(e) for s, e in zip(starts, ends)]


def med(xs):
    return float(statistics.median(xs))


def back_to_back_ms(fn, n, torch, groups=5, warm=5):
    """Median over `groups` groups of n launches of fn() back to back (after
    `warm` untimed groups, which carry the first milliseconds of a new load,
    while the clocks settle) of the mean ms per launch; each group sits between
    one pair of HIP events on the current stream (no markers between launches,
    so short kernels are not charged for them)."""
    for _ in range(warm * n):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(groups):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / n)
    return sorted(ts)[len(ts) // 2]


def rel_err_heads(got, ref):
    """Worst head's max|got - ref| / RMS(ref); inf when anything is not finite."""
    import numpy as np
    worst = 0.0
    for g, r in zip(got, ref):
        if not (np.isfinite(g).all() and np.isfinite(r).all()):
            return float("inf")
        rms = float(np.sqrt(np.mean(r * r)))
        worst = max(worst, float(np.abs(g - r).max()) / max(rms, 1e-30))
    return worst


class OracleChecks:
    """Host copies of sampled heads' inputs and the GPU's outputs for them, filled
    in by the GPU legs and compared in the CPU-baseline leg (the only leg that
    runs the oracle)."""

    def __init__(self):
        self.items = {}

    def add(self, name, inputs, got_o, got_s, heads=None, gate=None, timed=False, extra_o=None):
        """inputs: host q, k, v, alpha (or None with gate=(z, A)), beta, S0 as [B,T,H,.];
        got_o [n, T, d_v] (None: not compared), got_s [n, d_k, d_v], both for `heads`
        (ids b*H + h; None: all, in (b, h) order).  extra_o: {label: [n, T, d_v]}
        further outputs of the same heads compared against the same reference."""
        self.items[name] = dict(inputs=inputs, got_o=got_o, got_s=got_s, heads=heads, gate=gate,
                                timed=timed, extra_o=extra_o or {})


def cpu_baseline_leg(checks, threads, log):
    """Runs the oracle on every check: returns {name: (err_o, err_s)}, the errors
    of the extra outputs {name/label: err}, and the wall time of the timed check
    (the 64K prefill sample), which is the CPU baseline."""
    import oracle
    errs, extra, timed_s = {}, {}, None
    for name, c in checks.items.items():
        h = c["inputs"]
        alpha = h["alpha"] if c["gate"] is None else oracle.gate_alpha(*c["gate"])
        t0 = time.perf_counter()
        ro, rs = oracle.forward(h["q"], h["k"], h["v"], alpha, h["beta"], h["S0"], heads=c["heads"],
                                threads=threads, want_o=c["got_o"] is not None)
        if c["timed"]:
            timed_s = time.perf_counter() - t0
        eo = None
        if c["got_o"] is not None:
            eo = max(rel_err_heads(g[None].astype("float64"), r[None]) for g, r in zip(c["got_o"], ro))
            for label, go in c["extra_o"].items():
                extra[f"{name}/{label}"] = max(rel_err_heads(g[None].astype("float64"), r[None])
                                               for g, r in zip(go, ro))
        es = rel_err_heads(c["got_s"].astype("float64"), rs)
        errs[name] = (eo, es)
        log(f"parity {name}: o {eo if eo is None else f'{eo:.3e}'}  S {es:.3e}")
    for k, v in extra.items():
        log(f"parity {k}: o {v:.3e}")
    return errs, extra, timed_s


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--legs", default="all", help="comma-separated subset of " + ",".join(LEGS))
    ap.add_argument("--sample-heads", type=int, default=64, help="64K heads checked by the oracle (all 64)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="do not run the oracle (no parity, no baseline)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build measures one GPU only (asked for {max(args.gpus, world)}); "
              "every (sequence, head) chain is independent, so a multi-GPU run shards batch and heads, "
              "one process per GPU",
              file=sys.stderr)
        sys.exit(2)
    legs = set(LEGS) if args.legs == "all" else set(args.legs.split(","))
    unknown = legs - set(LEGS)
    if unknown:
        ap.error(f"unknown legs {sorted(unknown)}")

    import numpy as np
    import torch

    import gated_delta_rule_07_amd as kda
    import kda_inputs as ki

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kda.load_library()
    props = torch.cuda.get_device_properties(dev)
    checks = OracleChecks()
    bf16, f32 = torch.bfloat16, torch.float32

    def heads_of(t, heads):
        """[B,T,H,d] device tensor -> float32 numpy [n, T, d] for head ids b*H + h
        (gathers only the selected heads on the device)."""
        Bt, Tt, Ht, dt = t.shape
        rows = []
        for hid in heads:
            b_, h_ = divmod(int(hid), Ht)
            rows.append(t[b_, :, h_].float().cpu())
        return torch.stack(rows, 0).numpy()

    def states_of(t, heads):
        return t.reshape(-1, t.shape[-2], t.shape[-1])[heads].float().cpu().numpy()

    def host_heads(xin, heads):
        """Host copies of the selected heads' inputs as a [1, T, n, .] batch (for the oracle)."""
        out = {}
        H_ = xin["q"].shape[2]
        for n_ in ("q", "k", "v", "alpha", "beta"):
            t = xin[n_]
            out[n_] = torch.stack([t[hid // H_, :, hid % H_] for hid in heads], 1)[None].cpu()
        out["S0"] = None if xin["S0"] is None else torch.stack(
            [xin["S0"][hid // H_, hid % H_] for hid in heads], 0)[None].cpu()
        return out

    res = {}
    w = ki.WORKLOADS[2]
    B, T, H, dk, dv, C = w.B, w.T, w.H, w.dk, w.dv, w.chunk
    fl_canon = prefill_flops_per_th(dk, dv, C)         # the metric's count (chunk 64)
    fl_run = prefill_flops_per_th(dk, dv, RUN_CHUNK)   # the work of the chunk size the kernel runs

    def roofline(alg_bytes, per_th_bytes, kern_ms, ntok_heads, traffic_key=None, mfma_key=None):
        gbs = alg_bytes / (kern_ms / 1e3) / 1e9
        tf_canon = ntok_heads * fl_canon / (kern_ms / 1e3) / 1e12
        tf_run = ntok_heads * fl_run / (kern_ms / 1e3) / 1e12
        attainable = min(MFMA_BF16_PEAK_TFS, fl_canon / per_th_bytes * HBM_PEAK_GBS / 1e3)
        r = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
             "traffic": measured_traffic(traffic_key) if traffic_key else None,
             "kernel_ms": kern_ms, "algorithmic_bytes": alg_bytes, "bytes_per_token_head": per_th_bytes,
             "mfma_canonical_c64": {"flops_per_token_head": fl_canon, "tflops": tf_canon,
                                    "frac_of_peak": tf_canon / MFMA_BF16_PEAK_TFS,
                                    "attainable_tflops": attainable, "frac_of_attainable": tf_canon / attainable},
             "mfma_at_run_chunk": {"chunk": RUN_CHUNK, "flops_per_token_head": fl_run, "tflops": tf_run,
                                   "frac_of_peak": tf_run / MFMA_BF16_PEAK_TFS}}
        if mfma_key:
            ent = _profile_entry("mfma.json", mfma_key)
            if ent:
                issued = ent["flops_per_launch"] / (kern_ms / 1e3) / 1e12
                r["mfma_issued"] = {"tflops": issued, "frac_of_peak": issued / MFMA_BF16_PEAK_TFS,
                                    "mfma_busy_frac": ent.get("mfma_busy_frac"),
                                    "note": "rocprofv3 counters: all issued matrix-core work, masked "
                                            "halves and per-slab repeats included"}
        return r

    # ---------------- prefill: 64K tokens, B=2, H=32, d=128 ----------------
    if legs & {"prefill", "snapshots", "gated"}:
        log(f"generating prefill inputs B={B} T={T} H={H} d={dk}")
        x = ki.make_workload_prefill(2, seed=0, device=dev)
        o16 = torch.empty(B, T, H, dv, device=dev, dtype=bf16)
        o32 = torch.empty(B, T, H, dv, device=dev, dtype=f32)
        S_T = torch.empty(B, H, dk, dv, device=dev, dtype=f32)
        nh = min(args.sample_heads, B * H)
        heads = sorted(set(int(v) for v in np.linspace(0, B * H - 1, nh)))

    if "prefill" in legs:
        def step():
            kda.kda_chunk_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], chunk=C, o=o16, S_T=S_T)

        def step32():
            kda.kda_chunk_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], chunk=C, o=o32, S_T=S_T)

        step32()
        step()
        torch.cuda.synchronize()
        o16_exact = bool(torch.equal(o16, o32.to(bf16)))
        checks.add("prefill", host_heads(x, heads), heads_of(o32, heads), states_of(S_T, heads), heads=[*range(len(heads))],
                   timed=True, extra_o={"bf16 o": heads_of(o16, heads)})
        for _ in range(args.warmup):
            step()
        wall_ms, per = event_ms(step, args.steps, torch)
        kern_ms = med(per)
        ms_per_step = wall_ms / args.steps
        alg16, pth16 = prefill_bytes(B, T, H, dk, dv, 2)
        for _ in range(args.warmup):
            step32()
        wall32, per32 = event_ms(step32, args.steps, torch)
        alg32, pth32 = prefill_bytes(B, T, H, dk, dv, 4)
        res["prefill"] = dict(ms_per_step=ms_per_step, kern_ms=kern_ms, kern_mean_ms=sum(per) / len(per),
                              roof=roofline(alg16, pth16, kern_ms, B * T * H, "kda_prefill", "kda_prefill"),
                              o16_exact=o16_exact,
                              f32=dict(ms_per_step=wall32 / args.steps, kern_ms=med(per32),
                                       roof=roofline(alg32, pth32, med(per32), B * T * H, "kda_prefill_f32o")))
        log(f"prefill (bf16 o): {ms_per_step:.3f} ms/step, kernel median {kern_ms:.3f} ms "
            f"({alg16 / kern_ms / 1e6:.0f} GB/s); fp32 o: kernel {med(per32):.3f} ms; bf16 o == RNE(fp32 o): "
            f"{o16_exact}")

    # ------- the same prefill recording the state every 4096 tokens (prefix caching) -------
    if "snapshots" in legs:
        snap_pos = list(range(4096, T + 1, 4096))
        snaps = torch.empty(B, H, len(snap_pos), dk, dv, device=dev, dtype=f32)

        def sstep():
            kda.kda_chunk_fwd_snapshots(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"],
                                        snap_tokens=snap_pos, chunk=C, o=o16, S_T=S_T, snaps=snaps)

        sstep()
        torch.cuda.synchronize()
        snap_heads = [0, B * H // 2 + 5]
        sh_in = host_heads({n: (t[:, :snap_pos[0]] if n != "S0" else t) for n, t in x.items()}, snap_heads)
        checks.add("snapshot", sh_in, None, states_of(snaps[:, :, 0].contiguous(), snap_heads),
                   heads=[0, 1])
        snap_last_is_state = bool(torch.equal(snaps[:, :, -1], S_T))
        for _ in range(args.warmup):
            sstep()
        s_wall, s_per = event_ms(sstep, args.steps, torch)
        res["snapshots"] = dict(wall=s_wall / args.steps, kern=med(s_per), n=len(snap_pos), every=snap_pos[0],
                                bytes=B * H * len(snap_pos) * dk * dv * 4, last_is_state=snap_last_is_state)
        log(f"prefill + {len(snap_pos)} snapshots: kernel {med(s_per):.3f} ms; last == S_T: {snap_last_is_state}")

    # ------- the same prefill with the gate fused in (z and A instead of alpha) -------
    if "gated" in legs:
        def gate_check(name, z, A, hid):
            b_, h_ = divmod(hid, H)
            hin = {n: x[n][b_:b_ + 1, :, h_:h_ + 1].cpu() for n in ("q", "k", "v", "beta")}
            hin["S0"] = x["S0"][b_:b_ + 1, h_:h_ + 1].cpu()
            hin["alpha"] = None
            checks.add(name, hin, heads_of(o32, [hid]), states_of(S_T, [hid]),
                       gate=(z[b_:b_ + 1, :, h_:h_ + 1].cpu(), A[h_:h_ + 1].cpu()))

        gz, gA = ki.make_gate((B, T, H, dk), H, w.qkv_dtype, seed=0, device=dev)

        def gstep(o_=None):
            kda.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], gz, gA, x["beta"], x["S0"], chunk=C,
                                    o=o16 if o_ is None else o_, S_T=S_T)

        gstep(o32)
        torch.cuda.synchronize()
        for hid in (0, B * H // 2 + 5):
            gate_check(f"gated head {hid}", gz, gA, hid)
        for _ in range(args.warmup):
            gstep()
        g_wall, g_per = event_ms(gstep, args.steps, torch)
        g_bytes, g_pth = prefill_bytes(B, T, H, dk, dv, 2, a_bytes=2)  # bf16 z in place of fp32 alpha
        log(f"gated prefill: kernel {med(g_per):.3f} ms, {g_bytes / med(g_per) / 1e6:.0f} GB/s of {g_pth} B/token-head")
        del gz, gA

        # fast-forgetting heads (z ~ N(-3, 1), A ~ N(0, 0.3)): most 32-token chunks decay
        # below e^-10 in some channel (the range that needs no special handling in the
        # two-stage path's bounded factors; the single-kernel pipeline regroups them)
        fz, fA = ki.make_gate((B, T, H, dk), H, w.qkv_dtype, seed=1, device=dev, z_mu=-3.0, z_std=1.0, a_std=0.3)

        def fstep(o_=None):
            kda.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], fz, fA, x["beta"], x["S0"], chunk=C,
                                    o=o16 if o_ is None else o_, S_T=S_T)

        fstep(o32)
        torch.cuda.synchronize()
        f_heads = list(range(B * H))  # every head
        for hid in f_heads:
            gate_check(f"fast-forgetting head {hid}", fz, fA, hid)
        fstep()
        f_wall, f_per = event_ms(fstep, args.steps, torch)
        res["gated"] = dict(wall=g_wall / args.steps, kern=med(g_per), bytes=g_bytes, pth=g_pth,
                            fast_kern=med(f_per), fast_heads=f_heads)
        log(f"gated prefill, fast-forgetting heads: kernel {med(f_per):.3f} ms ({med(f_per) / med(g_per):.2f}x)")
        del fz, fA

    if legs & {"prefill", "snapshots", "gated"}:
        del x, o16, o32, S_T
        torch.cuda.empty_cache()

    # ------- the 4K-token prefill (B=1, H=8): a single pass, all heads -------
    if "prefill4k" in legs:
        w1 = ki.WORKLOADS[1]
        x4 = ki.make_workload_prefill(1, seed=0, device=dev)
        o4 = torch.empty(w1.B, w1.T, w1.H, w1.dv, device=dev, dtype=bf16)
        o4f = torch.empty(w1.B, w1.T, w1.H, w1.dv, device=dev, dtype=f32)
        S4 = torch.empty(w1.B, w1.H, w1.dk, w1.dv, device=dev, dtype=f32)

        def step4(o_=o4):
            kda.kda_chunk_fwd(x4["q"], x4["k"], x4["v"], x4["alpha"], x4["beta"], x4["S0"], chunk=w1.chunk,
                              o=o_, S_T=S4)

        step4(o4f)
        torch.cuda.synchronize()
        h4 = list(range(w1.B * w1.H))
        checks.add("prefill 4k", {n: t.cpu() for n, t in x4.items()}, heads_of(o4f, h4), states_of(S4, h4),
                   heads=h4)
        for _ in range(args.warmup):
            step4()
        w4, p4 = event_ms(step4, args.steps, torch)
        a4, pth4 = prefill_bytes(w1.B, w1.T, w1.H, w1.dk, w1.dv, 2)
        res["prefill4k"] = dict(wall=w4 / args.steps, kern=med(p4),
                                roof=roofline(a4, pth4, med(p4), w1.B * w1.T * w1.H))
        log(f"4K prefill: kernel {med(p4) * 1e3:.1f} us, {w1.B * w1.T / med(p4) * 1e3:.4g} tok/s")
        del x4, o4, o4f, S4

    # ------- the 1M-token prefill (B=1, H=32, alpha = sigmoid(N(4,1))) -------
    if "prefill1m" in legs:
        w3 = ki.WORKLOADS[3]
        log("generating 1M-token inputs")
        x1 = ki.make_workload_prefill(3, seed=0, device=dev)
        o1 = torch.empty(w3.B, w3.T, w3.H, w3.dv, device=dev, dtype=bf16)
        S1 = torch.empty(w3.B, w3.H, w3.dk, w3.dv, device=dev, dtype=f32)

        def step1m(o_=o1):
            kda.kda_chunk_fwd(x1["q"], x1["k"], x1["v"], x1["alpha"], x1["beta"], x1["S0"], chunk=w3.chunk,
                              o=o_, S_T=S1)

        h1 = [0, 11, 22, 31]
        o1f = torch.empty(w3.B, w3.T, w3.H, w3.dv, device=dev, dtype=f32)
        step1m(o1f)
        torch.cuda.synchronize()
        checks.add("prefill 1m", host_heads(x1, h1), heads_of(o1f, h1), states_of(S1, h1), heads=[0, 1, 2, 3])
        del o1f
        for _ in range(min(args.warmup, 2)):
            step1m()
        w1m, p1m = event_ms(step1m, max(3, args.steps // 2), torch)
        a1m, pth1m = prefill_bytes(w3.B, w3.T, w3.H, w3.dk, w3.dv, 2)
        res["prefill1m"] = dict(wall=w1m / max(3, args.steps // 2), kern=med(p1m),
                                roof=roofline(a1m, pth1m, med(p1m), w3.B * w3.T * w3.H, "kda_prefill_1m"),
                                heads=h1)
        log(f"1M prefill: kernel {med(p1m):.2f} ms, {w3.B * w3.T / med(p1m) * 1e3:.4g} tok/s")
        del x1, o1, S1
        torch.cuda.empty_cache()

    # ------- a packed batch of 16 sequences of mixed lengths (kda_chunk_fwd_varlen) -------
    if "varlen" in legs:
        gl = torch.Generator().manual_seed(17)
        v_lens = [int(1024 * 2 ** (4 * r)) for r in torch.rand(16, generator=gl).tolist()]  # 1K .. 16K tokens
        v_total = sum(v_lens)
        vx = ki.make_prefill(1, v_total, H, dk, dv, w.qkv_dtype, w.alpha_mu, w.s0_std, seed=3, device=dev)
        vflat = {n: vx[n][0] for n in ("q", "k", "v", "alpha", "beta")}
        v_S0 = torch.cat([vx["S0"]] * len(v_lens), 0).contiguous()
        v_cu = torch.tensor([0] + torch.cumsum(torch.tensor(v_lens), 0).tolist(), dtype=torch.int32, device=dev)
        v_o = torch.empty(v_total, H, dv, device=dev, dtype=bf16)
        v_of = torch.empty(v_total, H, dv, device=dev, dtype=f32)
        v_ST = torch.empty(len(v_lens), H, dk, dv, device=dev, dtype=f32)

        def vstep(o_=v_o):
            kda.kda_chunk_fwd_varlen(vflat["q"], vflat["k"], vflat["v"], vflat["alpha"], vflat["beta"], v_cu, v_S0,
                                     chunk=C, o=o_, S_T=v_ST)

        vstep(v_of)
        torch.cuda.synchronize()
        vb = int(min(range(len(v_lens)), key=lambda i: v_lens[i]))  # the shortest sequence, against the oracle
        vs0 = int(v_cu[vb])
        vhin = {n: vflat[n][vs0:vs0 + v_lens[vb]][None].cpu() for n in vflat}
        vhin["S0"] = v_S0[vb:vb + 1].cpu()
        checks.add("varlen", vhin, heads_of(v_of[vs0:vs0 + v_lens[vb]][None], [0, H - 1]),
                   states_of(v_ST[vb:vb + 1], [0, H - 1]), heads=[0, H - 1])
        for _ in range(args.warmup):
            vstep()
        _, vl_per = event_ms(vstep, args.steps, torch)
        res["varlen"] = dict(kern=med(vl_per), total=v_total, lens=v_lens)
        log(f"varlen: {len(v_lens)} sequences, {v_total} tokens ({min(v_lens)}..{max(v_lens)}): "
            f"{med(vl_per):.3f} ms, {v_total / med(vl_per) * 1e3:.4g} tok/s")
        del vx, vflat, v_o, v_of

    # ------- few long chains: the split prefill (kda_chunk_fwd_split) against the single pass -------
    if "split" in legs:
        split_res = []
        for sB, sT, sH, sseed in ((1, 16384, 2, 5), (1, 65536, 2, 6)):
            sx = ki.make_prefill(sB, sT, sH, dk, dv, w.qkv_dtype, w.alpha_mu, w.s0_std, seed=sseed, device=dev)
            n_parts, ws_bytes = kda.kda_chunk_fwd_split_plan(w.qkv_dtype, sB, sT, sH, dk, dv, chunk=C)
            s_ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
            s_o = torch.empty(sB, sT, sH, dv, device=dev, dtype=bf16)
            s_of = torch.empty(sB, sT, sH, dv, device=dev, dtype=f32)
            s_S = torch.empty(sB, sH, dk, dv, device=dev, dtype=f32)

            def one(sx=sx, s_o=s_o, s_S=s_S):
                kda.kda_chunk_fwd(sx["q"], sx["k"], sx["v"], sx["alpha"], sx["beta"], sx["S0"], chunk=C, o=s_o,
                                  S_T=s_S)

            def spl(o_=s_o, sx=sx, s_S=s_S, n_parts=n_parts, s_ws=s_ws):
                kda.kda_chunk_fwd_split(sx["q"], sx["k"], sx["v"], sx["alpha"], sx["beta"], sx["S0"], parts=n_parts,
                                        chunk=C, o=o_, S_T=s_S, workspace=s_ws)

            spl(s_of)
            torch.cuda.synchronize()
            sheads = [0, sB * sH - 1]
            name = f"split B={sB} T={sT} H={sH}"
            checks.add(name, {n: t.cpu() for n, t in sx.items()}, heads_of(s_of, sheads), states_of(s_S, sheads),
                       heads=sheads)
            for _ in range(args.warmup):
                one()
                spl()
            _, one_per = event_ms(one, args.steps, torch)
            _, spl_per = event_ms(spl, args.steps, torch)
            one_ms, spl_ms = med(one_per), med(spl_per)
            log(f"split prefill B={sB} T={sT} H={sH}: {n_parts} parts, {spl_ms:.3f} ms vs single pass "
                f"{one_ms:.3f} ms ({one_ms / spl_ms:.2f}x)")
            split_res.append({"workload": f"prefill B={sB} T={sT} H={sH} d={dk}, bf16 o (kda_chunk_fwd_split, "
                                          f"library's part count)", "parts": n_parts, "workspace_bytes": ws_bytes,
                              "ms": spl_ms, "single_pass_ms": one_ms, "speedup": one_ms / spl_ms,
                              "tokens_per_s": sB * sT / (spl_ms / 1e3), "check": name})
            del sx, s_ws, s_o, s_of, s_S
        res["split"] = split_res

    # ---------------- decode: B=256, H=32, d=128, 100 in-place steps ----------------
    if legs & {"decode", "spec"}:
        wd = ki.WORKLOADS[4]
        DB, DH = wd.B, wd.H
        S = ki.make_state(DB, DH, dk, dv, wd.s0_std, 1, dev)
    if "decode" in legs:
        nsteps = args.decode_steps
        log(f"generating decode inputs B={DB} H={DH} steps={nsteps}")
        toks = [ki.make_decode_token(DB, DH, dk, dv, wd.qkv_dtype, wd.alpha_mu, seed=0, step=s, device=dev)
                for s in range(nsteps)]
        od = torch.empty(nsteps, DB, DH, dv, device=dev, dtype=bf16)
        odf = torch.empty(nsteps, DB, DH, dv, device=dev, dtype=f32)
        # sampled states: the 100 tokens of one state are a sequence of 100 tokens
        dheads = sorted(set(int(v) for v in np.linspace(0, DB * DH - 1, 8)))
        S_init = S.reshape(DB * DH, dk, dv)[dheads].cpu()
        for s, tk in enumerate(toks):
            kda.kda_decode_step(tk["q"], tk["k"], tk["v"], tk["alpha"], tk["beta"], S, o=odf[s])
        torch.cuda.synchronize()

        def gather(name):
            return torch.stack([tk[name].reshape(DB * DH, -1)[dheads] for tk in toks], 0)[None].cpu()

        seq = {n: gather(n) for n in ("q", "k", "v", "alpha")}
        seq["beta"] = torch.stack([tk["beta"].reshape(DB * DH)[dheads] for tk in toks], 0)[None].cpu()
        seq["S0"] = S_init[None]
        checks.add("decode", seq, odf.reshape(nsteps, DB * DH, dv)[:, dheads].permute(1, 0, 2).cpu().numpy(),
                   states_of(S, dheads))

        def dstep_all():
            for s, tk in enumerate(toks):
                kda.kda_decode_step(tk["q"], tk["k"], tk["v"], tk["alpha"], tk["beta"], S, o=od[s])

        dstep_all()  # warm-up pass
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record()
        dstep_all()
        ev1.record()
        torch.cuda.synchronize()
        d_step_ms = ev0.elapsed_time(ev1) / nsteps
        state_bytes = 2 * DB * DH * dk * dv * 4
        io_bytes = DB * DH * (2 * (2 * dk + dv) + 4 * dk + 4 + 2 * dv)
        res["decode"] = dict(step_ms=d_step_ms, state_bytes=state_bytes, io_bytes=io_bytes, nsteps=nsteps)
        log(f"decode: {d_step_ms * 1e3:.1f} us/step over {nsteps} steps, "
            f"state {state_bytes / d_step_ms / 1e6:.0f} GB/s, all bytes {(state_bytes + io_bytes) / d_step_ms / 1e6:.0f} GB/s")
        del toks

    # ------- speculative decoding: 4 drafts per sequence, verify then commit -------
    if "spec" in legs:
        SK = 4
        dr = ki.make_prefill(DB, SK, DH, dk, dv, wd.qkv_dtype, wd.alpha_mu, 0.0, seed=5, device=dev)
        o_sp = torch.empty(DB, SK, DH, dv, device=dev, dtype=f32)
        u_sp = torch.empty(DB, DH, SK, dv, device=dev, dtype=f32)
        acc = torch.arange(DB, device=dev, dtype=torch.int32) % (SK + 1)  # 0..4 drafts accepted
        sp_seq = 4 * (SK + 1) - 1  # a sequence that accepts all 4 drafts; parity on its heads
        S_sp0 = S[sp_seq].clone()
        kda.kda_decode_verify(dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"], S, o=o_sp, u=u_sp)
        kda.kda_decode_commit(dr["k"], dr["alpha"], u_sp, acc, S)
        torch.cuda.synchronize()
        sphin = {n: t[sp_seq:sp_seq + 1].cpu() for n, t in dr.items() if n != "S0"}
        sphin["S0"] = S_sp0[None].cpu()
        checks.add("spec decode", sphin, heads_of(o_sp[sp_seq:sp_seq + 1], list(range(DH))),
                   states_of(S[sp_seq:sp_seq + 1], list(range(DH))))
        o_sp16 = torch.empty(DB, SK, DH, dv, device=dev, dtype=bf16)
        ver_ms = back_to_back_ms(
            lambda: kda.kda_decode_verify(dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"], S, o=o_sp16, u=u_sp),
            20, torch)
        com_ms = back_to_back_ms(lambda: kda.kda_decode_commit(dr["k"], dr["alpha"], u_sp, acc, S), 20, torch)
        n_commit = int((acc > 0).sum().item())
        ver_bytes = (DB * DH * dk * dv * 4 + DB * SK * DH * (2 * (2 * dk + dv) + 4 * dk + 4 + 2 * dv)
                     + DB * DH * SK * dv * 4)
        com_bytes = 2 * n_commit * DH * dk * dv * 4
        res["spec"] = dict(SK=SK, ver_ms=ver_ms, com_ms=com_ms, n_commit=n_commit, ver_bytes=ver_bytes,
                           com_bytes=com_bytes)
        log(f"spec decode ({SK} drafts): verify {ver_ms * 1e3:.1f} us ({ver_bytes / ver_ms / 1e6:.0f} GB/s), "
            f"commit {com_ms * 1e3:.1f} us ({com_bytes / com_ms / 1e6:.0f} GB/s)")

    if args.copy_probe:
        a = torch.empty(1 << 28, device=dev, dtype=f32)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("copy probe: 1 GiB read + 1 GiB written")
        del a, b

    # ---------------- the CPU baseline: the oracle on every sample above ----------------
    errs, extra, cpu = {}, {}, None
    if not args.no_cpu_baseline:
        import oracle
        threads = oracle.default_threads()
        log(f"CPU baseline: the oracle on the sampled heads ({threads} threads)")
        errs, extra, cpu_s = cpu_baseline_leg(checks, threads, log)
        if cpu_s is not None:
            nth = len(checks.items["prefill"]["inputs"]["q"][0, 0]) * T
            # one thread on one head of the same workload
            h1 = {n: (t[:, :, :1] if n != "S0" else t[:, :1]) for n, t in checks.items["prefill"]["inputs"].items()}
            t0 = time.perf_counter()
            oracle.forward(h1["q"], h1["k"], h1["v"], h1["alpha"], h1["beta"], h1["S0"], threads=1)
            one_s = time.perf_counter() - t0
            cpu = {"value": nth / cpu_s / H, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                   "sample": f"{nth // T} of {B * H} heads of the 64K workload, full T={T} ({nth} token-heads, "
                             f"{cpu_s:.1f} s wall on {threads} threads); tokens/s = token-heads/s / H",
                   "single_thread": {"value": T / one_s / H, "unit": "tokens/s", "cores": 1,
                                     "sample": f"1 head of the same workload, T={T} ({one_s:.1f} s wall)"},
                   "cpu": _cpu_model()}
            log(f"oracle: {nth / cpu_s:.4g} token-heads/s on {threads} threads, {T / one_s:.4g} on one")

    def perr(name, i):
        return errs[name][i] if name in errs else None

    out = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": f"prefill B={B} T={T} H={H} d_k=d_v={dk}; bf16 q/k/v and o, fp32 alpha/beta/state; "
                                  f"chunk {C} requested, run as {RUN_CHUNK}-token chunks",
                      "global_batch": B, "seq_len": T, "heads": H, "head_dim": dk, "chunk": RUN_CHUNK,
                      "chunk_requested": C, "parallelism": "none (1 GPU)"}}
    if "prefill" in res:
        r = res["prefill"]
        out["value"] = B * T / (r["ms_per_step"] / 1e3)
        out["ms_per_step"] = r["ms_per_step"]
        out["kernel_ms_median"] = r["kern_ms"]
        out["roofline"] = r["roof"]
        out["fp32_o"] = {"workload": "the same prefill with an fp32 o (1,796 B per token-head)",
                         "ms_per_step": r["f32"]["ms_per_step"], "kernel_ms": r["f32"]["kern_ms"],
                         "roofline": r["f32"]["roof"]}
    if "prefill4k" in res:
        r = res["prefill4k"]
        out["prefill_4k"] = {"workload": "prefill B=1 T=4096 H=8 d=128, bf16 o, single pass (kda_chunk_fwd)",
                             "kernel_ms": r["kern"], "ms_per_step": r["wall"],
                             "tokens_per_s": 4096 / (r["kern"] / 1e3), "roofline": r["roof"],
                             "parity_o": perr("prefill 4k", 0), "parity_S_T": perr("prefill 4k", 1)}
    if "prefill1m" in res:
        r = res["prefill1m"]
        out["prefill_1m"] = {"workload": "prefill B=1 T=1048576 H=32 d=128, alpha = sigmoid(N(4,1)), bf16 o",
                             "kernel_ms": r["kern"], "ms_per_step": r["wall"],
                             "tokens_per_s": 1048576 / (r["kern"] / 1e3), "roofline": r["roof"],
                             "parity_heads": r["heads"], "parity_o": perr("prefill 1m", 0),
                             "parity_S_T": perr("prefill 1m", 1)}
    if "decode" in res:
        r = res["decode"]
        tot = r["state_bytes"] + r["io_bytes"]
        dtr = measured_traffic("kda_decode")
        out["decode"] = {"workload": f"decode B=256 H=32 d=128, {r['nsteps']} in-place steps back to back, bf16 "
                                     f"q/k/v and o, fp32 state",
                         "us_per_step": r["step_ms"] * 1e3,
                         "state_gbps": r["state_bytes"] / r["step_ms"] / 1e6,
                         "roofline": {"bound": "hbm", "achieved": tot / r["step_ms"] / 1e6, "peak": HBM_PEAK_GBS,
                                      "unit": "GB/s", "frac": tot / r["step_ms"] / 1e6 / HBM_PEAK_GBS,
                                      "traffic": dtr, "kernel_us": r["step_ms"] * 1e3, "algorithmic_bytes": tot}}
    if "snapshots" in res:
        r = res["snapshots"]
        out["snapshots"] = {"workload": f"the 64K prefill (bf16 o), also recording the state after every {r['every']} "
                                        f"tokens ({r['n']} per sequence, kda_chunk_fwd_snapshots)",
                            "ms_per_step": r["wall"], "kernel_ms": r["kern"],
                            "overhead_vs_prefill": r["kern"] / res["prefill"]["kern_ms"] - 1 if "prefill" in res else None,
                            "snapshot_bytes": r["bytes"], "parity_first_snapshot": perr("snapshot", 1),
                            "last_snapshot_equals_S_T": r["last_is_state"]}
    if "gated" in res:
        r = res["gated"]
        fo = [errs[f"fast-forgetting head {h}"] for h in r["fast_heads"] if f"fast-forgetting head {h}" in errs]
        gerr = [errs[f"gated head {h}"] for h in (0, B * H // 2 + 5) if f"gated head {h}" in errs]
        out["gated"] = {"workload": "the 64K prefill with the gate fused in (kda_chunk_fwd_gated: bf16 z and per-head "
                                    "A in place of fp32 alpha), bf16 o",
                        "ms_per_step": r["wall"], "kernel_ms": r["kern"], "bytes_per_token_head": r["pth"],
                        "achieved_gbps": r["bytes"] / r["kern"] / 1e6,
                        "frac_hbm": r["bytes"] / r["kern"] / 1e6 / HBM_PEAK_GBS,
                        "vs_plain": r["kern"] / res["prefill"]["kern_ms"] if "prefill" in res else None,
                        "parity_o": max(e[0] for e in gerr) if gerr else None,
                        "parity_S_T": max(e[1] for e in gerr) if gerr else None,
                        "traffic": measured_traffic("kda_prefill_gated"),
                        "gate_recipe": "z ~ N(-4.5, 0.4) bf16, A ~ N(0, 0.1) per head",
                        "fast_forgetting": {"gate_recipe": "z ~ N(-3, 1), A ~ N(0, 0.3)", "kernel_ms": r["fast_kern"],
                                            "vs_gated": r["fast_kern"] / r["kern"], "parity_heads": r["fast_heads"],
                                            "parity_o": max(e[0] for e in fo) if fo else None,
                                            "parity_S_T": max(e[1] for e in fo) if fo else None}}
    if "split" in res:
        for s in res["split"]:
            name = s.pop("check")
            s["parity_o"], s["parity_S_T"] = perr(name, 0), perr(name, 1)
        out["split"] = res["split"]
    if "varlen" in res:
        r = res["varlen"]
        out["varlen"] = {"workload": f"packed batch of {len(r['lens'])} sequences, {r['total']} tokens (lengths "
                                     f"{min(r['lens'])}..{max(r['lens'])}), H={H} d={dk}, bf16 o, kda_chunk_fwd_varlen",
                         "kernel_ms": r["kern"], "tokens_per_s": r["total"] / (r["kern"] / 1e3), "lengths": r["lens"],
                         "parity_o": perr("varlen", 0), "parity_S_T": perr("varlen", 1)}
    if "spec" in res:
        r = res["spec"]
        d1 = res["decode"]["step_ms"] if "decode" in res else None
        out["spec_decode"] = {"workload": f"decode B=256 H=32 d=128 with {r['SK']} draft tokens per sequence: "
                                          f"kda_decode_verify (bf16 o), then kda_decode_commit with 0..{r['SK']} "
                                          f"accepted ({r['n_commit']} of 256 sequences commit); each time the "
                                          f"median of 5 groups of 20 launches back to back, after 100 untimed launches",
                              "verify_us": r["ver_ms"] * 1e3, "commit_us": r["com_ms"] * 1e3,
                              "verify_gbps": r["ver_bytes"] / r["ver_ms"] / 1e6,
                              "commit_gbps": r["com_bytes"] / r["com_ms"] / 1e6,
                              "sequential_decode_us": r["SK"] * d1 * 1e3 if d1 else None,
                              "parity_o": perr("spec decode", 0), "parity_S": perr("spec decode", 1)}
    all_errs = [v for pair in errs.values() for v in pair if v is not None]
    pr = res.get("prefill", {})
    out["parity"] = {"checked": bool(errs), "pass": (bool(errs) and max(all_errs) <= TOL_REL
                                                     and res.get("snapshots", {}).get("last_is_state", True)),
                     "tol_rel_rms": TOL_REL, "prefill_o_fp32": perr("prefill", 0), "prefill_S_T": perr("prefill", 1),
                     "prefill_o_bf16": extra.get("prefill/bf16 o"),
                     "prefill_o_bf16_is_rounded_fp32": pr.get("o16_exact"),
                     "decode_o": perr("decode", 0), "decode_S": perr("decode", 1),
                     "checks": {k: list(v) for k, v in errs.items()},
                     "note": "bf16 o is checked to be exactly the fp32 o rounded to nearest even; the tolerance "
                             "applies to the fp32 o (the rounding of a bf16 o alone can reach 2^-8 of |o|)"}
    out["cpu_baseline"] = cpu
    out["device"] = props.name
    out["source_hash"] = source_hash()
    out["legs"] = sorted(legs)
    print(json.dumps(out), flush=True)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
