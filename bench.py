#!/usr/bin/env python3
"""Benchmark libkda on one MI355X and print one JSON line.

One timed step is one kda_chunk_fwd call over the 64K-token prefill workload
(B=2, H=32, T=65536, d_k=d_v=128, bf16 q/k/v, fp32 alpha/beta/state, chunk 64,
fp32 o), with inputs resident in HBM.  The same run times the other calls on
their workloads (state snapshots, the fused gate, a packed batch, the split
prefill, batched and speculative decode) and reports each under its own key.

The GPU legs keep host copies of sampled heads' inputs and outputs; the last
leg, the CPU baseline, runs the fp64 oracle on all of them.  Its time on the
prefill sample, on this host's cores, is `cpu_baseline`; its comparisons are
the parity fields (max|GPU - oracle| / RMS(oracle) per head, worst head).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "KDA prefill tokens/s @T=64K,H=32,d=128 (%MFMA peak); decode state GB/s (%HBM)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 (fp16 is the same rate)
TOL_REL = 2e-2


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def prefill_counts(B, T, H, dk, dv, chunk, o_bytes):
    """Algorithmic bytes and FLOPs of one prefill call: the q/k/v/alpha/beta reads
    and o writes each token-head needs, plus one S0 read and S_T write per chain;
    FLOPs of the chunk form at chunk size `chunk`."""
    th = B * T * H
    per_th_bytes = 2 * (2 * dk + dv) + 4 * dk + 4 + o_bytes * dv
    state_bytes = 2 * 4 * dk * dv * B * H
    per_th_flops = 6 * dk * dv + chunk * (3 * dk + 2 * dv) + chunk * chunk / 3.0
    return th * per_th_bytes + state_bytes, th * per_th_flops, per_th_bytes, per_th_flops


def source_hash():
    h = hashlib.sha256()
    for f in sorted((ROOT / "gated_delta_rule_07_amd" / "csrc").glob("*")):
        h.update(f.read_bytes())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else None."""
    f = ROOT / "profiles" / "traffic.json"
    if not f.exists():
        return None
    try:
        d = json.loads(f.read_text())
    except ValueError:
        return None
    ent = d.get(kernel_key)
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent.get("bytes_per_launch")


def timed_launches(fn, n, torch):
    """Run fn() n times on the current stream; return (total_ms, mean per-launch ms)
    from HIP events recorded on that stream."""
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
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall_ms, sum(per) / len(per), starts[0].elapsed_time(ends[-1])


def back_to_back_ms(fn, n, torch):
    """Mean ms per launch of n launches of fn() back to back, between one pair of
    HIP events on the current stream (no markers between the launches, so short
    kernels are not charged for them)."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


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

    def add(self, name, inputs, got_o, got_s, heads=None, gate=None, per_step=False, timed=False):
        """inputs: host q, k, v, alpha (or None with gate=(z, A)), beta, S0 as [B,T,H,.];
        got_o [n, T, d_v] (None: not compared), got_s [n, d_k, d_v], both for `heads`
        (ids b*H + h; None: all, in (b, h) order).  per_step: normalise o per token
        over the heads (decode, where each head has one token per step)."""
        self.items[name] = dict(inputs=inputs, got_o=got_o, got_s=got_s, heads=heads, gate=gate,
                                per_step=per_step, timed=timed)


def cpu_baseline_leg(checks, threads, log):
    """Runs the oracle on every check: returns {name: (err_o, err_s)} and the wall
    time of the timed check (the prefill sample), which is the CPU baseline."""
    import oracle
    errs, timed_s = {}, None
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
            if c["per_step"]:
                eo = max(rel_err_heads(c["got_o"][:, t].reshape(1, -1), ro[:, t].reshape(1, -1))
                         for t in range(ro.shape[1]))
            else:
                eo = max(rel_err_heads(g[None].astype("float64"), r[None]) for g, r in zip(c["got_o"], ro))
        es = rel_err_heads(c["got_s"].astype("float64"), rs)
        errs[name] = (eo, es)
        log(f"parity {name}: o {eo if eo is None else f'{eo:.3e}'}  S {es:.3e}")
    return errs, timed_s


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--sample-heads", type=int, default=64, help="heads checked by the oracle (all 64 by default)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="do not report the oracle's time")
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

    import numpy as np
    import torch

    import gated_delta_rule_07_amd as kda
    import kda_inputs as ki

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kda.load_library()
    props = torch.cuda.get_device_properties(dev)
    checks = OracleChecks()

    def heads_of(t, heads):
        """[B,T,H,d] device tensor -> float32 numpy [n, T, d] for head ids b*H + h."""
        Bt, Tt, Ht, dt = t.shape
        return t.permute(0, 2, 1, 3).reshape(Bt * Ht, Tt, dt)[heads].float().cpu().numpy()

    def states_of(t, heads):
        return t.reshape(-1, t.shape[-2], t.shape[-1])[heads].float().cpu().numpy()

    # ---------------- prefill: 64K tokens, B=2, H=32, d=128 ----------------
    w = ki.WORKLOADS[2]
    B, T, H, dk, dv, C = w.B, w.T, w.H, w.dk, w.dv, w.chunk
    log(f"generating prefill inputs B={B} T={T} H={H} d={dk}")
    x = ki.make_workload_prefill(2, seed=0, device=dev)
    hx = {n: t.cpu() for n, t in x.items()}  # host copy for the oracle leg
    o = torch.empty(B, T, H, dv, device=dev, dtype=torch.float32)
    S_T = torch.empty(B, H, dk, dv, device=dev, dtype=torch.float32)

    def step():
        kda.kda_chunk_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], chunk=C, o=o, S_T=S_T)

    step()
    torch.cuda.synchronize()
    nh = min(args.sample_heads, B * H)
    heads = sorted(set(int(v) for v in np.linspace(0, B * H - 1, nh)))
    checks.add("prefill", hx, heads_of(o, heads), states_of(S_T, heads), heads=heads, timed=True)

    for _ in range(args.warmup):
        step()
    wall_ms, kern_ms, span_ms = timed_launches(step, args.steps, torch)
    ms_per_step = wall_ms / args.steps
    tokens_per_s = B * T / (ms_per_step / 1e3)
    alg_bytes, alg_flops, per_th_bytes, per_th_flops = prefill_counts(B, T, H, dk, dv, C, 4)
    achieved_gbs = alg_bytes / (kern_ms / 1e3) / 1e9
    tflops = alg_flops / (kern_ms / 1e3) / 1e12
    attainable = min(MFMA_BF16_PEAK_TFS, per_th_flops / per_th_bytes * HBM_PEAK_GBS / 1e3)
    log(f"prefill: {ms_per_step:.3f} ms/step (kernel {kern_ms:.3f} ms), {tokens_per_s:.4g} tok/s, "
        f"{achieved_gbs:.0f} GB/s, {tflops:.1f} TFLOP/s")

    # ------- the same prefill recording the state every 4096 tokens (prefix caching) -------
    snap_pos = list(range(4096, T + 1, 4096))
    snaps = torch.empty(B, H, len(snap_pos), dk, dv, device=dev, dtype=torch.float32)

    def sstep():
        kda.kda_chunk_fwd_snapshots(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], snap_tokens=snap_pos,
                                    chunk=C, o=o, S_T=S_T, snaps=snaps)

    sstep()
    torch.cuda.synchronize()
    snap_heads = [0, B * H // 2 + 5]
    checks.add("snapshot", {n: (t[:, :snap_pos[0]] if n != "S0" else t) for n, t in hx.items()}, None,
               states_of(snaps[:, :, 0].contiguous(), snap_heads), heads=snap_heads)
    snap_last_is_state = bool(torch.equal(snaps[:, :, -1], S_T))
    for _ in range(args.warmup):
        sstep()
    s_wall_ms, s_kern_ms, _ = timed_launches(sstep, args.steps, torch)
    snap_bytes = B * H * len(snap_pos) * dk * dv * 4
    log(f"prefill + {len(snap_pos)} snapshots: {s_wall_ms / args.steps:.3f} ms/step (kernel {s_kern_ms:.3f} ms, "
        f"{100 * (s_kern_ms / kern_ms - 1):+.1f}%); last == S_T: {snap_last_is_state}")

    # ------- the same prefill with the gate fused in (z and A instead of alpha) -------
    def gate_check(name, z, A, hid):
        b_, h_ = divmod(hid, H)
        hin = {n: hx[n][b_:b_ + 1, :, h_:h_ + 1] for n in ("q", "k", "v", "beta")}
        hin["S0"] = hx["S0"][b_:b_ + 1, h_:h_ + 1]
        hin["alpha"] = None
        checks.add(name, hin, heads_of(o, [hid]), states_of(S_T, [hid]),
                   gate=(z[b_:b_ + 1, :, h_:h_ + 1].cpu(), A[h_:h_ + 1].cpu()))

    gz, gA = ki.make_gate((B, T, H, dk), H, w.qkv_dtype, seed=0, device=dev)

    def gstep():
        kda.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], gz, gA, x["beta"], x["S0"], chunk=C, o=o, S_T=S_T)

    gstep()
    torch.cuda.synchronize()
    for hid in (0, B * H // 2 + 5):
        gate_check(f"gated head {hid}", gz, gA, hid)
    for _ in range(args.warmup):
        gstep()
    g_wall_ms, g_kern_ms, _ = timed_launches(gstep, args.steps, torch)
    g_per_th = per_th_bytes - 4 * dk + 2 * dk  # bf16 z in place of fp32 alpha; A is H floats per call
    g_bytes = g_per_th * B * T * H + 2 * B * H * dk * dv * 4
    log(f"gated prefill: {g_wall_ms / args.steps:.3f} ms/step (kernel {g_kern_ms:.3f} ms), "
        f"{g_bytes / g_kern_ms / 1e6:.0f} GB/s of {g_per_th} B/token-head")
    del gz, gA

    # fast-forgetting heads (z ~ N(-3, 1), A ~ N(0, 0.3)): most 32-token chunks decay
    # below e^-10 in some channel and are split into shorter segments
    fz, fA = ki.make_gate((B, T, H, dk), H, w.qkv_dtype, seed=1, device=dev, z_mu=-3.0, z_std=1.0, a_std=0.3)

    def fstep():
        kda.kda_chunk_fwd_gated(x["q"], x["k"], x["v"], fz, fA, x["beta"], x["S0"], chunk=C, o=o, S_T=S_T)

    fstep()
    torch.cuda.synchronize()
    f_head = 1 * H + 7
    gate_check("fast-forgetting", fz, fA, f_head)
    fstep()
    f_wall_ms, f_kern_ms, _ = timed_launches(fstep, args.steps, torch)
    log(f"gated prefill, fast-forgetting heads: kernel {f_kern_ms:.3f} ms ({f_kern_ms / g_kern_ms:.2f}x)")
    del fz, fA

    # ------- a packed batch of 16 sequences of mixed lengths (kda_chunk_fwd_varlen) -------
    gl = torch.Generator().manual_seed(17)
    v_lens = [int(1024 * 2 ** (4 * r)) for r in torch.rand(16, generator=gl).tolist()]  # 1K .. 16K tokens
    v_total = sum(v_lens)
    vx = ki.make_prefill(1, v_total, H, dk, dv, w.qkv_dtype, w.alpha_mu, w.s0_std, seed=3, device=dev)
    vflat = {n: vx[n][0] for n in ("q", "k", "v", "alpha", "beta")}
    v_S0 = torch.cat([vx["S0"]] * len(v_lens), 0).contiguous()
    v_cu = torch.tensor([0] + torch.cumsum(torch.tensor(v_lens), 0).tolist(), dtype=torch.int32, device=dev)
    v_o = torch.empty(v_total, H, dv, device=dev, dtype=torch.float32)
    v_ST = torch.empty(len(v_lens), H, dk, dv, device=dev, dtype=torch.float32)

    def vstep():
        kda.kda_chunk_fwd_varlen(vflat["q"], vflat["k"], vflat["v"], vflat["alpha"], vflat["beta"], v_cu, v_S0,
                                 chunk=C, o=v_o, S_T=v_ST)

    vstep()
    torch.cuda.synchronize()
    vb = int(min(range(len(v_lens)), key=lambda i: v_lens[i]))  # the shortest sequence, against the oracle
    vs0 = int(v_cu[vb])
    vhin = {n: vflat[n][vs0:vs0 + v_lens[vb]][None].cpu() for n in vflat}
    vhin["S0"] = v_S0[vb:vb + 1].cpu()
    checks.add("varlen", vhin, heads_of(v_o[vs0:vs0 + v_lens[vb]][None], [0, H - 1]),
               states_of(v_ST[vb:vb + 1], [0, H - 1]), heads=[0, H - 1])
    for _ in range(args.warmup):
        vstep()
    v_wall_ms, v_kern_ms, _ = timed_launches(vstep, args.steps, torch)
    v_tok_s = v_total / (v_kern_ms / 1e3)
    log(f"varlen: {len(v_lens)} sequences, {v_total} tokens ({min(v_lens)}..{max(v_lens)}): "
        f"{v_kern_ms:.3f} ms, {v_tok_s:.4g} tok/s")
    del vx, vflat

    # ------- few long chains: the split prefill (kda_chunk_fwd_split) against the single pass -------
    split_res = []
    for sB, sT, sH, sseed in ((1, 4096, 8, 5), (1, 65536, 2, 6)):
        sx = ki.make_prefill(sB, sT, sH, dk, dv, w.qkv_dtype, w.alpha_mu, w.s0_std, seed=sseed, device=dev)
        n_parts, ws_bytes = kda.kda_chunk_fwd_split_plan(w.qkv_dtype, sB, sT, sH, dk, dv, chunk=C)
        s_ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        s_o = torch.empty(sB, sT, sH, dv, device=dev, dtype=torch.float32)
        s_S = torch.empty(sB, sH, dk, dv, device=dev, dtype=torch.float32)

        def one(sx=sx, s_o=s_o, s_S=s_S):
            kda.kda_chunk_fwd(sx["q"], sx["k"], sx["v"], sx["alpha"], sx["beta"], sx["S0"], chunk=C, o=s_o, S_T=s_S)

        def spl(sx=sx, s_o=s_o, s_S=s_S, n_parts=n_parts, s_ws=s_ws):
            kda.kda_chunk_fwd_split(sx["q"], sx["k"], sx["v"], sx["alpha"], sx["beta"], sx["S0"], parts=n_parts,
                                    chunk=C, o=s_o, S_T=s_S, workspace=s_ws)

        spl()
        torch.cuda.synchronize()
        sheads = [0, sB * sH - 1]
        name = f"split B={sB} T={sT} H={sH}"
        checks.add(name, {n: t.cpu() for n, t in sx.items()}, heads_of(s_o, sheads), states_of(s_S, sheads),
                   heads=sheads)
        for _ in range(args.warmup):
            one()
            spl()
        _, one_ms, _ = timed_launches(one, args.steps, torch)
        _, spl_ms, _ = timed_launches(spl, args.steps, torch)
        log(f"split prefill B={sB} T={sT} H={sH}: {n_parts} parts, {spl_ms:.3f} ms vs single pass "
            f"{one_ms:.3f} ms ({one_ms / spl_ms:.2f}x)")
        split_res.append({"workload": f"prefill B={sB} T={sT} H={sH} d={dk} (kda_chunk_fwd_split, library's "
                                      f"part count)", "parts": n_parts, "workspace_bytes": ws_bytes,
                          "ms": spl_ms, "single_pass_ms": one_ms, "speedup": one_ms / spl_ms,
                          "tokens_per_s": sB * sT / (spl_ms / 1e3), "check": name})
        del sx, s_ws, s_o, s_S

    # ---------------- decode: B=256, H=32, d=128, 100 in-place steps ----------------
    wd = ki.WORKLOADS[4]
    DB, DH = wd.B, wd.H
    nsteps = args.decode_steps
    log(f"generating decode inputs B={DB} H={DH} steps={nsteps}")
    S = ki.make_state(DB, DH, dk, dv, wd.s0_std, 1, dev)
    toks = [ki.make_decode_token(DB, DH, dk, dv, wd.qkv_dtype, wd.alpha_mu, seed=0, step=s, device=dev)
            for s in range(nsteps)]
    od = torch.empty(nsteps, DB, DH, dv, device=dev, dtype=torch.float32)
    # sampled states: the 100 tokens of one state are a sequence of 100 tokens
    dheads = sorted(set(int(v) for v in np.linspace(0, DB * DH - 1, 8)))
    S_init = S.reshape(DB * DH, dk, dv)[dheads].cpu()
    for s, tk in enumerate(toks):
        kda.kda_decode_step(tk["q"], tk["k"], tk["v"], tk["alpha"], tk["beta"], S, o=od[s])
    torch.cuda.synchronize()

    def gather(name):
        return torch.stack([tk[name].reshape(DB * DH, -1)[dheads] for tk in toks], 0)[None].cpu()

    seq = {n: gather(n) for n in ("q", "k", "v", "alpha")}
    seq["beta"] = torch.stack([tk["beta"].reshape(DB * DH)[dheads] for tk in toks], 0)[None].cpu()
    seq["S0"] = S_init[None]
    checks.add("decode", seq, od.reshape(nsteps, DB * DH, dv)[:, dheads].permute(1, 0, 2).cpu().numpy(),
               states_of(S, dheads), per_step=True)

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
    d_total_ms = ev0.elapsed_time(ev1)
    # per-launch duration on the same stream: 20 launches back to back
    d_kern_ms = back_to_back_ms(
        lambda: kda.kda_decode_step(toks[0]["q"], toks[0]["k"], toks[0]["v"], toks[0]["alpha"],
                                    toks[0]["beta"], S, o=od[0]), 20, torch)
    d_step_ms = d_total_ms / nsteps
    state_bytes = 2 * DB * DH * dk * dv * 4
    io_bytes = DB * DH * (2 * (2 * dk + dv) + 4 * dk + 4 + 4 * dv)
    d_gbs_state = state_bytes / (d_step_ms / 1e3) / 1e9
    d_gbs_kernel = (state_bytes + io_bytes) / (d_kern_ms / 1e3) / 1e9
    log(f"decode: {d_step_ms * 1e3:.1f} us/step (kernel {d_kern_ms * 1e3:.1f} us), "
        f"state {d_gbs_state:.0f} GB/s, kernel {d_gbs_kernel:.0f} GB/s")

    # ------- speculative decoding: 4 drafts per sequence, verify then commit -------
    SK = 4
    dr = ki.make_prefill(DB, SK, DH, dk, dv, wd.qkv_dtype, wd.alpha_mu, 0.0, seed=5, device=dev)
    o_sp = torch.empty(DB, SK, DH, dv, device=dev, dtype=torch.float32)
    u_sp = torch.empty(DB, DH, SK, dv, device=dev, dtype=torch.float32)
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
    v_kern_ms = back_to_back_ms(
        lambda: kda.kda_decode_verify(dr["q"], dr["k"], dr["v"], dr["alpha"], dr["beta"], S, o=o_sp, u=u_sp),
        20, torch)
    c_kern_ms = back_to_back_ms(lambda: kda.kda_decode_commit(dr["k"], dr["alpha"], u_sp, acc, S), 20, torch)
    n_commit = int((acc > 0).sum().item())
    v_bytes = DB * DH * dk * dv * 4 + DB * SK * DH * (2 * (2 * dk + dv) + 4 * dk + 4 + 4 * dv) + DB * DH * SK * dv * 4
    c_bytes = 2 * n_commit * DH * dk * dv * 4
    log(f"spec decode ({SK} drafts): verify {v_kern_ms * 1e3:.1f} us ({v_bytes / v_kern_ms / 1e6:.0f} GB/s), "
        f"commit {c_kern_ms * 1e3:.1f} us ({c_bytes / c_kern_ms / 1e6:.0f} GB/s); {SK} decode steps "
        f"{SK * d_kern_ms * 1e3:.1f} us")

    if args.copy_probe:
        a = torch.empty(1 << 28, device=dev, dtype=torch.float32)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("copy probe: 1 GiB read + 1 GiB written")
        del a, b

    # ---------------- the CPU baseline: the oracle on every sample above ----------------
    import oracle
    threads = oracle.default_threads()
    log(f"CPU baseline: the oracle on the sampled heads ({threads} threads); prefill heads {heads}")
    errs, cpu_s = cpu_baseline_leg(checks, threads, log)
    e_o, e_s = errs["prefill"]
    cpu = None
    if not args.no_cpu_baseline:
        rate = len(heads) * T / cpu_s  # token-heads per second on this host
        cpu = {"value": rate / H, "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": f"{len(heads)} of {B * H} heads of the same workload, full T={T} "
                         f"({len(heads) * T} token-heads, {cpu_s:.1f} s wall); tokens/s = "
                         f"token-heads/s / H", "cpu": _cpu_model()}
    gated_err = [errs[f"gated head {hid}"] for hid in (0, B * H // 2 + 5)]
    e_go, e_gs = max(e[0] for e in gated_err), max(e[1] for e in gated_err)
    for r in split_res:
        r["parity_o"], r["parity_S_T"] = errs[r.pop("check")]
    all_errs = [v for pair in errs.values() for v in pair if v is not None]
    parity_ok = max(all_errs) <= TOL_REL and snap_last_is_state
    out = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"prefill B={B} T={T} H={H} d_k=d_v={dk} chunk={C}; bf16 q/k/v, "
                               f"fp32 alpha/beta/state, fp32 o",
                   "global_batch": B, "seq_len": T, "heads": H, "head_dim": dk, "chunk": C,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic("kda_prefill"),
                     "kernel_ms": kern_ms, "algorithmic_bytes": alg_bytes,
                     "bytes_per_token_head": per_th_bytes,
                     "mfma_tflops": tflops, "mfma_frac": tflops / MFMA_BF16_PEAK_TFS,
                     "flops_per_token_head": per_th_flops,
                     "attainable_tflops": attainable, "frac_of_attainable": tflops / attainable},
        "decode": {"workload": f"decode B={DB} H={DH} d={dk}, {nsteps} in-place steps, bf16 q/k/v, fp32 state",
                   "us_per_step": d_step_ms * 1e3, "state_gbps": d_gbs_state,
                   "roofline": {"bound": "hbm", "achieved": d_gbs_kernel, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": d_gbs_kernel / HBM_PEAK_GBS,
                                "traffic": measured_traffic("kda_decode"),
                                "kernel_us": d_kern_ms * 1e3, "algorithmic_bytes": state_bytes + io_bytes}},
        "snapshots": {"workload": f"the prefill above, also recording the state after every {snap_pos[0]} "
                                  f"tokens ({len(snap_pos)} per sequence, kda_chunk_fwd_snapshots)",
                      "ms_per_step": s_wall_ms / args.steps, "kernel_ms": s_kern_ms,
                      "overhead_vs_prefill": s_kern_ms / kern_ms - 1, "snapshot_bytes": snap_bytes,
                      "parity_first_snapshot": errs["snapshot"][1], "last_snapshot_equals_S_T": snap_last_is_state},
        "gated": {"workload": "the prefill above with the gate fused in (kda_chunk_fwd_gated: bf16 z and "
                              "per-head A in place of fp32 alpha)",
                  "ms_per_step": g_wall_ms / args.steps, "kernel_ms": g_kern_ms,
                  "bytes_per_token_head": g_per_th, "achieved_gbps": g_bytes / g_kern_ms / 1e6,
                  "frac_hbm": g_bytes / g_kern_ms / 1e6 / HBM_PEAK_GBS, "parity_o": e_go, "parity_S_T": e_gs,
                  "traffic": measured_traffic("kda_prefill_gated"),
                  "gate_recipe": "z ~ N(-4.5, 0.4) bf16, A ~ N(0, 0.1) per head",
                  "fast_forgetting": {"gate_recipe": "z ~ N(-3, 1), A ~ N(0, 0.3)", "kernel_ms": f_kern_ms,
                                      "vs_gated": f_kern_ms / g_kern_ms, "parity_o": errs["fast-forgetting"][0],
                                      "parity_S_T": errs["fast-forgetting"][1]}},
        "split": split_res,
        "varlen": {"workload": f"packed batch of {len(v_lens)} sequences, {v_total} tokens "
                               f"(lengths {min(v_lens)}..{max(v_lens)}), H={H} d={dk}, kda_chunk_fwd_varlen",
                   "kernel_ms": v_kern_ms, "tokens_per_s": v_tok_s, "lengths": v_lens,
                   "parity_o": errs["varlen"][0], "parity_S_T": errs["varlen"][1]},
        "spec_decode": {"workload": f"decode B={DB} H={DH} d={dk} with {SK} draft tokens per sequence: "
                                    f"kda_decode_verify, then kda_decode_commit with 0..{SK} accepted "
                                    f"({n_commit} of {DB} sequences commit)",
                        "verify_us": v_kern_ms * 1e3, "commit_us": c_kern_ms * 1e3,
                        "verify_gbps": v_bytes / v_kern_ms / 1e6, "commit_gbps": c_bytes / c_kern_ms / 1e6,
                        "sequential_decode_us": SK * d_kern_ms * 1e3,
                        "parity_o": errs["spec decode"][0], "parity_S": errs["spec decode"][1]},
        "parity": {"pass": parity_ok, "tol_rel_rms": TOL_REL, "prefill_o": e_o, "prefill_S_T": e_s,
                   "prefill_heads": heads, "decode_o": errs["decode"][0], "decode_S": errs["decode"][1],
                   "decode_states": dheads, "checks": {k: list(v) for k, v in errs.items()}},
        "cpu_baseline": cpu,
        "device": props.name,
        "source_hash": source_hash(),
    }
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
