"""KDA oracle: plain fp64 CPU recurrence, used as the correctness authority.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
(``gated_delta_rule_07_amd``) never imports it and shares no code with it.

The recurrence lives in ``kda_oracle.c`` (built with gcc into
``libkda_oracle.so``); this module marshals arrays, and ``gate_alpha`` forms
the retention from a gate pre-activation in numpy fp64.  What the recurrence
computes, with its citations, is documented at the top of the C file:
the "Kimi K3 Technical Report review" (jw9603.github.io), sections 3.2-3.3.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(worked example, closed forms, invariants, brute-force matrix products).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "kda_oracle.c"
_LIB = _HERE / "libkda_oracle.so"

F32, BF16, F64 = 0, 1, 2
ORDER_PAGE1, ORDER_LITERAL_P2 = 0, 1

# Deliberate mistakes the C oracle can plant (test use only).
MUTATIONS = {
    "no_decay": 1,
    "delta_sign": 2,
    "read_pre_update": 3,
    "decay_columns": 4,
    "predict_undecayed": 5,
    "drop_beta": 6,
    "read_with_k": 7,
}

_lib = None


def build(force: bool = False, verbose: bool = False) -> Path:
    """Compile the oracle with gcc (CPU only)."""
    if force or not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
        tmp = _LIB.with_suffix(".so.tmp%d" % os.getpid())
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
               str(_SRC), "-o", str(tmp), "-lm"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not _LIB.exists():
            build()
        lib = ctypes.CDLL(str(_LIB))
        vp, i32 = ctypes.c_void_p, ctypes.c_int
        lib.kda_oracle_forward.restype = i32
        lib.kda_oracle_forward.argtypes = [vp, vp, vp, i32, vp, i32, vp, i32, vp, i32, vp, vp,
                                           i32, i32, i32, i32, i32, vp, i32, i32, i32, i32, i32]
        lib.kda_oracle_decode_step.restype = i32
        lib.kda_oracle_decode_step.argtypes = [vp, vp, vp, i32, vp, i32, vp, i32, vp, vp,
                                               i32, i32, i32, i32, i32, i32]
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _as_array(x):
    """Return (contiguous numpy array, dtype code) holding the exact values."""
    if x is None:
        return None, F64
    mod = type(x).__module__
    if mod.startswith("torch"):
        import torch  # local: only needed when torch tensors are passed

        t = x.detach()
        if t.device.type != "cpu":
            t = t.cpu()
        t = t.contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16), BF16
        if t.dtype == torch.float32:
            return t.numpy(), F32
        if t.dtype == torch.float64:
            return t.numpy(), F64
        raise TypeError(f"oracle: unsupported torch dtype {t.dtype}")
    a = np.ascontiguousarray(x)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.float64:
        return a, F64
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"oracle: unsupported dtype {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def forward(q, k, v, alpha, beta, S0=None, *, heads=None, order="page1",
            mutation=None, threads=None, col_block=None, want_o=True, want_state=True):
    """Token-by-token KDA over [B,T,H,d] inputs.

    Returns ``(o, S_T)``: ``o`` is float64 ``[n_sel, T, d_v]`` and ``S_T`` float64
    ``[n_sel, d_k, d_v]``, where the selected heads are ``heads`` (ids ``b*H+h``)
    or all ``B*H`` of them in ``(b, h)`` order.
    """
    qa, qd = _as_array(q)
    ka, kd = _as_array(k)
    va, vd = _as_array(v)
    if not (qd == kd == vd):
        raise TypeError("oracle: q, k, v must share a dtype")
    aa, ad = _as_array(alpha)
    ba, bd = _as_array(beta)
    sa, sd = _as_array(S0)
    B, T, H, dk = qa.shape
    dv = va.shape[-1]
    if ka.shape != (B, T, H, dk) or aa.shape != (B, T, H, dk):
        raise ValueError("oracle: k/alpha shape mismatch")
    if va.shape != (B, T, H, dv) or ba.shape != (B, T, H):
        raise ValueError("oracle: v/beta shape mismatch")
    if sa is not None and sa.shape != (B, H, dk, dv):
        raise ValueError("oracle: S0 shape mismatch")
    if heads is None:
        harr, n_sel = None, B * H
    else:
        harr = np.ascontiguousarray(np.asarray(heads, dtype=np.int32))
        n_sel = int(harr.size)
    o = np.zeros((n_sel, T, dv), np.float64) if want_o else None
    st = np.zeros((n_sel, dk, dv), np.float64) if want_state else None
    ordc = {"page1": ORDER_PAGE1, "literal_p2": ORDER_LITERAL_P2}[order]
    mut = 0 if mutation is None else MUTATIONS[mutation]
    threads = int(threads or default_threads())
    if col_block is None:
        # independent state columns: split them when there are fewer heads than threads
        col_block = dv
        while n_sel * -(-dv // col_block) < 2 * threads and col_block > 8:
            col_block //= 2
    rc = _load().kda_oracle_forward(
        _ptr(qa), _ptr(ka), _ptr(va), qd, _ptr(aa), ad, _ptr(ba), bd, _ptr(sa), sd,
        _ptr(o), _ptr(st), B, T, H, dk, dv, _ptr(harr), n_sel,
        int(col_block), ordc, mut, threads)
    if rc != 0:
        raise ValueError("oracle: kda_oracle_forward rejected its arguments")
    return o, st


def _widen(x):
    """Exact fp64 values of a bf16 (uint16 bits), fp32 or fp64 array or tensor."""
    a, code = _as_array(x)
    if code == BF16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def gate_alpha(z, A):
    """Per-channel retention from a gate pre-activation, the lower-bounded decay
    of section 3.5 of the "Kimi K3 Technical Report review" (jw9603.github.io):
    the log-decay is g = g_min * Sigmoid(e^A z) with g_min = -5, and alpha = e^g,
    so alpha lies in (e^-5, 1).

    z: [..., H, d_k] (bf16, fp32 or fp64; bf16 widened exactly); A: [H], one
    log-scale per head.  Returns float64 alpha with z's shape.
    """
    zz = _widen(z)
    aa = _widen(A)
    x = np.exp(aa)[:, None] * zz          # e^A z, A broadcast over the head axis
    s = 1.0 / (1.0 + np.exp(-x))          # Sigmoid
    return np.exp(-5.0 * s)


def decode_step(q, k, v, alpha, beta, S, *, threads=None, col_block=None):
    """One decode step over [B,H,d] inputs; ``S`` (float64 [B,H,d_k,d_v]) is updated
    in place.  Returns ``o`` as float64 ``[B, H, d_v]``."""
    qa, qd = _as_array(q)
    ka, _ = _as_array(k)
    va, _ = _as_array(v)
    aa, ad = _as_array(alpha)
    ba, bd = _as_array(beta)
    if not (isinstance(S, np.ndarray) and S.dtype == np.float64 and S.flags.c_contiguous):
        raise TypeError("oracle: S must be a C-contiguous float64 numpy array")
    B, H, dk = qa.shape
    dv = va.shape[-1]
    if S.shape != (B, H, dk, dv):
        raise ValueError("oracle: S shape mismatch")
    o = np.zeros((B, H, dv), np.float64)
    rc = _load().kda_oracle_decode_step(
        _ptr(qa), _ptr(ka), _ptr(va), qd, _ptr(aa), ad, _ptr(ba), bd, _ptr(S), _ptr(o),
        B, H, dk, dv, int(col_block or 0), int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle: kda_oracle_decode_step rejected its arguments")
    return o
