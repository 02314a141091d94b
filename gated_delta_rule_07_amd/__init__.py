"""Python binding for libkda, the MI355X-native Kimi Delta Attention operator.

Argument marshalling only: every step of the operator runs in the HIP kernels of
``libkda.so`` (built by ``gated_delta_rule_07_amd.build``), called through its C
ABI (``include/kda.h``).  PyTorch supplies device memory and the current HIP
stream; nothing here computes any part of the recurrence, and there is no CPU
fallback: if the library is missing the calls raise.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

import torch

__all__ = ["kda_chunk_fwd", "kda_chunk_fwd_snapshots", "kda_chunk_fwd_varlen", "kda_chunk_fwd_gated",
           "kda_chunk_fwd_split", "kda_chunk_fwd_split_plan", "kda_chunk_fwd_run_chunk",
           "kda_chunk_fwd_split_noalloc", "KDA_SPLIT_SCRATCH_BYTES",
           "kda_decode_step", "kda_decode_step_gated",
           "kda_decode_verify",
           "kda_decode_commit", "kda_status_string", "kda_version",
           "kda_last_hip_error", "library_path", "load_library", "bind", "KdaError",
           "KDA_F32", "KDA_BF16", "KDA_MAX_SNAPSHOTS", "KDA_MAX_DRAFT"]

KDA_F32, KDA_BF16 = 0, 1
KDA_MAX_SNAPSHOTS = 128
KDA_MAX_DRAFT = 16
KDA_SPLIT_SCRATCH_BYTES = 64 << 20
_PKG = Path(__file__).resolve().parent
_LIB_PATH = _PKG / "libkda.so"
_lib = None


class KdaError(RuntimeError):
    """A libkda call returned a non-OK status."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {kda_status_string(status)}")


def library_path() -> Path:
    return _LIB_PATH


def load_library():
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        raise RuntimeError(f"libkda is not built ({_LIB_PATH} missing); run "
                           "`python -m gated_delta_rule_07_amd.build` first")
    _lib = bind(_LIB_PATH)
    return _lib


def bind(path) -> ctypes.CDLL:
    """Open a build of the C ABI at `path` and declare its argument types."""
    lib = ctypes.CDLL(str(path))
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.kda_chunk_fwd.restype = i32
    lib.kda_chunk_fwd.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, i32, vp,
                                  i32, i32, i32, i32, i32, i32, vp]
    lib.kda_chunk_fwd_snapshots.restype = i32
    lib.kda_chunk_fwd_snapshots.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, i32, vp, vp, i32, vp,
                                            i32, i32, i32, i32, i32, i32, vp]
    lib.kda_decode_step.restype = i32
    lib.kda_decode_step.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.kda_chunk_fwd_varlen.restype = i32
    lib.kda_chunk_fwd_varlen.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, i32, vp, vp, i32, i32,
                                         i32, i32, i32, i32, vp]
    lib.kda_chunk_fwd_gated.restype = i32
    lib.kda_chunk_fwd_gated.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, vp, i32, vp,
                                        i32, i32, i32, i32, i32, i32, vp]
    sz = ctypes.c_size_t
    lib.kda_chunk_fwd_split_plan.restype = i32
    lib.kda_chunk_fwd_split_plan.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                             ctypes.POINTER(i32), ctypes.POINTER(sz)]
    lib.kda_chunk_fwd_split.restype = i32
    lib.kda_chunk_fwd_split.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, i32, vp,
                                        i32, i32, i32, i32, i32, i32, i32, i32, vp, sz, vp]
    lib.kda_chunk_fwd_split_noalloc.restype = i32
    lib.kda_chunk_fwd_split_noalloc.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, i32, vp,
                                                i32, i32, i32, i32, i32, i32, i32, i32, vp]
    lib.kda_decode_step_gated.restype = i32
    lib.kda_decode_step_gated.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.kda_decode_verify.restype = i32
    lib.kda_decode_verify.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, vp]
    lib.kda_decode_commit.restype = i32
    lib.kda_decode_commit.argtypes = [vp, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [i32]
    lib.kda_last_hip_error.restype = i32
    lib.kda_last_hip_error.argtypes = []
    lib.kda_version.restype = i32
    lib.kda_version.argtypes = []
    lib.kda_chunk_fwd_run_chunk.restype = i32
    lib.kda_chunk_fwd_run_chunk.argtypes = [i32, i32, i32, i32, i32, ctypes.POINTER(i32)]
    return lib


def kda_chunk_fwd_run_chunk(qkv_dtype, H, d_k, d_v, chunk: int = 64) -> int:
    """Tokens per chunk a ``kda_chunk_fwd`` call with these sizes runs."""
    code = KDA_BF16 if qkv_dtype == torch.bfloat16 else KDA_F32 if qkv_dtype == torch.float32 else -1
    run = ctypes.c_int(0)
    st = load_library().kda_chunk_fwd_run_chunk(code, int(H), int(d_k), int(d_v), int(chunk), ctypes.byref(run))
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd_run_chunk")
    return run.value


def kda_status_string(status: int) -> str:
    return load_library().kda_status_string(int(status)).decode()


def kda_version() -> int:
    return load_library().kda_version()


def kda_last_hip_error() -> int:
    return load_library().kda_last_hip_error()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"libkda: q/k/v must be bfloat16 or float32, got {t.dtype}")


def _check(t: torch.Tensor, name: str, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"libkda: {name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"libkda: {name} must be on a HIP device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"libkda: {name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"libkda: {name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"libkda: {name} must be {dtype}, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _prefill_prep(q, k, v, alpha, beta, S0, o, S_T, o_dtype, want_state):
    _check(q, "q")
    dev = q.device
    for t, n in ((k, "k"), (v, "v")):
        _check(t, n, q.dtype, dev)
    if alpha is not None:  # None: the gated call, which checks z and A itself
        _check(alpha, "alpha", torch.float32, dev)
    _check(beta, "beta", torch.float32, dev)
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("libkda: q/k/v must be [B,T,H,d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if (k.shape != q.shape or (alpha is not None and alpha.shape != q.shape) or v.shape[:3] != q.shape[:3]
            or beta.shape != (B, T, H)):
        raise ValueError("libkda: inconsistent shapes")
    if S0 is not None:
        _check(S0, "S0", torch.float32, dev)
        if S0.shape != (B, H, dk, dv):
            raise ValueError("libkda: S0 must be [B,H,d_k,d_v]")
    if o is None:
        o = torch.empty(B, T, H, dv, device=dev, dtype=o_dtype)
    else:
        _check(o, "o", None, dev)
        if o.shape != (B, T, H, dv):
            raise ValueError("libkda: o must be [B,T,H,d_v]")
    if want_state and S_T is None:
        S_T = torch.empty(B, H, dk, dv, device=dev, dtype=torch.float32)
    elif S_T is not None:
        _check(S_T, "S_T", torch.float32, dev)
        if S_T.shape != (B, H, dk, dv):
            raise ValueError("libkda: S_T must be [B,H,d_k,d_v]")
    return dev, (B, T, H, dk, dv), o, S_T


def kda_chunk_fwd(q, k, v, alpha, beta, S0=None, *, chunk: int = 64, o=None, S_T=None,
                  o_dtype=torch.float32, want_state: bool = True, stream=None):
    """Prefill: returns ``(o, S_T)`` (``S_T`` is None when ``want_state`` is False).

    q, k: [B,T,H,d_k]; v: [B,T,H,d_v] (bf16 or fp32, same dtype); alpha: [B,T,H,d_k]
    fp32; beta: [B,T,H] fp32; S0: [B,H,d_k,d_v] fp32 or None (zeros).  ``o`` is
    float32 (default) or bfloat16 (``o_dtype``, or the dtype of a preallocated
    ``o``).  ``S_T`` may be preallocated (it may be ``S0`` for an in-place update).
    """
    lib = load_library()
    dev, (B, T, H, dk, dv), o, S_T = _prefill_prep(q, k, v, alpha, beta, S0, o, S_T, o_dtype, want_state)
    st = lib.kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(alpha), _ptr(beta),
                           _ptr(S0), _ptr(o), _dtype_code(o), _ptr(S_T), B, T, H, dk, dv, int(chunk),
                           _stream(dev, stream))
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd")
    return o, S_T


def kda_chunk_fwd_snapshots(q, k, v, alpha, beta, S0=None, *, snap_tokens, chunk: int = 64, o=None,
                            S_T=None, snaps=None, o_dtype=torch.float32, want_state: bool = True,
                            stream=None):
    """Prefill that also records the state after each count in ``snap_tokens``.

    Returns ``(o, S_T, snaps)`` with ``snaps`` [B,H,len(snap_tokens),d_k,d_v] fp32:
    ``snaps[:, :, j]`` is the state after the first ``snap_tokens[j]`` tokens.  The
    counts must be strictly increasing, in [1, T], and multiples of ``chunk`` (or T);
    at most ``KDA_MAX_SNAPSHOTS`` of them.  Other arguments as ``kda_chunk_fwd``.
    """
    lib = load_library()
    dev, (B, T, H, dk, dv), o, S_T = _prefill_prep(q, k, v, alpha, beta, S0, o, S_T, o_dtype, want_state)
    pos = [int(t) for t in snap_tokens]
    n = len(pos)
    if snaps is None:
        snaps = torch.empty(B, H, n, dk, dv, device=dev, dtype=torch.float32)
    else:
        _check(snaps, "snaps", torch.float32, dev)
        if snaps.shape != (B, H, n, dk, dv):
            raise ValueError("libkda: snaps must be [B,H,n_snap,d_k,d_v]")
    arr = (ctypes.c_int * max(n, 1))(*pos)
    st = lib.kda_chunk_fwd_snapshots(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(alpha), _ptr(beta),
                                     _ptr(S0), _ptr(o), _dtype_code(o), _ptr(S_T), arr, n,
                                     _ptr(snaps) if n > 0 else None, B, T, H, dk, dv, int(chunk),
                                     _stream(dev, stream))
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd_snapshots")
    return o, S_T, snaps


def kda_chunk_fwd_varlen(q, k, v, alpha, beta, cu_seqlens, S0=None, *, chunk: int = 64, o=None, S_T=None,
                         o_dtype=torch.float32, want_state: bool = True, stream=None):
    """Prefill over a packed batch: returns ``(o, S_T)``.

    q, k, alpha: [total_T,H,d_k]; v: [total_T,H,d_v]; beta: [total_T,H];
    cu_seqlens: int32 [N+1] on the device (sequence b is rows cu[b]..cu[b+1]);
    S0: [N,H,d_k,d_v] fp32 or None.  o: [total_T,H,d_v]; S_T: [N,H,d_k,d_v].
    """
    lib = load_library()
    _check(cu_seqlens, "cu_seqlens", torch.int32, q.device if isinstance(q, torch.Tensor) else None)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("libkda: cu_seqlens must be [N+1] with N >= 1")
    N = cu_seqlens.numel() - 1
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("libkda: packed q/k/v must be [total_T,H,d]")
    if S0 is not None and S0.shape[0] != N:
        raise ValueError("libkda: S0 must be [N,H,d_k,d_v]")
    if S_T is not None and S_T.shape[0] != N:
        raise ValueError("libkda: S_T must be [N,H,d_k,d_v]")
    # the packed rows are one [1,total_T,...] batch for the shared checks
    dev, (_, T, H, dk, dv), o4, _ = _prefill_prep(q[None], k[None], v[None], alpha[None], beta[None], None,
                                                  None if o is None else o[None], None, o_dtype, False)
    if S0 is not None:
        _check(S0, "S0", torch.float32, dev)
        if S0.shape != (N, H, dk, dv):
            raise ValueError("libkda: S0 must be [N,H,d_k,d_v]")
    if want_state and S_T is None:
        S_T = torch.empty(N, H, dk, dv, device=dev, dtype=torch.float32)
    elif S_T is not None:
        _check(S_T, "S_T", torch.float32, dev)
        if S_T.shape != (N, H, dk, dv):
            raise ValueError("libkda: S_T must be [N,H,d_k,d_v]")
    st = lib.kda_chunk_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(alpha), _ptr(beta), _ptr(S0),
                                  _ptr(o4), _dtype_code(o4), _ptr(S_T), _ptr(cu_seqlens), N, T, H, dk, dv,
                                  int(chunk), _stream(dev, stream))
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd_varlen")
    return o4[0], S_T


def kda_chunk_fwd_gated(q, k, v, z, A, beta, S0=None, *, chunk: int = 64, o=None, S_T=None,
                        o_dtype=torch.float32, want_state: bool = True, stream=None):
    """Prefill with the gate fused in: alpha = exp(-5 sigmoid(e^A z)) is formed in
    the kernels.  z: [B,T,H,d_k] in q's dtype; A: [H] fp32.  Returns ``(o, S_T)``;
    other arguments as ``kda_chunk_fwd``."""
    lib = load_library()
    dev, (B, T, H, dk, dv), o, S_T = _prefill_prep(q, k, v, None, beta, S0, o, S_T, o_dtype, want_state)
    _check(z, "z", q.dtype, dev)
    _check(A, "A", torch.float32, dev)
    if z.shape != q.shape or A.shape != (H,):
        raise ValueError("libkda: z must be shaped like q and A must be [H]")
    st = lib.kda_chunk_fwd_gated(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(z), _ptr(A), _ptr(beta),
                                 _ptr(S0), _ptr(o), _dtype_code(o), _ptr(S_T), B, T, H, dk, dv, int(chunk),
                                 _stream(dev, stream))
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd_gated")
    return o, S_T


def kda_chunk_fwd_split_plan(qkv_dtype, B, T, H, d_k, d_v, *, chunk: int = 64, parts: int = 0,
                             num_cus: int = 0):
    """``(parts, workspace_bytes)`` a split prefill of this shape would use
    (``parts`` 0: the library's choice for ``num_cus`` compute units, 0: the
    current device's)."""
    lib = load_library()
    code = KDA_BF16 if qkv_dtype == torch.bfloat16 else KDA_F32 if qkv_dtype == torch.float32 else -1
    n, ws = ctypes.c_int(0), ctypes.c_size_t(0)
    st = lib.kda_chunk_fwd_split_plan(code, B, T, H, d_k, d_v, int(chunk), int(parts), int(num_cus),
                                      ctypes.byref(n), ctypes.byref(ws))
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd_split_plan")
    return n.value, ws.value


def kda_chunk_fwd_split(q, k, v, alpha, beta, S0=None, *, parts: int = 0, num_cus: int = 0, chunk: int = 64,
                        o=None, S_T=None, workspace=None, o_dtype=torch.float32, want_state: bool = True,
                        stream=None):
    """Prefill with every sequence split into parts that run side by side (a
    two-level scan over the parts).  ``parts`` 0: the library's choice; the
    workspace (a uint8 device tensor) is allocated here when not given.  Returns
    ``(o, S_T)``; other arguments as ``kda_chunk_fwd``."""
    lib = load_library()
    dev, (B, T, H, dk, dv), o, S_T = _prefill_prep(q, k, v, alpha, beta, S0, o, S_T, o_dtype, want_state)
    n, need = kda_chunk_fwd_split_plan(q.dtype, B, T, H, dk, dv, chunk=chunk, parts=parts, num_cus=num_cus)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _check(workspace, "workspace", torch.uint8, dev)
    st = lib.kda_chunk_fwd_split(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(alpha), _ptr(beta),
                                 _ptr(S0), _ptr(o), _dtype_code(o), _ptr(S_T), B, T, H, dk, dv, int(chunk),
                                 n, 0, _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                 _stream(dev, stream))
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd_split")
    return o, S_T


def kda_chunk_fwd_split_noalloc(q, k, v, alpha, beta, S0=None, *, parts: int = 0, num_cus: int = 0,
                                chunk: int = 64, o=None, S_T=None, o_dtype=torch.float32, want_state: bool = True,
                                stream=None):
    """The split prefill with its workspace in the library's fixed per-GPU scratch
    array (``KDA_SPLIT_SCRATCH_BYTES``): the C call allocates nothing.  Pass
    preallocated ``o`` and ``S_T`` to keep this wrapper from allocating them.
    Calls that overlap on one GPU race.  Returns ``(o, S_T)``; other arguments as
    ``kda_chunk_fwd_split``."""
    lib = load_library()
    dev, (B, T, H, dk, dv), o, S_T = _prefill_prep(q, k, v, alpha, beta, S0, o, S_T, o_dtype, want_state)
    st = lib.kda_chunk_fwd_split_noalloc(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(alpha), _ptr(beta),
                                         _ptr(S0), _ptr(o), _dtype_code(o), _ptr(S_T), B, T, H, dk, dv, int(chunk),
                                         int(parts), int(num_cus), _stream(dev, stream))
    if st != 0:
        raise KdaError(st, "kda_chunk_fwd_split_noalloc")
    return o, S_T


def kda_decode_step_gated(q, k, v, z, A, beta, S, *, o=None, o_dtype=torch.float32, stream=None):
    """Decode with the gate fused in.  z: [B,H,d_k] in q's dtype; A: [H] fp32; the
    rest as ``kda_decode_step``.  Returns ``o``."""
    lib = load_library()
    _check(q, "q")
    dev = q.device
    for t, n in ((k, "k"), (v, "v"), (z, "z")):
        _check(t, n, q.dtype, dev)
    _check(A, "A", torch.float32, dev)
    _check(beta, "beta", torch.float32, dev)
    _check(S, "S", torch.float32, dev)
    if q.dim() != 3:
        raise ValueError("libkda: decode q/k/v must be [B,H,d]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or z.shape != q.shape or v.shape[:2] != (B, H) or beta.shape != (B, H) or A.shape != (H,):
        raise ValueError("libkda: inconsistent shapes")
    if S.shape != (B, H, dk, dv):
        raise ValueError("libkda: S must be [B,H,d_k,d_v]")
    if o is None:
        o = torch.empty(B, H, dv, device=dev, dtype=o_dtype)
    else:
        _check(o, "o", None, dev)
        if o.shape != (B, H, dv):
            raise ValueError("libkda: o must be [B,H,d_v]")
    st = lib.kda_decode_step_gated(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(z), _ptr(A), _ptr(beta),
                                   _ptr(S), _ptr(o), _dtype_code(o), B, H, dk, dv, _stream(dev, stream))
    if st != 0:
        raise KdaError(st, "kda_decode_step_gated")
    return o


def kda_decode_step(q, k, v, alpha, beta, S, *, o=None, o_dtype=torch.float32, stream=None):
    """Decode one token per (sequence, head); ``S`` ([B,H,d_k,d_v] fp32) is updated
    in place.  q, k: [B,H,d_k]; v: [B,H,d_v]; alpha: [B,H,d_k]; beta: [B,H].
    Returns ``o`` ([B,H,d_v], float32 by default or bfloat16)."""
    lib = load_library()
    _check(q, "q")
    dev = q.device
    for t, n in ((k, "k"), (v, "v")):
        _check(t, n, q.dtype, dev)
    _check(alpha, "alpha", torch.float32, dev)
    _check(beta, "beta", torch.float32, dev)
    _check(S, "S", torch.float32, dev)
    if q.dim() != 3:
        raise ValueError("libkda: decode q/k/v must be [B,H,d]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or alpha.shape != q.shape or v.shape[:2] != (B, H) or beta.shape != (B, H):
        raise ValueError("libkda: inconsistent shapes")
    if S.shape != (B, H, dk, dv):
        raise ValueError("libkda: S must be [B,H,d_k,d_v]")
    if o is None:
        o = torch.empty(B, H, dv, device=dev, dtype=o_dtype)
    else:
        _check(o, "o", None, dev)
        if o.shape != (B, H, dv):
            raise ValueError("libkda: o must be [B,H,d_v]")
    st = lib.kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(alpha), _ptr(beta),
                             _ptr(S), _ptr(o), _dtype_code(o), B, H, dk, dv, _stream(dev, stream))
    if st != 0:
        raise KdaError(st, "kda_decode_step")
    return o


def kda_decode_verify(q, k, v, alpha, beta, S, *, o=None, u=None, o_dtype=torch.float32, stream=None):
    """Speculative decoding, pass 1: apply K draft tokens per (sequence, head)
    without changing ``S``.  q, k: [B,K,H,d_k]; v: [B,K,H,d_v]; alpha: [B,K,H,d_k];
    beta: [B,K,H]; S: [B,H,d_k,d_v] fp32 (read only).  Returns ``(o, u)``: o
    [B,K,H,d_v] (o_t as if the first t drafts were accepted) and u [B,H,K,d_v]
    fp32, the write vectors ``kda_decode_commit`` needs."""
    lib = load_library()
    _check(q, "q")
    dev = q.device
    for t, n in ((k, "k"), (v, "v")):
        _check(t, n, q.dtype, dev)
    _check(alpha, "alpha", torch.float32, dev)
    _check(beta, "beta", torch.float32, dev)
    _check(S, "S", torch.float32, dev)
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("libkda: draft q/k/v must be [B,K,H,d]")
    B, K, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or alpha.shape != q.shape or v.shape[:3] != q.shape[:3] or beta.shape != (B, K, H):
        raise ValueError("libkda: inconsistent shapes")
    if S.shape != (B, H, dk, dv):
        raise ValueError("libkda: S must be [B,H,d_k,d_v]")
    if o is None:
        o = torch.empty(B, K, H, dv, device=dev, dtype=o_dtype)
    else:
        _check(o, "o", None, dev)
        if o.shape != (B, K, H, dv):
            raise ValueError("libkda: o must be [B,K,H,d_v]")
    if u is None:
        u = torch.empty(B, H, K, dv, device=dev, dtype=torch.float32)
    else:
        _check(u, "u", torch.float32, dev)
        if u.shape != (B, H, K, dv):
            raise ValueError("libkda: u must be [B,H,K,d_v]")
    st = lib.kda_decode_verify(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(alpha), _ptr(beta), _ptr(S),
                               _ptr(o), _dtype_code(o), _ptr(u), B, K, H, dk, dv, _stream(dev, stream))
    if st != 0:
        raise KdaError(st, "kda_decode_verify")
    return o, u


def kda_decode_commit(k, alpha, u, n_accept, S, *, stream=None):
    """Speculative decoding, pass 2: advance ``S`` in place over the accepted
    drafts, ``n_accept[b]`` of them for sequence b (int32 [B] on the device,
    clamped to [0, K]).  k, alpha: the drafts' [B,K,H,d_k] inputs of
    ``kda_decode_verify``; u: its [B,H,K,d_v] output.  Returns ``S``."""
    lib = load_library()
    _check(k, "k")
    dev = k.device
    _check(alpha, "alpha", torch.float32, dev)
    _check(u, "u", torch.float32, dev)
    _check(n_accept, "n_accept", torch.int32, dev)
    _check(S, "S", torch.float32, dev)
    if k.dim() != 4:
        raise ValueError("libkda: draft k must be [B,K,H,d_k]")
    B, K, H, dk = k.shape
    dv = S.shape[-1]
    if alpha.shape != k.shape or S.shape != (B, H, dk, dv) or u.shape != (B, H, K, dv) or n_accept.shape != (B,):
        raise ValueError("libkda: inconsistent shapes")
    st = lib.kda_decode_commit(_ptr(k), _dtype_code(k), _ptr(alpha), _ptr(u), _ptr(n_accept), _ptr(S),
                               B, K, H, dk, dv, _stream(dev, stream))
    if st != 0:
        raise KdaError(st, "kda_decode_commit")
    return S
