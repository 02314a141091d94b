"""CPU checks of the libkda boundary: the header compiles as C, the library
exports every declared symbol, and argument validation rejects bad calls with
the documented status codes before any HIP call is made (so these run without a
GPU; the pointers below are fake, aligned addresses that are never touched)."""
import ctypes
import re
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "kda.h"


def _lib():
    import gated_delta_rule_07_amd as kda
    if not kda.library_path().exists():
        pytest.skip("libkda.so not built")
    return kda.load_library()


def _declared():
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\*?\s+\*?(kda_[a-z_]+)\(", text, re.M)))


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-D__HIP_PLATFORM_AMD__",
                        "-I/opt/rocm/include", "-x", "c", str(HEADER)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_stream_arguments_are_hip_streams():
    """Every call that enqueues work takes its stream as a hipStream_t."""
    text = HEADER.read_text()
    assert "void* stream" not in text
    assert text.count("hipStream_t stream") >= 9


def test_product_library_has_no_test_switches():
    """Kernel choice never depends on the caller's environment or on a test hook:
    the product library reads no KDA_* variable and exports no test entry point
    (those live in libkda_testhooks.so only)."""
    lib = _lib()
    assert not hasattr(lib, "kda_test_force_prefill")
    blob = (ROOT / "gated_delta_rule_07_amd" / "libkda.so").read_bytes()
    assert b"KDA_PREFILL" not in blob
    for src in (ROOT / "gated_delta_rule_07_amd" / "csrc").glob("*"):
        text = src.read_text()
        assert "getenv" not in text, f"{src.name} reads the environment"
        assert "KDA_PHASE_MARK" not in text and "KDA_STEP_MARK" not in text, f"{src.name} carries timing hooks"
    hooks = ROOT / "gated_delta_rule_07_amd" / "libkda_testhooks.so"
    if hooks.exists():
        assert hasattr(ctypes.CDLL(str(hooks)), "kda_test_force_prefill")


def _run_chunk(lib, dtype, dk, dv, chunk, H=8):
    r = ctypes.c_int(-1)
    return lib.kda_chunk_fwd_run_chunk(dtype, H, dk, dv, chunk, ctypes.byref(r)), r.value


@pytest.mark.parametrize("dtype,dk,dv,chunk,want", [
    (1, 128, 128, 64, 32), (1, 128, 128, 32, 32), (1, 64, 64, 64, 32),   # the pipelined kernel
    (1, 128, 128, 16, 16), (1, 32, 32, 64, 64), (1, 16, 128, 32, 32),    # the generic kernel
    (1, 128, 16, 64, 64),                                                # d_v not a multiple of 32
    (0, 16, 16, 64, 64), (0, 32, 32, 32, 32),                            # fp32
    (0, 64, 64, 64, 32), (0, 128, 128, 64, 32), (0, 128, 128, 16, 16), (0, 128, 64, 32, 32),
])
def test_run_chunk(dtype, dk, dv, chunk, want):
    """The chunk size each supported call runs, including fp32 at every head size."""
    assert _run_chunk(_lib(), dtype, dk, dv, chunk) == (0, want)


def test_run_chunk_invalid():
    lib = _lib()
    assert _run_chunk(lib, 1, 48, 128, 64)[0] == 4
    assert _run_chunk(lib, 0, 128, 128, 48)[0] == 4
    assert _run_chunk(lib, 2, 128, 128, 64)[0] == 3
    assert _run_chunk(lib, 1, 128, 128, 64, H=0)[0] == 2
    assert lib.kda_chunk_fwd_run_chunk(1, 8, 128, 128, 64, None) == 1


def test_exports_every_declared_symbol():
    names = _declared()
    assert {"kda_chunk_fwd", "kda_decode_step", "kda_status_string", "kda_last_hip_error",
            "kda_version"} <= set(names)
    lib = _lib()
    for n in names:
        assert hasattr(lib, n), f"libkda.so does not export {n}"
    out = subprocess.run(["nm", "-D", "--defined-only", str(ROOT / "gated_delta_rule_07_amd" / "libkda.so")],
                         capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}\b", out), f"{n} is not a defined text symbol"


def test_status_strings_and_version():
    lib = _lib()
    for code in range(8):
        s = lib.kda_status_string(code).decode()
        assert s.startswith("KDA_")
    assert lib.kda_status_string(99).decode().startswith("KDA")
    assert lib.kda_version() >= 100
    assert lib.kda_last_hip_error() == 0


BASE = 1 << 40  # fake device addresses, 16-byte aligned, never dereferenced


def _addr(i):
    return ctypes.c_void_p(BASE + i * (1 << 32))


def _prefill(lib, **over):
    a = dict(q=_addr(0), k=_addr(1), v=_addr(2), dtype=1, alpha=_addr(3), beta=_addr(4), S0=_addr(5),
             o=_addr(6), odt=0, S_T=_addr(7), B=1, T=64, H=2, dk=128, dv=128, chunk=64)
    a.update(over)
    return lib.kda_chunk_fwd(a["q"], a["k"], a["v"], a["dtype"], a["alpha"], a["beta"], a["S0"], a["o"],
                             a["odt"], a["S_T"], a["B"], a["T"], a["H"], a["dk"], a["dv"], a["chunk"], None)


def _decode(lib, **over):
    a = dict(q=_addr(0), k=_addr(1), v=_addr(2), dtype=1, alpha=_addr(3), beta=_addr(4), S=_addr(5),
             o=_addr(6), odt=0, B=4, H=2, dk=128, dv=128)
    a.update(over)
    return lib.kda_decode_step(a["q"], a["k"], a["v"], a["dtype"], a["alpha"], a["beta"], a["S"], a["o"],
                               a["odt"], a["B"], a["H"], a["dk"], a["dv"], None)


@pytest.mark.parametrize("over,code", [
    (dict(dtype=7), 3), (dict(odt=9), 3),
    (dict(B=0), 2), (dict(H=0), 2), (dict(T=-1), 2),
    (dict(dk=48), 4), (dict(dv=256), 4), (dict(chunk=48), 4), (dict(chunk=128), 4),
    (dict(dtype=0, dk=128, chunk=48), 4),  # fp32 at d_k = 128 is built, chunk 48 is not
    (dict(q=None), 1), (dict(o=None), 1), (dict(beta=None), 1),
    (dict(k=ctypes.c_void_p(BASE + 8)), 5), (dict(S_T=ctypes.c_void_p(BASE + (7 << 32) + 4)), 5),
    (dict(o=_addr(0)), 6),                       # o aliases q
    (dict(S_T=_addr(1)), 6),                     # S_T aliases k
    (dict(S_T=ctypes.c_void_p(BASE + (5 << 32) + 16)), 6),  # S_T partially overlaps S0
])
def test_prefill_validation(over, code):
    assert _prefill(_lib(), **over) == code


@pytest.mark.parametrize("over,code", [
    (dict(dtype=2), 3), (dict(odt=-1), 3), (dict(B=0), 2), (dict(H=-3), 2),
    (dict(dk=8), 4), (dict(dv=100), 4),
    (dict(S=None), 1), (dict(o=None), 1),
    (dict(v=ctypes.c_void_p(BASE + (2 << 32) + 2)), 5),
    (dict(o=_addr(5)), 6),                       # o aliases the state
    (dict(S=_addr(3)), 6),                       # state aliases alpha
])
def test_decode_validation(over, code):
    assert _decode(_lib(), **over) == code


def _snap(lib, pos, n=None, snaps=_addr(8), **over):
    a = dict(q=_addr(0), k=_addr(1), v=_addr(2), dtype=1, alpha=_addr(3), beta=_addr(4), S0=_addr(5),
             o=_addr(6), odt=0, S_T=_addr(7), B=1, T=300, H=2, dk=128, dv=128, chunk=64)
    a.update(over)
    arr = None if pos is None else (ctypes.c_int * max(1, len(pos)))(*pos)
    n = (len(pos) if pos is not None else 1) if n is None else n
    return lib.kda_chunk_fwd_snapshots(a["q"], a["k"], a["v"], a["dtype"], a["alpha"], a["beta"], a["S0"],
                                       a["o"], a["odt"], a["S_T"], arr, n, snaps, a["B"], a["T"], a["H"],
                                       a["dk"], a["dv"], a["chunk"], None)


@pytest.mark.parametrize("pos,over,code", [
    ([64, 64], {}, 2),             # not strictly increasing
    ([128, 64], {}, 2),            # decreasing
    ([0], {}, 2),                  # before the first token
    ([320], {}, 2),                # past T
    ([100], {}, 2),                # not a multiple of the chunk, not T
    ([32], {}, 2),                 # multiple of 32 but chunk is 64
    (list(range(64, 64 * 130, 64)), dict(T=64 * 130), 2),  # more than KDA_MAX_SNAPSHOTS
    (None, {}, 1),                 # n_snap > 0 without a list
    ([64], dict(snaps=None), 1),   # no snapshot buffer
    ([64], dict(snaps=ctypes.c_void_p(BASE + (8 << 32) + 8)), 5),
    ([64], dict(snaps=_addr(6)), 6),   # snapshots alias o
    ([64], dict(snaps=_addr(7)), 6),   # snapshots alias S_T
    ([64], dict(snaps=_addr(3)), 6),   # snapshots alias alpha
    ([64], dict(snaps=_addr(5)), 6),   # snapshots alias S0
    ([64], dict(dtype=5), 3),          # the checks of kda_chunk_fwd still apply
])
def test_snapshot_validation(pos, over, code):
    lib = _lib()
    snaps = over.pop("snaps", _addr(8))
    assert _snap(lib, pos, snaps=snaps, **over) == code


def test_snapshot_negative_count_and_empty_list():
    lib = _lib()
    assert _snap(lib, [64], n=-1) == 2
    # n_snap = 0 with no list and no buffer is a plain prefill call: validation passes up
    # to the launch, which needs a device, so only the argument checks are exercised here
    assert _snap(lib, None, n=0, snaps=None, dtype=9) == 3


def _varlen(lib, **over):
    a = dict(q=_addr(0), k=_addr(1), v=_addr(2), dtype=1, alpha=_addr(3), beta=_addr(4), S0=_addr(5),
             o=_addr(6), odt=0, S_T=_addr(7), cu=_addr(8), N=3, T=300, H=2, dk=128, dv=128, chunk=64)
    a.update(over)
    return lib.kda_chunk_fwd_varlen(a["q"], a["k"], a["v"], a["dtype"], a["alpha"], a["beta"], a["S0"], a["o"],
                                    a["odt"], a["S_T"], a["cu"], a["N"], a["T"], a["H"], a["dk"], a["dv"],
                                    a["chunk"], None)


@pytest.mark.parametrize("over,code", [
    (dict(cu=None), 1), (dict(q=None), 1),
    (dict(N=0), 2), (dict(T=-5), 2), (dict(H=0), 2),
    (dict(dk=12), 4), (dict(chunk=8), 4), (dict(dtype=4), 3),
    (dict(cu=ctypes.c_void_p(BASE + (8 << 32) + 4)), 5),
    (dict(cu=_addr(6)), 6),   # offsets alias o
    (dict(cu=_addr(7)), 6),   # offsets alias S_T
    (dict(o=_addr(3)), 6),    # o aliases alpha
])
def test_varlen_validation(over, code):
    assert _varlen(_lib(), **over) == code


def _gated(lib, **over):
    a = dict(q=_addr(0), k=_addr(1), v=_addr(2), dtype=1, z=_addr(3), A=_addr(9), beta=_addr(4), S0=_addr(5),
             o=_addr(6), odt=0, S_T=_addr(7), B=1, T=64, H=2, dk=128, dv=128, chunk=64)
    a.update(over)
    return lib.kda_chunk_fwd_gated(a["q"], a["k"], a["v"], a["dtype"], a["z"], a["A"], a["beta"], a["S0"], a["o"],
                                   a["odt"], a["S_T"], a["B"], a["T"], a["H"], a["dk"], a["dv"], a["chunk"], None)


def _dgated(lib, **over):
    a = dict(q=_addr(0), k=_addr(1), v=_addr(2), dtype=1, z=_addr(3), A=_addr(9), beta=_addr(4), S=_addr(5),
             o=_addr(6), odt=0, B=4, H=2, dk=128, dv=128)
    a.update(over)
    return lib.kda_decode_step_gated(a["q"], a["k"], a["v"], a["dtype"], a["z"], a["A"], a["beta"], a["S"],
                                     a["o"], a["odt"], a["B"], a["H"], a["dk"], a["dv"], None)


@pytest.mark.parametrize("over,code", [
    (dict(z=None), 1), (dict(A=None), 1), (dict(q=None), 1),
    (dict(dtype=7), 3), (dict(B=0), 2), (dict(dk=40), 4),
    (dict(z=ctypes.c_void_p(BASE + (3 << 32) + 2)), 5), (dict(A=ctypes.c_void_p(BASE + (9 << 32) + 4)), 5),
    (dict(o=_addr(3)), 6),     # o aliases z
    (dict(S_T=_addr(9)), 6),   # S_T aliases A
])
def test_gated_prefill_validation(over, code):
    assert _gated(_lib(), **over) == code


@pytest.mark.parametrize("over,code", [
    (dict(z=None), 1), (dict(A=None), 1), (dict(dtype=2), 3), (dict(H=0), 2), (dict(dv=24), 4),
    (dict(z=ctypes.c_void_p(BASE + (3 << 32) + 8)), 5),
    (dict(o=_addr(9)), 6),     # o aliases A
    (dict(S=_addr(3)), 6),     # state aliases z
])
def test_gated_decode_validation(over, code):
    assert _dgated(_lib(), **over) == code


def _verify(lib, **over):
    a = dict(q=_addr(0), k=_addr(1), v=_addr(2), dtype=1, alpha=_addr(3), beta=_addr(4), S=_addr(5),
             o=_addr(6), odt=0, u=_addr(7), B=4, K=4, H=2, dk=128, dv=128)
    a.update(over)
    return lib.kda_decode_verify(a["q"], a["k"], a["v"], a["dtype"], a["alpha"], a["beta"], a["S"], a["o"],
                                 a["odt"], a["u"], a["B"], a["K"], a["H"], a["dk"], a["dv"], None)


def _commit(lib, **over):
    a = dict(k=_addr(1), dtype=1, alpha=_addr(3), u=_addr(7), n=_addr(8), S=_addr(5), B=4, K=4, H=2, dk=128, dv=128)
    a.update(over)
    return lib.kda_decode_commit(a["k"], a["dtype"], a["alpha"], a["u"], a["n"], a["S"], a["B"], a["K"], a["H"],
                                 a["dk"], a["dv"], None)


@pytest.mark.parametrize("over,code", [
    (dict(dtype=3), 3), (dict(odt=2), 3),
    (dict(K=0), 2), (dict(K=17), 2), (dict(B=0), 2),
    (dict(dk=24), 4), (dict(dv=512), 4),
    (dict(u=None), 1), (dict(S=None), 1), (dict(beta=None), 1),
    (dict(u=ctypes.c_void_p(BASE + (7 << 32) + 4)), 5),
    (dict(o=_addr(5)), 6),   # o aliases the state
    (dict(u=_addr(0)), 6),   # u aliases q
    (dict(u=_addr(6)), 6),   # u aliases o
])
def test_verify_validation(over, code):
    assert _verify(_lib(), **over) == code


@pytest.mark.parametrize("over,code", [
    (dict(dtype=-1), 3), (dict(K=0), 2), (dict(K=99), 2), (dict(H=0), 2), (dict(dk=100), 4),
    (dict(n=None), 1), (dict(S=None), 1), (dict(u=None), 1),
    (dict(n=ctypes.c_void_p(BASE + (8 << 32) + 4)), 5),
    (dict(S=_addr(7)), 6),   # state aliases u
    (dict(S=_addr(8)), 6),   # state aliases the accepted counts
    (dict(S=_addr(1)), 6),   # state aliases k
])
def test_commit_validation(over, code):
    assert _commit(_lib(), **over) == code


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    import gated_delta_rule_07_amd as kda
    if not kda.library_path().exists():
        pytest.skip("libkda.so not built")
    x = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        kda.kda_chunk_fwd(x, x, x, x, torch.zeros(1, 4, 1))


def test_gated_decode_binding_checks_o_before_any_launch(monkeypatch):
    """A caller-supplied o of the wrong shape is refused by the binding before the
    C ABI is reached (the ABI trusts B, H and d_v, so a small o would be written
    out of bounds).  The device checks are lifted so CPU tensors reach the shape
    check, and the library is replaced by one that fails if anything is called."""
    torch = pytest.importorskip("torch")
    import gated_delta_rule_07_amd as kda

    class NoLaunch:
        def __getattr__(self, name):
            raise AssertionError(f"{name} was called")

    def cpu_check(t, name, dtype=None, device=None):
        if dtype is not None and t.dtype != dtype:
            raise TypeError(name)

    monkeypatch.setattr(kda, "_check", cpu_check)
    monkeypatch.setattr(kda, "load_library", lambda: NoLaunch())
    B, H, d = 4, 2, 16
    q = torch.zeros(B, H, d, dtype=torch.bfloat16)
    A, beta, S = torch.zeros(H), torch.zeros(B, H), torch.zeros(B, H, d, d)
    for bad in (torch.zeros(B, H, d // 2), torch.zeros(B * H * d), torch.zeros(B, H + 1, d)):
        with pytest.raises(ValueError, match="o must be"):
            kda.kda_decode_step_gated(q, q, q, q, A, beta, S, o=bad)
        with pytest.raises(ValueError, match="o must be"):
            kda.kda_decode_step(q, q, q, torch.zeros(B, H, d), beta, S, o=bad)


def test_product_path_does_not_import_the_oracle():
    """The HIP product package never imports or links the oracle."""
    pkg = ROOT / "gated_delta_rule_07_amd"
    for f in [*pkg.rglob("*.py"), *pkg.rglob("*.hip"), *pkg.rglob("*.cpp"), *pkg.rglob("*.h")]:
        text = f.read_text()
        for bad in ("import oracle", "from oracle", "kda_oracle"):
            assert bad not in text, f"{f} mentions {bad}"


def _plan(lib, dtype=1, B=1, T=4096, H=8, dk=128, dv=128, chunk=64, parts=0, cus=256):
    n, ws = ctypes.c_int(-1), ctypes.c_size_t(0)
    st = lib.kda_chunk_fwd_split_plan(dtype, B, T, H, dk, dv, chunk, parts, cus, ctypes.byref(n), ctypes.byref(ws))
    return st, n.value, ws.value


TREE_PARTS = 9  # part counts from which the combine is a tree (a second (N | M) buffer)


def _ws_bytes(P, B=1, H=8, dk=128, dv=128):
    trans = (P - 1) * (dv + dk) * (2 if P >= TREE_PARTS else 1)
    return 4 * B * H * dk * (trans + P * dv)


def test_split_plan_choices():
    """The part count the library picks for 256 compute units, and the workspace
    it asks for (host logic only: an explicit compute-unit count makes no HIP call)."""
    lib = _lib()
    # 32 chains of 128 chunks: the single pass (its chain steps are short) is not beaten
    assert _plan(lib, B=1, T=4096, H=8) == (0, 1, 0)
    st, n, ws = _plan(lib, B=1, T=16384, H=2)     # 8 chains of 512 chunks: split
    assert st == 0 and 2 <= n <= 64 and ws == _ws_bytes(n, H=2)
    st, n, _ = _plan(lib, B=1, T=65536, H=2)      # 8 chains of 2048 chunks: many parts
    assert st == 0 and n >= 16
    assert _plan(lib, B=2, T=65536, H=32) == (0, 1, 0)   # 256 chains fill the GPU already
    assert _plan(lib, T=32)[:2] == (0, 1) and _plan(lib, T=0)[:2] == (0, 1)
    assert _plan(lib, dtype=0, dk=32, dv=32)[:2] == (0, 1)   # not a split shape: single pass
    assert _plan(lib, dtype=0, dk=32, dv=32, parts=4)[0] == 4
    assert _plan(lib, dk=32, parts=4)[0] == 4


@pytest.mark.parametrize("T", [33, 100, 1000, 4096, 5000])
def test_split_plan_explicit_counts(T):
    """Explicit counts give at most that many parts of whole 32-token chunks, at
    most one per chunk, and planning again with the result keeps it."""
    lib = _lib()
    nch = -(-T // 32)
    for P in (1, 2, 3, 5, 7, 64, 1000):
        st, n, ws = _plan(lib, T=T, parts=P)
        assert st == 0 and 1 <= n <= min(P, nch)
        assert ws == (_ws_bytes(n) if n > 1 else 0)
        assert _plan(lib, T=T, parts=n)[1] == n


def test_split_plan_invalid():
    lib = _lib()
    assert _plan(lib, parts=-1)[0] == 2
    assert _plan(lib, cus=-1)[0] == 2
    assert _plan(lib, dtype=5)[0] == 3
    assert _plan(lib, dk=48)[0] == 4
    assert lib.kda_chunk_fwd_split_plan(1, 1, 64, 1, 128, 128, 64, 0, 256, None, None) == 1


def _split(lib, parts=4, cus=256, ws=_addr(10), wsb=1 << 30, **over):
    a = dict(q=_addr(0), k=_addr(1), v=_addr(2), dtype=1, alpha=_addr(3), beta=_addr(4), S0=_addr(5),
             o=_addr(6), odt=0, S_T=_addr(7), B=1, T=4096, H=8, dk=128, dv=128, chunk=64)
    a.update(over)
    return lib.kda_chunk_fwd_split(a["q"], a["k"], a["v"], a["dtype"], a["alpha"], a["beta"], a["S0"], a["o"],
                                   a["odt"], a["S_T"], a["B"], a["T"], a["H"], a["dk"], a["dv"], a["chunk"],
                                   parts, cus, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(ws=None), 1),                                        # workspace needed
    (dict(wsb=_ws_bytes(4) - 16), 2),                          # workspace too small
    (dict(ws=ctypes.c_void_p(BASE + (10 << 32) + 8)), 5),      # misaligned workspace
    (dict(ws=_addr(0)), 6), (dict(ws=_addr(3)), 6),            # workspace aliases q, alpha
    (dict(ws=_addr(5)), 6),                                    # ... S0
    (dict(ws=_addr(6)), 6), (dict(ws=_addr(7)), 6),            # ... o, S_T
    (dict(parts=-1), 2), (dict(cus=-1), 2),
    (dict(dtype=0, dk=32, dv=32), 4),                          # fp32: no split kernel
    (dict(dk=32, parts=3), 4),                                 # bf16 d_k = 32: generic kernel
    (dict(q=None), 1), (dict(B=0), 2),
])
def test_split_validation(kw, code):
    assert _split(_lib(), **kw) == code


def _split_noalloc(lib, parts=4, cus=256, **over):
    a = dict(q=_addr(0), k=_addr(1), v=_addr(2), dtype=1, alpha=_addr(3), beta=_addr(4), S0=_addr(5),
             o=_addr(6), odt=0, S_T=_addr(7), B=1, T=4096, H=8, dk=128, dv=128, chunk=64)
    a.update(over)
    return lib.kda_chunk_fwd_split_noalloc(a["q"], a["k"], a["v"], a["dtype"], a["alpha"], a["beta"], a["S0"],
                                           a["o"], a["odt"], a["S_T"], a["B"], a["T"], a["H"], a["dk"], a["dv"],
                                           a["chunk"], parts, cus, None)


SCRATCH = 64 << 20  # KDA_SPLIT_SCRATCH_BYTES


@pytest.mark.parametrize("kw,code", [
    (dict(B=4, T=65536, H=32, parts=32), 2),   # the workspace of 32 parts exceeds the scratch
    (dict(B=2, T=65536, H=16, parts=9), 2),
    (dict(parts=-1), 2), (dict(cus=-1), 2),
    (dict(dtype=0, dk=32, dv=32), 4),          # fp32: no split kernel
    (dict(q=None), 1), (dict(o=_addr(0)), 6), (dict(dtype=9), 3),
])
def test_split_noalloc_validation(kw, code):
    """The allocation-free split refuses, before any HIP call, a part count whose
    workspace exceeds the library's scratch, and applies kda_chunk_fwd_split's checks."""
    parts = kw.pop("parts", 4)
    cus = kw.pop("cus", 256)
    if "B" in kw:
        assert _ws_bytes(parts, B=kw["B"], H=kw["H"]) > SCRATCH
    assert _split_noalloc(_lib(), parts=parts, cus=cus, **kw) == code


def test_split_noalloc_scratch_size_is_stated():
    assert "#define KDA_SPLIT_SCRATCH_BYTES ((size_t)64 << 20)" in HEADER.read_text()
    import gated_delta_rule_07_amd as kda
    assert kda.KDA_SPLIT_SCRATCH_BYTES == SCRATCH
