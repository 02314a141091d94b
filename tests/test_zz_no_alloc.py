"""The allocation-free split prefill (kda_chunk_fwd_split_noalloc) against the
split prefill with a caller workspace (kda_chunk_fwd_split): two calls in a row
through the C ABI, the second with a smaller input, each bit-equal to the
existing entry point (same kernels, same part count) and within the bf16
tolerance of the oracle on sampled heads; then the allocation-free call's own
part choice against the oracle (its single pass is the pipeline, which needs no
workspace, so it may choose parts where the allocating call would not).  (The
refusal of a split that needs more scratch than the library holds is a
host-side check, tested on the CPU.)"""
import pytest
import torch

import kda_inputs as ki
from kda_check import assert_close, gpu_o_heads, gpu_s_heads, log, oracle_prefill

pytestmark = pytest.mark.gpu


def _kda():
    import gated_delta_rule_07_amd as kda
    return kda


@pytest.mark.parametrize("o_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_split_matches_workspace_split(gpu, o_dtype):
    kda = _kda()
    for (B, T, H, parts, seed) in ((1, 4096, 8, 5, 40), (1, 1000, 2, 4, 41)):
        log(f"no-alloc split B={B} T={T} H={H} parts={parts} o={o_dtype}")
        x = ki.make_prefill(B, T, H, 128, 128, torch.bfloat16, 3.0, 0.1, seed=seed, device=gpu)
        args = (x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"])
        n, need = kda.kda_chunk_fwd_split_plan(torch.bfloat16, B, T, H, 128, 128, parts=parts)
        assert n >= 2 and 0 < need <= kda.KDA_SPLIT_SCRATCH_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device=gpu)
        o_ref, s_ref = kda.kda_chunk_fwd_split(*args, parts=n, workspace=ws, o_dtype=o_dtype)
        o = torch.full_like(o_ref, float("nan"))
        s = torch.full_like(s_ref, float("nan"))
        kda.kda_chunk_fwd_split_noalloc(*args, parts=parts, o=o, S_T=s)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
        heads = [0, B * H - 1]
        ro, rs = oracle_prefill(x, heads=heads)
        if o_dtype == torch.float32:
            assert_close(gpu_o_heads(o, heads), ro, True, "no-alloc o")
        assert_close(gpu_s_heads(s, heads), rs, True, "no-alloc S_T")
    # the library's part count for the allocation-free call
    x = ki.make_prefill(1, 4096, 8, 128, 128, torch.bfloat16, 3.0, 0.1, seed=42, device=gpu)
    o, s = kda.kda_chunk_fwd_split_noalloc(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["S0"], parts=0,
                                           o_dtype=o_dtype)
    torch.cuda.synchronize()
    heads = [0, 7]
    ro, rs = oracle_prefill(x, heads=heads)
    if o_dtype == torch.float32:
        assert_close(gpu_o_heads(o, heads), ro, True, "no-alloc o, library's parts")
    assert_close(gpu_s_heads(s, heads), rs, True, "no-alloc S_T, library's parts")
