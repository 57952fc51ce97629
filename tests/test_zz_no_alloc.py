"""The entry point that allocates nothing (nsa_compress_attention_noalloc)
against nsa_compress_attention through the C ABI: the same kernels on the
same table, so every output must agree bit for bit -- on two calls in a row
on one GPU, the second with a smaller batch (the static scratch keeps the
first call's table, which the second must not read)."""
import numpy as np
import pytest
import torch

import synth
from parity import gpu_prefix, log

import kv_compression_block_amd as nsa

pytestmark = pytest.mark.gpu


def _plan(wl):
    c, s = gpu_prefix(wl)
    return nsa.nsa_compress_attention_get_workspace(
        wl.act_seq_qlen, c, s, wl.N1, wl.N2, wl.D1, wl.D2, wl.scale, wl.l, wl.d, wl.lsel, wl.count,
        wl.torch_dtype)


def _outputs(plan, dtype):
    i = plan.info
    T1, N1, N2, D2 = i["total_q_tokens"], i["head_num"], i["kv_head_num"], i["d2"]
    return {"attention_out": torch.full((T1, N1, D2), 7.0, dtype=dtype, device="cuda"),
            "topk_indices": torch.full((T1, N2, i["select_block_count"]), 12345, dtype=torch.int32, device="cuda"),
            "softmax_max": torch.full((T1, N1, 8), 7.0, dtype=torch.float32, device="cuda"),
            "softmax_sum": torch.full((T1, N1, 8), 7.0, dtype=torch.float32, device="cuda")}


def _compare(wl):
    log(f"[case] no-alloc {wl.name}")
    inp = synth.make_inputs(wl, device="cuda")
    kc = nsa.nsa_compress(inp["k"], inp["w"], wl.act_seq_qlen, wl.l, wl.d)
    vc = nsa.nsa_compress(inp["v"], inp["w"], wl.act_seq_qlen, wl.l, wl.d)
    plan = _plan(wl)
    try:
        ref = nsa.nsa_compress_attention(plan, inp["q"], kc, vc, return_p_slc=True)
        outs = _outputs(plan, wl.torch_dtype)
        pslc = torch.full_like(ref[4], 7.0)
        got = nsa.nsa_compress_attention_noalloc(plan, inp["q"], kc, vc, outs, p_slc=pslc)
        torch.cuda.synchronize()
    finally:
        plan.destroy()
    for name, a, b in zip(("attention_out", "topk_indices", "softmax_max", "softmax_sum", "p_slc"),
                          got + (pslc,), ref):
        assert torch.equal(a, b), f"{wl.name}: {name} differs from nsa_compress_attention"


def test_no_alloc_matches_workspace_entry_point_twice():
    first = synth.small_variant(2, [1000, 2050, 64, 17])
    second = synth.small_variant(4, [700])          # smaller batch and fewer tokens
    assert second.B < first.B and second.T < first.T
    _compare(first)
    _compare(second)


def test_no_alloc_rejects_more_sequences_than_its_scratch_holds():
    wl = synth.WORKLOADS[0].with_seqlens([64] * 1025)
    plan = _plan(wl)
    try:
        outs = _outputs(plan, wl.torch_dtype)
        q = torch.zeros((wl.T, wl.N1, wl.D1), dtype=wl.torch_dtype, device="cuda")
        n2 = plan.info["total_cmp_tokens"]
        kc = torch.zeros((n2, wl.N2, wl.D1), dtype=wl.torch_dtype, device="cuda")
        vc = torch.zeros((n2, wl.N2, wl.D2), dtype=wl.torch_dtype, device="cuda")
        with pytest.raises(NotImplementedError, match="at most 1024 sequences"):
            nsa.nsa_compress_attention_noalloc(plan, q, kc, vc, outs)
    finally:
        plan.destroy()
