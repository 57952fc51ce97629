"""GPU parity of the selected-block attention (the consumer of
topk_indices; interface of "lite_boost.ops.rain_fusion_attention") against
the oracle.  Reading, shared with the oracle: token t, head h of KV group g
attends to the raw keys s <= t of its sequence whose block floor(s / l') is
listed in topk[t, g]; -1, repeats and out-of-range entries add nothing; no
key gives output 0 and lse -inf.

* seeded random block lists (padding, repeats, out-of-range entries) on the
  five workloads' shapes with short ragged sequences, an MHA case and
  float16: every token;
* the oracle's own top-k of the compressed branch as the block lists (the
  path as NSA runs it), small workloads;
* the batched workload at full size with random lists, sampled tokens;
* bitwise determinism.

Tolerances: attention_out as the compressed attention (2e-2 + 1e-2 |ref|);
softmax_lse 1e-3 absolute, -inf matched exactly.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_close_out, gpu_prefix, log, to_f64

import kv_compression_block_amd as nsa

pytestmark = pytest.mark.gpu

LSE_ATOL = 1e-3

SMALL = {
    0: synth.WORKLOADS[0],
    1: synth.small_variant(1, [900, 333]),
    2: synth.small_variant(2, [700, 1030, 64, 17]),
    3: synth.small_variant(3, [1500]),
    4: synth.small_variant(4, [1000, 600, 130]),
}
MHA = dataclasses.replace(synth.WORKLOADS[0], name="mha-select", N1=4, N2=4, seqlens=(400, 129, 3))
GQA3 = dataclasses.replace(synth.WORKLOADS[0], name="group-of-3-select", N1=12, N2=4, D1=128, D2=64,
                           seqlens=(520, 64))


def _plan(wl):
    c, s = gpu_prefix(wl)
    return nsa.nsa_compress_attention_get_workspace(
        wl.act_seq_qlen, c, s, wl.N1, wl.N2, wl.D1, wl.D2, wl.scale, wl.l, wl.d, wl.lsel, wl.count,
        wl.torch_dtype)


def _gpu(wl, q, k, v, topk):
    plan = _plan(wl)
    try:
        out, lse = nsa.nsa_select_attention(plan, q, k, v, torch.from_numpy(topk).to(q.device))
        torch.cuda.synchronize()
    finally:
        plan.destroy()
    return out, lse


def _compare(got_out, got_lse, ref):
    assert_close_out(to_f64(got_out), ref["out"], "selected attention out")
    gl = got_lse.double().cpu().numpy()
    rl = ref["lse"]
    ninf = np.isneginf(rl)
    assert np.array_equal(np.isneginf(gl), ninf), "lse: -inf rows differ"
    d = np.abs(gl[~ninf] - rl[~ninf])
    log(f"  lse: max|err| {d.max(initial=0):.3e}; {int(ninf.sum())} rows with no key")
    assert d.max(initial=0) <= LSE_ATOL


def _run(wl, topk, tokens=None):
    inp = synth.make_inputs(wl, device="cuda")
    bits = {k: synth.bits(v) for k, v in inp.items()}
    ref = oracle.select_attention(bits["q"], bits["k"], bits["v"], topk, wl.act_seq_qlen, wl.N1, wl.N2,
                                  wl.scale, wl.lsel, tokens=tokens, dtype=wl.dtype)
    out, lse = _gpu(wl, inp["q"], inp["k"], inp["v"], topk)
    if tokens is not None:
        t = torch.from_numpy(tokens).cuda()
        out, lse = out[t], lse[t]
    _compare(out, lse, ref)
    return inp


@pytest.mark.parametrize("name,wl,dtype", [(f"w{i}", SMALL[i], "bf16") for i in SMALL] +
                         [("mha", MHA, "bf16"), ("gqa3", GQA3, "bf16"), ("w4-f16", SMALL[4], "f16"),
                          ("w3-f16", SMALL[3], "f16")])
def test_random_block_lists_against_oracle(name, wl, dtype):
    wl = wl.with_dtype(dtype)
    log(f"[case] {wl.name}: selected attention, random block lists")
    _run(wl, synth.random_block_lists(wl, seed=len(name) * 7 + 3))


@pytest.mark.parametrize("wid", [0, 2, 4])
def test_oracle_topk_as_block_lists(wid):
    """The block lists NSA would use: the oracle's top-k of the compressed
    branch on the same inputs."""
    wl = SMALL[wid]
    log(f"[case] {wl.name}: selected attention over the oracle's top-k")
    inp = synth.make_inputs(wl, device="cuda")
    bits = {k: synth.bits(v) for k, v in inp.items()}
    topk = oracle.run(wl, bits["q"], bits["k"], bits["v"], bits["w"])["topk"]
    ref = oracle.select_attention(bits["q"], bits["k"], bits["v"], topk, wl.act_seq_qlen, wl.N1, wl.N2,
                                  wl.scale, wl.lsel, dtype=wl.dtype)
    out, lse = _gpu(wl, inp["q"], inp["k"], inp["v"], topk)
    _compare(out, lse, ref)


def test_full_size_batched_sampled():
    wl = synth.WORKLOADS[4]
    log(f"[case] full {wl.name}: selected attention, sampled tokens")
    _run(wl, synth.random_block_lists(wl, seed=5), tokens=synth.sample_tokens(wl, per_seq=4))


def test_select_attention_deterministic():
    wl = SMALL[2]
    inp = synth.make_inputs(wl, device="cuda")
    topk = synth.random_block_lists(wl, seed=8)
    a = _gpu(wl, inp["q"], inp["k"], inp["v"], topk)
    b = _gpu(wl, inp["q"], inp["k"], inp["v"], topk)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
