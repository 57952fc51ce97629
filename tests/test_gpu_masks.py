"""GPU parity with explicit atten_mask / topk_mask ("mindspore.ops.
nsa_compress_attention", Parameters: optional bool tensors of shape (S1,
S2)).  Reading, shared with the oracle: one matrix for every sequence,
indexed by (local query position, compressed entry or select block); True
masks the pair out and replaces that step's positional rule.

* masks that spell the positional rules give bitwise the same outputs as
  the mask-free path;
* random masks (with fully masked rows, rows that see blocks the causal
  rule hides, and rows without top-k candidates) against the oracle given
  the same masks, on the five workloads' shapes (short ragged sequences),
  in bf16 and one case in fp16;
* banded masks (a sliding window over the compressed blocks), so that row
  blocks start their key loop past the first tile, and causal masks with
  random holes past the first blocks (leading tiles kept whole by every
  token run without the mask);
* one mask at a time, and the fwd/select halves against the full call;
* a full-size workload with causal masks spelled out, against the
  mask-free path.
"""
import dataclasses
import zlib

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (assert_close_out, assert_pslc, assert_softmax_stats, assert_topk, gpu_prefix,
                    log, to_f64, upload_bits)

import kv_compression_block_amd as nsa

pytestmark = pytest.mark.gpu


def _plan(wl):
    c, s = gpu_prefix(wl)
    return nsa.nsa_compress_attention_get_workspace(
        wl.act_seq_qlen, c, s, wl.N1, wl.N2, wl.D1, wl.D2, wl.scale, wl.l, wl.d, wl.lsel, wl.count,
        wl.torch_dtype)


def _gpu(wl, q, kc, vc, am=None, tm=None):
    plan = _plan(wl)
    try:
        dev = q.device
        amt = None if am is None else torch.from_numpy(np.ascontiguousarray(am)).to(dev)
        tmt = None if tm is None else torch.from_numpy(np.ascontiguousarray(tm)).to(dev)
        res = nsa.nsa_compress_attention(plan, q, kc, vc, return_p_slc=True, atten_mask=amt,
                                         topk_mask=tmt)
        torch.cuda.synchronize()
    finally:
        plan.destroy()
    return dict(zip(["out", "topk", "max", "sum", "pslc"], res))


def _sizes(wl):
    nc = [nsa.nsa_compress_out_len(T, wl.l, wl.d) for T in wl.seqlens]
    return max(wl.seqlens), max(nc), max(-(-T // wl.lsel) for T in wl.seqlens)


def _causal_masks(wl, extra=(3, 5)):
    T_max, nc_max, s_max = _sizes(wl)
    t = np.arange(T_max + extra[0])[:, None]
    am = np.arange(nc_max + extra[1])[None, :] * wl.d + wl.l - 1 > t
    tm = np.arange(s_max + extra[1])[None, :] * wl.lsel > t
    return am, tm


def _random_masks(wl, seed, p=0.3, extra=(2, 7)):
    rng = np.random.default_rng(seed)
    T_max, nc_max, s_max = _sizes(wl)
    am = rng.random((T_max + extra[0], nc_max + extra[1])) < p
    tm = rng.random((T_max + extra[0], s_max + extra[1])) < p
    am[3, :] = True             # every block masked
    am[40, :] = False           # sees blocks the causal rule hides
    am[41, :nc_max // 2] = True # only late blocks
    tm[4, :] = True             # no candidate
    tm[50, :] = False
    return am, tm


def _check(wl, g, ref, am=None, tm=None):
    tokens = ref["tokens"]
    assert_close_out(to_f64(g["out"]), ref["out"], "attention_out")
    assert_softmax_stats(g["max"].cpu().numpy(), g["sum"].cpu().numpy(), ref["max"], ref["sum"])
    assert_pslc(g["pslc"].cpu().numpy(), ref["pslc"])
    assert_topk(wl, tokens, g["topk"].cpu().numpy(), ref["topk"], ref["pslc"], tie_rel=1e-4,
                topk_mask=tm)


def _inputs(wl):
    inp = synth.make_inputs(wl, device="cuda")
    bits = {k: synth.bits(v) for k, v in inp.items()}
    actq = np.asarray(wl.act_seq_qlen, dtype=np.int64)
    kc = oracle.round_to(oracle.compress(bits["k"], bits["w"], actq, wl.l, wl.d, wl.dtype), wl.dtype)
    vc = oracle.round_to(oracle.compress(bits["v"], bits["w"], actq, wl.l, wl.d, wl.dtype), wl.dtype)
    return inp, bits, kc, vc


def _oracle(wl, bits, kc, vc, am=None, tm=None):
    res = oracle.attention(bits["q"], np.arange(wl.T, dtype=np.int64), kc, vc, wl.act_seq_qlen,
                           oracle.cmp_prefix(wl.seqlens, wl.l, wl.d), wl.N1, wl.N2, wl.scale, wl.l,
                           wl.d, wl.lsel, wl.count, dtype=wl.dtype, atten_mask=am, topk_mask=tm)
    res["tokens"] = np.arange(wl.T, dtype=np.int64)
    return res


SMALL = {
    0: synth.WORKLOADS[0],
    1: synth.small_variant(1, [900, 333]),
    2: synth.small_variant(2, [700, 1030, 64, 17]),
    3: synth.small_variant(3, [1500]),
    4: synth.small_variant(4, [1000, 600, 130]),
}
MHA = dataclasses.replace(synth.WORKLOADS[0], name="mha-masks", N1=4, N2=4, seqlens=(400, 129))


def test_causal_masks_spelled_out_match_the_mask_free_path_bitwise():
    wl = SMALL[2]
    log(f"[case] {wl.name}: causal masks spelled out")
    inp, bits, kc, vc = _inputs(wl)
    kc_g, vc_g = upload_bits(kc, wl.dtype), upload_bits(vc, wl.dtype)
    am, tm = _causal_masks(wl)
    a = _gpu(wl, inp["q"], kc_g, vc_g)
    b = _gpu(wl, inp["q"], kc_g, vc_g, am, tm)
    for k in a:
        assert torch.equal(a[k], b[k]), k


@pytest.mark.parametrize("name,wl,dtype", [(f"w{i}", SMALL[i], "bf16") for i in SMALL] +
                         [("mha", MHA, "bf16"), ("w2-f16", SMALL[2], "f16"), ("w1-f16", SMALL[1], "f16")])
def test_random_masks_against_oracle(name, wl, dtype):
    wl = wl.with_dtype(dtype)
    log(f"[case] {wl.name}: random masks")
    inp, bits, kc, vc = _inputs(wl)
    am, tm = _random_masks(wl, seed=zlib.crc32(name.encode()))
    ref = _oracle(wl, bits, kc, vc, am, tm)
    g = _gpu(wl, inp["q"], upload_bits(kc, wl.dtype), upload_bits(vc, wl.dtype), am, tm)
    _check(wl, g, ref, am, tm)


def _band_masks(wl, width, extra=(1, 3)):
    """Each row keeps only the last ``width`` blocks it may see causally
    (a sliding window over compressed blocks) and the select blocks in the
    same range of positions: later row blocks start their key loop well
    past tile 0, at odd and even tiles."""
    T_max, nc_max, s_max = _sizes(wl)
    t = np.arange(T_max + extra[0])[:, None]
    i = np.arange(nc_max + extra[1])[None, :]
    nv = np.where(t >= wl.l - 1, (t - wl.l + 1) // wl.d + 1, 0)
    am = ~((i < nv) & (i >= nv - width))
    j = np.arange(s_max + extra[1])[None, :]
    tm = ~((j * wl.lsel <= t) & (j * wl.lsel >= t - width * wl.d))
    return am, tm


@pytest.mark.parametrize("wid,width", [(2, 40), (3, 70), (4, 33), ("mha", 50), (1, 100)])
def test_banded_masks_against_oracle(wid, width):
    wl = MHA if wid == "mha" else SMALL[wid]
    log(f"[case] {wl.name}: banded masks, width {width}")
    inp, bits, kc, vc = _inputs(wl)
    am, tm = _band_masks(wl, width)
    ref = _oracle(wl, bits, kc, vc, am, tm)
    g = _gpu(wl, inp["q"], upload_bits(kc, wl.dtype), upload_bits(vc, wl.dtype), am, tm)
    _check(wl, g, ref, am, tm)


@pytest.mark.parametrize("wid", [2, 3, 4])
def test_causal_masks_with_holes_against_oracle(wid):
    """The causal rule plus random holes past the first 96 blocks: leading
    key tiles that every token keeps whole take the mask-free body, the
    rest the masked one."""
    wl = SMALL[wid]
    log(f"[case] {wl.name}: causal masks with holes")
    inp, bits, kc, vc = _inputs(wl)
    am, tm = _causal_masks(wl)
    rng = np.random.default_rng(31 + wid)
    holes = rng.random(am.shape) < 0.2
    holes[:, :96] = False
    am = am | holes
    tm = tm | (rng.random(tm.shape) < 0.2)
    ref = _oracle(wl, bits, kc, vc, am, tm)
    g = _gpu(wl, inp["q"], upload_bits(kc, wl.dtype), upload_bits(vc, wl.dtype), am, tm)
    _check(wl, g, ref, am, tm)


@pytest.mark.parametrize("which", ["atten", "topk"])
def test_one_mask_at_a_time(which):
    wl = SMALL[4]
    log(f"[case] {wl.name}: only the {which} mask")
    inp, bits, kc, vc = _inputs(wl)
    am, tm = _random_masks(wl, seed=5)
    am = am if which == "atten" else None
    tm = tm if which == "topk" else None
    ref = _oracle(wl, bits, kc, vc, am, tm)
    g = _gpu(wl, inp["q"], upload_bits(kc, wl.dtype), upload_bits(vc, wl.dtype), am, tm)
    _check(wl, g, ref, am, tm)


def test_masked_halves_equal_the_full_call():
    wl = SMALL[3]
    log(f"[case] {wl.name}: fwd_masked + select_masked vs masked")
    inp, bits, kc, vc = _inputs(wl)
    kc_g, vc_g = upload_bits(kc, wl.dtype), upload_bits(vc, wl.dtype)
    am, tm = _random_masks(wl, seed=9)
    amt, tmt = torch.from_numpy(am).cuda(), torch.from_numpy(tm).cuda()
    full = _gpu(wl, inp["q"], kc_g, vc_g, am, tm)
    plan = _plan(wl)
    try:
        out, mx, sm = nsa.nsa_compress_attention_fwd(plan, inp["q"], kc_g, vc_g, atten_mask=amt)
        topk, pslc = nsa.nsa_compress_attention_select(plan, inp["q"], kc_g, mx, sm, return_p_slc=True,
                                                       atten_mask=amt, topk_mask=tmt)
        torch.cuda.synchronize()
    finally:
        plan.destroy()
    for k, v in (("out", out), ("max", mx), ("sum", sm), ("topk", topk), ("pslc", pslc)):
        assert torch.equal(full[k], v), k


def test_mask_shape_and_workspace_errors():
    wl = SMALL[0]
    inp, bits, kc, vc = _inputs(wl)
    kc_g, vc_g = upload_bits(kc, wl.dtype), upload_bits(vc, wl.dtype)
    am, tm = _causal_masks(wl, extra=(0, 0))
    plan = _plan(wl)
    try:
        with pytest.raises(ValueError):      # one column short
            nsa.nsa_compress_attention(plan, inp["q"], kc_g, vc_g,
                                       atten_mask=torch.from_numpy(am[:, :-1].copy()).cuda())
        with pytest.raises(ValueError):      # one row short
            nsa.nsa_compress_attention(plan, inp["q"], kc_g, vc_g,
                                       topk_mask=torch.from_numpy(tm[:-1].copy()).cuda())
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
        with pytest.raises(ValueError):      # the mask-free workspace is too small
            nsa.nsa_compress_attention(plan, inp["q"], kc_g, vc_g, workspace=ws,
                                       atten_mask=torch.from_numpy(am).cuda())
        torch.cuda.synchronize()
    finally:
        plan.destroy()


def test_full_size_causal_masks_sampled():
    """The batched workload at full size, in the launch configuration the
    benchmark times, with its causal masks spelled out: bitwise equal to
    the mask-free path on every row (that path meets the oracle in the
    full-size parity tests)."""
    wl = synth.WORKLOADS[4]
    log(f"[case] full {wl.name}: causal masks spelled out")
    inp = synth.make_inputs(wl, device="cuda")
    kc = nsa.nsa_compress(inp["k"], inp["w"], wl.act_seq_qlen, wl.l, wl.d)
    vc = nsa.nsa_compress(inp["v"], inp["w"], wl.act_seq_qlen, wl.l, wl.d)
    am, tm = _causal_masks(wl, extra=(0, 0))
    a = _gpu(wl, inp["q"], kc, vc)
    b = _gpu(wl, inp["q"], kc, vc, am, tm)
    for k in a:
        assert torch.equal(a[k], b[k]), k
