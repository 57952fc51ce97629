"""GPU parity of the split attention launch (nsa_compress_attention_fwd_split:
long row blocks cut into key-range pieces, merged by a second kernel)
against the oracle: attention_out, softmax max and sum, with the bounds of
the unsplit launch (the merge only reorders the same sums), on the oracle's
compressed K/V."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (assert_close_out, assert_softmax_stats, gpu_prefix, log, to_f64, upload_bits)
from test_gpu_parity import EDGES, SMALL

import kv_compression_block_amd as nsa

pytestmark = pytest.mark.gpu


def _plan(wl):
    c, s = gpu_prefix(wl)
    return nsa.nsa_compress_attention_get_workspace(
        wl.act_seq_qlen, c, s, wl.N1, wl.N2, wl.D1, wl.D2, wl.scale, wl.l, wl.d, wl.lsel, wl.count,
        wl.torch_dtype)


def _split(wl, q, kc, vc, tiles):
    plan = _plan(wl)
    try:
        out, mx, sm = nsa.nsa_compress_attention_fwd_split(plan, q, kc, vc, tiles)
        out2, mx2, sm2 = nsa.nsa_compress_attention_fwd_split(plan, q, kc, vc, tiles)
        torch.cuda.synchronize()
    finally:
        plan.destroy()
    assert torch.equal(out, out2) and torch.equal(mx, mx2) and torch.equal(sm, sm2), "not repeatable"
    return out, mx, sm


def _check(got, ref):
    out, mx, sm = got
    assert_close_out(to_f64(out), ref["out"], "attention_out")
    assert_softmax_stats(mx.cpu().numpy(), sm.cpu().numpy(), ref["max"], ref["sum"])


def _small(wl, tiles):
    log(f"[case] {wl.name}: split attention, {tiles} key tiles per piece")
    inp = synth.make_inputs(wl, device="cuda")
    bits = {k: synth.bits(v) for k, v in inp.items()}
    ref = oracle.run(wl, bits["q"], bits["k"], bits["v"], bits["w"])
    got = _split(wl, inp["q"], upload_bits(ref["kc_bits"], wl.dtype), upload_bits(ref["vc_bits"], wl.dtype),
                 tiles)
    _check(got, ref)


@pytest.mark.parametrize("tiles", [1, 3])
@pytest.mark.parametrize("wid", [0, 1, 2, 3, 4])
def test_split_small_workloads(wid, tiles):
    _small(SMALL[wid], tiles)


def test_split_f16():
    _small(SMALL[2].with_dtype("f16"), 2)


@pytest.mark.parametrize("name", ["short-and-empty-seqs", "negative-scale", "zero-scale", "group-of-3",
                                  "stride-64", "d192-group-16"])
def test_split_edge_cases(name):
    _small(EDGES[name], 1)


@pytest.mark.parametrize("wid,tiles", [(1, 4), (4, 8)])
def test_split_full_size_sampled(wid, tiles):
    wl = synth.WORKLOADS[wid]
    log(f"[case] full {wl.name}: split attention, {tiles} key tiles per piece")
    inp = synth.make_inputs(wl, device="cuda")
    kb, vb, wb = synth.bits(inp["k"]), synth.bits(inp["v"]), synth.bits(inp["w"])
    actq = np.asarray(wl.act_seq_qlen, dtype=np.int64)
    kc_b = oracle.round_to(oracle.compress(kb, wb, actq, wl.l, wl.d, wl.dtype), wl.dtype)
    vc_b = oracle.round_to(oracle.compress(vb, wb, actq, wl.l, wl.d, wl.dtype), wl.dtype)
    tokens = synth.sample_tokens(wl, per_seq=6)
    q_rows = synth.bits(inp["q"][torch.from_numpy(tokens).cuda()])
    ref = oracle.attention(q_rows, tokens, kc_b, vc_b, actq, oracle.cmp_prefix(wl.seqlens, wl.l, wl.d),
                           wl.N1, wl.N2, wl.scale, wl.l, wl.d, wl.lsel, wl.count, dtype=wl.dtype)
    out, mx, sm = _split(wl, inp["q"], upload_bits(kc_b, wl.dtype), upload_bits(vc_b, wl.dtype), tiles)
    tok_t = torch.from_numpy(tokens).cuda()
    _check((out[tok_t], mx[tok_t], sm[tok_t]), ref)
    assert torch.isfinite(out.float()).all()
    assert bool(((sm[..., 0] > 0) == torch.isfinite(mx[..., 0])).all())


def test_single_pass_matches_split_on_every_token():
    """The batched workload's longest and shortest sequences at full size:
    the single-pass launch (whose unrolled three-slot loop does most of the
    work there) against the split launch with 3 key tiles per piece (which
    never enters that loop), on every row.  Both consume the same compressed
    K/V and compute every score with the same MFMA sequence, so the softmax
    max agrees bit for bit; the sums differ only in summation order, the
    outputs also in where P is rounded."""
    base = synth.WORKLOADS[4]
    lens = (max(base.seqlens), min(base.seqlens))
    wl = base.with_seqlens(lens, name=f"{base.name}@lens{list(lens)}")
    log(f"[case] {wl.name}: single pass against split (3 tiles per piece), all tokens")
    inp = synth.make_inputs(wl, device="cuda")
    kc = nsa.nsa_compress(inp["k"], inp["w"], wl.act_seq_qlen, wl.l, wl.d)
    vc = nsa.nsa_compress(inp["v"], inp["w"], wl.act_seq_qlen, wl.l, wl.d)
    plan = _plan(wl)
    try:
        out1, mx1, sm1 = nsa.nsa_compress_attention_fwd(plan, inp["q"], kc, vc)
        torch.cuda.synchronize()
    finally:
        plan.destroy()
    out2, mx2, sm2 = _split(wl, inp["q"], kc, vc, 3)
    assert torch.equal(mx1, mx2), "softmax_max differs between the launches"
    fin = sm1 > 0
    assert torch.equal(fin, sm2 > 0)
    rel = ((sm1 - sm2).abs() / sm1.clamp_min(1e-30))[fin]
    log(f"  softmax sum: max rel diff {float(rel.max()):.3e}")
    assert float(rel.max()) <= 1e-5
    a, b = out1.double(), out2.double()
    d = (a - b).abs()
    log(f"  attention_out: max |diff| {float(d.max()):.3e}")
    assert bool((d <= 2e-2 + 1e-2 * b.abs()).all())
    # Each launch rounds every P to bfloat16 before P.V, relative to its own
    # running maximum (a piece starts a new one), so each output carries up
    # to 2^-9 * max|V| of rounding, plus its own rounding to bfloat16.
    vmax = float(vc.double().abs().max())
    assert bool((d <= 2.0 ** -8 * vmax + 2.0 ** -7 * b.abs()).all())
