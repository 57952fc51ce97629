"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

* small workloads (all tokens), the five workloads' head/dim/parameter
  settings with shorter, ragged sequences: compression, then attention,
  softmax statistics, importance scores and top-k -- staged (the GPU's
  attention consumes the oracle's compressed K/V) and end to end (the GPU's
  attention consumes its own compression, and the oracle is fed those same
  bits), both at the stated bounds;
* all tokens of shapes whose long sequences enter the attention kernel's
  unrolled three-slot loop (a workgroup whose first token sees at least
  four whole key tiles of 32 compressed entries: token >= 2063 for
  l = 32, d = 16 and >= 4127 for l = 64, d = 32): the MQA workload at full
  size, and the GQA-16, long-stride and group-64 settings with a sequence
  past that point;
* the five workloads at full size, in the launch configuration the
  benchmark times: compression in full, attention on whole workgroups (the
  first, a middle and the last 64-token run of every sequence) and on
  sampled tokens;
* edge cases: empty and short sequences, negative and zero scale, groups
  that are not powers of two, MHA, other remap stencils, count 1;
* bitwise determinism across runs;
* each of the above in float16 as well as bfloat16 (edge cases: those that
  reach a different code path per element type -- the sign flip of q for a
  negative scale, empty sequences, odd groups, D1 = 192, the widest stencil).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (assert_close_out, assert_pslc, assert_softmax_stats, assert_topk,
                    gpu_attention, gpu_compress, log, to_f64, token_meta, upload_bits, workgroup_runs)

pytestmark = pytest.mark.gpu

SMALL = {
    0: synth.WORKLOADS[0],
    1: synth.small_variant(1, [1500, 777]),
    2: synth.small_variant(2, [1000, 2050, 64, 17]),
    3: synth.small_variant(3, [3000]),
    4: synth.small_variant(4, [2000, 1500, 300]),
}

# Shapes whose longest sequence enters the unrolled loop of the attention
# kernel, compared on every token.
LOOP = {
    "mqa-full": synth.WORKLOADS[1],
    "gqa16-d128": synth.small_variant(2, [4500, 700]),
    "long-l64-d32": synth.small_variant(3, [5200]),
    "group64-d128": synth.small_variant(4, [4200, 300]),
}


def _check_all(wl, g, ref, tokens):
    """g: GPU outputs whose rows are the given tokens, in order; ref: the
    oracle on the compressed K/V the GPU consumed."""
    assert_close_out(to_f64(g["out"]), ref["out"], "attention_out")
    assert_softmax_stats(g["max"].cpu().numpy(), g["sum"].cpu().numpy(), ref["max"], ref["sum"])
    assert_pslc(g["pslc"].cpu().numpy(), ref["pslc"])
    assert_topk(wl, tokens, g["topk"].cpu().numpy(), ref["topk"], ref["pslc"])


def _oracle_attention(wl, q_bits, kc_bits, vc_bits, tokens=None):
    """Steps 1-7 of the oracle on the given compressed K/V bit patterns."""
    if tokens is None:
        tokens = np.arange(wl.T, dtype=np.int64)
    return oracle.attention(q_bits, tokens, kc_bits, vc_bits, np.asarray(wl.act_seq_qlen, dtype=np.int64),
                            oracle.cmp_prefix(wl.seqlens, wl.l, wl.d), wl.N1, wl.N2, wl.scale, wl.l, wl.d,
                            wl.lsel, wl.count, dtype=wl.dtype)


def _run_small(wl, end_to_end=True):
    log(f"[case] {wl.name}: generate on GPU")
    inp = synth.make_inputs(wl, device="cuda")
    bits = {k: synth.bits(v) for k, v in inp.items()}
    log(f"[case] {wl.name}: oracle")
    ref = oracle.run(wl, bits["q"], bits["k"], bits["v"], bits["w"])
    log(f"[case] {wl.name}: GPU compress")
    kc_g = gpu_compress(wl, inp["k"], inp["w"])
    vc_g = gpu_compress(wl, inp["v"], inp["w"])
    torch.cuda.synchronize()
    assert_close_out(to_f64(kc_g), ref["kc"], "compressed K")
    assert_close_out(to_f64(vc_g), ref["vc"], "compressed V")
    log(f"[case] {wl.name}: GPU attention on the oracle's compressed K/V")
    g = gpu_attention(wl, inp["q"], upload_bits(ref["kc_bits"], wl.dtype),
                      upload_bits(ref["vc_bits"], wl.dtype))
    _check_all(wl, g, ref, ref["tokens"])
    if end_to_end:
        log(f"[case] {wl.name}: GPU attention on its own compressed K/V, oracle on the same bits")
        ref2 = _oracle_attention(wl, bits["q"], synth.bits(kc_g), synth.bits(vc_g))
        g2 = gpu_attention(wl, inp["q"], kc_g, vc_g)
        _check_all(wl, g2, ref2, ref["tokens"])
    return inp, g


DTYPES = ["bf16", "f16"]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("wid", [0, 1, 2, 3, 4])
def test_small_workloads_all_tokens(wid, dtype):
    _run_small(SMALL[wid].with_dtype(dtype))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("name", sorted(LOOP))
def test_loop_shapes_all_tokens(name, dtype):
    wl = LOOP[name].with_dtype(dtype)
    first = {32: 2063, 64: 4127}[wl.l]
    assert max(wl.seqlens) > first + 64, "the case must reach the unrolled loop"
    _run_small(wl)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("wid", [1, 2, 3, 4])
def test_full_size_workloads_sampled(wid, dtype):
    wl = synth.WORKLOADS[wid].with_dtype(dtype)
    log(f"[case] full {wl.name}: generate on GPU")
    inp = synth.make_inputs(wl, device="cuda")
    kb, vb, wb = synth.bits(inp["k"]), synth.bits(inp["v"]), synth.bits(inp["w"])
    actq = np.asarray(wl.act_seq_qlen, dtype=np.int64)
    log(f"[case] full {wl.name}: oracle compress")
    kc_ref = oracle.compress(kb, wb, actq, wl.l, wl.d, dtype)
    vc_ref = oracle.compress(vb, wb, actq, wl.l, wl.d, dtype)
    log(f"[case] full {wl.name}: GPU compress")
    kc_g = gpu_compress(wl, inp["k"], inp["w"])
    vc_g = gpu_compress(wl, inp["v"], inp["w"])
    torch.cuda.synchronize()
    assert_close_out(to_f64(kc_g), kc_ref, "compressed K")
    assert_close_out(to_f64(vc_g), vc_ref, "compressed V")
    kc_gb, vc_gb = synth.bits(kc_g), synth.bits(vc_g)
    kc_b, vc_b = oracle.round_to(kc_ref, dtype), oracle.round_to(vc_ref, dtype)
    tokens = np.union1d(workgroup_runs(wl), synth.sample_tokens(wl, per_seq=6))
    tok_t = torch.from_numpy(tokens).cuda()
    q_rows = synth.bits(inp["q"][tok_t])
    for leg, kcb, vcb, kcd, vcd in (("oracle's", kc_b, vc_b, None, None), ("GPU's own", kc_gb, vc_gb, kc_g, vc_g)):
        log(f"[case] full {wl.name}: oracle attention on {len(tokens)} tokens, {leg} compressed K/V")
        ref = _oracle_attention(wl, q_rows, kcb, vcb, tokens)
        log(f"[case] full {wl.name}: GPU attention (all tokens) on the {leg} compressed K/V")
        if kcd is None:
            kcd, vcd = upload_bits(kcb, dtype), upload_bits(vcb, dtype)
        g = gpu_attention(wl, inp["q"], kcd, vcd)
        gs = {"out": g["out"][tok_t], "max": g["max"][tok_t], "sum": g["sum"][tok_t],
              "pslc": g["pslc"][tok_t], "topk": g["topk"][tok_t]}
        _check_all(wl, gs, ref, tokens)
    del kc_g, vc_g
    # Properties that hold for every row of the full output.
    log(f"[case] full {wl.name}: whole-output properties")
    assert torch.isfinite(g["out"].float()).all()
    gsum = g["sum"][..., 0]
    gmax = g["max"][..., 0]
    assert bool(((gsum > 0) == torch.isfinite(gmax)).all())
    topk = g["topk"]
    assert int(topk.max()) < max(-(-T // wl.lsel) for T in wl.seqlens)
    assert int(topk[:, :, 0].min()) == 0 or int(topk[:, :, 0].min()) >= 0


BASE = synth.Workload("edge", (300,), 8, 2, 64, 64, 32, 16, 64, 4, 0.125, seed=900)
EDGES = {
    "short-and-empty-seqs": dataclasses.replace(BASE, seqlens=(5, 0, 31, 32, 33, 47, 48, 200, 1, 130)),
    "negative-scale": dataclasses.replace(BASE, scale=-0.09, seqlens=(400, 77)),
    "zero-scale": dataclasses.replace(BASE, scale=0.0, seqlens=(333,)),
    "group-of-3": dataclasses.replace(BASE, N1=12, N2=4, D1=128, D2=64, seqlens=(520, 64)),
    "mha-group-1": dataclasses.replace(BASE, N1=4, N2=4, seqlens=(700, 129)),
    "group-of-32": dataclasses.replace(BASE, N1=64, N2=2, D1=128, D2=128, seqlens=(600,)),
    "stencil-R3": dataclasses.replace(BASE, l=48, d=16, lsel=48, count=8, seqlens=(900, 250)),
    "stencil-R8": dataclasses.replace(BASE, l=128, d=16, lsel=128, count=32, seqlens=(1500,)),
    "stride-64": dataclasses.replace(BASE, l=64, d=64, lsel=128, count=3, seqlens=(1000, 65)),
    "count-1": dataclasses.replace(BASE, count=1, seqlens=(500,)),
    "d192-group-16": dataclasses.replace(BASE, N1=16, N2=1, D1=192, D2=64, seqlens=(777,)),
}


F16_EDGES = ["short-and-empty-seqs", "negative-scale", "group-of-3", "d192-group-16", "stencil-R8"]


@pytest.mark.parametrize("name,dtype", [(n, "bf16") for n in sorted(EDGES)] +
                         [(n, "f16") for n in F16_EDGES])
def test_edge_cases(name, dtype):
    _run_small(dataclasses.replace(EDGES[name], name=name).with_dtype(dtype))


def test_topk_exact_ties():
    """q = 0: every score is 0, every visible P of a row is the same and the
    importance scores of all interior select blocks are bitwise equal.  The
    top-k must then pick the lowest-index interior blocks exactly (ties go to
    the lower index), both where at most 64 candidates tie (rows of up to ~66
    blocks) and where more do (rows past ~4200 tokens, up to 94 blocks)."""
    wl = dataclasses.replace(BASE, name="exact-ties", count=16, seqlens=(6000,))
    log(f"[case] {wl.name}: generate on GPU, q = 0")
    inp = synth.make_inputs(wl, device="cuda")
    inp["q"].zero_()
    bits = {k: synth.bits(v) for k, v in inp.items()}
    log(f"[case] {wl.name}: oracle")
    ref = oracle.run(wl, bits["q"], bits["k"], bits["v"], bits["w"])
    log(f"[case] {wl.name}: GPU attention on the oracle's compressed K/V")
    g = gpu_attention(wl, inp["q"], upload_bits(ref["kc_bits"], wl.dtype),
                      upload_bits(ref["vc_bits"], wl.dtype))
    _check_all(wl, g, ref, ref["tokens"])
    gi, ri = g["topk"].cpu().numpy(), ref["topk"]
    long_rows = 0
    for k, (t, S) in enumerate(token_meta(wl, ref["tokens"])):
        nvalid = min(t // wl.lsel + 1, S)
        kk = min(wl.count, nvalid)
        long_rows += nvalid >= 70
        for h in range(wl.N2):
            assert sorted(gi[k, h, :kk].tolist()) == sorted(ri[k, h, :kk].tolist()), (t, h, gi[k, h], ri[k, h])
    assert long_rows > 0


def test_bitwise_deterministic():
    wl = SMALL[2]
    log(f"[case] determinism {wl.name}")
    inp = synth.make_inputs(wl, device="cuda")
    kc1 = gpu_compress(wl, inp["k"], inp["w"])
    vc1 = gpu_compress(wl, inp["v"], inp["w"])
    a = gpu_attention(wl, inp["q"], kc1, vc1)
    kc2 = gpu_compress(wl, inp["k"], inp["w"])
    vc2 = gpu_compress(wl, inp["v"], inp["w"])
    b = gpu_attention(wl, inp["q"], kc2, vc2)
    assert torch.equal(kc1, kc2) and torch.equal(vc1, vc2)
    for k in a:
        assert torch.equal(a[k], b[k]), k
    # the debug output does not change anything else
    c = gpu_attention(wl, inp["q"], kc1, vc1, return_p_slc=False)
    for k in ("out", "topk", "max", "sum"):
        assert torch.equal(a[k], c[k]), k
