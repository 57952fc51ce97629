"""GPU parity of the backward of the compressed attention against the
oracle (the derivatives of the forward definition; the pages give no
backward formulas).  The GPU backward runs on the GPU forward's own
outputs (attention_out, softmax max and sum) over the oracle's compressed
K/V; the oracle recomputes the forward in float64.

Tolerance (gradients are sums of products of bf16-rounded factors; dS is
rounded to the element type before its MFMA, Delta uses the rounded
attention_out): per tensor, max |gpu - oracle| <= 2e-2 * max |oracle| and
||gpu - oracle||_2 <= 1e-2 * ||oracle||_2.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import gpu_prefix, log, to_f64, upload_bits

import kv_compression_block_amd as nsa

pytestmark = pytest.mark.gpu

SMALL = {
    0: synth.WORKLOADS[0],
    1: synth.small_variant(1, [900, 333]),
    2: synth.small_variant(2, [700, 1030, 64, 17]),
    3: synth.small_variant(3, [1500]),
    4: synth.small_variant(4, [1000, 600, 130]),
}
NEG = dataclasses.replace(synth.WORKLOADS[0], name="negative-scale-bwd", N1=8, N2=2, scale=-0.09,
                          seqlens=(400, 77))
# Sequences long enough (136-161 compressed entries, five or six key tiles)
# that the query-side kernel runs its steady state: the key-tile slots wrap
# around, and most waves take the loop without the visibility test.
LONG = dataclasses.replace(synth.small_variant(4, [2600, 333]), name="long-seqs-bwd", N1=16)
LONG192 = dataclasses.replace(synth.small_variant(1, [2200]), name="long-seq-d192-bwd")


def assert_grad_close(got: np.ndarray, ref: np.ndarray, what: str):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    scale = float(np.abs(ref).max(initial=0.0))
    dmax = float(np.abs(got - ref).max(initial=0.0))
    rel2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    log(f"  {what}: max|err| {dmax:.3e} of max|ref| {scale:.3e}; rel L2 {rel2:.3e}")
    assert dmax <= 2e-2 * scale + 1e-30, what
    assert rel2 <= 1e-2, what


def _run(wl, keys=("dq",)):
    log(f"[case] {wl.name}: backward")
    inp = synth.make_inputs(wl, device="cuda")
    bits = {k: synth.bits(v) for k, v in inp.items()}
    actq = np.asarray(wl.act_seq_qlen, dtype=np.int64)
    kc = oracle.round_to(oracle.compress(bits["k"], bits["w"], actq, wl.l, wl.d, wl.dtype), wl.dtype)
    vc = oracle.round_to(oracle.compress(bits["v"], bits["w"], actq, wl.l, wl.d, wl.dtype), wl.dtype)
    dout = synth.make_output_grad(wl, device="cuda")
    ref = oracle.attention_backward(bits["q"], kc, vc, synth.bits(dout), actq,
                                    oracle.cmp_prefix(wl.seqlens, wl.l, wl.d), wl.N1, wl.N2, wl.scale,
                                    wl.l, wl.d, wl.dtype)
    c, s = gpu_prefix(wl)
    plan = nsa.nsa_compress_attention_get_workspace(
        wl.act_seq_qlen, c, s, wl.N1, wl.N2, wl.D1, wl.D2, wl.scale, wl.l, wl.d, wl.lsel, wl.count,
        wl.torch_dtype)
    try:
        kc_g, vc_g = upload_bits(kc, wl.dtype), upload_bits(vc, wl.dtype)
        out, mx, sm = nsa.nsa_compress_attention_fwd(plan, inp["q"], kc_g, vc_g)
        dq, dk, dv = nsa.nsa_compress_attention_backward(plan, inp["q"], kc_g, vc_g, out, dout, mx, sm)
        torch.cuda.synchronize()
    finally:
        plan.destroy()
    got = {"dq": dq, "dkc": dk, "dvc": dv}
    for k in keys:
        assert_grad_close(got[k].double().cpu().numpy(), ref[k], k)
    return got


@pytest.mark.parametrize("name,wl,dtype", [(f"w{i}", SMALL[i], "bf16") for i in SMALL] +
                         [("neg", NEG, "bf16"), ("w2-f16", SMALL[2], "f16"), ("long", LONG, "bf16"),
                          ("long-f16", LONG, "f16"), ("long-d192", LONG192, "bf16")])
def test_backward_against_oracle(name, wl, dtype):
    _run(wl.with_dtype(dtype), keys=("dq", "dkc", "dvc"))


@pytest.mark.parametrize("name,wl,dtype", [("w2", SMALL[2], "bf16"), ("w3", SMALL[3], "bf16"),
                                           ("w4", SMALL[4], "bf16"), ("w2-f16", SMALL[2], "f16"),
                                           ("short", dataclasses.replace(SMALL[0], name="short-seqs",
                                                                         seqlens=(5, 0, 31, 32, 47, 200)), "bf16")])
def test_compress_backward_against_oracle(name, wl, dtype):
    """Gradients of the compression (d_input, d_weight) for a seeded float32
    output gradient, against the oracle."""
    wl = wl.with_dtype(dtype)
    log(f"[case] {wl.name}: compress backward")
    inp = synth.make_inputs(wl, device="cuda", tensors=("k", "w"))
    T2 = int(oracle.cmp_prefix(wl.seqlens, wl.l, wl.d)[-1])
    gen = torch.Generator(device="cpu")
    gen.manual_seed(1234)
    dy = torch.randn((T2, wl.N2, wl.D1), generator=gen, dtype=torch.float32)
    ref = oracle.compress_backward(synth.bits(inp["k"]), synth.bits(inp["w"]), dy.double().numpy(),
                                   wl.act_seq_qlen, wl.l, wl.d, wl.dtype)
    dx, dw = nsa.nsa_compress_backward(inp["k"], inp["w"], dy.cuda(), wl.act_seq_qlen, wl.l, wl.d)
    torch.cuda.synchronize()
    assert_grad_close(dx.double().cpu().numpy(), ref["dx"], "d_input")
    assert_grad_close(dw.double().cpu().numpy(), ref["dw"], "d_weight")
    dx2, dw2 = nsa.nsa_compress_backward(inp["k"], inp["w"], dy.cuda(), wl.act_seq_qlen, wl.l, wl.d)
    assert torch.equal(dx, dx2) and torch.equal(dw, dw2)


def test_backward_full_size_properties():
    """The batched varlen workload at its full size, in the launch
    configuration the benchmark times (GPU compression, forward, backward).
    No oracle at this size; instead properties of the derivatives that hold
    exactly at any size:
      * sum over a KV head's compressed entries of d_value equals the sum of
        d_attention_out over its query rows that see at least one block
        (each such row's probabilities sum to 1);
      * sum over the entries of d_key is zero (per row, sum_i dS_i =
        sum_i P_i dP_i - Delta = 0): the residual must sit far below the
        random-walk size of the terms (1/sqrt(#entries) of their summed
        magnitude), so only the rounding of P, dS and out is left;
      * d_query of rows that see no block is exactly zero, all gradients are
        finite, and a second call reproduces every bit."""
    wl = synth.WORKLOADS[4]
    log(f"[case] {wl.name}: full-size backward properties")
    inp = synth.make_inputs(wl, device="cuda")
    kc = nsa.nsa_compress(inp["k"], inp["w"], wl.act_seq_qlen, wl.l, wl.d)
    vc = nsa.nsa_compress(inp["v"], inp["w"], wl.act_seq_qlen, wl.l, wl.d)
    dout = synth.make_output_grad(wl, device="cuda", chunk_rows=16384)
    c, s = gpu_prefix(wl)
    plan = nsa.nsa_compress_attention_get_workspace(
        wl.act_seq_qlen, c, s, wl.N1, wl.N2, wl.D1, wl.D2, wl.scale, wl.l, wl.d, wl.lsel, wl.count,
        wl.torch_dtype)
    try:
        out, mx, sm = nsa.nsa_compress_attention_fwd(plan, inp["q"], kc, vc)
        dq, dk, dv = nsa.nsa_compress_attention_backward(plan, inp["q"], kc, vc, out, dout, mx, sm)
        dq2, dk2, dv2 = nsa.nsa_compress_attention_backward(plan, inp["q"], kc, vc, out, dout, mx, sm)
        torch.cuda.synchronize()
    finally:
        plan.destroy()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), name
    # rows that see a block: local token t >= l - 1
    seen = torch.zeros(wl.T, dtype=torch.bool, device="cuda")
    start = 0
    for T in wl.seqlens:
        seen[start + wl.l - 1:start + T] = True
        start += T
    assert bool((dq[~seen] == 0).all())
    G = wl.N1 // wl.N2
    for g in range(wl.N2):
        want = dout[seen, g * G:(g + 1) * G, :].double().sum((0, 1))
        got = dv[:, g, :].double().sum(0)
        rel = float(torch.linalg.norm(got - want) / torch.linalg.norm(want))
        log(f"  head {g}: |sum dV - sum dout| / |sum dout| = {rel:.3e}")
        assert rel <= 2e-3   # rounding of P to the element type: ~1e-4 seen
        zs = dk[:, g, :].double().sum(0)
        mag = dk[:, g, :].double().abs().sum(0)
        ratio = float(torch.linalg.norm(zs) / torch.linalg.norm(mag))
        walk = 1.0 / np.sqrt(dk.shape[0])
        log(f"  head {g}: |sum dK| / |sum |dK|| = {ratio:.3e} (random walk {walk:.3e})")
        assert ratio <= 0.1 * walk
