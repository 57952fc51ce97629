"""Chunked prefill on the GPU (nsa_compress_attention_get_workspace_kv):
each sequence's queries are the last Tq of its Tkv key/value tokens and
both causal rules are aligned bottom-right.  Parity against the oracle's
chunked mode (outputs, P_slc', top-k), on the oracle's compressed K/V, and
against the GPU's own full-prefill rows (bit for bit: a row's work does not
depend on which other rows share its workgroup); then every other call on
a chunked plan against the oracle's chunked mode: explicit masks (one mask
row per query), the split launch, selected-block attention over the raw
key/value tokens, and the backward."""
import functools
import zlib

import numpy as np
import pytest
import torch

import oracle
from parity import (assert_close_out, assert_pslc, assert_softmax_stats, log, to_f64, upload_bits)
from test_gpu_backward import assert_grad_close
from test_gpu_select_attn import _compare as compare_select

import kv_compression_block_amd as nsa

pytestmark = pytest.mark.gpu

CASES = {
    # N1, N2, D1, D2, l, d, lsel, count, scale, kv_lens, q_lens
    "gqa-d64": (8, 2, 64, 64, 32, 16, 64, 4, 0.125, [700, 333, 64, 45], [150, 333, 10, 45]),
    "group64-d128": (64, 1, 128, 128, 32, 16, 64, 16, 128 ** -0.5, [1500, 900], [300, 1]),
    "long-stride": (16, 1, 192, 128, 64, 32, 128, 8, 192 ** -0.5, [2100], [700]),
}


def _bits(rng, shape, std=1.0):
    return torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _plan(N1, N2, D1, D2, l, d, lsel, count, scale, kv_lens, q_lens):
    c = np.cumsum([nsa.nsa_compress_out_len(T, l, d) for T in kv_lens]).tolist()
    s = np.cumsum([-(-T // lsel) for T in kv_lens]).tolist()
    kv = np.cumsum(kv_lens).tolist() if kv_lens is not None else None
    return nsa.nsa_compress_attention_get_workspace(np.cumsum(q_lens).tolist(), c, s, N1, N2, D1, D2, scale,
                                                    l, d, lsel, count, torch.bfloat16, actual_seq_kvlen=kv)


def _topk_check(g_idx, r_idx, r_pslc, tie_rel=1e-4):
    for k in range(g_idx.shape[0]):
        for g in range(g_idx.shape[1]):
            gi, ri = g_idx[k, g], r_idx[k, g]
            kk = int((ri >= 0).sum())
            assert np.all(gi[kk:] == -1) and np.all(gi[:kk] >= 0), (k, g, gi, ri)
            assert len(set(gi[:kk].tolist())) == kk
            if kk == 0:
                continue
            ref = set(ri[:kk].tolist())
            sc = r_pslc[k, g].astype(np.float32).astype(np.float64)
            kth = min(sc[j] for j in ref)
            for pk in gi[:kk]:
                assert pk in ref or sc[pk] >= kth * (1 - tie_rel), (k, g, pk)


@pytest.mark.parametrize("name", sorted(CASES))
def test_chunked_prefill(name):
    N1, N2, D1, D2, l, d, lsel, count, scale, kv_lens, q_lens = CASES[name]
    log(f"[case] chunked {name}: kv {kv_lens} q {q_lens}")
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    k = _bits(rng, (sum(kv_lens), N2, D1))
    v = _bits(rng, (sum(kv_lens), N2, D2))
    w = _bits(rng, (l, N2), std=1.0 / l)
    q_full = _bits(rng, (sum(kv_lens), N1, D1))
    actkv = np.cumsum(kv_lens).astype(np.int64)
    kc = oracle.round_to(oracle.compress(k, w, actkv, l, d))
    vc = oracle.round_to(oracle.compress(v, w, actkv, l, d))
    starts = np.concatenate([[0], actkv[:-1]])
    rows = np.concatenate([s + np.arange(T - Tq, T) for s, T, Tq in zip(starts, kv_lens, q_lens)]).astype(np.int64)
    q_chunk = np.ascontiguousarray(q_full[rows])
    actc = oracle.cmp_prefix(kv_lens, l, d)
    ref = oracle.attention(q_chunk, np.arange(sum(q_lens), dtype=np.int64), kc, vc, np.cumsum(q_lens), actc,
                           N1, N2, scale, l, d, lsel, count, act_seq_kvlen=actkv)
    kc_g, vc_g = upload_bits(kc), upload_bits(vc)
    plan = _plan(N1, N2, D1, D2, l, d, lsel, count, scale, kv_lens, q_lens)
    try:
        out, topk, mx, sm, pslc = nsa.nsa_compress_attention(plan, upload_bits(q_chunk), kc_g, vc_g,
                                                             return_p_slc=True)
        torch.cuda.synchronize()
    finally:
        plan.destroy()
    assert_close_out(to_f64(out), ref["out"], "attention_out")
    assert_softmax_stats(mx.cpu().numpy(), sm.cpu().numpy(), ref["max"], ref["sum"])
    assert_pslc(pslc.cpu().numpy(), ref["pslc"])
    _topk_check(topk.cpu().numpy(), ref["topk"], ref["pslc"])
    # the same rows of the full prefill, computed by the GPU
    plan = _plan(N1, N2, D1, D2, l, d, lsel, count, scale, kv_lens, kv_lens)
    try:
        f_out, f_topk, f_mx, f_sm, f_pslc = nsa.nsa_compress_attention(plan, upload_bits(q_full), kc_g, vc_g,
                                                                       return_p_slc=True)
        torch.cuda.synchronize()
    finally:
        plan.destroy()
    r = torch.from_numpy(rows).cuda()
    assert torch.equal(out, f_out[r]) and torch.equal(mx, f_mx[r]) and torch.equal(sm, f_sm[r])
    assert torch.equal(topk, f_topk[r])
    assert torch.equal(pslc, f_pslc[r][..., :pslc.shape[-1]])


@functools.lru_cache(maxsize=None)
def _case(name):
    """Inputs of a chunked case: raw K/V of all key/value tokens, the
    queries of the chunks, the oracle's compressed K/V (rounded)."""
    N1, N2, D1, D2, l, d, lsel, count, scale, kv_lens, q_lens = CASES[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    k = _bits(rng, (sum(kv_lens), N2, D1))
    v = _bits(rng, (sum(kv_lens), N2, D2))
    w = _bits(rng, (l, N2), std=1.0 / l)
    q_full = _bits(rng, (sum(kv_lens), N1, D1))
    actkv = np.cumsum(kv_lens).astype(np.int64)
    kc = oracle.round_to(oracle.compress(k, w, actkv, l, d))
    vc = oracle.round_to(oracle.compress(v, w, actkv, l, d))
    starts = np.concatenate([[0], actkv[:-1]])
    rows = np.concatenate([s + np.arange(T - Tq, T) for s, T, Tq in zip(starts, kv_lens, q_lens)]).astype(np.int64)
    q_chunk = np.ascontiguousarray(q_full[rows])
    return dict(k=k, v=v, kc=kc, vc=vc, q=q_chunk, actkv=actkv, actq=np.cumsum(q_lens).astype(np.int64),
                actc=oracle.cmp_prefix(kv_lens, l, d), tokens=np.arange(sum(q_lens), dtype=np.int64))


def _oracle_fwd(name, **masks):
    N1, N2, D1, D2, l, d, lsel, count, scale, kv_lens, q_lens = CASES[name]
    c = _case(name)
    return oracle.attention(c["q"], c["tokens"], c["kc"], c["vc"], c["actq"], c["actc"], N1, N2, scale, l, d, lsel,
                            count, act_seq_kvlen=c["actkv"], **masks)


@pytest.mark.parametrize("name", sorted(CASES))
def test_chunked_explicit_masks(name):
    """One mask row per query (row t for the sequence's t-th query), random
    masks: the masked calls on a chunked plan against the oracle given the
    same masks and the same key/value positions."""
    N1, N2, D1, D2, l, d, lsel, count, scale, kv_lens, q_lens = CASES[name]
    log(f"[case] chunked {name}: explicit masks")
    c = _case(name)
    rng = np.random.default_rng(zlib.crc32(name.encode()) + 1)
    t_max = max(q_lens)
    ncm = max(nsa.nsa_compress_out_len(T, l, d) for T in kv_lens)
    smax_ = max(-(-T // lsel) for T in kv_lens)
    am = rng.random((t_max, ncm)) < 0.3
    tm = rng.random((t_max, smax_)) < 0.3
    ref = _oracle_fwd(name, atten_mask=am, topk_mask=tm)
    plan = _plan(N1, N2, D1, D2, l, d, lsel, count, scale, kv_lens, q_lens)
    try:
        out, topk, mx, sm, pslc = nsa.nsa_compress_attention(
            plan, upload_bits(c["q"]), upload_bits(c["kc"]), upload_bits(c["vc"]), return_p_slc=True,
            atten_mask=torch.from_numpy(am).cuda(), topk_mask=torch.from_numpy(tm).cuda())
        torch.cuda.synchronize()
    finally:
        plan.destroy()
    assert_close_out(to_f64(out), ref["out"], "attention_out")
    assert_softmax_stats(mx.cpu().numpy(), sm.cpu().numpy(), ref["max"], ref["sum"])
    assert_pslc(pslc.cpu().numpy(), ref["pslc"])
    _topk_check(topk.cpu().numpy(), ref["topk"], ref["pslc"])


@pytest.mark.parametrize("tiles", [1, 3])
@pytest.mark.parametrize("name", sorted(CASES))
def test_chunked_split_launch(name, tiles):
    N1, N2, D1, D2, l, d, lsel, count, scale, kv_lens, q_lens = CASES[name]
    log(f"[case] chunked {name}: split launch, {tiles} key tiles per piece")
    c = _case(name)
    ref = _oracle_fwd(name)
    plan = _plan(N1, N2, D1, D2, l, d, lsel, count, scale, kv_lens, q_lens)
    try:
        out, mx, sm = nsa.nsa_compress_attention_fwd_split(plan, upload_bits(c["q"]), upload_bits(c["kc"]),
                                                           upload_bits(c["vc"]), tiles)
        torch.cuda.synchronize()
    finally:
        plan.destroy()
    assert_close_out(to_f64(out), ref["out"], "attention_out")
    assert_softmax_stats(mx.cpu().numpy(), sm.cpu().numpy(), ref["max"], ref["sum"])


@pytest.mark.parametrize("name", sorted(CASES))
def test_chunked_select_attention(name):
    """Selected-block attention on a chunked plan: the raw key/value tensors
    hold every key/value token, query t of a sequence attends to listed keys
    at positions <= Tkv - Tq + t.  Block lists: the compressed branch's own
    chunked top-k, with some entries replaced by -1 and by repeats."""
    N1, N2, D1, D2, l, d, lsel, count, scale, kv_lens, q_lens = CASES[name]
    log(f"[case] chunked {name}: selected-block attention")
    c = _case(name)
    lists = _oracle_fwd(name)["topk"].copy()
    rng = np.random.default_rng(5)
    u = rng.random(lists.shape)
    lists = np.where(u < 0.1, -1, np.where(u < 0.15, np.roll(lists, 1, axis=2), lists)).astype(np.int32)
    ref = oracle.select_attention(c["q"], c["k"], c["v"], lists, c["actq"], N1, N2, scale, lsel,
                                  act_seq_kvlen=c["actkv"])
    plan = _plan(N1, N2, D1, D2, l, d, lsel, count, scale, kv_lens, q_lens)
    try:
        out, lse = nsa.nsa_select_attention(plan, upload_bits(c["q"]), upload_bits(c["k"]), upload_bits(c["v"]),
                                            torch.from_numpy(lists).cuda())
        torch.cuda.synchronize()
    finally:
        plan.destroy()
    compare_select(out, lse, ref)


@pytest.mark.parametrize("name", sorted(CASES))
def test_chunked_backward(name):
    N1, N2, D1, D2, l, d, lsel, count, scale, kv_lens, q_lens = CASES[name]
    log(f"[case] chunked {name}: backward")
    c = _case(name)
    rng = np.random.default_rng(zlib.crc32(name.encode()) + 2)
    dout = _bits(rng, (sum(q_lens), N1, D2))
    ref = oracle.attention_backward(c["q"], c["kc"], c["vc"], dout, c["actq"], c["actc"], N1, N2, scale, l, d,
                                    act_seq_kvlen=c["actkv"])
    plan = _plan(N1, N2, D1, D2, l, d, lsel, count, scale, kv_lens, q_lens)
    try:
        q, kc, vc = upload_bits(c["q"]), upload_bits(c["kc"]), upload_bits(c["vc"])
        out, mx, sm = nsa.nsa_compress_attention_fwd(plan, q, kc, vc)
        dq, dk, dv = nsa.nsa_compress_attention_backward(plan, q, kc, vc, out, upload_bits(dout), mx, sm)
        torch.cuda.synchronize()
    finally:
        plan.destroy()
    for key, got in (("dq", dq), ("dkc", dk), ("dvc", dv)):
        assert_grad_close(got.double().cpu().numpy(), ref[key], key)
