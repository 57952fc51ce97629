"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the oracle, to the tolerances stated below.

Tolerances:
* compressed K/V and attention_out: |gpu - oracle| <= 2e-2 + 1e-2 |oracle|
  (elementwise, the allclose form of max-abs 2e-2 / rel 1e-2);
* importance scores P_slc': |gpu - oracle| <= 1e-3 |oracle| + 1e-7, and exact
  zeros where the oracle is exactly zero;
* softmax max: |gpu - oracle| <= 1e-3 absolute, -inf matched exactly;
  softmax sum: relative 1e-3, 0 matched exactly;
* top-k, per (token, KV head) row: exactly min(count, #candidates) picks,
  the rest -1; picks are candidates and unique; every pick outside the
  oracle's set has an oracle score >= (1 - 1e-4) * the oracle's k-th
  score.

Every comparison feeds the oracle exactly the compressed K/V the GPU's
attention consumed: staged runs give the GPU the oracle's rounded
compression, end-to-end runs give the oracle the GPU's own compression
(its bit patterns).  The compression itself is compared with the oracle's
separately, at the compressed-K/V bound.  The same bounds serve both
element types: float16 keeps three more significant bits than bfloat16
everywhere the kernels round (P before P.V, O, compressed K/V).
"""
from __future__ import annotations

import numpy as np
import torch

import kv_compression_block_amd as nsa
import oracle
import synth

OUT_ATOL, OUT_RTOL = 2e-2, 1e-2
PSLC_RTOL, PSLC_ATOL = 1e-3, 1e-7
MAX_ATOL = 1e-3
SUM_RTOL = 1e-3


def log(msg: str) -> None:
    print(msg, flush=True)


def dtype_name(t: torch.Tensor) -> str:
    return {torch.bfloat16: "bf16", torch.float16: "f16"}[t.dtype]


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a bfloat16 or float16 tensor, widened by the
    oracle's decoder of that type."""
    return oracle.widen(synth.bits(t), dtype_name(t))


bf16_to_f64 = to_f64


def upload_bits(bits: np.ndarray, dtype: str = "bf16", device="cuda") -> torch.Tensor:
    return synth.from_bits(bits, dtype).to(device)


def gpu_compress(wl, x: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    return nsa.nsa_compress(x, w, wl.act_seq_qlen, wl.l, wl.d)


def gpu_prefix(wl):
    """Compressed and select prefix sums as the C library counts them."""
    c, s, pc, ps = [], [], 0, 0
    for T in wl.seqlens:
        pc += nsa.nsa_compress_out_len(T, wl.l, wl.d)
        ps += -(-T // wl.lsel)
        c.append(pc)
        s.append(ps)
    return c, s


def gpu_attention(wl, q, kc, vc, return_p_slc=True):
    c, s = gpu_prefix(wl)
    plan = nsa.nsa_compress_attention_get_workspace(
        wl.act_seq_qlen, c, s, wl.N1, wl.N2, wl.D1, wl.D2, wl.scale, wl.l, wl.d, wl.lsel, wl.count,
        q.dtype)
    try:
        res = nsa.nsa_compress_attention(plan, q, kc, vc, return_p_slc=return_p_slc)
        torch.cuda.synchronize()
    finally:
        plan.destroy()
    keys = ["out", "topk", "max", "sum", "pslc"]
    return dict(zip(keys, res))


def err_stats(got: np.ndarray, ref: np.ndarray):
    d = np.abs(got - ref)
    rel = d / np.maximum(np.abs(ref), 1e-30)
    return float(d.max(initial=0.0)), float(rel.max(initial=0.0))


def assert_close_out(got: np.ndarray, ref: np.ndarray, what: str):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    bad = np.abs(got - ref) > OUT_ATOL + OUT_RTOL * np.abs(ref)
    mabs, mrel = err_stats(got, ref)
    log(f"  {what}: max|err| {mabs:.3e}  max rel {mrel:.3e}  n={got.size}")
    assert not bad.any(), f"{what}: {int(bad.sum())} elements outside 2e-2 + 1e-2|ref|; first at {np.argwhere(bad)[0]}"


def assert_softmax_stats(gmax: np.ndarray, gsum: np.ndarray, rmax: np.ndarray, rsum: np.ndarray,
                         max_atol: float = MAX_ATOL, sum_rtol: float = SUM_RTOL):
    """gmax/gsum: [n, N1, 8] float32 from the GPU; rmax/rsum: [n, N1] oracle."""
    for k in range(8):
        assert np.array_equal(gmax[..., k], gmax[..., 0]) and np.array_equal(gsum[..., k], gsum[..., 0])
    gm, gs = gmax[..., 0].astype(np.float64), gsum[..., 0].astype(np.float64)
    ninf = np.isneginf(rmax)
    assert np.array_equal(np.isneginf(gm), ninf), "softmax_max: -inf rows differ"
    assert np.all(gs[ninf] == 0) and np.all(rsum[ninf] == 0)
    fin = ~ninf
    if fin.any():
        dm = np.abs(gm[fin] - rmax[fin])
        ds = np.abs(gs[fin] - rsum[fin]) / rsum[fin]
        log(f"  softmax max: max|err| {dm.max():.3e}; sum: max rel {ds.max():.3e}")
        assert dm.max() <= max_atol
        assert ds.max() <= sum_rtol


def assert_pslc(gp: np.ndarray, rp: np.ndarray, rtol: float = PSLC_RTOL):
    """[n, N2, S] both; S of the GPU may exceed nothing: same stride."""
    assert gp.shape == rp.shape, (gp.shape, rp.shape)
    zero = rp == 0
    assert np.all(gp[zero] == 0), f"P_slc: {int((gp[zero] != 0).sum())} non-zeros where the oracle is 0"
    bad = np.abs(gp - rp) > rtol * np.abs(rp) + PSLC_ATOL
    mabs, mrel = err_stats(gp[~zero], rp[~zero])
    log(f"  P_slc: max|err| {mabs:.3e}  max rel {mrel:.3e}")
    assert not bad.any(), f"P_slc: {int(bad.sum())} outside tolerance; first at {np.argwhere(bad)[0]}"


def workgroup_runs(wl, run: int = 16) -> np.ndarray:
    """Global tokens of whole workgroups at full size: per sequence three
    runs of ``run`` tokens that start at multiples of ``run`` -- the first,
    one in the middle and the last (possibly partial) one.  Workgroups of
    both kernels start at multiples of their token count (128 / G tokens for
    the attention kernel, 256 / G' for the top-k kernel, G' = G padded to a
    power of two), so with 16-token runs and groups of 16 or more every
    workgroup that touches a run has all its rows in it."""
    starts = np.concatenate([[0], np.cumsum(wl.seqlens)[:-1]])
    picks = []
    for s0, T in zip(starts, wl.seqlens):
        if T == 0:
            continue
        for a in (0, (T // 2) // run * run, (T - 1) // run * run):
            picks.extend(range(int(s0 + a), int(s0 + min(T, a + run))))
    return np.unique(np.array(picks, dtype=np.int64))


def token_meta(wl, tokens):
    """(local position, select-block count) of each global token."""
    starts = np.concatenate([[0], np.cumsum(wl.seqlens)[:-1]])
    ends = np.cumsum(wl.seqlens)
    out = []
    for tg in tokens:
        b = int(np.searchsorted(ends, tg, side="right"))
        T = wl.seqlens[b]
        out.append((int(tg - starts[b]), -(-T // wl.lsel)))
    return out


def assert_topk(wl, tokens, g_idx: np.ndarray, r_idx: np.ndarray, r_pslc: np.ndarray, tie_rel: float = 1e-4,
                topk_mask=None):
    """g_idx/r_idx: [n, N2, count]; r_pslc: oracle scores [n, N2, S].
    Candidates: j*l' <= t, or the unmasked j < S of row t of ``topk_mask``."""
    meta = token_meta(wl, tokens)
    n_diff = 0
    for k, (t, S) in enumerate(meta):
        if topk_mask is None:
            cands = set(range(min(t // wl.lsel + 1, S)))
        else:
            cands = set(int(j) for j in np.flatnonzero(~np.asarray(topk_mask[t, :S], dtype=bool)))
        nvalid = len(cands)
        kk = min(wl.count, nvalid)
        for g in range(wl.N2):
            gi = g_idx[k, g]
            ri = r_idx[k, g]
            assert np.all(gi[kk:] == -1), (tokens[k], g, gi)
            picks = gi[:kk]
            assert all(int(x) in cands for x in picks), (tokens[k], g, gi)
            assert len(set(picks.tolist())) == kk, (tokens[k], g, gi)
            if kk == 0:
                continue
            ref_set = set(ri[:kk].tolist())
            scores = r_pslc[k, g].astype(np.float32).astype(np.float64)
            kth = min(scores[j] for j in ref_set)
            for pk in picks:
                if pk not in ref_set:
                    n_diff += 1
                    assert scores[pk] >= kth * (1 - tie_rel), \
                        f"token {tokens[k]} g {g}: pick {pk} score {scores[pk]} < k-th {kth}"
    log(f"  top-k: {len(meta) * wl.N2} rows, {n_diff} near-tie substitutions")
