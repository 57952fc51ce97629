"""GPU parity of the compression alone ("aclnnNsaCompress", Formula) over
shapes the five workloads do not reach: head dims from 16 to 256 (so column
slabs of 2 to 16 chunks of 16 bytes), several heads, windows from l = d
to l = 8 d, l not a multiple of d, and ragged sequences (empty, shorter
than a window, one window, runs that end mid-run), in bfloat16 and float16.

Each case is compared with the oracle element by element at the
compressed-K/V bound (|gpu - oracle| <= 2e-2 + 1e-2 |oracle|).  Both sides
sum the same exact products; the kernel accumulates in float32 in
ascending window position and rounds once, the oracle sums in float64 and
rounds once, so the two round to the same element-type value except where
the float32 sum lands within its rounding error of a rounding boundary:
at most 1 % of the elements may differ in their bits, and those by one
unit in the last place.
"""
import numpy as np
import pytest
import torch

import kv_compression_block_amd as nsa
import oracle
import synth
from parity import log

pytestmark = pytest.mark.gpu

LENS = [0, 5, 47, 48, 300, 1000, 2013]
CASES = [
    # (N, D, l, d)
    (1, 16, 16, 16),
    (3, 48, 48, 32),
    (2, 80, 128, 16),
    (1, 256, 32, 16),
    (5, 128, 64, 64),
    (4, 192, 64, 32),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("N,D,l,d", CASES)
def test_compress_shapes_against_oracle(N, D, l, d, dtype):
    log(f"[case] compress N={N} D={D} l={l} d={d} {dtype}")
    rng = np.random.default_rng(1000 * N + D + 7 * l + d)
    T = sum(LENS)
    tdt = synth.TORCH_DTYPES[dtype]
    x = torch.tensor(rng.standard_normal((T, N, D)), dtype=torch.float32).to(tdt)
    w = torch.tensor(rng.uniform(0.0, 2.0 / l, (l, N)), dtype=torch.float32).to(tdt)
    act = np.cumsum(LENS).tolist()
    ref = oracle.compress(synth.bits(x), synth.bits(w), act, l, d, dtype)
    got_t = nsa.nsa_compress(x.cuda(), w.cuda(), act, l, d)
    torch.cuda.synchronize()
    assert tuple(got_t.shape) == ref.shape
    got_bits = synth.bits(got_t.cpu())
    got = oracle.widen(got_bits, dtype)
    bad = np.abs(got - ref) > 2e-2 + 1e-2 * np.abs(ref)
    assert not bad.any(), f"{int(bad.sum())} elements outside the bound"
    ref_bits = oracle.round_to(ref, dtype)
    diff = got_bits != ref_bits
    assert diff.mean() <= 0.01, f"{diff.mean():.4f} of the elements differ in their bits"
    if diff.any():
        ulps = np.abs(got_bits[diff].astype(np.int64) - ref_bits[diff].astype(np.int64))
        assert ulps.max() == 1, f"bit differences up to {ulps.max()} units in the last place"
