"""The importance pass (steps 4-7 of "mindspore.ops.nsa_compress_attention")
takes each row's softmax statistics either from softmax_max / softmax_sum or
from the per-row base-2 log-normaliser max * log2(e) + log2(sum) that every
forward call leaves in its workspace.  Both routes give the same top-k and
importance scores bit for bit: after the single-pass forward (the full call
takes the workspace route, so it must equal the two halves too), the split
forward, the masked forward, and at full size in the bench's launch."""
import numpy as np
import pytest
import torch

import synth
from parity import gpu_prefix, log
from test_gpu_parity import LOOP, SMALL

import kv_compression_block_amd as nsa

pytestmark = pytest.mark.gpu


def _plan(wl):
    c, s = gpu_prefix(wl)
    return nsa.nsa_compress_attention_get_workspace(
        wl.act_seq_qlen, c, s, wl.N1, wl.N2, wl.D1, wl.D2, wl.scale, wl.l, wl.d, wl.lsel, wl.count,
        wl.torch_dtype)


def _kv(wl, inp):
    kc = nsa.nsa_compress(inp["k"], inp["w"], wl.act_seq_qlen, wl.l, wl.d)
    vc = nsa.nsa_compress(inp["v"], inp["w"], wl.act_seq_qlen, wl.l, wl.d)
    return kc, vc


def _both_routes(plan, q, kc, ws, mx, sm, **masks):
    """Top-k and P_slc' from the explicit statistics and from the workspace."""
    a = nsa.nsa_compress_attention_select(plan, q, kc, mx, sm, workspace=ws, return_p_slc=True, **masks)
    b = nsa.nsa_compress_attention_select(plan, q, kc, None, None, workspace=ws, return_p_slc=True, **masks)
    torch.cuda.synchronize()
    return a, b


def _equal(a, b, what):
    for name, x, y in (("topk", a[0], b[0]), ("p_slc", a[1], b[1])):
        assert torch.equal(x, y), f"{what}: {name} differs between the two statistics routes"


def _case(wl, split_tiles=0):
    log(f"[case] {wl.name} ({wl.dtype}): statistics routes, split_tiles={split_tiles}")
    inp = synth.make_inputs(wl, device="cuda")
    kc, vc = _kv(wl, inp)
    plan = _plan(wl)
    try:
        if split_tiles:
            need = nsa.nsa_compress_attention_split_workspace(plan, split_tiles)
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            out, mx, sm = nsa.nsa_compress_attention_fwd_split(plan, inp["q"], kc, vc, split_tiles, workspace=ws)
        else:
            ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
            out, mx, sm = nsa.nsa_compress_attention_fwd(plan, inp["q"], kc, vc, workspace=ws)
        a, b = _both_routes(plan, inp["q"], kc, ws, mx, sm)
        _equal(a, b, wl.name)
        if not split_tiles:
            full = nsa.nsa_compress_attention(plan, inp["q"], kc, vc, return_p_slc=True)
            torch.cuda.synchronize()
            for name, x, y in (("out", full[0], out), ("topk", full[1], a[0]), ("max", full[2], mx),
                               ("sum", full[3], sm), ("p_slc", full[4], a[1])):
                assert torch.equal(x, y), f"{wl.name}: full call's {name} differs from the two halves"
    finally:
        plan.destroy()


@pytest.mark.parametrize("wid", [0, 1, 2, 3, 4])
def test_routes_equal_small(wid):
    _case(SMALL[wid])


@pytest.mark.parametrize("name", ["gqa16-d128", "group64-d128"])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_routes_equal_loop_shapes(name, dtype):
    _case(LOOP[name].with_dtype(dtype))


@pytest.mark.parametrize("wid,tiles", [(1, 1), (3, 3), (4, 3)])
def test_routes_equal_after_split_forward(wid, tiles):
    _case(SMALL[wid], split_tiles=tiles)


def test_routes_equal_after_masked_forward():
    wl = SMALL[2]
    log(f"[case] {wl.name}: statistics routes after the masked forward")
    inp = synth.make_inputs(wl, device="cuda")
    kc, vc = _kv(wl, inp)
    rng = np.random.default_rng(11)
    T_max = max(wl.seqlens)
    nc_max = max(nsa.nsa_compress_out_len(t, wl.l, wl.d) for t in wl.seqlens)
    s_max = max(-(-t // wl.lsel) for t in wl.seqlens)
    am = torch.from_numpy(rng.random((T_max, nc_max)) < 0.3).cuda()
    tm = torch.from_numpy(rng.random((T_max, s_max)) < 0.3).cuda()
    plan = _plan(wl)
    try:
        ws = torch.empty(plan.info["masked_workspace_bytes"], dtype=torch.uint8, device="cuda")
        out, mx, sm = nsa.nsa_compress_attention_fwd(plan, inp["q"], kc, vc, workspace=ws, atten_mask=am)
        a, b = _both_routes(plan, inp["q"], kc, ws, mx, sm, atten_mask=am, topk_mask=tm)
        _equal(a, b, wl.name + " masked")
    finally:
        plan.destroy()


def test_routes_equal_full_size_batched():
    """The batched workload at full size, in the launch the bench times."""
    _case(synth.WORKLOADS[4])
