"""Planning on the device (nsa_compress_attention_device_plan /
nsa_compress_attention_metadata): the table the device derives from device
prefix sums equals the host planner's bit for bit; every call on a
device-planned plan gives bitwise the outputs of the host-planned one; lengths
that fail a check set the status word and leave every output untouched; and
lengths that differ from the plan's but fit it are honoured."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from parity import gpu_prefix, log

import kv_compression_block_amd as nsa

pytestmark = pytest.mark.gpu

WL = synth.small_variant(2, [1000, 2050, 64, 17])            # GQA 16, ragged, one short sequence
MQA = synth.small_variant(1, [1500, 777])


def _host_plan(wl, kv_lens=None):
    """Plan from host prefix sums; kv_lens (per sequence) makes it chunked."""
    lens = kv_lens if kv_lens is not None else wl.seqlens
    c = np.cumsum([nsa.nsa_compress_out_len(T, wl.l, wl.d) for T in lens]).tolist()
    s = np.cumsum([-(-T // wl.lsel) for T in lens]).tolist()
    kv = None if kv_lens is None else np.cumsum(kv_lens).tolist()
    return nsa.nsa_compress_attention_get_workspace(wl.act_seq_qlen, c, s, wl.N1, wl.N2, wl.D1, wl.D2, wl.scale,
                                                    wl.l, wl.d, wl.lsel, wl.count, wl.torch_dtype,
                                                    actual_seq_kvlen=kv)


def _dev(vals):
    return torch.tensor(np.asarray(vals, dtype=np.int64), device="cuda")


def _metadata(dplan, wl, workspace, kv_lens=None, cmp=None, sel=None):
    lens = kv_lens if kv_lens is not None else wl.seqlens
    c = np.cumsum([nsa.nsa_compress_out_len(T, wl.l, wl.d) for T in lens]) if cmp is None else cmp
    s = np.cumsum([-(-T // wl.lsel) for T in lens]) if sel is None else sel
    nsa.nsa_compress_attention_metadata(dplan, _dev(wl.act_seq_qlen), _dev(c), _dev(s), workspace,
                                        actual_seq_kvlen=None if kv_lens is None else _dev(np.cumsum(kv_lens)))


def _status(plan, workspace):
    off = plan.info["status_offset"]
    return int(workspace[off:off + 4].cpu().view(torch.int32)[0])


@pytest.mark.parametrize("chunked", [False, True])
def test_device_table_equals_host_table(chunked):
    """The host path uploads its table (then a zero status word) into the
    workspace; the device planner writes the same bytes from device prefix
    sums."""
    wl = WL
    kv = [T + extra for T, extra in zip(wl.seqlens, (300, 0, 5, 1000))] if chunked else None
    log(f"[case] device table, chunked={chunked}")
    plan = _host_plan(wl, kv)
    dplan = nsa.nsa_compress_attention_device_plan(plan)
    try:
        n = (plan.info["batch"] + 1) * 64
        inp = synth.make_inputs(wl, device="cuda")
        T2 = plan.info["total_cmp_tokens"]
        kc = torch.zeros((T2, wl.N2, wl.D1), dtype=wl.torch_dtype, device="cuda")
        vc = torch.zeros((T2, wl.N2, wl.D2), dtype=wl.torch_dtype, device="cuda")
        ws_h = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
        nsa.nsa_compress_attention_fwd(plan, inp["q"], kc, vc, workspace=ws_h)
        ws_d = torch.full((plan.workspace_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
        ws_d[plan.info["status_offset"]:n] = 0
        _metadata(dplan, wl, ws_d, kv_lens=kv)
        torch.cuda.synchronize()
        assert _status(dplan, ws_d) == 0
        assert torch.equal(ws_h[:n], ws_d[:n]), "device table differs from the host table"
    finally:
        dplan.destroy()
        plan.destroy()


def _outputs(wl, plan, value=7.0):
    i = plan.info
    T1, N1, N2 = i["total_q_tokens"], i["head_num"], i["kv_head_num"]
    return {"attention_out": torch.full((T1, N1, wl.D2), value, dtype=wl.torch_dtype, device="cuda"),
            "topk_indices": torch.full((T1, N2, wl.count), 12345, dtype=torch.int32, device="cuda"),
            "softmax_max": torch.full((T1, N1, 8), value, dtype=torch.float32, device="cuda"),
            "softmax_sum": torch.full((T1, N1, 8), value, dtype=torch.float32, device="cuda")}


def _all_calls(wl, plan, inp, kc, vc, ws_fn, dout):
    """Every call kind on one plan; ws_fn(bytes) gives the workspace."""
    res = {}
    o = _outputs(wl, plan)
    nsa.nsa_compress_attention(plan, inp["q"], kc, vc, workspace=ws_fn(plan.workspace_bytes), outputs=o)
    res.update({f"full.{k}": v for k, v in o.items()})
    need = nsa.nsa_compress_attention_split_workspace(plan, 2)
    out, mx, sm = nsa.nsa_compress_attention_fwd_split(plan, inp["q"], kc, vc, 2, workspace=ws_fn(need))
    res.update({"split.out": out, "split.max": mx, "split.sum": sm})
    out_s, lse = nsa.nsa_select_attention(plan, inp["q"], inp["k"], inp["v"], o["topk_indices"],
                                          workspace=ws_fn(plan.workspace_bytes))
    res.update({"select.out": out_s, "select.lse": lse})
    dq, dk, dv = nsa.nsa_compress_attention_backward(plan, inp["q"], kc, vc, o["attention_out"], dout,
                                                     o["softmax_max"], o["softmax_sum"],
                                                     workspace=ws_fn(plan.info["backward_workspace_bytes"]))
    res.update({"bwd.dq": dq, "bwd.dk": dk, "bwd.dv": dv})
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("wl", [WL, MQA], ids=["gqa16", "mqa"])
def test_device_planned_calls_match_host_planned_bitwise(wl):
    log(f"[case] device-planned calls, {wl.name}")
    inp = synth.make_inputs(wl, device="cuda")
    kc = nsa.nsa_compress(inp["k"], inp["w"], wl.act_seq_qlen, wl.l, wl.d)
    vc = nsa.nsa_compress(inp["v"], inp["w"], wl.act_seq_qlen, wl.l, wl.d)
    dout = synth.make_output_grad(wl, device="cuda")
    plan = _host_plan(wl)
    dplan = nsa.nsa_compress_attention_device_plan(plan)
    try:
        host = _all_calls(wl, plan, inp, kc, vc, lambda n: torch.empty(n, dtype=torch.uint8, device="cuda"), dout)
        # one workspace, large enough for every call, holding the metadata
        big = max(nsa.nsa_compress_attention_split_workspace(plan, 2), plan.info["backward_workspace_bytes"])
        ws = torch.empty(big, dtype=torch.uint8, device="cuda")
        _metadata(dplan, wl, ws)
        dev = _all_calls(wl, dplan, inp, kc, vc, lambda n: ws, dout)
        assert _status(dplan, ws) == 0
    finally:
        dplan.destroy()
        plan.destroy()
    for k in host:
        assert torch.equal(host[k], dev[k]), k


def test_device_plan_rejects_lengths_that_fail_a_check():
    """A wrong compressed length (one sequence off by one) sets bit 4 of
    the status word; every call on that workspace then leaves its outputs as
    they were."""
    wl = WL
    log("[case] device plan, bad lengths")
    inp = synth.make_inputs(wl, device="cuda")
    kc = nsa.nsa_compress(inp["k"], inp["w"], wl.act_seq_qlen, wl.l, wl.d)
    vc = nsa.nsa_compress(inp["v"], inp["w"], wl.act_seq_qlen, wl.l, wl.d)
    plan = _host_plan(wl)
    dplan = nsa.nsa_compress_attention_device_plan(plan)
    try:
        c, s = gpu_prefix(wl)
        bad = np.array(c, dtype=np.int64)
        bad[1:] += 1                                      # sequence 1 one entry too long
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
        _metadata(dplan, wl, ws, cmp=bad)
        o = _outputs(wl, dplan)
        nsa.nsa_compress_attention(dplan, inp["q"], kc, vc, workspace=ws, outputs=o)
        torch.cuda.synchronize()
        st = _status(dplan, ws)
        log(f"  status word {st:#x}")
        assert st & 4, st
        ref = _outputs(wl, dplan)
        for k in o:
            assert torch.equal(o[k], ref[k]), f"{k} was written despite the failed check"
    finally:
        dplan.destroy()
        plan.destroy()


def test_device_plan_honours_other_lengths_that_fit():
    """Lengths in another order give the same totals and launch sizes: the
    device plan made from [1000, 2050, 64, 17] then computes exactly what a
    host plan made from the new lengths computes."""
    wl = WL
    other = dataclasses.replace(wl, seqlens=(2050, 17, 1000, 64), name=wl.name + "-reordered")
    log("[case] device plan, reordered lengths")
    inp = synth.make_inputs(other, device="cuda")
    kc = nsa.nsa_compress(inp["k"], inp["w"], other.act_seq_qlen, other.l, other.d)
    vc = nsa.nsa_compress(inp["v"], inp["w"], other.act_seq_qlen, other.l, other.d)
    plan = _host_plan(wl)
    dplan = nsa.nsa_compress_attention_device_plan(plan)
    plan2 = _host_plan(other)
    try:
        ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device="cuda")
        _metadata(dplan, other, ws)
        got = nsa.nsa_compress_attention(dplan, inp["q"], kc, vc, workspace=ws)
        ref = nsa.nsa_compress_attention(plan2, inp["q"], kc, vc)
        torch.cuda.synchronize()
        assert _status(dplan, ws) == 0
    finally:
        plan2.destroy()
        dplan.destroy()
        plan.destroy()
    for a, b, k in zip(got, ref, ("out", "topk", "max", "sum")):
        assert torch.equal(a, b), k
