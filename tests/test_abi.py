"""The C-ABI library loads, exports what include/nsa_cmp.h declares, and
rejects every invalid argument with the documented status before touching a
device (these tests make no compute call and need no GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import kv_compression_block_amd as nsa
from kv_compression_block_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nsa_cmp.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nsa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = _lib.load()
    declared = header_functions()
    assert declared == sorted(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_symbols_visible_in_dynamic_table():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    for name in header_functions():
        assert re.search(rf"\bT {name}$", out, re.M), name


@pytest.mark.parametrize("T,l,d,n", [(0, 32, 16, 0), (31, 32, 16, 0), (32, 32, 16, 1), (48, 32, 16, 2),
                                     (8192, 32, 16, 511), (65536, 64, 32, 2047), (5, 0, 16, -1),
                                     (-1, 32, 16, -1)])
def test_compress_out_len(T, l, d, n):
    assert _lib.load().nsa_compress_out_len(T, l, d) == n


def _arr(vals):
    return (ctypes.c_int64 * len(vals))(*vals)


def _ws(B, qlen, clen, slen, N1=16, N2=1, D1=128, D2=128, scale=0.1, l=32, d=16, lsel=64, cnt=16, dtype=0):
    ws = ctypes.c_size_t(0)
    plan = ctypes.c_void_p(0)
    st = _lib.load().nsa_compress_attention_get_workspace(
        B, _arr(qlen) if qlen is not None else None, _arr(clen) if clen is not None else None,
        _arr(slen) if slen is not None else None, N1, N2, D1, D2, scale, l, d, lsel, cnt, dtype,
        ctypes.byref(ws), ctypes.byref(plan))
    return st, ws.value, plan


def _good(**kw):
    base = dict(B=2, qlen=[100, 300], clen=[5, 16], slen=[2, 6])
    base.update(kw)
    return base


@pytest.mark.parametrize("dtype", [_lib.NSA_DTYPE_BF16, _lib.NSA_DTYPE_FP16])
def test_get_workspace_ok_and_plan_info(dtype):
    st, ws, plan = _ws(**_good(dtype=dtype))
    assert st == _lib.NSA_OK and plan.value and ws > 0
    info = _lib.PlanInfo()
    assert _lib.load().nsa_plan_get_info(plan, ctypes.byref(info)) == 0
    assert (info.total_q_tokens, info.total_cmp_tokens, info.total_sel_blocks, info.max_sel_blocks) == (300, 16, 6, 4)
    assert info.dtype == dtype
    _lib.load().nsa_plan_destroy(plan)


CONSTRAINT_CASES = [
    dict(l=24), dict(l=0), dict(l=144), dict(d=8), dict(d=80), dict(lsel=72), dict(lsel=144),
    dict(cnt=0), dict(cnt=33), dict(l=32, d=48), dict(lsel=16, l=32), dict(l=48, d=32, lsel=48),
    dict(D1=100), dict(D2=40), dict(D1=64, D2=128), dict(N1=6, N2=4), dict(N1=2, N2=4), dict(N2=0),
    dict(scale=float("inf")), dict(scale=float("nan")),
]


@pytest.mark.parametrize("kw", CONSTRAINT_CASES)
def test_get_workspace_constraint_violations(kw):
    args = _good()
    args.update(kw)
    st, _, plan = _ws(**args)
    assert st == _lib.NSA_ERR_CONSTRAINT, _lib.load().nsa_last_error()
    assert not plan.value
    assert _lib.load().nsa_last_error()


@pytest.mark.parametrize("kw", [
    dict(qlen=[100, 90], clen=[5, 5], slen=[2, 2]),          # decreasing prefix sums
    dict(clen=[5, 17]),                                      # wrong compressed length
    dict(slen=[2, 5]),                                       # wrong select length
    dict(B=0, qlen=[0], clen=[0], slen=[0]),                 # empty
])
def test_get_workspace_shape_errors(kw):
    args = _good()
    args.update(kw)
    st, _, plan = _ws(**args)
    assert st == _lib.NSA_ERR_SHAPE, _lib.load().nsa_last_error()
    assert not plan.value


def test_get_workspace_nullptr_dtype_unsupported():
    assert _ws(**_good(qlen=None))[0] == _lib.NSA_ERR_NULLPTR
    assert _ws(**_good(dtype=7))[0] == _lib.NSA_ERR_DTYPE
    assert _ws(**_good(D1=256, D2=128))[0] == _lib.NSA_ERR_UNSUPPORTED     # legal, not built
    assert _ws(**_good(N1=128, N2=1))[0] == _lib.NSA_ERR_UNSUPPORTED       # group > 64


def test_compute_call_rejects_before_touching_the_device():
    st, ws, plan = _ws(**_good())
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    # NULL outputs
    assert lib.nsa_compress_attention(plan, fake, fake, fake, None, fake, fake, fake, None, fake, ws, None) \
        == _lib.NSA_ERR_NULLPTR
    # workspace too small
    assert lib.nsa_compress_attention(plan, fake, fake, fake, fake, fake, fake, fake, None, fake, ws - 1, None) \
        == _lib.NSA_ERR_WORKSPACE
    # misaligned query
    odd = ctypes.c_void_p(0x1002)
    assert lib.nsa_compress_attention(plan, odd, fake, fake, fake, fake, fake, fake, None, fake, ws, None) \
        == _lib.NSA_ERR_CONSTRAINT
    assert lib.nsa_compress_attention(None, fake, fake, fake, fake, fake, fake, fake, None, fake, ws, None) \
        == _lib.NSA_ERR_NULLPTR
    lib.nsa_plan_destroy(plan)
    lib.nsa_plan_destroy(None)


def test_select_statistics_both_or_neither():
    """The importance pass reads softmax_max and softmax_sum, or (both NULL)
    the per-row array the forward left in the workspace; one without the
    other is refused before any device work."""
    st, ws, plan = _ws(**_good())
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    for smax, ssum in ((fake, None), (None, fake)):
        assert lib.nsa_compress_attention_select(plan, fake, fake, smax, ssum, fake, None, fake, ws, None) \
            == _lib.NSA_ERR_NULLPTR
        assert "both" in lib.nsa_last_error().decode()
        m = _lib.Masks()
        assert lib.nsa_compress_attention_select_masked(plan, fake, fake, ctypes.byref(m), smax, ssum, fake, None,
                                                        fake, ws, None) == _lib.NSA_ERR_NULLPTR
    lib.nsa_plan_destroy(plan)


def test_workspace_holds_table_and_row_biases():
    """Phase one's workspace: the table (64 B per sequence plus a status
    entry, rounded to 256 B), then one float32 per (query token, head)."""
    for N1, B, qlen, clen, slen in ((16, 2, [100, 300], [5, 16], [2, 6]), (64, 1, [4097], [255], [65])):
        st, ws, plan = _ws(**_good(N1=N1, B=B, qlen=qlen, clen=clen, slen=slen))
        assert st == _lib.NSA_OK
        table = ((B + 1) * 64 + 255) // 256 * 256
        assert ws == table + (qlen[-1] * N1 * 4 + 255) // 256 * 256
        _lib.load().nsa_plan_destroy(plan)


@pytest.mark.parametrize("kw,status", [
    (dict(l=24), _lib.NSA_ERR_CONSTRAINT), (dict(l=160), _lib.NSA_ERR_CONSTRAINT),
    (dict(d=48, l=32), _lib.NSA_ERR_CONSTRAINT), (dict(D=72), _lib.NSA_ERR_CONSTRAINT),
    (dict(D=272), _lib.NSA_ERR_CONSTRAINT), (dict(out_tokens=99), _lib.NSA_ERR_SHAPE),
    (dict(total=301), _lib.NSA_ERR_SHAPE), (dict(B=0), _lib.NSA_ERR_SHAPE),
    (dict(dtype=3), _lib.NSA_ERR_DTYPE), (dict(dtype=-1), _lib.NSA_ERR_DTYPE),
    (dict(inp=None), _lib.NSA_ERR_NULLPTR),
])
def test_compress_validation(kw, status):
    a = dict(inp=ctypes.c_void_p(0x1000), B=2, total=300, N=1, D=128, l=32, d=16, dtype=0, out_tokens=16)
    a.update(kw)
    st = _lib.load().nsa_compress(a["inp"], ctypes.c_void_p(0x2000), _arr([100, 300]), a["B"], a["total"],
                                  a["N"], a["D"], a["l"], a["d"], a["dtype"], ctypes.c_void_p(0x3000),
                                  a["out_tokens"], None)
    assert st == status, _lib.load().nsa_last_error()


def test_status_strings_and_python_exception_mapping():
    lib = _lib.load()
    for code in range(8):
        assert lib.nsa_status_string(code).decode().startswith("NSA_")
    with pytest.raises(ValueError):
        nsa.nsa_compress_attention_get_workspace([100, 300], [5, 16], [2, 6], 16, 1, 128, 128, 0.1,
                                                 24, 16, 64, 16)
    with pytest.raises(ValueError):
        nsa.nsa_compress_attention_get_workspace([100, 300], [5, 17], [2, 6], 16, 1, 128, 128, 0.1,
                                                 32, 16, 64, 16)
    with pytest.raises(TypeError):
        nsa.nsa_compress_attention_get_workspace([100, 300], [5, 16], [2, 6], 16, 1, 128, 128, "x",
                                                 32, 16, 64, 16)
    with pytest.raises(NotImplementedError):
        nsa.nsa_compress_attention_get_workspace([100, 300], [5, 16], [2, 6], 16, 1, 256, 128, 0.1,
                                                 32, 16, 64, 16)
    plan = nsa.nsa_compress_attention_get_workspace([100, 300], [5, 16], [2, 6], 16, 1, 128, 128, 0.1,
                                                    32, 16, 64, 16)
    assert plan.info["total_q_tokens"] == 300 and plan.workspace_bytes > 0
    plan.destroy()


def test_masked_calls_reject_before_touching_the_device():
    """Masks smaller than the plan's longest sequence / largest counts give
    NSA_ERR_SHAPE, a workspace below masked_workspace_bytes gives
    NSA_ERR_WORKSPACE; both before any launch."""
    st, ws, plan = _ws(**_good())          # sequences of 100 and 200 tokens
    lib = _lib.load()
    info = _lib.PlanInfo()
    assert lib.nsa_plan_get_info(plan, ctypes.byref(info)) == 0
    assert info.masked_workspace_bytes > info.workspace_bytes
    fake = ctypes.c_void_p(0x1000)
    big = info.masked_workspace_bytes

    def call(m, wsb, fn="nsa_compress_attention_masked"):
        if fn == "nsa_compress_attention_masked":
            return lib.nsa_compress_attention_masked(plan, fake, fake, fake, ctypes.byref(m), fake, fake,
                                                     fake, fake, None, fake, wsb, None)
        if fn == "nsa_compress_attention_fwd_masked":
            return lib.nsa_compress_attention_fwd_masked(plan, fake, fake, fake, ctypes.byref(m), fake,
                                                         fake, fake, fake, wsb, None)
        return lib.nsa_compress_attention_select_masked(plan, fake, fake, ctypes.byref(m), fake, fake,
                                                        fake, None, fake, wsb, None)

    short_rows = _lib.Masks(0x2000, 199, 11, None, 0, 0)     # needs 200 rows, 11 columns
    short_cols = _lib.Masks(0x2000, 200, 10, None, 0, 0)
    topk_short = _lib.Masks(None, 0, 0, 0x3000, 200, 3)       # needs 4 select blocks
    good = _lib.Masks(0x2000, 200, 11, 0x3000, 200, 4)
    for fn in ("nsa_compress_attention_masked", "nsa_compress_attention_fwd_masked",
               "nsa_compress_attention_select_masked"):
        assert call(short_rows, big, fn) == _lib.NSA_ERR_SHAPE, lib.nsa_last_error()
        assert call(short_cols, big, fn) == _lib.NSA_ERR_SHAPE
        assert call(good, big - 1, fn) == _lib.NSA_ERR_WORKSPACE
    assert call(topk_short, big) == _lib.NSA_ERR_SHAPE
    assert call(topk_short, big, "nsa_compress_attention_select_masked") == _lib.NSA_ERR_SHAPE
    lib.nsa_plan_destroy(plan)


def test_select_attention_rejects_before_touching_the_device():
    lib = _lib.load()
    fake = ctypes.c_void_p(0x1000)
    st, ws, plan = _ws(**_good())
    assert lib.nsa_select_attention(plan, fake, fake, fake, None, fake, fake, fake, ws, None) \
        == _lib.NSA_ERR_NULLPTR
    assert lib.nsa_select_attention(plan, fake, fake, fake, fake, fake, fake, fake, ws - 1, None) \
        == _lib.NSA_ERR_WORKSPACE
    lib.nsa_plan_destroy(plan)
    st, ws, plan = _ws(**_good(lsel=48, slen=[3, 8]))   # l' = 48: legal, not a multiple of 32
    assert st == _lib.NSA_OK, lib.nsa_last_error()
    assert lib.nsa_select_attention(plan, fake, fake, fake, fake, fake, fake, fake, ws, None) \
        == _lib.NSA_ERR_UNSUPPORTED
    lib.nsa_plan_destroy(plan)


def test_split_workspace_host_checks():
    """The split attention's workspace query is host only: piece lengths
    outside [1, 2^20] are refused, and shorter pieces need at least as much
    workspace (more partial slots)."""
    import synth
    wl = synth.WORKLOADS[1]
    c, s, pc, ps = [], [], 0, 0
    for T in wl.seqlens:
        pc += nsa.nsa_compress_out_len(T, wl.l, wl.d)
        ps += -(-T // wl.lsel)
        c.append(pc)
        s.append(ps)
    plan = nsa.nsa_compress_attention_get_workspace(wl.act_seq_qlen, c, s, wl.N1, wl.N2, wl.D1, wl.D2, wl.scale,
                                                    wl.l, wl.d, wl.lsel, wl.count, wl.torch_dtype)
    try:
        for bad in (0, -3, (1 << 20) + 1):
            with pytest.raises(ValueError):
                nsa.nsa_compress_attention_split_workspace(plan, bad)
        sizes = [nsa.nsa_compress_attention_split_workspace(plan, t) for t in (64, 8, 4, 1)]
        assert sizes[0] >= plan.workspace_bytes
        assert sizes == sorted(sizes)
        assert sizes[-1] > sizes[0]
    finally:
        plan.destroy()


def test_chunked_plan_host_checks():
    """Chunked-prefill plans: fewer key/value than query tokens is a shape
    error; the plan records the key/value total, and the split launch sizes
    its workspace for it like for any plan."""
    kw = dict(head_num=4, kv_head_num=1, d1=64, d2=64, scale_value=0.125, compress_block_size=32,
              compress_stride=16, select_block_size=64, select_block_count=4)
    c = [nsa.nsa_compress_out_len(300, 32, 16)]
    s = [-(-300 // 64)]
    with pytest.raises(ValueError):
        nsa.nsa_compress_attention_get_workspace([301], c, s, actual_seq_kvlen=[300], **kw)
    plan = nsa.nsa_compress_attention_get_workspace([100], c, s, actual_seq_kvlen=[300], **kw)
    try:
        assert plan.info["total_q_tokens"] == 100 and plan.info["total_cmp_tokens"] == c[0]
        assert plan.info["total_kv_tokens"] == 300
        assert nsa.nsa_compress_attention_split_workspace(plan, 4) > plan.workspace_bytes
    finally:
        plan.destroy()


def test_device_plan_host_checks():
    """A device-planned plan reports itself and the status word's place (the
    entry after the table); the metadata call refuses a plain plan, and the
    no-allocation call refuses a device-planned one, before any launch."""
    kw = dict(head_num=8, kv_head_num=2, d1=64, d2=64, scale_value=0.125, compress_block_size=32,
              compress_stride=16, select_block_size=64, select_block_count=4)
    lens = [300, 45, 1000]
    c = list(np.cumsum([nsa.nsa_compress_out_len(T, 32, 16) for T in lens]))
    s = list(np.cumsum([-(-T // 64) for T in lens]))
    plan = nsa.nsa_compress_attention_get_workspace(list(np.cumsum(lens)), c, s, **kw)
    dplan = nsa.nsa_compress_attention_device_plan(plan)
    try:
        assert plan.info["device_metadata"] == 0 and dplan.info["device_metadata"] == 1
        assert plan.info["status_offset"] == dplan.info["status_offset"] == 64 * len(lens)
        assert plan.workspace_bytes == dplan.workspace_bytes >= 64 * (len(lens) + 1)
        lib = _lib.load()
        fake = ctypes.c_void_p(4096)
        st = lib.nsa_compress_attention_metadata(plan.handle, fake, None, fake, fake, fake, 1 << 20, None)
        assert st == _lib.NSA_ERR_CONSTRAINT
        st = lib.nsa_compress_attention_metadata(dplan.handle, None, None, fake, fake, fake, 1 << 20, None)
        assert st == _lib.NSA_ERR_NULLPTR
        st = lib.nsa_compress_attention_metadata(dplan.handle, fake, None, fake, fake, fake, 16, None)
        assert st == _lib.NSA_ERR_WORKSPACE
        st = lib.nsa_compress_attention_noalloc(dplan.handle, *([fake] * 8), None)
        assert st == _lib.NSA_ERR_CONSTRAINT
    finally:
        dplan.destroy()
        plan.destroy()
