"""MI355X (gfx950) compressed branch of Native Sparse Attention.

A thin Python binding over ``libnsa_cmp.so`` (C ABI in include/nsa_cmp.h).
PyTorch is used only to own device memory and to name the current HIP
stream; every step of the computation runs in the library's HIP kernels.
The functions here only check Python-level types, marshal pointers and
sizes, and allocate output tensors.

Entry points (same names as the C ABI):

* ``nsa_compress`` -- NSA compression of K or V ("aclnnNsaCompress");
* ``nsa_compress_attention_get_workspace`` -- first phase: validation,
  workspace size, plan;
* ``nsa_compress_attention`` -- second phase: attention output, top-k
  indices, softmax max/sum (and optionally the importance scores);
* ``compress_attention`` -- both phases in one call with the argument list
  of ``mindspore.ops.nsa_compress_attention``;
* ``nsa_select_attention`` -- attention over the raw keys of the blocks
  that ``topk_indices`` lists (the consumer of the top-k).

The second-phase calls take optional ``atten_mask`` / ``topk_mask``: 2-D
bool (or uint8) GPU tensors indexed by (local query position, compressed
entry / select block), shared by all sequences; True masks the pair out and
a given mask replaces that step's positional rule.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import Masks, NsaError, PlanInfo  # noqa: F401

__all__ = ["nsa_compress_out_len", "nsa_compress", "nsa_compress_attention_get_workspace",
           "nsa_compress_attention", "nsa_compress_attention_noalloc", "nsa_compress_attention_fwd",
           "nsa_compress_attention_select",
           "nsa_compress_attention_split_workspace", "nsa_compress_attention_fwd_split",
           "nsa_select_attention", "nsa_compress_attention_backward", "nsa_compress_backward", "compress_attention", "Plan",
           "nsa_compress_attention_device_plan", "nsa_compress_attention_metadata", "NsaError", "library_path"]


def library_path() -> str:
    return _lib.LIB_PATH


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return _lib.NSA_DTYPE_BF16
    if dt == torch.float16:
        return _lib.NSA_DTYPE_FP16
    raise TypeError(f"q/k/v must be bfloat16 or float16 tensors, got {dt}")


def _stream_ptr(device: torch.device, stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _empty(shape, dtype: torch.dtype, device: torch.device, stream) -> torch.Tensor:
    """A tensor the binding allocates for a call on ``stream``.  The caching
    allocator ties a block to the stream current at allocation; when the
    kernels run on another stream the block is recorded on it too, so it is
    not handed out again while they may still use it."""
    t = torch.empty(shape, dtype=dtype, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        t.record_stream(stream)
    return t


def _prefix(arr, name: str) -> "ctypes.Array":
    if isinstance(arr, torch.Tensor):
        arr = arr.tolist()
    try:
        vals = [int(x) for x in arr]
    except TypeError as e:
        raise TypeError(f"{name} must be a sequence of ints") from e
    return (ctypes.c_int64 * max(1, len(vals)))(*vals), len(vals)


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need_tensor(t, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def nsa_compress_out_len(seq_len: int, compress_block_size: int, compress_stride: int) -> int:
    n = _lib.load().nsa_compress_out_len(int(seq_len), int(compress_block_size), int(compress_stride))
    if n < 0:
        raise ValueError("invalid arguments to nsa_compress_out_len")
    return int(n)


def nsa_compress(input: torch.Tensor, weight: torch.Tensor, act_seq_len: Sequence[int],
                 compress_block_size: int, compress_stride: int,
                 out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Compress a TND tensor ``input [T, N, D]`` with ``weight [l, N]``.

    ``act_seq_len`` holds the sequences' token counts as prefix sums.
    Returns ``[sum_b n_cmp_b, N, D]`` in the input dtype."""
    _need_tensor(input, "input")
    _need_tensor(weight, "weight")
    if input.dim() != 3:
        raise ValueError(f"input must be [T, N, D], got shape {tuple(input.shape)}")
    if weight.dtype != input.dtype:
        raise TypeError("weight must have the input's dtype")
    T, N, D = input.shape
    l, dd = int(compress_block_size), int(compress_stride)
    if tuple(weight.shape) != (l, N):
        raise ValueError(f"weight must be [{l}, {N}], got {tuple(weight.shape)}")
    pre, B = _prefix(act_seq_len, "act_seq_len")
    prev, T2 = 0, 0
    lib = _lib.load()
    for x in list(pre)[:B]:
        n = lib.nsa_compress_out_len(int(x) - prev, l, dd)
        prev = int(x)
        T2 += max(0, int(n))
    if out is None:
        out = _empty((T2, N, D), input.dtype, input.device, stream)
    else:
        _need_tensor(out, "out")
    st = _lib.load().nsa_compress(_ptr(input), _ptr(weight), pre, B, T, N, D, l, dd,
                                  _dtype_code(input.dtype), _ptr(out), out.shape[0],
                                  _stream_ptr(input.device, stream))
    _lib.check(st)
    return out


class Plan:
    """Owns an nsa_plan handle (first phase of the attention operator)."""

    def __init__(self, handle: ctypes.c_void_p, workspace_bytes: int):
        self._h = handle
        self.workspace_bytes = int(workspace_bytes)
        info = PlanInfo()
        _lib.check(_lib.load().nsa_plan_get_info(self._h, ctypes.byref(info)))
        self.info = {name: getattr(info, name) for name, _ in PlanInfo._fields_}

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise ValueError("plan was destroyed")
        return self._h

    def destroy(self) -> None:
        if self._h is not None:
            _lib.load().nsa_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def nsa_compress_attention_get_workspace(actual_seq_qlen, actual_cmp_seq_kvlen, actual_sel_seq_kvlen,
                                         head_num: int, kv_head_num: int, d1: int, d2: int,
                                         scale_value: float, compress_block_size: int,
                                         compress_stride: int, select_block_size: int,
                                         select_block_count: int,
                                         dtype: torch.dtype = torch.bfloat16, actual_seq_kvlen=None) -> Plan:
    """Validates and plans steps 2-7.  ``actual_seq_kvlen`` (prefix sums of
    key/value tokens, optional): each sequence's queries are then its last
    tokens (chunked prefill), and the compressed/select lengths follow the
    key/value tokens."""
    if not isinstance(scale_value, (int, float)):
        raise TypeError("scale_value must be a float")
    for name, v in (("head_num", head_num), ("kv_head_num", kv_head_num), ("d1", d1), ("d2", d2),
                    ("compress_block_size", compress_block_size), ("compress_stride", compress_stride),
                    ("select_block_size", select_block_size), ("select_block_count", select_block_count)):
        if not isinstance(v, int) or isinstance(v, bool):
            raise TypeError(f"{name} must be an int")
    q, B = _prefix(actual_seq_qlen, "actual_seq_qlen")
    c, Bc = _prefix(actual_cmp_seq_kvlen, "actual_cmp_seq_kvlen")
    s, Bs = _prefix(actual_sel_seq_kvlen, "actual_sel_seq_kvlen")
    if not (B == Bc == Bs):
        raise ValueError("the three prefix-sum lists must have the same length")
    ws = ctypes.c_size_t(0)
    h = ctypes.c_void_p(0)
    rest = (head_num, kv_head_num, d1, d2, float(scale_value), compress_block_size, compress_stride,
            select_block_size, select_block_count, _dtype_code(dtype), ctypes.byref(ws), ctypes.byref(h))
    if actual_seq_kvlen is None:
        st = _lib.load().nsa_compress_attention_get_workspace(B, q, c, s, *rest)
    else:
        kv, Bk = _prefix(actual_seq_kvlen, "actual_seq_kvlen")
        if Bk != B:
            raise ValueError("actual_seq_kvlen must have the length of actual_seq_qlen")
        st = _lib.load().nsa_compress_attention_get_workspace_kv(B, q, kv, c, s, *rest)
    _lib.check(st)
    return Plan(h, ws.value)


def nsa_compress_attention_device_plan(plan: Plan) -> Plan:
    """A copy of ``plan`` whose execute calls read their per-sequence table
    from the workspace, where ``nsa_compress_attention_metadata`` writes it
    from device prefix sums (no host-to-device copy per call)."""
    h = ctypes.c_void_p(0)
    _lib.check(_lib.load().nsa_compress_attention_device_plan(plan.handle, ctypes.byref(h)))
    return Plan(h, plan.workspace_bytes)


def _device_prefix(t, name: str, B: int):
    _need_tensor(t, name)
    if t.dtype != torch.int64 or t.dim() != 1 or t.numel() != B:
        raise ValueError(f"{name} must be a 1-D int64 GPU tensor of {B} prefix sums")
    return _ptr(t)


def nsa_compress_attention_metadata(plan: Plan, actual_seq_qlen: torch.Tensor, actual_cmp_seq_kvlen: torch.Tensor,
                                    actual_sel_seq_kvlen: torch.Tensor, workspace: torch.Tensor,
                                    actual_seq_kvlen: Optional[torch.Tensor] = None, stream=None) -> None:
    """Writes the per-sequence table of a device-planned ``plan`` into
    ``workspace`` from int64 GPU prefix sums, with a status word at byte
    ``plan.info["status_offset"]`` (0 when the lengths pass the plan's
    checks; otherwise every later call on this workspace leaves its outputs
    untouched)."""
    B = plan.info["batch"]
    _need_tensor(workspace, "workspace")
    args = [_device_prefix(actual_seq_qlen, "actual_seq_qlen", B),
            None if actual_seq_kvlen is None else _device_prefix(actual_seq_kvlen, "actual_seq_kvlen", B),
            _device_prefix(actual_cmp_seq_kvlen, "actual_cmp_seq_kvlen", B),
            _device_prefix(actual_sel_seq_kvlen, "actual_sel_seq_kvlen", B)]
    st = _lib.load().nsa_compress_attention_metadata(plan.handle, *args, _ptr(workspace),
                                                     workspace.numel() * workspace.element_size(),
                                                     _stream_ptr(workspace.device, stream))
    _lib.check(st)


def _check_qkv(plan: Plan, query, key, value=None):
    info = plan.info
    _need_tensor(query, "query")
    _need_tensor(key, "key")
    T1, N1, D1, N2, T2 = (info["total_q_tokens"], info["head_num"], info["d1"], info["kv_head_num"],
                          info["total_cmp_tokens"])
    if tuple(query.shape) != (T1, N1, D1):
        raise ValueError(f"query must be {(T1, N1, D1)}, got {tuple(query.shape)}")
    if tuple(key.shape) != (T2, N2, D1):
        raise ValueError(f"key must be {(T2, N2, D1)}, got {tuple(key.shape)}")
    if query.dtype != key.dtype:
        raise TypeError("query and key must share a dtype")
    if _dtype_code(query.dtype) != info["dtype"]:
        raise TypeError(f"the plan was made for dtype code {info['dtype']}, "
                        f"query is {query.dtype}")
    if value is not None:
        _need_tensor(value, "value")
        if tuple(value.shape) != (T2, N2, info["d2"]):
            raise ValueError(f"value must be {(T2, N2, info['d2'])}, got {tuple(value.shape)}")
        if value.dtype != query.dtype:
            raise TypeError("query and value must share a dtype")


def _workspace(plan: Plan, workspace, dev, stream, masked: bool = False):
    need = plan.info["masked_workspace_bytes"] if masked else plan.workspace_bytes
    if workspace is None and plan.info["device_metadata"]:
        raise ValueError("a device-planned plan needs the workspace nsa_compress_attention_metadata wrote")
    if workspace is None:
        workspace = _empty((max(need, 1),), torch.uint8, dev, stream)
    return workspace, workspace.numel() * workspace.element_size()


def _masks(atten_mask, topk_mask):
    """An nsa_masks struct (and the tensors it points at), or None."""
    if atten_mask is None and topk_mask is None:
        return None, ()
    m = Masks()
    keep = []
    for name, t in (("atten_mask", atten_mask), ("topk_mask", topk_mask)):
        if t is None:
            continue
        _need_tensor(t, name)
        if t.dim() != 2:
            raise ValueError(f"{name} must be 2-D (query position, column), got shape {tuple(t.shape)}")
        if t.dtype not in (torch.bool, torch.uint8):
            raise TypeError(f"{name} must be a bool or uint8 tensor, got {t.dtype}")
        keep.append(t)
        pre = name.split("_")[0]
        setattr(m, name, t.data_ptr())
        setattr(m, f"{pre}_rows", t.shape[0])
        setattr(m, f"{pre}_cols", t.shape[1])
    return m, tuple(keep)


def _alloc_outputs(plan: Plan, query, outputs, want_pslc: bool, stream=None):
    info = plan.info
    T1, N1, N2, D2 = info["total_q_tokens"], info["head_num"], info["kv_head_num"], info["d2"]
    cnt, S = info["select_block_count"], info["max_sel_blocks"]
    dev = query.device
    o = dict(outputs or {})
    if o.get("attention_out") is None:
        o["attention_out"] = _empty((T1, N1, D2), query.dtype, dev, stream)
    if o.get("topk_indices") is None:
        o["topk_indices"] = _empty((T1, N2, cnt), torch.int32, dev, stream)
    if o.get("softmax_max") is None:
        o["softmax_max"] = _empty((T1, N1, 8), torch.float32, dev, stream)
    if o.get("softmax_sum") is None:
        o["softmax_sum"] = _empty((T1, N1, 8), torch.float32, dev, stream)
    if want_pslc and o.get("p_slc") is None:
        o["p_slc"] = _empty((T1, N2, max(S, 1)), torch.float32, dev, stream)
    return o


def nsa_compress_attention(plan: Plan, query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                           workspace: Optional[torch.Tensor] = None, return_p_slc: bool = False,
                           outputs: Optional[dict] = None, stream=None, atten_mask=None,
                           topk_mask=None):
    """Second phase.  Returns (attention_out, topk_indices, softmax_max,
    softmax_sum) and, with ``return_p_slc``, the importance scores
    [T1, N2, S] as a fifth element."""
    _check_qkv(plan, query, key, value)
    o = _alloc_outputs(plan, query, outputs, return_p_slc, stream)
    m, _keep = _masks(atten_mask, topk_mask)
    ws, ws_bytes = _workspace(plan, workspace, query.device, stream, m is not None)
    lib = _lib.load()
    args = (_ptr(o["attention_out"]), _ptr(o["topk_indices"]), _ptr(o["softmax_max"]),
            _ptr(o["softmax_sum"]), _ptr(o.get("p_slc") if return_p_slc else None), _ptr(ws),
            ws_bytes, _stream_ptr(query.device, stream))
    if m is None:
        st = lib.nsa_compress_attention(plan.handle, _ptr(query), _ptr(key), _ptr(value), *args)
    else:
        st = lib.nsa_compress_attention_masked(plan.handle, _ptr(query), _ptr(key), _ptr(value),
                                               ctypes.byref(m), *args)
    _lib.check(st)
    res = (o["attention_out"], o["topk_indices"], o["softmax_max"], o["softmax_sum"])
    return res + (o["p_slc"],) if return_p_slc else res


def nsa_compress_attention_noalloc(plan: Plan, query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                                   outputs: dict, p_slc: Optional[torch.Tensor] = None, stream=None):
    """``nsa_compress_attention`` for callers that cannot allocate: nothing
    is allocated here or in the library (its scratch is a static per-GPU
    table of at most 1024 sequences, shared by every call on that GPU, so
    calls that overlap on one GPU race).  ``outputs`` must hold
    attention_out, topk_indices, softmax_max and softmax_sum of the plan's
    shapes; ``p_slc`` optionally receives the importance scores.  Returns
    (attention_out, topk_indices, softmax_max, softmax_sum)."""
    _check_qkv(plan, query, key, value)
    info = plan.info
    T1, N1, N2, D2 = info["total_q_tokens"], info["head_num"], info["kv_head_num"], info["d2"]
    want = {"attention_out": ((T1, N1, D2), query.dtype), "topk_indices": ((T1, N2, info["select_block_count"]),
                                                                          torch.int32),
            "softmax_max": ((T1, N1, 8), torch.float32), "softmax_sum": ((T1, N1, 8), torch.float32)}
    for name, (shape, dt) in want.items():
        t = outputs.get(name) if outputs else None
        if t is None:
            raise ValueError(f"outputs[{name!r}] must be given: this entry point allocates nothing")
        _need_tensor(t, name)
        if tuple(t.shape) != shape or t.dtype != dt:
            raise ValueError(f"outputs[{name!r}] must be {dt} {shape}")
    if p_slc is not None:
        _need_tensor(p_slc, "p_slc")
        if tuple(p_slc.shape) != (T1, N2, max(info["max_sel_blocks"], 1)) or p_slc.dtype != torch.float32:
            raise ValueError("p_slc must be float32 [T1, N2, max select blocks]")
    st = _lib.load().nsa_compress_attention_noalloc(
        plan.handle, _ptr(query), _ptr(key), _ptr(value), _ptr(outputs["attention_out"]),
        _ptr(outputs["topk_indices"]), _ptr(outputs["softmax_max"]), _ptr(outputs["softmax_sum"]), _ptr(p_slc),
        _stream_ptr(query.device, stream))
    _lib.check(st)
    return outputs["attention_out"], outputs["topk_indices"], outputs["softmax_max"], outputs["softmax_sum"]


def nsa_compress_attention_fwd(plan: Plan, query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                               workspace: Optional[torch.Tensor] = None, outputs: Optional[dict] = None,
                               stream=None, atten_mask=None):
    """Steps 1-3 only: returns (attention_out, softmax_max, softmax_sum)."""
    _check_qkv(plan, query, key, value)
    o = _alloc_outputs(plan, query, outputs, False, stream)
    m, _keep = _masks(atten_mask, None)
    ws, ws_bytes = _workspace(plan, workspace, query.device, stream, m is not None)
    lib = _lib.load()
    args = (_ptr(o["attention_out"]), _ptr(o["softmax_max"]), _ptr(o["softmax_sum"]), _ptr(ws),
            ws_bytes, _stream_ptr(query.device, stream))
    if m is None:
        st = lib.nsa_compress_attention_fwd(plan.handle, _ptr(query), _ptr(key), _ptr(value), *args)
    else:
        st = lib.nsa_compress_attention_fwd_masked(plan.handle, _ptr(query), _ptr(key), _ptr(value),
                                                   ctypes.byref(m), *args)
    _lib.check(st)
    return o["attention_out"], o["softmax_max"], o["softmax_sum"]


def nsa_compress_attention_split_workspace(plan: Plan, key_tiles_per_piece: int) -> int:
    """Workspace bytes of ``nsa_compress_attention_fwd_split`` for this plan."""
    n = ctypes.c_size_t(0)
    _lib.check(_lib.load().nsa_compress_attention_split_workspace(plan.handle, int(key_tiles_per_piece),
                                                                   ctypes.byref(n)))
    return n.value


def nsa_compress_attention_fwd_split(plan: Plan, query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                                     key_tiles_per_piece: int, workspace: Optional[torch.Tensor] = None,
                                     outputs: Optional[dict] = None, stream=None):
    """Steps 1-3 with the key range of long row blocks split into pieces of
    at most ``key_tiles_per_piece`` tiles of 32 compressed blocks, merged by
    a second kernel: returns (attention_out, softmax_max, softmax_sum)."""
    _check_qkv(plan, query, key, value)
    o = _alloc_outputs(plan, query, outputs, False, stream)
    need = nsa_compress_attention_split_workspace(plan, key_tiles_per_piece)
    if workspace is None and plan.info["device_metadata"]:
        raise ValueError("a device-planned plan needs the workspace nsa_compress_attention_metadata wrote")
    if workspace is None:
        workspace = _empty((max(need, 1),), torch.uint8, query.device, stream)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _lib.load().nsa_compress_attention_fwd_split(
        plan.handle, _ptr(query), _ptr(key), _ptr(value), _ptr(o["attention_out"]), _ptr(o["softmax_max"]),
        _ptr(o["softmax_sum"]), int(key_tiles_per_piece), _ptr(workspace), ws_bytes,
        _stream_ptr(query.device, stream))
    _lib.check(st)
    return o["attention_out"], o["softmax_max"], o["softmax_sum"]


def nsa_compress_attention_select(plan: Plan, query: torch.Tensor, key: torch.Tensor,
                                  softmax_max: Optional[torch.Tensor], softmax_sum: Optional[torch.Tensor],
                                  workspace: Optional[torch.Tensor] = None, return_p_slc: bool = False,
                                  outputs: Optional[dict] = None, stream=None, atten_mask=None,
                                  topk_mask=None):
    """Steps 4-7 from the first half's softmax statistics: returns
    topk_indices (and the importance scores with ``return_p_slc``).  The
    atten_mask must be the one the first half was given.  With
    ``softmax_max`` and ``softmax_sum`` both None the statistics are the
    per-row array the first half wrote into ``workspace`` (which must then
    be that call's workspace)."""
    _check_qkv(plan, query, key)
    if (softmax_max is None) != (softmax_sum is None):
        raise ValueError("give softmax_max and softmax_sum together, or neither (then the forward's workspace)")
    if softmax_max is None and workspace is None:
        raise ValueError("without softmax_max / softmax_sum the statistics come from the forward call's "
                         "workspace: pass it")
    for t, name in ((softmax_max, "softmax_max"), (softmax_sum, "softmax_sum")):
        if t is None:
            continue
        _need_tensor(t, name)
        if t.dtype != torch.float32 or tuple(t.shape) != (plan.info["total_q_tokens"], plan.info["head_num"], 8):
            raise ValueError(f"{name} must be float32 [T1, N1, 8]")
    o = _alloc_outputs(plan, query, outputs, return_p_slc, stream)
    m, _keep = _masks(atten_mask, topk_mask)
    ws, ws_bytes = _workspace(plan, workspace, query.device, stream, m is not None)
    lib = _lib.load()
    args = (_ptr(softmax_max), _ptr(softmax_sum), _ptr(o["topk_indices"]),
            _ptr(o.get("p_slc") if return_p_slc else None), _ptr(ws), ws_bytes,
            _stream_ptr(query.device, stream))
    if m is None:
        st = lib.nsa_compress_attention_select(plan.handle, _ptr(query), _ptr(key), *args)
    else:
        st = lib.nsa_compress_attention_select_masked(plan.handle, _ptr(query), _ptr(key),
                                                      ctypes.byref(m), *args)
    _lib.check(st)
    return (o["topk_indices"], o["p_slc"]) if return_p_slc else o["topk_indices"]


def compress_attention(query, key, value, scale_value, head_num, compress_block_size,
                       compress_stride, select_block_size, select_block_count, *,
                       actual_seq_qlen, actual_cmp_seq_kvlen, actual_sel_seq_kvlen,
                       topk_mask=None, atten_mask=None, return_p_slc: bool = False):
    """Both phases with the argument list of the MindSpore operator.  With
    no mask tensors the causal rules are generated from positions."""
    _need_tensor(query, "query")
    _need_tensor(key, "key")
    if query.dim() != 3 or key.dim() != 3 or value.dim() != 3:
        raise ValueError("query, key and value must be TND (3-D)")
    plan = nsa_compress_attention_get_workspace(
        actual_seq_qlen, actual_cmp_seq_kvlen, actual_sel_seq_kvlen, int(head_num),
        int(key.shape[1]), int(query.shape[2]), int(value.shape[2]), scale_value,
        int(compress_block_size), int(compress_stride), int(select_block_size),
        int(select_block_count), query.dtype)
    try:
        return nsa_compress_attention(plan, query, key, value, return_p_slc=return_p_slc,
                                      atten_mask=atten_mask, topk_mask=topk_mask)
    finally:
        plan.destroy()


def nsa_select_attention(plan: Plan, query: torch.Tensor, key: torch.Tensor, value: torch.Tensor,
                         topk_indices: torch.Tensor, workspace: Optional[torch.Tensor] = None,
                         outputs: Optional[dict] = None, stream=None):
    """Selected-block attention over the raw ``key [Tkv, N2, D1]`` /
    ``value [Tkv, N2, D2]`` (the plan's key/value tokens: Tkv = T1 unless the
    plan is chunked) for the blocks that ``topk_indices [T1, N2, count]``
    lists.  Returns (attention_out [T1, N1, D2], softmax_lse [T1, N1] float32)."""
    info = plan.info
    T1, N1, N2, D1, D2 = (info["total_q_tokens"], info["head_num"], info["kv_head_num"], info["d1"],
                          info["d2"])
    Tkv = info["total_kv_tokens"]
    for t, name in ((query, "query"), (key, "key"), (value, "value"), (topk_indices, "topk_indices")):
        _need_tensor(t, name)
    if tuple(query.shape) != (T1, N1, D1):
        raise ValueError(f"query must be {(T1, N1, D1)}, got {tuple(query.shape)}")
    if tuple(key.shape) != (Tkv, N2, D1) or tuple(value.shape) != (Tkv, N2, D2):
        raise ValueError(f"key/value must be {(Tkv, N2, D1)} / {(Tkv, N2, D2)}, got "
                         f"{tuple(key.shape)} / {tuple(value.shape)}")
    if key.dtype != query.dtype or value.dtype != query.dtype:
        raise TypeError("query, key and value must share a dtype")
    if _dtype_code(query.dtype) != info["dtype"]:
        raise TypeError(f"the plan was made for dtype code {info['dtype']}, query is {query.dtype}")
    if topk_indices.dtype != torch.int32 or tuple(topk_indices.shape) != (T1, N2, info["select_block_count"]):
        raise ValueError(f"topk_indices must be int32 {(T1, N2, info['select_block_count'])}")
    o = dict(outputs or {})
    if o.get("attention_out") is None:
        o["attention_out"] = _empty((T1, N1, D2), query.dtype, query.device, stream)
    if o.get("softmax_lse") is None:
        o["softmax_lse"] = _empty((T1, N1), torch.float32, query.device, stream)
    ws, ws_bytes = _workspace(plan, workspace, query.device, stream)
    st = _lib.load().nsa_select_attention(plan.handle, _ptr(query), _ptr(key), _ptr(value), _ptr(topk_indices),
                                          _ptr(o["attention_out"]), _ptr(o["softmax_lse"]), _ptr(ws), ws_bytes,
                                          _stream_ptr(query.device, stream))
    _lib.check(st)
    return o["attention_out"], o["softmax_lse"]


def nsa_compress_attention_backward(plan: Plan, query, key, value, attention_out, d_attention_out,
                                    softmax_max, softmax_sum, workspace: Optional[torch.Tensor] = None,
                                    stream=None):
    """Gradients of the compressed attention output with respect to query,
    key and value (the compressed ones), float32: (d_query [T1, N1, D1],
    d_key [T2, N2, D1], d_value [T2, N2, D2])."""
    _check_qkv(plan, query, key, value)
    info = plan.info
    T1, N1, N2, D1, D2, T2 = (info["total_q_tokens"], info["head_num"], info["kv_head_num"], info["d1"],
                              info["d2"], info["total_cmp_tokens"])
    for t, name in ((attention_out, "attention_out"), (d_attention_out, "d_attention_out")):
        _need_tensor(t, name)
        if tuple(t.shape) != (T1, N1, D2) or t.dtype != query.dtype:
            raise ValueError(f"{name} must be {(T1, N1, D2)} of the query's dtype")
    for t, name in ((softmax_max, "softmax_max"), (softmax_sum, "softmax_sum")):
        _need_tensor(t, name)
        if t.dtype != torch.float32 or tuple(t.shape) != (T1, N1, 8):
            raise ValueError(f"{name} must be float32 [T1, N1, 8]")
    dev = query.device
    dq = _empty((T1, N1, D1), torch.float32, dev, stream)
    dk = _empty((T2, N2, D1), torch.float32, dev, stream)
    dv = _empty((T2, N2, D2), torch.float32, dev, stream)
    need = info["backward_workspace_bytes"]
    if workspace is None and info["device_metadata"]:
        raise ValueError("a device-planned plan needs the workspace nsa_compress_attention_metadata wrote")
    if workspace is None:
        workspace = _empty((max(need, 1),), torch.uint8, dev, stream)
    st = _lib.load().nsa_compress_attention_backward(
        plan.handle, _ptr(query), _ptr(key), _ptr(value), _ptr(attention_out), _ptr(d_attention_out),
        _ptr(softmax_max), _ptr(softmax_sum), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream_ptr(dev, stream))
    _lib.check(st)
    return dq, dk, dv


def nsa_compress_backward(input: torch.Tensor, weight: torch.Tensor, d_output: torch.Tensor,
                          act_seq_len: Sequence[int], compress_block_size: int, compress_stride: int,
                          stream=None):
    """Gradients of nsa_compress: (d_input [T, N, D], d_weight [l, N]), float32,
    for the float32 gradient ``d_output [T2, N, D]`` of its output."""
    _need_tensor(input, "input")
    _need_tensor(weight, "weight")
    _need_tensor(d_output, "d_output")
    if input.dim() != 3 or weight.dtype != input.dtype:
        raise ValueError("input must be [T, N, D] and weight of the input's dtype")
    if d_output.dtype != torch.float32:
        raise TypeError("d_output must be float32")
    T, N, D = input.shape
    l, dd = int(compress_block_size), int(compress_stride)
    pre, B = _prefix(act_seq_len, "act_seq_len")
    dx = _empty((T, N, D), torch.float32, input.device, stream)
    dw = _empty((l, N), torch.float32, input.device, stream)
    st = _lib.load().nsa_compress_backward(_ptr(input), _ptr(weight), _ptr(d_output), pre, B, T, N, D, l, dd,
                                           _dtype_code(input.dtype), d_output.shape[0], _ptr(dx), _ptr(dw),
                                           _stream_ptr(input.device, stream))
    _lib.check(st)
    return dx, dw
