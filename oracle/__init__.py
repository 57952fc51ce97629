"""CPU oracle for the compressed branch of NSA -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It wraps ``nsa_oracle.c`` (plain C,
float64 on exactly widened bfloat16 or float16 inputs) through ctypes and shares no code with
the HIP library in ``kv_compression_block_amd``.

Every function here either marshals arrays or chains the C steps in the
order the operator pages give them:

* ``compress``  -- the NSA Compress formula ("aclnnNsaCompress", Formula);
* ``attention`` -- steps 1-7 of "mindspore.ops.nsa_compress_attention"
  (scores, mask, softmax, output, importance remap, group sum, top-k);
* ``select_attention`` -- attention over the raw keys of the selected
  blocks, the consumer of the top-k indices (interface of
  "lite_boost.ops.rain_fusion_attention");
* ``attention_backward`` / ``compress_backward`` -- the derivatives of the
  compressed attention output and of the compression, for training.

The compressed keys/values that feed attention are the compression results
rounded to the element type of the inputs (round to nearest, ties to even),
because that is the dtype the attention operator takes for its key and value
inputs.  ``dtype`` is "bf16" or "f16" throughout.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nsa_oracle.c")
_LIB = os.path.join(_HERE, "libnsa_oracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile nsa_oracle.c with gcc (no -ffast-math: IEEE semantics kept)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-D_DEFAULT_SOURCE", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-Werror", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.nsa_oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.nsa_oracle_bf16_to_double.restype = ctypes.c_double
    lib.nsa_oracle_double_to_bf16.argtypes = [ctypes.c_double]
    lib.nsa_oracle_double_to_bf16.restype = ctypes.c_uint16
    lib.nsa_oracle_round_to_bf16.argtypes = [P, P, I64]
    lib.nsa_oracle_round_to_bf16.restype = None
    lib.nsa_oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.nsa_oracle_f16_to_double.restype = ctypes.c_double
    lib.nsa_oracle_double_to_f16.argtypes = [ctypes.c_double]
    lib.nsa_oracle_double_to_f16.restype = ctypes.c_uint16
    lib.nsa_oracle_round_to_f16.argtypes = [P, P, I64]
    lib.nsa_oracle_round_to_f16.restype = None
    lib.nsa_oracle_stage_reset.argtypes = []
    lib.nsa_oracle_stage_reset.restype = None
    lib.nsa_oracle_stage_seconds.argtypes = [P]
    lib.nsa_oracle_stage_seconds.restype = None
    lib.nsa_oracle_threads.argtypes = []
    lib.nsa_oracle_threads.restype = ctypes.c_int
    lib.nsa_oracle_n_cmp.argtypes = [I64, I64, I64]
    lib.nsa_oracle_n_cmp.restype = I64
    lib.nsa_oracle_compress.argtypes = [P, P, P, I64, I64, I64, I64, I64, ctypes.c_int, P]
    lib.nsa_oracle_compress.restype = ctypes.c_int
    lib.nsa_oracle_attention.argtypes = [P, P, I64, P, P, P, P, I64,
                                         I64, I64, I64, I64, ctypes.c_double,
                                         I64, I64, I64, I64, ctypes.c_int,
                                         P, P, P, P, I64, P]
    lib.nsa_oracle_attention.restype = ctypes.c_int
    lib.nsa_oracle_attention_masked.argtypes = [P, P, I64, P, P, P, P, P, I64,
                                                I64, I64, I64, I64, ctypes.c_double,
                                                I64, I64, I64, I64, ctypes.c_int,
                                                P, I64, I64, P, I64, I64,
                                                P, P, P, P, I64, P]
    lib.nsa_oracle_attention_masked.restype = ctypes.c_int
    lib.nsa_oracle_select_attention.argtypes = [P, P, P, P, P, I64, P, I64, I64, I64, I64, I64,
                                                ctypes.c_double, I64, I64, ctypes.c_int, P, P]
    lib.nsa_oracle_select_attention.restype = ctypes.c_int
    lib.nsa_oracle_select_attention_kv.argtypes = [P, P, P, P, P, I64, P, P, I64, I64, I64, I64, I64,
                                                   ctypes.c_double, I64, I64, ctypes.c_int, P, P]
    lib.nsa_oracle_select_attention_kv.restype = ctypes.c_int
    lib.nsa_oracle_attention_backward.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, I64,
                                                  ctypes.c_double, I64, I64, ctypes.c_int, P, P, P]
    lib.nsa_oracle_attention_backward.restype = ctypes.c_int
    lib.nsa_oracle_attention_backward_kv.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, I64,
                                                     ctypes.c_double, I64, I64, ctypes.c_int, P, P, P]
    lib.nsa_oracle_attention_backward_kv.restype = ctypes.c_int
    lib.nsa_oracle_compress_backward.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, ctypes.c_int, P, P]
    lib.nsa_oracle_compress_backward.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected 16-bit float bit patterns as uint16, got {a.dtype}")
    return a


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def threads() -> int:
    return int(_load().nsa_oracle_threads())


STAGES = ("compress", "attention (steps 1-3)", "remap + group sum (steps 4-5)", "top-k (steps 6-7)")


def stage_reset() -> None:
    """Zero the per-stage timers (instrumentation only)."""
    _load().nsa_oracle_stage_reset()


def stage_seconds() -> dict:
    """Thread-seconds spent per stage since the last reset: compression, then
    steps 1-3, 4-5 and 6-7 of the attention call (summed over threads)."""
    out = np.zeros(4, dtype=np.float64)
    _load().nsa_oracle_stage_seconds(_ptr(out))
    return dict(zip(STAGES, (float(x) for x in out)))


def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns."""
    b = _u16(bits)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_bf16(x) -> np.ndarray:
    """Round float64 values to bfloat16 bit patterns (nearest, ties to even)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().nsa_oracle_round_to_bf16(_ptr(x), _ptr(out), x.size)
    return out


def f16_to_f64(bits) -> np.ndarray:
    """Exact widening of float16 (IEEE binary16) bit patterns, element by
    element through the C decoder."""
    b = _u16(bits)
    lib = _load()
    flat = b.reshape(-1)
    # 65536 patterns at most: decode each distinct one once.
    uniq, inv = np.unique(flat, return_inverse=True)
    vals = np.array([lib.nsa_oracle_f16_to_double(int(u)) for u in uniq], dtype=np.float64)
    return vals[inv].reshape(b.shape)


def to_f16(x) -> np.ndarray:
    """Round float64 values to float16 bit patterns (nearest, ties to even)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().nsa_oracle_round_to_f16(_ptr(x), _ptr(out), x.size)
    return out


DTYPES = {"bf16": 0, "f16": 1}


def _code(dtype: str) -> int:
    if dtype not in DTYPES:
        raise ValueError(f"dtype must be one of {sorted(DTYPES)}, got {dtype!r}")
    return DTYPES[dtype]


def widen(bits, dtype: str = "bf16") -> np.ndarray:
    """Exact float64 values of bit patterns of element type ``dtype``."""
    return f16_to_f64(bits) if _code(dtype) == 1 else bf16_to_f64(bits)


def round_to(x, dtype: str = "bf16") -> np.ndarray:
    """Round float64 values to bit patterns of element type ``dtype``."""
    return to_f16(x) if _code(dtype) == 1 else to_bf16(x)


def n_cmp(T: int, l: int, d: int) -> int:
    return int(_load().nsa_oracle_n_cmp(T, l, d))


def cmp_prefix(seqlens: Sequence[int], l: int, d: int) -> np.ndarray:
    """Prefix sums of the compressed lengths of each sequence."""
    return np.cumsum([n_cmp(int(T), l, d) for T in seqlens]).astype(np.int64)


def sel_prefix(seqlens: Sequence[int], lsel: int) -> np.ndarray:
    """Prefix sums of the number of select blocks, ceil(T / l'), per sequence."""
    return np.cumsum([-(-int(T) // lsel) for T in seqlens]).astype(np.int64)


def compress(x_bits, w_bits, act_seq_len, l: int, d: int, dtype: str = "bf16") -> np.ndarray:
    """x: [T, N, D] bits, w: [l, N] bits, both of element type ``dtype``
    -> [T2, N, D] float64."""
    x = _u16(x_bits)
    w = _u16(w_bits)
    T, N, D = x.shape
    if w.shape != (l, N):
        raise ValueError(f"weight shape {w.shape} != {(l, N)}")
    act = _i64(act_seq_len)
    if act[-1] != T:
        raise ValueError("prefix sums do not end at the token count")
    starts = np.concatenate([[0], act[:-1]])
    T2 = int(sum(n_cmp(int(e - s), l, d) for s, e in zip(starts, act)))
    out = np.empty((T2, N, D), dtype=np.float64)
    rc = _load().nsa_oracle_compress(_ptr(x), _ptr(w), _ptr(act), len(act), N, D, l, d,
                                     _code(dtype), _ptr(out))
    if rc != 0:
        raise ValueError(f"nsa_oracle_compress returned {rc}")
    return out


def attention(q_rows_bits, tokens, kc_bits, vc_bits, act_seq_qlen, act_cmp_seq_kvlen,
              N1: int, N2: int, scale: float, l: int, d: int, lsel: int, count: int,
              s_stride: Optional[int] = None, dtype: str = "bf16",
              atten_mask=None, topk_mask=None, act_seq_kvlen=None) -> dict:
    """Steps 1-7 for the listed global tokens.

    ``act_seq_kvlen`` (prefix sums, optional): chunked prefill -- each
    sequence's queries are the last of its key/value tokens, so query t has
    position Tkv - Tq + t in both causal rules, and the select blocks follow
    the key/value tokens (``tokens`` still index the query rows).

    q_rows_bits: [n_tok, N1, D1] bits of those tokens' query rows; q, kc and
    vc are all of element type ``dtype``.  ``atten_mask`` / ``topk_mask``:
    None (the positional rules) or 2-D boolean arrays indexed by (local
    query position, compressed entry / select block), True = masked out,
    shared by all sequences.
    Returns dict(out [n,N1,D2], max [n,N1], sum [n,N1],
                 pslc [n,N2,s_stride], topk [n,N2,count] int32).
    """
    q = _u16(q_rows_bits)
    kc = _u16(kc_bits)
    vc = _u16(vc_bits)
    tok = _i64(tokens)
    n_tok = len(tok)
    D1 = kc.shape[2]
    D2 = vc.shape[2]
    if q.shape != (n_tok, N1, D1):
        raise ValueError(f"q rows shape {q.shape} != {(n_tok, N1, D1)}")
    actq = _i64(act_seq_qlen)
    actc = _i64(act_cmp_seq_kvlen)
    actkv = actq if act_seq_kvlen is None else _i64(act_seq_kvlen)
    starts = np.concatenate([[0], actkv[:-1]])
    s_sel_max = int(max(-(-(int(e - s)) // lsel) for s, e in zip(starts, actkv)))
    if s_stride is None:
        s_stride = max(1, s_sel_max)
    out = np.empty((n_tok, N1, D2), dtype=np.float64)
    smax = np.empty((n_tok, N1), dtype=np.float64)
    ssum = np.empty((n_tok, N1), dtype=np.float64)
    pslc = np.empty((n_tok, N2, s_stride), dtype=np.float64)
    topk = np.empty((n_tok, N2, count), dtype=np.int32)

    def mask_arg(m):
        if m is None:
            return None, ctypes.c_void_p(0), 0, 0
        m = np.ascontiguousarray(np.asarray(m, dtype=bool)).view(np.uint8)
        if m.ndim != 2:
            raise ValueError("masks are 2-D (query position, column)")
        return m, _ptr(m), m.shape[0], m.shape[1]

    am, amp, amr, amc = mask_arg(atten_mask)
    tm, tmp, tmr, tmc = mask_arg(topk_mask)
    rc = _load().nsa_oracle_attention_masked(_ptr(q), _ptr(tok), n_tok, _ptr(kc), _ptr(vc),
                                             _ptr(actq), None if act_seq_kvlen is None else _ptr(actkv),
                                             _ptr(actc), len(actq),
                                             N1, N2, D1, D2, float(scale), l, d, lsel, count,
                                             _code(dtype), amp, amr, amc, tmp, tmr, tmc,
                                             _ptr(out), _ptr(smax), _ptr(ssum), _ptr(pslc),
                                             s_stride, _ptr(topk))
    del am, tm
    if rc != 0:
        raise ValueError(f"nsa_oracle_attention returned {rc}")
    return {"out": out, "max": smax, "sum": ssum, "pslc": pslc, "topk": topk}


def run(wl, q_bits, k_bits, v_bits, w_bits, tokens=None, atten_mask=None,
        topk_mask=None) -> dict:
    """The whole path for a workload: compress K and V, round them to the
    workload's element type, then steps 1-7 for ``tokens`` (all tokens when
    None).  ``kc_bits``/``vc_bits`` are the rounded compressed tensors."""
    dt = getattr(wl, "dtype", "bf16")
    actq = np.asarray(wl.act_seq_qlen, dtype=np.int64)
    kc = compress(k_bits, w_bits, actq, wl.l, wl.d, dt)
    vc = compress(v_bits, w_bits, actq, wl.l, wl.d, dt)
    kc_b = round_to(kc, dt)
    vc_b = round_to(vc, dt)
    if tokens is None:
        tokens = np.arange(wl.T, dtype=np.int64)
        q_rows = q_bits
    else:
        tokens = np.asarray(tokens, dtype=np.int64)
        q_rows = q_bits[tokens]
    res = attention(q_rows, tokens, kc_b, vc_b, actq, cmp_prefix(wl.seqlens, wl.l, wl.d),
                    wl.N1, wl.N2, wl.scale, wl.l, wl.d, wl.lsel, wl.count, dtype=dt,
                    atten_mask=atten_mask, topk_mask=topk_mask)
    res.update({"kc": kc, "vc": vc, "kc_bits": kc_b, "vc_bits": vc_b, "tokens": tokens})
    return res


def select_attention(q_bits, k_bits, v_bits, topk, act_seq_qlen, N1: int, N2: int, scale: float,
                     lsel: int, tokens=None, dtype: str = "bf16", act_seq_kvlen=None) -> dict:
    """Selected-block attention for the listed global tokens (all when None).

    q: [T, N1, D1], k: [Tkv, N2, D1], v: [Tkv, N2, D2] bits of element type
    ``dtype`` (Tkv = T unless ``act_seq_kvlen`` gives chunked prefill: each
    sequence's queries are then the last of its key/value tokens); topk:
    [T, N2, count] int32 block indices (-1 unused).
    Returns dict(out [n, N1, D2], lse [n, N1]) in float64."""
    q, k, v = _u16(q_bits), _u16(k_bits), _u16(v_bits)
    topk = np.ascontiguousarray(topk, dtype=np.int32)
    T = q.shape[0]
    Tkv = T if act_seq_kvlen is None else int(np.asarray(act_seq_kvlen)[-1])
    D1, D2 = q.shape[2], v.shape[2]
    if k.shape != (Tkv, N2, D1) or v.shape[:2] != (Tkv, N2) or q.shape[1] != N1:
        raise ValueError("shapes of q, k, v do not match")
    if topk.ndim != 3 or topk.shape[:2] != (T, N2):
        raise ValueError(f"topk must be [{T}, {N2}, count], got {topk.shape}")
    count = topk.shape[2]
    actq = _i64(act_seq_qlen)
    tok = _i64(np.arange(T) if tokens is None else tokens)
    out = np.empty((len(tok), N1, D2), dtype=np.float64)
    lse = np.empty((len(tok), N1), dtype=np.float64)
    actkv = None if act_seq_kvlen is None else _i64(act_seq_kvlen)
    rc = _load().nsa_oracle_select_attention_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(topk), _ptr(tok), len(tok),
                                                _ptr(actq), None if actkv is None else _ptr(actkv), len(actq),
                                                N1, N2, D1, D2, float(scale), lsel, count, _code(dtype),
                                                _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError(f"nsa_oracle_select_attention returned {rc}")
    return {"out": out, "lse": lse}


def attention_backward(q_bits, kc_bits, vc_bits, dout_bits, act_seq_qlen, act_cmp_seq_kvlen,
                       N1: int, N2: int, scale: float, l: int, d: int, dtype: str = "bf16",
                       act_seq_kvlen=None) -> dict:
    """Gradients of steps 1-3 with respect to q, kc and vc for the gradient
    dout [T1, N1, D2] of attention_out (all of element type ``dtype``);
    ``act_seq_kvlen`` (optional prefix sums) puts each sequence's queries at
    the end of its key/value tokens (chunked prefill).
    Returns dict(dq [T1,N1,D1], dkc [T2,N2,D1], dvc [T2,N2,D2]) in float64."""
    q, kc, vc, do = _u16(q_bits), _u16(kc_bits), _u16(vc_bits), _u16(dout_bits)
    T1, D1 = q.shape[0], q.shape[2]
    T2, D2 = kc.shape[0], vc.shape[2]
    if q.shape[1] != N1 or kc.shape[1:] != (N2, D1) or vc.shape[:2] != (T2, N2) or do.shape != (T1, N1, D2):
        raise ValueError("shapes of q, kc, vc, dout do not match")
    actq, actc = _i64(act_seq_qlen), _i64(act_cmp_seq_kvlen)
    dq = np.empty((T1, N1, D1)); dkc = np.empty((T2, N2, D1)); dvc = np.empty((T2, N2, D2))
    actkv = None if act_seq_kvlen is None else _i64(act_seq_kvlen)
    rc = _load().nsa_oracle_attention_backward_kv(_ptr(q), _ptr(kc), _ptr(vc), _ptr(do), _ptr(actq),
                                                  None if actkv is None else _ptr(actkv), _ptr(actc), len(actq),
                                                  N1, N2, D1, D2, float(scale), l, d, _code(dtype),
                                                  _ptr(dq), _ptr(dkc), _ptr(dvc))
    if rc != 0:
        raise ValueError(f"nsa_oracle_attention_backward returned {rc}")
    return {"dq": dq, "dkc": dkc, "dvc": dvc}


def compress_backward(x_bits, w_bits, dy, act_seq_len, l: int, d: int, dtype: str = "bf16") -> dict:
    """Gradients of the compression for the output gradient dy [T2, N, D]
    (float64): dict(dx [T, N, D], dw [l, N]) in float64."""
    x, w = _u16(x_bits), _u16(w_bits)
    T, N, D = x.shape
    dy = np.ascontiguousarray(dy, dtype=np.float64)
    act = _i64(act_seq_len)
    starts = np.concatenate([[0], act[:-1]])
    T2 = int(sum(n_cmp(int(e - s0), l, d) for s0, e in zip(starts, act)))
    if dy.shape != (T2, N, D) or w.shape != (l, N):
        raise ValueError(f"dy must be {(T2, N, D)} and w {(l, N)}")
    dx = np.empty((T, N, D)); dw = np.empty((l, N))
    rc = _load().nsa_oracle_compress_backward(_ptr(x), _ptr(w), _ptr(dy), _ptr(act), len(act), N, D, l, d,
                                              _code(dtype), _ptr(dx), _ptr(dw))
    if rc != 0:
        raise ValueError(f"nsa_oracle_compress_backward returned {rc}")
    return {"dx": dx, "dw": dw}
