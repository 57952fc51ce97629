"""Seeded synthetic inputs for the compressed branch of Native Sparse Attention.

This module only draws numbers.  It holds none of the method's arithmetic:
no compression, no visibility rule, no attention, no remap and no top-k.
Both the HIP path (through its tests and the benchmark) and the CPU oracle
consume what it produces, so it is the one piece of code they share.

Recipe (the same for every workload):

* q, k and v are drawn as float32 normals with a workload-specific standard
  deviation, then rounded to the workload's element type (bfloat16 or
  float16) with round-to-nearest-even (torch's float32 conversion).
* the compression weight ``w[l, N2]`` is drawn as float32 U(0, w_hi) and
  rounded the same way.
* each tensor has its own ``torch.Generator`` seeded from (workload seed,
  tensor id) with ids q=0, k=1, v=2, w=3.  Draws happen in token-major
  chunks, so a tensor's values depend only on the seed, the chunk size and
  the device type (CPU and GPU generators differ; a test always compares
  the two sides on the same bytes, copied across when needed).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "w": 3}
TORCH_DTYPES = {"bf16": torch.bfloat16, "f16": torch.float16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes, method parameters and value distributions of one input set."""

    name: str
    seqlens: tuple          # per-sequence token counts (TND varlen)
    N1: int                 # query heads
    N2: int                 # key/value heads
    D1: int                 # q/k head dim
    D2: int                 # v head dim
    l: int                  # compress_block_size
    d: int                  # compress_stride
    lsel: int               # select_block_size (l')
    count: int              # select_block_count
    scale: float            # scale_value
    q_std: float = 1.0
    kv_std: float = 1.0
    w_hi: float = 1.0 / 16  # weight ~ U(0, w_hi)
    seed: int = 0
    dtype: str = "bf16"     # element type of q, k, v and the weight: "bf16" or "f16"

    @property
    def B(self) -> int:
        return len(self.seqlens)

    @property
    def T(self) -> int:
        return int(sum(self.seqlens))

    @property
    def act_seq_qlen(self) -> List[int]:
        """Token counts as the prefix sums the operator takes."""
        return [int(x) for x in np.cumsum(self.seqlens)]

    def with_seqlens(self, seqlens, name: Optional[str] = None) -> "Workload":
        return dataclasses.replace(self, seqlens=tuple(int(s) for s in seqlens),
                                   name=name or f"{self.name}-lens{list(seqlens)}")

    @property
    def torch_dtype(self) -> torch.dtype:
        return TORCH_DTYPES[self.dtype]

    def with_dtype(self, dtype: str) -> "Workload":
        if dtype not in TORCH_DTYPES:
            raise ValueError(f"dtype must be one of {sorted(TORCH_DTYPES)}, got {dtype!r}")
        if dtype == self.dtype:
            return self
        return dataclasses.replace(self, dtype=dtype, name=f"{self.name}-{dtype}")

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "T": self.T, "N1": self.N1,
                "N2": self.N2, "D1": self.D1, "D2": self.D2, "l": self.l, "d": self.d,
                "lsel": self.lsel, "count": self.count, "scale": self.scale,
                "dtype": self.dtype}


def _batched_lens_16() -> tuple:
    # 16 lengths drawn uniformly from the multiples of 128 in [8192, 32768].
    return tuple(int(x) for x in np.random.default_rng(4).integers(64, 257, 16) * 128)


# The five workloads.  Where a workload names no scale, head_dim**-0.5 is
# used (the convention the sparse-attention wrappers state as their default).
WORKLOADS = {
    0: Workload("tiny-T512-N4x1-D64", (512,), 4, 1, 64, 64, 32, 16, 64, 4, 1.0 / 8,
                q_std=1.0, kv_std=1.0, w_hi=2.0 / 32, seed=100),
    1: Workload("mqa-T8192-N16x1-D192x128", (8192,), 16, 1, 192, 128, 32, 16, 64, 16,
                192 ** -0.5, w_hi=1.0 / 16, seed=101),
    2: Workload("varlen-gqa-B4-N64x4-D128", (4096, 16384, 1024, 10752), 64, 4, 128, 128,
                32, 16, 64, 16, 128 ** -0.5, w_hi=1.0 / 16, seed=102),
    3: Workload("long-T65536-N64x4-D192x128", (65536,), 64, 4, 192, 128, 64, 32, 128, 32,
                192 ** -0.5, w_hi=1.0 / 32, seed=103),
    4: Workload("batched-varlen-B16-N64x1-D128", _batched_lens_16(), 64, 1, 128, 128,
                32, 16, 64, 16, 128 ** -0.5, kv_std=0.5, w_hi=1.0 / 16, seed=104),
}


def small_variant(wid: int, seqlens) -> Workload:
    """Workload ``wid`` with shorter, ragged sequences (same heads, dims and
    method parameters) -- for full-output comparisons the oracle finishes in
    seconds."""
    base = WORKLOADS[wid]
    return dataclasses.replace(base, seqlens=tuple(int(s) for s in seqlens),
                               name=f"{base.name}@lens{list(seqlens)}")


def _seed(wl: Workload, tensor: str) -> int:
    return (wl.seed * 1_000_003 + TENSOR_IDS[tensor] * 7919) & 0x7FFF_FFFF_FFFF


def _draw(shape, seed: int, device, kind: str, a: float, chunk_rows: int,
          dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """Draw ``shape`` values in row chunks, round each chunk to ``dtype``."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = torch.empty(shape, dtype=dtype, device=device)
    rows = shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        sub = (r1 - r0,) + tuple(shape[1:])
        if kind == "normal":
            x = torch.randn(sub, generator=gen, device=device, dtype=torch.float32)
            if a != 1.0:
                x.mul_(a)
        else:  # uniform on [0, a)
            x = torch.rand(sub, generator=gen, device=device, dtype=torch.float32)
            x.mul_(a)
        out[r0:r1] = x.to(dtype)
        del x
    return out


def make_inputs(wl: Workload, device="cpu", chunk_rows: int = 8192,
                tensors=("q", "k", "v", "w")) -> dict:
    """Tensors q [T,N1,D1], k [T,N2,D1], v [T,N2,D2] and w [l,N2] of the
    workload's element type."""
    T = wl.T
    dt = wl.torch_dtype
    out = {}
    if "q" in tensors:
        out["q"] = _draw((T, wl.N1, wl.D1), _seed(wl, "q"), device, "normal", wl.q_std,
                         chunk_rows, dt)
    if "k" in tensors:
        out["k"] = _draw((T, wl.N2, wl.D1), _seed(wl, "k"), device, "normal", wl.kv_std,
                         chunk_rows, dt)
    if "v" in tensors:
        out["v"] = _draw((T, wl.N2, wl.D2), _seed(wl, "v"), device, "normal", wl.kv_std,
                         chunk_rows, dt)
    if "w" in tensors:
        out["w"] = _draw((wl.l, wl.N2), _seed(wl, "w"), device, "uniform", wl.w_hi,
                         chunk_rows, dt)
    return out


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The raw bfloat16 bit patterns of a CPU tensor as a uint16 numpy array."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bf16_bits(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    """The raw bit patterns of a bfloat16 or float16 tensor as uint16."""
    assert t.dtype in (torch.bfloat16, torch.float16)
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray, dtype: str = "bf16") -> torch.Tensor:
    """A CPU tensor of element type ``dtype`` holding the bit patterns ``a``."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(
        TORCH_DTYPES[dtype])


def sample_tokens(wl: Workload, per_seq: int, rng_seed: int = 7) -> np.ndarray:
    """Global token indices: the first and last tokens of every sequence,
    tokens around the first compressed block and the first selected-block
    boundaries, plus ``per_seq`` seeded random positions per sequence."""
    rng = np.random.default_rng(rng_seed)
    starts = np.concatenate([[0], np.cumsum(wl.seqlens)[:-1]])
    picks = []
    for s0, T in zip(starts, wl.seqlens):
        fixed = [0, 1, wl.l - 2, wl.l - 1, wl.l, wl.lsel - 1, wl.lsel,
                 wl.count * wl.lsel - 1, wl.count * wl.lsel, T // 2, T - 2, T - 1]
        rand = rng.integers(0, T, per_seq) if T > 0 else []
        for t in list(fixed) + list(rand):
            if 0 <= t < T:
                picks.append(int(s0 + t))
    return np.unique(np.array(picks, dtype=np.int64))


def random_block_lists(wl: Workload, seed: int = 11, p_pad: float = 0.15, p_repeat: float = 0.05,
                       p_bad: float = 0.03) -> np.ndarray:
    """[T, N2, count] int32 lists of select-block indices drawn uniformly
    from [0, ceil(T_b / l')) of each token's sequence, with seeded -1 padding,
    repeats, and entries outside that range (past it, or negative other
    than -1) -- inputs for the attention over selected blocks."""
    rng = np.random.default_rng(seed)
    out = np.empty((wl.T, wl.N2, wl.count), dtype=np.int64)
    s0 = 0
    for T in wl.seqlens:
        S = max(1, -(-T // wl.lsel))
        blk = rng.integers(0, S, (T, wl.N2, wl.count))
        u = rng.random((T, wl.N2, wl.count))
        rep = np.roll(blk, 1, axis=2)
        blk = np.where(u < p_repeat, rep, blk)
        blk = np.where((u >= p_repeat) & (u < p_repeat + p_bad),
                       np.where(rng.random(blk.shape) < 0.5, S + rng.integers(0, 3, blk.shape), -7), blk)
        blk = np.where(rng.random(blk.shape) < p_pad, -1, blk)
        out[s0:s0 + T] = blk
        s0 += T
    return out.astype(np.int32)


def make_output_grad(wl: Workload, device="cpu", seed: int = 77, chunk_rows: int = 8192) -> torch.Tensor:
    """A seeded N(0, 1) gradient for attention_out [T, N1, D2] in the
    workload's element type (for the backward)."""
    return _draw((wl.T, wl.N1, wl.D2), (wl.seed * 1_000_003 + seed * 7919) & 0x7FFF_FFFF_FFFF, device,
                 "normal", 1.0, chunk_rows, wl.torch_dtype)
