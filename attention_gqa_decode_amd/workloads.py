"""Seeded synthetic workloads for grouped-query attention decode and causal prefill.

This module only draws inputs: shapes, seeds and random bf16 tensors.  It holds none of
the attention arithmetic, so the tests, the benchmark and the CPU oracle can all take
their inputs from it without sharing any of the method's code.

Workloads (shapes follow the Llama-3 head layout of page "필수 LLM 최적화 기법(2)"
section 1-1 (32 query heads, 8 KV heads), the 256K-context case of the LeanAttention
digest's evaluation section, and ragged continuous batches of that digest's scheduling
discussion):

* ``tiny``       decode B=1,  Hq=8,  KH=2 (G=4), Hsz=128, L=1024
* ``llama3_8b``  decode B=16, Hq=32, KH=8 (G=4), Hsz=128, L=8192 for every request
* ``long_mqa``   decode B=1,  Hq=8,  KH=1 (G=8), Hsz=128, L=262144 (and x8 scores)
* ``ragged``     decode B=32, Hq=32, KH=8, Hsz=128, L_b log-uniform in [512, 65536]
* ``prefill``    causal prefill B=1, ISL=8192, Hq=32, KH=8, Hsz=128

Values are i.i.d. N(0, 1) drawn in fp32 from a seeded ``torch.Generator`` and rounded to
bf16 (round-to-nearest-even).  Ragged lengths come from ``numpy.random.default_rng``.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class DecodeShape:
    name: str
    B: int
    Hq: int
    KH: int
    Hsz: int
    seqlens: tuple  # per-request context length L_b
    score_mult: float = 1.0  # multiplies the default 1/sqrt(Hsz) softmax scale
    seed: int = 0

    @property
    def G(self) -> int:
        return self.Hq // self.KH

    @property
    def S(self) -> int:
        """KV capacity per (b, kv head): the longest request."""
        return max(self.seqlens) if self.seqlens else 0


@dataclasses.dataclass(frozen=True)
class PrefillShape:
    name: str
    B: int
    ISL: int
    Hq: int
    KH: int
    Hsz: int
    seed: int = 0


def ragged_seqlens(B: int, seed: int, lo: int = 512, hi: int = 65536) -> tuple:
    """Per-request lengths floor(exp(U(ln lo, ln hi))) from numpy's default_rng(seed)."""
    rng = np.random.default_rng(seed)
    L = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), B))).astype(np.int64)
    return tuple(int(x) for x in L)


def decode_workload(name: str, seed: int | None = None) -> DecodeShape:
    if name == "tiny":
        return DecodeShape("tiny", 1, 8, 2, 128, (1024,), seed=1001 if seed is None else seed)
    if name == "llama3_8b":
        return DecodeShape("llama3_8b", 16, 32, 8, 128, (8192,) * 16, seed=1002 if seed is None else seed)
    if name == "long_mqa":
        return DecodeShape("long_mqa", 1, 8, 1, 128, (262144,), seed=1003 if seed is None else seed)
    if name == "long_mqa_x8":
        return DecodeShape("long_mqa_x8", 1, 8, 1, 128, (262144,), score_mult=8.0,
                           seed=1003 if seed is None else seed)
    if name == "ragged":
        s = 0 if seed is None else seed
        return DecodeShape("ragged", 32, 32, 8, 128, ragged_seqlens(32, s), seed=1004 + s)
    raise KeyError(name)


def ragged_sweep_point(G: int, Hsz: int, seed: int = 0) -> DecodeShape:
    """Ragged batch with Hq=32, KH=32/G, Hsz, at the same total KV bytes as the base point.

    Every seeded length is scaled by (8/KH)*(128/Hsz) so KH*Hsz*sum(L) stays fixed and
    the length mix keeps its shape.
    """
    KH = 32 // G
    f = (8 / KH) * (128 / Hsz)
    base = ragged_seqlens(32, seed)
    L = tuple(max(1, int(round(x * f))) for x in base)
    return DecodeShape(f"ragged_G{G}_H{Hsz}", 32, 32, KH, Hsz, L, seed=2000 + 100 * G + Hsz)


def prefill_workload(name: str = "prefill", seed: int | None = None) -> PrefillShape:
    if name == "prefill":
        return PrefillShape("prefill", 1, 8192, 32, 8, 128, seed=1005 if seed is None else seed)
    raise KeyError(name)


def _generator(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def randn_bf16(shape, seed: int, device="cpu") -> torch.Tensor:
    """N(0,1) in fp32 from a seeded generator on ``device``, rounded to bf16 (RNE)."""
    g = _generator(device, seed)
    return torch.randn(shape, generator=g, dtype=torch.float32, device=device).to(torch.bfloat16)


def decode_inputs(shape: DecodeShape, device="cpu", S: int | None = None):
    """(q [B][Hq][Hsz], k [B][KH][S][Hsz], v [B][KH][S][Hsz], seqlens int32 [B]).

    q, k, v are bf16 tensors on ``device``; seqlens is a CPU int32 tensor.  Slots past
    L_b in each (b, kv head) row are filled too (they must never be read).
    """
    S = shape.S if S is None else S
    q = randn_bf16((shape.B, shape.Hq, shape.Hsz), shape.seed, device)
    k = randn_bf16((shape.B, shape.KH, S, shape.Hsz), shape.seed + 7919, device)
    v = randn_bf16((shape.B, shape.KH, S, shape.Hsz), shape.seed + 15485863, device)
    sl = torch.tensor(shape.seqlens, dtype=torch.int32)
    return q, k, v, sl


def prefill_inputs(shape: PrefillShape, device="cpu"):
    """(q [B][Hq][ISL][Hsz], k [B][KH][ISL][Hsz], v [B][KH][ISL][Hsz]) bf16 on ``device``."""
    q = randn_bf16((shape.B, shape.Hq, shape.ISL, shape.Hsz), shape.seed, device)
    k = randn_bf16((shape.B, shape.KH, shape.ISL, shape.Hsz), shape.seed + 7919, device)
    v = randn_bf16((shape.B, shape.KH, shape.ISL, shape.Hsz), shape.seed + 15485863, device)
    return q, k, v


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> its bit patterns as a numpy uint16 array (copied to host)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def decode_inputs_fp8(shape: DecodeShape, device="cpu", k_scale: float = 1.0, v_scale: float = 1.0, S: int | None = None):
    """(q bf16, k, v as uint8 OCP E4M3 codes, seqlens): K/V ~ N(0,1) stored as K/k_scale, V/v_scale.

    The codes come from torch's round-to-nearest-even conversion to float8_e4m3fn after
    clamping to the format's range (|x| <= 448); the attended key is k_scale * code value.
    """
    S = shape.S if S is None else S
    q = randn_bf16((shape.B, shape.Hq, shape.Hsz), shape.seed, device)
    g = _generator(device, shape.seed + 7919)
    k = torch.randn((shape.B, shape.KH, S, shape.Hsz), generator=g, dtype=torch.float32, device=device)
    k = (k / k_scale).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    g = _generator(device, shape.seed + 15485863)
    v = torch.randn((shape.B, shape.KH, S, shape.Hsz), generator=g, dtype=torch.float32, device=device)
    v = (v / v_scale).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    sl = torch.tensor(shape.seqlens, dtype=torch.int32)
    return q, k, v, sl


def codes(t: torch.Tensor) -> np.ndarray:
    """uint8 tensor -> numpy uint8 array (copied to host)."""
    assert t.dtype == torch.uint8
    return t.detach().contiguous().cpu().numpy()


def paged_layout(k: torch.Tensor, v: torch.Tensor, seqlens, block_size: int, seed: int, spare: int = 7):
    """Scatter a contiguous [B][KH][S][Hsz] cache into block pools through a random block map.

    Returns (k_pool, v_pool [num_blocks][KH][block_size][Hsz], block_table int32 [B][max_blocks]
    on k's device).  Request b's logical block i lands in a random physical block; table
    entries past a request's last block are -1 (never read); `spare` extra blocks stay zero.
    """
    B, KH, S, Hsz = k.shape
    nb = [(int(L) + block_size - 1) // block_size for L in seqlens]
    total = sum(nb) + spare
    perm = np.random.default_rng(seed).permutation(total)
    mb = max(max(nb), 1) + 2
    table = np.full((B, mb), -1, dtype=np.int32)
    kp = torch.zeros((total, KH, block_size, Hsz), dtype=k.dtype, device=k.device)
    vp = torch.zeros_like(kp)
    # logical blocks in request order (b, then i) take perm[0], perm[1], ...
    bi = [(b, i) for b in range(B) for i in range(nb[b])]
    if bi:
        for o, (b, i) in enumerate(bi):
            table[b, i] = perm[o]
        nmax = max(nb)
        rows = nmax * block_size  # every request's blocks, zero past its length
        keep = torch.arange(rows, device=k.device)[None, :] < torch.tensor([int(L) for L in seqlens],
                                                                           device=k.device)[:, None]
        dst = torch.from_numpy(perm[:len(bi)].astype(np.int64)).to(k.device)
        src_b = torch.tensor([b for b, _ in bi], device=k.device)
        src_i = torch.tensor([i for _, i in bi], device=k.device)
        for pool, x in ((kp, k), (vp, v)):
            xp = torch.zeros((B, KH, rows, Hsz), dtype=x.dtype, device=x.device)
            n = min(rows, S)
            xp[:, :, :n] = torch.where(keep[:, None, :n, None], x[:, :, :n], torch.zeros((), dtype=x.dtype, device=x.device))
            blocks = xp.view(B, KH, nmax, block_size, Hsz).permute(0, 2, 1, 3, 4)  # [B][block][KH][bs][Hsz]
            pool[dst] = blocks[src_b, src_i]
    return kp, vp, torch.from_numpy(table).to(k.device)

