"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI, run the
oracle on the same bf16 bytes, and compare."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import attention_gqa_decode_amd as A
import oracle
from attention_gqa_decode_amd.workloads import bits

DECODE_TOL = 2e-3  # max |err| on fp32 outputs, bf16 unit-scale inputs


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_decode(q, k, v, seqlens, **kw):
    out = A.attn_decode_ex(q, k, v, seqlens, **kw)
    torch.cuda.synchronize()
    return out.cpu().double().numpy()


def oracle_decode(q, k, v, seqlens, KH, scale, rows=None):
    Hq = q.shape[1]
    return oracle.decode(bits(q), bits(k), bits(v), np.asarray(seqlens), Hq, KH, scale, rows=rows)


def decode_err(q, k, v, seqlens, scale_mult=1.0, rows=None, **kw):
    """max |GPU - oracle| over the listed rows (all rows if None)."""
    KH, Hsz = k.shape[1], k.shape[3]
    scale = scale_mult / math.sqrt(Hsz)
    got = gpu_decode(q, k, v, seqlens, scale=scale if scale_mult != 1.0 else 0.0, **kw)
    ref = oracle_decode(q, k, v, seqlens, KH, scale, rows)
    B, Hq, _ = q.shape
    flat_g, flat_r = got.reshape(B * Hq, Hsz), ref.reshape(B * Hq, Hsz)
    sel = np.arange(B * Hq) if rows is None else np.asarray(rows)
    assert np.all(np.isfinite(flat_g[sel])), "non-finite GPU output"
    return float(np.abs(flat_g[sel] - flat_r[sel]).max()), got


def bf16_half_ulp(x: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |x|: 2**(floor(log2|x|) - 8); tiny floor for x ~ 0."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.ldexp(1.0, (np.floor(np.log2(ax)) - 8).astype(np.int64))
