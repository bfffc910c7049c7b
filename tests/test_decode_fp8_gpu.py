"""GPU parity of the FP8 E4M3 KV-cache decode against the fp64 oracle.

The caches hold OCP E4M3 codes with one scale per tensor; the oracle decodes the same
codes exactly (its decoder is pinned against torch's float8_e4m3fn on all 256 codes).
Every E4M3 value is a bf16 value, so the kernel widens K and V exactly and the bar is the
bf16 path's: max |err| <= 2e-3 on the fp32 outputs.
"""
import math

import numpy as np
import pytest
import torch

import attention_gqa_decode_amd as A
import oracle
from attention_gqa_decode_amd import workloads as W
from attention_gqa_decode_amd.workloads import bits, codes
from gpu_util import DECODE_TOL, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def fp8_err(shape, k_scale=1.0, v_scale=1.0, rows=None, S=None, **kw):
    q, k, v, sl = W.decode_inputs_fp8(shape, device="cuda", k_scale=k_scale, v_scale=v_scale, S=S)
    scale = shape.score_mult / math.sqrt(shape.Hsz)
    out = A.attn_decode_ex(q, k, v, sl.tolist(), scale=scale if shape.score_mult != 1.0 else 0.0,
                           k_scale=k_scale, v_scale=v_scale, **kw)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy().reshape(shape.B * shape.Hq, shape.Hsz)
    ref = oracle.decode_fp8(bits(q), codes(k), codes(v), sl.numpy(), shape.Hq, shape.KH, scale, k_scale, v_scale,
                            rows=rows).reshape(shape.B * shape.Hq, shape.Hsz)
    sel = np.arange(shape.B * shape.Hq) if rows is None else np.asarray(rows)
    assert np.all(np.isfinite(got[sel]))
    return float(np.abs(got[sel] - ref[sel]).max()), (q, k, v, sl)


@pytest.mark.parametrize("Hsz", [64, 128, 256])
@pytest.mark.parametrize("G", [1, 4, 8, 16])
def test_fp8_shapes_ragged(Hsz, G):
    s = W.DecodeShape("f", 4, 2 * G, 2, Hsz, (1, 333, 1000, 64), seed=40 + G + Hsz)
    note(f"fp8 decode Hsz={Hsz} G={G}")
    err, _ = fp8_err(s)
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL


@pytest.mark.parametrize("k_scale,v_scale", [(0.5, 2.0), (0.0625, 0.125), (3.0, 0.7)])
def test_fp8_scales(k_scale, v_scale):
    s = W.DecodeShape("f", 3, 16, 4, 128, (3000, 5, 777), seed=50)
    note(f"fp8 decode k_scale={k_scale} v_scale={v_scale}")
    err, _ = fp8_err(s, k_scale=k_scale, v_scale=v_scale)
    assert err <= DECODE_TOL


@pytest.mark.parametrize("T,P", [(16, 7), (64, 300), (1024, 3)])
def test_fp8_forced_splits(T, P):
    s = W.DecodeShape("f", 2, 8, 2, 128, (4000, 999), seed=51)
    err, _ = fp8_err(s, tile_keys=T, num_ctas=P)
    assert err <= DECODE_TOL


def test_fp8_equals_bf16_path_on_the_same_values():
    # widening the codes to bf16 outside the library and taking the bf16 path must give
    # the same numbers up to the order of fp32 additions
    s = W.DecodeShape("f", 2, 16, 4, 128, (2500, 1300), seed=52)
    q, k, v, sl = W.decode_inputs_fp8(s, device="cuda", k_scale=0.5, v_scale=2.0)
    a = A.attn_decode_ex(q, k, v, sl.tolist(), k_scale=0.5, v_scale=2.0)
    kb = k.view(torch.float8_e4m3fn).to(torch.bfloat16)
    vb = v.view(torch.float8_e4m3fn).to(torch.bfloat16)
    b = A.attn_decode_ex(q, kb, vb, sl.tolist(), scale=0.5 / math.sqrt(128))
    torch.cuda.synchronize()
    assert (a - 2.0 * b).abs().max().item() <= 1e-5


def test_fp8_torch_float8_tensor_accepted():
    s = W.DecodeShape("f", 1, 8, 2, 128, (300,), seed=53)
    q, k, v, sl = W.decode_inputs_fp8(s, device="cuda")
    a = A.attn_decode_ex(q, k, v, sl.tolist())
    b = A.attn_decode_ex(q, k.view(torch.float8_e4m3fn), v.view(torch.float8_e4m3fn), sl.tolist())
    torch.cuda.synchronize()
    assert torch.equal(a, b) or (a - b).abs().max().item() <= 1e-5


@pytest.mark.parametrize("name", ["llama3_8b", "long_mqa", "long_mqa_x8", "ragged"])
def test_fp8_full_size_workloads(name):
    s = W.decode_workload(name)
    note(f"fp8 decode full-size {name}")
    rows = None if name != "ragged" else np.random.default_rng(54).choice(s.B * s.Hq, 128, replace=False)
    err, t = fp8_err(s, rows=rows)
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL
    del t
    torch.cuda.empty_cache()


def test_fp8_wide_head():
    # one long head split over 300 CTAs: the wide merge kernel applies the value scale
    shape = W.DecodeShape("w", 1, 8, 1, 128, (40000,), seed=95)
    err, _ = fp8_err(shape, k_scale=0.5, v_scale=2.0, tile_keys=64, num_ctas=300)
    note(f"fp8 wide head: max err {err:.3e}")
    assert err <= DECODE_TOL
