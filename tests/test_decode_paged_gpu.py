"""GPU parity of decode over a paged KV cache (block tables).

The pools [num_blocks][KH][block_size][Hsz] are filled from a contiguous cache through a
random block permutation; the paged result must match the contiguous path (same numbers
up to fp32 summation order) and the fp64 oracle on the contiguous data (max |err| <= 2e-3).
The layout follows the block-table design of "필수 LLM 최적화 기법(2)", section 3
(PagedAttention: fixed-size KV blocks found through a lookup table).
"""
import math

import numpy as np
import pytest
import torch

import attention_gqa_decode_amd as A
from attention_gqa_decode_amd import workloads as W
from gpu_util import DECODE_TOL, gpu_decode, note, oracle_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def to_paged(k, v, seqlens, bs, seed):
    return W.paged_layout(k, v, seqlens, bs, seed)


@pytest.mark.parametrize("bs", [16, 32, 64, 256])
@pytest.mark.parametrize("Hsz", [64, 128])
def test_paged_matches_contiguous_and_oracle(bs, Hsz):
    sl = [1000, 0, 1, 333, 4097]
    note(f"paged decode bs={bs} Hsz={Hsz}")
    shape = W.DecodeShape("p", len(sl), 16, 4, Hsz, tuple(sl), seed=60 + bs + Hsz)
    q, k, v, _ = W.decode_inputs(shape, device="cuda")
    kp, vp, table = to_paged(k, v, sl, bs, seed=bs)
    got = A.attn_decode_paged(q, kp, vp, table, sl)
    torch.cuda.synchronize()
    got = got.cpu().double().numpy()
    base = gpu_decode(q, k, v, sl)
    assert np.abs(got - base).max() <= 1e-5
    ref = oracle_decode(q, k, v, sl, 4, 1 / math.sqrt(Hsz))
    err = float(np.abs(got - ref).max())
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL
    assert np.all(got[1] == 0)


@pytest.mark.parametrize("T,P", [(16, 5), (48, 200), (1024, 2)])
def test_paged_forced_splits(T, P):
    sl = [3000, 1777]
    shape = W.DecodeShape("p", 2, 8, 2, 128, tuple(sl), seed=61)
    q, k, v, _ = W.decode_inputs(shape, device="cuda")
    kp, vp, table = to_paged(k, v, sl, 16, seed=T + P)
    got = A.attn_decode_paged(q, kp, vp, table, sl, tile_keys=T, num_ctas=P)
    torch.cuda.synchronize()
    ref = oracle_decode(q, k, v, sl, 2, 1 / math.sqrt(128))
    assert np.abs(got.cpu().double().numpy() - ref).max() <= DECODE_TOL


def test_paged_fp8():
    sl = [2500, 640, 3]
    shape = W.DecodeShape("p", 3, 16, 4, 128, tuple(sl), seed=62)
    q, k, v, _ = W.decode_inputs_fp8(shape, device="cuda", k_scale=0.5, v_scale=2.0)
    kp, vp, table = to_paged(k, v, sl, 32, seed=62)
    got = A.attn_decode_paged(q, kp, vp, table, sl, k_scale=0.5, v_scale=2.0)
    base = A.attn_decode_ex(q, k, v, sl, k_scale=0.5, v_scale=2.0)
    torch.cuda.synchronize()
    assert (got - base).abs().max().item() <= 1e-5


def test_paged_full_size_llama3():
    s = W.decode_workload("llama3_8b")
    note("paged decode full-size llama3_8b, block size 16")
    q, k, v, sl = W.decode_inputs(s, device="cuda")
    sl = sl.tolist()
    kp, vp, table = to_paged(k, v, sl, 16, seed=63)
    got = A.attn_decode_paged(q, kp, vp, table, sl)
    torch.cuda.synchronize()
    ref = oracle_decode(q, k, v, sl, s.KH, 1 / math.sqrt(s.Hsz))
    err = float(np.abs(got.cpu().double().numpy() - ref).max())
    note(f"  max err {err:.3e}")
    assert err <= DECODE_TOL
    del q, k, v, kp, vp
    torch.cuda.empty_cache()


def test_paged_wide_head():
    # 16-key blocks, one long head split over 200 CTAs (wide merge kernel)
    sl = [30000, 100]
    shape = W.DecodeShape("p", 2, 8, 1, 128, tuple(sl), seed=62)
    q, k, v, _ = W.decode_inputs(shape, device="cuda")
    kp, vp, table = to_paged(k, v, sl, 16, seed=62)
    got = A.attn_decode_paged(q, kp, vp, table, sl, tile_keys=64, num_ctas=200)
    torch.cuda.synchronize()
    got = got.cpu().double().numpy()
    base = gpu_decode(q, k, v, sl, tile_keys=64, num_ctas=200)
    assert np.abs(got - base).max() <= 1e-5
    ref = oracle_decode(q, k, v, sl, 1, 1 / math.sqrt(128))
    err = float(np.abs(got - ref).max())
    note(f"paged wide head: max err {err:.3e}")
    assert err <= DECODE_TOL
