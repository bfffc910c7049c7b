"""GPU parity of decode with the context lengths in device memory (``seqlens_on_device``).

The LeanTile plan is then built on the device in front of the decode kernel, so the call
reads nothing on the host and can be captured in a HIP graph whose replays see new
lengths.  The same oracle bar as host lengths (max |err| <= 2e-3 on fp32 outputs); against
the host-length path the results agree to fp32 summation order (1e-5).  Lengths outside
[0, kv_stride] are clamped into it on the device.
"""
import math

import numpy as np
import pytest
import torch

import attention_gqa_decode_amd as A
import oracle
from attention_gqa_decode_amd import workloads as W
from attention_gqa_decode_amd.workloads import bits
from gpu_util import DECODE_TOL, gpu_decode, note, oracle_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def inputs(B, Hq, KH, Hsz, seqlens, seed, S=None):
    shape = W.DecodeShape("d", B, Hq, KH, Hsz, tuple(seqlens), seed=seed)
    q, k, v, sl = W.decode_inputs(shape, device="cuda", S=S)
    return q, k, v, sl.tolist()


def dev(sl):
    return torch.tensor(sl, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("sl,KH,G,Hsz,kw", [
    ([1000, 0, 1, 333, 4097], 2, 4, 128, {}),
    ([8192] * 4, 2, 4, 128, dict(tile_keys=64, num_ctas=100)),
    ([65536], 1, 8, 128, dict(tile_keys=64, num_ctas=300)),            # one head over 300 CTAs (wide merge)
    ([100, 2000, 40000, 7], 2, 2, 64, dict(num_ctas=2000, tile_keys=16)),
    ([3000, 1, 0, 700], 4, 4, 256, dict(schedule=A.ATTN_SCHEDULE_FIXED_SPLIT, num_splits=20)),
    ([3000, 1, 0, 700], 4, 4, 128, dict(schedule=A.ATTN_SCHEDULE_FIXED_SPLIT)),
    ([0, 0, 0], 2, 4, 128, {}),                                          # an all-empty batch
])
def test_device_seqlens_match_oracle_and_host_path(sl, KH, G, Hsz, kw):
    note(f"device seqlens decode sl={sl} KH={KH} G={G} Hsz={Hsz} {kw}")
    q, k, v, sl = inputs(len(sl), G * KH, KH, Hsz, sl, seed=300 + len(sl) + Hsz, S=max(max(sl), 1))
    got = gpu_decode(q, k, v, dev(sl), **kw)
    ref = oracle_decode(q, k, v, sl, KH, 1 / math.sqrt(Hsz))
    err = float(np.abs(got - ref).max())
    note(f"  max err {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= DECODE_TOL
    host = gpu_decode(q, k, v, sl, **kw)
    assert np.abs(got - host).max() <= 1e-5
    for b, L in enumerate(sl):
        if L == 0:
            assert np.all(got[b] == 0)


def test_device_seqlens_are_clamped_into_the_cache():
    # 9000 > S = 5000 reads as 5000, -3 as 0: never an access outside the cache
    q, k, v, _ = inputs(3, 8, 2, 128, [5000, 5000, 5000], seed=310)
    got = gpu_decode(q, k, v, dev([9000, -3, 1234]))
    ref = oracle_decode(q, k, v, [5000, 0, 1234], 2, 1 / math.sqrt(128))
    assert np.abs(got - ref).max() <= DECODE_TOL
    assert np.all(got[1] == 0)


def test_device_seqlens_paged_fp8_and_multi_token():
    # paged cache
    sl = [3000, 17, 900]
    shape = W.DecodeShape("p", 3, 8, 2, 128, tuple(sl), seed=311)
    q, k, v, _ = W.decode_inputs(shape, device="cuda")
    kp, vp, table = W.paged_layout(k, v, sl, 16, 311)
    got = A.attn_decode_paged(q, kp, vp, table, dev(sl), num_ctas=64)
    torch.cuda.synchronize()
    ref = oracle_decode(q, k, v, sl, 2, 1 / math.sqrt(128))
    assert np.abs(got.cpu().double().numpy() - ref).max() <= DECODE_TOL
    # FP8 cache with scales
    shape = W.DecodeShape("f", 2, 8, 2, 128, (2500, 600), seed=312)
    q, k8, v8, sl8 = W.decode_inputs_fp8(shape, device="cuda", k_scale=0.5, v_scale=2.0)
    got = A.attn_decode_ex(q, k8, v8, dev(sl8.tolist()), k_scale=0.5, v_scale=2.0, num_ctas=50)
    torch.cuda.synchronize()
    ref = oracle.decode_fp8(bits(q), W.codes(k8), W.codes(v8), sl8.numpy(), 8, 2, 1 / math.sqrt(128), 0.5, 2.0)
    assert np.abs(got.cpu().double().numpy() - ref.reshape(got.shape)).max() <= DECODE_TOL
    # multi-token (gamma = 4): the drafted tokens' causal limits come from the device lengths
    sl = [1000, 37]
    shape = W.DecodeShape("m", 2, 8, 2, 128, tuple(sl), seed=313)
    qm = W.randn_bf16((2, 8, 4, 128), 313, "cuda")
    _, k, v, _ = W.decode_inputs(shape, device="cuda")
    got = A.attn_decode_multi(qm, k, v, dev(sl), tile_keys=16, num_ctas=40)
    torch.cuda.synchronize()
    ref = oracle.decode_multi(bits(qm), bits(k), bits(v), sl, 2, 1 / math.sqrt(128))
    assert np.abs(got.cpu().double().numpy() - ref.reshape(got.shape)).max() <= DECODE_TOL


def test_graph_capture_with_device_seqlens():
    """One decode call captured in a graph (plan kernel, decode kernel, wide merge kernel) with
    a caller workspace; every replay, with new lengths written into the device tensor in
    between and eager work around it, matches the eager call and the oracle."""
    B, KH, G, Hsz, S = 3, 1, 8, 128, 40000
    q, k, v, _ = inputs(B, G * KH, KH, Hsz, [S] * B, seed=320)
    ws = torch.zeros(A.attn_decode_workspace_bytes(B, G * KH, KH, Hsz, 256) // 4 + 1, dtype=torch.int32, device="cuda")
    sl_dev = dev([S, 100, 7])
    out = torch.empty((B, G * KH, Hsz), dtype=torch.float32, device="cuda")
    kw = dict(workspace=ws, num_ctas=256, tile_keys=64)
    A.attn_decode_ex(q, k, v, sl_dev, out, **kw)  # warm-up outside the capture (device queries, attributes)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.attn_decode_ex(q, k, v, sl_dev, out, **kw)
    torch.cuda.synchronize()
    for step, sl in enumerate([[S, 100, 7], [123, S, 0], [30000, 1, 20001], [S, S, S]]):
        sl_dev.copy_(torch.tensor(sl, dtype=torch.int32))
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().double().numpy()
        eager = gpu_decode(q, k, v, sl, num_ctas=256, tile_keys=64)  # eager work between replays
        ref = oracle_decode(q, k, v, sl, KH, 1 / math.sqrt(Hsz))
        err = float(np.abs(got - ref).max())
        note(f"graph replay {step} sl={sl}: max err {err:.3e}")
        assert err <= DECODE_TOL
        assert np.abs(got - eager).max() <= 1e-5
