"""attn_decode_noalloc (the decode entry point that allocates nothing: its workspace is a
fixed device array inside the library) against attn_decode_ex on the same inputs, through
the C ABI.  Two calls in a row, the second smaller; a head split over many workgroups (the
wide merge), device seqlens, multi-token queries, graph capture with replays, and the
size and argument checks.  Bar: max |err| <= 2e-3 against the fp64 oracle, and the two
entry points agree to fp32 rounding (1e-5)."""
import math

import numpy as np
import pytest
import torch

import attention_gqa_decode_amd as A
from attention_gqa_decode_amd import workloads as W
from gpu_util import DECODE_TOL, note, oracle_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def inputs(B, Hq, KH, Hsz, seqlens, seed):
    shape = W.DecodeShape("n", B, Hq, KH, Hsz, tuple(seqlens), seed=seed)
    q, k, v, sl = W.decode_inputs(shape, device="cuda")
    return q, k, v, sl.tolist()


def check_against_ex(q, k, v, sl, rows=None, **kw):
    out = torch.empty((q.shape[0], q.shape[1], q.shape[-1]) if q.dim() == 3 else tuple(q.shape),
                      dtype=torch.float32, device="cuda")
    out.fill_(float("nan"))
    A.attn_decode_noalloc(q, k, v, sl, out, **kw)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    if q.dim() == 3:
        ref_ex = A.attn_decode_ex(q, k, v, sl, **kw)
    else:
        ref_ex = A.attn_decode_multi(q, k, v, sl, **kw)
    torch.cuda.synchronize()
    ref_ex = ref_ex.cpu().double().numpy()
    assert np.all(np.isfinite(got))
    assert np.abs(got - ref_ex).max() <= 1e-5
    if q.dim() == 3:
        KH, Hsz = k.shape[1], k.shape[3]
        ref = oracle_decode(q, k, v, sl if not isinstance(sl, torch.Tensor) else sl.tolist(), KH,
                            1 / math.sqrt(Hsz), rows=rows)
        g = got.reshape(-1, Hsz)
        r = ref.reshape(-1, Hsz)
        sel = np.arange(g.shape[0]) if rows is None else np.asarray(rows)
        err = float(np.abs(g[sel] - r[sel]).max())
        note(f"  max err vs oracle {err:.3e}")
        assert err <= DECODE_TOL
    return got


def test_two_calls_second_smaller():
    note("noalloc: ragged batch, then a smaller forced split")
    q, k, v, sl = inputs(6, 32, 8, 128, [9000, 17, 2500, 20000, 0, 777], seed=901)
    check_against_ex(q, k, v, sl)
    q, k, v, sl = inputs(2, 8, 2, 64, [3000, 5], seed=902)
    check_against_ex(q, k, v, sl, tile_keys=16, num_ctas=100)


def test_wide_head_and_lse():
    # one kv head over every workgroup: the wide merge reads the scratch's partials
    note("noalloc: long context over all workgroups")
    q, k, v, sl = inputs(1, 8, 1, 128, [131072], seed=903)
    lse = torch.empty(8, dtype=torch.float32, device="cuda")
    check_against_ex(q, k, v, sl, out_lse=lse)
    assert torch.isfinite(lse).all()


def test_device_seqlens_and_multi_token():
    note("noalloc: device seqlens, then 4 drafted tokens")
    q, k, v, sl = inputs(3, 16, 4, 128, [4000, 4, 650], seed=904)
    dev = torch.tensor(sl, dtype=torch.int32, device="cuda")
    out = torch.empty((3, 16, 128), dtype=torch.float32, device="cuda")
    A.attn_decode_noalloc(q, k, v, dev, out)
    torch.cuda.synchronize()
    ref = oracle_decode(q, k, v, sl, 4, 1 / math.sqrt(128))
    assert np.abs(out.cpu().double().numpy() - ref).max() <= DECODE_TOL
    qm = W.randn_bf16((3, 16, 4, 128), 905, "cuda")
    check_against_ex(qm, k, v, sl)


def test_graph_capture_replays():
    # captured with the host plan baked in; every replay must match the eager result, with
    # eager work on the same device between replays
    note("noalloc: captured in a graph, replayed 4 times")
    q, k, v, sl = inputs(4, 32, 8, 128, [6000, 300, 12000, 64], seed=906)
    out = torch.empty((4, 32, 128), dtype=torch.float32, device="cuda")
    ref = A.attn_decode_ex(q, k, v, sl)
    torch.cuda.synchronize()
    ref = ref.cpu().double().numpy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        A.attn_decode_noalloc(q, k, v, sl, out)  # first call on this stream outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.attn_decode_noalloc(q, k, v, sl, out)
    for i in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().double().numpy()
        assert np.abs(got - ref).max() <= 1e-5, f"replay {i}"
        A.attn_decode_ex(q[:1].contiguous(), k[:1].contiguous(), v[:1].contiguous(), sl[:1])  # eager work between
        torch.cuda.synchronize()


def test_size_and_argument_checks():
    q, k, v, sl = inputs(2, 128, 2, 128, [20000, 20000], seed=907)  # 64 columns
    out = torch.empty((2, 128, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(A.AttnError) as e:  # 4096 workgroups x 2 slots x 33 KB > the scratch
        A.attn_decode_noalloc(q, k, v, sl, out, num_ctas=4096, tile_keys=16)
    assert e.value.status == A.ATTN_ERR_WORKSPACE
    a, _keep = A._decode_args(q, k, v, sl, out, q_len=1, multi=False, paged=False, block_table=None, scale=0.0,
                              tile_keys=0, num_ctas=0, schedule=0, num_splits=0, k_scale=0.0, v_scale=0.0,
                              out_lse=None, workspace=torch.zeros(1 << 20, dtype=torch.uint8, device="cuda"))
    import ctypes
    assert A.lib().attn_decode_noalloc(ctypes.byref(a), None) == A.ATTN_ERR_SHAPE
    with pytest.raises(ValueError):
        A.attn_decode_noalloc(q, k, v, sl, None)
