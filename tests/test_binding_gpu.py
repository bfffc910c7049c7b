"""The Python binding rejects tensors the library would misuse (wrong dtype, shape, device or
layout of out, out_lse, workspace) before anything reaches the library."""
import pytest
import torch

import attention_gqa_decode_amd as A
from attention_gqa_decode_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def small():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    s = W.DecodeShape("binding", 2, 8, 2, 64, (100, 37), seed=77)
    return W.decode_inputs(s, device="cuda")


@pytest.mark.parametrize("bad", [
    lambda B, Hq, Hsz: torch.empty((B, Hq, Hsz), dtype=torch.bfloat16, device="cuda"),   # wrong dtype
    lambda B, Hq, Hsz: torch.empty((B, Hq, Hsz - 4), dtype=torch.float32, device="cuda"),  # too small
    lambda B, Hq, Hsz: torch.empty((B, Hq, Hsz), dtype=torch.float32),                    # host memory
    lambda B, Hq, Hsz: torch.empty((B, Hsz, Hq), dtype=torch.float32, device="cuda").transpose(1, 2),  # strided
])
def test_bad_out_is_rejected(small, bad):
    q, k, v, sl = small
    B, Hq, Hsz = q.shape
    out = bad(B, Hq, Hsz)
    for call in (lambda: A.attn_decode_ex(q, k, v, sl.tolist(), out=out),
                 lambda: A.attn_decode(q, k[:, :, :100].contiguous(), v[:, :, :100].contiguous(), sl.tolist(), out=out),
                 lambda: A.PreparedDecode(q, k, v, sl.tolist(), out)):
        with pytest.raises((TypeError, ValueError)):
            call()


def test_bad_multi_out_is_rejected(small):
    _, k, v, sl = small
    q = W.randn_bf16((2, 8, 3, 64), 5, "cuda")
    with pytest.raises(ValueError):
        A.attn_decode_multi(q, k, v, sl.tolist(), out=torch.empty((2, 8, 64), dtype=torch.float32, device="cuda"))


def test_bad_lse_and_workspace_are_rejected(small):
    q, k, v, sl = small
    with pytest.raises(ValueError):
        A.attn_decode_ex(q, k, v, sl.tolist(), out_lse=torch.empty(3, dtype=torch.float32, device="cuda"))
    with pytest.raises(TypeError):
        A.attn_decode_ex(q, k, v, sl.tolist(), out_lse=torch.empty(16, dtype=torch.float64, device="cuda"))
    with pytest.raises(TypeError):
        A.attn_decode_ex(q, k, v, sl.tolist(), workspace=torch.zeros(1 << 16, dtype=torch.float32))
    outs = torch.zeros((2, 4, 64), dtype=torch.float32, device="cuda")
    lses = torch.zeros((2, 4), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        A.attn_merge_shards(outs, lses, lse_out=torch.empty(3, dtype=torch.float32, device="cuda"))
    with pytest.raises(TypeError):
        A.attn_merge_shards(outs, lses, out=torch.empty((4, 64), dtype=torch.float32))
