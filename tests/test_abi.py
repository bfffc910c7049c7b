"""CPU tests of the C ABI: the library loads, exports every declared symbol, and rejects bad
arguments synchronously (before any HIP call, so these run without a GPU).

Only argument combinations that fail validation are passed; the fake device addresses
below are never dereferenced.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import attention_gqa_decode_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_gqa.h")
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["attn_decode", "attn_decode_ex", "attn_decode_workspace_bytes", "attn_prefill_causal",
              "attn_decode_plan", "attn_hbm_copy_probe", "attn_device_info", "attn_release",
              "attn_status_string", "attn_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = A.lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_no_oracle_symbols_in_library():
    lib = A.lib()
    for n in ["oracle_decode_f64", "oracle_prefill_causal_f64", "oracle_bf16_to_f64"]:
        assert not hasattr(lib, n)


def test_status_strings():
    lib = A.lib()
    for code in [0, -1, -2, -3, -4, -5, -6]:
        assert lib.attn_status_string(code).decode() not in ("", "unknown status")
    assert lib.attn_status_string(-99).decode() == "unknown status"


def call_decode(q=FAKE, k=FAKE, v=FAKE, sl=(4, 4), B=2, Hq=8, KH=2, Hsz=128, out=FAKE):
    lib = A.lib()
    arr = None if sl is None else np.ascontiguousarray(sl, dtype=np.int32)
    return lib.attn_decode(q, k, v, None if arr is None else arr.ctypes.data, B, Hq, KH, Hsz, out, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), A.ATTN_ERR_NULL),
    (dict(k=None), A.ATTN_ERR_NULL),
    (dict(v=None), A.ATTN_ERR_NULL),
    (dict(out=None), A.ATTN_ERR_NULL),
    (dict(sl=None), A.ATTN_ERR_NULL),
    (dict(B=0, sl=(4,)), A.ATTN_ERR_SHAPE),
    (dict(Hq=6, KH=4), A.ATTN_ERR_SHAPE),
    (dict(KH=0), A.ATTN_ERR_SHAPE),
    (dict(Hsz=96), A.ATTN_ERR_UNSUPPORTED),
    (dict(Hsz=512), A.ATTN_ERR_UNSUPPORTED),
    (dict(Hq=256, KH=2), A.ATTN_ERR_UNSUPPORTED),              # G = 128 > 64 query columns
    (dict(Hq=128, KH=2, Hsz=256), A.ATTN_ERR_UNSUPPORTED),     # 64 columns x 256 > 8192
    (dict(B=257, sl=(1,) * 257), A.ATTN_ERR_UNSUPPORTED),
    (dict(q=FAKE + 2), A.ATTN_ERR_ALIGN),
    (dict(out=FAKE + 4), A.ATTN_ERR_ALIGN),
    (dict(v=FAKE + 8), A.ATTN_ERR_ALIGN),
    (dict(sl=(4, -1)), A.ATTN_ERR_SHAPE),
])
def test_decode_rejects_bad_arguments(kw, status):
    assert call_decode(**kw) == status
    assert A.lib().attn_last_error().decode() != ""


def ex_args(**kw):
    a = A.attn_decode_args()
    sl = np.ascontiguousarray(kw.pop("seqlens", (4, 4)), dtype=np.int32)
    a.q = a.k_cache = a.v_cache = a.out = FAKE
    a.seqlens = sl.ctypes.data
    a.B, a.Hq, a.KH, a.Hsz = 2, 8, 2, 128
    for k, v in kw.items():
        setattr(a, k, v)
    return a, sl


@pytest.mark.parametrize("kw,status", [
    (dict(kv_stride=3), A.ATTN_ERR_SHAPE),           # L_b = 4 > stride
    (dict(kv_stride=-1), A.ATTN_ERR_SHAPE),
    (dict(tile_keys=-5), A.ATTN_ERR_SHAPE),
    (dict(num_ctas=-1), A.ATTN_ERR_SHAPE),
    (dict(scale=float("inf")), A.ATTN_ERR_SHAPE),
    (dict(scale=float("nan")), A.ATTN_ERR_SHAPE),
    (dict(workspace=FAKE + 4, workspace_bytes=1 << 20), A.ATTN_ERR_ALIGN),
    # 2 x 2 segments of 16 LeanTiles over 6 CTAs: heads are split, so slots are needed
    (dict(seqlens=(4096, 4096), workspace=FAKE, workspace_bytes=16, num_ctas=6), A.ATTN_ERR_WORKSPACE),
    (dict(seqlens=(4096, 4096), workspace=FAKE, workspace_bytes=32768, num_ctas=6), A.ATTN_ERR_WORKSPACE),
    (dict(num_ctas=4097), A.ATTN_ERR_UNSUPPORTED),
    (dict(schedule=3), A.ATTN_ERR_SHAPE),
    (dict(schedule=-1), A.ATTN_ERR_SHAPE),
    (dict(num_splits=-2), A.ATTN_ERR_SHAPE),
    (dict(schedule=2, num_ctas=16), A.ATTN_ERR_SHAPE),       # the fixed split sets P itself
    (dict(schedule=2, num_splits=2000), A.ATTN_ERR_UNSUPPORTED),  # B*KH*splits > ATTN_MAX_CTAS
    (dict(kv_dtype=2), A.ATTN_ERR_SHAPE),
    (dict(kv_dtype=1, k_scale=float("inf")), A.ATTN_ERR_SHAPE),
    (dict(kv_dtype=1, v_scale=float("nan")), A.ATTN_ERR_SHAPE),
    (dict(kv_dtype=0, k_scale=0.5), A.ATTN_ERR_SHAPE),           # scales belong to FP8 caches
    (dict(block_table=FAKE, block_size=24, max_blocks_per_seq=4, num_blocks=8), A.ATTN_ERR_UNSUPPORTED),
    (dict(block_table=FAKE, block_size=8, max_blocks_per_seq=4, num_blocks=8), A.ATTN_ERR_UNSUPPORTED),
    (dict(block_table=FAKE, block_size=16, max_blocks_per_seq=0, num_blocks=8), A.ATTN_ERR_SHAPE),
    (dict(block_table=FAKE, block_size=16, max_blocks_per_seq=4, num_blocks=0), A.ATTN_ERR_SHAPE),
    (dict(block_table=FAKE, block_size=16, max_blocks_per_seq=4, num_blocks=8, kv_stride=64), A.ATTN_ERR_SHAPE),
    (dict(block_table=FAKE + 2, block_size=16, max_blocks_per_seq=4, num_blocks=8), A.ATTN_ERR_ALIGN),
    (dict(block_size=16), A.ATTN_ERR_SHAPE),                      # block geometry without a table
    (dict(q_len=-1), A.ATTN_ERR_SHAPE),
    (dict(out_lse=FAKE + 2), A.ATTN_ERR_ALIGN),
    (dict(q_len=17), A.ATTN_ERR_UNSUPPORTED),                     # G * q_len = 68 > 64 query columns
    (dict(Hsz=256, q_len=9), A.ATTN_ERR_UNSUPPORTED),             # 36 columns x 256 > 8192
    (dict(Hq=2, KH=2, q_len=5), A.ATTN_ERR_SHAPE),                 # 4 cached keys < 5 query tokens
    (dict(seqlens=(4, 70), block_table=FAKE, block_size=16, max_blocks_per_seq=4, num_blocks=8),
     A.ATTN_ERR_SHAPE),                                           # 70 keys > 4 blocks x 16
    (dict(seqlens_on_device=1), A.ATTN_ERR_SHAPE),                # device seqlens need kv_stride
    (dict(seqlens_on_device=1, kv_stride=1 << 30, tile_keys=1), A.ATTN_ERR_UNSUPPORTED),  # > 2^31 tiles
])
def test_decode_ex_rejects_bad_arguments(kw, status):
    a, _sl = ex_args(**kw)
    assert A.lib().attn_decode_ex(ctypes.byref(a), None) == status


def test_decode_ex_device_seqlens_alignment():
    a, _sl = ex_args(seqlens_on_device=1, kv_stride=64)
    a.seqlens = FAKE + 2  # a device address, never read on the host
    assert A.lib().attn_decode_ex(ctypes.byref(a), None) == A.ATTN_ERR_ALIGN


def test_decode_ex_null_args():
    assert A.lib().attn_decode_ex(None, None) == A.ATTN_ERR_NULL


@pytest.mark.parametrize("args,status", [
    ((None, FAKE, FAKE, 1, 16, 8, 2, 128, FAKE), A.ATTN_ERR_NULL),
    ((FAKE, FAKE, FAKE, 0, 16, 8, 2, 128, FAKE), A.ATTN_ERR_SHAPE),
    ((FAKE, FAKE, FAKE, 1, -1, 8, 2, 128, FAKE), A.ATTN_ERR_SHAPE),
    ((FAKE, FAKE, FAKE, 1, 16, 8, 3, 128, FAKE), A.ATTN_ERR_SHAPE),
    ((FAKE, FAKE, FAKE, 1, 16, 8, 2, 512, FAKE), A.ATTN_ERR_UNSUPPORTED),
    ((FAKE, FAKE, FAKE, 1, 16, 8, 2, 96, FAKE), A.ATTN_ERR_UNSUPPORTED),
    ((FAKE + 2, FAKE, FAKE, 1, 16, 8, 2, 128, FAKE), A.ATTN_ERR_ALIGN),
    ((FAKE, FAKE, FAKE, 1, 0, 8, 2, 128, FAKE), A.ATTN_OK),  # empty prompt: nothing to do, no launch
])
def test_prefill_argument_checks(args, status):
    assert A.lib().attn_prefill_causal(*args, None) == status


def test_merge_shards_argument_checks():
    lib = A.lib()
    assert lib.attn_merge_shards(None, FAKE, 2, 8, 128, FAKE, None, None) == A.ATTN_ERR_NULL
    assert lib.attn_merge_shards(FAKE, FAKE, 0, 8, 128, FAKE, None, None) == A.ATTN_ERR_SHAPE
    assert lib.attn_merge_shards(FAKE, FAKE, 2, -1, 128, FAKE, None, None) == A.ATTN_ERR_SHAPE
    assert lib.attn_merge_shards(FAKE, FAKE, 2, 8, 6, FAKE, None, None) == A.ATTN_ERR_SHAPE
    assert lib.attn_merge_shards(FAKE + 4, FAKE, 2, 8, 128, FAKE, None, None) == A.ATTN_ERR_ALIGN
    assert lib.attn_merge_shards(FAKE, FAKE + 2, 2, 8, 128, FAKE, None, None) == A.ATTN_ERR_ALIGN


def test_copy_probe_argument_checks():
    lib = A.lib()
    assert lib.attn_hbm_copy_probe(None, FAKE, 64, None) == A.ATTN_ERR_NULL
    assert lib.attn_hbm_copy_probe(FAKE, FAKE, 65, None) == A.ATTN_ERR_SHAPE
    assert lib.attn_hbm_copy_probe(FAKE + 8, FAKE, 64, None) == A.ATTN_ERR_ALIGN


def test_plan_argument_checks():
    with pytest.raises(A.AttnError) as e:
        A.attn_decode_plan([4, 4], 2, 0, 4)
    assert e.value.status == A.ATTN_ERR_SHAPE
    with pytest.raises(A.AttnError) as e:
        A.attn_decode_plan([4, -4], 2, 16, 4)
    assert e.value.status == A.ATTN_ERR_SHAPE


def test_workspace_bytes_formula():
    # the counter region, then 2 slots per CTA, each G*Hsz (O) + 2G (m, l) floats rounded up to 4
    assert A.ATTN_DECODE_COUNTER_BYTES == 2 * A.ATTN_MAX_CTAS * 4  # one arrival counter per partial slot
    C = A.ATTN_DECODE_COUNTER_BYTES + A.ATTN_DECODE_PLAN_BYTES
    assert A.attn_decode_workspace_bytes(16, 32, 8, 128, 100) == C + 2 * 100 * ((4 * 128 + 8 + 3) & ~3) * 4
    assert A.attn_decode_workspace_bytes(1, 8, 1, 64, 7) == C + 2 * 7 * ((8 * 64 + 16 + 3) & ~3) * 4
    assert A.attn_decode_workspace_bytes(1, 8, 3, 64, 7) == 0  # Hq % KH != 0
    assert A.attn_decode_workspace_bytes(1, 8, 1, 64, A.ATTN_MAX_CTAS + 1) == 0
    # multi-token: slots hold G * q_len states
    assert A.attn_decode_multi_workspace_bytes(16, 32, 8, 128, 4, 100) == C + 2 * 100 * ((16 * 128 + 32 + 3) & ~3) * 4
    assert A.attn_decode_multi_workspace_bytes(16, 32, 8, 128, 5, 100) == C + 2 * 100 * ((20 * 128 + 40 + 3) & ~3) * 4
    assert A.attn_decode_multi_workspace_bytes(16, 32, 8, 128, 17, 100) == 0  # 68 columns
    assert A.attn_decode_multi_workspace_bytes(16, 32, 8, 256, 9, 100) == 0   # 36 columns x 256
    assert A.attn_decode_workspace_bytes(1, 64, 1, 128, 10) == C + 2 * 10 * ((64 * 128 + 128 + 3) & ~3) * 4


def test_python_binding_validates_cache_capacity():
    import torch
    # CPU tensors are rejected before anything reaches the library
    with pytest.raises(TypeError):
        A.attn_decode(torch.zeros(1, 8, 128, dtype=torch.bfloat16), torch.zeros(1, 2, 4, 128, dtype=torch.bfloat16),
                      torch.zeros(1, 2, 4, 128, dtype=torch.bfloat16), [4])


def _no_gpu() -> bool:
    import torch
    return torch.cuda.device_count() == 0  # counts devices without initialising one


@pytest.mark.skipif(not _no_gpu(), reason="needs a host without a GPU: there every HIP runtime call fails")
def test_hip_failure_after_validation_is_reported():
    # Valid arguments pass validation; the first HIP runtime call after it (the device query for
    # the default workgroup count) fails on a host without a GPU, and the failure comes back as
    # ATTN_ERR_HIP with the call and the HIP error text, not as a crash or a silent success.
    lib = A.lib()
    assert call_decode() == A.ATTN_ERR_HIP
    msg = lib.attn_last_error().decode()
    assert "hipGetDevice" in msg and "(" in msg, msg
    # an explicit stream-K count needs no device query; the failure then comes from the launch path
    a, _sl = ex_args(num_ctas=1, schedule=A.ATTN_SCHEDULE_STREAM_K)
    assert lib.attn_decode_ex(ctypes.byref(a), None) == A.ATTN_ERR_HIP
    assert lib.attn_last_error().decode() != ""
    cus, lds = ctypes.c_int(), ctypes.c_int()
    assert lib.attn_device_info(ctypes.byref(cus), ctypes.byref(lds)) == A.ATTN_ERR_HIP
    # the size query reports failure as 0 bytes
    assert A.attn_decode_workspace_bytes(2, 8, 2, 128, 0) == 0


def test_workspace_check_uses_the_clamped_cta_count():
    # 2 requests x 2 kv heads x 1 tile = 4 tiles: an explicit num_ctas of 64 is clamped to 4,
    # no head is split, so no workspace is needed and a tiny caller workspace is accepted by
    # validation (on a GPU-less host the call then fails at its first HIP call, not with
    # ATTN_ERR_WORKSPACE)
    a, _sl = ex_args(num_ctas=64, schedule=A.ATTN_SCHEDULE_STREAM_K, workspace=FAKE, workspace_bytes=16)
    st = A.lib().attn_decode_ex(ctypes.byref(a), None) if _no_gpu() else None
    if st is not None:
        assert st == A.ATTN_ERR_HIP
    # 2 requests of 4096 keys over 64 CTAs at T=256: heads are split, the workspace is checked
    # against the final count before any HIP call
    a, _sl = ex_args(seqlens=(4096, 4096), num_ctas=64, tile_keys=256, schedule=A.ATTN_SCHEDULE_STREAM_K,
                     workspace=FAKE, workspace_bytes=32768 + 8192)
    assert A.lib().attn_decode_ex(ctypes.byref(a), None) == A.ATTN_ERR_WORKSPACE


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # no fallback path: without the built HIP library every entry point stops at lib()
    monkeypatch.setattr(A, "_lib", None)
    monkeypatch.setattr(A, "LIB_PATH", str(tmp_path / "libattn_gqa.so"))
    with pytest.raises(RuntimeError, match="is missing"):
        A.lib()
