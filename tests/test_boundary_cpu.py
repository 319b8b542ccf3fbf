"""The C-ABI library on the CPU: it loads, exports every symbol the public
header declares, and its host-side validation returns the documented codes.
No compute call is made (there is no GPU here)."""

import ctypes
import glob
import math
import os
import re
import subprocess

import pytest

import compressive_memory_transformers_segment_amd as ia
from compressive_memory_transformers_segment_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    syms = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        syms.update(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(infini_attn_\w+)\s*\(", text, re.M))
    return syms


def desc(**kw):
    base = dict(batch=1, n_q_heads=4, n_kv_heads=2, seq_len=300, d_k=64, d_v=64,
                dtype=ia.BF16, eps=1e-6, stream=None, device=0)
    base.update(kw)
    return ia.make_desc(**base)


def test_library_exports_every_header_symbol():
    lib = ia.load()
    syms = header_symbols()
    assert syms == set(_lib.EXPORTS), syms
    for s in syms:
        assert hasattr(lib, s), f"missing export {s}"
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], stdout=subprocess.PIPE,
                        text=True, check=True).stdout
    for s in syms:
        assert re.search(rf"\bT {s}$", nm, re.M), f"{s} not a defined text symbol"


def test_library_is_built_for_gfx950_only():
    # Offload bundle entry ids embedded by hipcc in the library we built.
    blob = open(_lib.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx\w+)", blob))
    assert targets == {b"gfx950"}, targets


@pytest.mark.parametrize("fields,seg,mode,expect", [
    (dict(), 64, ia.LINEAR, 0),
    (dict(), 64, ia.DELTA, 0),
    (dict(seq_len=0), 64, ia.LINEAR, 0),
    (dict(batch=0), 64, ia.LINEAR, 0),
    (dict(dtype=ia.F32, d_k=32, d_v=32), 1, ia.LINEAR, 0),
    (dict(d_k=128, d_v=128), 2048, ia.DELTA, 0),
    (dict(n_kv_heads=3), 64, ia.LINEAR, _lib.ERR_INVALID),
    (dict(n_q_heads=0), 64, ia.LINEAR, _lib.ERR_INVALID),
    (dict(batch=-1), 64, ia.LINEAR, _lib.ERR_INVALID),
    (dict(seq_len=-5), 64, ia.LINEAR, _lib.ERR_INVALID),
    (dict(), 0, ia.LINEAR, _lib.ERR_INVALID),
    (dict(), -3, ia.LINEAR, _lib.ERR_INVALID),
    (dict(), 64, 2, _lib.ERR_INVALID),
    (dict(dtype=7), 64, ia.LINEAR, _lib.ERR_INVALID),
    (dict(eps=0.0), 64, ia.LINEAR, _lib.ERR_INVALID),
    (dict(eps=-1e-6), 64, ia.LINEAR, _lib.ERR_INVALID),
    (dict(eps=float("nan")), 64, ia.LINEAR, _lib.ERR_INVALID),
    (dict(eps=float("inf")), 64, ia.LINEAR, _lib.ERR_INVALID),
    (dict(device=-1), 64, ia.LINEAR, _lib.ERR_INVALID),
    (dict(d_v=32), 64, ia.LINEAR, _lib.ERR_UNSUPPORTED),
    (dict(d_k=48, d_v=48), 64, ia.LINEAR, _lib.ERR_UNSUPPORTED),
    (dict(d_k=256, d_v=256), 64, ia.LINEAR, _lib.ERR_UNSUPPORTED),
    (dict(batch=2, n_q_heads=40000, n_kv_heads=1), 64, ia.LINEAR, _lib.ERR_UNSUPPORTED),
    (dict(seq_len=70000), 1, ia.LINEAR, _lib.ERR_UNSUPPORTED),
    (dict(seq_len=(1 << 30) + 1), 1 << 30, ia.LINEAR, _lib.ERR_UNSUPPORTED),
    (dict(), 2**31 - 1, ia.DELTA, 0),
])
def test_check_codes(fields, seg, mode, expect):
    assert ia.infini_attn_check(desc(**fields), seg, mode) == expect


def test_check_null_descriptor():
    lib = ia.load()
    assert lib.infini_attn_check(None, 64, 0) == _lib.ERR_INVALID


def test_workspace_size():
    d = desc(batch=2, n_q_heads=8, n_kv_heads=2, seq_len=700, d_k=64, d_v=64, dtype=ia.BF16)
    S = math.ceil(700 / 300)
    up = lambda x: (x + 255) // 256 * 256
    heads = 2 * 2
    # z snapshots, M^T snapshots (bf16), sigma(k) sums, G/H, V^T in 64-key tiles,
    # z snapshots as bf16 hi/lo rows
    assert ia.infini_attn_workspace_size(d, 300) == (
        up(heads * (S + 1) * 64 * 4) + up(heads * S * 64 * 64 * 2) + up(heads * S * 1 * 64 * 4)
        + up(heads * S * 2 * 64 * 64 * 4) + up(heads * S * math.ceil(300 / 64) * 64 * 64 * 2)
        + up(heads * S * 2 * 64 * 2))
    d32 = desc(dtype=ia.F32, d_k=32, d_v=32, seq_len=256, n_q_heads=2, n_kv_heads=2)
    assert ia.infini_attn_workspace_size(d32, 64) == up(2 * 5 * 32 * 4) + up(2 * 4 * 32 * 32 * 4)
    # 2048-row segments: sigma(k) sums in 4 row ranges of 512
    d4 = desc(batch=1, n_q_heads=32, n_kv_heads=8, seq_len=32768, d_k=128, d_v=128)
    assert ia.infini_attn_workspace_size(d4, 2048) == (
        up(8 * 17 * 128 * 4) + up(8 * 16 * 128 * 128 * 2) + up(8 * 16 * 4 * 128 * 4)
        + up(8 * 16 * 2 * 128 * 128 * 4) + up(8 * 16 * 32 * 128 * 64 * 2)
        + up(8 * 16 * 2 * 128 * 2))
    with pytest.raises(ia.InfiniAttnError):
        ia.infini_attn_workspace_size(desc(), 0)


def test_workspace_of_a_segment_longer_than_the_call():
    """seg_len >= L is one segment of L rows: the workspace is that of
    seg_len = L, also for seg_len near the int32 limit (no 32-bit overflow in
    the tile counts, no request sized by rows that do not exist)."""
    d = desc(batch=1, n_q_heads=32, n_kv_heads=8, seq_len=4096, d_k=128, d_v=128)
    ref = ia.infini_attn_workspace_size(d, 4096)
    for seg in (4097, 1 << 24, 2**31 - 1):
        assert ia.infini_attn_workspace_size(d, seg) == ref
    d200 = desc(seq_len=200)
    assert ia.infini_attn_workspace_size(d200, 2**31 - 1) == ia.infini_attn_workspace_size(d200, 200)


def test_create_without_device_reports_hip_error():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible")
    with pytest.raises(ia.InfiniAttnError) as ei:
        ia.infini_attn_create(desc())
    assert ei.value.status == _lib.ERR_HIP


def test_create_rejects_bad_descriptor_before_touching_a_device():
    with pytest.raises(ia.InfiniAttnError) as ei:
        ia.infini_attn_create(desc(n_kv_heads=3))
    assert ei.value.status == _lib.ERR_INVALID
    lib = ia.load()
    assert lib.infini_attn_create(None, ctypes.byref(desc())) == _lib.ERR_INVALID


def test_destroy_null_and_forward_null_handle():
    ia.infini_attn_destroy(None)
    lib = ia.load()
    assert lib.infini_attn_forward(None, None, None, None, None, None, None, 64, 0,
                                   None) == _lib.ERR_INVALID
    assert lib.infini_attn_backward(None, None, None, None, None, None, None, 64, 0, None, None,
                                    None, None, None, None, None, None, None) == _lib.ERR_INVALID


def test_strerror():
    assert ia.strerror(0) == "ok"
    assert "invalid" in ia.strerror(_lib.ERR_INVALID)
    assert "unsupported" in ia.strerror(_lib.ERR_UNSUPPORTED)
    assert "HIP" in ia.strerror(_lib.ERR_HIP)
    assert "memory" in ia.strerror(_lib.ERR_OOM)
    assert ia.strerror(12345) == "unknown status"


def test_product_path_has_no_oracle_or_cpu_fallback():
    pkg = os.path.join(ROOT, "compressive_memory_transformers_segment_amd")
    for f in glob.glob(os.path.join(pkg, "**", "*.py"), recursive=True):
        text = open(f).read()
        assert "import oracle" not in text and "from oracle" not in text, f
