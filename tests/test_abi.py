"""CPU tests of the C ABI: the library loads, exports every function that
include/s2attn.h declares, and rejects bad arguments before touching the GPU.

No call here reaches a kernel launch: every call either fails argument
validation or is an empty (B == 0 or N == 0) call, both of which return
before any HIP runtime call.
"""
import ctypes
import os
import re

import pytest

from grouped_shifted_attention_amd import _lib
from grouped_shifted_attention_amd.build import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "s2attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB_PATH), reason="libs2attn.so not built")

EINVAL, EUNSUP = _lib.S2ATTN_EINVAL, _lib.S2ATTN_EUNSUPPORTED


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(s2attn_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("s2attn_fwd", "s2attn_bwd", "s2attn_fwd_rope", "s2attn_bwd_rope", "s2attn_strerror"):
        assert n in names


def test_library_exports_every_declared_symbol():
    handle = ctypes.CDLL(LIB_PATH)
    for name in declared_functions():
        assert hasattr(handle, name), name
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def test_status_codes_match_header():
    text = open(HEADER).read()
    for name, val in (("S2ATTN_OK", 0), ("S2ATTN_EINVAL", -1), ("S2ATTN_EUNSUPPORTED", -2), ("S2ATTN_EHIP", -3)):
        m = re.search(rf"#define {name} \(?(-?\d+)\)?", text)
        assert m and int(m.group(1)) == val


def test_strerror():
    L = _lib.lib()
    assert L.s2attn_strerror(0) == b"success"
    assert L.s2attn_strerror(-1) == b"invalid argument"
    assert L.s2attn_strerror(-2) == b"unsupported configuration"
    assert L.s2attn_strerror(-3) == b"HIP runtime error"
    assert L.s2attn_strerror(7) == b"unknown status"


FAKE = 0x10000  # 16-byte-aligned non-null address; never dereferenced here


def fwd(B=1, N=256, H=4, Hkv=4, D=64, G=64, shift=32, ptrs=None):
    q = k = v = out = lse = FAKE
    if ptrs:
        q, k, v, out, lse = ptrs
    return _lib.lib().s2attn_fwd(q, k, v, out, lse, B, N, H, Hkv, D, G, shift, None)


def detail():
    return _lib.lib().s2attn_last_error().decode()


@pytest.mark.parametrize("kw,msg", [
    (dict(N=250), "multiple of G"),
    (dict(G=0), "G must be"),
    (dict(shift=64), "shift"),
    (dict(shift=-1), "shift"),
    (dict(H=3, Hkv=3), "even"),
    (dict(H=4, Hkv=1), "even"),
    (dict(H=4, Hkv=3, shift=0), "multiple of Hkv"),
    (dict(B=-1), ">= 0"),
    (dict(H=0), ">= 1"),
    (dict(D=0), "D must be"),
    (dict(H=262144, Hkv=262144, D=128, shift=0), "H * D too large"),
])
def test_fwd_rejects_bad_shapes(kw, msg):
    assert fwd(**kw) == EINVAL
    assert msg in detail()


@pytest.mark.parametrize("D", [32, 96, 256])
def test_fwd_unsupported_head_dim(D):
    assert fwd(D=D) == EUNSUP


def test_fwd_rejects_null_and_misaligned_pointers():
    assert fwd(ptrs=(0, FAKE, FAKE, FAKE, FAKE)) == EINVAL and "q is NULL" in detail()
    assert fwd(ptrs=(FAKE + 2, FAKE, FAKE, FAKE, FAKE)) == EINVAL and "aligned" in detail()


def test_fwd_rejects_overlapping_output():
    q_bytes = 1 * 256 * 4 * 64 * 2
    base = 0x1000000
    # out overlaps q
    assert fwd(ptrs=(base, base + 4 * q_bytes, base + 8 * q_bytes, base + q_bytes - 256, 0)) == EINVAL
    assert "overlaps" in detail()
    # lse overlaps out
    assert fwd(ptrs=(base, base + 4 * q_bytes, base + 8 * q_bytes, base + 12 * q_bytes,
                     base + 12 * q_bytes + 16)) == EINVAL


def test_empty_calls_succeed_without_pointers():
    L = _lib.lib()
    assert fwd(B=0, ptrs=(0, 0, 0, 0, 0)) == 0
    assert fwd(N=0, ptrs=(0, 0, 0, 0, 0)) == 0
    assert L.s2attn_bwd(None, None, None, None, None, None, None, None, None,
                        0, 256, 4, 4, 64, 64, 32, None, 0, None) == 0
    assert L.s2attn_fwd_rope(None, None, None, None, None, 1, 0, 4, 4, 64, 64, 32,
                             10000.0, 8.0, None, 0, None) == 0


def test_bwd_checks_workspace():
    L = _lib.lib()
    B, N, H, Hkv, D, G, sh = 1, 256, 4, 4, 64, 64, 32
    need = L.s2attn_bwd_workspace_size(B, N, H, Hkv, D)
    # -Delta and -lse*log2(e) (fp32), each 256-byte aligned; nothing else
    assert need == 2 * ((B * H * N * 4 + 255) // 256 * 256)
    step = 1 << 24
    p = [0x10000000 + i * step for i in range(10)]
    st = L.s2attn_bwd(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], B, N, H, Hkv, D, G, sh,
                      p[9], need - 1, None)
    assert st == EINVAL and "workspace too small" in detail()
    st = L.s2attn_bwd(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], B, N, H, Hkv, D, G, sh,
                      p[9] + 16, need, None)
    assert st == EINVAL and "256-byte" in detail()


def test_rope_arguments_are_checked():
    L = _lib.lib()
    for base, s in ((0.0, 8.0), (10000.0, 0.0), (float("inf"), 8.0), (10000.0, float("nan"))):
        st = L.s2attn_fwd_rope(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 256, 4, 4, 64, 64, 32, base, s, FAKE, 1 << 20, None)
        assert st == EINVAL


def test_workspace_sizes():
    L = _lib.lib()
    B, N, H, Hkv, D = 1, 32768, 64, 8, 128
    fr = L.s2attn_fwd_rope_workspace_size(B, N, H, Hkv, D)
    br = L.s2attn_bwd_rope_workspace_size(B, N, H, Hkv, D)
    b = L.s2attn_bwd_workspace_size(B, N, H, Hkv, D)
    assert fr >= B * N * Hkv * D * 2
    assert b == 2 * B * H * N * 4  # the two row statistics only
    assert br >= b + B * N * H * D * 2 + B * N * Hkv * D * 2  # plus the rotated q and k
    assert L.s2attn_bwd_workspace_size(0, N, H, Hkv, D) == 0


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libs2attn.so")
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()


def test_general_entry_points_check_the_head_pattern():
    L = _lib.lib()
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, 1, 256, 4, 4, 64, 64, 32)
    assert L.s2attn_fwd_ex(*args, 2, 0.0, 1.0, None, 0, None) == EINVAL
    assert "head_pattern" in detail()
    # Alternate heads need no even head count; an empty call validates only.
    assert L.s2attn_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 0, 3, 3, 64, 64, 32, 1, 0.0, 1.0, None, 0, None) == 0
    assert L.s2attn_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 0, 3, 3, 64, 64, 32, 0, 0.0, 1.0, None, 0, None) == EINVAL
    assert L.s2attn_fwd_ex(*args, 1, -1.0, 1.0, FAKE, 1 << 20, None) == EINVAL  # bad RoPE base


# ------------------------------------------------- LoRA q/k/v projections

def _lora(M=512, d_in=128, wq=256, wkv=128, r=16, scale=1.0, ws=True, ws_bytes=None, **ptrs):
    L = _lib.lib()
    need = L.s2attn_lora_qkv_workspace_size(M, r)
    p = {n: FAKE + i * (1 << 28) for i, n in enumerate(
        ("x", "wq", "wk", "wv", "aq", "ak", "av", "bq", "bk", "bv", "q", "k", "v", "ws"))}
    p.update(ptrs)
    return L.s2attn_lora_qkv_fwd(p["x"], M, d_in, p["wq"], p["wk"], p["wv"], wq, wkv,
                                 p["aq"], p["ak"], p["av"], p["bq"], p["bk"], p["bv"], r, scale,
                                 p["q"], p["k"], p["v"], p["ws"] if ws else None,
                                 need if ws_bytes is None else ws_bytes, None)


def test_lora_workspace_size():
    L = _lib.lib()
    assert L.s2attn_lora_qkv_workspace_size(1000, 64) == 1000 * 3 * 64 * 2  # already a multiple of 256
    assert L.s2attn_lora_qkv_workspace_size(3, 8) == 256
    assert L.s2attn_lora_qkv_workspace_size(1000, 0) == 0
    assert L.s2attn_lora_qkv_workspace_size(0, 64) == 0


@pytest.mark.parametrize("kw", [
    dict(M=-1), dict(d_in=96), dict(d_in=0), dict(wq=100), dict(wkv=32), dict(r=12), dict(r=2048),
    dict(r=-8), dict(scale=float("nan")), dict(scale=float("inf")),
])
def test_lora_rejects_bad_shapes(kw):
    assert _lora(**kw) == EINVAL


def test_lora_rejects_bad_buffers():
    assert _lora(x=None) == EINVAL
    assert _lora(bq=None) == EINVAL
    assert _lora(q=FAKE + 8) == EINVAL                      # not 16-byte aligned
    assert _lora(ws=False) == EINVAL                         # r > 0 needs the workspace
    assert _lora(ws_bytes=100) == EINVAL
    assert _lora(q=FAKE) == EINVAL                          # output overlaps x
    assert _lora(k=FAKE + 10 * (1 << 28)) == EINVAL         # k overlaps q
    assert b"overlaps" in _lib.lib().s2attn_last_error()


def test_lora_empty_call_is_a_no_op():
    assert _lora(M=0) == _lib.S2ATTN_OK


def test_lora_without_adapter_needs_no_workspace():
    # r = 0 with NULL adapters and workspace passes validation; M = 0 keeps it
    # from launching.
    assert _lora(M=0, r=0, aq=None, ak=None, av=None, bq=None, bk=None, bv=None, ws=False) == _lib.S2ATTN_OK


def _lora_bwd(M=512, d_in=128, wq=256, wkv=128, r=16, scale=1.0, ws=True, ws_bytes=None, **ptrs):
    L = _lib.lib()
    need = L.s2attn_lora_qkv_bwd_workspace_size(M, d_in, wq, wkv, r)
    names = ("x", "wq", "wk", "wv", "aq", "ak", "av", "bq", "bk", "bv", "t", "dq", "dk", "dv",
             "dx", "daq", "dak", "dav", "dbq", "dbk", "dbv", "ws")
    p = {n: FAKE + i * (1 << 28) for i, n in enumerate(names)}
    p.update(ptrs)
    return L.s2attn_lora_qkv_bwd(p["x"], M, d_in, p["wq"], p["wk"], p["wv"], wq, wkv,
                                 p["aq"], p["ak"], p["av"], p["bq"], p["bk"], p["bv"], r, scale, p["t"],
                                 p["dq"], p["dk"], p["dv"], p["dx"], p["daq"], p["dak"], p["dav"],
                                 p["dbq"], p["dbk"], p["dbv"], p["ws"] if ws else None,
                                 need if ws_bytes is None else ws_bytes, None)


def test_lora_bwd_workspace_size():
    L = _lib.lib()
    # s x A-sized bf16 block, then 1 split x max(d_in, widths) x r fp32 partials.
    assert L.s2attn_lora_qkv_bwd_workspace_size(1000, 128, 256, 128, 16) == 96000 + 16384
    assert L.s2attn_lora_qkv_bwd_workspace_size(1000, 128, 256, 128, 0) == 0
    assert L.s2attn_lora_qkv_bwd_workspace_size(0, 128, 256, 128, 16) == 0


@pytest.mark.parametrize("kw", [
    dict(M=-1), dict(d_in=96), dict(wq=100), dict(wkv=0), dict(r=12), dict(r=2048), dict(scale=float("nan")),
])
def test_lora_bwd_rejects_bad_shapes(kw):
    assert _lora_bwd(**kw) == EINVAL


def test_lora_bwd_rejects_bad_buffers():
    assert _lora_bwd(t=None) == EINVAL                        # r > 0 needs the forward's x A
    assert _lora_bwd(dbv=None) == EINVAL
    assert _lora_bwd(ws=False) == EINVAL
    assert _lora_bwd(ws_bytes=1000) == EINVAL
    assert _lora_bwd(dx=FAKE + 11 * (1 << 28)) == EINVAL      # dx overlaps dq
    assert b"overlaps" in _lib.lib().s2attn_last_error()
    assert _lora_bwd(M=0) == _lib.S2ATTN_OK


def test_noalloc_rejects_shapes_beyond_its_scratch():
    # 5 * 4 * 2^20 rows of statistics need 160 MiB: rejected before any HIP call.
    L = _lib.lib()
    st = L.s2attn_bwd_noalloc(*([FAKE] * 9), 5, 1 << 20, 4, 4, 64, 1024, 512, None)
    assert st == EINVAL and "scratch" in detail()
    assert L.s2attn_bwd_noalloc(*([FAKE] * 9), 0, 256, 4, 4, 64, 64, 32, None) == 0  # empty call


def test_hip_error_status_path(monkeypatch):
    # A HIP failure after the argument checks maps to S2ATTN_EHIP with its
    # detail; the hook fails the call before any HIP call, so this runs
    # without a GPU.
    L = _lib.lib()
    monkeypatch.setenv("S2ATTN_TEST_HIP_ERROR", "719")
    B, N, H, Hkv, D, G, sh = 1, 256, 4, 4, 64, 64, 32
    st = L.s2attn_fwd(FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000, None, B, N, H, Hkv, D, G, sh, None)
    assert st == _lib.S2ATTN_EHIP and "HIP error 719" in detail()
    p = [0x10000000 + i * (1 << 24) for i in range(10)]
    need = L.s2attn_bwd_workspace_size(B, N, H, Hkv, D)
    st = L.s2attn_bwd(*p[:9], B, N, H, Hkv, D, G, sh, p[9], need, None)
    assert st == _lib.S2ATTN_EHIP and "injected" in detail()
    st = L.s2attn_bwd_noalloc(*p[:9], B, N, H, Hkv, D, G, sh, None)
    assert st == _lib.S2ATTN_EHIP
    with pytest.raises(_lib.S2AttnError, match="HIP error 719"):
        _lib.check(st)
    # invalid arguments are still reported as such, ahead of the hook
    st = L.s2attn_fwd(FAKE, FAKE, FAKE, FAKE, None, B, N, H, Hkv, D, 100, sh, None)
    assert st == EINVAL
    monkeypatch.setenv("S2ATTN_TEST_HIP_ERROR", "0")
    assert L.s2attn_fwd(FAKE, FAKE, FAKE, FAKE, None, 0, N, H, Hkv, D, G, sh, None) == 0
