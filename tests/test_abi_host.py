"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch.
(Addresses below are fake integers; a rejected call never dereferences them.)"""
import ctypes
import os
import re

import pytest

import tiled_online_softmax_fwd_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULL, SHAPE, HEAD, DTYPE, ALIGN, TILE, SCALE, ALIAS = 0, 1, 2, 3, 4, 5, 6, 7, 8
WORKSPACE = 10


def declared_functions():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(attn_\w+)\s*\(", src, flags=re.M))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert names == set(A.EXPORTS), names ^ set(A.EXPORTS)
    lib = A.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert A.version() == 100
    assert A.lib().attn_status_string(0) == b"ok"
    assert A.lib().attn_status_string(9) == b"HIP runtime error"
    assert A.lib().attn_status_string(123) == b"unknown status"


def test_default_tiles():
    assert A.default_tiles(A.BF16, 128, True) == (256, 64)
    assert A.default_tiles(A.F16, 64, True) == (128, 128)
    assert A.default_tiles(A.F32, 64, False) == (128, 64)
    with pytest.raises(A.AttnError):
        A.default_tiles(A.BF16, 96)
    with pytest.raises(A.AttnError):
        A.default_tiles(9, 64)


BASE = dict(q=0x10000, k=0x20000, v=0x30000, o=0x40000, lse=0x50000)


def chk(B=1, H=2, N=8, d=64, scale=0.125, causal=0, dtype=A.BF16, br=0, bc=0, kv_order=0, ref_slack=0, **ptrs):
    p = dict(BASE)
    p.update(ptrs)
    return A.check_args(p["q"], p["k"], p["v"], p["o"], p["lse"], B, H, N, d, scale, causal, None, dtype,
                        br, bc, kv_order, ref_slack)


def test_valid_arguments_pass():
    assert chk() == OK
    assert chk(dtype=A.F32) == OK and chk(dtype=A.F16_OUT_F32) == OK and chk(d=128) == OK
    assert chk(lse=None) == OK
    for dtype in (A.F32, A.F16, A.BF16, A.F16_OUT_F32, A.BF16_OUT_F32):
        for d in (64, 128):
            for br in (16, 32, 64, 128):
                for bc in (16, 32, 64, 128):
                    for order in (0, 1):
                        assert chk(dtype=dtype, d=d, br=br, bc=bc, kv_order=order) == OK
    for bc in (32, 64, 128):
        assert chk(dtype=A.BF16, d=128, br=256, bc=bc) == OK
    assert chk(dtype=A.F16, d=64, br=256, bc=64) == OK
    # bc alone: the default br falls back to 128 where no 256-row tile exists
    for dtype in (A.F32, A.BF16):
        for d in (64, 128):
            for bc in (16, 32, 64, 128):
                assert chk(dtype=dtype, d=d, bc=bc) == OK


def test_rejections():
    assert chk(q=None) == NULL and chk(o=None) == NULL
    assert chk(B=-1) == SHAPE and chk(N=-5) == SHAPE
    assert chk(B=1 << 16, H=1 << 10, N=1 << 6) == SHAPE
    assert chk(d=96) == HEAD and chk(d=0) == HEAD
    assert chk(dtype=5) == DTYPE and chk(dtype=-1) == DTYPE
    assert chk(q=0x10008) == ALIGN and chk(lse=0x50002) == ALIGN
    assert chk(br=48) == TILE and chk(bc=256) == TILE and chk(kv_order=2) == TILE
    assert chk(ref_slack=-1) == TILE and chk(ref_slack=16) == TILE
    assert chk(ref_slack=8) == OK and chk(ref_slack=15) == OK
    assert chk(br=256, bc=128) == TILE and chk(br=256, dtype=A.F32) == TILE      # not compiled
    for bad in (float("inf"), float("-inf"), float("nan")):
        assert chk(scale=bad) == SCALE
    for fine in (0.0, -0.0, -0.125, 1e-30, -3.0):     # every finite scale is accepted
        assert chk(scale=fine) == OK
    assert chk(o=0x10000 + 16) == ALIAS                     # o inside q
    assert chk(lse=0x40000 + 64) == ALIAS                   # lse inside o
    assert A.lib().attn_last_error() != b""


def test_zero_sizes_need_no_pointers():
    assert chk(B=0, q=None, k=None, v=None, o=None) == OK
    assert chk(N=0, q=None, k=None, v=None, o=None) == OK
    assert chk(N=0, d=96) == HEAD         # shape rules still apply


def test_no_cpu_fallback_exists():
    """The binding has no code path that computes attention itself."""
    src = open(os.path.join(ROOT, "tiled_online_softmax_fwd_amd", "__init__.py")).read()
    for banned in (r"softmax\(", r"matmul", r"\boracle\b", r"einsum", r"import numpy", r"\bexp\(", r"\bbmm\("):
        assert not re.search(banned, src), banned


def test_decode_argument_checks():
    L = A.lib()
    q, k, v, o = (ctypes.c_void_p(x) for x in (0x10000, 0x20000, 0x30000, 0x40000))
    ws = ctypes.c_void_p(0x100000)
    need = L.attn_decode_workspace_bytes(1, 2, 3, 100, 64, 0)
    assert need > 0 and L.attn_decode_workspace_bytes(1, 2, 3, 100, 96, 0) == 0

    def dec(q=q, k=k, v=v, o=o, lse=None, B=1, H=2, Nq=3, Nk=100, d=64, scale=0.1, dtype=A.BF16, ws=ws,
            nws=None, splits=0):
        return L.attn_decode_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, scale, 0, None, dtype, None, ws,
                                 need if nws is None else nws, splits)
    # rejected before anything is launched (no GPU touched)
    assert dec(dtype=A.F32) == DTYPE
    assert dec(d=96) == HEAD
    assert dec(scale=float("inf")) == SCALE and dec(scale=float("nan")) == SCALE
    assert dec(Nq=-1) == SHAPE
    assert dec(splits=1025) == TILE
    assert dec(q=None) == NULL
    assert dec(k=None) == NULL
    assert dec(q=ctypes.c_void_p(0x10008)) == ALIGN
    assert dec(ws=None) == WORKSPACE
    assert dec(nws=need - 4) == WORKSPACE
    assert dec(ws=ctypes.c_void_p(0x20000 + 64)) == ALIAS    # inside k
    assert dec(o=ctypes.c_void_p(0x10000)) == ALIAS          # o == q
    assert dec(Nq=0, q=None, o=None) == OK                                          # empty: no-op


def test_sparse_argument_checks():
    """attn_fwd_sparse rejects, before any launch: fp32 inputs, a block that is
    not a positive multiple of 32, kv_order 1, a tile without a block-sparse
    instance, a NULL block_mask, and o overlapping the flags."""
    L = A.lib()
    base = 1 << 20
    q, k, v, o, lse, bm = base, base + (1 << 24), base + (2 << 24), base + (3 << 24), base + (4 << 24), base + (5 << 24)

    def call(dtype=A.BF16, block=64, opts=None, bmask=bm, N=256, d=128, oo=o):
        return L.attn_fwd_sparse(q, k, v, oo, lse, 1, 2, N, d, 0.1, 0, None, bmask, block, dtype, None,
                                 ctypes.byref(opts) if opts is not None else None)

    assert call(dtype=A.F32) == DTYPE
    for blk in (0, -64, 16, 48, 100):
        assert call(block=blk) == SHAPE, blk
    assert call(opts=A.make_opts(kv_order=1)) == TILE
    for br, bc in ((32, 32), (64, 128), (256, 128), (16, 64), (128, 32)):
        assert call(opts=A.make_opts(br, bc)) == TILE, (br, bc)
    assert call(bmask=None) == NULL
    assert call(bmask=o + 64) == ALIAS
    assert call(d=96) == HEAD
    assert call(N=0, bmask=None) == OK          # empty problem: no-op before any pointer check


def test_decode_default_chunking():
    """The library's default key chunking, read back through the workspace size
    (B*H*splits*Nq*(d+1) floats): about 1024 one-wave workgroups, fewer (down to
    about 512) where that keeps chunks at 1024 keys or more, never chunks under
    256 keys; an explicit count is kept, in whole 32-key tiles."""
    L = A.lib()
    L.attn_decode_workspace_bytes.restype = ctypes.c_size_t

    def chunks(B, H, Nq, Nk, d, splits=0):
        n = L.attn_decode_workspace_bytes(B, H, Nq, Nk, d, splits)
        per = B * H * Nq * (d + 1) * 4
        assert n % per == 0
        return n // per
    assert chunks(8, 32, 1, 8192, 128) == 4        # 1024 workgroups of 2048 keys
    assert chunks(8, 32, 1, 8192, 64) == 4
    assert chunks(8, 32, 16, 8192, 128) == 4
    assert chunks(1, 32, 1, 65536, 128) == 32      # 1024 workgroups of 2048 keys
    assert chunks(2, 8, 1, 32768, 128) == 32       # 512 workgroups of 1024 keys
    assert chunks(1, 8, 1, 16384, 128) == 64       # 512 workgroups of 256 keys
    assert chunks(1, 1, 1, 100, 64) == 1           # a short cache stays whole
    assert chunks(8, 32, 1, 1001, 128) == 2
    assert chunks(8, 32, 1, 8192, 128, 3) == 3     # an explicit count is taken as given
    assert chunks(1, 2, 3, 100, 64, 3) == 2        # ... in whole 32-key tiles: 4 tiles give 2 chunks of 2
