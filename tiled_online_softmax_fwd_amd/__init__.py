"""Python binding of libattn.so, the gfx950 exact-attention forward library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of include/attn.h.  PyTorch is used for device memory
and streams; tensors are passed by data_ptr() on torch's current HIP stream.
There is no fallback: if the library is missing or the GPU is absent, calls
raise.
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

# attn_dtype
F32, F16, BF16, F16_OUT_F32, BF16_OUT_F32 = 0, 1, 2, 3, 4
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_HEAD_DIM",
          4: "ATTN_ERR_DTYPE", 5: "ATTN_ERR_ALIGN", 6: "ATTN_ERR_TILE", 7: "ATTN_ERR_SCALE",
          8: "ATTN_ERR_ALIAS", 9: "ATTN_ERR_HIP", 10: "ATTN_ERR_WORKSPACE"}
EXPORTS = ("attn_fwd", "attn_fwd_ex", "attn_fwd_sparse", "attn_check_args", "attn_default_tiles", "attn_naive_fwd",
           "attn_naive_workspace_bytes", "attn_decode_fwd", "attn_decode_workspace_bytes", "attn_decode_fwd_noalloc",
           "attn_bwd", "attn_bwd_workspace_bytes", "attn_probe_mfma",
           "attn_status_string", "attn_last_error", "attn_version")


class AttnError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class attn_opts(ctypes.Structure):
    _fields_ = [("br", ctypes.c_int), ("bc", ctypes.c_int), ("kv_order", ctypes.c_int),
                ("ref_slack", ctypes.c_int), ("generic_loop", ctypes.c_int), ("reserved", ctypes.c_int * 3)]


_lib = None


def lib():
    """Load libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not built; run __graft_entry__.build() or "
                               "python tiled_online_softmax_fwd_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        common = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i]
        L.attn_fwd.argtypes = common + [vp]
        L.attn_fwd_ex.argtypes = common + [vp, ctypes.POINTER(attn_opts)]
        L.attn_check_args.argtypes = common + [ctypes.POINTER(attn_opts)]
        L.attn_fwd_sparse.argtypes = common[:12] + [vp, i, i, vp, ctypes.POINTER(attn_opts)]
        L.attn_default_tiles.argtypes = [i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
        L.attn_naive_fwd.argtypes = common + [vp, vp, ctypes.c_size_t]
        L.attn_naive_workspace_bytes.argtypes = [i, i, i, i]
        L.attn_naive_workspace_bytes.restype = ctypes.c_size_t
        L.attn_decode_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, vp, vp, ctypes.c_size_t, i]
        L.attn_decode_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, i, vp, i]
        L.attn_decode_workspace_bytes.argtypes = [i, i, i, i, i, i]
        L.attn_decode_workspace_bytes.restype = ctypes.c_size_t
        L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp, vp, ctypes.c_size_t]
        L.attn_bwd_workspace_bytes.argtypes = [i, i, i]
        L.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.attn_probe_mfma.argtypes = [i, vp, ctypes.POINTER(ctypes.c_double)]
        L.attn_probe_mfma.restype = ctypes.c_int
        L.attn_status_string.argtypes = [i]
        L.attn_status_string.restype = ctypes.c_char_p
        L.attn_last_error.argtypes = []
        L.attn_last_error.restype = ctypes.c_char_p
        L.attn_version.argtypes = []
        for fn in (L.attn_fwd, L.attn_fwd_ex, L.attn_fwd_sparse, L.attn_check_args, L.attn_default_tiles,
                   L.attn_naive_fwd, L.attn_decode_fwd, L.attn_decode_fwd_noalloc, L.attn_bwd, L.attn_version):
            fn.restype = ctypes.c_int
        _lib = L
    return _lib


def _raise(st):
    if st != 0:
        raise AttnError(st, lib().attn_last_error().decode())


def make_opts(br=0, bc=0, kv_order=0, ref_slack=0, generic_loop=0):
    o = attn_opts()
    o.br, o.bc, o.kv_order, o.ref_slack = int(br or 0), int(bc or 0), int(kv_order or 0), int(ref_slack or 0)
    o.generic_loop = int(bool(generic_loop))
    return o


def default_tiles(dtype, d, causal=False):
    br, bc = ctypes.c_int(), ctypes.c_int()
    _raise(lib().attn_default_tiles(int(dtype), int(d), int(bool(causal)), ctypes.byref(br), ctypes.byref(bc)))
    return br.value, bc.value


def _torch():
    import torch
    return torch


def _dtype_code(t, out_f32):
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float16:
        return F16_OUT_F32 if out_f32 else F16
    if t.dtype == torch.bfloat16:
        return BF16_OUT_F32 if out_f32 else BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, name, device, dtypes, shape):
    """Raise ValueError unless t lives on `device`, is contiguous, has one of
    `dtypes` and exactly `shape`: the library writes through the raw pointer."""
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(x) for x in dtypes)}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}, got {list(t.shape)}")
    return t


def _mask_arg(mask, name, device, shape):
    """uint8/bool [B, N] padding mask on `device` (made contiguous), or None."""
    if mask is None:
        return None
    torch = _torch()
    if mask.device != device:
        raise ValueError(f"{name} must be on {device}, got {mask.device}")
    return _check(mask.contiguous(), name, device, (torch.uint8, torch.bool), shape)


def _workspace(ws, need, device):
    """Caller workspace on `device` (any dtype, contiguous) of at least `need`
    bytes, or a new one; returns (tensor, size in bytes)."""
    torch = _torch()
    if ws is None:
        ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=device)
    if ws.device != device or not ws.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes, {need} needed")
    return ws, nbytes


def _prep(q, k, v, key_padding_mask, out, lse, out_f32, want_lse):
    torch = _torch()
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if not q.is_cuda:
        raise ValueError("q, k, v must be GPU tensors")
    dev = q.device
    B, H, N, d = q.shape
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _check(t, nm, dev, (q.dtype,), (B, H, N, d))
    code = _dtype_code(q, out_f32)
    odt = torch.float32 if (out_f32 or q.dtype == torch.float32) else q.dtype
    if out is None:
        out = torch.empty((B, H, N, d), dtype=odt, device=dev)
    _check(out, "out", dev, (odt,), (B, H, N, d))
    if lse is None and want_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if lse is not None:
        _check(lse, "lse", dev, (torch.float32,), (B, H, N))
    key_padding_mask = _mask_arg(key_padding_mask, "key_padding_mask", dev, (B, N))
    return B, H, N, d, code, out, lse, key_padding_mask


def fwd(q, k, v, *, scale=None, causal=False, key_padding_mask=None, out=None, lse=None,
        out_fp32=False, br=None, bc=None, kv_order=0, ref_slack=0, generic_loop=False, want_lse=True,
        stream=None):
    """Exact attention forward through attn_fwd_ex.  Returns (out, lse)."""
    torch = _torch()
    B, H, N, d, code, out, lse, mask = _prep(q, k, v, key_padding_mask, out, lse, out_fp32, want_lse)
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    s = stream if stream is not None else torch.cuda.current_stream(q.device).cuda_stream
    opts = make_opts(br, bc, kv_order, ref_slack, generic_loop)
    st = lib().attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, float(scale),
                           int(bool(causal)), _ptr(mask), code, ctypes.c_void_p(s), ctypes.byref(opts))
    _raise(st)
    return out, lse


def fwd_sparse(q, k, v, block_mask, *, block=64, scale=None, causal=False, key_padding_mask=None, out=None,
               lse=None, out_fp32=False, br=None, bc=None, ref_slack=0, want_lse=True, stream=None):
    """Block-sparse forward through attn_fwd_sparse: block_mask is a
    [B, H, ceil(N / block), ceil(N / block)] uint8/bool GPU tensor (non-zero =
    the block of pairs is attended).  Returns (out, lse)."""
    torch = _torch()
    B, H, N, d, code, out, lse, mask = _prep(q, k, v, key_padding_mask, out, lse, out_fp32, want_lse)
    nb = (N + int(block) - 1) // int(block) if block and int(block) > 0 else 0
    block_mask = _mask_arg(block_mask, "block_mask", q.device, (B, H, nb, nb))
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    s = stream if stream is not None else torch.cuda.current_stream(q.device).cuda_stream
    opts = make_opts(br, bc, 0, ref_slack)
    st = lib().attn_fwd_sparse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, float(scale),
                               int(bool(causal)), _ptr(mask), _ptr(block_mask), int(block), code,
                               ctypes.c_void_p(s), ctypes.byref(opts))
    _raise(st)
    return out, lse


def naive_fwd(q, k, v, *, scale=None, causal=False, key_padding_mask=None, out=None, lse=None,
              out_fp32=False, workspace=None, want_lse=True, stream=None):
    """Materialising baseline through attn_naive_fwd.  Returns (out, lse)."""
    torch = _torch()
    B, H, N, d, code, out, lse, mask = _prep(q, k, v, key_padding_mask, out, lse, out_fp32, want_lse)
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    need = lib().attn_naive_workspace_bytes(B, H, N, code)
    workspace, ws_bytes = _workspace(workspace, need, q.device)
    s = stream if stream is not None else torch.cuda.current_stream(q.device).cuda_stream
    st = lib().attn_naive_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, float(scale),
                              int(bool(causal)), _ptr(mask), code, ctypes.c_void_p(s),
                              _ptr(workspace), ws_bytes)
    _raise(st)
    return out, lse


def decode_fwd(q, k, v, *, scale=None, causal=False, key_padding_mask=None, out=None, lse=None,
               out_fp32=False, num_splits=0, workspace=None, want_lse=True, stream=None):
    """Query block q [B,H,Nq,d] against a key/value cache k, v [B,H,Nk,d] through
    attn_decode_fwd (16-bit inputs).  Returns (out, lse)."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("q [B,H,Nq,d] and k, v [B,H,Nk,d] do not match")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    if not q.is_cuda:
        raise ValueError("q, k, v must be GPU tensors")
    dev = q.device
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _check(q, "q", dev, (q.dtype,), (B, H, Nq, d))
    _check(k, "k", dev, (q.dtype,), (B, H, Nk, d))
    _check(v, "v", dev, (q.dtype,), (B, H, Nk, d))
    code = _dtype_code(q, out_fp32)
    odt = torch.float32 if (out_fp32 or q.dtype == torch.float32) else q.dtype
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=odt, device=dev)
    _check(out, "out", dev, (odt,), (B, H, Nq, d))
    if lse is None and want_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    if lse is not None:
        _check(lse, "lse", dev, (torch.float32,), (B, H, Nq))
    mask = _mask_arg(key_padding_mask, "key_padding_mask", dev, (B, Nk))
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    need = lib().attn_decode_workspace_bytes(B, H, Nq, Nk, d, int(num_splits))
    workspace, ws_bytes = _workspace(workspace, need, dev)
    s = stream if stream is not None else torch.cuda.current_stream(q.device).cuda_stream
    st = lib().attn_decode_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, d, float(scale),
                               int(bool(causal)), _ptr(mask), code, ctypes.c_void_p(s), _ptr(workspace),
                               ws_bytes, int(num_splits))
    _raise(st)
    return out, lse


def bwd(q, k, v, o, dout, lse, *, scale=None, causal=False, key_padding_mask=None, workspace=None, stream=None):
    """Gradient of fwd w.r.t. q, k, v through attn_bwd (bf16 or f16 inputs; o and
    lse as returned by fwd with the same arguments).  Returns fp32 (dq, dk, dv)."""
    torch = _torch()
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("the backward takes bf16 or fp16 tensors")
    if q.dim() != 4 or not q.is_cuda:
        raise ValueError("q must be a [B, H, N, d] GPU tensor")
    dev = q.device
    B, H, N, d = q.shape
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check(t, nm, dev, (q.dtype,), (B, H, N, d))
    _check(lse, "lse", dev, (torch.float32,), (B, H, N))
    code = BF16 if q.dtype == torch.bfloat16 else F16
    if scale is None:
        scale = 1.0 / (d ** 0.5)
    dq = torch.empty((B, H, N, d), dtype=torch.float32, device=q.device)
    dk = torch.empty_like(dq)
    dv = torch.empty_like(dq)
    mask = _mask_arg(key_padding_mask, "key_padding_mask", dev, (B, N))
    need = lib().attn_bwd_workspace_bytes(B, H, N)
    workspace, ws_bytes = _workspace(workspace, need, dev)
    s = stream if stream is not None else torch.cuda.current_stream(q.device).cuda_stream
    st = lib().attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                        B, H, N, d, float(scale), int(bool(causal)), _ptr(mask), code, ctypes.c_void_p(s),
                        _ptr(workspace), ws_bytes)
    _raise(st)
    return dq, dk, dv


def check_args(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, N, d, scale, causal, mask_ptr, dtype,
               br=0, bc=0, kv_order=0, ref_slack=0):
    """Host-only argument check with raw integer addresses; returns the status."""
    opts = make_opts(br, bc, kv_order, ref_slack)
    c = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib().attn_check_args(c(q_ptr), c(k_ptr), c(v_ptr), c(o_ptr), c(lse_ptr), B, H, N, d,
                                 float(scale), int(causal), c(mask_ptr), int(dtype), ctypes.byref(opts))


def probe_mfma(reps, stream=None):
    """Launch the matrix-core ceiling probe on the current stream; returns its
    floating-point operation count (time it with events on the same stream)."""
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    fl = ctypes.c_double()
    _raise(lib().attn_probe_mfma(int(reps), ctypes.c_void_p(s), ctypes.byref(fl)))
    return fl.value


def version():
    return lib().attn_version()
