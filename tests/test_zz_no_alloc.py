"""GPU: attn_decode_fwd_noalloc (the cache path without a caller workspace,
for callers that cannot allocate) against attn_decode_fwd through the C ABI,
on two calls in a row (the second smaller, so it reuses the array the first
one filled), plus the limit check.  The two entry points share the kernels
and the split rule, so the results must be bitwise equal."""
import ctypes

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    import torch
    assert torch.cuda.is_available()
    import tiled_online_softmax_fwd_amd as A
    A.lib()
    return A


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def both(A, B, H, Nq, Nk, d, dtype, causal, seed, mask=None):
    import torch
    kv = synth.make_qkv(B, H, Nk, d, dtype, seed)
    qq = synth.make_qkv(B, H, Nq, d, dtype, seed, variant=1)
    q, k, v = (synth.to_torch(x, dtype) for x in (qq.q, kv.k, kv.v))
    code = A.BF16 if dtype == "bf16" else A.F16
    scale = float(np.float32(d ** -0.5))
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    m = None if mask is None else torch.from_numpy(mask).cuda()
    outs = []
    for noalloc in (False, True):
        o = torch.full((B, H, Nq, d), float("nan"), dtype=q.dtype, device="cuda")
        lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
        if noalloc:
            st = A.lib().attn_decode_fwd_noalloc(ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), B, H, Nq, Nk, d, scale,
                                                 int(causal), ptr(m), code, stream, 0)
        else:
            need = A.lib().attn_decode_workspace_bytes(B, H, Nq, Nk, d, 0)
            ws = torch.empty((max(need, 16),), dtype=torch.uint8, device="cuda")
            st = A.lib().attn_decode_fwd(ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), B, H, Nq, Nk, d, scale,
                                         int(causal), ptr(m), code, stream, ptr(ws), ws.numel(), 0)
        assert st == 0, A.lib().attn_last_error()
        torch.cuda.synchronize()
        outs.append((o, lse))
    return outs


def test_noalloc_equals_workspace_entry_two_calls(A):
    import torch
    # the decode benchmark's shape, then a smaller call with a padding mask
    cases = [(8, 32, 1, 8192, 128, "bf16", False, None),
             (2, 3, 5, 1000, 64, "f16", True, np.array([[0] * 990 + [1] * 10, [1] * 1000], np.uint8))]
    for B, H, Nq, Nk, d, dtype, causal, mask in cases:
        print(f"[case] noalloc vs workspace B{B} H{H} Nq{Nq} Nk{Nk} d{d} {dtype} causal={causal}", flush=True)
        (o1, l1), (o2, l2) = both(A, B, H, Nq, Nk, d, dtype, causal, 110, mask)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        assert not torch.isnan(o2).any()


def test_noalloc_rejects_sizes_beyond_its_array(A):
    import torch
    # 40000 query rows against a 64-key cache: 40000 x 129 x 4 bytes of partial
    # results, more than the 16 MiB array.  Refused before anything is
    # launched, with a message that names the limit; the tensors are real and
    # sized for the call, so nothing could go out of bounds either way.
    B, H, Nq, Nk, d = 1, 1, 40000, 64, 128
    need = A.lib().attn_decode_workspace_bytes(B, H, Nq, Nk, d, 0)
    assert need > 16 << 20
    q = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, H, Nk, d), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((B, H, Nk, d), dtype=torch.bfloat16, device="cuda")
    o = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
    print("[case] noalloc limit", need, flush=True)
    st = A.lib().attn_decode_fwd_noalloc(ptr(q), ptr(k), ptr(v), ptr(o), None, B, H, Nq, Nk, d,
                                         0.088, 0, None, A.BF16, None, 0)
    assert st == 10, st      # ATTN_ERR_WORKSPACE
    assert b"16777216" in A.lib().attn_last_error()
