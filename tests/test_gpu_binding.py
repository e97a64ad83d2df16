"""The Python binding checks every caller-supplied tensor (device, contiguity,
dtype, exact shape, workspace bytes) before anything reaches the library, which
writes through the raw pointers.  Each bad case must raise ValueError."""
import numpy as np
import pytest

import synth


def attn_mod():
    import tiled_online_softmax_fwd_amd as A
    return A


def test_cpu_inputs_rejected_before_the_library():
    """Host tensors never reach the ABI (no GPU needed)."""
    import torch
    A = attn_mod()
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        A.fwd(q, q, q)
    with pytest.raises(ValueError):
        A.decode_fwd(q, q, q)
    with pytest.raises(ValueError):
        A.bwd(q, q, q, q, q, torch.zeros((1, 1, 8)))


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available()
    attn_mod().lib()
    return torch.device("cuda", torch.cuda.current_device())


def qkv(dev, B=1, H=2, N=64, d=64, dtype="bf16"):
    return synth.upload(synth.make_qkv(B, H, N, d, dtype, 80))


@pytest.mark.gpu
def test_forward_rejects_bad_outputs_and_masks(dev):
    import torch
    A = attn_mod()
    q, k, v = qkv(dev)
    B, H, N, d = q.shape
    cases = {
        "bf16 out with out_fp32": dict(out=torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev), out_fp32=True),
        "fp32 out for bf16 output": dict(out=torch.empty((B, H, N, d), dtype=torch.float32, device=dev)),
        "out shape": dict(out=torch.empty((B, H, N - 1, d), dtype=torch.bfloat16, device=dev)),
        "out on host": dict(out=torch.empty((B, H, N, d), dtype=torch.bfloat16)),
        "out strided": dict(out=torch.empty((B, H, d, N), dtype=torch.bfloat16, device=dev).transpose(2, 3)),
        "lse dtype": dict(lse=torch.empty((B, H, N), dtype=torch.bfloat16, device=dev)),
        "lse shape": dict(lse=torch.empty((B, H, N + 1), dtype=torch.float32, device=dev)),
        "lse on host": dict(lse=torch.empty((B, H, N), dtype=torch.float32)),
        "mask on host": dict(key_padding_mask=torch.zeros((B, N), dtype=torch.uint8)),
        "mask shape": dict(key_padding_mask=torch.zeros((B, N + 3), dtype=torch.uint8, device=dev)),
        "mask dtype": dict(key_padding_mask=torch.zeros((B, N), dtype=torch.int32, device=dev)),
    }
    for what, kw in cases.items():
        print("[case] forward:", what, flush=True)
        with pytest.raises(ValueError):
            A.fwd(q, k, v, **kw)
        with pytest.raises(ValueError):
            A.naive_fwd(q, k, v, **kw)
    print("[case] forward: strided k", flush=True)
    kt = torch.empty((B, H, d, N), dtype=q.dtype, device=dev).transpose(2, 3)
    with pytest.raises(ValueError):
        A.fwd(q, kt, v)


@pytest.mark.gpu
def test_workspaces_are_checked_in_bytes(dev):
    import torch
    A = attn_mod()
    q, k, v = qkv(dev)
    B, H, N, d = q.shape
    need = A.lib().attn_naive_workspace_bytes(B, H, N, A.BF16)
    print("[case] naive workspace: fp32 tensor of exactly the bytes needed", flush=True)
    ws = torch.empty(((need + 3) // 4,), dtype=torch.float32, device=dev)
    A.naive_fwd(q, k, v, workspace=ws)
    torch.cuda.synchronize()
    print("[case] naive workspace: one element short / on host", flush=True)
    with pytest.raises(ValueError):
        A.naive_fwd(q, k, v, workspace=torch.empty((need // 4 - 1,), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        A.naive_fwd(q, k, v, workspace=torch.empty((need,), dtype=torch.uint8))
    need_d = A.lib().attn_decode_workspace_bytes(B, H, 1, N, d, 0)
    qd = q[:, :, :1].contiguous()
    print("[case] decode workspace short / out shape", flush=True)
    with pytest.raises(ValueError):
        A.decode_fwd(qd, k, v, workspace=torch.empty((max(need_d - 1, 0),), dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError):
        A.decode_fwd(qd, k, v, out=torch.empty((B, H, 2, d), dtype=q.dtype, device=dev))
    need_b = A.lib().attn_bwd_workspace_bytes(B, H, N)
    o, lse = A.fwd(q, k, v)
    print("[case] backward lse dtype / shape / workspace", flush=True)
    with pytest.raises(ValueError):
        A.bwd(q, k, v, o, o, lse.to(torch.bfloat16))
    with pytest.raises(ValueError):
        A.bwd(q, k, v, o, o, lse[:, :, :-1].contiguous())
    with pytest.raises(ValueError):
        A.bwd(q, k, v, o, o, lse, workspace=torch.empty((max(need_b - 1, 0),), dtype=torch.uint8, device=dev))


@pytest.mark.gpu
def test_block_mask_is_checked(dev):
    import torch
    A = attn_mod()
    q, k, v = qkv(dev, N=128, d=128)
    B, H, N, d = q.shape
    nb = N // 64
    print("[case] block mask on host / wrong shape", flush=True)
    with pytest.raises(ValueError):
        A.fwd_sparse(q, k, v, torch.ones((B, H, nb, nb), dtype=torch.uint8), block=64)
    with pytest.raises(ValueError):
        A.fwd_sparse(q, k, v, torch.ones((B, H, nb, nb + 1), dtype=torch.uint8, device=dev), block=64)
