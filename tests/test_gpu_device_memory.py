"""The library allocates no device memory: the forward keeps only its
streaming state (the score matrix is never stored, and no workspace exists),
and the cache path and the gradient use the caller's workspace.  Checked as the
device's free memory (hipMemGetInfo through torch) across repeated calls at the
B1 H32 N8192 d128 causal shape, after one warm-up call that loads the code
objects.  Inputs are zeros: only allocation is observed here.

Every case prints what it runs (flushed) before touching the GPU.
"""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    import torch
    assert torch.cuda.is_available()
    import tiled_online_softmax_fwd_amd as A
    A.lib()
    return A


def say(*a):
    print("[case]", *a, flush=True)


def free_bytes():
    import torch
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


def test_forward_and_cache_path_allocate_nothing(attn):
    import torch
    B, H, N, d = 1, 32, 8192, 128
    q, k, v = (torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    qd = torch.zeros((8, 32, 1, d), dtype=torch.bfloat16, device="cuda")
    kd, vd = (torch.zeros((8, 32, 8192, d), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    od = torch.empty_like(qd)
    ld = torch.empty((8, 32, 1), dtype=torch.float32, device="cuda")
    need = attn.lib().attn_decode_workspace_bytes(8, 32, 1, 8192, d, 0)
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")

    def run():
        attn.fwd(q, k, v, causal=True, out=o, lse=lse)
        attn.decode_fwd(qd, kd, vd, out=od, lse=ld, workspace=ws)

    say("device memory: forward and cache path", B, H, N, d)
    run()
    before = free_bytes()
    for _ in range(5):
        run()
    after = free_bytes()
    assert after == before, f"free device memory changed by {before - after} bytes"


def test_backward_allocates_nothing_beyond_its_outputs(attn):
    """The gradient's outputs are torch tensors; once the first call's blocks
    sit in torch's cache, further calls change the free device memory only if
    the library itself allocates."""
    import torch
    B, H, N, d = 1, 8, 4096, 128
    q, k, v, g = (torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda") for _ in range(4))
    o, lse = attn.fwd(q, k, v, causal=True)
    need = attn.lib().attn_bwd_workspace_bytes(B, H, N)
    ws = torch.empty((max(need, 16),), dtype=torch.uint8, device="cuda")
    say("device memory: backward", B, H, N, d)
    grads = attn.bwd(q, k, v, o, g, lse, causal=True, workspace=ws)
    del grads
    before = free_bytes()
    for _ in range(3):
        grads = attn.bwd(q, k, v, o, g, lse, causal=True, workspace=ws)
        del grads
    after = free_bytes()
    assert after == before, f"free device memory changed by {before - after} bytes"
