"""moe_permute_noalloc (static scratch, no workspace) against moe_permute on the GPU.

Two calls in a row through the C ABI, the second with a smaller input, each bit-exact against
moe_permute on the same routing (integer outputs), with and without the shared-expert group.
The first call of the process on the device also looks the scratch array's address up.
"""
import numpy as np
import pytest
import torch

import sparse_moe_transformer_02_amd as moe

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _routing(T, K, N_r, seed, hot=0):
    g = torch.Generator(device=DEV).manual_seed(seed)
    s = torch.rand((T, N_r), generator=g, device=DEV)
    if hot:
        s[:, :hot] += 1.0
    return torch.topk(s, K, dim=1).indices.to(torch.int32).contiguous()


def _outputs(T, K, N_r, S):
    i32 = dict(dtype=torch.int32, device=DEV)
    return dict(counts=torch.full((N_r,), -7, **i32), offsets=torch.full((N_r + (2 if S else 1),), -7, **i32),
                row_token=torch.full((S + T * K,), -7, **i32), slot_row=torch.full((T * K,), -7, **i32))


@pytest.mark.parametrize("S_on", [False, True])
def test_noalloc_matches_permute_twice(S_on):
    cases = [(16384, 8, 256, 1, 8), (777, 8, 256, 2, 0)]     # second call smaller, ragged
    for T, K, N_r, seed, hot in cases:
        print(f"noalloc case T={T} K={K} N_r={N_r} shared={S_on}", flush=True)
        idx = _routing(T, K, N_r, seed, hot)
        S = T if S_on else 0
        ref = moe.moe_permute(idx, N_r, shared_rows=S)
        out = _outputs(T, K, N_r, S)
        moe.moe_permute_noalloc(idx, N_r, shared_rows=S, **out)
        torch.cuda.synchronize()
        for name, r in zip(("counts", "offsets", "row_token", "slot_row"), ref):
            assert np.array_equal(out[name].cpu().numpy(), r.cpu().numpy()), (T, name)
        assert int(out["counts"].sum()) == T * K


def test_noalloc_rejects_oversize_before_launch():
    T, K, N_r = 262208, 8, 256
    assert moe.moe_permute_workspace_size(T, K, N_r) > moe.moe_permute_noalloc_max_bytes()
    idx = torch.zeros((T, K), dtype=torch.int32, device=DEV)
    with pytest.raises(moe.MoeError):
        moe.moe_permute_noalloc(idx, N_r, shared_rows=0, **_outputs(T, K, N_r, 0))
