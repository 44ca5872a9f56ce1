"""moe_permute_noalloc (the dispatch layout without a workspace, for callers
that cannot allocate device memory) against moe_permute on the same inputs:
every output bit-exact, on two calls in a row on one GPU (the second with a
smaller batch, so stale scratch contents from the first call would show), plus
the host-side refusal of a batch whose scratch would not fit."""

import numpy as np
import pytest
import torch

import expert_routing_router_amd as M
from tests.gpu_util import dev, host, log

pytestmark = pytest.mark.gpu


def _idx(T, N, K, seed):
    rng = np.random.default_rng(seed)
    # distinct experts per token, skewed towards the low ids (ragged loads)
    p = 1.0 / np.arange(1, N + 1) ** 0.8
    p /= p.sum()
    return np.stack([rng.choice(N, K, replace=False, p=p) for _ in range(T)]).astype(np.int32)


def _outputs(desc, idx, u, noalloc):
    T, K, N = desc.T, desc.top_k, desc.n_routed
    offsets = torch.full((N + 1,), -7, dtype=torch.int32, device="cuda")
    row_token = torch.full((T * K,), -7, dtype=torch.int32, device="cuda")
    slot_row = torch.full((T * K,), -7, dtype=torch.int32, device="cuda")
    counts = torch.full((N,), -7, dtype=torch.int32, device="cuda")
    x_perm = torch.zeros((T * K, desc.d), dtype=torch.bfloat16, device="cuda")
    if noalloc:
        M.moe_permute_noalloc(desc, idx, offsets, row_token, slot_row, counts, u=u, x_perm=x_perm)
    else:
        ws = torch.empty(M.moe_workspace_bytes(desc), dtype=torch.uint8, device="cuda")
        M.moe_permute(desc, idx, offsets, row_token, slot_row, ws, counts=counts, u=u, x_perm=x_perm)
    torch.cuda.synchronize()
    return [host(t) for t in (offsets, row_token, slot_row, counts)] + [x_perm.view(torch.int16).cpu().numpy()]


def test_noalloc_permute_matches_workspace_permute():
    N, K, d = 256, 8, 256
    for T, seed in ((8192, 1), (1000, 2)):        # the second call is smaller
        log("moe_permute_noalloc T=%d N=%d K=%d" % (T, N, K))
        desc = M.make_desc(T=T, d=d, n_routed=N, top_k=K, n_groups=8, topk_groups=4, group_topk=2,
                           n_shared=1, inter=2048)
        idx = dev(_idx(T, N, K, seed), "i32")
        u = torch.randn((T, d), device="cuda").to(torch.bfloat16)
        got = _outputs(desc, idx, u, True)
        want = _outputs(desc, idx, u, False)
        for a, b, name in zip(got, want, ("offsets", "row_token", "slot_row", "counts", "x_perm")):
            assert np.array_equal(a, b), (T, name)
        assert got[3].sum() == T * K and got[0][-1] == T * K


def test_noalloc_permute_refuses_oversized_batch():
    desc = M.make_desc(T=1 << 18, d=8, n_routed=256, top_k=1, n_shared=0, inter=64, in_dtype="f32",
                       router_dtype="f32", expert_dtype="f32")
    assert M.moe_validate(desc) == M.MOE_OK
    one = torch.empty(16, dtype=torch.int32, device="cuda")
    st = M.lib().moe_permute_noalloc(desc, one.data_ptr(), one.data_ptr(), one.data_ptr(), one.data_ptr(),
                                     None, None, None, None)
    assert st == M.MOE_EWORKSPACE
