"""moe_build_indices_noalloc (the form whose scratch is the library's static
device array, for callers that cannot allocate) against moe_build_indices,
through the C ABI: every output bit-exact, on two calls in a row on the same
output buffers, the second with fewer tokens and experts (the scratch keeps
the first call's counts, which must not leak into the second), and the
refusal of a call whose scratch would exceed the static array."""
import ctypes

import numpy as np
import pytest
import torch

from tests.gpu_util import host, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _routing(T, E, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    return idx, rng.random((T, k)).astype(np.float32)


def _outputs(T, k, L, H, quant):
    R = T * k
    o = {"offsets": torch.empty(L + 1, dtype=torch.int32, device=DEV),
         "sorted_token": torch.empty(R, dtype=torch.int32, device=DEV),
         "row_of_slot": torch.empty(R, dtype=torch.int32, device=DEV),
         "sorted_weight": torch.empty(R, dtype=torch.float32, device=DEV)}
    if H:
        o["x_perm"] = torch.empty((R, H), dtype=torch.uint8 if quant else torch.bfloat16, device=DEV)
        if quant:
            o["x_perm_scale"] = torch.empty((R, H // 128), dtype=torch.float32, device=DEV)
    return o


def _compare(a, b, n_rows):
    for key in ("offsets", "row_of_slot"):
        assert torch.equal(a[key], b[key]), key
    for key in ("sorted_token", "sorted_weight", "x_perm", "x_perm_scale"):
        if key in a:
            assert torch.equal(a[key][:n_rows], b[key][:n_rows]), key


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixture_experts_ffn_top_amd as m
    m.lib()
    return m


def test_noalloc_matches_workspace_form_twice(moe):
    cases = [  # (T, E, k, start, L, H, xperm): the second is smaller
        (8192, 256, 8, 0, 256, 512, "fp8"),
        (300, 40, 3, 4, 24, 256, "bf16"),
    ]
    big_T, big_k = cases[0][0], cases[0][2]
    bufs = _outputs(big_T, big_k, 256, 512, True)        # the noalloc calls write into these, both times
    for T, E, k, start, L, H, xp in cases:
        say(f"[noalloc] T={T} E={E} k={k} start={start} L={L} H={H} {xp}")
        idx, w = _routing(T, E, k, T)
        it, wt = torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV)
        g = torch.Generator(device=DEV)
        g.manual_seed(T)
        x = torch.randn((T, H), generator=g, device=DEV).to(torch.bfloat16)
        mask = (torch.rand((T,), generator=g, device=DEV) > 0.2).to(torch.uint8)
        want = moe.build_indices(it, L, expert_start=start, weights=wt, token_mask=mask, x=x, xperm_dtype=xp)
        R = T * k
        view = {"offsets": bufs["offsets"][:L + 1], "sorted_token": bufs["sorted_token"][:R],
                "row_of_slot": bufs["row_of_slot"][:R], "sorted_weight": bufs["sorted_weight"][:R]}
        if xp == "fp8":
            view["x_perm"] = bufs["x_perm"][:R]
            view["x_perm_scale"] = bufs["x_perm_scale"][:R, : H // 128]
        else:
            view["x_perm"] = bufs["x_perm"].view(-1)[: R * H * 2].view(torch.bfloat16).view(R, H)
        got = moe.build_indices(it, L, expert_start=start, weights=wt, token_mask=mask, x=x, xperm_dtype=xp,
                                noalloc=True, out=view)
        torch.cuda.synchronize()
        n = int(host(want["offsets"])[-1])
        assert n > 0
        _compare(want, got, n)


def test_noalloc_refuses_beyond_its_scratch(moe):
    lib = moe.lib()
    T, k, L = 1 << 20, 4, 1024      # 8192 blocks x 1024 experts x 4 bytes = 32 MiB of counts
    need = lib.moe_build_indices_workspace_bytes(T, k, L)
    assert need > 16 * 1024 * 1024
    a = moe.IndexArgs(num_tokens=T, n_experts_per_tok=k, experts_start_idx=0, n_local_experts=L,
                      expert_indices=16, expert_offsets=32, sorted_token=48, row_of_slot=64)
    st = lib.moe_build_indices_noalloc(ctypes.byref(a), None)
    assert st == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    assert b"static scratch" in lib.moe_last_error_message()
    a.workspace, a.workspace_bytes = 80, 1 << 20
    assert lib.moe_build_indices_noalloc(ctypes.byref(a), None) == moe.MOE_ERR_INVALID_ARGUMENT
