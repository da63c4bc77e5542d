"""moe_permute_noalloc (no workspace: the library's per-device scratch array)
against moe_permute (caller's workspace), through the C ABI: bit-identical
counts, offsets, rows, permutation and gathered rows, on two calls in a row, the
second smaller than the first, so that the second runs on what the first left
in the scratch array."""
import numpy as np
import pytest
import torch

from mixture_experts_ffn_08_amd import _lib
from support import host, log

pytestmark = pytest.mark.gpu


def routed(T, k, E, seed):
    """Seeded top-k expert lists: k distinct experts per token, skewed toward low ids."""
    g = torch.Generator().manual_seed(seed)
    keys = torch.rand(T, E, generator=g) + torch.linspace(0.5, 0.0, E)
    return keys.topk(k, dim=1).indices.to(torch.int32).contiguous()


def permute_both(T, k, E, d, phi, seed):
    idx = routed(T, k, E, seed).cuda()
    x = torch.randn(T, d, generator=torch.Generator().manual_seed(seed + 1)).to(torch.bfloat16).cuda()
    cap = _lib.moe_capacity(T, k, E, phi)
    outs = []
    for noalloc in (False, True):
        o = dict(counts=torch.full((E,), -7, dtype=torch.int32, device="cuda"),
                 offsets=torch.full((E + 1,), -7, dtype=torch.int32, device="cuda"),
                 row_of=torch.full((T, k), -7, dtype=torch.int32, device="cuda"),
                 perm_token=torch.full((T * k,), -7, dtype=torch.int32, device="cuda"),
                 x_perm=torch.zeros((T * k, d), dtype=torch.bfloat16, device="cuda"))
        if noalloc:
            _lib.moe_permute_noalloc(idx, T, k, E, cap, x, d, o["counts"], o["offsets"], o["row_of"],
                                     o["perm_token"], o["x_perm"])
        else:
            ws = torch.empty(max(_lib.moe_permute_workspace_bytes(T, k, E), 1), dtype=torch.uint8, device="cuda")
            _lib.moe_permute(idx, T, k, E, cap, x, d, o["counts"], o["offsets"], o["row_of"], o["perm_token"],
                             o["x_perm"], ws)
        torch.cuda.synchronize()
        outs.append({key: host(v) for key, v in o.items()})
    return outs, cap


@pytest.mark.parametrize("first,second", [
    ((16384, 8, 128, 2048, None), (3000, 4, 64, 256, 1.0)),     # many blocks, then fewer (capacity cut)
    ((9000, 8, 256, 256, 1.25), (700, 2, 8, 128, None)),         # E = 256 under capacity, then E = 8
    ((2048, 8, 256, 128, None), (40, 2, 8, 128, 0.5)),           # then a one-block dispatch
])
def test_noalloc_permute_matches_workspace_permute(first, second):
    for T, k, E, d, phi in (first, second):
        (ref, got), cap = permute_both(T, k, E, d, phi, seed=T + E)
        R = int(ref["offsets"][-1])
        for key in ("counts", "offsets", "row_of"):
            assert np.array_equal(got[key], ref[key]), key
        assert np.array_equal(got["perm_token"][:R], ref["perm_token"][:R])
        assert np.array_equal(got["x_perm"][:R], ref["x_perm"][:R])
        assert int(ref["counts"].sum()) == T * k
        log(f"[noalloc T={T} k={k} E={E} cap={cap}] R={R} bit-identical to moe_permute")


def test_noalloc_permute_rejects_beyond_its_scratch():
    T, k, E = 1 << 18, 8, 256
    need = _lib.moe_permute_workspace_bytes(T, k, E)
    assert need > (4 << 20)
    dummy = torch.zeros(1, dtype=torch.int32, device="cuda")
    status = _lib.load().moe_permute_noalloc(dummy.data_ptr(), T, k, E, -1, 0, _lib.MOE_BF16, 128,
                                             dummy.data_ptr(), dummy.data_ptr(), dummy.data_ptr(),
                                             dummy.data_ptr(), 0, 0)
    assert status == _lib.MOE_ERR_UNSUPPORTED
    assert "scratch" in _lib.last_error()
