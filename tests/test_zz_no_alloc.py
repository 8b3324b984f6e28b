"""The grouping entry point that allocates nothing (ft_permute_noalloc) against
ft_permute with a caller workspace, through the C ABI: bit-identical offsets,
perm and inv on two calls in a row (the second smaller, so stale contents of
the library's fixed scratch array would show), and the size limit rejected on
the host before any launch."""
import numpy as np
import pytest

from moe_expert_offload_amd import ft
from tests.gpu_helpers import dev, host, torch_mod

pytestmark = pytest.mark.gpu


def _keys(P, G, seed):
    rng = np.random.default_rng(seed)
    k = rng.integers(0, G, size=P).astype(np.int32)
    k[rng.random(P) < 0.05] = -1  # pairs left out
    return k


def _both(key, P, G):
    torch = torch_mod()
    kd = dev(key)
    out = {}
    for name in ("ws", "noalloc"):
        off = torch.full((G + 1,), -7, dtype=torch.int32, device="cuda")
        perm = torch.full((max(P, 1),), -7, dtype=torch.int32, device="cuda")
        inv = torch.full((max(P, 1),), -7, dtype=torch.int32, device="cuda")
        if name == "ws":
            wsb = ft.ft_permute_workspace_bytes(P, G)
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            ft.ft_permute(kd, P, G, off, perm, inv, ws, wsb)
        else:
            ft.ft_permute_noalloc(kd, P, G, off, perm, inv)
        torch.cuda.synchronize()
        out[name] = (host(off), host(perm), host(inv))
    return out


def test_noalloc_matches_workspace_form_twice():
    cases = [(49152, 256, 1), (5000, 1024, 2)]  # 8192 tokens x top-6 over 256 experts, then smaller
    for P, G, seed in cases:
        print("[case] permute_noalloc P", P, "groups", G, flush=True)
        key = _keys(P, G, seed)
        r = _both(key, P, G)
        off_w, perm_w, inv_w = r["ws"]
        off_n, perm_n, inv_n = r["noalloc"]
        assert np.array_equal(off_w, off_n)
        n = int(off_w[G])
        assert n == int((key >= 0).sum())
        assert np.array_equal(perm_w[:n], perm_n[:n])
        assert np.array_equal(inv_w, inv_n)


def test_noalloc_rejects_beyond_its_scratch():
    torch = torch_mod()
    cap = ft.ft_permute_noalloc_max_scratch_bytes()
    assert cap == 1 << 20
    P, G = 70000, 1024  # needs 274 blocks x 4 KB of counts, more than 1 MiB
    assert ft.ft_permute_workspace_bytes(P, G) > cap
    t = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(ft.FtError) as ei:
        ft.ft_permute_noalloc(t, P, G, t, t, t)
    assert ei.value.status == ft.FT_EINVAL
