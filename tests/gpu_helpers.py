"""Helpers of the GPU tests: device tensors, pinned host pools, contexts.

Inputs come from moe_expert_offload_amd.synth (seeded); expected values come
from the oracle only.
"""
from __future__ import annotations

import numpy as np

from moe_expert_offload_amd import ft
from moe_expert_offload_amd.pool import HostPool
from moe_expert_offload_amd.synth import Shape, fill_mxfp4_records_torch, fill_records_torch


def torch_mod():
    import torch
    return torch


def dev_u16(a):
    """numpy uint16 (bf16 words) -> CUDA tensor with the same bits."""
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


def dev(a):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


class PinnedPool(HostPool):
    """A pinned host pool of expert records: uint16 [rows, record_elems] (bf16) or
    uint8 [rows, record_bytes] (MXFP4)."""

    def __init__(self, shape: Shape, rows: int):
        super().__init__(rows, shape.record_bytes, shape.pool_dtype)
        self.shape = shape

    def fill_device_random(self, seed_key: int, seed: int = 0):
        if self.shape.mxfp4:
            fill_mxfp4_records_torch(self.view, self.shape.d, self.shape.d_ff, seed_key, seed)
        else:
            fill_records_torch(self.view, seed_key, seed)


class Engine:
    """A context over a pinned pool, a device slot buffer and a device workspace."""

    def __init__(self, shape: Shape, pool: PinnedPool, n_slots: int, T_max: int, frac_q16: int,
                 min_fill=1, max_fetch=-1, cpu_threads=0, prefill_overlap=0, L_phys=0):
        torch = torch_mod()
        self.shape = shape
        self.fshape = ft.make_shape(shape.L, shape.E, shape.d, shape.d_ff, shape.k,
                                    ft.FT_W_MXFP4 if shape.mxfp4 else ft.FT_W_BF16)
        self.cfg = ft.make_config(frac_q16, min_fill, max_fetch, cpu_threads, prefill_overlap, T_max, L_phys)
        S = shape.record_bytes
        self.slots = torch.empty(max(n_slots, 1) * S, dtype=torch.uint8, device="cuda")
        wsb = ft.ft_workspace_bytes(self.fshape, T_max)
        self.ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        assert self.slots.data_ptr() % 256 == 0 and self.ws.data_ptr() % 256 == 0
        self.ctx = ft.ft_create(self.fshape, self.cfg, pool.ptr, pool.nbytes, self.slots, n_slots, self.ws, wsb)
        self.copy = torch.cuda.Stream()

    def destroy(self):
        if self.ctx:
            ft.ft_destroy(self.ctx)
            self.ctx = None


def tile_cover_tokens(idx, E):
    """Tokens whose outputs reach every expert group of a chunk's grouping (pairs
    grouped stably by expert, as the oracle groups them): the first row of every
    non-empty group; rows 31 and 32 and the last row of the largest group (the
    32-row sub-tile edge and the ragged tail); rows 255 and 256 of every group that
    passes 256 rows (the two sides of the 256-row pass edge)."""
    from oracle.permute import group_pairs
    off, perm, _ = group_pairs(idx, E)
    k = idx.shape[1]
    sizes = np.diff(off)
    rows = []
    for g in range(E):
        if sizes[g] == 0:
            continue
        rows.append(off[g])
        if sizes[g] > 256:
            rows += [off[g] + 255, off[g] + 256]
    big = int(np.argmax(sizes))
    rows += [off[big] + r for r in (31, 32, sizes[big] - 1) if r < sizes[big]]
    return np.unique(perm[np.asarray(rows, np.int64)] // k), sizes
