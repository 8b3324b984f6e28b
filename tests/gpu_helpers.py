"""Helpers of the GPU tests: device tensors, pinned host pools, contexts.

Inputs come from moe_expert_offload_amd.synth (seeded); expected values come
from the oracle only.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from moe_expert_offload_amd import ft
from moe_expert_offload_amd.synth import Shape


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


class PinnedPool:
    """A pinned host pool of expert records from ft_pool_alloc, viewed as uint16 [rows, record_elems]."""

    def __init__(self, shape: Shape, rows: int):
        self.shape = shape
        self.rows = rows
        self.nbytes = rows * shape.record_bytes
        self.ptr = ft.ft_pool_alloc(self.nbytes)
        buf = (C.c_uint16 * (self.nbytes // 2)).from_address(self.ptr)
        self.view = np.ctypeslib.as_array(buf).reshape(rows, shape.record_elems)

    def fill_numpy(self, records):
        self.view[:] = records

    def fill_device_random(self, seed: int, std: float = 0.02, chunk: int = 16):
        """Fill with N(0, std^2) rounded to bf16, generated on the GPU (fast for big pools)."""
        torch = torch_mod()
        g = torch.Generator(device="cuda")
        host_t = torch.from_numpy(self.view.reshape(-1).view(np.int16))
        n = self.shape.record_elems
        for r0 in range(0, self.rows, chunk):
            r1 = min(self.rows, r0 + chunk)
            g.manual_seed(seed * 1_000_003 + r0)
            w = torch.randn((r1 - r0) * n, generator=g, device="cuda", dtype=torch.float32).mul_(std)
            host_t[r0 * n:r1 * n].copy_(w.to(torch.bfloat16).view(torch.int16))
        torch.cuda.synchronize()

    def free(self):
        if self.ptr:
            ft.ft_pool_free(self.ptr)
            self.ptr = 0


class Engine:
    """A context over a pinned pool, a device slot buffer and a device workspace."""

    def __init__(self, shape: Shape, pool: PinnedPool, n_slots: int, T_max: int, frac_q16: int,
                 min_fill=1, max_fetch=-1, cpu_threads=0, prefill_overlap=0, L_phys=0):
        torch = torch_mod()
        self.shape = shape
        self.fshape = ft.make_shape(shape.L, shape.E, shape.d, shape.d_ff, shape.k)
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
