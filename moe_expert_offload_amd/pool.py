"""Pinned host pool of expert records (memory plumbing around ft_pool_alloc).

The pool is page-locked host memory from hipHostMalloc, viewed from Python as a
uint16 array [rows, record_elems] (bf16 words).  Row (l mod L_phys) * E + e holds
the record of layer l, expert e.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import ft


class HostPool:
    def __init__(self, record_elems: int, rows: int):
        self.record_elems = record_elems
        self.rows = rows
        self.nbytes = rows * record_elems * 2
        self.ptr = ft.ft_pool_alloc(self.nbytes)
        buf = (C.c_uint16 * (self.nbytes // 2)).from_address(self.ptr)
        self.view = np.ctypeslib.as_array(buf).reshape(rows, record_elems)

    def free(self):
        if self.ptr:
            self.view = None
            ft.ft_pool_free(self.ptr)
            self.ptr = 0

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.free()
