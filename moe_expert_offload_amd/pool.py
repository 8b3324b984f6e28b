"""Pinned host pool of expert records (memory plumbing around ft_pool_alloc).

The pool is page-locked host memory from hipHostMalloc, viewed from Python as an
array [rows, record_bytes / itemsize] of `dtype` (uint16 bf16 words for bf16
records, uint8 for MXFP4 records).  Row (l mod L_phys) * E + e holds the record of
layer l, expert e.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import ft


class HostPool:
    def __init__(self, rows: int, record_bytes: int, dtype=np.uint16):
        dtype = np.dtype(dtype)
        if record_bytes % dtype.itemsize:
            raise ValueError("record size is not a whole number of elements")
        self.rows = rows
        self.record_bytes = record_bytes
        self.nbytes = rows * record_bytes
        self.ptr = ft.ft_pool_alloc(self.nbytes)
        buf = (C.c_uint8 * self.nbytes).from_address(self.ptr)
        self.view = np.ctypeslib.as_array(buf).view(dtype).reshape(rows, record_bytes // dtype.itemsize)

    def free(self):
        if self.ptr:
            self.view = None
            ft.ft_pool_free(self.ptr)
            self.ptr = 0

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.free()
