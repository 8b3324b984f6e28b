"""Thin ctypes binding of libft (C ABI in include/ft.h).

Argument marshalling only: every call goes to the HIP/C++ library.  Functions
keep the C names; tensor arguments may be torch tensors (their data_ptr() is
passed), numpy arrays (host memory), raw integer addresses, or None for NULL.
Streams are torch streams, raw handles, or None (the current torch stream).
Loading fails loudly when the built library is missing.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libft.so")

FT_OK = 0
FT_EINVAL = -1
FT_ENOMEM = -2
FT_EBUSY = -3
FT_ENOPIN = -4
FT_ECAP = -5
FT_EHIP = -6
FT_EUNSUPPORTED = -7
FT_ENOPROFILE = -8
FT_WOVERLAP_OFF = 1
FT_PLAN_CAP = 512
FT_W_BF16 = 0
FT_W_MXFP4 = 1
FT_PLACE_LRU = 0
FT_PLACE_HOTSET = 1
FT_PLACE_STATIC = 2

EXPORTED = [
    "ft_strerror", "ft_last_error", "ft_record_bytes", "ft_workspace_bytes", "ft_frac_q16",
    "ft_qstar_split", "ft_pool_alloc", "ft_pool_free", "ft_bench_bw", "ft_create", "ft_destroy",
    "ft_get_stats", "ft_reset_stats", "ft_get_config", "ft_n_slots", "ft_router_topk",
    "ft_permute_workspace_bytes", "ft_permute", "ft_grouped_ffn", "ft_grouped_ffn_mx_workspace_bytes",
    "ft_grouped_ffn_mx", "ft_combine",
    "ft_expert_cache_lookup", "ft_expert_cache_fill", "ft_expert_cache_resize",
    "ft_expert_cache_where", "ft_moe_decode_layer", "ft_moe_prefill_begin", "ft_moe_prefill_layer",
    "ft_moe_prefill_end", "ft_prefill_slot", "ft_profile_enable", "ft_profile_read", "ft_host_experts",
    "ft_frac_q16_contended", "ft_fetch_fraction_q16", "ft_recommend_hybrid", "ft_bench_bw_contended",
    "ft_bw_profile_path", "ft_bw_profile_save", "ft_bw_profile_load", "ft_expert_cache_prefill_on_demand",
    "ft_replay_placement", "ft_layer_routing", "ft_decode_graph_create",
    "ft_decode_graph_launch", "ft_decode_graph_status", "ft_decode_graph_destroy", "ft_permute_noalloc", "ft_permute_noalloc_max_scratch_bytes",
]


FT_E_MAX = 1024


class ft_prefill_plan(C.Structure):
    _fields_ = [("layer", C.c_int32), ("n_u", C.c_int32), ("n_h", C.c_int32), ("n_rounds", C.c_int32),
                ("group_expert", C.c_int32 * FT_E_MAX), ("group_slot", C.c_int32 * FT_E_MAX),
                ("round_end", C.c_int32 * FT_E_MAX)]


class ft_bw_profile(C.Structure):
    _fields_ = [("B_P", C.c_double), ("B_H", C.c_double), ("pcie_ov", C.c_double), ("cpu_ov", C.c_double),
                ("fmt", C.c_int32)]


class ft_shape(C.Structure):
    _fields_ = [("L", C.c_int32), ("E", C.c_int32), ("d", C.c_int32), ("d_ff", C.c_int32),
                ("k", C.c_int32), ("fmt", C.c_int32)]


class ft_config(C.Structure):
    _fields_ = [("frac_q16", C.c_uint32), ("min_fill", C.c_int32), ("max_fetch", C.c_int32),
                ("cpu_threads", C.c_int32), ("prefill_overlap", C.c_int32), ("T_max", C.c_int32),
                ("L_phys", C.c_int32)]


_A = C.c_int32 * FT_PLAN_CAP


class ft_plan(C.Structure):
    _fields_ = [("layer", C.c_int32), ("T", C.c_int32), ("k", C.c_int32), ("n_u", C.c_int32),
                ("n_h", C.c_int32), ("n_m", C.c_int32), ("q", C.c_int32), ("n_c", C.c_int32),
                ("avail", C.c_int32), ("U", _A), ("H", _A), ("M", _A), ("F_slot", _A), ("G_slot", _A),
                ("route_slot", _A), ("pair_group", _A), ("idx", _A), ("gates", C.c_float * FT_PLAN_CAP)]


class ft_step_stats(C.Structure):
    _fields_ = [("layer", C.c_int32), ("T", C.c_int32), ("n_u", C.c_int32), ("hits", C.c_int32),
                ("misses", C.c_int32), ("q", C.c_int32), ("n_c", C.c_int32), ("cpu_caller_items", C.c_int32),
                ("h2d_bytes", C.c_int64), ("t_route_us", C.c_double), ("t_ctrl_us", C.c_double),
                ("t_cpu_us", C.c_double), ("t_total_us", C.c_double), ("t_issue_us", C.c_double),
                ("t_cpu_work_us", C.c_double), ("t_submit_us", C.c_double), ("t_between_us", C.c_double)]


class ft_stats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in ("calls", "unique_hits", "unique_misses", "fills", "cpu_experts",
                                         "reads", "read_hits", "read_fills", "read_cpu", "h2d_bytes",
                                         "prefill_layers", "resizes")]


class ft_profile(C.Structure):
    _fields_ = [("launches", C.c_int64), ("ms_gateup", C.c_double), ("ms_down", C.c_double),
                ("bytes_gateup", C.c_double), ("bytes_down", C.c_double), ("flops_gateup", C.c_double),
                ("flops_down", C.c_double)]


class FtError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {status} ({msg})")
        self.status = status


_lib = None
P = C.c_void_p
I = C.c_int32


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libft.so not built at {LIB_PATH}; run `python -m moe_expert_offload_amd.build`")
        L = C.CDLL(LIB_PATH)
        sig = {
            "ft_strerror": (C.c_char_p, [C.c_int]),
            "ft_last_error": (C.c_char_p, []),
            "ft_record_bytes": (C.c_size_t, [C.POINTER(ft_shape)]),
            "ft_workspace_bytes": (C.c_size_t, [C.POINTER(ft_shape), I]),
            "ft_frac_q16": (C.c_uint32, [C.c_double, C.c_double]),
            "ft_frac_q16_contended": (C.c_uint32, [C.c_double, C.c_double]),
            "ft_fetch_fraction_q16": (C.c_uint32, [C.POINTER(ft_bw_profile)]),
            "ft_recommend_hybrid": (I, [C.POINTER(C.c_double), C.POINTER(C.c_double), I, C.c_double]),
            "ft_bench_bw_contended": (C.c_int, [C.POINTER(ft_shape), P, I, P, I, C.POINTER(C.c_double),
                                                C.POINTER(C.c_double)]),
            "ft_bw_profile_path": (C.c_int, [I, I, C.c_char_p, C.c_char_p, C.c_size_t]),
            "ft_expert_cache_prefill_on_demand": (C.c_int, [P, I, P, I, C.POINTER(ft_prefill_plan)]),
            "ft_bw_profile_save": (C.c_int, [C.c_char_p, C.POINTER(ft_bw_profile)]),
            "ft_bw_profile_load": (C.c_int, [C.c_char_p, I, C.POINTER(ft_bw_profile)]),
            "ft_qstar_split": (I, [I, C.c_uint32, I, I, I]),
            "ft_pool_alloc": (C.c_int, [C.c_size_t, C.POINTER(P)]),
            "ft_pool_free": (C.c_int, [P]),
            "ft_bench_bw": (C.c_int, [C.POINTER(ft_shape), P, I, P, I, C.POINTER(C.c_double), C.POINTER(C.c_double)]),
            "ft_replay_placement": (C.c_int, [I, C.POINTER(ft_shape), I, P, I, I, I, C.POINTER(C.c_int64),
                                              C.POINTER(C.c_int64)]),
            "ft_create": (C.c_int, [C.POINTER(ft_shape), C.POINTER(ft_config), P, C.c_size_t, P, I, P, C.c_size_t, C.POINTER(P)]),
            "ft_destroy": (C.c_int, [P]),
            "ft_get_stats": (C.c_int, [P, C.POINTER(ft_stats)]),
            "ft_reset_stats": (C.c_int, [P]),
            "ft_get_config": (C.c_int, [P, C.POINTER(ft_config)]),
            "ft_n_slots": (I, [P]),
            "ft_router_topk": (C.c_int, [P, P, P, I, I, I, I, P, P, P, P]),
            "ft_permute_workspace_bytes": (C.c_size_t, [I, I]),
            "ft_permute": (C.c_int, [P, I, I, P, P, P, P, C.c_size_t, P]),
            "ft_permute_noalloc": (C.c_int, [P, I, I, P, P, P, P]),
            "ft_permute_noalloc_max_scratch_bytes": (C.c_size_t, []),
            "ft_grouped_ffn": (C.c_int, [P, I, I, I, I, P, P, P, P, I, I, I, I, P, P, I, P]),
            "ft_grouped_ffn_mx_workspace_bytes": (C.c_size_t, [I, I, I, I]),
            "ft_grouped_ffn_mx": (C.c_int, [P, I, I, I, I, P, P, P, P, I, I, I, I, I, P, C.c_size_t, P, I, P]),
            "ft_combine": (C.c_int, [P, P, P, P, I, I, I, P, P]),
            "ft_expert_cache_lookup": (C.c_int, [P, I, P, I, C.POINTER(ft_plan)]),
            "ft_expert_cache_fill": (C.c_int, [P, C.POINTER(ft_plan), P, P, P]),
            "ft_expert_cache_resize": (C.c_int, [P, P, I]),
            "ft_expert_cache_where": (I, [P, I, I]),
            "ft_moe_decode_layer": (C.c_int, [P, I, P, I, P, P, P, P, C.POINTER(ft_plan), C.POINTER(ft_step_stats)]),
            "ft_moe_prefill_begin": (C.c_int, [P, P]),
            "ft_moe_prefill_layer": (C.c_int, [P, I, P, I, P, P, P, P]),
            "ft_moe_prefill_end": (C.c_int, [P]),
            "ft_prefill_slot": (I, [P, I, I]),
            "ft_layer_routing": (C.c_int, [P, P, P, I, P]),
            "ft_decode_graph_create": (C.c_int, [P, I, P, C.POINTER(P), P, P, C.POINTER(P)]),
            "ft_decode_graph_launch": (C.c_int, [P, P]),
            "ft_decode_graph_status": (C.c_int, [P]),
            "ft_decode_graph_destroy": (C.c_int, [P]),
            "ft_profile_enable": (C.c_int, [P, I]),
            "ft_profile_read": (C.c_int, [P, C.POINTER(ft_profile)]),
            "ft_host_experts": (C.c_int, [P, I, I, I, I, C.POINTER(P), P, P, P, I, I, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if hasattr(t, "ctypes"):
        return t.ctypes.data
    raise TypeError(f"cannot pass {type(t)} as a pointer")


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(fn, st):
    if st < 0:
        raise FtError(fn, st, lib().ft_last_error().decode(errors="replace"))
    return st


# ---- plain calls ---------------------------------------------------------------

def ft_strerror(st):
    return lib().ft_strerror(st).decode()


def ft_last_error():
    return lib().ft_last_error().decode(errors="replace")


def make_shape(L, E, d, d_ff, k, fmt=FT_W_BF16):
    return ft_shape(L, E, d, d_ff, k, fmt)


def make_config(frac_q16=65536, min_fill=1, max_fetch=-1, cpu_threads=0, prefill_overlap=0, T_max=1, L_phys=0):
    return ft_config(frac_q16, min_fill, max_fetch, cpu_threads, prefill_overlap, T_max, L_phys)


def ft_record_bytes(shape):
    return lib().ft_record_bytes(C.byref(shape))


def ft_workspace_bytes(shape, T_max):
    return lib().ft_workspace_bytes(C.byref(shape), T_max)


def ft_frac_q16(B_P, B_H):
    return lib().ft_frac_q16(float(B_P), float(B_H))


def ft_frac_q16_contended(pcie_ov, cpu_ov):
    return lib().ft_frac_q16_contended(float(pcie_ov), float(cpu_ov))


def ft_fetch_fraction_q16(profile):
    return lib().ft_fetch_fraction_q16(C.byref(profile))


def ft_recommend_hybrid(B_P, B_H, threshold=2.0):
    """B_P, B_H: sequences (one entry per benched workload of a format); True for hybrid."""
    n = len(B_P)
    arr = C.c_double * max(n, 1)
    r = lib().ft_recommend_hybrid(arr(*B_P), arr(*B_H), n, float(threshold))
    return bool(_check("ft_recommend_hybrid", r))


def ft_bench_bw_contended(shape, host_pool, n_records, dev_scratch, threads=0):
    po, co = C.c_double(), C.c_double()
    _check("ft_bench_bw_contended", lib().ft_bench_bw_contended(C.byref(shape), _ptr(host_pool), n_records,
                                                                _ptr(dev_scratch), threads, C.byref(po),
                                                                C.byref(co)))
    return po.value, co.value


def ft_bw_profile_path(device, fmt, directory):
    buf = C.create_string_buffer(4096)
    _check("ft_bw_profile_path", lib().ft_bw_profile_path(device, fmt, directory.encode(), buf, 4096))
    return buf.value.decode()


def ft_bw_profile_save(path, profile):
    return _check("ft_bw_profile_save", lib().ft_bw_profile_save(path.encode(), C.byref(profile)))


def ft_bw_profile_load(path, fmt):
    """The stored profile, or None when there is no usable one (FT_ENOPROFILE)."""
    p = ft_bw_profile()
    st = lib().ft_bw_profile_load(path.encode(), fmt, C.byref(p))
    if st == FT_ENOPROFILE:
        return None
    _check("ft_bw_profile_load", st)
    return p


def ft_qstar_split(m, frac_q16, min_fill, max_fetch, avail):
    return _check("ft_qstar_split", lib().ft_qstar_split(m, frac_q16, min_fill, max_fetch, avail))


def ft_pool_alloc(nbytes):
    p = P()
    _check("ft_pool_alloc", lib().ft_pool_alloc(nbytes, C.byref(p)))
    return p.value


def ft_pool_free(ptr):
    _check("ft_pool_free", lib().ft_pool_free(ptr))


def ft_bench_bw(shape, host_pool, n_records, dev_scratch, threads=0):
    bp, bh = C.c_double(), C.c_double()
    _check("ft_bench_bw", lib().ft_bench_bw(C.byref(shape), _ptr(host_pool), n_records, _ptr(dev_scratch),
                                            threads, C.byref(bp), C.byref(bh)))
    return bp.value, bh.value


def ft_replay_placement(policy, shape, n_slots, ids, prompt):
    """(decode reads, decode misses) of a trace ids int32 [requests, prompt + decode, L, k]
    under one placement policy (FT_PLACE_*).  Host only."""
    import numpy as np
    a = np.ascontiguousarray(ids, dtype=np.int32)
    if a.ndim != 4 or a.shape[2] != shape.L or a.shape[3] != shape.k or a.shape[1] < prompt:
        raise ValueError("ids must be [requests, prompt + decode, L, k]")
    reads, misses = C.c_int64(), C.c_int64()
    _check("ft_replay_placement", lib().ft_replay_placement(
        policy, C.byref(shape), n_slots, a.ctypes.data_as(C.c_void_p), a.shape[0], prompt, a.shape[1] - prompt,
        C.byref(reads), C.byref(misses)))
    return reads.value, misses.value


def ft_create(shape, config, host_pool=None, pool_bytes=0, dev_slots=None, n_slots=0, dev_workspace=None,
              workspace_bytes=0):
    out = P()
    _check("ft_create", lib().ft_create(C.byref(shape), C.byref(config), _ptr(host_pool), pool_bytes,
                                        _ptr(dev_slots), n_slots, _ptr(dev_workspace), workspace_bytes,
                                        C.byref(out)))
    return out.value


def ft_destroy(ctx):
    return _check("ft_destroy", lib().ft_destroy(ctx))


def ft_get_stats(ctx):
    s = ft_stats()
    _check("ft_get_stats", lib().ft_get_stats(ctx, C.byref(s)))
    return {n: getattr(s, n) for n, _ in ft_stats._fields_}


def ft_reset_stats(ctx):
    return _check("ft_reset_stats", lib().ft_reset_stats(ctx))


def ft_get_config(ctx):
    c = ft_config()
    _check("ft_get_config", lib().ft_get_config(ctx, C.byref(c)))
    return c


def ft_n_slots(ctx):
    return lib().ft_n_slots(ctx)


def ft_router_topk(x, w_router, allowed, T, d, E, k, idx, gates, logits, stream=None):
    return _check("ft_router_topk", lib().ft_router_topk(_ptr(x), _ptr(w_router), _ptr(allowed), T, d, E, k,
                                                         _ptr(idx), _ptr(gates), _ptr(logits), _stream(stream)))


def ft_permute_workspace_bytes(P_, n_groups):
    return lib().ft_permute_workspace_bytes(P_, n_groups)


def ft_permute(key, P_, n_groups, offsets, perm, inv, workspace, workspace_bytes, stream=None):
    return _check("ft_permute", lib().ft_permute(_ptr(key), P_, n_groups, _ptr(offsets), _ptr(perm), _ptr(inv),
                                                 _ptr(workspace), workspace_bytes, _stream(stream)))


def ft_permute_noalloc(key, P_, n_groups, offsets, perm, inv, stream=None):
    return _check("ft_permute_noalloc", lib().ft_permute_noalloc(_ptr(key), P_, n_groups, _ptr(offsets), _ptr(perm),
                                                                 _ptr(inv), _stream(stream)))


def ft_permute_noalloc_max_scratch_bytes():
    return lib().ft_permute_noalloc_max_scratch_bytes()


def ft_grouped_ffn(x, T, d, d_ff, k, slots, group_slot, offsets, perm, n_groups, g_begin, g_end,
                   max_rows_per_group, h_ws, out, form=0, stream=None):
    return _check("ft_grouped_ffn", lib().ft_grouped_ffn(
        _ptr(x), T, d, d_ff, k, _ptr(slots), _ptr(group_slot), _ptr(offsets), _ptr(perm), n_groups, g_begin,
        g_end, max_rows_per_group, _ptr(h_ws), _ptr(out), form, _stream(stream)))


def ft_grouped_ffn_mx_workspace_bytes(T, d, d_ff, n_rows):
    return lib().ft_grouped_ffn_mx_workspace_bytes(T, d, d_ff, n_rows)


def ft_grouped_ffn_mx(x, T, d, d_ff, k, slots, group_slot, offsets, perm, n_groups, g_begin, g_end,
                      max_rows_per_group, n_rows, workspace, workspace_bytes, out, form, stream=None):
    return _check("ft_grouped_ffn_mx", lib().ft_grouped_ffn_mx(
        _ptr(x), T, d, d_ff, k, _ptr(slots), _ptr(group_slot), _ptr(offsets), _ptr(perm), n_groups, g_begin,
        g_end, max_rows_per_group, n_rows, _ptr(workspace), workspace_bytes, _ptr(out), form, _stream(stream)))


def ft_combine(out, inv, gates, cpu_partial, T, k, d, y, stream=None):
    return _check("ft_combine", lib().ft_combine(_ptr(out), _ptr(inv), _ptr(gates), _ptr(cpu_partial), T, k, d,
                                                 _ptr(y), _stream(stream)))


def ft_host_experts(x, T, d, d_ff, records, use_off, use_t, use_g, n_exp, threads, partial, fmt=FT_W_BF16):
    """records: sequence of host addresses (or numpy arrays); other arrays numpy."""
    recs = (P * max(n_exp, 1))(*[_ptr(r) for r in records])
    return _check("ft_host_experts", lib().ft_host_experts(_ptr(x), T, d, d_ff, fmt, recs, _ptr(use_off),
                                                           _ptr(use_t), _ptr(use_g), n_exp, threads, _ptr(partial)))


def ft_expert_cache_prefill_on_demand(ctx, layer, idx_host, T):
    """Decisions of one on-demand prefill layer: (U_groups, n_h, rounds) with rounds a list of
    {"fill": [(e, slot)], "compute": [(e, slot)]} in the plan's group order."""
    p = ft_prefill_plan()
    _check("ft_expert_cache_prefill_on_demand", lib().ft_expert_cache_prefill_on_demand(
        ctx, layer, _ptr(idx_host), T, C.byref(p)))
    groups = [(p.group_expert[g], p.group_slot[g]) for g in range(p.n_u)]
    rounds, g0 = [], 0
    for r in range(p.n_rounds):
        g1 = p.round_end[r]
        rounds.append({"fill": [gs for i, gs in enumerate(groups[g0:g1], g0) if i >= p.n_h],
                       "compute": groups[g0:g1]})
        g0 = g1
    return groups, p.n_h, rounds


def ft_expert_cache_lookup(ctx, layer, idx_host, T, plan=None):
    plan = ft_plan() if plan is None else plan
    _check("ft_expert_cache_lookup", lib().ft_expert_cache_lookup(ctx, layer, _ptr(idx_host), T, C.byref(plan)))
    return plan


def ft_expert_cache_fill(ctx, plan, copy_stream=None, wait_event=None, done_event=None):
    return _check("ft_expert_cache_fill", lib().ft_expert_cache_fill(
        ctx, C.byref(plan), _stream(copy_stream), _ptr(wait_event), _ptr(done_event)))


def ft_expert_cache_resize(ctx, new_dev_slots, n_slots):
    return _check("ft_expert_cache_resize", lib().ft_expert_cache_resize(ctx, _ptr(new_dev_slots), n_slots))


def ft_expert_cache_where(ctx, layer, expert):
    return lib().ft_expert_cache_where(ctx, layer, expert)


def ft_moe_decode_layer(ctx, layer, x, T, w_router, allowed, y, compute=None, plan=None, stats=None):
    return _check("ft_moe_decode_layer", lib().ft_moe_decode_layer(
        ctx, layer, _ptr(x), T, _ptr(w_router), _ptr(allowed), _ptr(y), _stream(compute),
        C.byref(plan) if plan is not None else None, C.byref(stats) if stats is not None else None))


def ft_moe_prefill_begin(ctx, copy=None):
    return _check("ft_moe_prefill_begin", lib().ft_moe_prefill_begin(ctx, _stream(copy)))


def ft_moe_prefill_layer(ctx, layer, x, T, w_router, y, compute=None, copy=None):
    return _check("ft_moe_prefill_layer", lib().ft_moe_prefill_layer(
        ctx, layer, _ptr(x), T, _ptr(w_router), _ptr(y), _stream(compute), _stream(copy)))


def ft_moe_prefill_end(ctx):
    return _check("ft_moe_prefill_end", lib().ft_moe_prefill_end(ctx))


def ft_layer_routing(ctx, idx, gates, T, stream=None):
    return _check("ft_layer_routing", lib().ft_layer_routing(ctx, _ptr(idx), _ptr(gates), T, _stream(stream)))


def ft_decode_graph_create(ctx, T, x, w_router, allowed, y):
    """w_router: sequence of L device tensors or addresses."""
    arr = (P * len(w_router))(*[_ptr(w) for w in w_router])
    out = P()
    _check("ft_decode_graph_create", lib().ft_decode_graph_create(ctx, T, _ptr(x), arr, _ptr(allowed), _ptr(y),
                                                                  C.byref(out)))
    return out.value


def ft_decode_graph_launch(graph, stream=None):
    return _check("ft_decode_graph_launch", lib().ft_decode_graph_launch(graph, _stream(stream)))


def ft_decode_graph_status(graph):
    return _check("ft_decode_graph_status", lib().ft_decode_graph_status(graph))


def ft_decode_graph_destroy(graph):
    return _check("ft_decode_graph_destroy", lib().ft_decode_graph_destroy(graph))


def ft_prefill_slot(ctx, layer, expert):
    return lib().ft_prefill_slot(ctx, layer, expert)


def ft_profile_enable(ctx, on=True):
    return _check("ft_profile_enable", lib().ft_profile_enable(ctx, 1 if on else 0))


def ft_profile_read(ctx):
    p = ft_profile()
    _check("ft_profile_read", lib().ft_profile_read(ctx, C.byref(p)))
    return {n: getattr(p, n) for n, _ in ft_profile._fields_}


def plan_dict(plan):
    """Plan fields as Python lists (host)."""
    n = plan.T * plan.k
    return {
        "layer": plan.layer, "U": list(plan.U[:plan.n_u]), "H": list(plan.H[:plan.n_h]),
        "M": list(plan.M[:plan.n_m]), "q": plan.q, "n_c": plan.n_c, "avail": plan.avail,
        "F_slot": list(plan.F_slot[:plan.q]), "G_slot": list(plan.G_slot[:plan.n_h + plan.q]),
        "route_slot": list(plan.route_slot[:n]), "pair_group": list(plan.pair_group[:n]),
        "idx": list(plan.idx[:n]), "gates": list(plan.gates[:n]),
    }
