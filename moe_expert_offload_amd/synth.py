"""Seeded synthetic inputs for the routed MoE layer and its decode traces.

This module is the only code shared by the HIP path's harness and the CPU
oracle.  It holds no step of the method: it draws random numbers, rounds them
to the storage formats the layer consumes (bf16), lays expert weights out as
host records, and generates routing traces.

Citations: [FT] is the paper "FreeToken: Efficient Edge-Native MoE Serving with
Bandwidth-Adaptive Execution" (arXiv 2608.16157).

Record layout (one complete (layer, expert) pair, [FT] §3 and §4.2 "Expert banks"
-- every tensor needed to evaluate one layer-expert pair sits in one record so a
cache fill is one contiguous copy): bf16 words, row-major,

    [ W_gate (d_ff x d) | W_up (d_ff x d) | W_down (d x d_ff) ]

Host pool: records indexed by the flattened id  row = l_phys * E + e  ([FT] §4.2,
banks use l*E+e as their leading dimension).  When the logical pool does not
fit host memory the pool holds L_phys < L physical layers and logical layer l
reads physical layer l mod L_phys; keys, bytes moved and timing are unchanged.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

STREAM_ROUTER = 0
STREAM_EXPERT = 1
STREAM_X = 2
STREAM_TRACE = 3


@dataclass(frozen=True)
class Shape:
    """Shape of one stack of routed MoE layers."""

    L: int
    E: int
    d: int
    d_ff: int
    k: int
    mxfp4: bool = False  # expert records in MXFP4 (else bf16)

    @property
    def record_elems(self) -> int:
        return 3 * self.d * self.d_ff

    @property
    def record_bytes(self) -> int:
        return mxfp4_record_bytes(self.d, self.d_ff) if self.mxfp4 else 2 * self.record_elems

    @property
    def pool_dtype(self):
        return np.uint8 if self.mxfp4 else np.uint16


@dataclass(frozen=True)
class Workload:
    """One synthetic workload (sizes and distributions of the pages' configurations)."""

    name: str
    seed_key: int
    shape: Shape
    T: int
    cache_rate: float  # fraction of the L*E (layer, expert) pairs the GPU cache holds
    zipf_alpha: float = 1.1
    reuse: float = 0.6
    steps: int = 512

    @property
    def n_slots(self) -> int:
        # N = floor(rate * L * E)
        return int(np.floor(self.cache_rate * self.shape.L * self.shape.E + 1e-9))


WORKLOADS = {w.name: w for w in (
    # single layer, all experts resident
    Workload("layer-d256-E8-top2", 1, Shape(1, 8, 256, 512, 2), 16, 1.0),
    # decode: 40 layers, d=2048, E=128, top-8, d_ff=768, cache at 37 %, batch 1 and 8
    Workload("decode-L40-d2048-E128-top8", 2, Shape(40, 128, 2048, 768, 8), 1, 0.37),
    Workload("decode-L40-d2048-E128-top8-b8", 2, Shape(40, 128, 2048, 768, 8), 8, 0.37),
    # decode: 43 layers, d=4096, E=256, top-6, d_ff=2048, cache at 11 %
    Workload("decode-L43-d4096-E256-top6", 3, Shape(43, 256, 4096, 2048, 6), 1, 0.11),
    # prefill: 8192-token chunk through the same 43-layer shape
    Workload("prefill8k-L43-d4096-E256-top6", 4, Shape(43, 256, 4096, 2048, 6), 8192, 0.11),
    # the 43-layer shape with MXFP4 experts: 16384-token prefill (two 8192-token chunks)
    # and batch-1 decode
    Workload("mxfp4-prefill8k-L43-d4096-E256-top6", 5, Shape(43, 256, 4096, 2048, 6, True), 8192, 0.11),
    Workload("mxfp4-decode-L43-d4096-E256-top6", 5, Shape(43, 256, 4096, 2048, 6, True), 1, 0.11),
)}


def generator(seed_key: int, stream: int, *extra: int, seed: int = 0) -> np.random.Generator:
    """PCG64 stream keyed by (workload seed key, stream, extra...) under one base seed."""
    ss = np.random.SeedSequence(entropy=seed, spawn_key=(seed_key, stream) + tuple(int(e) for e in extra))
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float values to bf16 (round to nearest, ties to even); returns uint16 words."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 words to float32 (exact)."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def router_weights(w: Workload, layer: int, seed: int = 0) -> np.ndarray:
    """W_r for one layer: bf16 words [E, d], values N(0, 0.02^2)."""
    s = w.shape
    g = generator(w.seed_key, STREAM_ROUTER, layer, seed=seed)
    return f32_to_bf16_bits(g.normal(0.0, 0.02, size=(s.E, s.d)))


def expert_record(w: Workload, layer_phys: int, expert: int, seed: int = 0) -> np.ndarray:
    """One expert record (bf16 words, layout in the module docstring), values N(0, 0.02^2)."""
    s = w.shape
    g = generator(w.seed_key, STREAM_EXPERT, layer_phys, expert, seed=seed)
    return f32_to_bf16_bits(g.normal(0.0, 0.02, size=s.record_elems))


def host_pool_numpy(w: Workload, L_phys: int, seed: int = 0) -> np.ndarray:
    """The whole host pool as uint16 [L_phys * E, record_elems] (small workloads only)."""
    s = w.shape
    pool = np.empty((L_phys * s.E, s.record_elems), dtype=np.uint16)
    for lp in range(L_phys):
        for e in range(s.E):
            pool[lp * s.E + e] = expert_record(w, lp, e, seed=seed)
    return pool


def tokens(w: Workload, step: int, layer: int, T: int | None = None, seed: int = 0) -> np.ndarray:
    """Layer input x for (step or chunk, layer): bf16 words [T, d], values N(0, 1)."""
    s = w.shape
    T = w.T if T is None else T
    g = generator(w.seed_key, STREAM_X, step, layer, seed=seed)
    return f32_to_bf16_bits(g.normal(0.0, 1.0, size=(T, s.d)))


def zipf_reuse_trace(L: int, E: int, k: int, B: int, steps: int, alpha: float, reuse: float,
                     rng: np.random.Generator) -> np.ndarray:
    """Routing trace int16 [steps, L, B, k] (expert ids ascending within a row).

    Per layer a random permutation assigns popularity ranks; rank r has weight
    (r+1)^-alpha.  Each batch stream is independent.  Step 0 draws k distinct
    experts without replacement from the popularity law; every later step keeps
    each of the previous step's k experts independently with probability
    `reuse` and draws the rest without replacement, excluding the kept ones.
    Sequential draws without replacement are taken as the top-k of
    log-weight + Gumbel noise, which has the same law.
    """
    ranks = np.stack([rng.permutation(E) for _ in range(L)])  # ranks[l, r] = expert of rank r
    logw_rank = -alpha * np.log(np.arange(1, E + 1, dtype=np.float64))
    logw = np.empty((L, E))
    logw[np.arange(L)[:, None], ranks] = logw_rank[None, :]
    out = np.empty((steps, L, B, k), dtype=np.int16)
    prev = None
    li = np.arange(L)[:, None, None]
    bi = np.arange(B)[None, :, None]
    for s in range(steps):
        key = logw[:, None, :] + rng.gumbel(size=(L, B, E))
        if prev is not None:
            keep = rng.random((L, B, k)) < reuse
            kk = np.where(keep, np.inf, key[li, bi, prev])
            key[li, bi, prev] = kk
        sel = np.argpartition(-key, k - 1, axis=2)[:, :, :k]
        sel.sort(axis=2)
        out[s] = sel.astype(np.int16)
        prev = sel
    return out


def trace_for(w: Workload, seed: int = 0, steps: int | None = None) -> np.ndarray:
    s = w.shape
    g = generator(w.seed_key, STREAM_TRACE, seed=seed)
    return zipf_reuse_trace(s.L, s.E, s.k, w.T, w.steps if steps is None else steps,
                            w.zipf_alpha, w.reuse, g)


def allowed_mask(trace_row: np.ndarray, E: int) -> np.ndarray:
    """uint8 [B, E]: 1 where the trace routes token b to expert e."""
    B = trace_row.shape[0]
    m = np.zeros((B, E), dtype=np.uint8)
    m[np.arange(B)[:, None], trace_row.astype(np.int64)] = 1
    return m


# ---- GPU-side generation for pools and activations too large for NumPy ---------
# torch's CUDA generator, seeded per chunk; values N(0, std^2) rounded to bf16 by
# torch's round-to-nearest-even conversion.  Used for the large workloads, where
# the oracle reads the same host memory afterwards.

def fill_records_torch(view, seed_key: int, seed: int = 0, std: float = 0.02, chunk_rows: int = 16):
    """Fills a uint16 [rows, record_elems] host array (pinned or not) with N(0, std^2) bf16."""
    import torch
    rows, n = view.shape
    host_t = torch.from_numpy(view.reshape(-1).view(np.int16))
    g = torch.Generator(device="cuda")
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        g.manual_seed(((seed * 1_000_003 + seed_key) * 1_000_003 + r0) & 0x7FFFFFFFFFFFFFFF)
        w = torch.randn((r1 - r0) * n, generator=g, device="cuda", dtype=torch.float32).mul_(std)
        host_t[r0 * n:r1 * n].copy_(w.to(torch.bfloat16).view(torch.int16))
    torch.cuda.synchronize()


def tokens_torch(seed_key: int, chunk: int, layer: int, T: int, d: int, seed: int = 0):
    """Layer input on the GPU: bf16 bits as an int16 CUDA tensor [T, d], values N(0, 1)."""
    import torch
    g = torch.Generator(device="cuda")
    g.manual_seed(((seed * 1_000_003 + seed_key * 7919 + chunk) * 1_000_003 + layer) & 0x7FFFFFFFFFFFFFFF)
    return torch.randn((T, d), generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16).view(torch.int16)


# ---- MXFP4 expert records --------------------------------------------------------
# Weights N(0, 0.02^2) converted to OCP MXFP4 (E2M1 elements, E8M0 scale per 32
# consecutive elements along each matrix's reduction axis; shared exponent
# floor(log2 max|v|) - 2, elements rounded to nearest even and clamped to +-6).
# Record bytes: [gate codes d_ff x d/2 | up codes d_ff x d/2 | down codes d x d_ff/2 |
# gate scales d_ff x d/32 | up scales d_ff x d/32 | down scales d x d_ff/32], the
# lower-index element of each pair in the low nibble.

# magnitudes 0 .5 1 1.5 2 3 4 6; midpoints with the tie direction of round-half-even
_E2M1_STEPS = ((0.25, False), (0.75, True), (1.25, False), (1.75, True), (2.5, False), (3.5, True), (5.0, False))


def mxfp4_record_bytes(d: int, d_ff: int) -> int:
    return 3 * d * d_ff // 2 + 3 * d * d_ff // 32


def _mx_quantize_np(w):
    """w [rows, cols] float64 -> (codes uint8 [rows, cols], scales uint8 [rows, cols/32])."""
    rows, cols = w.shape
    b = w.reshape(rows, cols // 32, 32)
    amax = np.abs(b).max(axis=2)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.clip(ex.astype(np.int64) - 1 - 2, -127, 127)
    a = np.minimum(np.abs(b) / np.exp2(e)[..., None], 6.0)
    mag = np.zeros(a.shape, np.uint8)
    for t, incl in _E2M1_STEPS:
        mag += (a >= t) if incl else (a > t)
    codes = np.where((b < 0) & (mag > 0), mag | 8, mag).astype(np.uint8)
    zero = amax == 0
    scales = np.where(zero, 0, e + 127).astype(np.uint8)
    codes[zero] = 0
    return codes.reshape(rows, cols), scales


def _pack_nibbles_np(codes):
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def mxfp4_record_from_weights(wg, wu, wd):
    """Pack float weights (W_gate [d_ff,d], W_up [d_ff,d], W_down [d,d_ff]) into an MXFP4 record."""
    parts_c, parts_s = [], []
    for w in (wg, wu, wd):
        c, sc = _mx_quantize_np(np.asarray(w, np.float64))
        parts_c.append(_pack_nibbles_np(c).reshape(-1))
        parts_s.append(sc.reshape(-1))
    return np.concatenate(parts_c + parts_s)


def mxfp4_expert_record(w: Workload, layer_phys: int, expert: int, seed: int = 0) -> np.ndarray:
    """One MXFP4 expert record (uint8), from N(0, 0.02^2) weights."""
    s = w.shape
    g = generator(w.seed_key, STREAM_EXPERT, layer_phys, expert, seed=seed)
    wg = g.normal(0.0, 0.02, size=(s.d_ff, s.d))
    wu = g.normal(0.0, 0.02, size=(s.d_ff, s.d))
    wd = g.normal(0.0, 0.02, size=(s.d, s.d_ff))
    return mxfp4_record_from_weights(wg, wu, wd)


def fill_mxfp4_records_torch(view, d: int, d_ff: int, seed_key: int, seed: int = 0, chunk_rows: int = 8):
    """Fills a uint8 [rows, record_bytes] host array with MXFP4 records of N(0, 0.02^2)
    weights generated and converted on the GPU (same conversion as above)."""
    import torch
    rows, nbytes = view.shape
    assert nbytes == mxfp4_record_bytes(d, d_ff)
    host_t = torch.from_numpy(view.reshape(-1))
    g = torch.Generator(device="cuda")

    def quant(w):  # w [n, R, C] float32 -> codes packed [n, R*C/2], scales [n, R*C/32]
        n, R, Cc = w.shape
        b = w.reshape(n, R, Cc // 32, 32)
        amax = b.abs().amax(dim=3)
        _, ex = torch.frexp(torch.where(amax > 0, amax, torch.ones_like(amax)))
        e = (ex.to(torch.int32) - 3).clamp(-127, 127)
        a = (b.abs() / torch.exp2(e.to(torch.float32)).unsqueeze(-1)).clamp(max=6.0)
        mag = torch.zeros_like(a, dtype=torch.uint8)
        for t, incl in _E2M1_STEPS:
            mag += (a >= t).to(torch.uint8) if incl else (a > t).to(torch.uint8)
        codes = torch.where((b < 0) & (mag > 0), mag | 8, mag)
        zero = amax == 0
        codes = torch.where(zero.unsqueeze(-1), torch.zeros_like(codes), codes)
        scales = torch.where(zero, torch.zeros_like(e), e + 127).to(torch.uint8)
        codes = codes.reshape(n, R, Cc)
        packed = codes[:, :, 0::2] | (codes[:, :, 1::2] << 4)
        return packed.reshape(n, -1), scales.reshape(n, -1)

    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        n = r1 - r0
        g.manual_seed(((seed * 1_000_003 + seed_key) * 1_000_003 + 7 * r0 + 1) & 0x7FFFFFFFFFFFFFFF)
        wg = torch.randn((n, d_ff, d), generator=g, device="cuda").mul_(0.02)
        wu = torch.randn((n, d_ff, d), generator=g, device="cuda").mul_(0.02)
        wd = torch.randn((n, d, d_ff), generator=g, device="cuda").mul_(0.02)
        cg, sg = quant(wg)
        cu, su = quant(wu)
        cd, sd = quant(wd)
        rec = torch.cat([cg, cu, cd, sg, su, sd], dim=1)
        host_t[r0 * nbytes:r1 * nbytes].copy_(rec.reshape(-1))
    torch.cuda.synchronize()
