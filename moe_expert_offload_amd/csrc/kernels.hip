// HIP kernels of the routed MoE layer for gfx950 (CDNA4, wavefront 64).
//
// Citations: [FT] = "FreeToken: Efficient Edge-Native MoE Serving with
// Bandwidth-Adaptive Execution" (arXiv 2608.16157).
//
//   router      fp32 logits in a fixed summation order + wavefront top-k    [FT] §3.2
//   permute     stable grouping of (token, rank) pairs by expert            (grouped evaluation, [FT] §3.2)
//   ffn rows    grouped SwiGLU FFN, row-streaming form for few tokens/expert (decode, [FT] §3.2)
//   ffn mfma    grouped SwiGLU FFN on bf16 MFMA tiles for many tokens/expert (prefill, [FT] §3.1)
//   combine     gate-weighted sum in rank order + the host partial          ([FT] §3.2 exact merge)
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <mutex>

#include "device_common.h"
#include "internal.h"

using namespace ft::dev;

namespace {

using ft::DecideArgs;
using ft::DevPlan;
using ft::plan_term;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }


// sum of the 8 products of two packed bf16x8 vectors, added into acc (any order), with
// the packed bf16 dot instruction (fp32 accumulation), no unpacking
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot8_pk(uint4 a, uint4 b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w), acc, false);
  return acc;
}

__device__ __forceinline__ float dot8_f(uint4 a, float4 h0, float4 h1, float acc) {
  acc = fmaf(bf_lo(a.x), h0.x, acc);
  acc = fmaf(bf_hi(a.x), h0.y, acc);
  acc = fmaf(bf_lo(a.y), h0.z, acc);
  acc = fmaf(bf_hi(a.y), h0.w, acc);
  acc = fmaf(bf_lo(a.z), h1.x, acc);
  acc = fmaf(bf_hi(a.z), h1.y, acc);
  acc = fmaf(bf_lo(a.w), h1.z, acc);
  acc = fmaf(bf_hi(a.w), h1.w, acc);
  return acc;
}


// ============================================================================
// Router
// ============================================================================

// Element i of a dot product belongs to lane (i mod 512) / 8; a lane adds its
// products in increasing i (chunk j = 0,1,..., then r = 0..7 inside the chunk);
// positions past d contribute +0.0 products.  The 64 lane sums are combined by
// a_l += a_(l xor o), o = 32..1.  Every fp32 step is an IEEE add of an exact
// bf16 x bf16 product, so the bits do not depend on FMA contraction.
template <int TT, int TE>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ w,
                                                            int T, int d, int E,
                                                            float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TT;
  const int e0 = (blockIdx.y * 4 + wave) * TE;
  if (e0 >= E) return;
  float acc[TT][TE];
#pragma unroll
  for (int a = 0; a < TT; ++a)
#pragma unroll
    for (int b = 0; b < TE; ++b) acc[a][b] = 0.0f;
  const int J = (d + 511) >> 9;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  for (int j = 0; j < J; ++j) {
    const int i0 = j * 512 + lane * 8;
    const bool in = i0 < d;
    uint4 xv[TT], wv[TE];
#pragma unroll
    for (int a = 0; a < TT; ++a) xv[a] = (in && t0 + a < T) ? ld16(x + (size_t)(t0 + a) * d + i0) : zero;
#pragma unroll
    for (int b = 0; b < TE; ++b) wv[b] = (in && e0 + b < E) ? ld16(w + (size_t)(e0 + b) * d + i0) : zero;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
#pragma unroll
      for (int a = 0; a < TT; ++a) {
        const uint32_t xw = (r >> 1) == 0 ? xv[a].x : (r >> 1) == 1 ? xv[a].y : (r >> 1) == 2 ? xv[a].z : xv[a].w;
        const float xf = (r & 1) ? bf_hi(xw) : bf_lo(xw);
#pragma unroll
        for (int b = 0; b < TE; ++b) {
          const uint32_t ww = (r >> 1) == 0 ? wv[b].x : (r >> 1) == 1 ? wv[b].y : (r >> 1) == 2 ? wv[b].z : wv[b].w;
          const float wf = (r & 1) ? bf_hi(ww) : bf_lo(ww);
          acc[a][b] = acc[a][b] + xf * wf;  // product exact in fp32
        }
      }
    }
  }
#pragma unroll
  for (int a = 0; a < TT; ++a)
#pragma unroll
    for (int b = 0; b < TE; ++b) {
      float v = acc[a][b];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v = v + __shfl_xor(v, o, WAVE);
      acc[a][b] = v;
    }
  if (lane == 0) {
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
      for (int b = 0; b < TE; ++b)
        if (t0 + a < T && e0 + b < E) logits[(size_t)(t0 + a) * E + e0 + b] = acc[a][b];
  }
}

// Order-preserving 64-bit key of (logit, expert): larger key = ranks first
// (logit descending, then index ascending).  -0.0 and +0.0 map to one key.
__device__ __forceinline__ unsigned long long rank_key(float v, int e) {
  uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (uint32_t)(0x7fffffff - e);
}

template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
  return ((unsigned long long)hi << 32) | lo;
}

// v from the lane DPP control CTRL names, in the rows ROWS selects; other lanes keep v
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned long long dpp_rows_u64(unsigned long long v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)v, (int)(uint32_t)v, CTRL, ROWS, 0xf, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(v >> 32), (int)(uint32_t)(v >> 32), CTRL,
                                                           ROWS, 0xf, false);
  return ((unsigned long long)hi << 32) | lo;
}

// Maximum over a wavefront whose 64 lanes are all active, all in DPP: within each
// row of 16 lanes (swap neighbours, swap pairs, mirror the half rows, mirror the
// row), then lane 15 of rows 0 and 2 into rows 1 and 3 and lane 31 into rows 2 and
// 3, which leaves the maximum in lane 63; returned to every lane.
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  unsigned long long w;
  w = dpp_u64<0xb1>(v);  // quad_perm [1,0,3,2]
  v = w > v ? w : v;
  w = dpp_u64<0x4e>(v);  // quad_perm [2,3,0,1]
  v = w > v ? w : v;
  w = dpp_u64<0x141>(v);  // row_half_mirror
  v = w > v ? w : v;
  w = dpp_u64<0x140>(v);  // row_mirror
  v = w > v ? w : v;
  w = dpp_rows_u64<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = w > v ? w : v;
  w = dpp_rows_u64<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  v = w > v ? w : v;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((unsigned long long)hi << 32) | lo;
}

// The logit a rank key was made from (zero comes back as +0, which the gate
// arithmetic cannot tell from -0).
__device__ __forceinline__ float key_logit(unsigned long long key) {
  const uint32_t u = (uint32_t)(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Top-k of one token by one wavefront: k rounds of a wave arg-max over the
// allowed experts (NS per lane), each winner removed; softmax over the k winners.
// Lanes 0..k-1 write the k ids and gates to idx/gates (global or shared memory).
// The logits are loaded together with the mask rather than behind it, and a
// wavefront with two tokens loads both before it selects.
template <int NS>
struct TopkIn {
  float v[NS];
  uint8_t ok[NS];
};

template <int NS>
__device__ __forceinline__ void topk_load(const float* __restrict__ lg, const uint8_t* __restrict__ allowed, int E,
                                          int lane, TopkIn<NS>& in) {
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int e = lane + 64 * s;
    in.v[s] = e < E ? lg[e] : 0.0f;
    in.ok[s] = e < E && (allowed == nullptr || allowed[e] != 0);
  }
}

template <int NS>
__device__ __forceinline__ void topk_pick(const TopkIn<NS>& in, int k, int lane, int32_t* idx, float* gates) {
  unsigned long long key[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) key[s] = in.ok[s] ? rank_key(in.v[s], lane + 64 * s) : 0ull;
  // winner r goes to lane r (value and expert); the largest logit is uniform
  float my_v = 0.0f, top = 0.0f;
  int my_e = -1;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if (r < k) {
      unsigned long long b = key[0];
#pragma unroll
      for (int s = 1; s < NS; ++s) b = key[s] > b ? key[s] : b;
      b = wave_max_u64(b);
      if (b != 0ull) {
        const int e = 0x7fffffff - (int)(uint32_t)(b & 0xffffffffu);
#pragma unroll
        for (int s = 0; s < NS; ++s)
          if (lane + 64 * s == e) key[s] = 0ull;
        const float v = key_logit(b);
        if (r == 0) top = v;
        if (lane == r) {
          my_v = v;
          my_e = e;
        }
      }
    }
  }
  // softmax over the k winners, one per lane, summed by a butterfly over 8 lanes
  const float z = (lane < k && my_e >= 0) ? expf(my_v - top) : 0.0f;
  float sum = z;
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) sum += __shfl_xor(sum, o, WAVE);
  if (lane < k) {
    idx[lane] = my_e;
    gates[lane] = my_e >= 0 ? z / sum : 0.0f;
  }
}

// Tokens first, first + step, ... of logits [T, E] by one wavefront, two at a time.
template <int NS>
__device__ __forceinline__ void topk_tokens_ns(const float* __restrict__ logits, const uint8_t* __restrict__ allowed,
                                               int T, int E, int k, int first, int step, int lane, int32_t* idx,
                                               float* gates) {
  for (int t = first; t < T; t += 2 * step) {
    const int t1 = t + step;
    TopkIn<NS> a, b;
    topk_load<NS>(logits + (size_t)t * E, allowed ? allowed + (size_t)t * E : nullptr, E, lane, a);
    if (t1 < T) topk_load<NS>(logits + (size_t)t1 * E, allowed ? allowed + (size_t)t1 * E : nullptr, E, lane, b);
    topk_pick<NS>(a, k, lane, idx + (size_t)t * k, gates + (size_t)t * k);
    if (t1 < T) topk_pick<NS>(b, k, lane, idx + (size_t)t1 * k, gates + (size_t)t1 * k);
  }
}

__device__ __forceinline__ void topk_tokens(const float* __restrict__ logits, const uint8_t* __restrict__ allowed,
                                            int T, int E, int k, int first, int step, int lane, int32_t* idx,
                                            float* gates) {
  if (E <= 64)
    topk_tokens_ns<1>(logits, allowed, T, E, k, first, step, lane, idx, gates);
  else if (E <= 128)
    topk_tokens_ns<2>(logits, allowed, T, E, k, first, step, lane, idx, gates);
  else if (E <= 256)
    topk_tokens_ns<4>(logits, allowed, T, E, k, first, step, lane, idx, gates);
  else if (E <= 512)
    topk_tokens_ns<8>(logits, allowed, T, E, k, first, step, lane, idx, gates);
  else
    topk_tokens_ns<16>(logits, allowed, T, E, k, first, step, lane, idx, gates);
}

__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ logits,
                                                          const uint8_t* __restrict__ allowed,
                                                          int T, int E, int k,
                                                          int32_t* __restrict__ idx,
                                                          float* __restrict__ gates) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_tokens(logits, allowed, t + 1, E, k, t, 1, lane, idx, gates);
}

// ---- device-side cache decisions ([FT] §4.1 "Device-side cache control") ----------
// Exclusive prefix sum over the 256 threads of a block; *total gets the block sum.
__device__ int block_excl_scan_256(int v, int* total) {
  __shared__ int ws[4];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o, WAVE);
    if (lane >= o) inc += t;
  }
  if (lane == 63) ws[wv] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    base += w < wv ? ws[w] : 0;
    tot += ws[w];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// q* of [FT] Eqs. (1)-(4) in Q16 with the floor and caps; the same integer rule as
// ft_qstar_split on the host.
__device__ int qstar_device(int m, uint32_t frac_q16, int min_fill, int max_fetch, int avail) {
  if (m <= 0) return 0;
  const long long fq = frac_q16, one = 65536;
  const long long lo = ((long long)m * fq) >> 16;
  const long long f0 = lo * (one - fq), h0 = (long long)(m - lo) * fq;
  const long long f1 = (lo + 1) * (one - fq), h1 = (long long)(m - lo - 1) * fq;
  const long long ms0 = f0 > h0 ? f0 : h0, ms1 = f1 > h1 ? f1 : h1;
  long long q = ms1 < ms0 ? lo + 1 : lo;
  if (q > m) q = m;
  const long long floor_fill = min_fill < m ? min_fill : m;
  if (q < floor_fill) q = floor_fill;
  if (max_fetch >= 0 && q > max_fetch) q = max_fetch;
  if (avail < 0) avail = 0;
  if (q > avail) q = avail;
  if (q < 0) q = 0;
  return (int)q;
}

// Cache state one decision reads, loaded before the top-k so that its latency
// overlaps it: the layer's row of `where` (E <= 1024: four entries per thread),
// every slot's key and stamp when n_slots <= 4096 (sixteen per thread; larger
// caches are read during the victim search), and the recency clock.
struct DecidePre {
  int32_t wh[4];
  int32_t key[16];
  long long st[16];
  long long clock;
};

__device__ __forceinline__ void decide_prefetch(const DecideArgs& a, DecidePre& pf) {
  const int tid = threadIdx.x, E = a.dc.E, base = a.layer * E, n = a.dc.n_slots;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid + 256 * j;
    pf.wh[j] = e < E ? a.dc.where[base + e] : -1;
  }
  if (n <= 4096) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int sl = tid + 256 * j;
      pf.key[j] = sl < n ? a.dc.slot_key[sl] : -1;
      pf.st[j] = sl < n ? a.dc.slot_stamp[sl] : 0;
    }
  }
  pf.clock = *a.dc.clock;
}

// Victim order (stamp asc, slot asc) as one unsigned key: stamps are >= -1 and far
// below 2^39, slots below 2^24; ~0 marks a slot that is not a candidate.
__device__ __forceinline__ unsigned long long victim_key(long long st, int sl) {
  return ((unsigned long long)(st + 1) << 24) | (unsigned long long)sl;
}

__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) {
  return ~wave_max_u64(~v);
}

// The decisions of one decode call, by the 256 threads of one block, for the P
// routed ids in s_id (shared memory): dedup in first-occurrence order, classify
// against `where`, q from the split, the q least recently used slots not holding
// a hit (by (stamp, slot)), eviction and admission, stamps of H then F in
// first-occurrence order, the slot rewrite, and the stable grouping of the pairs
// by G = H then F.  Same rule as ExpertCache::lookup.  Every decision is made in
// shared memory from the prefetched state.  Global memory is only written, and
// only after the last barrier: a barrier waits for the block's stores in flight,
// so stores issued before one would put their round trip on the critical path.
__device__ void decide_block(const DecideArgs& a, const int32_t* s_id, int P, const DecidePre& pf) {
  __shared__ int32_t s_u[FT_PLAN_CAP], s_g[FT_PLAN_CAP], s_h[FT_PLAN_CAP], s_m[FT_PLAN_CAP];
  __shared__ int32_t s_vold[FT_PLAN_CAP];
  __shared__ int32_t s_where[1024], s_first[1024], s_pos[1024];
  __shared__ unsigned long long s_best[2][4];
  __shared__ uint32_t s_hash;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int E = a.dc.E, base = a.layer * E, n_sl = a.dc.n_slots;
  DevPlan* pl = a.plan;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid + 256 * j;
    if (e < E) {
      s_where[e] = pf.wh[j];
      s_first[e] = 0x7fffffff;
      s_pos[e] = -1;
    }
  }
  if (tid == 0) s_hash = 0u;
  // a token that allows fewer than k experts leaves -1 ids: no decisions, no groups
  int bad = 0;
  for (int i = tid; i < P; i += 256) bad |= s_id[i] < 0 || s_id[i] >= E;
  if (__syncthreads_or(bad)) {
    if (tid == 0) {
      pl->n_u = -1;
      pl->n_h = 0;
      pl->n_g = 0;
      pl->q = 0;
      if (a.pub) a.pub->n_u = -1;
    }
    return;
  }
  for (int i = tid; i < P; i += 256) atomicMin(&s_first[s_id[i]], i);
  __syncthreads();
  // Calls of at most 64 pairs (every decode call of up to 8 tokens) take the
  // counting steps with ballots, one pair or one distinct expert per lane; every
  // wavefront computes the same values and wavefront 0 stores them.  Larger calls
  // take block-wide scans, two per thread.
  const bool small = P <= 64;
  const unsigned long long lt = (1ull << lane) - 1ull;
  const int i0 = small ? lane : 2 * tid, i1 = 2 * tid + 1;
  // U: first occurrences in pair order
  int n_u, ex;
  const int f0 = i0 < P && s_first[s_id[i0]] == i0, f1 = !small && i1 < P && s_first[s_id[i1]] == i1;
  if (small) {
    const unsigned long long b = __ballot(f0);
    n_u = __popcll(b);
    ex = __popcll(b & lt);
    if (f0 && wv == 0) s_u[ex] = s_id[i0];
  } else {
    ex = block_excl_scan_256(f0 + f1, &n_u);
    if (f0) s_u[ex] = s_id[i0];
    if (f1) s_u[ex + f0] = s_id[i1];
  }
  __syncthreads();
  // classify against the residency before this call; H and M keep U order
  const int u0 = small ? lane : 2 * tid, u1 = 2 * tid + 1;
  const int e0 = u0 < n_u ? s_u[u0] : 0, e1 = !small && u1 < n_u ? s_u[u1] : 0;
  const int p0 = u0 < n_u ? s_where[e0] : -1, p1 = !small && u1 < n_u ? s_where[e1] : -1;
  const int h0 = u0 < n_u && p0 >= 0, h1 = !small && u1 < n_u && p1 >= 0;
  const int m0 = u0 < n_u && !h0, m1 = !small && u1 < n_u && !h1;
  int n_h, n_m, xh, xm;
  if (small) {
    const unsigned long long bh = __ballot(h0), bm = __ballot(m0);
    n_h = __popcll(bh);
    n_m = __popcll(bm);
    xh = __popcll(bh & lt);
    xm = __popcll(bm & lt);
  } else {
    int tot;
    ex = block_excl_scan_256((h0 + h1) | ((m0 + m1) << 16), &tot);
    n_h = tot & 0xffff;
    n_m = tot >> 16;
    xh = ex & 0xffff;
    xm = ex >> 16;
  }
  if (!small || wv == 0) {
    if (h0) {
      s_h[xh] = e0;
      s_g[xh] = p0;
      s_pos[e0] = xh;  // group of a hit: its rank in H
    }
    if (h1) {
      s_h[xh + h0] = e1;
      s_g[xh + h0] = p1;
      s_pos[e1] = xh + h0;
    }
    if (m0) s_m[xm] = e0;
    if (m1) s_m[xm + m0] = e1;
  }
  const int avail = n_sl - n_h;
  const int q = qstar_device(n_m, a.fq, a.min_fill, a.max_fetch, avail);
  __syncthreads();
  // victims: q rounds of the smallest victim key above the previous pick, over the
  // slots that hold neither a hit of this call nor a prefill reservation
  const bool in_regs = n_sl <= 4096;
  unsigned long long vk[16];
  if (q > 0 && in_regs) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int sl = tid + 256 * j, key = pf.key[j];
      const bool hit = key >= base && key < base + E && s_pos[key - base] >= 0;
      vk[j] = (sl < n_sl && !hit && key != -2) ? victim_key(pf.st[j], sl) : ~0ull;
    }
  }
  unsigned long long prev = 0ull;
  for (int r = 0; r < q; ++r) {
    unsigned long long best = ~0ull;
    if (in_regs) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if ((r == 0 || vk[j] > prev) && vk[j] < best) best = vk[j];
    } else {
      for (int sl = tid; sl < n_sl; sl += 256) {
        const int key = a.dc.slot_key[sl];
        if (key == -2 || (key >= base && key < base + E && s_pos[key - base] >= 0)) continue;
        const unsigned long long v = victim_key(a.dc.slot_stamp[sl], sl);
        if ((r == 0 || v > prev) && v < best) best = v;
      }
    }
    best = wave_min_u64(best);
    if (lane == 0) s_best[r & 1][wv] = best;
    __syncthreads();
    best = s_best[r & 1][0];
#pragma unroll
    for (int w = 1; w < 4; ++w) best = s_best[r & 1][w] < best ? s_best[r & 1][w] : best;
    if (best == ~0ull) {
      // fewer candidates than q (cannot happen while q <= avail and no prefill
      // reservation exists): publish an invalid plan, change nothing
      if (tid == 0) {
        pl->n_u = -1;
        pl->n_h = 0;
        pl->n_g = 0;
        pl->q = 0;
        if (a.pub) a.pub->n_u = -1;
      }
      return;
    }
    const int bsl = (int)(best & 0xffffffull);
    // the owner of the slot records it and the key it held
    if (bsl % 256 == tid) {
      s_g[n_h + r] = bsl;
      s_vold[r] = in_regs ? pf.key[0] : a.dc.slot_key[bsl];
      if (in_regs) {
#pragma unroll
        for (int j = 1; j < 16; ++j)
          if (bsl == tid + 256 * j) s_vold[r] = pf.key[j];
      }
    }
    prev = best;
  }
  __syncthreads();
  // admission of F = M[0:q]: its group is n_h + r (in shared memory; the device
  // state is written at the end)
  for (int r = tid; r < q; r += 256) s_pos[s_m[r]] = n_h + r;
  __syncthreads();
  // stamps: H and F in first-occurrence order (written at the end)
  const int r0 = u0 < n_u && s_pos[e0] >= 0, r1 = !small && u1 < n_u && s_pos[e1] >= 0;
  int n_res;
  if (small) {
    const unsigned long long b = __ballot(r0);
    n_res = __popcll(b);
    ex = __popcll(b & lt);
  } else {
    ex = block_excl_scan_256(r0 + r1, &n_res);
  }
  const int n_g = n_h + q;
  // the host takes the same decisions from the published ids; it checks them
  // against a hash of the device's (plan_term summed over the sequence of values)
  const int n_seq = 5 + n_u + n_h + n_m + n_g + 2 * P;
  uint32_t part = 0u;
  for (int j = tid; j < n_seq; j += 256) {
    int v, r = j;
    if (r < 5) {
      v = r == 0 ? n_u : r == 1 ? n_h : r == 2 ? n_m : r == 3 ? q : avail;
    } else if ((r -= 5) < n_u) {
      v = s_u[r];
    } else if ((r -= n_u) < n_h) {
      v = s_h[r];
    } else if ((r -= n_h) < n_m) {
      v = s_m[r];
    } else if ((r -= n_m) < n_g) {
      v = s_g[r];
    } else if ((r -= n_g) < P) {
      const int g = s_pos[s_id[r]];
      v = g >= 0 ? s_g[g] : -1;
    } else {
      v = s_pos[s_id[r - P]];
    }
    part += plan_term(j, v);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o, WAVE);
  if (lane == 0) atomicAdd(&s_hash, part);
  __syncthreads();
  // ---- stores: no barrier from here on
  // eviction and admission; the keys involved are all distinct
  for (int r = tid; r < q; r += 256) {
    const int sl = s_g[n_h + r], old = s_vold[r], e = s_m[r];
    if (old >= 0) a.dc.where[old] = -1;
    a.dc.slot_key[sl] = base + e;
    a.dc.where[base + e] = sl;
  }
  if (!small || wv == 0) {
    if (r0) a.dc.slot_stamp[s_g[s_pos[e0]]] = pf.clock + ex + 1;
    if (r1) a.dc.slot_stamp[s_g[s_pos[e1]]] = pf.clock + ex + r0 + 1;
  }
  if (tid == 0) *a.dc.clock = pf.clock + n_res;
  // slot rewrite and stable grouping of the pairs by G
  if (small) {
    // lane i holds pair i: per group v, the pairs in it are ranked by ballot
    if (wv == 0) {
      const int g = lane < P ? s_pos[s_id[lane]] : -1;
      int run = 0, pos = -1;
      for (int v = 0; v < n_g; ++v) {
        const unsigned long long b = __ballot(g == v);
        if (g == v) pos = run + __popcll(b & lt);
        if (lane == 0) pl->offsets[v] = run;
        run += __popcll(b);
      }
      if (lane == 0) pl->offsets[n_g] = run;
      if (lane < P) {
        pl->pair_group[lane] = g;
        pl->route_slot[lane] = g >= 0 ? s_g[g] : -1;
        pl->inv[lane] = g >= 0 ? pos : -1;
        if (g >= 0) pl->perm[pos] = lane;
      }
    }
  } else {
    // counted directly per pair and per group
    for (int i = tid; i < P; i += 256) {
      const int g = s_pos[s_id[i]];
      pl->pair_group[i] = g;
      pl->route_slot[i] = g >= 0 ? s_g[g] : -1;
      if (g < 0) {
        pl->inv[i] = -1;
      } else {
        int pos = 0;
        for (int j = 0; j < P; ++j) {
          const int gj = s_pos[s_id[j]];
          pos += (gj >= 0 && gj < g) || (gj == g && j < i);
        }
        pl->perm[pos] = i;
        pl->inv[i] = pos;
      }
    }
    for (int g = tid; g <= n_g; g += 256) {
      int off = 0;
      for (int j = 0; j < P; ++j) {
        const int gj = s_pos[s_id[j]];
        off += gj >= 0 && gj < g;
      }
      pl->offsets[g] = off;
    }
  }
  for (int i = tid; i < n_u; i += 256) pl->U[i] = s_u[i];
  for (int i = tid; i < n_h; i += 256) pl->H[i] = s_h[i];
  for (int i = tid; i < n_m; i += 256) pl->M[i] = s_m[i];
  for (int i = tid; i < n_g; i += 256) pl->G_slot[i] = s_g[i];
  for (int i = tid; i < q; i += 256) pl->F_slot[i] = s_g[n_h + i];
  if (tid == 0) {
    pl->P = P;
    pl->n_u = n_u;
    pl->n_h = n_h;
    pl->n_m = n_m;
    pl->q = q;
    pl->n_c = n_m - q;
    pl->avail = avail;
    pl->n_g = n_g;
    pl->hash = s_hash;
    if (a.pub != nullptr) {
      a.pub->n_u = n_u;
      a.pub->q = q;
      a.pub->hash = s_hash;
    }
  }
}

// key[i] = map[idx[i]]: the group of each routed pair from a per-expert table.
__global__ __launch_bounds__(256) void remap_kernel(const int32_t* __restrict__ idx, const int32_t* __restrict__ map,
                                                    int n_map, int P, int32_t* __restrict__ key) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < P) {
    const int e = idx[i];
    key[i] = (e >= 0 && e < n_map) ? map[e] : -1;
  }
}

// ---- decode fills over PCIe ([FT] §3.2, the F set) ----------------------------------
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Copies n16 16-byte units from pinned host memory (read by the GPU over PCIe) to
// device memory, the grid's threads striding over them.
__device__ __forceinline__ void h2d_stride_copy(const u32x4_t* __restrict__ src, u32x4_t* __restrict__ dst,
                                                size_t n16) {
  const size_t step = (size_t)gridDim.x * blockDim.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += step)
    dst[i] = __builtin_nontemporal_load(src + i);
}

// The fills of one decode call: records M[0:q] of the layer (layer_base points at
// its expert 0 in the pinned pool) into slots F_slot[0:q], as the device decisions
// in `plan` chose them; nothing when the plan is invalid or q is 0.
__global__ __launch_bounds__(256) void fill_kernel(const uint8_t* __restrict__ layer_base, size_t S, int E,
                                                   uint8_t* __restrict__ slots, int n_slots,
                                                   const DevPlan* __restrict__ plan) {
  const int q = plan->n_u < 0 ? 0 : plan->q;
  if (q <= 0 || q > FT_PLAN_CAP) return;
  for (int r = 0; r < q; ++r) {
    const int e = plan->M[r], sl = plan->F_slot[r];
    if (e < 0 || e >= E || sl < 0 || sl >= n_slots) continue;
    h2d_stride_copy(reinterpret_cast<const u32x4_t*>(layer_base + (size_t)e * S),
                    reinterpret_cast<u32x4_t*>(slots + (size_t)sl * S), S / 16);
  }
}

__global__ __launch_bounds__(256) void h2d_copy_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                       size_t bytes) {
  h2d_stride_copy(reinterpret_cast<const u32x4_t*>(src), reinterpret_cast<u32x4_t*>(dst), bytes / 16);
}

constexpr int kFillBlocks = 64;  // enough reads in flight for the link; more only congest it

// Decode router in one launch.  Logits: wavefront w of block (bx, by) computes
// the TE experts from (4 bx + w) TE on for the TT tokens from by TT on, with the
// arithmetic order of router_logits_kernel (lane l owns elements (i mod 512)/8 ==
// l, adds its products in increasing i, then a butterfly), loading JB chunks of
// 512 elements per operand at once.  Several logits per wavefront keep the grid at
// a few tens of blocks: every block's arrival (a device-scope fence and atomic on
// one counter) lengthens the wait of the last one.  The last block
// to arrive (device-scope fence + ticket counter, no waiting) does the top-k of
// every token, the cache decisions when asked, copies x to pinned host memory and
// publishes there.  `ticket` is a zeroed device counter, reset by the last block.
__device__ __forceinline__ uint4 keep_if(uint4 v, bool c) {
  return make_uint4(c ? v.x : 0u, c ? v.y : 0u, c ? v.z : 0u, c ? v.w : 0u);
}

template <int TT, int TE>
__global__ __launch_bounds__(256) void router_decode_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, const uint8_t* __restrict__ allowed,
    int T, int d, int E, int k, float* __restrict__ logits, int32_t* __restrict__ idx,
    float* __restrict__ gates, unsigned int* __restrict__ ticket, int32_t* pub_idx, float* pub_gates,
    uint16_t* pub_x, uint32_t* pub_flag, uint32_t seq, DecideArgs da, int decide) {
  constexpr int JB = 40 / (TT + TE) < 8 ? 40 / (TT + TE) : 8;  // at most 40 16-byte loads in flight
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.y * TT;
  const int e0 = (blockIdx.x * 4 + wave) * TE;
  if (e0 < E) {
    float acc[TT][TE];
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
      for (int b = 0; b < TE; ++b) acc[a][b] = 0.0f;
    const int J = (d + 511) >> 9;
    for (int j0 = 0; j0 < J; j0 += JB) {
      // every load is issued unconditionally from a clamped (in-bounds) address and
      // the operands past the ends are zeroed afterwards: loads under a branch come
      // out one behind the other
      uint4 xv[JB][TT], wv[JB][TE];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const int i0 = (j0 + jj) * 512 + lane * 8;
        const bool in = j0 + jj < J && i0 < d;
        const int ic = in ? i0 : 0;
#pragma unroll
        for (int a = 0; a < TT; ++a) {
          const int ta = t0 + a < T ? t0 + a : T - 1;
          xv[jj][a] = ld16(x + (size_t)ta * d + ic);
        }
#pragma unroll
        for (int b = 0; b < TE; ++b) {
          const int eb = e0 + b < E ? e0 + b : E - 1;
          wv[jj][b] = ld16(w + (size_t)eb * d + ic);
        }
      }
      // only the positions past d need zeros (as in router_logits_kernel); the
      // logits of tokens and experts past the ends are not stored
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const bool in = j0 + jj < J && (j0 + jj) * 512 + lane * 8 < d;
#pragma unroll
        for (int a = 0; a < TT; ++a) xv[jj][a] = keep_if(xv[jj][a], in);
#pragma unroll
        for (int b = 0; b < TE; ++b) wv[jj][b] = keep_if(wv[jj][b], in);
      }
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        if (j0 + jj >= J) continue;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
#pragma unroll
          for (int a = 0; a < TT; ++a) {
            const uint32_t xw = (r >> 1) == 0 ? xv[jj][a].x : (r >> 1) == 1 ? xv[jj][a].y
                              : (r >> 1) == 2 ? xv[jj][a].z : xv[jj][a].w;
            const float xf = (r & 1) ? bf_hi(xw) : bf_lo(xw);
#pragma unroll
            for (int b = 0; b < TE; ++b) {
              const uint32_t ww = (r >> 1) == 0 ? wv[jj][b].x : (r >> 1) == 1 ? wv[jj][b].y
                                : (r >> 1) == 2 ? wv[jj][b].z : wv[jj][b].w;
              const float wf = (r & 1) ? bf_hi(ww) : bf_lo(ww);
              acc[a][b] = acc[a][b] + xf * wf;  // same order as router_logits_kernel
            }
          }
        }
      }
    }
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
      for (int b = 0; b < TE; ++b) {
        float v = acc[a][b];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) v = v + __shfl_xor(v, o, WAVE);
        if (lane == 0 && t0 + a < T && e0 + b < E) logits[(size_t)(t0 + a) * E + e0 + b] = v;
      }
  }
  __threadfence();
  __shared__ int last;
  __syncthreads();
  if (threadIdx.x == 0) last = atomicAdd(ticket, 1u) == gridDim.x * gridDim.y - 1;
  __syncthreads();
  if (!last) return;
  __threadfence();
  __shared__ int32_t s_ids[FT_PLAN_CAP];
  __shared__ float s_gates[FT_PLAN_CAP];
  // the cache state (written by earlier launches) is loaded here, not by every
  // block: all blocks reading the same few kilobytes at once slows their logits
  DecidePre pf;
  if (decide) decide_prefetch(da, pf);
  topk_tokens(logits, allowed, T, E, k, wave, 4, lane, s_ids, s_gates);
  __syncthreads();
  if (decide) decide_block(da, s_ids, T * k, pf);
  // Every store of the block's results comes after its last barrier, so their
  // round trips (the host copies' over PCIe) overlap: ids and gates, their host
  // copies, and x for the host's CPU branch.
  const int P = T * k;
  for (int i = threadIdx.x; i < P; i += 256) {
    idx[i] = s_ids[i];
    gates[i] = s_gates[i];
    if (pub_idx != nullptr) {
      pub_idx[i] = s_ids[i];
      pub_gates[i] = s_gates[i];
    }
  }
  if (pub_x != nullptr)
    for (int i = threadIdx.x * 8; i < T * d; i += 256 * 8)
      *reinterpret_cast<uint4*>(pub_x + i) = ld16(x + i);
  __threadfence_system();
  __syncthreads();
  if (threadIdx.x == 0) {
    *ticket = 0u;
    if (pub_flag != nullptr) {
      // every published value is visible before the host sees the sequence number
      __threadfence_system();
      *reinterpret_cast<volatile uint32_t*>(pub_flag) = seq;
    }
  }
}

// ============================================================================
// Permutation: stable counting sort of pair ids by group key
// ============================================================================
constexpr int PB = 256;

// Exclusive prefix sum of v over the 1024 threads of a block; returns the
// exclusive value of this thread and writes the block total to *total.
__device__ int block_exclusive_scan_1024(int v, int* total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(inc, o, WAVE);
    if (lane >= o) inc += u;
  }
  if (lane == 63) wsum[wv] = inc;
  __syncthreads();
  if (wv == 0) {
    int s = lane < 16 ? wsum[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int u = __shfl_up(s, o, WAVE);
      if (lane >= o) s += u;
    }
    if (lane < 16) wsum[lane] = s;  // inclusive per-wave totals
  }
  __syncthreads();
  const int base = wv > 0 ? wsum[wv - 1] : 0;
  *total = wsum[15];
  __syncthreads();
  return base + inc - v;
}

__global__ __launch_bounds__(PB) void perm_count_kernel(const int32_t* __restrict__ key, int P, int G,
                                                        int32_t* __restrict__ counts) {
  extern __shared__ int32_t hist[];
  for (int i = threadIdx.x; i < G; i += PB) hist[i] = 0;
  __syncthreads();
  const int p = blockIdx.x * PB + threadIdx.x;
  if (p < P) {
    const int g = key[p];
    if (g >= 0 && g < G) atomicAdd(&hist[g], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G; i += PB) counts[(size_t)blockIdx.x * G + i] = hist[i];
}

// One block of 1024 threads (G <= 1024): per-group running bases over blocks,
// then the exclusive scan of the group totals; counts[b][g] becomes the absolute
// first position of block b's pairs of group g.
__global__ __launch_bounds__(1024) void perm_scan_kernel(int nblk, int G, int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets) {
  const int g = threadIdx.x;
  int run = 0;
  if (g < G)
    for (int b = 0; b < nblk; ++b) {
      const int c = counts[(size_t)b * G + g];
      counts[(size_t)b * G + g] = run;
      run += c;
    }
  int total;
  const int base = block_exclusive_scan_1024(g < G ? run : 0, &total);
  if (g < G) {
    offsets[g] = base;
    for (int b = 0; b < nblk; ++b) counts[(size_t)b * G + g] += base;
  }
  if (g == 0) offsets[G] = total;
}

__global__ __launch_bounds__(PB) void perm_scatter_kernel(const int32_t* __restrict__ key, int P, int G,
                                                          const int32_t* __restrict__ base,
                                                          int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ inv) {
  __shared__ int32_t ks[PB];
  const int p = blockIdx.x * PB + threadIdx.x;
  int g = p < P ? key[p] : -1;
  if (g >= G) g = -1;
  ks[threadIdx.x] = g;
  __syncthreads();
  if (p >= P) return;
  if (g < 0) {
    inv[p] = -1;
    return;
  }
  int rank = 0;
  for (int q = 0; q < (int)threadIdx.x; ++q) rank += (ks[q] == g);
  const int pos = base[(size_t)blockIdx.x * G + g] + rank;
  perm[pos] = p;
  inv[p] = pos;
}

// All of the grouping in one block for P <= 1024 and G <= 1024 (decode).  key
// and gslot_src may live in pinned host memory; gslot_src (n_gslot entries) is
// copied to gslot_dst on the device for the FFN kernels.
__global__ __launch_bounds__(1024) void perm_small_kernel(const int32_t* key, int P, int G,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ perm,
                                                          int32_t* __restrict__ inv,
                                                          const int32_t* gslot_src,
                                                          int32_t* __restrict__ gslot_dst, int n_gslot) {
  __shared__ int32_t cnt[1024];
  __shared__ int32_t ks[1024];
  const int tid = threadIdx.x;
  cnt[tid] = 0;
  int g = tid < P ? key[tid] : -1;
  if (g >= G) g = -1;
  ks[tid] = g;
  if (gslot_src != nullptr && tid < n_gslot) gslot_dst[tid] = gslot_src[tid];
  __syncthreads();
  if (g >= 0) atomicAdd(&cnt[g], 1);
  __syncthreads();
  int total;
  const int base = block_exclusive_scan_1024(tid < G ? cnt[tid] : 0, &total);
  if (tid < G) {
    offsets[tid] = base;
    cnt[tid] = base;
  }
  if (tid == 0) offsets[G] = total;
  __syncthreads();
  if (tid < P) {
    if (g < 0) {
      inv[tid] = -1;
    } else {
      int rank = 0;
      for (int q = 0; q < tid; ++q) rank += (ks[q] == g);
      const int pos = cnt[g] + rank;
      perm[pos] = tid;
      inv[tid] = pos;
    }
  }
}

// ============================================================================
// Grouped SwiGLU FFN, row-streaming form (few tokens per expert)
// ============================================================================
// gate/up: one wavefront per RG row pairs (gate and up rows r .. r + RG - 1; RG = 2 for
// one token per group beyond d = 2048, where a wavefront's token row then serves twice
// the weights: 0.64 -> 0.67 of HBM peak at the 43-layer d = 4096 shape; 1 elsewhere,
// since at d = 2048 two pairs measured slower).  Lane l reads the 16-byte pieces l,
// l+64, ... of each row, so a wavefront streams 1 KB per load; the rows are held in
// registers while every token of the group is applied to them.  SX: the block stages
// the token rows of a batch in LDS once and its 4 wavefronts read them from there
// instead of each loading them from memory, a quarter of the x loads (one token per
// call: 0.68 -> 0.71 of HBM peak at d = 4096; 8 tokens: 71 -> 48 us per launch at d = 2048).
// down: one wavefront per 4 consecutive rows of W_down, read as one contiguous span
// (6 KB at d_ff = 768), each 16-byte piece added into the sum of the row it lies in;
// the group's h rows are staged in LDS once per block (64 KB at most per batch), their
// loads leaving together with the wave's first weight pieces.
// Both read the group's metadata in one round of independent loads and the record
// through a buffer resource (masked pieces read as zeros), weights before anything
// the arithmetic needs.

template <int NT, int JC, int RG = 1, bool SX = false>
__global__ __launch_bounds__(256) void ffn_gateup_rows_kernel(
    const uint16_t* __restrict__ x, int d, int d_ff, int k, const uint16_t* __restrict__ slots,
    size_t rec_elems, const int32_t* __restrict__ group_slot, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, int g_begin, int blocks_per_group, float* __restrict__ h,
    const int32_t* __restrict__ g_lo, const int32_t* __restrict__ g_hi, int one_token) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = g_begin + blockIdx.x / blocks_per_group;
  const int row0 = ((blockIdx.x % blocks_per_group) * 4 + wave) * RG;
  const int glo = g_lo != nullptr ? *g_lo : INT_MIN;
  const int ghi = g_hi != nullptr ? *g_hi : INT_MAX;
  const int slot = group_slot[g];
  const int r0 = offsets[g];
  const int r1 = offsets[g + 1];
  if (g < glo || g >= ghi || r1 <= r0) return;  // the whole block
  if (!SX && row0 >= d_ff) return;
  const int n = r1 - r0;
  const __amdgpu_buffer_rsrc_t rec = buf_rsrc(slots + (size_t)slot * rec_elems, (uint32_t)(rec_elems * 2));
  uint32_t og[RG], ou[RG];
  bool rin[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    rin[r] = row0 + r < d_ff;
    og[r] = (uint32_t)(row0 + r) * (uint32_t)d * 2u;
    ou[r] = (uint32_t)(d_ff + row0 + r) * (uint32_t)d * 2u;
  }
  const int J = (d + 511) >> 9;
  if constexpr (SX) {
    // The rows of x of a batch of up to NT tokens of the group are staged in LDS once per
    // block (their loads leave after the wavefront's first weight pieces) and its 4
    // wavefronts read them from there instead of each loading them from memory.
    extern __shared__ uint4 sxv[];  // [NT][d / 8] pieces of 8 bf16
    const int dp = d >> 3;          // pieces per row
    if constexpr (NT == 1) {
      // calls of one token (the launcher's condition): every group is one row of x,
      // which the block stages once, its loads leaving after the first weight pieces;
      // a group of more rows (the stated bound not kept) takes them one after another
      auto one_row = [&](int t) {
        const uint16_t* xrow = one_token ? x : x + (size_t)(perm[r0 + t] / k) * d;
        uint4 gw[RG][JC], uw[RG][JC];
#pragma unroll
        for (int r = 0; r < RG; ++r)
#pragma unroll
          for (int jj = 0; jj < JC; ++jj) {
            const int i0 = jj * 512 + lane * 8;
            const bool in = rin[r] && jj < J && i0 < d;
            gw[r][jj] = buf_ld16(rec, in ? og[r] + (uint32_t)i0 * 2u : kOOB);
            uw[r][jj] = buf_ld16(rec, in ? ou[r] + (uint32_t)i0 * 2u : kOOB);
          }
        const __amdgpu_buffer_rsrc_t xrs = buf_rsrc(xrow, (uint32_t)d * 2u);
        uint4 xs[4];  // d <= 8192: at most 4 pieces per thread
#pragma unroll
        for (int u = 0; u < 4; ++u) xs[u] = buf_ld16(xrs, (uint32_t)(threadIdx.x + 256 * u) * 16u);
        if (t > 0) __syncthreads();  // the previous row is no longer read
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if ((int)threadIdx.x + 256 * u < dp) sxv[threadIdx.x + 256 * u] = xs[u];
        __syncthreads();
        float ag[RG], au[RG];
#pragma unroll
        for (int r = 0; r < RG; ++r) ag[r] = au[r] = 0.0f;
        for (int j0 = 0; j0 < J; j0 += JC) {
          if (j0 > 0) {
#pragma unroll
            for (int r = 0; r < RG; ++r)
#pragma unroll
              for (int jj = 0; jj < JC; ++jj) {
                const int i0 = (j0 + jj) * 512 + lane * 8;
                const bool in = rin[r] && (j0 + jj < J) && i0 < d;
                gw[r][jj] = buf_ld16(rec, in ? og[r] + (uint32_t)i0 * 2u : kOOB);
                uw[r][jj] = buf_ld16(rec, in ? ou[r] + (uint32_t)i0 * 2u : kOOB);
              }
          }
#pragma unroll
          for (int jj = 0; jj < JC; ++jj) {
            const int i0 = (j0 + jj) * 512 + lane * 8;
            if ((j0 + jj < J) && i0 < d) {
              const uint4 xv = sxv[(j0 + jj) * 64 + lane];
#pragma unroll
              for (int r = 0; r < RG; ++r) {
                ag[r] = dot8_pk(gw[r][jj], xv, ag[r]);
                au[r] = dot8_pk(uw[r][jj], xv, au[r]);
              }
            }
          }
        }
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          const float zg = wave_sum(ag[r]);
          const float zu = wave_sum(au[r]);
          if (lane == 0 && rin[r]) h[(size_t)(r0 + t) * d_ff + row0 + r] = silu(zg) * zu;
        }
      };
      one_row(0);
      for (int t = 1; t < n; ++t) one_row(t);
      return;
    }
    constexpr int SU = 8;  // staged pieces per thread: NT * d <= 16384 elements
    for (int tb = 0; tb < n; tb += NT) {
      const int nt = min(NT, n - tb);
      uint4 gw[RG][JC], uw[RG][JC];
#pragma unroll
      for (int r = 0; r < RG; ++r)
#pragma unroll
        for (int jj = 0; jj < JC; ++jj) {
          const int i0 = jj * 512 + lane * 8;
          const bool in = rin[r] && jj < J && i0 < d;
          gw[r][jj] = buf_ld16(rec, in ? og[r] + (uint32_t)i0 * 2u : kOOB);
          uw[r][jj] = buf_ld16(rec, in ? ou[r] + (uint32_t)i0 * 2u : kOOB);
        }
      uint4 xs[SU];
#pragma unroll
      for (int u = 0; u < SU; ++u) {
        const int q = threadIdx.x + 256 * u, i = q / dp;
        const uint16_t* xrow = one_token ? x : x + (size_t)(perm[r0 + tb + min(i, nt - 1)] / k) * d;
        xs[u] = q < nt * dp ? ld16(xrow + 8 * (q - i * dp)) : make_uint4(0, 0, 0, 0);
      }
      __syncthreads();  // the previous batch's rows are no longer read
#pragma unroll
      for (int u = 0; u < SU; ++u)
        if ((int)threadIdx.x + 256 * u < nt * dp) sxv[threadIdx.x + 256 * u] = xs[u];
      __syncthreads();
      float ag[NT][RG], au[NT][RG];
#pragma unroll
      for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int r = 0; r < RG; ++r) ag[i][r] = au[i][r] = 0.0f;
      for (int j0 = 0; j0 < J; j0 += JC) {
        if (j0 > 0) {
#pragma unroll
          for (int r = 0; r < RG; ++r)
#pragma unroll
            for (int jj = 0; jj < JC; ++jj) {
              const int i0 = (j0 + jj) * 512 + lane * 8;
              const bool in = rin[r] && (j0 + jj < J) && i0 < d;
              gw[r][jj] = buf_ld16(rec, in ? og[r] + (uint32_t)i0 * 2u : kOOB);
              uw[r][jj] = buf_ld16(rec, in ? ou[r] + (uint32_t)i0 * 2u : kOOB);
            }
        }
#pragma unroll
        for (int jj = 0; jj < JC; ++jj) {
          const int i0 = (j0 + jj) * 512 + lane * 8;
          if ((j0 + jj < J) && i0 < d) {
#pragma unroll
            for (int i = 0; i < NT; ++i) {
              if (i >= nt) continue;
              const uint4 xv = sxv[i * dp + (j0 + jj) * 64 + lane];
#pragma unroll
              for (int r = 0; r < RG; ++r) {
                ag[i][r] = dot8_pk(gw[r][jj], xv, ag[i][r]);
                au[i][r] = dot8_pk(uw[r][jj], xv, au[i][r]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if (i >= nt) continue;
#pragma unroll
        for (int r = 0; r < RG; ++r) {
          const float zg = wave_sum(ag[i][r]);
          const float zu = wave_sum(au[i][r]);
          if (lane == 0 && rin[r]) h[(size_t)(r0 + tb + i) * d_ff + row0 + r] = silu(zg) * zu;
        }
      }
    }
    return;
  }
  for (int tb = 0; tb < n; tb += NT) {
    float ag[NT][RG], au[NT][RG];
    const uint16_t* xr[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        ag[i][r] = 0.0f;
        au[i][r] = 0.0f;
      }
      xr[i] = nullptr;
    }
    for (int j0 = 0; j0 < J; j0 += JC) {
      uint4 gw[RG][JC], uw[RG][JC];
#pragma unroll
      for (int r = 0; r < RG; ++r)
#pragma unroll
        for (int jj = 0; jj < JC; ++jj) {
          const int i0 = (j0 + jj) * 512 + lane * 8;
          const bool in = rin[r] && (j0 + jj < J) && i0 < d;
          gw[r][jj] = buf_ld16(rec, in ? og[r] + (uint32_t)i0 * 2u : kOOB);
          uw[r][jj] = buf_ld16(rec, in ? ou[r] + (uint32_t)i0 * 2u : kOOB);
        }
      if (j0 == 0) {  // token rows, looked up once the first weights are in flight
#pragma unroll
        for (int i = 0; i < NT; ++i)
          xr[i] = tb + i >= n ? nullptr : one_token ? x : x + (size_t)(perm[r0 + tb + i] / k) * d;
      }
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if (xr[i] == nullptr) continue;
#pragma unroll
        for (int jj = 0; jj < JC; ++jj) {
          const int i0 = (j0 + jj) * 512 + lane * 8;
          if ((j0 + jj < J) && i0 < d) {
            const uint4 xv = ld16(xr[i] + i0);
#pragma unroll
            for (int r = 0; r < RG; ++r) {
              ag[i][r] = dot8_pk(gw[r][jj], xv, ag[i][r]);
              au[i][r] = dot8_pk(uw[r][jj], xv, au[i][r]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (tb + i >= n) continue;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        const float zg = wave_sum(ag[i][r]);
        const float zu = wave_sum(au[i][r]);
        if (lane == 0 && rin[r]) h[(size_t)(r0 + tb + i) * d_ff + row0 + r] = silu(zg) * zu;
      }
    }
  }
}

template <int NT>
__global__ __launch_bounds__(256) void ffn_down_rows_kernel(
    int d, int d_ff, const uint16_t* __restrict__ slots, size_t rec_elems,
    const int32_t* __restrict__ group_slot, const int32_t* __restrict__ offsets, int g_begin,
    int blocks_per_group, const float* __restrict__ h, float* __restrict__ out, const int32_t* __restrict__ g_lo,
    const int32_t* __restrict__ g_hi) {
  constexpr int RW = 4;  // W_down rows per wavefront
  extern __shared__ float sh[];  // h rows of a batch of tokens [nt][d_ff], read by all 4 wavefronts
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = g_begin + blockIdx.x / blocks_per_group;
  const int row0 = ((blockIdx.x % blocks_per_group) * 4 + wave) * RW;
  const int glo = g_lo != nullptr ? *g_lo : INT_MIN;
  const int ghi = g_hi != nullptr ? *g_hi : INT_MAX;
  const int slot = group_slot[g];
  const int r0 = offsets[g];
  const int r1 = offsets[g + 1];
  if (g < glo || g >= ghi || r1 <= r0) return;  // the whole block: it stages h below
  const int n = r1 - r0;
  const __amdgpu_buffer_rsrc_t rec = buf_rsrc(slots + (size_t)slot * rec_elems, (uint32_t)(rec_elems * 2));
  const int span = row0 < d ? min(RW, d - row0) * d_ff : 0;  // elements of this wave's rows, contiguous
  const uint32_t base = ((uint32_t)2 * d_ff * d + (uint32_t)row0 * d_ff) * 2u;
  const int J = (span + 511) >> 9;
  const int per = min(NT, max(1, 16384 / d_ff));  // token rows per batch: at most 64 KB of h
  for (int tb = 0; tb < n; tb += per) {
    const int nt = min(per, n - tb);
    const int tot = nt * d_ff;  // floats of h in this batch
    const float* hb = h + (size_t)(r0 + tb) * d_ff;
    // The batch's first 16 KB of h (4 pieces per thread, zeros past its end) and the
    // wave's first 8 weight pieces are all requested before anything waits, h first:
    // staging h then waits for h alone, and the weights' round trip overlaps it.
    const __amdgpu_buffer_rsrc_t hrs = buf_rsrc(hb, (uint32_t)tot * 4u);
    uint4 hv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) hv[u] = buf_ld16(hrs, (uint32_t)(threadIdx.x + 256 * u) * 16u);
    uint4 wv[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int e0 = jj * 512 + lane * 8;
      wv[jj] = buf_ld16(rec, (jj < J && e0 < span) ? base + (uint32_t)e0 * 2u : kOOB);
    }
    __syncthreads();  // the previous batch's h is no longer read
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = (threadIdx.x + 256 * u) * 4;
      if (i < tot) *reinterpret_cast<uint4*>(sh + i) = hv[u];
    }
    for (int i = (threadIdx.x + 1024) * 4; i < tot; i += 256 * 4)  // batches of more than 16 KB
      *reinterpret_cast<float4*>(sh + i) = *reinterpret_cast<const float4*>(hb + i);
    __syncthreads();
    float acc[NT][RW];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int r = 0; r < RW; ++r) acc[i][r] = 0.0f;
    for (int j0 = 0; j0 < J; j0 += 8) {
      if (j0 > 0) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int e0 = (j0 + jj) * 512 + lane * 8;
          wv[jj] = buf_ld16(rec, (j0 + jj < J && e0 < span) ? base + (uint32_t)e0 * 2u : kOOB);
        }
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const int e0 = (j0 + jj) * 512 + lane * 8;
        if (j0 + jj >= J || e0 >= span) continue;
        const int rr = e0 / d_ff;  // a piece never straddles two rows (d_ff % 8 == 0)
        const int col = e0 - rr * d_ff;
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          if (i >= nt) continue;
          const float* hr = sh + i * d_ff + col;
          const float v = dot8_f(wv[jj], *reinterpret_cast<const float4*>(hr),
                                 *reinterpret_cast<const float4*>(hr + 4), 0.0f);
#pragma unroll
          for (int r = 0; r < RW; ++r) acc[i][r] += rr == r ? v : 0.0f;
        }
      }
    }
    if (span == 0) continue;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (i >= nt) continue;
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const float sum = wave_sum(acc[i][r]);
        if (lane == 0 && row0 + r < d) out[(size_t)(r0 + tb + i) * d + row0 + r] = sum;
      }
    }
  }
}

// ============================================================================
// Grouped SwiGLU FFN, MFMA tile form (many tokens per expert)
// ============================================================================
// v_mfma_f32_32x32x16_bf16 lane layout (checked on gfx950): lane l supplies
// A[l%32][(l/32)*8 .. +7] and B^T[l%32][(l/32)*8 .. +7]; accumulator element v
// of lane l is C[(v/4)*8 + (l/32)*4 + v%4][l%32].
//
// Block: 256 threads = 4 waves, one per SIMD.  One pass covers up to 256 rows of
// one expert (8 row subtiles of 32; the usual ~200 tokens of an 8k chunk in one
// pass) and 256 weight rows ("B columns"), 64 per wave: every weight element is
// read from HBM once per pass.  Both operands go straight from memory into LDS
// (`buffer_load ... lds`, 16 bytes per lane, no registers in between).  K runs in
// stages of 32 elements.  Token rows go through 4 buffers ([256][32] bf16, 16 KB), the
// loads of stage s + 3 in flight while stage s multiplies.  Weights go through 3
// buffers of double stages ([256][64] bf16, 32 KB): each weight row is read 128 bytes
// at a time, since a stream of 64-byte pieces of many rows reaches only ~4.5 TB/s
// where 128-byte pieces reach ~6.3 TB/s (probe at one block per compute unit); half a
// double stage is issued per stage, two to four stages ahead.  160 KB of LDS in all.
// In a buffer, 16-byte piece p of row r sits at piece p ^ swz(r), so the 8 or 16
// lanes of one LDS read phase hit as many different bank groups.  Inside a stage,
// MFMA slice i (0, 1) takes in lane group g the elements 16i + 8g .. +7.
//
// The loop's loads are issued by inline asm and waited for by one explicit
// `s_waitcnt vmcnt` per stage: the compiler's own waits drain every load at the
// loop head and before any LDS read that follows an LDS-direct load.  The 8 loads
// of a stage go out one after each MFMA pair, so their issue overlaps the MFMAs
// instead of stalling the wavefront in front of them.
constexpr int XM = 256;                 // rows per pass
constexpr int XK = 32;                  // K elements per stage
constexpr int XNB = 4;                  // token-row buffers
constexpr int XB = XM * XK;             // one token-row buffer, bf16 elements (16 KB)
constexpr int WK = 64;                  // K elements per weight double stage (128 bytes of a row)
constexpr int WNB = 3;                  // weight double-stage buffers
constexpr int WB = XM * WK;             // one weight buffer, bf16 elements (32 KB)

typedef __attribute__((address_space(3))) uint16_t lds_u16;

// Physical position of 16-byte piece p of token-row buffer row r: p ^ swz(r).  A read
// phase of 8 lanes (rows r..r+7, 32 banks) or of 16 lanes (rows r..r+15, 64 banks)
// then touches 8 or 16 different bank groups.
__device__ __forceinline__ int lds_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }
// The same for the 8 pieces of a weight buffer row (128 bytes).
__device__ __forceinline__ int lds_swz_w(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ bf16x8_t lds_frag(const uint16_t* buf, int r, int piece) {
  const uint4 u = *reinterpret_cast<const uint4*>(buf + r * XK + ((piece ^ lds_swz(r)) * 8));
  return __builtin_bit_cast(bf16x8_t, u);
}
__device__ __forceinline__ bf16x8_t lds_frag_w(const uint16_t* buf, int r, int piece) {
  const uint4 u = *reinterpret_cast<const uint4*>(buf + r * WK + ((piece ^ lds_swz_w(r)) * 8));
  return __builtin_bit_cast(bf16x8_t, u);
}


// Token rows: load q (0..3) of wave w covers buffer rows 16 (4w + q) + lane/4, physical
// piece lane%4.  Weights: load u (0..7) of wave w covers buffer rows 64w + 8u + lane/8,
// physical piece lane%8.  The lane's source piece is the logical one stored there.
__device__ __forceinline__ int lds_load_row(int wave, int q, int lane) { return 16 * (4 * wave + q) + (lane >> 2); }
__device__ __forceinline__ int lds_load_piece(int r, int lane) { return (lane & 3) ^ lds_swz(r); }
__device__ __forceinline__ int lds_wload_row(int wave, int u, int lane) { return 64 * wave + 8 * u + (lane >> 3); }
__device__ __forceinline__ int lds_wload_piece(int r, int lane) { return (lane & 7) ^ lds_swz_w(r); }

// acc[a][c] += A(row subtile a) x B(column subtile c of this wave) over one stage; the
// stage's weights are half `half` (K elements 32 half .. +31) of a weight buffer.
// Slice 1's operands are read from LDS while slice 0 multiplies; `issue(t)` sends
// load t (0..7) of a later stage after the t-th MFMA pair.
template <int NSUB, typename F>
__device__ __forceinline__ void mfma_stage_bf16(f32x16_t (&acc)[8][2], const uint16_t* sa, const uint16_t* sb,
                                                int half, int wave, int lane, F&& issue) {
  const int m = lane & 31, g = lane >> 5;
  const int pb = 4 * half + g;
  bf16x8_t fa[2][NSUB], fb[2][2];
  fb[0][0] = lds_frag_w(sb, wave * 64 + m, pb);
  fb[0][1] = lds_frag_w(sb, wave * 64 + 32 + m, pb);
#pragma unroll
  for (int a = 0; a < NSUB; ++a) fa[0][a] = lds_frag(sa, a * 32 + m, g);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int a = 0; a < NSUB; ++a) {
      acc[a][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i][a], fb[i][0], acc[a][0], 0, 0, 0);
      acc[a][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i][a], fb[i][1], acc[a][1], 0, 0, 0);
      if (i == 0) {
        if (a == 0) {
          fb[1][0] = lds_frag_w(sb, wave * 64 + m, pb + 2);
          fb[1][1] = lds_frag_w(sb, wave * 64 + 32 + m, pb + 2);
        }
        fa[1][a] = lds_frag(sa, a * 32 + m, 2 + g);
        __builtin_amdgcn_sched_barrier(0);  // keep these reads here, ahead of slice 1
      }
      const int t = i * NSUB + a;
      if (t < 8) issue(t);
    }
  }
  if (2 * NSUB < 8) {
#pragma unroll
    for (int t = 2 * NSUB; t < 8; ++t) issue(t);
  }
}

// The grid is persistent: a block takes logical blocks b, b + grid, b + 2 grid, ...
// (in the XCD-aware order, so the tiles running on one XCD at a time belong to few
// experts and share its L2), each split into passes of up to XM rows; a pass is one
// "item".  The loads go out three stages ahead (token rows) and two to four stages
// ahead (weights) across item boundaries, so the first stages of the next item are in
// flight while the current one finishes and runs its epilogue.
struct MfmaArgs {
  const uint16_t* x;       // gate/up: token rows [T][d]
  const uint16_t* h;       // down: h rows [n_rows][d_ff] in perm order
  const uint16_t* slots;
  const int32_t* group_slot;
  const int32_t* offsets;
  const int32_t* perm;
  uint16_t* h_out;         // gate/up output
  float* out;              // down output
  size_t rec_elems;
  int T, n_rows, d, d_ff, k, g_begin, n_tiles, n_blocks;
};

struct MfmaItem {
  int g, n0, r0, m0, rows, nsub;
  __amdgpu_buffer_rsrc_t rw;  // the group's weight rows
  uint32_t roff[4], woff[8];  // this lane's load offsets (bytes, K position 0)
};

// Advances (i, m0) over this block's passes and sets up the next item; false at the end.
template <bool DOWN>
__device__ __forceinline__ bool next_item(const MfmaArgs& A, int& i, int& m0, MfmaItem& it, int wave, int lane) {
  const int tile = DOWN ? 256 : 128;
  for (;;) {
    const int hb = blockIdx.x + i * gridDim.x;
    if (hb >= A.n_blocks) return false;
    const int lb = xcd_logical_block(hb, A.n_blocks);
    const int g = A.g_begin + lb / A.n_tiles;
    const int r0 = A.offsets[g];
    const int n = A.offsets[g + 1] - r0;
    if (m0 >= n) {  // this logical block is done (or empty): the next one
      ++i;
      m0 = 0;
      continue;
    }
    it.g = g;
    it.n0 = (lb % A.n_tiles) * tile;
    it.r0 = r0;
    it.m0 = m0;
    it.rows = min(XM, n - m0);
    it.nsub = (it.rows + 31) >> 5;
    const uint16_t* rec = A.slots + (size_t)A.group_slot[g] * A.rec_elems;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = lds_load_row(wave, q, lane), rr = min(r, it.rows - 1);  // rows past the end load a valid row
      it.roff[q] = DOWN ? (uint32_t)((size_t)(r0 + m0 + rr) * A.d_ff + lds_load_piece(r, lane) * 8) * 2u
                        : (uint32_t)((size_t)(A.perm[r0 + m0 + rr] / A.k) * A.d + lds_load_piece(r, lane) * 8) * 2u;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int bc = lds_wload_row(wave, u, lane);
      if (DOWN)  // B column bc is output column n0 + bc
        it.woff[u] = (uint32_t)((size_t)(it.n0 + bc) * A.d_ff + lds_wload_piece(bc, lane) * 8) * 2u;
      else {  // B column bc: wave bc/64, gate or up (bc/32)&1, column bc%32
        const int wrow = ((bc >> 5) & 1) * A.d_ff + it.n0 + (bc >> 6) * 32 + (bc & 31);
        it.woff[u] = (uint32_t)((size_t)wrow * A.d + lds_wload_piece(bc, lane) * 8) * 2u;
      }
    }
    it.rw = DOWN ? buf_rsrc(rec + (size_t)2 * A.d_ff * A.d, (uint32_t)((size_t)A.d * A.d_ff * 2))
                 : buf_rsrc(rec, (uint32_t)((size_t)2 * A.d * A.d_ff * 2));
    m0 += XM;
    return true;
  }
}

// Writes one item's results from the accumulators.
template <bool DOWN>
__device__ __forceinline__ void mfma_epilogue(const MfmaArgs& A, const MfmaItem& it, const f32x16_t (&acc)[8][2],
                                              int wave, int lane) {
  int g4 = (lane >> 5) * 4;
  asm volatile("" : "+v"(g4));  // keeps the row indices below out of the loop
  if (DOWN) {  // wave w: columns n0 + 64w .. +63
    const int col = it.n0 + wave * 64 + (lane & 31);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      if (a >= it.nsub) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = a * 32 + (v >> 2) * 8 + g4 + (v & 3);
        if (row < it.rows) {
          float* o = A.out + (size_t)(it.r0 + it.m0 + row) * A.d + col;
          o[0] = acc[a][0][v];
          o[32] = acc[a][1][v];
        }
      }
    }
  } else {  // wave w: columns n0 + 32w .. +31 of both W_gate and W_up
    const int col = it.n0 + wave * 32 + (lane & 31);
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      if (a >= it.nsub) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = a * 32 + (v >> 2) * 8 + g4 + (v & 3);
        if (row < it.rows)
          A.h_out[(size_t)(it.r0 + it.m0 + row) * A.d_ff + col] =
              f32_to_bf16_rne(silu_fast(acc[a][0][v]) * acc[a][1][v]);
      }
    }
  }
}

// Token-row load q of stage st of item it into buffer st % XNB (lx: this wave's part).
__device__ __forceinline__ void mfma_load_x(__amdgpu_buffer_rsrc_t rx, const MfmaItem& it, int st, int q,
                                            uint32_t klast, uint32_t lx) {
  const uint32_t kbyte = min((uint32_t)st * (uint32_t)(XK * 2), klast);
  lds_load16(rx, it.roff[q], kbyte, lx + (uint32_t)((st % XNB) * XB * 2 + q * 1024));
}

// Weight load u of double stage ds of item it into weight buffer `slot` (lw: this
// wave's part).
__device__ __forceinline__ void mfma_load_w(const MfmaItem& it, int ds, int u, uint32_t klast, uint32_t lw,
                                            int slot) {
  const uint32_t kbyte = min((uint32_t)ds * (uint32_t)(WK * 2), klast);
  lds_load16(it.rw, it.woff[u], kbyte, lw + (uint32_t)(slot * WB * 2 + u * 1024));
}

__device__ __forceinline__ int mod3(int v) { return v % 3; }

// The K loop of one item (kdim a multiple of 128, so every item starts in token-row
// buffer 0; weight double stage ds sits in buffer (wbase + ds) % 3, wbase carried from
// item to item).  Stage s issues the token rows of stage s + 3 and half s % 2 of the
// weights of double stage s / 2 + 2, of this item or, past its end, of the next one
// (re-reading this item's last stage when there is none).  At the top of stage s its
// own loads (rows issued at s - 3, weights at or before s - 3) are older than the 16
// of the two stages before it.  Anything else the compiler issues in between only adds
// newer operations, which keeps the count safe.
template <int NSUB>
__device__ __forceinline__ void mfma_item_bf16(f32x16_t (&acc)[8][2], __amdgpu_buffer_rsrc_t rx, const MfmaItem& cur,
                                               const MfmaItem& nxt, bool has_nxt, uint16_t* sx, uint16_t* sw,
                                               int kdim, int wave, int lane, uint32_t lx, uint32_t lw, int wbase) {
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      acc[a][0][v] = 0.0f;
      acc[a][1][v] = 0.0f;
    }
  const int nst = kdim / XK, nds = kdim / WK;
  const uint32_t klast_x = (uint32_t)(kdim - XK) * 2u, klast_w = (uint32_t)(kdim - WK) * 2u;
  for (int s0 = 0; s0 < nst; s0 += XNB) {
#pragma unroll
    for (int j = 0; j < XNB; ++j) {
      const int st = s0 + j;
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"((XNB - 2) * 8) : "memory");
      __syncthreads();  // every wave's loads of this stage have landed; stage s - 1 is done
      const int sn = st + XNB - 1;
      const bool x_cur = sn < nst || !has_nxt;
      const MfmaItem& xi = x_cur ? cur : nxt;
      const int xs = x_cur ? sn : sn - nst;
      const int dn = (st >> 1) + 2, wh = st & 1;
      const bool w_cur = dn < nds || !has_nxt;
      const MfmaItem& wi = w_cur ? cur : nxt;
      const int wd = w_cur ? dn : dn - nds;
      const int wslot = mod3(wbase + dn);
      mfma_stage_bf16<NSUB>(acc, sx + j * XB, sw + mod3(wbase + (st >> 1)) * WB, wh, wave, lane, [&](int t) {
        if (t < 4)
          mfma_load_x(rx, xi, xs, t, klast_x, lx);
        else
          mfma_load_w(wi, wd, 4 * wh + (t - 4), klast_w, lw, wslot);
      });
    }
  }
}

template <bool DOWN>
__device__ __forceinline__ void mfma_persistent(const MfmaArgs& A, uint16_t* sx, uint16_t* sw) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kdim = DOWN ? A.d_ff : A.d;
  const __amdgpu_buffer_rsrc_t rx = DOWN ? buf_rsrc(A.h, (uint32_t)((size_t)A.n_rows * A.d_ff * 2))
                                         : buf_rsrc(A.x, (uint32_t)((size_t)A.T * A.d * 2));
  int ci = 0, cm = 0;  // cursor over this block's passes
  MfmaItem cur, nxt;
  if (!next_item<DOWN>(A, ci, cm, cur, wave, lane)) return;  // block-uniform
  bool has_nxt = next_item<DOWN>(A, ci, cm, nxt, wave, lane);
  const uint32_t lx = (uint32_t)(uintptr_t)(lds_u16*)sx + (uint32_t)(4 * wave * 1024);
  const uint32_t lw = (uint32_t)(uintptr_t)(lds_u16*)sw + (uint32_t)(8 * wave * 1024);
  const uint32_t klast_x = (uint32_t)(kdim - XK) * 2u, klast_w = (uint32_t)(kdim - WK) * 2u;
  // the loads stages -4 .. -1 would have issued, in the same order: weights of double
  // stages 0 and 1 (in halves), token rows of stages 0, 1, 2
#pragma unroll
  for (int u = 0; u < 4; ++u) mfma_load_w(cur, 0, u, klast_w, lw, 0);
#pragma unroll
  for (int j = 0; j < 3; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) mfma_load_x(rx, cur, j, q, klast_x, lx);
    const int ds = (j + 1) >> 1, h = (j + 1) & 1;  // (0, 1), (1, 0), (1, 1)
#pragma unroll
    for (int u = 0; u < 4; ++u) mfma_load_w(cur, ds, 4 * h + u, klast_w, lw, ds);
  }
  int wbase = 0;
  const int nds = kdim / WK;
  for (;;) {
    f32x16_t acc[8][2];
    switch (cur.nsub) {
      case 1: mfma_item_bf16<1>(acc, rx, cur, nxt, has_nxt, sx, sw, kdim, wave, lane, lx, lw, wbase); break;
      case 2: mfma_item_bf16<2>(acc, rx, cur, nxt, has_nxt, sx, sw, kdim, wave, lane, lx, lw, wbase); break;
      case 3: mfma_item_bf16<3>(acc, rx, cur, nxt, has_nxt, sx, sw, kdim, wave, lane, lx, lw, wbase); break;
      case 4: mfma_item_bf16<4>(acc, rx, cur, nxt, has_nxt, sx, sw, kdim, wave, lane, lx, lw, wbase); break;
      case 5: mfma_item_bf16<5>(acc, rx, cur, nxt, has_nxt, sx, sw, kdim, wave, lane, lx, lw, wbase); break;
      case 6: mfma_item_bf16<6>(acc, rx, cur, nxt, has_nxt, sx, sw, kdim, wave, lane, lx, lw, wbase); break;
      case 7: mfma_item_bf16<7>(acc, rx, cur, nxt, has_nxt, sx, sw, kdim, wave, lane, lx, lw, wbase); break;
      default: mfma_item_bf16<8>(acc, rx, cur, nxt, has_nxt, sx, sw, kdim, wave, lane, lx, lw, wbase); break;
    }
    mfma_epilogue<DOWN>(A, cur, acc, wave, lane);  // the next item's first stages are in flight
    if (!has_nxt) break;
    cur = nxt;
    has_nxt = next_item<DOWN>(A, ci, cm, nxt, wave, lane);
    wbase = mod3(wbase + nds);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // no LDS load is left in flight when the block ends
}

// h[i][c] = silu(sum_k x[t_i][k] Wg[c][k]) * (sum_k x[t_i][k] Wu[c][k]) for the 128
// columns c of each strip (wave w: columns n0 + 32w .. +31 of both W_gate and W_up,
// B columns 64w .. +31 and 64w + 32 .. +63 of the weight buffer), h in bf16.
__global__ __launch_bounds__(256) void ffn_gateup_mfma_kernel(MfmaArgs A) {
  __shared__ __attribute__((aligned(1024))) uint16_t sX[XNB * XB];
  __shared__ __attribute__((aligned(1024))) uint16_t sW[WNB * WB];
  mfma_persistent<false>(A, sX, sW);
}

// out[i][c] = sum_r h[i][r] Wd[c][r] for the 256 columns of each strip (wave w:
// columns n0 + 64w .. +63), h rows in perm order.
__global__ __launch_bounds__(256) void ffn_down_mfma_kernel(MfmaArgs A) {
  __shared__ __attribute__((aligned(1024))) uint16_t sX[XNB * XB];
  __shared__ __attribute__((aligned(1024))) uint16_t sW[WNB * WB];
  mfma_persistent<true>(A, sX, sW);
}

// ============================================================================
// Combine: y[t] = sum_j (in rank order) g[t,j] out[inv[t,j]] + cpu_partial[t]
// ============================================================================
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ out,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ gates,
                                                      const float* __restrict__ cpu, int T, int k,
                                                      int d, float* __restrict__ y) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (t >= T || c >= d) return;
  // every load first (k <= 8): the pairs' positions and gates, then their rows and the
  // host partial, so the call waits for memory once; then the sum in rank order
  int pos[8];
  float g[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    pos[j] = j < k ? inv[(size_t)t * k + j] : -1;
    g[j] = j < k ? gates[(size_t)t * k + j] : 0.0f;
  }
  float4 o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    o[j] = pos[j] >= 0 ? *reinterpret_cast<const float4*>(out + (size_t)pos[j] * d + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  const float4 p = cpu != nullptr ? *reinterpret_cast<const float4*>(cpu + (size_t)t * d + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (pos[j] < 0) continue;
    acc.x = fmaf(g[j], o[j].x, acc.x);
    acc.y = fmaf(g[j], o[j].y, acc.y);
    acc.z = fmaf(g[j], o[j].z, acc.z);
    acc.w = fmaf(g[j], o[j].w, acc.w);
  }
  if (cpu != nullptr) {
    acc.x += p.x;
    acc.y += p.y;
    acc.z += p.z;
    acc.w += p.w;
  }
  *reinterpret_cast<float4*>(y + (size_t)t * d + c) = acc;
}


}  // namespace

namespace ft {

int launch_router(const uint16_t* x, const uint16_t* w, const uint8_t* allowed, int T, int d,
                  int E, int k, int32_t* idx, float* gates, float* logits_ws, void* stream) {
  if (T < 0 || d <= 0 || d % 8 != 0 || E <= 0 || E > 1024 || k < 1 || k > 8 || k > E)
    return fail(FT_EINVAL, "router: need d%8==0, 1<=k<=min(E,8), E<=1024");
  if (T == 0) return FT_OK;
  if (!x || !w || !idx || !gates || !logits_ws || !aligned16(x) || !aligned16(w))
    return fail(FT_EINVAL, "router: null or unaligned pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T >= 64) {
    dim3 grid((T + 7) / 8, (E + 31) / 32);
    router_logits_kernel<8, 8><<<grid, 256, 0, s>>>(x, w, T, d, E, logits_ws);
  } else {
    dim3 grid(T, (E + 15) / 16);
    router_logits_kernel<1, 4><<<grid, 256, 0, s>>>(x, w, T, d, E, logits_ws);
  }
  if (int rc = launched("router_logits")) return rc;
  router_topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits_ws, allowed, T, E, k, idx, gates);
  return launched("router_topk");
}

int launch_remap(const int32_t* idx, const int32_t* map, int n_map, int P, int32_t* key, void* stream) {
  if (P < 0 || n_map < 1 || !idx || !map || !key) return fail(FT_EINVAL, "remap: bad argument");
  if (P == 0) return FT_OK;
  remap_kernel<<<(P + 255) / 256, 256, 0, static_cast<hipStream_t>(stream)>>>(idx, map, n_map, P, key);
  return launched("remap");
}

int launch_fill(const uint8_t* layer_base, size_t S, int E, uint8_t* slots, int n_slots, const DevPlan* plan,
                void* stream) {
  if (!layer_base || !slots || !plan || S == 0 || S % 16 || E <= 0 || n_slots < 0)
    return fail(FT_EINVAL, "fill: bad argument");
  if ((reinterpret_cast<uintptr_t>(layer_base) | reinterpret_cast<uintptr_t>(slots)) & 15)
    return fail(FT_EINVAL, "fill: unaligned pointer");
  fill_kernel<<<kFillBlocks, 256, 0, static_cast<hipStream_t>(stream)>>>(layer_base, S, E, slots, n_slots, plan);
  return launched("fill");
}

int launch_h2d_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes % 16 || ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15))
    return fail(FT_EINVAL, "h2d_copy: need 16-byte aligned pointers and sizes");
  if (bytes == 0) return FT_OK;
  h2d_copy_kernel<<<kFillBlocks, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint8_t*>(src), static_cast<uint8_t*>(dst), bytes);
  return launched("h2d_copy");
}

int launch_router_decode(const uint16_t* x, const uint16_t* w, const uint8_t* allowed, int T, int d,
                         int E, int k, float* logits_ws, int32_t* idx, float* gates,
                         unsigned int* ticket, int32_t* pub_idx, float* pub_gates, uint16_t* pub_x,
                         uint32_t* pub_flag, uint32_t seq, void* stream, const DecideArgs* da) {
  if (T < 1 || T > 64 || d <= 0 || d % 8 != 0 || E <= 0 || E > 1024 || k < 1 || k > 8 || k > E)
    return fail(FT_EINVAL, "router: need T<=64, d%8==0, 1<=k<=min(E,8), E<=1024");
  if (!aligned16(x) || !aligned16(w) || (pub_x && !aligned16(pub_x)))
    return fail(FT_EINVAL, "router: unaligned pointer");
  if (da && (T * k > FT_PLAN_CAP || !da->plan || !da->dc.where || da->dc.n_slots >= (1 << 24) ||
             (da->dc.n_slots > 0 && (!da->dc.slot_key || !da->dc.slot_stamp))))
    return fail(FT_EINVAL, "router: bad decision arguments");
  DecideArgs none{};
  const DecideArgs dargs = da ? *da : none;
  const int dec = da ? 1 : 0;
  // tokens per wavefront: all of them up to 8.  Experts per wavefront: more of them
  // means fewer blocks to wait for at the ticket but longer logits per block; the
  // choice measured best at E = 128 and 256 (one token: 2 per wavefront, 16 or 32
  // blocks; eight tokens: 1 per wavefront, 32 blocks at E = 128)
  const int tt = T == 1 ? 1 : T <= 4 ? 4 : 8;
  const int te = T == 1 ? (E <= 64 ? 1 : E <= 256 ? 2 : 4) : (E <= 128 ? 1 : E <= 256 ? 2 : 4);
  const dim3 grid((E + 4 * te - 1) / (4 * te), (T + tt - 1) / tt);
  hipStream_t s = static_cast<hipStream_t>(stream);
#define FT_ROUTER_DECODE(TT_, TE_)                                                                                 \
  router_decode_kernel<TT_, TE_><<<grid, 256, 0, s>>>(x, w, allowed, T, d, E, k, logits_ws, idx, gates, ticket, \
                                                       pub_idx, pub_gates, pub_x, pub_flag, seq, dargs, dec)
  if (tt == 1) {
    if (te == 1) FT_ROUTER_DECODE(1, 1); else if (te == 2) FT_ROUTER_DECODE(1, 2); else FT_ROUTER_DECODE(1, 4);
  } else if (tt == 4) {
    if (te == 1) FT_ROUTER_DECODE(4, 1); else if (te == 2) FT_ROUTER_DECODE(4, 2); else FT_ROUTER_DECODE(4, 4);
  } else {
    if (te == 1) FT_ROUTER_DECODE(8, 1); else if (te == 2) FT_ROUTER_DECODE(8, 2); else FT_ROUTER_DECODE(8, 4);
  }
#undef FT_ROUTER_DECODE
  return launched("router_decode");
}

size_t permute_ws_bytes(int P, int n_groups) {
  const size_t nblk = (size_t)((P + PB - 1) / PB);
  return (nblk > 0 ? nblk : 1) * (size_t)(n_groups > 0 ? n_groups : 1) * sizeof(int32_t);
}

int launch_permute(const int32_t* key, int P, int n_groups, int32_t* offsets, int32_t* perm,
                   int32_t* inv, void* ws, size_t ws_bytes, void* stream, const int32_t* gslot_src,
                   int32_t* gslot_dst, int n_gslot) {
  if (P < 0 || n_groups < 1 || n_groups > 1024) return fail(FT_EINVAL, "permute: need 1<=n_groups<=1024");
  if (n_gslot < 0 || n_gslot > 1024 || (n_gslot > 0 && (!gslot_src || !gslot_dst)))
    return fail(FT_EINVAL, "permute: bad group-slot copy");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (P <= 1024) {
    perm_small_kernel<<<1, 1024, 0, s>>>(key, P, n_groups, offsets, perm, inv, n_gslot > 0 ? gslot_src : nullptr,
                                         gslot_dst, n_gslot);
    return launched("perm_small");
  }
  if (ws_bytes < permute_ws_bytes(P, n_groups)) return fail(FT_ENOMEM, "permute: workspace too small");
  if (n_gslot > 0) {
    if (hipMemcpyAsync(gslot_dst, gslot_src, (size_t)n_gslot * 4, hipMemcpyDefault, s) != hipSuccess)
      return fail(FT_EHIP, "permute: group-slot copy failed");
  }
  const int nblk = (P + PB - 1) / PB;
  int32_t* counts = static_cast<int32_t*>(ws);
  perm_count_kernel<<<nblk, PB, n_groups * sizeof(int32_t), s>>>(key, P, n_groups, counts);
  if (int rc = launched("perm_count")) return rc;
  perm_scan_kernel<<<1, 1024, 0, s>>>(nblk, n_groups, counts, offsets);
  if (int rc = launched("perm_scan")) return rc;
  perm_scatter_kernel<<<nblk, PB, 0, s>>>(key, P, n_groups, counts, perm, inv);
  return launched("perm_scatter");
}

// Launches a kernel with dynamic shared memory; with timing events, start/stop
// bracket the kernel itself.
int launch_ffn_rows(const uint16_t* x, int d, int d_ff, int k, const uint16_t* slots,
                    const int32_t* group_slot, const int32_t* offsets, const int32_t* perm,
                    int g_begin, int g_end, int max_rows, float* h, float* out, void* stream,
                    void* const* ev, const int32_t* g_lo, const int32_t* g_hi, int one_token) {
  if (d <= 0 || d_ff <= 0 || d % 8 || d_ff % 8 || k < 1) return fail(FT_EINVAL, "ffn_rows: bad shape");
  const int ng = g_end - g_begin;
  if (ng <= 0) return FT_OK;
  if (!aligned16(x) || !aligned16(slots) || !aligned16(h) || !aligned16(out))
    return fail(FT_EINVAL, "ffn_rows: unaligned pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t rec_elems = (size_t)3 * d * d_ff;
  if ((size_t)rec_elems * 2 >= ((size_t)1 << 31)) return fail(FT_EINVAL, "ffn_rows: record over 2 GiB");
  if (d_ff > 16384) return fail(FT_EINVAL, "ffn_rows: need d_ff <= 16384");
  const int bpg_up = (d_ff + 3) / 4;
  const int bpg_dn = (d + 15) / 16;
  const int nt = max_rows <= 1 ? 1 : max_rows <= 2 ? 2 : max_rows <= 4 ? 4 : 8;
  // the token rows of a batch staged in LDS once per block: in calls of one token (every
  // group is its row) up to d = 8192, else while a batch's rows fit 32 KB
  const bool one_row = one_token && d <= 8192;
#define FT_GU_ROWS(NT_, JC_, RG_, SX_, BPG_, SHM_)                                                    \
  timed_launch_shm(ffn_gateup_rows_kernel<NT_, JC_, RG_, SX_>, dim3(ng * (BPG_)), dim3(256), (SHM_), s, ev, 0, \
                   x, d, d_ff, k, slots, rec_elems, group_slot, offsets, perm, g_begin, (BPG_), h, g_lo, g_hi, \
                   one_token)
#define FT_ROWS_LAUNCH(NT)                                                                          \
  if constexpr (NT == 1) {                                                                          \
    if (one_row && d > 2048) FT_GU_ROWS(1, 4, 2, true, (d_ff + 7) / 8, (size_t)d * 2);             \
    else if (one_row) FT_GU_ROWS(1, 4, 1, true, bpg_up, (size_t)d * 2);                             \
    else if (d > 2048) FT_GU_ROWS(1, 4, 2, false, (d_ff + 7) / 8, 0);                               \
    else FT_GU_ROWS(1, 4, 1, false, bpg_up, 0);                                                     \
  } else {                                                                                          \
    if (NT * d <= 16384 && d <= 2048) FT_GU_ROWS(NT, 4, 1, true, bpg_up, (size_t)NT * d * 2);      \
    else if (NT * d <= 16384) FT_GU_ROWS(NT, 8, 1, true, bpg_up, (size_t)NT * d * 2);               \
    else if (d <= 2048) FT_GU_ROWS(NT, 4, 1, false, bpg_up, 0);                                     \
    else FT_GU_ROWS(NT, 8, 1, false, bpg_up, 0);                                                    \
  }                                                                                                 \
  if (int rc = launched("ffn_gateup_rows")) return rc;                                              \
  timed_launch_shm(ffn_down_rows_kernel<NT>, dim3(ng * bpg_dn), dim3(256),                         \
                   (size_t)std::min(NT, std::max(1, 16384 / d_ff)) * d_ff * 4, s, ev, 1, d, d_ff, slots, \
                   rec_elems, group_slot, offsets, g_begin, bpg_dn, (const float*)h, out, g_lo, g_hi);   \
  return launched("ffn_down_rows");
  switch (nt) {
    case 1: { FT_ROWS_LAUNCH(1) }
    case 2: { FT_ROWS_LAUNCH(2) }
    case 4: { FT_ROWS_LAUNCH(4) }
    default: { FT_ROWS_LAUNCH(8) }
  }
#undef FT_ROWS_LAUNCH
#undef FT_GU_ROWS
}

int launch_ffn_mfma(const uint16_t* x, int T, int d, int d_ff, int k, const uint16_t* slots,
                    const int32_t* group_slot, const int32_t* offsets, const int32_t* perm,
                    int g_begin, int g_end, int n_rows, uint16_t* h, float* out,
                    void* stream, void* const* ev) {
  if (d % 256 != 0 || d_ff % 128 != 0 || k < 1 || T < 0 || n_rows < 0)
    return fail(FT_EINVAL, "ffn_mfma: need d%256==0 and d_ff%128==0");
  const int ng = g_end - g_begin;
  if (ng <= 0) return FT_OK;
  if (!aligned16(x) || !aligned16(slots) || !aligned16(h) || !aligned16(out))
    return fail(FT_EINVAL, "ffn_mfma: unaligned pointer");
  // the kernels address x, h and a record through 32-bit buffer offsets
  const size_t lim = (size_t)1 << 31;
  if ((size_t)T * d * 2 >= lim || (size_t)n_rows * d_ff * 2 >= lim || (size_t)3 * d * d_ff * 2 >= lim)
    return fail(FT_EINVAL, "ffn_mfma: x, h or a record over 2 GiB");
  // one block per compute unit (160 KB of LDS each), a multiple of the 8 XCDs
  static int n_cu = 0;
  if (n_cu <= 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
      n_cu = 256;
  }
  auto grid_for = [&](int nb) { return nb <= n_cu ? nb : (n_cu / 8) * 8; };
  hipStream_t s = static_cast<hipStream_t>(stream);
  MfmaArgs A{};
  A.x = x;
  A.h = h;
  A.slots = slots;
  A.group_slot = group_slot;
  A.offsets = offsets;
  A.perm = perm;
  A.h_out = h;
  A.out = out;
  A.rec_elems = (size_t)3 * d * d_ff;
  A.T = T;
  A.n_rows = n_rows;
  A.d = d;
  A.d_ff = d_ff;
  A.k = k;
  A.g_begin = g_begin;
  A.n_tiles = d_ff / 128;
  A.n_blocks = ng * A.n_tiles;
  timed_launch(ffn_gateup_mfma_kernel, dim3(grid_for(A.n_blocks)), dim3(256), s, ev, 0, A);
  if (int rc = launched("ffn_gateup_mfma")) return rc;
  A.n_tiles = d / 256;
  A.n_blocks = ng * A.n_tiles;
  timed_launch(ffn_down_mfma_kernel, dim3(grid_for(A.n_blocks)), dim3(256), s, ev, 1, A);
  return launched("ffn_down_mfma");
}

int launch_combine(const float* out, const int32_t* inv, const float* gates,
                   const float* cpu_partial, int T, int k, int d, float* y, void* stream) {
  if (T < 0 || k < 1 || k > 8 || d <= 0 || d % 4 != 0) return fail(FT_EINVAL, "combine: bad shape (1 <= k <= 8, d % 4 == 0)");
  if (T == 0) return FT_OK;
  if (T > 65535) return fail(FT_EINVAL, "combine: T > 65535");
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid((d / 4 + 255) / 256, T);
  combine_kernel<<<grid, 256, 0, s>>>(out, inv, gates, cpu_partial, T, k, d, y);
  return launched("combine");
}

}  // namespace ft

// ============================================================================
// Grouping without allocation
// ============================================================================
// ft_permute_noalloc: ft_permute with its per-block group counts in a fixed
// device array instead of a caller workspace.  Each GPU the library runs on
// holds its own copy of the array until the process ends; host code reaches it
// only through the address hipGetSymbolAddress returns on that device (the
// array's name is a host-side stand-in, not a device address).
namespace {

constexpr size_t kNoAllocScratchBytes = size_t(1) << 20;  // P <= 65536 pairs at any n_groups <= 1024
constexpr int kMaxDevices = 64;
static __device__ __align__(256) int32_t scratch[kNoAllocScratchBytes / sizeof(int32_t)];

std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device with that
// device current; null with the error set on failure.
void* scratch_for_current_device() {
  int dev = -1;
  const hipError_t ge = hipGetDevice(&dev);
  if (ge != hipSuccess) {
    ft::set_error(std::string("permute_noalloc: hipGetDevice: ") + hipGetErrorString(ge));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    ft::set_error("permute_noalloc: device index beyond the library's table");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      ft::set_error(std::string("permute_noalloc: hipGetSymbolAddress: ") + hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_dev[dev] = ptr;
  }
  return g_scratch_dev[dev];
}

}  // namespace

extern "C" {

size_t ft_permute_noalloc_max_scratch_bytes(void) { return kNoAllocScratchBytes; }

int ft_permute_noalloc(const int32_t* key, int32_t P, int32_t n_groups, int32_t* offsets, int32_t* perm,
                       int32_t* inv, void* stream) {
  if (P < 0 || n_groups < 1 || n_groups > 1024) return ft::fail(FT_EINVAL, "permute_noalloc: need P >= 0 and 1<=n_groups<=1024");
  if ((P > 0 && (!key || !perm || !inv)) || !offsets) return ft::fail(FT_EINVAL, "permute_noalloc: null pointer");
  const size_t need = ft::permute_ws_bytes(P, n_groups);
  if (need > kNoAllocScratchBytes)
    return ft::fail(FT_EINVAL, "permute_noalloc: P and n_groups need " + std::to_string(need) +
                                   " bytes of scratch, more than its fixed " +
                                   std::to_string(kNoAllocScratchBytes));
  void* ws = scratch_for_current_device();
  if (!ws) return FT_EHIP;
  return ft::launch_permute(key, P, n_groups, offsets, perm, inv, ws, kNoAllocScratchBytes, stream);
}

}  // extern "C"
