// MXFP4 experts on gfx950: row-streaming decode kernels with in-register E2M1
// dequantisation, MXFP8 activation quantisation, and the grouped SwiGLU FFN on
// the scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 activations x E2M1
// weights, one E8M0 scale per lane per operand).
//
// [FT] = "FreeToken: Efficient Edge-Native MoE Serving with Bandwidth-Adaptive
// Execution" (arXiv 2608.16157): §5.1 the experts are natively MXFP4; §4.1 the
// kernels dequantise in place.  Formats follow OCP Microscaling Formats v1.0.
//
// Record (bytes): [gate codes d_ff x d/2 | up codes d_ff x d/2 | down codes d x d_ff/2 |
// gate scales d_ff x d/32 | up scales d_ff x d/32 | down scales d x d_ff/32], two
// E2M1 codes per byte with the lower-index element in the low nibble; a weight
// block is 32 consecutive elements of a row (one 16-byte piece of codes).
//
// Scaled-MFMA operand layout of the mixed E4M3 x E2M1 form (checked on gfx950):
// the E2M1 operand (weights, B) takes in lane group g = l/32 the 32 elements
// k = 32g .. 32g+31 of its 64-element K step (16 bytes, low nibble first); the
// E4M3 operand (activations, A) takes in lane group g the elements {16g .. 16g+15}
// (bytes 0..15) and {32+16g .. 32+16g+15} (bytes 16..31).  The E8M0 scale a lane
// group g passes, for either operand, multiplies the elements k = 32g .. 32g+31,
// whichever lane holds them: both operands use blocks of 32 consecutive elements.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cmath>

#include "internal.h"

namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// E2M1 code (4 bits) -> fp32: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1(uint32_t c) {
  const uint32_t m = c & 7u;
  const uint32_t bits = m >= 2u ? ((m << 22) + (126u << 23)) : (m == 1u ? 0x3f000000u : 0u);
  return __uint_as_float(bits | ((c & 8u) << 28));
}

// 2^(s - 127) for an E8M0 byte (s < 255).
__device__ __forceinline__ float e8m0(uint32_t s) { return s ? __uint_as_float(s << 23) : 1.17549435e-38f * 0.5f; }

// sum over the 32 elements of one weight block (16 code bytes) times 32 bf16 activations
__device__ __forceinline__ float block_dot_bf16(uint4 codes, const uint16_t* __restrict__ xb) {
  const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 xv = *reinterpret_cast<const uint4*>(xb + 8 * q);  // 8 bf16 = elements 8q..8q+7
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int b = 0; b < 4; ++b) {  // code byte b of word q -> elements 8q+2b, 8q+2b+1
      const uint32_t byte = (cw[q] >> (8 * b)) & 0xffu;
      acc = fmaf(e2m1(byte & 0xfu), bf_lo(xw[b]), acc);
      acc = fmaf(e2m1(byte >> 4), bf_hi(xw[b]), acc);
    }
  }
  return acc;
}

__device__ __forceinline__ float block_dot_f32(uint4 codes, const float* __restrict__ hb) {
  const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 h0 = *reinterpret_cast<const float4*>(hb + 8 * q);
    const float4 h1 = *reinterpret_cast<const float4*>(hb + 8 * q + 4);
    const float hv[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint32_t byte = (cw[q] >> (8 * b)) & 0xffu;
      acc = fmaf(e2m1(byte & 0xfu), hv[2 * b], acc);
      acc = fmaf(e2m1(byte >> 4), hv[2 * b + 1], acc);
    }
  }
  return acc;
}

struct MxRec {
  size_t g_codes, u_codes, d_codes, g_sc, u_sc, d_sc, bytes;
};
__device__ __host__ inline MxRec mx_rec(int d, int d_ff) {
  MxRec r;
  const size_t c = (size_t)d * d_ff / 2, s = (size_t)d * d_ff / 32;
  r.g_codes = 0;
  r.u_codes = c;
  r.d_codes = 2 * c;
  r.g_sc = 3 * c;
  r.u_sc = 3 * c + s;
  r.d_sc = 3 * c + 2 * s;
  r.bytes = 3 * c + 3 * s;
  return r;
}

// ---- decode: one wavefront per weight row, lane l takes blocks l, l+64, ... ----
template <int NT>
__global__ __launch_bounds__(256) void mx_gateup_rows_kernel(
    const uint16_t* __restrict__ x, int d, int d_ff, int k, const uint8_t* __restrict__ slots,
    const int32_t* __restrict__ group_slot, const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
    int g_begin, int blocks_per_group, float* __restrict__ h) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = g_begin + blockIdx.x / blocks_per_group;
  const int row = (blockIdx.x % blocks_per_group) * 4 + wave;
  if (row >= d_ff) return;
  const int r0 = offsets[g];
  const int n = offsets[g + 1] - r0;
  if (n <= 0) return;
  const MxRec R = mx_rec(d, d_ff);
  const uint8_t* rec = slots + (size_t)group_slot[g] * R.bytes;
  const uint8_t* gc = rec + R.g_codes + (size_t)row * (d / 2);
  const uint8_t* uc = rec + R.u_codes + (size_t)row * (d / 2);
  const uint8_t* gs = rec + R.g_sc + (size_t)row * (d / 32);
  const uint8_t* us = rec + R.u_sc + (size_t)row * (d / 32);
  const int nb = d / 32;  // blocks per row
  for (int tb = 0; tb < n; tb += NT) {
    float ag[NT], au[NT];
    const uint16_t* xr[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      ag[i] = 0.0f;
      au[i] = 0.0f;
      xr[i] = (tb + i < n) ? x + (size_t)(perm[r0 + tb + i] / k) * d : nullptr;
    }
    for (int b = lane; b < nb; b += 64) {
      const uint4 cgv = *reinterpret_cast<const uint4*>(gc + 16 * b);
      const uint4 cuv = *reinterpret_cast<const uint4*>(uc + 16 * b);
      const float sg = e8m0(gs[b]), su = e8m0(us[b]);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if (xr[i] == nullptr) continue;
        ag[i] = fmaf(block_dot_bf16(cgv, xr[i] + 32 * b), sg, ag[i]);
        au[i] = fmaf(block_dot_bf16(cuv, xr[i] + 32 * b), su, au[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (tb + i >= n) continue;
      const float zg = wave_sum(ag[i]);
      const float zu = wave_sum(au[i]);
      if (lane == 0) h[(size_t)(r0 + tb + i) * d_ff + row] = silu(zg) * zu;
    }
  }
}

template <int NT>
__global__ __launch_bounds__(256) void mx_down_rows_kernel(
    int d, int d_ff, const uint8_t* __restrict__ slots, const int32_t* __restrict__ group_slot,
    const int32_t* __restrict__ offsets, int g_begin, int blocks_per_group, const float* __restrict__ h,
    float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = g_begin + blockIdx.x / blocks_per_group;
  const int row = (blockIdx.x % blocks_per_group) * 4 + wave;
  if (row >= d) return;
  const int r0 = offsets[g];
  const int n = offsets[g + 1] - r0;
  if (n <= 0) return;
  const MxRec R = mx_rec(d, d_ff);
  const uint8_t* rec = slots + (size_t)group_slot[g] * R.bytes;
  const uint8_t* dc = rec + R.d_codes + (size_t)row * (d_ff / 2);
  const uint8_t* ds = rec + R.d_sc + (size_t)row * (d_ff / 32);
  const int nb = d_ff / 32;
  for (int tb = 0; tb < n; tb += NT) {
    float acc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] = 0.0f;
    for (int b = lane; b < nb; b += 64) {
      const uint4 cv = *reinterpret_cast<const uint4*>(dc + 16 * b);
      const float sc = e8m0(ds[b]);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if (tb + i >= n) continue;
        acc[i] = fmaf(block_dot_f32(cv, h + (size_t)(r0 + tb + i) * d_ff + 32 * b), sc, acc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (tb + i >= n) continue;
      const float s = wave_sum(acc[i]);
      if (lane == 0) out[(size_t)(r0 + tb + i) * d + row] = s;
    }
  }
}

// ---- MXFP8 (E4M3) activation quantisation ----------------------------------------
// value -> E4M3 code (round half to even, |v| clamped to 448 first)
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: subnormal steps of 2^-9
    code = (uint32_t)rintf(a * 512.0f);  // 0..8 (8 is the smallest normal, code 0x08)
  } else {
    uint32_t u = __float_as_uint(a);
    const uint32_t lsb = (u >> 20) & 1u;
    u += 0x7ffffu + lsb;  // round the 23-bit mantissa to 3 bits, ties to even
    const int e = (int)(u >> 23) - 127;
    code = (uint32_t)((e + 7) << 3) | ((u >> 20) & 7u);
    if (code > 0x7eu) code = 0x7eu;
  }
  return code == 0u ? 0u : (code | sign);
}

// One thread per activation block of 32 consecutive elements.  Scale
// X = 2^(floor(log2 amax) - 8) (OCP MX conversion for E4M3).
template <typename In>
__device__ __forceinline__ float ld_act(const In* p);
template <>
__device__ __forceinline__ float ld_act<uint16_t>(const uint16_t* p) { return __uint_as_float((uint32_t)(*p) << 16); }
template <>
__device__ __forceinline__ float ld_act<float>(const float* p) { return *p; }

template <typename In>
__global__ __launch_bounds__(256) void mx_quant_act_kernel(const In* __restrict__ in, int rows, int n,
                                                           const int32_t* __restrict__ row_of, int k_div,
                                                           uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  const int nblk = n / 32;
  const long long id = (long long)blockIdx.x * 256 + threadIdx.x;
  if (id >= (long long)rows * nblk) return;
  const int r = (int)(id / nblk), b = (int)(id % nblk);
  const size_t src_row = row_of ? (size_t)(row_of[r] / k_div) : (size_t)r;
  const In* src = in + src_row * n + 32 * b;
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = ld_act<In>(src + i);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  uint32_t s = 0;
  float inv = 0.0f;
  if (amax > 0.0f) {
    int e2;
    (void)frexpf(amax, &e2);  // amax = m 2^e2, m in [0.5, 1): floor(log2 amax) = e2 - 1
    int e = e2 - 1 - 8;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    s = (uint32_t)(e + 127);
    inv = ldexpf(1.0f, -e);
  }
  uint32_t packed[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    packed[w] = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) packed[w] |= (amax > 0.0f ? e4m3_code(v[4 * w + j] * inv) : 0u) << (8 * j);
  }
  uint4* dst = reinterpret_cast<uint4*>(q + (size_t)r * n + 32 * b);
  dst[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  dst[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
  sc[(size_t)r * nblk + b] = (uint8_t)s;
}

// ---- scaled-MFMA grouped FFN ---------------------------------------------------------
// Tile: up to 256 rows of one expert x a column tile; 8 waves (4 along M x 2 along N);
// K staged in steps of 128 (two MFMA steps) through LDS with register prefetch.
constexpr int MTBM = 256;
constexpr int MKB = 128;            // K elements per stage
constexpr int ALD = MKB + 16;       // LDS bytes per A row (fp8, padded)
constexpr int BLD = MKB / 2 + 16;   // LDS bytes per B row (fp4, padded)

__device__ __forceinline__ int xcd_logical_block(int b, int nb) {
  const int q = nb >> 3, r = nb & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

__device__ __forceinline__ v8i_t a_frag(const uint8_t* row, int ks, int grp) {
  // bytes {64ks + 16g .. +15} and {64ks + 32 + 16g .. +15} of the staged row
  const uint4 lo = *reinterpret_cast<const uint4*>(row + 64 * ks + 16 * grp);
  const uint4 hi = *reinterpret_cast<const uint4*>(row + 64 * ks + 32 + 16 * grp);
  v8i_t r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

__device__ __forceinline__ v8i_t b_frag(const uint8_t* row, int ks, int grp) {
  // 32 E2M1 codes = 16 bytes at K element 64ks + 32g
  const uint4 v = *reinterpret_cast<const uint4*>(row + 32 * ks + 16 * grp);
  v8i_t r;
  r[0] = (int)v.x; r[1] = (int)v.y; r[2] = (int)v.z; r[3] = (int)v.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

// h[i][n0 + c] = silu(x_i . Wg[n0+c]) * (x_i . Wu[n0+c]) with x in MXFP8 (xq, xs) and
// W in MXFP4; 64 columns per block (each N-wave 32 gate + the same 32 up columns).
__global__ __launch_bounds__(512) void mx_gateup_mfma_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, int d, int d_ff, int k,
    const uint8_t* __restrict__ slots, const int32_t* __restrict__ group_slot,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm, int g_begin, int n_tiles, int n_blocks,
    float* __restrict__ h) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[MTBM * ALD];
  __shared__ __attribute__((aligned(16))) uint8_t sB[128 * BLD];
  __shared__ uint32_t sAs[MTBM];   // 4 activation scales per row per stage
  __shared__ uint32_t sBs[128];    // 4 weight scales per row per stage
  const int lb = xcd_logical_block(blockIdx.x, n_blocks);
  const int g = g_begin + lb / n_tiles;
  const int n0 = (lb % n_tiles) * 64;
  const int r0 = offsets[g];
  const int n = offsets[g + 1] - r0;
  if (n <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const MxRec R = mx_rec(d, d_ff);
  const uint8_t* rec = slots + (size_t)group_slot[g] * R.bytes;
  // B: 128 rows (0..63 gate, 64..127 up) x 64 code bytes per stage: one 16-byte piece per thread
  const int brow = tid >> 2, bq = tid & 3;
  const uint8_t* bcode = rec + (brow < 64 ? R.g_codes + (size_t)(n0 + brow) * (d / 2)
                                          : R.u_codes + (size_t)(n0 + brow - 64) * (d / 2)) + 16 * bq;
  const uint8_t* bsc = rec + (brow < 64 ? R.g_sc + (size_t)(n0 + brow) * (d / 32)
                                        : R.u_sc + (size_t)(n0 + brow - 64) * (d / 32));
  for (int m0 = 0; m0 < n; m0 += MTBM) {
    // A: 256 rows x 128 bytes per stage: four 16-byte pieces per thread (rows tid/8 + 64 i)
    const uint8_t* arow[4];
    const uint8_t* asrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 64 * i;
      const bool in = m0 + r < n;
      const size_t xr = in ? (size_t)(perm[r0 + m0 + r] / k) : 0;
      arow[i] = in ? xq + xr * d + 16 * (tid & 7) : nullptr;
      asrow[i] = in ? xs + xr * (d / 32) : nullptr;
    }
    const bool wave_active = (m0 + wm * 64) < n;
    f32x16_t acc[4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][v] = 0.0f;
    const uint4 zero = make_uint4(0, 0, 0, 0);
    uint4 pa[4], pb;
    uint32_t pas = 0, pbs = 0;
    auto load_stage = [&](int k0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pa[i] = arow[i] ? *reinterpret_cast<const uint4*>(arow[i] + k0) : zero;
      pb = *reinterpret_cast<const uint4*>(bcode + k0 / 2);
      // scales: threads 0..255 fetch 4 activation scales of row tid, 256..383 the weight scales
      if (tid < 256) {
        const int r = tid;
        const bool in = m0 + r < n;
        pas = in ? *reinterpret_cast<const uint32_t*>(xs + (size_t)(perm[r0 + m0 + r] / k) * (d / 32) + k0 / 32) : 0u;
      } else if (tid < 384) {
        const int r = tid - 256;
        const uint8_t* sp = rec + (r < 64 ? R.g_sc + (size_t)(n0 + r) * (d / 32) : R.u_sc + (size_t)(n0 + r - 64) * (d / 32));
        pbs = *reinterpret_cast<const uint32_t*>(sp + k0 / 32);
      }
    };
    (void)asrow;
    (void)bsc;
    load_stage(0);
    for (int k0 = 0; k0 < d; k0 += MKB) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&sA[((tid >> 3) + 64 * i) * ALD + 16 * (tid & 7)]) = pa[i];
      *reinterpret_cast<uint4*>(&sB[brow * BLD + 16 * bq]) = pb;
      if (tid < 256) sAs[tid] = pas;
      else if (tid < 384) sBs[tid - 256] = pbs;
      __syncthreads();
      if (k0 + MKB < d) load_stage(k0 + MKB);
      if (wave_active) {
        const int grp = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int ra0 = wm * 64 + (lane & 31), ra1 = ra0 + 32;
          const int rbg = wn * 32 + (lane & 31), rbu = 64 + rbg;
          const v8i_t a0 = a_frag(&sA[ra0 * ALD], ks, grp);
          const v8i_t a1 = a_frag(&sA[ra1 * ALD], ks, grp);
          const v8i_t bg = b_frag(&sB[rbg * BLD], ks, grp);
          const v8i_t bu = b_frag(&sB[rbu * BLD], ks, grp);
          const int sh = 8 * (2 * ks + grp);
          const int sa0 = (sAs[ra0] >> sh) & 0xff, sa1 = (sAs[ra1] >> sh) & 0xff;
          const int sbg = (sBs[rbg] >> sh) & 0xff, sbu = (sBs[rbu] >> sh) & 0xff;
          acc[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, bg, acc[0], 0, 4, 0, sa0, 0, sbg);
          acc[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, bg, acc[1], 0, 4, 0, sa1, 0, sbg);
          acc[2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, bu, acc[2], 0, 4, 0, sa0, 0, sbu);
          acc[3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, bu, acc[3], 0, 4, 0, sa1, 0, sbu);
        }
      }
    }
    if (wave_active) {
      const int col = n0 + wn * 32 + (lane & 31);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wm * 64 + mb * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
          if (row < n) h[(size_t)(r0 + row) * d_ff + col] = silu(acc[mb][v]) * acc[2 + mb][v];
        }
    }
  }
}

// out[i][n0 + c] = hq_i . Wd[n0+c] with h in MXFP8 (rows in perm order) and W in MXFP4;
// 128 columns per block (each N-wave 64).
__global__ __launch_bounds__(512) void mx_down_mfma_kernel(
    const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs, int d, int d_ff,
    const uint8_t* __restrict__ slots, const int32_t* __restrict__ group_slot,
    const int32_t* __restrict__ offsets, int g_begin, int n_tiles, int n_blocks, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[MTBM * ALD];
  __shared__ __attribute__((aligned(16))) uint8_t sB[128 * BLD];
  __shared__ uint32_t sAs[MTBM];
  __shared__ uint32_t sBs[128];
  const int lb = xcd_logical_block(blockIdx.x, n_blocks);
  const int g = g_begin + lb / n_tiles;
  const int n0 = (lb % n_tiles) * 128;
  const int r0 = offsets[g];
  const int n = offsets[g + 1] - r0;
  if (n <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
  const MxRec R = mx_rec(d, d_ff);
  const uint8_t* rec = slots + (size_t)group_slot[g] * R.bytes;
  const int brow = tid >> 2, bq = tid & 3;
  const uint8_t* bcode = rec + R.d_codes + (size_t)(n0 + brow) * (d_ff / 2) + 16 * bq;
  for (int m0 = 0; m0 < n; m0 += MTBM) {
    const uint8_t* arow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 64 * i;
      arow[i] = (m0 + r < n) ? hq + (size_t)(r0 + m0 + r) * d_ff + 16 * (tid & 7) : nullptr;
    }
    const bool wave_active = (m0 + wm * 64) < n;
    f32x16_t acc[4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][v] = 0.0f;
    const uint4 zero = make_uint4(0, 0, 0, 0);
    uint4 pa[4], pb;
    uint32_t pas = 0, pbs = 0;
    auto load_stage = [&](int k0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) pa[i] = arow[i] ? *reinterpret_cast<const uint4*>(arow[i] + k0) : zero;
      pb = *reinterpret_cast<const uint4*>(bcode + k0 / 2);
      if (tid < 256) {
        const int r = tid;
        pas = (m0 + r < n) ? *reinterpret_cast<const uint32_t*>(hs + (size_t)(r0 + m0 + r) * (d_ff / 32) + k0 / 32) : 0u;
      } else if (tid < 384) {
        const int r = tid - 256;
        pbs = *reinterpret_cast<const uint32_t*>(rec + R.d_sc + (size_t)(n0 + r) * (d_ff / 32) + k0 / 32);
      }
    };
    load_stage(0);
    for (int k0 = 0; k0 < d_ff; k0 += MKB) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(&sA[((tid >> 3) + 64 * i) * ALD + 16 * (tid & 7)]) = pa[i];
      *reinterpret_cast<uint4*>(&sB[brow * BLD + 16 * bq]) = pb;
      if (tid < 256) sAs[tid] = pas;
      else if (tid < 384) sBs[tid - 256] = pbs;
      __syncthreads();
      if (k0 + MKB < d_ff) load_stage(k0 + MKB);
      if (wave_active) {
        const int grp = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int ra0 = wm * 64 + (lane & 31), ra1 = ra0 + 32;
          const int rb0 = wn * 64 + (lane & 31), rb1 = rb0 + 32;
          const v8i_t a0 = a_frag(&sA[ra0 * ALD], ks, grp);
          const v8i_t a1 = a_frag(&sA[ra1 * ALD], ks, grp);
          const v8i_t b0 = b_frag(&sB[rb0 * BLD], ks, grp);
          const v8i_t b1 = b_frag(&sB[rb1 * BLD], ks, grp);
          const int sh = 8 * (2 * ks + grp);
          const int sa0 = (sAs[ra0] >> sh) & 0xff, sa1 = (sAs[ra1] >> sh) & 0xff;
          const int sb0 = (sBs[rb0] >> sh) & 0xff, sb1 = (sBs[rb1] >> sh) & 0xff;
          acc[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b0, acc[0], 0, 4, 0, sa0, 0, sb0);
          acc[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b0, acc[1], 0, 4, 0, sa1, 0, sb0);
          acc[2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a0, b1, acc[2], 0, 4, 0, sa0, 0, sb1);
          acc[3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a1, b1, acc[3], 0, 4, 0, sa1, 0, sb1);
        }
      }
    }
    if (wave_active) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int col = n0 + wn * 64 + nb * 32 + (lane & 31);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int row = m0 + wm * 64 + mb * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
            if (row < n) out[(size_t)(r0 + row) * d + col] = acc[nb * 2 + mb][v];
          }
      }
    }
  }
}

inline int launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return ft::fail(FT_EHIP, std::string(what) + ": " + hipGetErrorString(e));
  return FT_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename... KArgs, typename... Args>
inline void timed_launch(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t s, void* const* ev, int which,
                         Args... args) {
  if (ev) {
    hipExtLaunchKernelGGL(kern, grid, block, 0, s, static_cast<hipEvent_t>(ev[2 * which]),
                          static_cast<hipEvent_t>(ev[2 * which + 1]), 0, args...);
  } else {
    hipLaunchKernelGGL(kern, grid, block, 0, s, args...);
  }
}

}  // namespace

namespace ft {

size_t mx_record_bytes(int d, int d_ff) { return mx_rec(d, d_ff).bytes; }

int launch_mx_ffn_rows(const uint16_t* x, int d, int d_ff, int k, const uint8_t* slots, const int32_t* group_slot,
                       const int32_t* offsets, const int32_t* perm, int g_begin, int g_end, int max_rows, float* h,
                       float* out, void* stream, void* const* ev) {
  if (d % 64 || d_ff % 64 || k < 1) return fail(FT_EINVAL, "mx_ffn_rows: need d%64==0 and d_ff%64==0");
  const int ng = g_end - g_begin;
  if (ng <= 0) return FT_OK;
  if (!aligned16(x) || !aligned16(slots) || !aligned16(h) || !aligned16(out))
    return fail(FT_EINVAL, "mx_ffn_rows: unaligned pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int bpg_up = (d_ff + 3) / 4, bpg_dn = (d + 3) / 4;
  const int nt = max_rows <= 1 ? 1 : max_rows <= 2 ? 2 : max_rows <= 4 ? 4 : 8;
#define FT_MX_ROWS(NT)                                                                                        \
  timed_launch(mx_gateup_rows_kernel<NT>, dim3(ng * bpg_up), dim3(256), s, ev, 0, x, d, d_ff, k, slots,      \
               group_slot, offsets, perm, g_begin, bpg_up, h);                                              \
  if (int rc = launched("mx_gateup_rows")) return rc;                                                        \
  timed_launch(mx_down_rows_kernel<NT>, dim3(ng * bpg_dn), dim3(256), s, ev, 1, d, d_ff, slots, group_slot,  \
               offsets, g_begin, bpg_dn, (const float*)h, out);                                               \
  return launched("mx_down_rows");
  switch (nt) {
    case 1: { FT_MX_ROWS(1) }
    case 2: { FT_MX_ROWS(2) }
    case 4: { FT_MX_ROWS(4) }
    default: { FT_MX_ROWS(8) }
  }
#undef FT_MX_ROWS
}

size_t mx_act_ws_bytes(int rows, int n) { return (size_t)rows * n + (size_t)rows * (n / 32); }

int launch_mx_quant_bf16(const uint16_t* x, int rows, int n, uint8_t* q, uint8_t* sc, void* stream) {
  if (n % 64) return fail(FT_EINVAL, "mx_quant: need n%64==0");
  if (rows <= 0) return FT_OK;
  const long long nthreads = (long long)rows * (n / 32);
  mx_quant_act_kernel<uint16_t><<<(unsigned)((nthreads + 255) / 256), 256, 0, static_cast<hipStream_t>(stream)>>>(
      x, rows, n, nullptr, 1, q, sc);
  return launched("mx_quant_act");
}

int launch_mx_ffn_mfma(const uint16_t* x, int T, int d, int d_ff, int k, const uint8_t* slots,
                       const int32_t* group_slot, const int32_t* offsets, const int32_t* perm, int g_begin, int g_end,
                       int n_rows, uint8_t* xq, uint8_t* xs, float* h, uint8_t* hq, uint8_t* hs, float* out,
                       void* stream, void* const* ev) {
  if (d % 128 || d_ff % 128 || k < 1) return fail(FT_EINVAL, "mx_ffn_mfma: need d%128==0 and d_ff%128==0");
  const int ng = g_end - g_begin;
  if (ng <= 0 || n_rows <= 0) return FT_OK;
  if (!aligned16(x) || !aligned16(slots) || !aligned16(xq) || !aligned16(hq) || !aligned16(h) || !aligned16(out) ||
      ((reinterpret_cast<uintptr_t>(xs) | reinterpret_cast<uintptr_t>(hs)) & 3u))
    return fail(FT_EINVAL, "mx_ffn_mfma: unaligned pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (int rc = launch_mx_quant_bf16(x, T, d, xq, xs, s)) return rc;
  const int tiles_up = d_ff / 64, nb_up = ng * tiles_up;
  timed_launch(mx_gateup_mfma_kernel, dim3(nb_up), dim3(512), s, ev, 0, (const uint8_t*)xq, (const uint8_t*)xs, d,
               d_ff, k, slots, group_slot, offsets, perm, g_begin, tiles_up, nb_up, h);
  if (int rc = launched("mx_gateup_mfma")) return rc;
  // h rows are in permuted order already
  const long long nthreads = (long long)n_rows * (d_ff / 32);
  mx_quant_act_kernel<float><<<(unsigned)((nthreads + 255) / 256), 256, 0, s>>>(h, n_rows, d_ff, nullptr, 1, hq, hs);
  if (int rc = launched("mx_quant_h")) return rc;
  const int tiles_dn = d / 128, nb_dn = ng * tiles_dn;
  timed_launch(mx_down_mfma_kernel, dim3(nb_dn), dim3(512), s, ev, 1, (const uint8_t*)hq, (const uint8_t*)hs, d, d_ff,
               slots, group_slot, offsets, g_begin, tiles_dn, nb_dn, out);
  return launched("mx_down_mfma");
}

}  // namespace ft
