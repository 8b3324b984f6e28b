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

#include <algorithm>
#include <climits>
#include <cmath>

#include "device_common.h"
#include "internal.h"

using namespace ft::dev;

namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));

// 2^(s - 127) for an E8M0 byte (s < 255).
__device__ __forceinline__ float e8m0(uint32_t s) { return s ? __uint_as_float(s << 23) : 1.17549435e-38f * 0.5f; }

// gfx950 converts two E2M1 codes (byte `sel` of a word, the low nibble first) to a
// pair of bf16 or fp32 values in one instruction; with scale 1 both are exact.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// acc + sum over the 8 elements of one code word times 4 words of bf16 pairs
// (element 2b of the word in the low half of xw[b]); products summed in pairs.
__device__ __forceinline__ float word_dot_bf16(uint32_t cw, const uint32_t (&xw)[4], float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 0),
                                        __builtin_bit_cast(bf16x2_t, xw[0]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 1),
                                        __builtin_bit_cast(bf16x2_t, xw[1]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 2),
                                        __builtin_bit_cast(bf16x2_t, xw[2]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, 1.0f, 3),
                                        __builtin_bit_cast(bf16x2_t, xw[3]), acc, false);
  return acc;
}

// sum over the 32 elements of one weight block (16 code bytes) times 32 bf16
// activations held in registers (4 x 8 bf16, elements 8q .. 8q + 7 in xv[q])
__device__ __forceinline__ float block_dot_bf16_r(uint4 codes, const uint4 (&xv)[4]) {
  const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t xw[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
    acc = word_dot_bf16(cw[q], xw, acc);
  }
  return acc;
}

// acc + sum over the 8 elements of one code word times 8 fp32 values
__device__ __forceinline__ float word_dot_f32(uint32_t cw, float4 h0, float4 h1, float acc) {
  f32x2_t w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0);
  acc = fmaf(w.x, h0.x, acc);
  acc = fmaf(w.y, h0.y, acc);
  w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1);
  acc = fmaf(w.x, h0.z, acc);
  acc = fmaf(w.y, h0.w, acc);
  w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2);
  acc = fmaf(w.x, h1.x, acc);
  acc = fmaf(w.y, h1.y, acc);
  w = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3);
  acc = fmaf(w.x, h1.z, acc);
  acc = fmaf(w.y, h1.w, acc);
  return acc;
}

__device__ __forceinline__ float block_dot_f32(uint4 codes, const float* __restrict__ hb) {
  const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
  float acc = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 h0 = *reinterpret_cast<const float4*>(hb + 8 * q);
    const float4 h1 = *reinterpret_cast<const float4*>(hb + 8 * q + 4);
    acc = word_dot_f32(cw[q], h0, h1, acc);
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

// ---- decode: row-streaming form ---------------------------------------------------
// gate/up: one wavefront per 2 row pairs (gate and up rows r, r+1; 1 pair beyond
// d = 4096); lane l takes the 32-element blocks l, l+64, ... of each row (16 code
// bytes and one scale byte each) and reads the token's activations for them once.
// down: one wavefront per 4 consecutive rows of W_down, whose codes (and scales) are
// one contiguous span; lane l takes blocks l, l+64, ... of the span, each added into
// the sum of the row it lies in.  Both read the group's metadata in one round of
// independent loads, then every code block and scale of the lane through a buffer
// resource (masked ones read as zeros), before anything the arithmetic needs.

template <int NB, int RG>  // NB: blocks per lane and row (d <= 2048 * NB); RG row pairs per wavefront
__global__ __launch_bounds__(256) void mx_gateup_rows_kernel(
    const uint16_t* __restrict__ x, int d, int d_ff, int k, const uint8_t* __restrict__ slots,
    const int32_t* __restrict__ group_slot, const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm,
    int g_begin, int blocks_per_group, float* __restrict__ h, const int32_t* __restrict__ g_lo,
    const int32_t* __restrict__ g_hi, int one_token) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = g_begin + blockIdx.x / blocks_per_group;
  const int row0 = ((blockIdx.x % blocks_per_group) * 4 + wave) * RG;
  const int glo = g_lo != nullptr ? *g_lo : INT_MIN;
  const int ghi = g_hi != nullptr ? *g_hi : INT_MAX;
  const int slot = group_slot[g];
  const int r0 = offsets[g];
  const int r1 = offsets[g + 1];
  if (row0 >= d_ff || g < glo || g >= ghi || r1 <= r0) return;
  const int n = r1 - r0;
  const MxRec R = mx_rec(d, d_ff);
  const __amdgpu_buffer_rsrc_t rec = buf_rsrc(slots + (size_t)slot * R.bytes, (uint32_t)R.bytes);
  const int nb = d / 32;  // blocks per row
  uint4 cg[RG][NB], cu[RG][NB];
  uint32_t sg[RG][NB], su[RG][NB];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int row = row0 + r;
    const uint32_t gc = (uint32_t)(R.g_codes + (size_t)row * (d / 2)), uc = (uint32_t)(R.u_codes + (size_t)row * (d / 2));
    const uint32_t gs = (uint32_t)(R.g_sc + (size_t)row * nb), us = (uint32_t)(R.u_sc + (size_t)row * nb);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int b = lane + 64 * j;
      const bool in = row < d_ff && b < nb;
      cg[r][j] = buf_ld16(rec, in ? gc + 16u * b : kOOB);
      cu[r][j] = buf_ld16(rec, in ? uc + 16u * b : kOOB);
      sg[r][j] = buf_ld8(rec, in ? gs + b : kOOB);
      su[r][j] = buf_ld8(rec, in ? us + b : kOOB);
    }
  }
  // one token at a time: its 32 activations per block of the lane are read once and
  // applied to all RG row pairs
  for (int t = 0; t < n; ++t) {
    const uint16_t* xr = one_token ? x : x + (size_t)(perm[r0 + t] / k) * d;
    uint4 xv[NB][4];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int b = lane + 64 * j;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xv[j][q] = b < nb ? *reinterpret_cast<const uint4*>(xr + 32 * b + 8 * q) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      float ag = 0.0f, au = 0.0f;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        if (lane + 64 * j >= nb) continue;
        ag = fmaf(block_dot_bf16_r(cg[r][j], xv[j]), e8m0(sg[r][j]), ag);
        au = fmaf(block_dot_bf16_r(cu[r][j], xv[j]), e8m0(su[r][j]), au);
      }
      const float zg = wave_sum(ag);
      const float zu = wave_sum(au);
      if (lane == 0 && row0 + r < d_ff) h[(size_t)(r0 + t) * d_ff + row0 + r] = silu(zg) * zu;
    }
  }
}

// h rows staged in LDS with each 32-element block at a stride of 36 floats: a lane
// reads the 32 consecutive values of its block, and at that stride the 16-byte reads
// of 16 consecutive lanes (blocks) fall on distinct banks (a 32-float stride would put
// every lane of the wavefront on the same banks).
constexpr int kHStride = 36;

// Token rows of h a down block stages at once: at most 64 KB of padded rows.
__host__ __device__ inline int mx_down_rows_per_batch(int nt_max, int d_ff) {
  const int per_row = (d_ff / 32) * kHStride;
  const int fit = 16384 / per_row;
  return nt_max < (fit > 1 ? fit : 1) ? nt_max : (fit > 1 ? fit : 1);
}

// C64: d_ff = 2048 with RW = 8 (64 blocks per row, NB = 8): lane l owns block l of
// every one of its rows, so it reads its 32 h values of a token from LDS once.
template <int NT, int NB, int RW, bool C64 = false>  // NB: blocks per lane over RW rows (RW * d_ff <= 2048 * NB)
__global__ __launch_bounds__(256) void mx_down_rows_kernel(
    int d, int d_ff, const uint8_t* __restrict__ slots, const int32_t* __restrict__ group_slot,
    const int32_t* __restrict__ offsets, int g_begin, int blocks_per_group, const float* __restrict__ h,
    float* __restrict__ out, const int32_t* __restrict__ g_lo, const int32_t* __restrict__ g_hi) {
  extern __shared__ float sh[];  // h rows of a batch of tokens, [nt][d_ff / 32][kHStride]
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
  const MxRec R = mx_rec(d, d_ff);
  const __amdgpu_buffer_rsrc_t rec = buf_rsrc(slots + (size_t)slot * R.bytes, (uint32_t)R.bytes);
  const int nb = d_ff / 32;                              // blocks per row
  const int span = row0 < d ? min(RW, d - row0) * nb : 0;  // blocks of this wave's rows, contiguous
  const uint32_t dc = (uint32_t)(R.d_codes + (size_t)row0 * (d_ff / 2)), ds = (uint32_t)(R.d_sc + (size_t)row0 * nb);
  uint4 cv[NB];
  uint32_t sv[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int p = lane + 64 * j;
    const bool in = p < span;
    cv[j] = buf_ld16(rec, in ? dc + 16u * p : kOOB);
    sv[j] = buf_ld8(rec, in ? ds + p : kOOB);
  }
  const int per = mx_down_rows_per_batch(NT, d_ff);
  const int tok_stride = nb * kHStride;
  for (int tb = 0; tb < n; tb += per) {
    const int nt = min(per, n - tb);
    __syncthreads();  // the previous batch's h is no longer read
    for (int i = threadIdx.x * 4; i < nt * d_ff; i += 256 * 4) {
      const int ti = i / d_ff, e = i - ti * d_ff;
      *reinterpret_cast<float4*>(sh + ti * tok_stride + (e >> 5) * kHStride + (e & 31)) =
          *reinterpret_cast<const float4*>(h + (size_t)(r0 + tb) * d_ff + i);
    }
    __syncthreads();
    float acc[NT][RW];
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int r = 0; r < RW; ++r) acc[i][r] = 0.0f;
    if constexpr (C64) {
      // row j of the wave is code block j of the lane; its h block is block `lane`
      // one code word (8 elements) of every row at a time against the same 8 h values
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        if (i >= nt) continue;
        const float* hb = sh + i * tok_stride + lane * kHStride;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 h0 = *reinterpret_cast<const float4*>(hb + 8 * q);
          const float4 h1 = *reinterpret_cast<const float4*>(hb + 8 * q + 4);
#pragma unroll
          for (int j = 0; j < RW; ++j) {
            uint32_t w = q == 0 ? cv[j].x : q == 1 ? cv[j].y : q == 2 ? cv[j].z : cv[j].w;
            // converted where used: hoisted out of the token loop, the conversions of all
            // rows would hold 256 values per lane
            asm volatile("" : "+v"(w));
            acc[i][j] = word_dot_f32(w, h0, h1, acc[i][j]);
          }
        }
#pragma unroll
        for (int j = 0; j < RW; ++j) acc[i][j] *= e8m0(sv[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int p = lane + 64 * j;
        if (p >= span) continue;
        const int rr = p / nb, cb = p - rr * nb;
        const float sc = e8m0(sv[j]);
#pragma unroll
        for (int i = 0; i < NT; ++i) {
          if (i >= nt) continue;
          const float v = block_dot_f32(cv[j], sh + i * tok_stride + cb * kHStride) * sc;
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
// Block: 512 threads = 8 waves, two per SIMD.  One pass covers up to 256 rows of one
// expert (8 row subtiles of 32) and 256 weight rows ("B columns"), so every weight
// byte is read from HBM once per pass; the waves split them 4 x 2 (see q_stage).  K
// runs in stages of 128 elements = two scaled MFMAs per row subtile and column
// subtile.  MFMA i (0, 1) of a stage
// takes as its K positions 0..31 the stage's block i and as positions 32..63 its
// block i + 2 (any pairing is exact as long as both operands and both scales follow
// it); then a lane's E2M1 codes for an MFMA are one 16-byte piece of a weight row.
//
// All four operand streams of a stage (token-row codes and scales, weight codes and
// scales) go straight from memory into one LDS stage buffer (`buffer_load ... lds`,
// no registers in between), two stages ahead, through three buffers of 50 KB.  Wave w
// loads token rows 32 w .. +31 and B columns 32 w .. +31, and the scales of 64 token
// rows (waves 0-3) or 64 B columns (waves 4-7), all shared behind the stage barrier: 7
// loads per wave per stage, spread over the stage's MFMAs, waited for by one explicit
// `s_waitcnt vmcnt` at the top of the stage they feed.  With two waves per SIMD, one
// wave's MFMAs run while the other waits on the issue of its loads.  (Loads into
// registers leave the waits to the compiler, which drains every load at the head of
// the K loop: the memory latency then lands on every few stages.)
//
// Stage buffer (bytes): token-row codes, row r at 128 r with 16-byte piece p at
// physical piece p ^ swz8(r) | their scales, 4 bytes per row (the stage's 4 blocks) |
// weight codes, column c at 64 c with piece p at physical piece p ^ swz4(c) | weight
// scales, 4 bytes per column.  The swizzles put the 8 or 16 lanes of one LDS read
// phase (consecutive rows, one logical piece) on as many different bank groups.
constexpr int QM = 256;                    // rows per pass
constexpr int QK = 128;                    // K elements per stage
constexpr int QXS = QM * QK;               // offset of the token-row scales in a stage buffer
constexpr int QWC = QXS + QM * 4;          // offset of the weight codes
constexpr int QWS = QWC + 256 * (QK / 2);  // offset of the weight scales
constexpr int QSTAGE = QWS + 256 * 4;      // one stage buffer: 51200 bytes
constexpr int QNB = 3;                     // stage buffers
constexpr int QWAVES = 8;                  // waves per block, two per SIMD
constexpr int QLOADS = 7;                  // loads per wave per stage

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ int swz8(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int swz4(int c) { return ((c >> 1) ^ (c >> 3)) & 3; }

// This lane's loads of one pass: buffer resources and byte offsets at K position 0.
struct QLoads {
  __amdgpu_buffer_rsrc_t rx, rxs, rw;  // token-row codes, their scales, the expert record
  uint32_t xo[4], wo[2], so;           // so: token-row scales (waves 0-3) or weight scales (4-7)
};

// Load t (0..6) of stage st into the stage buffer at LDS byte address lb: token-row
// codes of rows 32 w + 8 t .. +7 (t < 4), weight codes of columns 32 w + 16 (t - 4)
// .. +15 (t = 4, 5), and the scales of token rows 64 w .. +63 (waves 0-3) or of weight
// columns 64 (w - 4) .. +63 (waves 4-7).
__device__ __forceinline__ void q_issue(const QLoads& L, int t, int st, uint32_t lb, int wave) {
  if (t < 4)
    lds_load16(L.rx, L.xo[t], (uint32_t)st * QK, lb + (uint32_t)(4096 * wave + 1024 * t));
  else if (t < 6)
    lds_load16(L.rw, L.wo[t - 4], (uint32_t)st * (QK / 2), lb + (uint32_t)(QWC + 2048 * wave + 1024 * (t - 4)));
  else if (wave < 4)
    lds_load4(L.rxs, L.so, (uint32_t)st * 4, lb + (uint32_t)(QXS + 256 * wave));
  else
    lds_load4(L.rw, L.so, (uint32_t)st * 4, lb + (uint32_t)(QWS + 256 * (wave - 4)));
}

// Lane l of load t covers, for token-row codes, buffer row 32 w + 8 t + l/8 at physical
// piece l%8, and for weight codes column 32 w + 16 u + l/4 at physical piece l%4; it
// reads the logical piece stored there.
__device__ __forceinline__ int q_xrow(int wave, int t, int lane) { return 32 * wave + 8 * t + (lane >> 3); }
__device__ __forceinline__ int q_xpiece(int r, int lane) { return (lane & 7) ^ swz8(r); }
__device__ __forceinline__ int q_wcol(int wave, int u, int lane) { return 32 * wave + 16 * u + (lane >> 2); }
__device__ __forceinline__ int q_wpiece(int c, int lane) { return (lane & 3) ^ swz4(c); }

__device__ __forceinline__ i32x4_t lds_piece(const uint8_t* row, int phys) {
  return *reinterpret_cast<const i32x4_t*>(row + 16 * phys);
}

__device__ __forceinline__ v8i_t fp4_operand(i32x4_t c) {
  v8i_t r;
  r[0] = c.x; r[1] = c.y; r[2] = c.z; r[3] = c.w;
  r[4] = 0; r[5] = 0; r[6] = 0; r[7] = 0;
  return r;
}

// A operand of row r for both MFMAs of a stage (lane group g: pieces 2i + g and
// 2i + g + 4 for MFMA i), and the row's 4 scale bytes.
struct QA {
  v8i_t f[2];
  uint32_t s;
};

__device__ __forceinline__ void q_read_a(QA& q, const uint8_t* buf, int r, int g) {
  const uint8_t* row = buf + 128 * r;
  const int z = swz8(r);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const i32x4_t lo = lds_piece(row, (2 * i + g) ^ z), hi = lds_piece(row, (2 * i + g + 4) ^ z);
    q.f[i][0] = lo.x; q.f[i][1] = lo.y; q.f[i][2] = lo.z; q.f[i][3] = lo.w;
    q.f[i][4] = hi.x; q.f[i][5] = hi.y; q.f[i][6] = hi.z; q.f[i][7] = hi.w;
  }
  q.s = *reinterpret_cast<const uint32_t*>(buf + QXS + 4 * r);
}

// After MFMA mi of the nm of a stage, the loads t with t nm / 7 == mi, pinned there:
// the wave's 7 loads spread evenly over its MFMAs.  The 56 loads of a block's stage
// occupy the compute unit's address unit for about as long as the MFMAs run; bunched,
// they back up and stall the issuing wave, MFMAs included (the scheduler would bunch
// them behind the first few MFMAs).
template <typename F>
__device__ __forceinline__ void q_issue_at(int mi, int nm, F& issue) {
  bool any = false;
#pragma unroll
  for (int t = 0; t < QLOADS; ++t)
    if (t * nm / QLOADS == mi) {
      issue(t);
      any = true;
    }
  if (any) __builtin_amdgcn_sched_barrier(0);
}

// acc[i][j] += A(row subtile i of this wave) x B(column subtile j of this wave) over
// one stage, as MFMAs m0 .. m0 + 7 of the stage's nm.  The four column subtiles take K
// half 0, then K half 1, so that the two MFMAs into one accumulator are four apart.
template <typename F>
__device__ __forceinline__ void q_mma(f32x16_t (&acc)[2][4], const QA& q, int i, const v8i_t (&b)[4][2],
                                      const int (&sb)[4][2], int g, int m0, int nm, F& issue) {
  const int sa[2] = {(int)((q.s >> (16 * g)) & 0xff), (int)((q.s >> (16 * g + 8)) & 0xff)};
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(q.f[h], b[j][h], acc[i][j], 0, 4, 0, sa[h], 0,
                                                                  sb[j][h]);
      q_issue_at(m0 + 4 * h + j, nm, issue);
    }
}

// One stage held in `buf`.  The 8 waves form a 4 x 2 grid: wave w takes the row
// subtiles w/2, w/2 + 4 (NA of them, 0 to 2) and the B columns 128 (w%2) .. +127 (four
// column subtiles).  The two waves of a SIMD (w and w + 4) then hold row subtiles
// {q, q + 2, q + 4, q + 6} (q = w%4 / 2) between them, as even a split of the pass's
// rows over the SIMDs as 32-row subtiles allow.  The wave's B operands and scales first,
// then its row subtiles, subtile i + 1 read from LDS while subtile i multiplies;
// `issue(t)` sends load t of a later stage.
template <int NA, typename F>
__device__ __forceinline__ void q_stage(f32x16_t (&acc)[2][4], const uint8_t* buf, int wave, int lane, F&& issue) {
  if (NA == 0) {
#pragma unroll
    for (int t = 0; t < QLOADS; ++t) issue(t);
    return;
  }
  const int m = lane & 31, g = lane >> 5, wr = wave >> 1, wc = wave & 1;
  v8i_t b[4][2];
  int sb[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = 128 * wc + 32 * j + m;
    const uint8_t* col = buf + QWC + 64 * c;
    const uint32_t s = *reinterpret_cast<const uint32_t*>(buf + QWS + 4 * c);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      b[j][h] = fp4_operand(lds_piece(col, (2 * g + h) ^ swz4(c)));
      sb[j][h] = (int)((s >> (16 * g + 8 * h)) & 0xff);
    }
  }
  QA q0, q1;
  q_read_a(q0, buf, 32 * wr + m, g);
  if (NA > 1) q_read_a(q1, buf, 32 * (wr + 4) + m, g);
  q_mma(acc, q0, 0, b, sb, g, 0, 8 * NA, issue);
  if (NA > 1) q_mma(acc, q1, 1, b, sb, g, 8, 8 * NA, issue);
}

// K loop of one pass over nst stages.  Stage s waits for its own loads (issued two
// stages earlier; only the 7 of stage s + 1 are younger), passes the barrier (every
// wave's part has landed and stage s - 1, whose buffer the loads of stage s + 2 now
// overwrite, is done), then multiplies.  Past the last stage the loads re-read it, so
// that every stage issues the same 7.
template <int NA>
__device__ __forceinline__ void q_pass(f32x16_t (&acc)[2][4], const QLoads& L, const uint8_t* sq, uint32_t lds0,
                                       int nst, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
#pragma unroll
  for (int t = 0; t < QLOADS; ++t) q_issue(L, t, 0, lds0, wave);
#pragma unroll
  for (int t = 0; t < QLOADS; ++t) q_issue(L, t, min(1, nst - 1), lds0 + QSTAGE, wave);
  int b = 0;
  for (int st = 0; st < nst; ++st) {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(QLOADS) : "memory");
    __syncthreads();
    const int sn = min(st + 2, nst - 1);
    const int bn = b == 0 ? 2 : b - 1;  // (st + 2) % 3
    const uint32_t lbn = lds0 + (uint32_t)(bn * QSTAGE);
    q_stage<NA>(acc, sq + b * QSTAGE, wave, lane, [&](int t) { q_issue(L, t, sn, lbn, wave); });
    b = b == 2 ? 0 : b + 1;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // no load is left in flight and every wave is done with the buffers
}

// na: row subtiles of this wave (0, 1 or 2; see q_stage).
__device__ __forceinline__ void q_pass_n(int na, f32x16_t (&acc)[2][4], const QLoads& L, const uint8_t* sq,
                                         uint32_t lds0, int nst, int wave, int lane) {
  switch (na) {
    case 0: q_pass<0>(acc, L, sq, lds0, nst, wave, lane); break;
    case 1: q_pass<1>(acc, L, sq, lds0, nst, wave, lane); break;
    default: q_pass<2>(acc, L, sq, lds0, nst, wave, lane); break;
  }
}

// Row subtiles of wave w for a pass of nsub: those of w/2 and w/2 + 4 below nsub.
__device__ __forceinline__ int q_na(int nsub, int wave) {
  const int wr = wave >> 1;
  return (wr < nsub ? 1 : 0) + (wr + 4 < nsub ? 1 : 0);
}

// E8M0 scale code of a block with maximum magnitude amax, and 2^-e to multiply its
// elements by (OCP MX conversion for E4M3; an all-zero block gets code 0).
__device__ __forceinline__ uint32_t mx8_scale(float amax, float* inv) {
  if (!(amax > 0.0f)) {
    *inv = 0.0f;
    return 0u;
  }
  int e2;
  (void)frexpf(amax, &e2);
  int e = e2 - 1 - 8;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  *inv = ldexpf(1.0f, -e);
  return (uint32_t)(e + 127);
}

// h = silu(x Wg^T) * (x Wu^T) for the 128 columns of this block's strip (wave w:
// columns n0 + 32w .. +31 of both W_gate and W_up), written in MXFP8: codes hq
// [rows, d_ff] and scales hs [rows, d_ff/32] (a wave's 32 columns are one block).
__global__ __launch_bounds__(512) void mx_gateup_mfma_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs, int T, int d, int d_ff, int k,
    const uint8_t* __restrict__ slots, const int32_t* __restrict__ group_slot,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ perm, int g_begin, int n_tiles, int n_blocks,
    uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  __shared__ __attribute__((aligned(1024))) uint8_t sQ[QNB * QSTAGE];
  const int lb = xcd_logical_block(blockIdx.x, n_blocks);
  const int g = g_begin + lb / n_tiles;
  const int n0 = (lb % n_tiles) * 128;
  const int r0 = offsets[g];
  const int n = offsets[g + 1] - r0;
  if (n <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, grp = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const MxRec R = mx_rec(d, d_ff);
  const uint8_t* rec = slots + (size_t)group_slot[g] * R.bytes;
  QLoads L;
  L.rx = buf_rsrc(xq, (uint32_t)((size_t)T * d));
  L.rxs = buf_rsrc(xs, (uint32_t)((size_t)T * (d / 32)));
  L.rw = buf_rsrc(rec, (uint32_t)R.bytes);
  // B column c (column subtile j = (c/32) % 4 of the waves with w%2 = c/128): W_gate
  // for even j, W_up for odd j, row n0 + 64 (c/128) + 32 (j/2) + c%32
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = q_wcol(wave, u, lane);
    const size_t wrow = (size_t)(n0 + 64 * (c >> 7) + 32 * ((c >> 6) & 1) + (c & 31));
    L.wo[u] = (uint32_t)(((c >> 5) & 1 ? R.u_codes : R.g_codes) + wrow * (d / 2) + q_wpiece(c, lane) * 16);
  }
  if (wave >= 4) {
    const int c = 64 * (wave - 4) + lane;
    const size_t wrow = (size_t)(n0 + 64 * (c >> 7) + 32 * ((c >> 6) & 1) + (c & 31));
    L.so = (uint32_t)(((c >> 5) & 1 ? R.u_sc : R.g_sc) + wrow * (d / 32));
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)sQ;
  const int nst = d / QK;
  for (int m0 = 0; m0 < n; m0 += QM) {
    const int rows = min(QM, n - m0);
    const int nsub = (rows + 31) >> 5;
    // rows past the group's end load a valid row (their products land in rows never stored)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = q_xrow(wave, t, lane);
      L.xo[t] = (uint32_t)((size_t)(perm[r0 + m0 + min(r, rows - 1)] / k) * d + q_xpiece(r, lane) * 16);
    }
    if (wave < 4) L.so = (uint32_t)((size_t)(perm[r0 + m0 + min(64 * wave + lane, rows - 1)] / k) * (d / 32));
    f32x16_t acc[2][4];
    q_pass_n(q_na(nsub, wave), acc, L, sQ, lds0, nst, wave, lane);
    // MXFP8 conversion of h: column subtiles 2p (gate) and 2p + 1 (up) of a wave give
    // h for the 32 output columns n0 + 64 (w%2) + 32 p, one block of every row.  A
    // 32 x 32 subtile goes through this wave's corner of LDS (the pass ended with a
    // barrier, so the staging buffers are free) so that each lane then holds 16
    // consecutive values of one row: lanes 2r and 2r+1 share row r's block.
    float* tile = reinterpret_cast<float*>(sQ) + wave * 32 * 36;
    int g4 = grp * 4;
    asm volatile("" : "+v"(g4));  // keeps the row indices below out of the prologue
    const int tr = lane >> 1, th = lane & 1, wr = wave >> 1, wc = wave & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (wr + 4 * i >= nsub) continue;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          tile[((v >> 2) * 8 + g4 + (v & 3)) * 36 + (lane & 31)] = silu_fast(acc[i][2 * p][v]) * acc[i][2 * p + 1][v];
        float hv[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 t4 = *reinterpret_cast<const float4*>(tile + tr * 36 + 16 * th + 4 * q);
          hv[4 * q] = t4.x; hv[4 * q + 1] = t4.y; hv[4 * q + 2] = t4.z; hv[4 * q + 3] = t4.w;
        }
        float amax = 0.0f;
#pragma unroll
        for (int q = 0; q < 16; ++q) amax = fmaxf(amax, fabsf(hv[q]));
        amax = fmaxf(amax, __shfl_xor(amax, 1, WAVE));
        float inv;
        const uint32_t sc = mx8_scale(amax, &inv);
        uint32_t pk[4];
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          pk[w4] = 0u;
#pragma unroll
          for (int j = 0; j < 4; ++j) pk[w4] |= (sc ? e4m3_code(hv[4 * w4 + j] * inv) : 0u) << (8 * j);
        }
        const int row = 32 * (wr + 4 * i) + tr;
        const int c0 = n0 + 64 * wc + 32 * p;
        if (row < rows) {
          const size_t gr = (size_t)(r0 + m0 + row);
          *reinterpret_cast<uint4*>(hq + gr * d_ff + c0 + 16 * th) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
          if (th == 0) hs[gr * (d_ff / 32) + c0 / 32] = (uint8_t)sc;
        }
      }
    }
    __syncthreads();  // the next row pass restages into the same LDS
  }
}

// out[i][c] = hq_i . Wd[c] for the 256 columns of this block's strip (wave w: columns
// n0 + 64w .. +63), h in MXFP8 with rows in perm order.
__global__ __launch_bounds__(512) void mx_down_mfma_kernel(
    const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs, int n_rows, int d, int d_ff,
    const uint8_t* __restrict__ slots, const int32_t* __restrict__ group_slot,
    const int32_t* __restrict__ offsets, int g_begin, int n_tiles, int n_blocks, float* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t sQ[QNB * QSTAGE];
  const int lb = xcd_logical_block(blockIdx.x, n_blocks);
  const int g = g_begin + lb / n_tiles;
  const int n0 = (lb % n_tiles) * 256;
  const int r0 = offsets[g];
  const int n = offsets[g + 1] - r0;
  if (n <= 0) return;
  const int tid = threadIdx.x, lane = tid & 63, grp = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const MxRec R = mx_rec(d, d_ff);
  const uint8_t* rec = slots + (size_t)group_slot[g] * R.bytes;
  QLoads L;
  L.rx = buf_rsrc(hq, (uint32_t)((size_t)n_rows * d_ff));
  L.rxs = buf_rsrc(hs, (uint32_t)((size_t)n_rows * (d_ff / 32)));
  L.rw = buf_rsrc(rec, (uint32_t)R.bytes);
  // B column c is output column n0 + c
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int c = q_wcol(wave, u, lane);
    L.wo[u] = (uint32_t)(R.d_codes + (size_t)(n0 + c) * (d_ff / 2) + q_wpiece(c, lane) * 16);
  }
  if (wave >= 4) L.so = (uint32_t)(R.d_sc + (size_t)(n0 + 64 * (wave - 4) + lane) * (d_ff / 32));
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_u8*)sQ;
  const int nst = d_ff / QK;
  const int col = n0 + 128 * (wave & 1) + (lane & 31);  // column subtile j: col + 32 j
  for (int m0 = 0; m0 < n; m0 += QM) {
    const int rows = min(QM, n - m0);
    const int nsub = (rows + 31) >> 5;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int r = q_xrow(wave, t, lane);
      L.xo[t] = (uint32_t)((size_t)(r0 + m0 + min(r, rows - 1)) * d_ff + q_xpiece(r, lane) * 16);
    }
    if (wave < 4) L.so = (uint32_t)((size_t)(r0 + m0 + min(64 * wave + lane, rows - 1)) * (d_ff / 32));
    f32x16_t acc[2][4];
    q_pass_n(q_na(nsub, wave), acc, L, sQ, lds0, nst, wave, lane);
    int g4 = grp * 4;
    asm volatile("" : "+v"(g4));
    const int wr = wave >> 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (wr + 4 * i >= nsub) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 32 * (wr + 4 * i) + (v >> 2) * 8 + g4 + (v & 3);
        if (row < rows) {
          float* o = out + (size_t)(r0 + m0 + row) * d + col;
          o[0] = acc[i][0][v];
          o[32] = acc[i][1][v];
          o[64] = acc[i][2][v];
          o[96] = acc[i][3][v];
        }
      }
    }
  }
}


}  // namespace

namespace ft {

size_t mx_record_bytes(int d, int d_ff) { return mx_rec(d, d_ff).bytes; }

int launch_mx_ffn_rows(const uint16_t* x, int d, int d_ff, int k, const uint8_t* slots, const int32_t* group_slot,
                       const int32_t* offsets, const int32_t* perm, int g_begin, int g_end, int max_rows, float* h,
                       float* out, void* stream, void* const* ev, const int32_t* g_lo, const int32_t* g_hi,
                       int one_token) {
  if (d % 64 || d_ff % 64 || k < 1) return fail(FT_EINVAL, "mx_ffn_rows: need d%64==0 and d_ff%64==0");
  const int ng = g_end - g_begin;
  if (ng <= 0) return FT_OK;
  if (!aligned16(x) || !aligned16(slots) || !aligned16(h) || !aligned16(out))
    return fail(FT_EINVAL, "mx_ffn_rows: unaligned pointer");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mx_rec(d, d_ff).bytes >= ((size_t)1 << 31)) return fail(FT_EINVAL, "mx_ffn_rows: record over 2 GiB");
  if (d > 8192 || d_ff > 4096) return fail(FT_EINVAL, "mx_ffn_rows: need d <= 8192 and d_ff <= 4096");
  // gate/up: 2 row pairs per wavefront up to d = 4096 (2 blocks per lane), 1 beyond
  const int rg = d <= 4096 ? 2 : 1;
  const int bpg_up = (d_ff + 4 * rg - 1) / (4 * rg);
  const int nt = max_rows <= 1 ? 1 : max_rows <= 2 ? 2 : max_rows <= 4 ? 4 : 8;
  // blocks per lane: gate/up ceil(d/32/64); down ceil(RW*d_ff/32/64) with RW = 8 rows per
  // wavefront up to d_ff = 2048, 4 beyond
  const int nbu = (d / 32 + 63) / 64;
  const int rw = d_ff <= 2048 ? 8 : 4;
  const int nbd = (rw * (d_ff / 32) + 63) / 64;
  const int bpg_dn = (d + 4 * rw - 1) / (4 * rw);
#define FT_MX_UP(NB)                                                                                         \
  timed_launch(mx_gateup_rows_kernel<NB, NB <= 2 ? 2 : 1>, dim3(ng * bpg_up), dim3(256), s, ev, 0, x, d, d_ff, k, \
               slots, group_slot, offsets, perm, g_begin, bpg_up, h, g_lo, g_hi, one_token)
#define FT_MX_DN(NT, NB, RW)                                                                                 \
  timed_launch_shm(mx_down_rows_kernel<NT, NB, RW>, dim3(ng * bpg_dn), dim3(256),                             \
                   (size_t)mx_down_rows_per_batch(NT, d_ff) * (d_ff / 32) * kHStride * 4, s, ev, 1, d,         \
                   d_ff, slots, group_slot, offsets, g_begin, bpg_dn, (const float*)h, out, g_lo, g_hi)
#define FT_MX_DN64(NT)                                                                                       \
  timed_launch_shm(mx_down_rows_kernel<NT, 8, 8, true>, dim3(ng * bpg_dn), dim3(256),                          \
                   (size_t)mx_down_rows_per_batch(NT, d_ff) * (d_ff / 32) * kHStride * 4, s, ev, 1, d,         \
                   d_ff, slots, group_slot, offsets, g_begin, bpg_dn, (const float*)h, out, g_lo, g_hi)
#define FT_MX_ROWS(NT)                                                     \
  if (nbu <= 1) FT_MX_UP(1); else if (nbu <= 2) FT_MX_UP(2); else FT_MX_UP(4);            \
  if (int rc = launched("mx_gateup_rows")) return rc;                      \
  if (rw == 8 && d_ff == 2048) {                                          \
    FT_MX_DN64(NT);                                                        \
  } else if (rw == 8) {                                                    \
    if (nbd <= 1) FT_MX_DN(NT, 1, 8); else if (nbd <= 2) FT_MX_DN(NT, 2, 8);  \
    else if (nbd <= 4) FT_MX_DN(NT, 4, 8); else FT_MX_DN(NT, 8, 8);         \
  } else {                                                                 \
    FT_MX_DN(NT, 8, 4);                                                    \
  }                                                                        \
  return launched("mx_down_rows");
  switch (nt) {
    case 1: { FT_MX_ROWS(1) }
    case 2: { FT_MX_ROWS(2) }
    case 4: { FT_MX_ROWS(4) }
    default: { FT_MX_ROWS(8) }
  }
#undef FT_MX_UP
#undef FT_MX_DN
#undef FT_MX_ROWS
#undef FT_MX_DN64
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
                       int n_rows, uint8_t* xq, uint8_t* xs, float* /*h*/, uint8_t* hq, uint8_t* hs, float* out,
                       void* stream, void* const* ev) {
  if (d % 256 || d_ff % 128 || k < 1) return fail(FT_EINVAL, "mx_ffn_mfma: need d%256==0 and d_ff%128==0");
  const int ng = g_end - g_begin;
  if (ng <= 0 || n_rows <= 0) return FT_OK;
  if (!aligned16(x) || !aligned16(slots) || !aligned16(xq) || !aligned16(hq) || !aligned16(out) ||
      ((reinterpret_cast<uintptr_t>(xs) | reinterpret_cast<uintptr_t>(hs)) & 3u))
    return fail(FT_EINVAL, "mx_ffn_mfma: unaligned pointer");
  if ((size_t)T * d >= (1u << 31) || (size_t)n_rows * d_ff >= (1u << 31) || mx_rec(d, d_ff).bytes >= (1u << 31))
    return fail(FT_EINVAL, "mx_ffn_mfma: activations or a record over 2 GiB");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (int rc = launch_mx_quant_bf16(x, T, d, xq, xs, s)) return rc;
  const int tiles_up = d_ff / 128, nb_up = ng * tiles_up;
  timed_launch(mx_gateup_mfma_kernel, dim3(nb_up), dim3(64 * QWAVES), s, ev, 0, (const uint8_t*)xq,
               (const uint8_t*)xs, T, d, d_ff, k, slots, group_slot, offsets, perm, g_begin, tiles_up, nb_up, hq, hs);
  if (int rc = launched("mx_gateup_mfma")) return rc;
  const int tiles_dn = d / 256, nb_dn = ng * tiles_dn;
  timed_launch(mx_down_mfma_kernel, dim3(nb_dn), dim3(64 * QWAVES), s, ev, 1, (const uint8_t*)hq,
               (const uint8_t*)hs, n_rows, d, d_ff, slots, group_slot, offsets, g_begin, tiles_dn, nb_dn, out);
  return launched("mx_down_mfma");
}

}  // namespace ft
