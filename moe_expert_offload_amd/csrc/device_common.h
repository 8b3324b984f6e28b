// Device and launch helpers shared by the kernel sources (kernels.hip, kernels_mx.hip):
// vector types, buffer-resource loads, wavefront sums, SiLU, the XCD-aware block order,
// the LDS-direct loads of the MFMA kernels, and the launch wrappers.  gfx950 only.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "internal.h"

namespace ft {
namespace dev {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Buffer loads over one expert record: a scalar resource (base, size in bytes) and a
// 32-bit byte offset per lane; the hardware range check returns zeros for offsets
// past the size, so masked pieces cost no branch (kOOB is past every record).
constexpr uint32_t kOOB = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}
__device__ __forceinline__ uint32_t buf_ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
// The same through the hardware exp2 and reciprocal (a few ulp), for values that are
// rounded right after (to bf16 or MXFP8 in the prefill MFMA epilogues).
__device__ __forceinline__ float silu_fast(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// Blocks are dealt to the 8 XCDs round-robin; remap so that consecutive logical
// blocks share an XCD (and its L2).
__device__ __forceinline__ int xcd_logical_block(int b, int nb) {
  const int q = nb >> 3, r = nb & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// One load from buffer `rs` at byte offset off + kbytes straight into LDS at byte
// address lds + 16 * lane (lds_load16) or lds + 4 * lane (lds_load4); no register is
// written, and the caller waits for it with an explicit `s_waitcnt vmcnt`.
// Out-of-range offsets read zeros.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t kbytes, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(m0), "v"(off), "s"(rs), "s"(kbytes) : "memory", "m0");
}
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t kbytes, uint32_t lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(m0), "v"(off), "s"(rs), "s"(kbytes) : "memory", "m0");
}

inline int launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return ft::fail(FT_EHIP, std::string(what) + ": " + hipGetErrorString(e));
  return FT_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Launches a kernel; with timing events, start/stop bracket the kernel itself.
template <typename... KArgs, typename... Args>
inline void timed_launch_shm(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t shm, hipStream_t s,
                             void* const* ev, int which, Args... args) {
  if (ev) {
    hipExtLaunchKernelGGL(kern, grid, block, shm, s, static_cast<hipEvent_t>(ev[2 * which]),
                          static_cast<hipEvent_t>(ev[2 * which + 1]), 0, args...);
  } else {
    hipLaunchKernelGGL(kern, grid, block, shm, s, args...);
  }
}
template <typename... KArgs, typename... Args>
inline void timed_launch(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t s, void* const* ev,
                         int which, Args... args) {
  timed_launch_shm(kern, grid, block, 0, s, ev, which, args...);
}

}  // namespace dev
}  // namespace ft
