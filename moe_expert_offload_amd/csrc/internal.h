// Internal declarations shared by the libft sources (not part of the C ABI).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/ft.h"

namespace ft {

// Thread-local error message for ft_last_error().
void set_error(const std::string& msg);
int fail(int status, const std::string& msg);

// ---- kernel launchers (kernels.hip); all asynchronous on `stream` ----------
// Each returns FT_OK or FT_EHIP (launch error) / FT_EINVAL (bad sizes).

int launch_router(const uint16_t* x, const uint16_t* w, const uint8_t* allowed, int T, int d,
                  int E, int k, int32_t* idx, float* gates, float* logits_ws, void* stream);

// Decisions of one decode call as the device computes them ([FT] §4.1
// "Device-side cache control"), with the grouping of the routed pairs: the
// grouped FFN and the combine read offsets/perm/inv/G_slot from here.
struct DevPlan {
  int32_t P, n_u, n_h, n_m, q, n_c, avail, n_g;
  uint32_t hash;  // plan_term hash of the decisions (the host compares it with its own)
  int32_t U[FT_PLAN_CAP], H[FT_PLAN_CAP], M[FT_PLAN_CAP], F_slot[FT_PLAN_CAP], G_slot[FT_PLAN_CAP];
  int32_t route_slot[FT_PLAN_CAP], pair_group[FT_PLAN_CAP];
  int32_t offsets[FT_PLAN_CAP + 1], perm[FT_PLAN_CAP], inv[FT_PLAN_CAP];
};

// Hash of a plan: the sum over j of plan_term(j, v_j) for the sequence n_u, n_h,
// n_m, q, avail, U, H, M, G_slot (n_h + q entries), route_slot and pair_group (P
// entries each); a sum, so threads can form it in any order.
#ifdef __HIPCC__
#define FT_HD __host__ __device__
#else
#define FT_HD
#endif
FT_HD inline uint32_t plan_term(int j, int32_t v) {
  uint32_t h = (uint32_t)v + 0x9e3779b9u * (uint32_t)(j + 1);
  h ^= h >> 16;
  h *= 0x85ebca6bu;
  h ^= h >> 13;
  h *= 0xc2b2ae35u;
  h ^= h >> 16;
  return h;
}

// Residency state of the cache in device memory (mirrors ExpertCache).
struct DevCache {
  int32_t* where;       // [L*E] slot or -1
  int32_t* slot_key;    // [n_slots] l*E+e, or -1 empty
  int64_t* slot_stamp;  // [n_slots] recency stamp, -1 empty
  int64_t* clock;       // [1]
  int32_t n_slots, E;
};

// What the decode router does after the top-k when decisions run on the device.
struct DecideArgs {
  DevCache dc;
  DevPlan* plan;  // device
  DevPlan* pub;   // pinned host copy for the host (scalars and the first P / n_u entries)
  int32_t layer;
  uint32_t fq;
  int32_t min_fill, max_fetch;
};

// key[i] = map[idx[i]] (-1 for ids outside [0, n_map)).
int launch_remap(const int32_t* idx, const int32_t* map, int n_map, int P, int32_t* key, void* stream);

// Decode fills read by the GPU from the pinned pool over PCIe: records M[0:q] of a
// layer (layer_base = its expert 0, S bytes each) into slots F_slot[0:q] of the
// device plan; stream-ordered after the router that wrote the plan.
int launch_fill(const uint8_t* layer_base, size_t S, int E, uint8_t* slots, int n_slots, const DevPlan* plan,
                void* stream);
// Plain copy of pinned host memory to device memory by the same kernel reads.
int launch_h2d_copy(const void* src, void* dst, size_t bytes, void* stream);

// Decode router in one launch (T <= 64): also publishes idx, gates and x to
// pinned host memory (pub_* may be null), then writes seq to *pub_flag; ticket
// is a zeroed device counter (left zeroed).  With `da`, the last
// block also takes the cache decisions of the call on the device (dedup,
// classify, split, victims, slot rewrite, stamps) and the grouping of the pairs,
// updates the device state and publishes the plan before the flag.
int launch_router_decode(const uint16_t* x, const uint16_t* w, const uint8_t* allowed, int T, int d,
                         int E, int k, float* logits_ws, int32_t* idx, float* gates,
                         unsigned int* ticket, int32_t* pub_idx, float* pub_gates, uint16_t* pub_x,
                         uint32_t* pub_flag, uint32_t seq, void* stream, const DecideArgs* da = nullptr);

size_t permute_ws_bytes(int P, int n_groups);
// For P <= 1024 one block does everything and ws is not used; key may then live
// in pinned host memory.  Optionally copies n_gslot group slots gslot_src -> gslot_dst.
int launch_permute(const int32_t* key, int P, int n_groups, int32_t* offsets, int32_t* perm,
                   int32_t* inv, void* ws, size_t ws_bytes, void* stream,
                   const int32_t* gslot_src = nullptr, int32_t* gslot_dst = nullptr, int n_gslot = 0);

// Row-streaming (GEMV-like) grouped FFN: h fp32 [rows, d_ff], out fp32 [rows, d].
// ev (nullable): four hipEvent_t, start/stop of the gate/up kernel then of the down kernel.
// g_lo, g_hi (nullable, device): when given, only groups from *g_lo and below *g_hi
// run (the launch covers [g_begin, g_end) as a bound, for plans the host has not
// seen).  one_token: x holds one token row, every pair's (no permutation lookup).
int launch_ffn_rows(const uint16_t* x, int d, int d_ff, int k, const uint16_t* slots,
                    const int32_t* group_slot, const int32_t* offsets, const int32_t* perm,
                    int g_begin, int g_end, int max_rows, float* h, float* out, void* stream,
                    void* const* ev = nullptr, const int32_t* g_lo = nullptr, const int32_t* g_hi = nullptr,
                    int one_token = 0);

// MFMA tile grouped FFN: h bf16 [rows, d_ff] (in the fp32-sized workspace), out fp32 [rows, d].
// n_rows: rows of h and out (offsets[n_groups] at most; bounds the h reads)
int launch_ffn_mfma(const uint16_t* x, int T, int d, int d_ff, int k, const uint16_t* slots,
                    const int32_t* group_slot, const int32_t* offsets, const int32_t* perm,
                    int g_begin, int g_end, int n_rows, uint16_t* h, float* out, void* stream,
                    void* const* ev = nullptr);

// ---- MXFP4 experts (kernels_mx.hip) ------------------------------------------------
size_t mx_record_bytes(int d, int d_ff);

// Row-streaming grouped FFN over MXFP4 records, bf16 x: h fp32 [rows, d_ff], out fp32 [rows, d].
int launch_mx_ffn_rows(const uint16_t* x, int d, int d_ff, int k, const uint8_t* slots, const int32_t* group_slot,
                       const int32_t* offsets, const int32_t* perm, int g_begin, int g_end, int max_rows, float* h,
                       float* out, void* stream, void* const* ev = nullptr, const int32_t* g_lo = nullptr,
                       const int32_t* g_hi = nullptr, int one_token = 0);

// Bytes of an MXFP8 copy of rows x n activations (codes then one scale per 32).
size_t mx_act_ws_bytes(int rows, int n);

// Scaled-MFMA grouped FFN: converts x [T, d] to MXFP8 (xq codes [T, d], xs scales
// [T, d/32]), gate/up into h fp32 [n_rows, d_ff], h to MXFP8 (hq, hs), then down
// into out fp32 [n_rows, d], rows in perm order.  n_rows = offsets[g_end]: rows
// [0, n_rows) of h are converted (those before offsets[g_begin] are not used).
int launch_mx_ffn_mfma(const uint16_t* x, int T, int d, int d_ff, int k, const uint8_t* slots,
                       const int32_t* group_slot, const int32_t* offsets, const int32_t* perm, int g_begin, int g_end,
                       int n_rows, uint8_t* xq, uint8_t* xs, float* h, uint8_t* hq, uint8_t* hs, float* out,
                       void* stream, void* const* ev = nullptr);

int launch_combine(const float* out, const int32_t* inv, const float* gates,
                   const float* cpu_partial, int T, int k, int d, float* y, void* stream);

// ---- host expert kernel (cpu_exec.cpp) ----------------------------------------
// One batch of CPU-branch work: experts `n_exp`, each with a record pointer and a
// list of (token, gate) uses.  Computes partial[t] += sum gate * FFN_e(x[t]).
struct CpuUse {
  int32_t t;
  float gate;
};
struct CpuExpert {
  const void* rec;  // one record in the context's format (FT_W_BF16 or FT_W_MXFP4)
  int32_t n_use;
  CpuUse use[64];
};

class CpuPool;
CpuPool* cpu_pool_create(int threads);
void cpu_pool_destroy(CpuPool*);
int cpu_pool_threads(const CpuPool*);
// Starts the work asynchronously; x is bf16 [T, d]; partial fp32 [T, d] is
// overwritten (zeroed first); fmt is the records' ft_wfmt.  Returns immediately.
void cpu_pool_submit(CpuPool*, const uint16_t* x, int T, int d, int d_ff, int fmt, const CpuExpert* ex,
                     int n_exp, float* partial);
// Blocks until the submitted work is done (the caller works on it too).
void cpu_pool_wait(CpuPool*);
// Microseconds from the last submit to the completion of its last work item.
double cpu_pool_last_work_us(const CpuPool*);
// Work items the calling thread did itself in the last call.
int cpu_pool_last_caller_items(const CpuPool*);
const char* cpu_simd_name();

}  // namespace ft
