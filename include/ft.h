/*
 * ft.h -- C ABI of libft: a routed mixture-of-experts layer served from an
 * elastic GPU expert cache over a host-resident expert pool, on one AMD
 * Instinct MI355X (gfx950).
 *
 * Citations:
 *   [FT]  the paper "FreeToken: Efficient Edge-Native MoE Serving with
 *         Bandwidth-Adaptive Execution" (arXiv 2608.16157), by section/equation.
 *   [AIN] the page "FreeToken: bandwidth-adaptive edge MoE serving"
 *         (ai-infrastructure.net), by section heading.
 *
 * Conventions
 *   - Every call returns an int status: FT_OK (0), a negative error code, or a
 *     positive warning.  No exception crosses the ABI.  ft_last_error() gives a
 *     thread-local message for the last failing call on the calling thread.
 *   - "device" pointers are HIP device allocations (e.g. torch CUDA tensors on
 *     ROCm); "host" pointers are ordinary host memory; "pinned" pointers are
 *     page-locked host memory from hipHostMalloc (ft_pool_alloc) or torch
 *     pin_memory.  The caller owns every buffer it passes in; the library never
 *     frees caller memory.
 *   - Streams and events are passed as void* (hipStream_t / hipEvent_t).  A NULL
 *     stream is HIP's default stream.  Kernel launches are asynchronous: a
 *     launch error returns FT_EHIP, a fault inside a kernel surfaces at the next
 *     synchronising call.
 *   - bf16 tensors are arrays of uint16 words (the top half of an IEEE binary32).
 *     Matrices are row-major.
 *   - A context (ft_ctx_t) may be used by one host thread at a time.
 *
 * Expert record (the unit of residency, [FT] §3: a slot holds every tensor of
 * one (layer, expert) pair; [FT] §4.2: banks are indexed by l*E + e): one
 * contiguous record per expert, row-major.
 *   FT_W_BF16:  [ W_gate (d_ff x d) | W_up (d_ff x d) | W_down (d x d_ff) ] in bf16,
 *               S = 6 * d * d_ff bytes.
 *   FT_W_MXFP4 ([FT] §5.1: routed experts natively MXFP4; format of the OCP
 *               Microscaling Formats v1.0): bytes
 *               [ gate codes d_ff x d/2 | up codes d_ff x d/2 | down codes d x d_ff/2 |
 *                 gate scales d_ff x d/32 | up scales d_ff x d/32 | down scales d x d_ff/32 ],
 *               E2M1 codes two per byte (lower-index element in the low nibble),
 *               one E8M0 scale per 32 consecutive elements along each matrix's
 *               reduction axis (d for gate/up, d_ff for down); weight value =
 *               e2m1(code) * 2^(scale - 127).  S = 3*d*d_ff/2 + 3*d*d_ff/32 bytes.
 * S = ft_record_bytes(shape).  The host pool holds L_phys*E records; logical
 * layer l, expert e reads record (l mod L_phys)*E + e.
 *
 * MXFP4 arithmetic: decode (the row-streaming form) and the CPU branch apply the
 * exactly dequantised weights to the bf16 activations.  Prefill (the MFMA form)
 * runs on gfx950's scaled MFMA with E4M3 x E2M1 operands: x and the SwiGLU output
 * h are converted to MXFP8 (E4M3 elements, one E8M0 scale per 32 consecutive
 * elements along the reduction axis, shared exponent floor(log2 max|v|) - 8,
 * elements rounded to nearest even and clamped to +-448, an all-zero block gets
 * scale 0 and zero codes) before each contraction; fp32 accumulation.
 */
#ifndef FT_H
#define FT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define FT_OK 0
#define FT_EINVAL (-1)        /* bad argument, shape or state */
#define FT_ENOMEM (-2)        /* a host or pinned allocation failed, or a buffer is too small */
#define FT_EBUSY (-3)         /* not at a safe point ([FT] §3.3: rebuild only at a safe point) */
#define FT_ENOPIN (-4)        /* host pool is not pinned memory; fills are impossible ([FT] §4.2) */
#define FT_ECAP (-5)          /* prefill overlap requested with fewer than 2E slots
                                 ([AIN] "Failure modes": asserted at construction) */
#define FT_EHIP (-6)          /* a HIP call failed */
#define FT_EUNSUPPORTED (-7)  /* format or mode not built */
#define FT_ENOPROFILE (-8)    /* no usable bandwidth profile (missing, unreadable, or for another
                                 expert format: [AIN] "How to maintain it", no guessing) */
#define FT_WOVERLAP_OFF 1     /* warning: resize left fewer than 2E slots, prefill overlap
                                 disabled ([AIN] "Failure modes": warn-and-disable on rebuild) */

#define FT_PLAN_CAP 512       /* max routed pairs T*k in one decode call */

typedef enum { FT_W_BF16 = 0, FT_W_MXFP4 = 1 } ft_wfmt;

/* Layer-stack shape.  L layers, E routed experts per layer, hidden size d,
 * expert hidden size d_ff, k experts per token.  d and d_ff must be multiples of 8
 * (FT_W_BF16); FT_W_MXFP4 needs d % 256 == 0 and d_ff % 128 == 0. */
typedef struct {
  int32_t L, E, d, d_ff, k;
  int32_t fmt; /* ft_wfmt: expert record format */
} ft_shape;

/* Engine configuration ([AIN] "How to use it", flags table).
 *   frac_q16        fetch fraction phi = B_P/B_H in Q16, computed once ([FT] Eq. 4;
 *                   ft_frac_q16).
 *   min_fill        fills kept per call even when the split gives fewer, capped at m
 *                   ([FT] §3.2 "always retains at least one fill"; 0 = the shipped rule).
 *   max_fetch       -1: q from the split; n >= 0: at most n fills per call (0 never fetches).
 *   cpu_threads     worker threads of the CPU branch (0 = one per CPU of the affinity mask
 *                   except the first, which is left to the calling thread).
 *   prefill_overlap 1 = full-layer double-buffered prefill ([FT] §3.1); needs >= 2E slots.
 *   T_max           largest T of any call (sizes the workspace).
 *   L_phys          physical layers in the host pool (0 = L). */
typedef struct {
  uint32_t frac_q16;
  int32_t min_fill;
  int32_t max_fetch;
  int32_t cpu_threads;
  int32_t prefill_overlap;
  int32_t T_max;
  int32_t L_phys;
} ft_config;

/* Decisions of one decode call ([FT] §3.2, §4.1 "Device-side cache control").
 * U: distinct routed experts in first-occurrence order over (t, j), t-major.
 * H: hits, M: misses (both in U order).  F = M[0:q] is filled into F_slot[i];
 * C = M[q:] runs on the host.  G = H followed by F are the experts evaluated on
 * the GPU, in slots G_slot.  route_slot[t*k+j] is the slot of the pair's expert
 * or -1 (host); pair_group[t*k+j] its index in G or -1.  idx/gates are the
 * router's output for the call (filled by ft_moe_decode_layer). */
typedef struct {
  int32_t layer, T, k;
  int32_t n_u, n_h, n_m, q, n_c, avail;
  int32_t U[FT_PLAN_CAP];
  int32_t H[FT_PLAN_CAP];
  int32_t M[FT_PLAN_CAP];
  int32_t F_slot[FT_PLAN_CAP];
  int32_t G_slot[FT_PLAN_CAP];
  int32_t route_slot[FT_PLAN_CAP];
  int32_t pair_group[FT_PLAN_CAP];
  int32_t idx[FT_PLAN_CAP];
  float gates[FT_PLAN_CAP];
} ft_plan;

/* The decisions of one on-demand prefill layer ([FT] §3.1: the fallback when the
 * slot pool cannot spare two full layers, and the serial loading left when the
 * second buffer is off).  The chunk's distinct routed experts U (first occurrence
 * over (t, j), t-major) are computed in group order: the n_h hits (U order), then
 * the misses in rounds of at most the slots not holding a hit, each round's
 * misses loaded into LRU victims (victim order before the round, M order).  Round
 * r computes groups [r ? round_end[r-1] : 0, round_end[r]); its loads are its
 * groups at or after n_h.  Experts are < FT_E_MAX. */
#define FT_E_MAX 1024
typedef struct {
  int32_t layer, n_u, n_h, n_rounds;
  int32_t group_expert[FT_E_MAX];
  int32_t group_slot[FT_E_MAX];
  int32_t round_end[FT_E_MAX];
} ft_prefill_plan;

/* Per-call measurements (host clock, microseconds). */
typedef struct {
  int32_t layer, T, n_u, hits, misses, q, n_c;
  int32_t cpu_caller_items; /* CPU-branch work items the calling thread did itself */
  int64_t h2d_bytes;
  double t_route_us;   /* router launch until its results reached the host */
  double t_ctrl_us;    /* cache decisions */
  double t_cpu_us;     /* CPU branch, from post to completion */
  double t_total_us;   /* whole call, host side */
  double t_issue_us;   /* issuing the fills and the GPU work after the decisions */
  double t_cpu_work_us; /* CPU branch, from post to its last work item */
  double t_submit_us;   /* posting the CPU branch to the worker threads */
  double t_between_us;  /* caller's own time since the previous decode call returned (0 on the first) */
} ft_step_stats;

/* Cumulative counters since create or the last resize ([AIN] "How to run it in
 * production": a rebuild resets hit/miss counters).  unique_* count distinct
 * experts per call; read_* count routed (token, expert) pairs. */
typedef struct {
  int64_t calls, unique_hits, unique_misses, fills, cpu_experts;
  int64_t reads, read_hits, read_fills, read_cpu;
  int64_t h2d_bytes, prefill_layers, resizes;
} ft_stats;

typedef struct ft_ctx* ft_ctx_t;

/* ---- errors ------------------------------------------------------------- */
const char* ft_strerror(int status);
const char* ft_last_error(void);

/* ---- sizes and the split ----------------------------------------------- */

/* Bytes of one expert record (S), 0 for an invalid shape. */
size_t ft_record_bytes(const ft_shape* shape);

/* Device workspace bytes a context needs for calls of up to T_max tokens. */
size_t ft_workspace_bytes(const ft_shape* shape, int32_t T_max);

/* [FT] Eq. (4): phi = B_P / B_H in Q16, rounded half to even; 0 when B_P <= 0,
 * 65536 when B_P >= B_H (no residual host bandwidth, [FT] Eq. 2).  Bandwidths in
 * any common unit. */
uint32_t ft_frac_q16(double B_P, double B_H);

/* Fetch count q for m unique misses ([FT] §3.2 Eqs. 1-4; [AIN] "The split, and
 * what it is actually optimising"): lo = floor(m*fq/2^16); pick lo or lo+1,
 * whichever has the smaller max(f*(2^16-fq), (m-f)*fq), lo on a tie; cap at m;
 * raise to min(min_fill, m); cap at max_fetch when max_fetch >= 0; cap at avail
 * (slots that may be evicted).  Returns q >= 0, or FT_EINVAL for m < 0 or
 * frac_q16 > 65536. */
int32_t ft_qstar_split(int32_t m, uint32_t frac_q16, int32_t min_fill, int32_t max_fetch,
                       int32_t avail);

/* ---- host pool -------------------------------------------------------------
 * [FT] §3.3 pins the pool after filling it; here pinned memory must be allocated
 * first (hipHostMalloc) and filled afterwards.  ft_pool_alloc returns pinned,
 * host-cached, device-accessible memory owned by the caller, to be released with
 * ft_pool_free.  Errors: FT_ENOMEM, FT_EHIP. */
int ft_pool_alloc(size_t bytes, void** out);
int ft_pool_free(void* ptr);

/* ---- bandwidth profile ([AIN] "How to use it", "How to maintain it") --------
 * A machine's profile for one expert format: B_P and B_H measured apart, and the
 * contended pair measured together (pcie_ov: the PCIe rate while the CPU expert
 * kernel runs; cpu_ov: the CPU kernel's rate while the PCIe reads run; 0 when not
 * measured).  Bytes per second. */
typedef struct {
  double B_P, B_H, pcie_ov, cpu_ov;
  int32_t fmt; /* ft_wfmt the profile was measured with */
} ft_bw_profile;

/* pcie_ov / (pcie_ov + cpu_ov) in Q16, rounded half to even: 0 when pcie_ov <= 0,
 * 65536 when cpu_ov <= 0.  Equals ft_frac_q16(B_P, B_H) when the contention is
 * total (cpu_ov = B_H - B_P, pcie_ov = B_P). */
uint32_t ft_frac_q16_contended(double pcie_ov, double cpu_ov);

/* The fetch fraction a profile gives: the contended pair when both rates are
 * positive, else Eq. (4) from B_P and B_H.  0 for a null profile. */
uint32_t ft_fetch_fraction_q16(const ft_bw_profile* profile);

/* The hybrid gate ([AIN] "Why use it"): 1 (hybrid) only when every one of the n
 * benched workloads of a format has B_H > threshold * B_P, else 0 (plain offload;
 * also for n = 0).  FT_EINVAL for n < 0, null arrays with n > 0, or threshold <= 0. */
int32_t ft_recommend_hybrid(const double* B_P, const double* B_H, int32_t n, double threshold);

/* Measures the contended pair: record reads over PCIe into dev_scratch (records
 * [0, n_records/2) of the pool, one launch per record, kept in flight) while the
 * host expert kernel runs over records [n_records/2, n_records) at one token
 * (`threads` workers, 0 = all); each rate counts only work done while the other
 * side ran.  n_records >= 2; dev_scratch holds n_records/2 records. */
int ft_bench_bw_contended(const ft_shape* shape, const void* host_pool, int32_t n_records,
                          void* dev_scratch, int32_t threads, double* pcie_ov, double* cpu_ov);

/* Profile files, one per GPU and expert format: `out` gets
 * "<dir>/ft_bw_<GPU UUID in hex>_<bf16|mxfp4>.txt" (FT_ENOMEM if out_len is too
 * small).  save writes the profile as text; load reads one back and returns
 * FT_ENOPROFILE when the file is missing or unreadable, lacks B_P or B_H, or was
 * measured for a format other than `fmt`. */
int ft_bw_profile_path(int32_t device, int32_t fmt, const char* dir, char* out, size_t out_len);
int ft_bw_profile_save(const char* path, const ft_bw_profile* profile);
int ft_bw_profile_load(const char* path, int32_t fmt, ft_bw_profile* profile);

/* Measures B_P (whole records read by the GPU from the pinned pool over PCIe into
 * device memory, as the decode fills move them, `n_records` of them, one launch
 * each, on a fresh stream) and B_H (the host expert kernel over the same records at one
 * token, `threads` workers; 0 = all) in bytes per second ([FT] §3.2, Table 1:
 * both measured on the deployed tensor shapes).  Each is the fastest of several
 * passes after a warm-up pass (B_H: passes over at least 100 ms).  dev_scratch
 * must hold n_records records. */
int ft_bench_bw(const ft_shape* shape, const void* host_pool, int32_t n_records,
                void* dev_scratch, int32_t threads, double* B_P, double* B_H);

/* ---- context -----------------------------------------------------------------
 * host_pool: pinned pool of L_phys*E records (may be NULL for a decisions-only
 * context: lookups and resizes work, device calls return FT_EINVAL).
 * dev_slots: device buffer of n_slots records (the elastic cache, [FT] §3).
 * dev_workspace: device buffer of at least ft_workspace_bytes(shape, T_max).
 * The library allocates its pinned staging buffers and starts its CPU worker
 * pool here, and reads every page of the host pool once (in parallel) so that
 * the CPU branch takes no first-touch page faults while serving.  Errors: FT_EINVAL (shape/config), FT_ECAP (prefill_overlap and
 * n_slots < 2E), FT_ENOPIN (host_pool not pinned), FT_ENOMEM, FT_EHIP. */
int ft_create(const ft_shape* shape, const ft_config* config, const void* host_pool,
              size_t pool_bytes, void* dev_slots, int32_t n_slots, void* dev_workspace,
              size_t workspace_bytes, ft_ctx_t* out);
int ft_destroy(ft_ctx_t ctx);

int ft_get_stats(ft_ctx_t ctx, ft_stats* out);
int ft_reset_stats(ft_ctx_t ctx);
int ft_get_config(ft_ctx_t ctx, ft_config* out);
int32_t ft_n_slots(ft_ctx_t ctx);

/* ---- kernels (stateless; usable without a context) -------------------------- */

/* Router ([FT] §3.2: the router runs on the GPU and picks k experts per token).
 * x: device bf16 [T, d]; w_router: device bf16 [E, d]; allowed: device uint8
 * [T, E] or NULL (only allowed experts are ranked; each row must allow >= k).
 * Logits are fp32 in a fixed order: element i belongs to lane (i mod 512)/8 of 64
 * lanes, each lane adds its products in increasing i, then a_l += a_(l xor o) for
 * o = 32..1, result lane 0.  Top-k by (logit desc, index asc), renormalised
 * softmax gates.  Outputs (device): idx int32 [T, k] in rank order, gates fp32
 * [T, k], logits fp32 [T, E].  Requires 1 <= k <= min(E, 8), E <= 1024,
 * d % 8 == 0.  logits is required (it is the router's scratch between its two
 * kernels); pass the same buffer back to read the logits. */
int ft_router_topk(const void* x, const void* w_router, const uint8_t* allowed, int32_t T,
                   int32_t d, int32_t E, int32_t k, int32_t* idx, float* gates, float* logits,
                   void* stream);

/* Stable grouping of P pairs by key (device int32 [P], -1 = left out) into
 * n_groups groups: offsets int32 [n_groups+1] (exclusive prefix sum of counts),
 * perm int32 [P] (pair ids ordered by (key, id); entries past offsets[n_groups]
 * are unspecified), inv int32 [P] (position in perm or -1).  workspace: device,
 * ft_permute_workspace_bytes(P, n_groups) bytes. */
size_t ft_permute_workspace_bytes(int32_t P, int32_t n_groups);
int ft_permute(const int32_t* key, int32_t P, int32_t n_groups, int32_t* offsets,
               int32_t* perm, int32_t* inv, void* workspace, size_t workspace_bytes,
               void* stream);

/* ft_permute for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels
 * and results, with the per-block group counts in a fixed device array of the
 * library (ft_permute_noalloc_max_scratch_bytes() = 1 MiB, enough for P <= 65536
 * at any n_groups <= 1024) instead of a workspace.  Calls no allocating routine.
 * Each GPU has its own array, held until the process ends and shared by every
 * call on that GPU: calls that overlap on one GPU (different streams, or host
 * threads) race on it.  FT_EINVAL when ft_permute_workspace_bytes(P, n_groups)
 * exceeds the array, for bad sizes or null pointers; FT_EHIP when the array's
 * device address cannot be looked up. */
size_t ft_permute_noalloc_max_scratch_bytes(void);
int ft_permute_noalloc(const int32_t* key, int32_t P, int32_t n_groups, int32_t* offsets,
                       int32_t* perm, int32_t* inv, void* stream);

/* Grouped SwiGLU expert FFN over groups [g_begin, g_end):
 *   out[i] = W_down (silu(W_gate x_t) * (W_up x_t))  for i in [offsets[g], offsets[g+1]),
 *   t = perm[i] / k, with the record at slots + group_slot[g] * S.
 * x: device bf16 [T, d]; out: device fp32 [offsets[n_groups], d] (rows in perm
 * order); h_ws: device, offsets[n_groups] * d_ff * 4 bytes.  form: 0 auto, 1 the
 * bandwidth-bound row-streaming form (few tokens per expert), 2 the MFMA tile form
 * (many tokens per expert; needs d % 256 == 0 and d_ff % 128 == 0).
 * max_rows_per_group: the most rows a group holds; the row form batches that many
 * tokens per pass over the weights (a group holding more is still computed, in
 * further passes). */
int ft_grouped_ffn(const void* x, int32_t T, int32_t d, int32_t d_ff, int32_t k,
                   const void* slots, const int32_t* group_slot, const int32_t* offsets,
                   const int32_t* perm, int32_t n_groups, int32_t g_begin, int32_t g_end,
                   int32_t max_rows_per_group, void* h_ws, float* out, int32_t form,
                   void* stream);

/* The same grouped SwiGLU FFN over FT_W_MXFP4 records ([FT] §5.1 experts natively
 * MXFP4; §4.1 dequantisation inside the kernels).  form 1: row-streaming, exactly
 * dequantised weights applied to the bf16 x (the decode form); form 2: scaled MFMA,
 * x and h converted to MXFP8 first (the prefill form; see "MXFP4 arithmetic" above).
 * form 1 needs d, d_ff % 64 == 0, form 2 d % 256 == 0 and d_ff % 128 == 0.
 * n_rows = offsets[n_groups] (rows of out).
 * workspace: device, at least ft_grouped_ffn_mx_workspace_bytes(T, d, d_ff, n_rows)
 * bytes, 256-byte aligned; FT_ENOMEM when smaller.  It holds, each part starting at
 * a 256-byte boundary: h fp32 [n_rows, d_ff]; x in MXFP8, codes [T, d] then scales
 * [T, d/32]; h in MXFP8, codes [n_rows, d_ff] then scales [n_rows, d_ff/32]
 * (form 1 writes h fp32 only; form 2 writes the two MXFP8 parts only, converting
 * h inside the gate/up kernel).  These are readable after the call. */
size_t ft_grouped_ffn_mx_workspace_bytes(int32_t T, int32_t d, int32_t d_ff, int32_t n_rows);
int ft_grouped_ffn_mx(const void* x, int32_t T, int32_t d, int32_t d_ff, int32_t k,
                      const void* slots, const int32_t* group_slot, const int32_t* offsets,
                      const int32_t* perm, int32_t n_groups, int32_t g_begin, int32_t g_end,
                      int32_t max_rows_per_group, int32_t n_rows, void* workspace,
                      size_t workspace_bytes, float* out, int32_t form, void* stream);

/* Gate-weighted combine and exact merge ([FT] §3.2: the GPU and CPU partial sums
 * merge into the exact MoE output):  y[t] = sum_{j: inv[t*k+j] >= 0, in j order}
 * gates[t*k+j] * out[inv[t*k+j]]  +  cpu_partial[t]  (cpu_partial may be NULL).
 * All device; y fp32 [T, d]; 1 <= k <= 8 and d % 4 == 0, else FT_EINVAL. */
int ft_combine(const float* out, const int32_t* inv, const float* gates,
               const float* cpu_partial, int32_t T, int32_t k, int32_t d, float* y,
               void* stream);

/* Host expert kernel, the CPU branch of a decode call ([FT] §3.2: experts of C run
 * in place from the host pool and return gate-weighted per-token partials; §4.1:
 * persistent workers with SIMD kernels that dequantise in place).  For n_exp experts
 * with records `records[i]` of format fmt (ft_wfmt; host or pinned) and uses u in
 * [use_off[i], use_off[i+1]) of token use_t[u] with gate use_g[u]:
 * partial[t] = sum over uses of g * FFN_i(x[t]), fp32, overwritten (MXFP4 weights
 * exactly dequantised, activations bf16).  x: host bf16 [T, d].  threads: workers
 * of a pool made for this call (0 = default count).  At most 64 uses per expert. */
int ft_host_experts(const void* x, int32_t T, int32_t d, int32_t d_ff, int32_t fmt,
                    const void* const* records, const int32_t* use_off, const int32_t* use_t,
                    const float* use_g, int32_t n_exp, int32_t threads, float* partial);

/* ---- expert cache -------------------------------------------------------------- */

/* Decisions of one decode call for routed ids idx_host (host int32 [T, k]):
 * dedup, classify, split (ft_qstar_split with avail = n_slots - |H|), victims
 * (non-hit slots by (recency, slot), empty first), LRU update (H and F touched in
 * U order) and the slot rewrite ([FT] §3.2, §4.1).  Updates the residency state
 * and counters; copies nothing.  T*k <= FT_PLAN_CAP. */
int ft_expert_cache_lookup(ft_ctx_t ctx, int32_t layer, const int32_t* idx_host, int32_t T,
                           ft_plan* plan);

/* The decisions of one on-demand prefill layer (see ft_prefill_plan) for the
 * chunk's routed ids idx_host [T, k], in a decisions-only context with an
 * on-demand prefill open: updates residency and copies nothing.  FT_ECAP when a
 * miss has no slot. */
int ft_expert_cache_prefill_on_demand(ft_ctx_t ctx, int32_t layer, const int32_t* idx_host, int32_t T,
                                      ft_prefill_plan* plan);

/* Copies the q records of plan->F into their slots with hipMemcpyAsync on
 * `copy` (pinned host -> device; [FT] §3.2: fills proceed at the full PCIe rate).
 * Waits on wait_event first if not NULL; records done_event after if not NULL. */
int ft_expert_cache_fill(ft_ctx_t ctx, const ft_plan* plan, void* copy, void* wait_event,
                         void* done_event);

/* Rebuilds the cache over new_dev_slots (n_slots records; may equal the old
 * buffer) at a safe point ([FT] §3.3): all slots empty, counters reset, recency
 * clock kept.  FT_EBUSY if work the library issued is still running or a prefill
 * is open.  Returns FT_WOVERLAP_OFF when prefill overlap had to be disabled
 * (n_slots < 2E). */
int ft_expert_cache_resize(ft_ctx_t ctx, void* new_dev_slots, int32_t new_n_slots);

/* Residency of one (layer, expert): slot or -1. */
int32_t ft_expert_cache_where(ft_ctx_t ctx, int32_t layer, int32_t expert);

/* ---- layer forward ----------------------------------------------------------------- */

/* One decode call of one MoE layer ([FT] §3.2, "In execution order"; §4.1,
 * device-side cache control), every GPU step on `compute`: the router takes the
 * call's decisions on the device (dedup, classify, q*, victims, stamps, grouping)
 * and publishes ids, gates, x and a hash of the plan to pinned host memory; the
 * fills of F are read by the GPU from the pinned pool over PCIe into the chosen
 * slots; the grouped FFN of G = H then F.  Meanwhile the host controller takes
 * the same decisions from the published ids (FT_EHIP if they differ from the
 * device's) and runs the CPU branch (C) on the worker pool; then the merge of the
 * CPU partial and the combine into y.  Returns when y is enqueued on `compute`
 * (the CPU branch has finished).  The pool must be GPU-readable pinned memory
 * (hipHostMalloc).
 * x: device bf16 [T, d]; w_router: device bf16 [E, d]; allowed: device uint8
 * [T, E] or NULL; y: device fp32 [T, d].  plan, stats: host, may be NULL.
 * T <= min(T_max, FT_PLAN_CAP / k, 64). */
int ft_moe_decode_layer(ft_ctx_t ctx, int32_t layer, const void* x, int32_t T,
                        const void* w_router, const uint8_t* allowed, float* y, void* compute,
                        ft_plan* plan, ft_step_stats* stats);

/* ---- graph-resident decode step ([FT] §4.1 "Graph-resident CPU execution") -------
 * One decode step through every layer (0..L-1 in order) replayed from one HIP graph.
 * Per layer, on one chain: the router with the device's cache decisions, the fills of
 * F read over PCIe, the grouped FFN of G = H then F, and the combine; forked off after
 * the router, a host node that takes the host controller's decisions from the
 * published ids, checks them against the device's (plan hash) and runs the CPU branch
 * (C) on the worker pool; the combine waits for both.  The same kernels, decisions
 * and arithmetic as ft_moe_decode_layer.
 * Fixed buffers, owned by the caller, read or written at every launch: x device bf16
 * [L, T, d] (layer l's input at x + l*T*d), allowed device uint8 [L, T, E] or NULL,
 * y device fp32 [L, T, d]; w_router: host array of L device pointers (bf16 [E, d]).
 * The caller writes each step's inputs into x (and allowed) before the launch.
 * create: captures and instantiates the graph for T tokens (1 <= T <= min(T_max,
 * FT_PLAN_CAP / k, 64)).
 * launch: enqueues one step on `stream` (asynchronous) after everything the context
 * issued before; first returns the error, if any, that an earlier step's host node
 * met (FT_EHIP: the device's decisions differed from the host's; FT_EINVAL: a token
 * allowed fewer than k experts).  The device keeps deciding for that step's later
 * layers while the host nodes stop, so the cache was emptied; that step's y is
 * undefined from the failing layer on.  Re-captures the graph
 * when a resize or a larger cache state changed what the kernels were built with.
 * While steps are in flight the host nodes update the context's host state: make no
 * other call on the context (except further launches on the same stream) until the
 * stream is synchronised.  status: the error an earlier step's host node met, or
 * FT_OK (clears it).  FT_EBUSY while a prefill is open. */
typedef struct ft_decode_graph* ft_decode_graph_t;
int ft_decode_graph_create(ft_ctx_t ctx, int32_t T, const void* x, const void* const* w_router,
                           const uint8_t* allowed, float* y, ft_decode_graph_t* out);
int ft_decode_graph_launch(ft_decode_graph_t graph, void* stream);
int ft_decode_graph_status(ft_decode_graph_t graph);
int ft_decode_graph_destroy(ft_decode_graph_t graph);

/* Prefill ([FT] §3.1; §5.3 "Pipelined prefill"), layers in order 0..L-1.
 * Full-layer double buffering, with overlap on and at least 2E slots:
 * begin: reserve two buffers of E slots (victim order) and start loading layer 0
 * on `copy`.  layer: start loading layer l+1 into the other buffer once layer
 * l-1's compute is done, then compute layer l (router, grouping, grouped FFN,
 * combine) from its buffer once its load landed.  end: waits for any layer load
 * still in flight; then the layers the two buffers hold stay resident for decode:
 * L-2 and L-1 after a whole pass; after a pass ended early at n layers, layer n-1
 * and layer n (streamed in while n-1 computed); a buffer whose load was not issued
 * completely (a failed call) holds no layer and its slots become empty.
 * On-demand, with overlap off or fewer than 2E slots (the pages' fallback): begin
 * reserves nothing; layer routes, brings the ids to the host, takes the decisions
 * of ft_expert_cache_prefill_on_demand, runs the hits' FFN, then per round loads
 * the round's misses on `copy` and runs their FFN once they landed, and combines;
 * FT_ECAP when a miss has no slot.  end only closes the prefill.
 * In a decisions-only context begin/end change residency only (no copies). */
int ft_moe_prefill_begin(ft_ctx_t ctx, void* copy);
int ft_moe_prefill_layer(ft_ctx_t ctx, int32_t layer, const void* x, int32_t T,
                         const void* w_router, float* y, void* compute, void* copy);
int ft_moe_prefill_end(ft_ctx_t ctx);

/* The routed ids (int32 [T, k]) and gates (fp32 [T, k]) of the context's last
 * successful ft_moe_decode_layer or ft_moe_prefill_layer call ([FT] §3.2: the
 * router's top-k and renormalised gates), copied out of the device workspace into
 * idx and gates (device or host memory; either may be NULL) with hipMemcpyAsync on
 * `stream`, which the caller orders after that call (its compute stream does).  T
 * must be that call's T.  FT_EINVAL before any layer call or for another T. */
int ft_layer_routing(ft_ctx_t ctx, int32_t* idx, float* gates, int32_t T, void* stream);

/* Device slot of expert e in the buffer serving `layer` during prefill, or -1. */
int32_t ft_prefill_slot(ft_ctx_t ctx, int32_t layer, int32_t expert);

/* ---- kernel timing ---------------------------------------------------------------
 * When enabled, each of the two kernels of every grouped-FFN launch issued by
 * ft_moe_decode_layer and ft_moe_prefill_layer is launched with start and stop
 * events that bracket the kernel itself (hipExtLaunchKernel), and
 * its algorithmic bytes and flops are recorded: per expert group of n rows,
 *   gate/up: 2*d*d_ff*2 weight bytes + n*d*2 (x) + n*d_ff*hb (h), 2*2*n*d*d_ff flops
 *   down:    d*d_ff*2 weight bytes + n*d_ff*hb (h) + n*d*4 (out), 2*n*d*d_ff flops
 * with hb = 4 in the row-streaming form and 2 in the MFMA form; groups with n = 0
 * count nothing.  enable(1) clears what was recorded; read() waits for the
 * recorded events and sums them. */
typedef struct {
  int64_t launches;
  double ms_gateup, ms_down;
  double bytes_gateup, bytes_down;
  double flops_gateup, flops_down;
} ft_profile;
int ft_profile_enable(ft_ctx_t ctx, int32_t on);
int ft_profile_read(ft_ctx_t ctx, ft_profile* out);

/* ---- placement replay ([FT] §5.3 "Expert locality", Fig. 4b) ---------------------
 * Replays a routing trace against one placement policy at a cache of n_slots
 * (layer, expert) pairs and counts the decode-time expert reads and how many of
 * them miss the GPU.  Host only; touches no device.
 *   ids int32 [n_requests][prompt + decode][L][k], expert ids in [0, E): requests
 *   served one after another at batch 1, `prompt` prefill tokens then `decode`
 *   decode steps each; only the decode steps are counted (k reads per step and
 *   layer).
 * Policies:
 *   FT_PLACE_LRU     the engine's global LRU (the controller ft_moe_decode_layer
 *                    uses) with every miss filled (q = m); each prefill is the
 *                    engine's: two full-layer buffers when n_slots >= 2E (the last
 *                    two layers stay), else on-demand loading of each layer's routed
 *                    experts (FT_ECAP when a miss finds no slot).  The cache
 *                    persists across requests.
 *   FT_PLACE_HOTSET  after each prefill the resident set becomes the n_slots pairs
 *                    that prefill routed most often (ties to the lower l*E + e, pairs
 *                    never routed fill the rest in that order); fixed during decode.
 *   FT_PLACE_STATIC  routing-blind: the last n_slots pairs in l*E + e order.
 * E <= FT_E_MAX, 1 <= k <= min(8, E).  FT_EINVAL for bad arguments or ids. */
#define FT_PLACE_LRU 0
#define FT_PLACE_HOTSET 1
#define FT_PLACE_STATIC 2
int ft_replay_placement(int32_t policy, const ft_shape* shape, int32_t n_slots, const int32_t* ids,
                        int32_t n_requests, int32_t prompt, int32_t decode, int64_t* reads,
                        int64_t* misses);

#ifdef __cplusplus
}
#endif
#endif /* FT_H */
