// C ABI of libft: context, decode and prefill orchestration, cache control,
// bandwidth probe.  See include/ft.h for the contract of each call.
//
// [FT] = "FreeToken: Efficient Edge-Native MoE Serving with Bandwidth-Adaptive
// Execution" (arXiv 2608.16157).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstring>
#include <string>
#include <vector>

#include "cache.h"
#include "internal.h"

namespace ft {

namespace {
thread_local std::string g_last_error;
}

void set_error(const std::string& msg) { g_last_error = msg; }
int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

}  // namespace ft

using ft::fail;

namespace {

double now_us() {
  return std::chrono::duration<double, std::micro>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

#define FT_HIP(call)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess) return fail(FT_EHIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
  } while (0)

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool shape_ok(const ft_shape* s) {
  return s && s->L > 0 && s->E > 0 && s->E <= 1024 && s->d > 0 && s->d % 8 == 0 && s->d_ff > 0 &&
         s->d_ff % 8 == 0 && s->k >= 1 && s->k <= 8 && s->k <= s->E && s->fmt == FT_W_BF16;
}

// Workspace carve: offsets of each device array for calls of up to T_max tokens.
struct Carve {
  size_t idx, gates, logits, key, gslot, bufslot, offsets, perm, inv, pws, h, out, cpu, total;
  size_t pws_bytes;
  int g_max;
};

Carve carve(const ft_shape* s, int T_max) {
  Carve c{};
  const size_t P = (size_t)T_max * s->k;
  const int t_dec = std::max(1, std::min(std::min(T_max, FT_PLAN_CAP / s->k), 64));
  c.g_max = std::max(s->E, std::min((int)P, FT_PLAN_CAP));
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  c.idx = take(P * 4);
  c.gates = take(P * 4);
  c.logits = take((size_t)T_max * s->E * 4);
  c.key = take(P * 4);
  c.gslot = take((size_t)c.g_max * 4);
  c.bufslot = take((size_t)2 * s->E * 4);
  c.offsets = take((size_t)(c.g_max + 1) * 4);
  c.perm = take(P * 4);
  c.inv = take(P * 4);
  c.pws_bytes = ft::permute_ws_bytes((int)P, c.g_max);
  c.pws = take(c.pws_bytes);
  c.h = take(P * s->d_ff * 4);
  c.out = take(P * s->d * 4);
  c.cpu = take((size_t)t_dec * s->d * 4);
  c.total = o;
  return c;
}

}  // namespace

struct ft_ctx {
  ft_shape shape{};
  ft_config cfg{};
  size_t S = 0, rec_elems = 0;
  const uint16_t* pool = nullptr;
  size_t pool_bytes = 0;
  int L_phys = 0;
  uint16_t* slots = nullptr;
  uint8_t* ws = nullptr;
  size_t ws_bytes = 0;
  Carve cv{};
  int t_dec = 0;
  int device = 0;
  bool dev = false;  // device path available
  bool overlap = false;

  // pinned staging
  int32_t* h_idx = nullptr;
  float* h_gates = nullptr;
  uint16_t* h_x = nullptr;
  int32_t* h_key = nullptr;
  int32_t* h_gslot = nullptr;
  float* h_partial = nullptr;

  hipEvent_t ev_route = nullptr, ev_fill = nullptr, ev_done = nullptr;
  hipEvent_t ev_pf_fill[2] = {nullptr, nullptr}, ev_pf_comp[2] = {nullptr, nullptr};

  ft::ExpertCache* cache = nullptr;
  ft::CpuPool* cpu = nullptr;
  std::vector<ft::CpuExpert> cpu_ex;
  ft_plan scratch_plan{};
  int prefill_next = -1;

  template <typename T>
  T* wsp(size_t off) const { return reinterpret_cast<T*>(ws + off); }
  const uint16_t* record(int layer, int e) const {
    return pool + ((size_t)(layer % L_phys) * shape.E + e) * rec_elems;
  }
  uint16_t* slot_ptr(int s) const { return slots + (size_t)s * rec_elems; }
};

extern "C" {

const char* ft_strerror(int st) {
  switch (st) {
    case FT_OK: return "ok";
    case FT_EINVAL: return "invalid argument";
    case FT_ENOMEM: return "out of memory or buffer too small";
    case FT_EBUSY: return "not at a safe point";
    case FT_ENOPIN: return "host pool is not pinned";
    case FT_ECAP: return "prefill overlap needs at least 2E slots";
    case FT_EHIP: return "HIP error";
    case FT_EUNSUPPORTED: return "unsupported";
    case FT_WOVERLAP_OFF: return "warning: prefill overlap disabled";
    default: return "unknown status";
  }
}

const char* ft_last_error(void) { return ft::g_last_error.c_str(); }

size_t ft_record_bytes(const ft_shape* s) {
  if (!shape_ok(s)) return 0;
  return (size_t)6 * s->d * s->d_ff;
}

size_t ft_workspace_bytes(const ft_shape* s, int32_t T_max) {
  if (!shape_ok(s) || T_max < 1) return 0;
  return carve(s, T_max).total;
}

int ft_pool_alloc(size_t bytes, void** out) {
  if (!out || bytes == 0) return fail(FT_EINVAL, "pool_alloc: null out or zero size");
  void* p = nullptr;
  hipError_t e = hipHostMalloc(&p, bytes, hipHostMallocDefault);
  if (e != hipSuccess || !p) return fail(FT_ENOMEM, std::string("hipHostMalloc: ") + hipGetErrorString(e));
  *out = p;
  return FT_OK;
}

int ft_pool_free(void* p) {
  if (!p) return FT_OK;
  FT_HIP(hipHostFree(p));
  return FT_OK;
}

int ft_create(const ft_shape* shape, const ft_config* config, const void* host_pool,
              size_t pool_bytes, void* dev_slots, int32_t n_slots, void* dev_workspace,
              size_t workspace_bytes, ft_ctx_t* out) {
  if (!out) return fail(FT_EINVAL, "create: null out");
  *out = nullptr;
  if (!shape_ok(shape)) return fail(shape && shape->fmt != FT_W_BF16 ? FT_EUNSUPPORTED : FT_EINVAL, "create: bad shape");
  if (!config || config->T_max < 1 || config->frac_q16 > 65536u || n_slots < 0 || config->max_fetch < -1)
    return fail(FT_EINVAL, "create: bad config");
  if (config->prefill_overlap && n_slots < 2 * shape->E)
    return fail(FT_ECAP, "create: prefill overlap needs n_slots >= 2E");
  ft_ctx* c = new ft_ctx();
  c->shape = *shape;
  c->cfg = *config;
  c->L_phys = config->L_phys > 0 ? std::min(config->L_phys, shape->L) : shape->L;
  c->cfg.L_phys = c->L_phys;
  c->S = ft_record_bytes(shape);
  c->rec_elems = c->S / 2;
  c->overlap = config->prefill_overlap != 0;
  c->t_dec = std::max(1, std::min(std::min(config->T_max, FT_PLAN_CAP / shape->k), 64));
  c->cache = new ft::ExpertCache(shape->L, shape->E, n_slots);
  c->cv = carve(shape, config->T_max);
  if (host_pool != nullptr || dev_slots != nullptr || dev_workspace != nullptr) {
    auto bail = [&](int st, const std::string& m) {
      ft_destroy(c);
      return fail(st, m);
    };
    if (!host_pool || !dev_workspace || (n_slots > 0 && !dev_slots))
      return bail(FT_EINVAL, "create: host_pool, dev_slots and dev_workspace go together");
    if (pool_bytes < (size_t)c->L_phys * shape->E * c->S) return bail(FT_ENOMEM, "create: host pool too small");
    if (workspace_bytes < c->cv.total) return bail(FT_ENOMEM, "create: workspace too small");
    if ((reinterpret_cast<uintptr_t>(dev_slots) | reinterpret_cast<uintptr_t>(dev_workspace)) & 255)
      return bail(FT_EINVAL, "create: device buffers must be 256-byte aligned");
    hipPointerAttribute_t attr;
    hipError_t pe = hipPointerGetAttributes(&attr, host_pool);
    if (pe != hipSuccess || attr.type != hipMemoryTypeHost) {
      (void)hipGetLastError();
      return bail(FT_ENOPIN, "create: host pool is not pinned host memory");
    }
    if (hipGetDevice(&c->device) != hipSuccess) return bail(FT_EHIP, "create: hipGetDevice failed");
    c->pool = static_cast<const uint16_t*>(host_pool);
    c->pool_bytes = pool_bytes;
    c->slots = static_cast<uint16_t*>(dev_slots);
    c->ws = static_cast<uint8_t*>(dev_workspace);
    c->ws_bytes = workspace_bytes;
    const size_t P = (size_t)FT_PLAN_CAP;
    if (hipHostMalloc((void**)&c->h_idx, P * 4) != hipSuccess ||
        hipHostMalloc((void**)&c->h_gates, P * 4) != hipSuccess ||
        hipHostMalloc((void**)&c->h_x, (size_t)c->t_dec * shape->d * 2) != hipSuccess ||
        hipHostMalloc((void**)&c->h_key, P * 4) != hipSuccess ||
        hipHostMalloc((void**)&c->h_gslot, (size_t)(c->cv.g_max + 2 * shape->E) * 4) != hipSuccess ||
        hipHostMalloc((void**)&c->h_partial, (size_t)c->t_dec * shape->d * 4) != hipSuccess)
      return bail(FT_ENOMEM, "create: pinned staging allocation failed");
    hipEvent_t* evs[] = {&c->ev_route, &c->ev_fill, &c->ev_done, &c->ev_pf_fill[0], &c->ev_pf_fill[1],
                         &c->ev_pf_comp[0], &c->ev_pf_comp[1]};
    for (hipEvent_t* e : evs)
      if (hipEventCreateWithFlags(e, hipEventDisableTiming) != hipSuccess)
        return bail(FT_EHIP, "create: hipEventCreate failed");
    c->cpu = ft::cpu_pool_create(config->cpu_threads);
    c->cfg.cpu_threads = ft::cpu_pool_threads(c->cpu);
    c->dev = true;
  }
  *out = c;
  return FT_OK;
}

int ft_destroy(ft_ctx_t c) {
  if (!c) return FT_OK;
  if (c->dev) {
    (void)hipSetDevice(c->device);
    (void)hipDeviceSynchronize();
  }
  if (c->cpu) ft::cpu_pool_destroy(c->cpu);
  hipEvent_t evs[] = {c->ev_route, c->ev_fill, c->ev_done, c->ev_pf_fill[0], c->ev_pf_fill[1],
                      c->ev_pf_comp[0], c->ev_pf_comp[1]};
  for (hipEvent_t e : evs)
    if (e) (void)hipEventDestroy(e);
  void* pins[] = {c->h_idx, c->h_gates, c->h_x, c->h_key, c->h_gslot, c->h_partial};
  for (void* p : pins)
    if (p) (void)hipHostFree(p);
  delete c->cache;
  delete c;
  return FT_OK;
}

int ft_get_stats(ft_ctx_t c, ft_stats* out) {
  if (!c || !out) return fail(FT_EINVAL, "get_stats: null");
  *out = c->cache->stats;
  return FT_OK;
}

int ft_reset_stats(ft_ctx_t c) {
  if (!c) return fail(FT_EINVAL, "reset_stats: null");
  const int64_t r = c->cache->stats.resizes;
  c->cache->stats = ft_stats{};
  c->cache->stats.resizes = r;
  return FT_OK;
}

int ft_get_config(ft_ctx_t c, ft_config* out) {
  if (!c || !out) return fail(FT_EINVAL, "get_config: null");
  *out = c->cfg;
  out->prefill_overlap = c->overlap ? 1 : 0;
  return FT_OK;
}

int32_t ft_n_slots(ft_ctx_t c) { return c ? c->cache->n_slots() : FT_EINVAL; }

int32_t ft_expert_cache_where(ft_ctx_t c, int32_t layer, int32_t expert) {
  return c ? c->cache->where(layer, expert) : -1;
}

int32_t ft_prefill_slot(ft_ctx_t c, int32_t layer, int32_t expert) {
  return c ? c->cache->prefill_slot(layer, expert) : -1;
}

// ---- stateless kernels --------------------------------------------------------

int ft_router_topk(const void* x, const void* w_router, const uint8_t* allowed, int32_t T, int32_t d,
                   int32_t E, int32_t k, int32_t* idx, float* gates, float* logits, void* stream) {
  if (!logits && T > 0) return fail(FT_EINVAL, "router: logits buffer is required");
  return ft::launch_router(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router), allowed, T, d,
                           E, k, idx, gates, logits, stream);
}

size_t ft_permute_workspace_bytes(int32_t P, int32_t n_groups) { return ft::permute_ws_bytes(P, n_groups); }

int ft_permute(const int32_t* key, int32_t P, int32_t n_groups, int32_t* offsets, int32_t* perm,
               int32_t* inv, void* workspace, size_t workspace_bytes, void* stream) {
  return ft::launch_permute(key, P, n_groups, offsets, perm, inv, workspace, workspace_bytes, stream);
}

int ft_grouped_ffn(const void* x, int32_t T, int32_t d, int32_t d_ff, int32_t k, const void* slots,
                   const int32_t* group_slot, const int32_t* offsets, const int32_t* perm,
                   int32_t n_groups, int32_t g_begin, int32_t g_end, int32_t max_rows_per_group,
                   void* h_ws, float* out, int32_t form, void* stream) {
  if (T < 0 || g_begin < 0 || g_end > n_groups || g_begin > g_end) return fail(FT_EINVAL, "grouped_ffn: bad group range");
  const bool mfma_ok = d % 128 == 0 && d_ff % 64 == 0;
  if (form == 0) form = (mfma_ok && max_rows_per_group >= 32) ? 2 : 1;
  if (form == 2) {
    if (!mfma_ok) return fail(FT_EINVAL, "grouped_ffn: MFMA form needs d%128==0 and d_ff%64==0");
    return ft::launch_ffn_mfma(static_cast<const uint16_t*>(x), d, d_ff, k, static_cast<const uint16_t*>(slots),
                               group_slot, offsets, perm, g_begin, g_end, max_rows_per_group,
                               static_cast<uint16_t*>(h_ws), out, stream);
  }
  if (form != 1) return fail(FT_EINVAL, "grouped_ffn: form must be 0, 1 or 2");
  return ft::launch_ffn_rows(static_cast<const uint16_t*>(x), d, d_ff, k, static_cast<const uint16_t*>(slots),
                             group_slot, offsets, perm, g_begin, g_end, max_rows_per_group,
                             static_cast<float*>(h_ws), out, stream);
}

int ft_combine(const float* out, const int32_t* inv, const float* gates, const float* cpu_partial,
               int32_t T, int32_t k, int32_t d, float* y, void* stream) {
  return ft::launch_combine(out, inv, gates, cpu_partial, T, k, d, y, stream);
}

// ---- cache control --------------------------------------------------------------

int ft_expert_cache_lookup(ft_ctx_t c, int32_t layer, const int32_t* idx_host, int32_t T, ft_plan* plan) {
  if (!c || !idx_host || !plan) return fail(FT_EINVAL, "lookup: null argument");
  return c->cache->lookup(layer, idx_host, T, c->shape.k, c->cfg.frac_q16, c->cfg.min_fill,
                          c->cfg.max_fetch, plan);
}

int ft_expert_cache_fill(ft_ctx_t c, const ft_plan* p, void* copy, void* wait_event, void* done_event) {
  if (!c || !p) return fail(FT_EINVAL, "fill: null argument");
  if (!c->dev) return fail(FT_EINVAL, "fill: context has no device path");
  if (p->q < 0 || p->q > p->n_m || p->layer < 0 || p->layer >= c->shape.L) return fail(FT_EINVAL, "fill: bad plan");
  FT_HIP(hipSetDevice(c->device));
  hipStream_t cs = static_cast<hipStream_t>(copy);
  if (wait_event) FT_HIP(hipStreamWaitEvent(cs, static_cast<hipEvent_t>(wait_event), 0));
  for (int i = 0; i < p->q; ++i) {
    if (p->F_slot[i] < 0 || p->F_slot[i] >= c->cache->n_slots()) return fail(FT_EINVAL, "fill: slot out of range");
    FT_HIP(hipMemcpyAsync(c->slot_ptr(p->F_slot[i]), c->record(p->layer, p->M[i]), c->S, hipMemcpyHostToDevice, cs));
  }
  c->cache->stats.h2d_bytes += (int64_t)p->q * (int64_t)c->S;
  if (done_event) FT_HIP(hipEventRecord(static_cast<hipEvent_t>(done_event), cs));
  return FT_OK;
}

int ft_expert_cache_resize(ft_ctx_t c, void* new_dev_slots, int32_t n) {
  if (!c || n < 0) return fail(FT_EINVAL, "resize: bad argument");
  if (c->cache->prefill_open()) return fail(FT_EBUSY, "resize: a prefill is open");
  if (c->dev) {
    if (n > 0 && (!new_dev_slots || (reinterpret_cast<uintptr_t>(new_dev_slots) & 255)))
      return fail(FT_EINVAL, "resize: need a 256-byte aligned slot buffer");
    FT_HIP(hipSetDevice(c->device));
    hipEvent_t evs[] = {c->ev_route, c->ev_fill, c->ev_done, c->ev_pf_fill[0], c->ev_pf_fill[1],
                        c->ev_pf_comp[0], c->ev_pf_comp[1]};
    for (hipEvent_t e : evs) {
      const hipError_t q = hipEventQuery(e);
      if (q == hipErrorNotReady) return fail(FT_EBUSY, "resize: issued work still running");
      if (q != hipSuccess) return fail(FT_EHIP, std::string("resize: hipEventQuery: ") + hipGetErrorString(q));
    }
    c->slots = static_cast<uint16_t*>(new_dev_slots);
  }
  c->cache->resize(n);
  c->cache->stats.resizes += 1;
  if (c->overlap && n < 2 * c->shape.E) {
    c->overlap = false;
    ft::set_error("resize: fewer than 2E slots, prefill overlap disabled");
    return FT_WOVERLAP_OFF;
  }
  return FT_OK;
}

// ---- decode ------------------------------------------------------------------------

int ft_moe_decode_layer(ft_ctx_t c, int32_t layer, const void* x, int32_t T, const void* w_router,
                        const uint8_t* allowed, float* y, void* compute, void* copy, ft_plan* plan_out,
                        ft_step_stats* st) {
  const double t0 = now_us();
  if (!c || !x || !w_router || !y) return fail(FT_EINVAL, "decode: null argument");
  if (!c->dev) return fail(FT_EINVAL, "decode: context has no device path");
  const int k = c->shape.k, d = c->shape.d, E = c->shape.E;
  if (layer < 0 || layer >= c->shape.L || T < 1 || T > c->t_dec) return fail(FT_EINVAL, "decode: bad layer or T");
  if (c->cache->prefill_open()) return fail(FT_EBUSY, "decode: a prefill is open");
  const int P = T * k;
  FT_HIP(hipSetDevice(c->device));
  hipStream_t cs = static_cast<hipStream_t>(compute);
  hipStream_t ps = static_cast<hipStream_t>(copy);
  int32_t* d_idx = c->wsp<int32_t>(c->cv.idx);
  float* d_gates = c->wsp<float>(c->cv.gates);
  // order after everything this context issued before, whatever the stream
  FT_HIP(hipStreamWaitEvent(cs, c->ev_done, 0));
  if (int rc = ft::launch_router(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router), allowed,
                                 T, d, E, k, d_idx, d_gates, c->wsp<float>(c->cv.logits), cs))
    return rc;
  FT_HIP(hipMemcpyAsync(c->h_idx, d_idx, (size_t)P * 4, hipMemcpyDeviceToHost, cs));
  FT_HIP(hipMemcpyAsync(c->h_gates, d_gates, (size_t)P * 4, hipMemcpyDeviceToHost, cs));
  FT_HIP(hipMemcpyAsync(c->h_x, x, (size_t)T * d * 2, hipMemcpyDeviceToHost, cs));
  FT_HIP(hipEventRecord(c->ev_route, cs));
  FT_HIP(hipEventSynchronize(c->ev_route));
  const double t1 = now_us();
  for (int i = 0; i < P; ++i)
    if (c->h_idx[i] < 0) return fail(FT_EINVAL, "decode: a token allows fewer than k experts");

  ft_plan* p = plan_out ? plan_out : &c->scratch_plan;
  if (int rc = c->cache->lookup(layer, c->h_idx, T, k, c->cfg.frac_q16, c->cfg.min_fill, c->cfg.max_fetch, p))
    return rc;
  std::memcpy(p->idx, c->h_idx, (size_t)P * 4);
  std::memcpy(p->gates, c->h_gates, (size_t)P * 4);
  const int n_h = p->n_h, q = p->q, n_c = p->n_c, n_g = n_h + q;
  const double t2 = now_us();

  // CPU branch first ([FT] §3.2, "In execution order")
  if (n_c > 0) {
    c->cpu_ex.resize(n_c);
    for (int i = 0; i < n_c; ++i) {
      ft::CpuExpert& ex = c->cpu_ex[i];
      const int e = p->M[q + i];
      ex.rec = c->record(layer, e);
      ex.n_use = 0;
      for (int pr = 0; pr < P; ++pr)
        if (c->h_idx[pr] == e && ex.n_use < 64) ex.use[ex.n_use++] = ft::CpuUse{pr / k, c->h_gates[pr]};
    }
    ft::cpu_pool_submit(c->cpu, c->h_x, T, d, c->shape.d_ff, c->cpu_ex.data(), n_c, c->h_partial);
  }
  // fills of F on the copy stream
  if (q > 0) {
    FT_HIP(hipStreamWaitEvent(ps, c->ev_route, 0));
    for (int i = 0; i < q; ++i)
      FT_HIP(hipMemcpyAsync(c->slot_ptr(p->F_slot[i]), c->record(layer, p->M[i]), c->S, hipMemcpyHostToDevice, ps));
    FT_HIP(hipEventRecord(c->ev_fill, ps));
    c->cache->stats.h2d_bytes += (int64_t)q * (int64_t)c->S;
  }
  // GPU path: grouping, grouped FFN of H, then of F once filled
  int32_t* d_key = c->wsp<int32_t>(c->cv.key);
  int32_t* d_gslot = c->wsp<int32_t>(c->cv.gslot);
  int32_t* d_off = c->wsp<int32_t>(c->cv.offsets);
  int32_t* d_perm = c->wsp<int32_t>(c->cv.perm);
  int32_t* d_inv = c->wsp<int32_t>(c->cv.inv);
  float* d_h = c->wsp<float>(c->cv.h);
  float* d_out = c->wsp<float>(c->cv.out);
  std::memcpy(c->h_key, p->pair_group, (size_t)P * 4);
  std::memcpy(c->h_gslot, p->G_slot, (size_t)std::max(n_g, 1) * 4);
  int max_rows = 0;
  {
    int cnt[FT_PLAN_CAP] = {0};
    for (int i = 0; i < P; ++i)
      if (p->pair_group[i] >= 0) max_rows = std::max(max_rows, ++cnt[p->pair_group[i]]);
  }
  FT_HIP(hipMemcpyAsync(d_key, c->h_key, (size_t)P * 4, hipMemcpyHostToDevice, cs));
  if (n_g > 0) FT_HIP(hipMemcpyAsync(d_gslot, c->h_gslot, (size_t)n_g * 4, hipMemcpyHostToDevice, cs));
  if (int rc = ft::launch_permute(d_key, P, std::max(n_g, 1), d_off, d_perm, d_inv, c->ws + c->cv.pws,
                                  c->cv.pws_bytes, cs))
    return rc;
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  if (n_h > 0)
    if (int rc = ft::launch_ffn_rows(xs, d, c->shape.d_ff, k, c->slots, d_gslot, d_off, d_perm, 0, n_h, max_rows,
                                     d_h, d_out, cs))
      return rc;
  if (q > 0) {
    FT_HIP(hipStreamWaitEvent(cs, c->ev_fill, 0));
    if (int rc = ft::launch_ffn_rows(xs, d, c->shape.d_ff, k, c->slots, d_gslot, d_off, d_perm, n_h, n_g, max_rows,
                                     d_h, d_out, cs))
      return rc;
  }
  // merge of the CPU partial, then the combine
  const float* cpu_part = nullptr;
  double t_cpu = 0.0;
  if (n_c > 0) {
    ft::cpu_pool_wait(c->cpu);
    t_cpu = now_us() - t2;
    float* d_cpu = c->wsp<float>(c->cv.cpu);
    FT_HIP(hipMemcpyAsync(d_cpu, c->h_partial, (size_t)T * d * 4, hipMemcpyHostToDevice, cs));
    cpu_part = d_cpu;
  }
  if (int rc = ft::launch_combine(d_out, d_inv, d_gates, cpu_part, T, k, d, y, cs)) return rc;
  FT_HIP(hipEventRecord(c->ev_done, cs));
  if (st) {
    st->layer = layer;
    st->T = T;
    st->n_u = p->n_u;
    st->hits = n_h;
    st->misses = p->n_m;
    st->q = q;
    st->n_c = n_c;
    st->h2d_bytes = (int64_t)q * (int64_t)c->S;
    st->t_route_us = t1 - t0;
    st->t_ctrl_us = t2 - t1;
    st->t_cpu_us = t_cpu;
    st->t_total_us = now_us() - t0;
  }
  return FT_OK;
}

// ---- prefill -----------------------------------------------------------------------

static int enqueue_layer_load(ft_ctx_t c, int layer, hipStream_t ps) {
  const std::vector<int32_t>& b = c->cache->prefill_buffer(layer & 1);
  const int E = c->shape.E;
  int e = 0;
  while (e < E) {
    int run = 1;
    while (e + run < E && b[e + run] == b[e] + run) ++run;
    FT_HIP(hipMemcpyAsync(c->slot_ptr(b[e]), c->record(layer, e), (size_t)run * c->S, hipMemcpyHostToDevice, ps));
    e += run;
  }
  c->cache->stats.h2d_bytes += (int64_t)E * (int64_t)c->S;
  return FT_OK;
}

int ft_moe_prefill_begin(ft_ctx_t c, void* copy) {
  if (!c) return fail(FT_EINVAL, "prefill_begin: null");
  if (!c->overlap) return fail(FT_EUNSUPPORTED, "prefill_begin: overlap disabled; on-demand prefill is not built");
  if (!c->dev) return c->cache->prefill_begin();  // decisions-only context: residency only
  FT_HIP(hipSetDevice(c->device));
  if (int rc = c->cache->prefill_begin()) return rc;
  hipStream_t ps = static_cast<hipStream_t>(copy);
  const int E = c->shape.E;
  for (int b = 0; b < 2; ++b)
    std::memcpy(c->h_gslot + c->cv.g_max + b * E, c->cache->prefill_buffer(b).data(), (size_t)E * 4);
  // the buffers may hold slots that earlier compute still reads
  FT_HIP(hipStreamWaitEvent(ps, c->ev_done, 0));
  FT_HIP(hipMemcpyAsync(c->wsp<int32_t>(c->cv.bufslot), c->h_gslot + c->cv.g_max, (size_t)2 * E * 4,
                        hipMemcpyHostToDevice, ps));
  if (int rc = enqueue_layer_load(c, 0, ps)) return rc;
  FT_HIP(hipEventRecord(c->ev_pf_fill[0], ps));
  c->prefill_next = 0;
  return FT_OK;
}

int ft_moe_prefill_layer(ft_ctx_t c, int32_t layer, const void* x, int32_t T, const void* w_router, float* y,
                         void* compute, void* copy) {
  if (!c || !x || !w_router || !y) return fail(FT_EINVAL, "prefill_layer: null argument");
  if (!c->cache->prefill_open()) return fail(FT_EINVAL, "prefill_layer: no open prefill");
  if (layer != c->prefill_next) return fail(FT_EINVAL, "prefill_layer: layers must come in order 0..L-1");
  if (T < 1 || T > c->cfg.T_max) return fail(FT_EINVAL, "prefill_layer: T out of range");
  FT_HIP(hipSetDevice(c->device));
  hipStream_t cs = static_cast<hipStream_t>(compute);
  hipStream_t ps = static_cast<hipStream_t>(copy);
  const int k = c->shape.k, d = c->shape.d, E = c->shape.E, d_ff = c->shape.d_ff;
  const int b = layer & 1;
  // stream layer l+1 into the other buffer once layer l-1 (its last reader) is done
  if (layer + 1 < c->shape.L) {
    if (layer >= 1) FT_HIP(hipStreamWaitEvent(ps, c->ev_pf_comp[(layer - 1) & 1], 0));
    if (int rc = enqueue_layer_load(c, layer + 1, ps)) return rc;
    FT_HIP(hipEventRecord(c->ev_pf_fill[(layer + 1) & 1], ps));
  }
  FT_HIP(hipStreamWaitEvent(cs, c->ev_pf_fill[b], 0));
  const int P = T * k;
  int32_t* d_idx = c->wsp<int32_t>(c->cv.idx);
  float* d_gates = c->wsp<float>(c->cv.gates);
  int32_t* d_off = c->wsp<int32_t>(c->cv.offsets);
  int32_t* d_perm = c->wsp<int32_t>(c->cv.perm);
  int32_t* d_inv = c->wsp<int32_t>(c->cv.inv);
  const int32_t* d_buf = c->wsp<int32_t>(c->cv.bufslot) + (size_t)b * E;
  if (int rc = ft::launch_router(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router), nullptr, T,
                                 d, E, k, d_idx, d_gates, c->wsp<float>(c->cv.logits), cs))
    return rc;
  if (int rc = ft::launch_permute(d_idx, P, E, d_off, d_perm, d_inv, c->ws + c->cv.pws, c->cv.pws_bytes, cs))
    return rc;
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  if (d % 128 == 0 && d_ff % 64 == 0) {
    if (int rc = ft::launch_ffn_mfma(xs, d, d_ff, k, c->slots, d_buf, d_off, d_perm, 0, E, T,
                                     c->wsp<uint16_t>(c->cv.h), c->wsp<float>(c->cv.out), cs))
      return rc;
  } else {
    if (int rc = ft::launch_ffn_rows(xs, d, d_ff, k, c->slots, d_buf, d_off, d_perm, 0, E, 8,
                                     c->wsp<float>(c->cv.h), c->wsp<float>(c->cv.out), cs))
      return rc;
  }
  if (int rc = ft::launch_combine(c->wsp<float>(c->cv.out), d_inv, d_gates, nullptr, T, k, d, y, cs)) return rc;
  FT_HIP(hipEventRecord(c->ev_pf_comp[b], cs));
  FT_HIP(hipEventRecord(c->ev_done, cs));
  c->prefill_next = layer + 1;
  c->cache->stats.prefill_layers += 1;
  return FT_OK;
}

int ft_moe_prefill_end(ft_ctx_t c) {
  if (!c) return fail(FT_EINVAL, "prefill_end: null");
  if (!c->cache->prefill_open()) return fail(FT_EINVAL, "prefill_end: no open prefill");
  if (c->dev) {
    // a prefetch of the next layer may still be writing a buffer that is about to
    // return to the pool
    FT_HIP(hipSetDevice(c->device));
    FT_HIP(hipEventSynchronize(c->ev_pf_fill[0]));
    FT_HIP(hipEventSynchronize(c->ev_pf_fill[1]));
  }
  // the last two layers processed stay resident (all L layers in a full prefill)
  c->cache->prefill_end(c->dev ? std::max(c->prefill_next, 0) : c->shape.L);
  c->prefill_next = -1;
  return FT_OK;
}

// ---- bandwidth probe ---------------------------------------------------------------

int ft_bench_bw(const ft_shape* shape, const void* host_pool, int32_t n_records, void* dev_scratch,
                int32_t threads, double* B_P, double* B_H) {
  if (!shape_ok(shape) || !host_pool || !dev_scratch || n_records < 1 || !B_P || !B_H)
    return fail(FT_EINVAL, "bench_bw: bad argument");
  const size_t S = ft_record_bytes(shape);
  const size_t bytes = S * (size_t)n_records;
  hipStream_t s = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  FT_HIP(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
  auto cleanup = [&]() {
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    (void)hipStreamDestroy(s);
  };
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    cleanup();
    return fail(FT_EHIP, "bench_bw: event create failed");
  }
  float best_ms = 1e30f;
  for (int rep = 0; rep < 4; ++rep) {
    (void)hipEventRecord(e0, s);
    for (int i = 0; i < n_records; ++i)
      (void)hipMemcpyAsync(static_cast<uint8_t*>(dev_scratch) + (size_t)i * S,
                           static_cast<const uint8_t*>(host_pool) + (size_t)i * S, S, hipMemcpyHostToDevice, s);
    (void)hipEventRecord(e1, s);
    if (hipEventSynchronize(e1) != hipSuccess) {
      cleanup();
      return fail(FT_EHIP, "bench_bw: copy failed");
    }
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, e0, e1);
    if (rep > 0) best_ms = std::min(best_ms, ms);
  }
  cleanup();
  *B_P = (double)bytes / (best_ms * 1e-3);

  ft::CpuPool* pool = ft::cpu_pool_create(threads);
  std::vector<uint16_t> x((size_t)shape->d, 0x3c00);  // 2^-7 in bf16 words
  std::vector<float> part((size_t)shape->d);
  std::vector<ft::CpuExpert> ex(n_records);
  for (int i = 0; i < n_records; ++i) {
    ex[i].rec = static_cast<const uint16_t*>(host_pool) + (size_t)i * (S / 2);
    ex[i].n_use = 1;
    ex[i].use[0] = ft::CpuUse{0, 1.0f};
  }
  double best_us = 1e30;
  for (int rep = 0; rep < 4; ++rep) {
    const double a = now_us();
    ft::cpu_pool_submit(pool, x.data(), 1, shape->d, shape->d_ff, ex.data(), n_records, part.data());
    ft::cpu_pool_wait(pool);
    const double b = now_us() - a;
    if (rep > 0) best_us = std::min(best_us, b);
  }
  ft::cpu_pool_destroy(pool);
  *B_H = (double)bytes / (best_us * 1e-6);
  return FT_OK;
}

}  // extern "C"
