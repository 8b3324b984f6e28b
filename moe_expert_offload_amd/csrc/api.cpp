// C ABI of libft: context, decode and prefill orchestration, cache control,
// bandwidth probe.  See include/ft.h for the contract of each call.
//
// [FT] = "FreeToken: Efficient Edge-Native MoE Serving with Bandwidth-Adaptive
// Execution" (arXiv 2608.16157).
#include <hip/hip_runtime.h>
#include <immintrin.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <chrono>
#include <cstring>
#include <string>
#include <thread>
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

void prefault_host(const void* p, size_t bytes, int threads) {
  if (!p || bytes == 0) return;
  threads = std::max(1, std::min(threads, 64));
  const size_t page = 4096;
  const size_t chunk = ((bytes / threads) / page + 1) * page;
  std::vector<std::thread> ts;
  for (int i = 0; i < threads; ++i) {
    const size_t b = (size_t)i * chunk;
    if (b >= bytes) break;
    const size_t e = std::min(bytes, b + chunk);
    ts.emplace_back([p, b, e, page] {
      const volatile uint8_t* q = static_cast<const volatile uint8_t*>(p);
      uint8_t acc = 0;
      for (size_t o = b; o < e; o += page) acc ^= q[o];
      (void)acc;
    });
  }
  for (auto& t : ts) t.join();
}

bool shape_ok(const ft_shape* s) {
  if (!s || s->L <= 0 || s->E <= 0 || s->E > 1024 || s->d <= 0 || s->d % 8 || s->d_ff <= 0 || s->d_ff % 8 ||
      s->k < 1 || s->k > 8 || s->k > s->E)
    return false;
  if (s->fmt == FT_W_BF16) return true;
  return s->fmt == FT_W_MXFP4 && s->d % 256 == 0 && s->d_ff % 128 == 0;
}

bool is_mx(const ft_shape* s) { return s->fmt == FT_W_MXFP4; }

// Workspace carve: offsets of each device array for calls of up to T_max tokens.
struct Carve {
  size_t ticket, idx, gates, logits, key, gslot, bufslot, offsets, perm, inv, pws, h, out, cpu, total;
  size_t xq, xs, hq, hs;  // MXFP8 copies of x and h (MXFP4 experts only)
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
  c.ticket = take(4);
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
  if (is_mx(s)) {
    c.xq = take((size_t)T_max * s->d);
    c.xs = take((size_t)T_max * (s->d / 32));
    c.hq = take(P * s->d_ff);
    c.hs = take(P * (s->d_ff / 32));
  }
  c.total = o;
  return c;
}

}  // namespace

struct ft_ctx {
  ft_shape shape{};
  ft_config cfg{};
  size_t S = 0;  // record bytes
  bool mx = false;
  const uint8_t* pool = nullptr;
  size_t pool_bytes = 0;
  int L_phys = 0;
  uint8_t* slots = nullptr;
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
  int32_t* h_pf_idx = nullptr;  // pinned: routed ids of an on-demand prefill layer (T_max x k)
  ft_prefill_plan pf_plan{};    // decisions of the current on-demand prefill layer
  float* h_partial = nullptr;
  uint32_t* h_flag = nullptr;  // router's publication sequence number
  uint32_t route_seq = 0;
  double last_return_us = 0.0;  // host clock when the previous decode call returned

  // device copy of the residency state and the device-side plan ([FT] §4.1)
  ft::DevCache dc{};
  int dev_cap = 0;               // slots the device arrays hold
  std::atomic<bool> dev_dirty{true};  // host state changed since the last upload (graph host nodes set it too)
  ft::DevPlan* d_plan = nullptr;  // device
  ft::DevPlan* h_plan = nullptr;  // pinned publication

  hipEvent_t ev_route = nullptr, ev_done = nullptr, ev_hffn = nullptr;
  hipEvent_t ev_pf_fill[2] = {nullptr, nullptr}, ev_pf_comp[2] = {nullptr, nullptr};
  hipStream_t side = nullptr;  // decode of 4 or more tokens: the hits' FFN beside the fills

  ft::ExpertCache* cache = nullptr;
  ft::CpuPool* cpu = nullptr;
  std::vector<ft::CpuExpert> cpu_ex;
  ft_plan scratch_plan{};
  int prefill_next = -1;
  int last_T = 0;  // T of the last successful layer call (its ids and gates stay in the workspace)

  // kernel timing (ft_profile_enable)
  struct ProfRec {
    hipEvent_t ev[4];
    double bytes_up, bytes_dn, flops_up, flops_dn;
    int32_t* offsets;  // pinned copy of the group offsets (prefill) or null
    int n_groups, hb;
  };
  bool prof_on = false;
  std::vector<ProfRec> prof;
  std::vector<hipEvent_t> ev_free;
  std::vector<int32_t*> off_free;

  template <typename T>
  T* wsp(size_t off) const { return reinterpret_cast<T*>(ws + off); }
  const uint8_t* record(int layer, int e) const { return pool + ((size_t)(layer % L_phys) * shape.E + e) * S; }
  uint8_t* slot_ptr(int s) const { return slots + (size_t)s * S; }
};

namespace {

// Three timing events for one grouped-FFN launch, or null when timing is off.
ft_ctx::ProfRec* prof_begin(ft_ctx* c) {
  if (!c->prof_on) return nullptr;
  ft_ctx::ProfRec r{};
  for (int i = 0; i < 4; ++i) {
    if (!c->ev_free.empty()) {
      r.ev[i] = c->ev_free.back();
      c->ev_free.pop_back();
    } else if (hipEventCreate(&r.ev[i]) != hipSuccess) {
      return nullptr;
    }
  }
  c->prof.push_back(r);
  return &c->prof.back();
}

// Algorithmic bytes and flops of one launch from its rows per group (see ft.h).
// Per group of n rows: the expert's weights once, the n activation rows read, the
// n result rows written.  hb: bytes per h element between the two kernels.  MXFP4
// weights cost 1/2 + 1/32 byte per element; the MFMA form reads x and h as MXFP8
// (1 + 1/32 bytes per element) after its conversion kernels.
void prof_account(ft_ctx* c, ft_ctx::ProfRec* r, const int* rows, int n_groups, int hb) {
  const double d = c->shape.d, dff = c->shape.d_ff;
  const double wb = c->mx ? (0.5 + 1.0 / 32.0) : 2.0;                   // weight bytes per element
  const bool mx8 = c->mx && hb == 1;                                      // MXFP8 activations
  const double xb = mx8 ? 1.0 + 1.0 / 32.0 : 2.0, hin = mx8 ? 1.0 + 1.0 / 32.0 : hb, hout = mx8 ? 4.0 : hb;
  r->bytes_up = r->bytes_dn = r->flops_up = r->flops_dn = 0.0;
  for (int g = 0; g < n_groups; ++g) {
    const double n = rows[g];
    if (n <= 0) continue;
    r->bytes_up += 2.0 * d * dff * wb + n * d * xb + n * dff * hout;
    r->bytes_dn += d * dff * wb + n * dff * hin + n * d * 4.0;
    r->flops_up += 4.0 * n * d * dff;
    r->flops_dn += 2.0 * n * d * dff;
  }
}

// Copies the host residency state to the device arrays the decode router's
// decisions work on (at create and after every host-side change: resize, prefill,
// stand-alone lookups).  Synchronous; only called at safe points.
int upload_cache(ft_ctx* c) {
  const ft::ExpertCache& h = *c->cache;
  const int n = h.n_slots();
  if (n > c->dev_cap) {
    if (c->dc.slot_key) (void)hipFree(c->dc.slot_key);
    if (c->dc.slot_stamp) (void)hipFree(c->dc.slot_stamp);
    c->dc.slot_key = nullptr;
    c->dc.slot_stamp = nullptr;
    c->dev_cap = 0;
    if (hipMalloc((void**)&c->dc.slot_key, (size_t)n * 4) != hipSuccess ||
        hipMalloc((void**)&c->dc.slot_stamp, (size_t)n * 8) != hipSuccess)
      return fail(FT_ENOMEM, "device cache state allocation failed");
    c->dev_cap = n;
  }
  c->dc.n_slots = n;
  const int64_t clk = h.clock();
  if ((n > 0 && (hipMemcpy(c->dc.slot_key, h.slot_keys().data(), (size_t)n * 4, hipMemcpyHostToDevice) != hipSuccess ||
                 hipMemcpy(c->dc.slot_stamp, h.slot_stamps().data(), (size_t)n * 8, hipMemcpyHostToDevice) !=
                     hipSuccess)) ||
      hipMemcpy(c->dc.where, h.where_table().data(), h.where_table().size() * 4, hipMemcpyHostToDevice) !=
          hipSuccess ||
      hipMemcpy(c->dc.clock, &clk, 8, hipMemcpyHostToDevice) != hipSuccess)
    return fail(FT_EHIP, "device cache state upload failed");
  c->dev_dirty = false;
  return FT_OK;
}

// Hash of a host plan, as the device computes it for its decisions (plan_term).
uint32_t host_plan_hash(const ft_plan& h, int P) {
  uint32_t x = 0u;
  int j = 0;
  auto add = [&](int32_t v) { x += ft::plan_term(j++, v); };
  add(h.n_u);
  add(h.n_h);
  add(h.n_m);
  add(h.q);
  add(h.avail);
  for (int i = 0; i < h.n_u; ++i) add(h.U[i]);
  for (int i = 0; i < h.n_h; ++i) add(h.H[i]);
  for (int i = 0; i < h.n_m; ++i) add(h.M[i]);
  for (int i = 0; i < h.n_h + h.q; ++i) add(h.G_slot[i]);
  for (int i = 0; i < P; ++i) add(h.route_slot[i]);
  for (int i = 0; i < P; ++i) add(h.pair_group[i]);
  return x;
}

}  // namespace

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
    case FT_ENOPROFILE: return "no usable bandwidth profile";
    case FT_WOVERLAP_OFF: return "warning: prefill overlap disabled";
    default: return "unknown status";
  }
}

const char* ft_last_error(void) { return ft::g_last_error.c_str(); }

size_t ft_record_bytes(const ft_shape* s) {
  if (!shape_ok(s)) return 0;
  if (is_mx(s)) return ft::mx_record_bytes(s->d, s->d_ff);
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
  if (!shape_ok(shape))
    return fail(shape && shape->fmt != FT_W_BF16 && shape->fmt != FT_W_MXFP4 ? FT_EUNSUPPORTED : FT_EINVAL,
                "create: bad shape");
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
  c->mx = is_mx(shape);
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
    c->pool = static_cast<const uint8_t*>(host_pool);
    c->pool_bytes = pool_bytes;
    c->slots = static_cast<uint8_t*>(dev_slots);
    c->ws = static_cast<uint8_t*>(dev_workspace);
    c->ws_bytes = workspace_bytes;
    const size_t P = (size_t)FT_PLAN_CAP;
    if (hipHostMalloc((void**)&c->h_idx, P * 4) != hipSuccess ||
        hipHostMalloc((void**)&c->h_gates, P * 4) != hipSuccess ||
        hipHostMalloc((void**)&c->h_x, (size_t)c->t_dec * shape->d * 2) != hipSuccess ||
        hipHostMalloc((void**)&c->h_key, P * 4) != hipSuccess ||
        hipHostMalloc((void**)&c->h_gslot, (size_t)(c->cv.g_max + 2 * shape->E) * 4) != hipSuccess ||
        hipHostMalloc((void**)&c->h_partial, (size_t)c->t_dec * shape->d * 4) != hipSuccess ||
        hipHostMalloc((void**)&c->h_flag, 256) != hipSuccess ||
        hipHostMalloc((void**)&c->h_pf_idx, (size_t)c->cfg.T_max * shape->k * 4) != hipSuccess)
      return bail(FT_ENOMEM, "create: pinned staging allocation failed");
    hipEvent_t* evs[] = {&c->ev_route, &c->ev_done, &c->ev_hffn, &c->ev_pf_fill[0], &c->ev_pf_fill[1],
                         &c->ev_pf_comp[0], &c->ev_pf_comp[1]};
    for (hipEvent_t* e : evs)
      if (hipEventCreateWithFlags(e, hipEventDisableTiming) != hipSuccess)
        return bail(FT_EHIP, "create: hipEventCreate failed");
    if (hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) != hipSuccess)
      return bail(FT_EHIP, "create: hipStreamCreate failed");
    if (hipMemset(c->ws + c->cv.ticket, 0, 4) != hipSuccess) return bail(FT_EHIP, "create: hipMemset failed");
    if (hipMalloc((void**)&c->dc.where, (size_t)shape->L * shape->E * 4) != hipSuccess ||
        hipMalloc((void**)&c->dc.clock, 8) != hipSuccess ||
        hipMalloc((void**)&c->d_plan, sizeof(ft::DevPlan)) != hipSuccess ||
        hipHostMalloc((void**)&c->h_plan, sizeof(ft::DevPlan)) != hipSuccess)
      return bail(FT_ENOMEM, "create: device cache state allocation failed");
    c->dc.E = shape->E;
    *c->h_flag = 0;
    c->cpu = ft::cpu_pool_create(config->cpu_threads);
    c->cfg.cpu_threads = ft::cpu_pool_threads(c->cpu);
    // Pinned host memory is mapped into the process lazily: the first CPU access
    // to each page faults (about a microsecond per 4 KB page, serialised per
    // thread).  Touch the whole pool once here, in parallel, so the CPU branch
    // never faults on the hot path.
    prefault_host(host_pool, (size_t)c->L_phys * shape->E * c->S, c->cfg.cpu_threads + 1);
    c->dev = true;
    if (int rc = upload_cache(c)) {
      ft_destroy(c);
      return rc;
    }
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
  hipEvent_t evs[] = {c->ev_route, c->ev_done, c->ev_hffn, c->ev_pf_fill[0], c->ev_pf_fill[1],
                      c->ev_pf_comp[0], c->ev_pf_comp[1]};
  for (hipEvent_t e : evs)
    if (e) (void)hipEventDestroy(e);
  if (c->side) (void)hipStreamDestroy(c->side);
  for (auto& r : c->prof) {
    for (hipEvent_t e : r.ev) c->ev_free.push_back(e);
    if (r.offsets) c->off_free.push_back(r.offsets);
  }
  for (hipEvent_t e : c->ev_free) (void)hipEventDestroy(e);
  for (int32_t* o : c->off_free) (void)hipHostFree(o);
  void* pins[] = {c->h_idx,     c->h_gates, c->h_x,    c->h_key, c->h_gslot,
                  c->h_partial, c->h_flag,  c->h_plan, c->h_pf_idx};
  for (void* p : pins)
    if (p) (void)hipHostFree(p);
  void* devs[] = {c->dc.where, c->dc.slot_key, c->dc.slot_stamp, c->dc.clock, c->d_plan};
  for (void* p : devs)
    if (p) (void)hipFree(p);
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

int ft_layer_routing(ft_ctx_t c, int32_t* idx, float* gates, int32_t T, void* stream) {
  if (!c || !c->dev) return fail(FT_EINVAL, "layer_routing: no context with a device path");
  if (c->last_T <= 0 || T != c->last_T) return fail(FT_EINVAL, "layer_routing: no layer call of this T");
  FT_HIP(hipSetDevice(c->device));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t n = (size_t)T * c->shape.k;
  if (idx) FT_HIP(hipMemcpyAsync(idx, c->wsp<int32_t>(c->cv.idx), n * 4, hipMemcpyDefault, s));
  if (gates) FT_HIP(hipMemcpyAsync(gates, c->wsp<float>(c->cv.gates), n * 4, hipMemcpyDefault, s));
  return FT_OK;
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
  const bool mfma_ok = d % 256 == 0 && d_ff % 128 == 0;
  if (form == 0) form = (mfma_ok && max_rows_per_group >= 32) ? 2 : 1;
  if (form == 2) {
    if (!mfma_ok) return fail(FT_EINVAL, "grouped_ffn: MFMA form needs d%256==0 and d_ff%128==0");
    // rows of h are pairs (t, j) of the T tokens: at most T * k
    return ft::launch_ffn_mfma(static_cast<const uint16_t*>(x), T, d, d_ff, k, static_cast<const uint16_t*>(slots),
                               group_slot, offsets, perm, g_begin, g_end, T * k, static_cast<uint16_t*>(h_ws), out,
                               stream);
  }
  if (form != 1) return fail(FT_EINVAL, "grouped_ffn: form must be 0, 1 or 2");
  return ft::launch_ffn_rows(static_cast<const uint16_t*>(x), d, d_ff, k, static_cast<const uint16_t*>(slots),
                             group_slot, offsets, perm, g_begin, g_end, max_rows_per_group,
                             static_cast<float*>(h_ws), out, stream, nullptr, nullptr, nullptr, T == 1);
}

size_t ft_grouped_ffn_mx_workspace_bytes(int32_t T, int32_t d, int32_t d_ff, int32_t n_rows) {
  if (T < 0 || d <= 0 || d_ff <= 0 || n_rows < 0) return 0;
  return align256((size_t)n_rows * d_ff * 4) + align256(ft::mx_act_ws_bytes(T, d)) +
         align256(ft::mx_act_ws_bytes(n_rows, d_ff));
}

int ft_grouped_ffn_mx(const void* x, int32_t T, int32_t d, int32_t d_ff, int32_t k, const void* slots,
                      const int32_t* group_slot, const int32_t* offsets, const int32_t* perm, int32_t n_groups,
                      int32_t g_begin, int32_t g_end, int32_t max_rows_per_group, int32_t n_rows, void* workspace,
                      size_t workspace_bytes, float* out, int32_t form, void* stream) {
  if (T < 0 || g_begin < 0 || g_end > n_groups || g_begin > g_end) return fail(FT_EINVAL, "grouped_ffn_mx: bad group range");
  if (d <= 0 || d_ff <= 0 || d % 64 || d_ff % 64) return fail(FT_EINVAL, "grouped_ffn_mx: need d%64==0 and d_ff%64==0");
  if (form == 2 && (d % 256 || d_ff % 128))
    return fail(FT_EINVAL, "grouped_ffn_mx: the MFMA form needs d%256==0 and d_ff%128==0");
  if (n_rows < 0 || !workspace || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return fail(FT_EINVAL, "grouped_ffn_mx: need n_rows >= 0 and a 256-byte aligned workspace");
  if (workspace_bytes < ft_grouped_ffn_mx_workspace_bytes(T, d, d_ff, n_rows))
    return fail(FT_ENOMEM, "grouped_ffn_mx: workspace too small");
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* h = reinterpret_cast<float*>(ws);
  uint8_t* xq = ws + align256((size_t)n_rows * d_ff * 4);
  uint8_t* xs = xq + (size_t)T * d;
  uint8_t* hq = xq + align256(ft::mx_act_ws_bytes(T, d));
  uint8_t* hs = hq + (size_t)n_rows * d_ff;
  const uint8_t* sl = static_cast<const uint8_t*>(slots);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (form == 1)
    return ft::launch_mx_ffn_rows(xb, d, d_ff, k, sl, group_slot, offsets, perm, g_begin, g_end, max_rows_per_group,
                                  h, out, stream, nullptr, nullptr, nullptr, T == 1);
  if (form == 2)
    return ft::launch_mx_ffn_mfma(xb, T, d, d_ff, k, sl, group_slot, offsets, perm, g_begin, g_end, n_rows, xq, xs, h,
                                  hq, hs, out, stream);
  return fail(FT_EINVAL, "grouped_ffn_mx: form must be 1 or 2");
}

int ft_combine(const float* out, const int32_t* inv, const float* gates, const float* cpu_partial,
               int32_t T, int32_t k, int32_t d, float* y, void* stream) {
  return ft::launch_combine(out, inv, gates, cpu_partial, T, k, d, y, stream);
}

int ft_host_experts(const void* x, int32_t T, int32_t d, int32_t d_ff, int32_t fmt, const void* const* records,
                    const int32_t* use_off, const int32_t* use_t, const float* use_g, int32_t n_exp,
                    int32_t threads, float* partial) {
  if (!x || !partial || T < 1 || d <= 0 || d_ff <= 0 || n_exp < 0 || (n_exp > 0 && (!records || !use_off)))
    return fail(FT_EINVAL, "host_experts: bad argument");
  if (fmt != FT_W_BF16 && fmt != FT_W_MXFP4) return fail(FT_EUNSUPPORTED, "host_experts: unknown format");
  if (fmt == FT_W_MXFP4 && (d % 32 || d_ff % 32)) return fail(FT_EINVAL, "host_experts: MXFP4 needs d, d_ff % 32 == 0");
  std::vector<ft::CpuExpert> ex(n_exp);
  for (int i = 0; i < n_exp; ++i) {
    const int n = use_off[i + 1] - use_off[i];
    if (n < 0 || n > 64 || !records[i]) return fail(FT_EINVAL, "host_experts: 0..64 uses per expert");
    ex[i].rec = records[i];
    ex[i].n_use = n;
    for (int u = 0; u < n; ++u) {
      const int t = use_t[use_off[i] + u];
      if (t < 0 || t >= T) return fail(FT_EINVAL, "host_experts: token out of range");
      ex[i].use[u] = ft::CpuUse{t, use_g[use_off[i] + u]};
    }
  }
  if (n_exp == 0) {
    std::memset(partial, 0, sizeof(float) * (size_t)T * d);
    return FT_OK;
  }
  ft::CpuPool* pool = ft::cpu_pool_create(threads);
  ft::cpu_pool_submit(pool, static_cast<const uint16_t*>(x), T, d, d_ff, fmt, ex.data(), n_exp, partial);
  ft::cpu_pool_wait(pool);
  ft::cpu_pool_destroy(pool);
  return FT_OK;
}

// ---- cache control --------------------------------------------------------------

int ft_expert_cache_lookup(ft_ctx_t c, int32_t layer, const int32_t* idx_host, int32_t T, ft_plan* plan) {
  if (!c || !idx_host || !plan) return fail(FT_EINVAL, "lookup: null argument");
  c->dev_dirty = true;  // the device copy is refreshed before the next decode call
  return c->cache->lookup(layer, idx_host, T, c->shape.k, c->cfg.frac_q16, c->cfg.min_fill,
                          c->cfg.max_fetch, plan);
}

int ft_expert_cache_prefill_on_demand(ft_ctx_t c, int32_t layer, const int32_t* idx_host, int32_t T,
                                      ft_prefill_plan* plan) {
  if (!c || !idx_host || !plan || T < 0) return fail(FT_EINVAL, "prefill_on_demand: null argument");
  if (c->dev) return fail(FT_EINVAL, "prefill_on_demand: a device context runs its prefill through ft_moe_prefill_layer");
  return c->cache->prefill_on_demand(layer, idx_host, T * c->shape.k, plan);
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
    hipEvent_t evs[] = {c->ev_route, c->ev_done, c->ev_hffn, c->ev_pf_fill[0], c->ev_pf_fill[1],
                        c->ev_pf_comp[0], c->ev_pf_comp[1]};
    for (hipEvent_t e : evs) {
      const hipError_t q = hipEventQuery(e);
      if (q == hipErrorNotReady) return fail(FT_EBUSY, "resize: issued work still running");
      if (q != hipSuccess) return fail(FT_EHIP, std::string("resize: hipEventQuery: ") + hipGetErrorString(q));
    }
    c->slots = static_cast<uint8_t*>(new_dev_slots);
  }
  c->cache->resize(n);
  c->cache->stats.resizes += 1;
  c->dev_dirty = true;
  if (c->overlap && n < 2 * c->shape.E) {
    c->overlap = false;
    ft::set_error("resize: fewer than 2E slots, prefill overlap disabled");
    return FT_WOVERLAP_OFF;
  }
  return FT_OK;
}

// ---- decode ------------------------------------------------------------------------

int ft_moe_decode_layer(ft_ctx_t c, int32_t layer, const void* x, int32_t T, const void* w_router,
                        const uint8_t* allowed, float* y, void* compute, ft_plan* plan_out,
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
  int32_t* d_idx = c->wsp<int32_t>(c->cv.idx);
  float* d_gates = c->wsp<float>(c->cv.gates);
  // order after everything this context issued before, whatever the stream
  FT_HIP(hipStreamWaitEvent(cs, c->ev_done, 0));
  if (c->dev_dirty) {
    FT_HIP(hipStreamSynchronize(cs));
    if (int rc = upload_cache(c)) return rc;
  }
  // [FT] §4.1 device-side cache control: the router's last block takes this call's
  // decisions on the device and groups the pairs, so the fills and the grouped FFN
  // are queued right behind it without waiting for the host.  It publishes ids,
  // gates, x and the plan to pinned host memory, then a sequence number.
  const uint32_t seq = ++c->route_seq == 0 ? ++c->route_seq : c->route_seq;
  ft::DecideArgs da{};
  da.dc = c->dc;
  da.plan = c->d_plan;
  da.pub = c->h_plan;
  da.layer = layer;
  da.fq = c->cfg.frac_q16;
  da.min_fill = c->cfg.min_fill;
  da.max_fetch = c->cfg.max_fetch;
  if (int rc = ft::launch_router_decode(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_router),
                                        allowed, T, d, E, k, c->wsp<float>(c->cv.logits), d_idx, d_gates,
                                        c->wsp<unsigned int>(c->cv.ticket), c->h_idx, c->h_gates, c->h_x,
                                        c->h_flag, seq, cs, &da))
    return rc;
  FT_HIP(hipEventRecord(c->ev_route, cs));
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  float* d_h = c->wsp<float>(c->cv.h);
  float* d_out = c->wsp<float>(c->cv.out);
  const int nt_bound = T;  // rows per group are at most T
  // grouped FFN over groups [g0, g1) on stream s, further bounded on the device by
  // *g_lo and *g_hi when given
  auto ffn = [&](hipStream_t s, int g0, int g1, const int32_t* g_lo, const int32_t* g_hi,
                 const int* rows_of) -> int {
    ft_ctx::ProfRec* r = prof_begin(c);
    if (r) {
      if (rows_of) {
        prof_account(c, r, rows_of + g0, g1 - g0, 4);
      } else {
        r->bytes_up = r->bytes_dn = r->flops_up = r->flops_dn = 0.0;  // filled in once the plan is known
      }
    }
    void* const* ev = r ? reinterpret_cast<void* const*>(r->ev) : nullptr;
    if (c->mx)
      return ft::launch_mx_ffn_rows(xs, d, c->shape.d_ff, k, c->slots, c->d_plan->G_slot, c->d_plan->offsets,
                                    c->d_plan->perm, g0, g1, nt_bound, d_h, d_out, s, ev, g_lo, g_hi, T == 1);
    return ft::launch_ffn_rows(xs, d, c->shape.d_ff, k, reinterpret_cast<const uint16_t*>(c->slots),
                               c->d_plan->G_slot, c->d_plan->offsets, c->d_plan->perm, g0, g1, nt_bound, d_h,
                               d_out, s, ev, g_lo, g_hi, T == 1);
  };
  // The fills of F are read by the GPU from the pinned pool over PCIe into the victim
  // slots the device chose, right behind the router.  The grouped FFN of G = H then F
  // is launched for every possible group and bounded on the device by the plan.
  // With 4 or more tokens the hits' FFN (bounded by n_h) runs on a side stream beside
  // the fills, since it reads only slots that no fill of this call writes, and the
  // FFN of F follows the fills once the host has seen q (below).  With fewer tokens
  // the hits' FFN is too short to pay for the two cross-stream waits (measured on
  // one MI355X, 40 layers d=2048 E=128 top-8 at one fetch fraction: the split takes
  // batch 8 from 271 to 282 tok/s, batch 1 from 146 down to 134), and the whole FFN
  // follows the fills.
  const bool split_h = T >= 4;
  const size_t prof_h = c->prof.size();
  if (split_h) {
    FT_HIP(hipStreamWaitEvent(c->side, c->ev_route, 0));
    if (int rc = ffn(c->side, 0, P, nullptr, &c->d_plan->n_h, nullptr)) return rc;
    FT_HIP(hipEventRecord(c->ev_hffn, c->side));
  }
  if (int rc = ft::launch_fill(c->record(layer, 0), c->S, E, c->slots, c->cache->n_slots(), c->d_plan, cs))
    return rc;
  if (split_h) {
    // everything issued so far is behind ev_done, also when this call ends in an error
    FT_HIP(hipStreamWaitEvent(cs, c->ev_hffn, 0));
    FT_HIP(hipEventRecord(c->ev_done, cs));
  } else {
    if (int rc = ffn(cs, 0, P, nullptr, &c->d_plan->n_g, nullptr)) return rc;
  }
  // wait for the publication (bounded spin on the sequence number, the event is
  // the fallback)
  {
    bool seen = false;
    const double spin_end = now_us() + 2000.0;
    for (int i = 0;; ++i) {
      if (__atomic_load_n(c->h_flag, __ATOMIC_ACQUIRE) == seq) {
        seen = true;
        break;
      }
      _mm_pause();
      if ((i & 1023) == 1023 && now_us() > spin_end) break;
    }
    if (!seen) {
      FT_HIP(hipEventSynchronize(c->ev_route));
      if (__atomic_load_n(c->h_flag, __ATOMIC_ACQUIRE) != seq)
        return fail(FT_EHIP, "decode: router finished without publishing its result");
    }
  }
  const double t1 = now_us();
  // From here on the device has already acted on its own decisions (fills into its
  // victim slots are queued).  If the host cannot confirm them, no slot's contents
  // can be trusted: empty the cache (the next call uploads the empty state, after
  // this call's queued work) before reporting the error.
  auto distrust = [&](int st, const char* msg) {
    c->cache->clear_residency();
    c->dev_dirty = true;
    return fail(st, msg);
  };
  // a token that allows fewer than k experts: the device took no decisions (no
  // fills, no groups), so residency is unchanged on both sides
  for (int i = 0; i < P; ++i)
    if (c->h_idx[i] < 0) return fail(FT_EINVAL, "decode: a token allows fewer than k experts");
  const ft::DevPlan& dp = *c->h_plan;
  // the host controller takes the same decisions from the same ids: it keeps the
  // counters and the state for safe-point operations, and checks the device
  ft_plan* p = plan_out ? plan_out : &c->scratch_plan;
  if (int rc = c->cache->lookup(layer, c->h_idx, T, k, c->cfg.frac_q16, c->cfg.min_fill, c->cfg.max_fetch, p)) {
    c->cache->clear_residency();
    c->dev_dirty = true;
    return rc;
  }
  if (dp.n_u != p->n_u || dp.q != p->q || dp.hash != host_plan_hash(*p, P))
    return distrust(FT_EHIP, "decode: device and host cache decisions differ");
  std::memcpy(p->idx, c->h_idx, (size_t)P * 4);
  std::memcpy(p->gates, c->h_gates, (size_t)P * 4);
  const int n_h = p->n_h, q = p->q, n_c = p->n_c, n_g = n_h + q;
  const double t2 = now_us();

  // CPU branch first ([FT] §3.2, "In execution order")
  const double t_sub0 = now_us();
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
    ft::cpu_pool_submit(c->cpu, c->h_x, T, d, c->shape.d_ff, c->shape.fmt, c->cpu_ex.data(), n_c, c->h_partial);
  }
  const double t_sub1 = now_us();
  int rows_of[FT_PLAN_CAP] = {0};
  for (int i = 0; i < P; ++i)
    if (p->pair_group[i] >= 0) ++rows_of[p->pair_group[i]];
  c->cache->stats.h2d_bytes += (int64_t)q * (int64_t)c->S;
  if (prof_h < c->prof.size()) prof_account(c, &c->prof[prof_h], rows_of, split_h ? n_h : n_g, 4);
  // the FFN of F = groups [n_h, n_g), behind the fills
  if (split_h && q > 0)
    if (int rc = ffn(cs, n_h, n_g, nullptr, nullptr, rows_of)) return rc;
  // merge of the CPU partial, then the combine
  const double t3 = now_us();
  const float* cpu_part = nullptr;
  double t_cpu = 0.0, t_cpu_work = 0.0;
  if (n_c > 0) {
    ft::cpu_pool_wait(c->cpu);
    t_cpu = now_us() - t2;
    t_cpu_work = ft::cpu_pool_last_work_us(c->cpu);
    if (st) st->cpu_caller_items = ft::cpu_pool_last_caller_items(c->cpu);
    cpu_part = c->h_partial;  // the combine reads the host partial from pinned memory
  }
  if (int rc = ft::launch_combine(d_out, c->d_plan->inv, d_gates, cpu_part, T, k, d, y, cs)) return rc;
  FT_HIP(hipEventRecord(c->ev_done, cs));
  if (st) {
    st->layer = layer;
    st->T = T;
    st->n_u = p->n_u;
    st->hits = n_h;
    st->misses = p->n_m;
    st->q = q;
    st->n_c = n_c;
    if (n_c == 0) st->cpu_caller_items = 0;
    st->h2d_bytes = (int64_t)q * (int64_t)c->S;
    st->t_route_us = t1 - t0;
    st->t_ctrl_us = t2 - t1;
    st->t_cpu_us = t_cpu;
    st->t_total_us = now_us() - t0;
    st->t_issue_us = t3 - t2;
    st->t_cpu_work_us = t_cpu_work;
    st->t_submit_us = t_sub1 - t_sub0;
    st->t_between_us = c->last_return_us > 0.0 ? t0 - c->last_return_us : 0.0;
  }
  c->last_T = T;
  c->last_return_us = now_us();
  return FT_OK;
}

}  // extern "C"

// ---- graph-resident decode step ------------------------------------------------------
// [FT] §4.1 "Graph-resident CPU execution": a whole decode step replayed from one HIP
// graph.  Per layer: the router with the device's decisions, the fills, the grouped
// FFN and the combine on one chain; forked off after the router, a host node that
// takes the host controller's decisions from the published ids, checks them against
// the device's (plan hash) and runs the CPU branch; the combine waits for both.

struct ft_decode_graph {
  ft_ctx* c = nullptr;
  int T = 0;
  const uint16_t* x = nullptr;
  std::vector<const uint16_t*> w_router;
  const uint8_t* allowed = nullptr;
  float* y = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipStream_t cap = nullptr, side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  // what the captured kernels have baked in; a change (resize, a larger device state)
  // means a new capture
  const uint8_t* slots = nullptr;
  int n_slots = -1;
  ft::DevCache dc{};
  struct NodeArg {
    ft_decode_graph* g;
    int layer;
  };
  std::vector<NodeArg> args;
  // first error a host node met since the last report, and its message; the message is
  // written and read under the lock (host nodes run on the runtime's callback thread)
  std::atomic<int> status{FT_OK};
  std::mutex error_lock;
  std::string error;
  ft_plan plan{};
};

namespace {

// The host node of one layer.  Runs on the runtime's callback thread once the layer's
// router finished (its publication to pinned memory is complete); calls no HIP API.
void decode_graph_host_node(void* p) {
  auto* a = static_cast<ft_decode_graph::NodeArg*>(p);
  ft_decode_graph* g = a->g;
  ft_ctx* c = g->c;
  const int T = g->T, k = c->shape.k, d = c->shape.d, P = T * k, layer = a->layer;
  std::memset(c->h_partial, 0, sizeof(float) * (size_t)T * d);
  if (g->status.load(std::memory_order_relaxed) != FT_OK) return;  // after an error, no more decisions
  // The device keeps deciding (and filling) for this step's later layers while the
  // host nodes stop: after any error no slot's contents can be trusted.
  auto failed = [&](int st, const char* msg, bool) {
    c->cache->clear_residency();
    c->dev_dirty = true;
    std::lock_guard<std::mutex> lk(g->error_lock);
    if (g->status.load(std::memory_order_relaxed) == FT_OK) {
      g->error = msg;
      g->status.store(st, std::memory_order_release);
    }
  };
  for (int i = 0; i < P; ++i)
    if (c->h_idx[i] < 0) return failed(FT_EINVAL, "decode graph: a token allows fewer than k experts", false);
  ft_plan* pl = &g->plan;
  if (c->cache->lookup(layer, c->h_idx, T, k, c->cfg.frac_q16, c->cfg.min_fill, c->cfg.max_fetch, pl) != FT_OK)
    return failed(FT_EINVAL, "decode graph: host lookup failed", true);
  const ft::DevPlan& dp = *c->h_plan;
  if (dp.n_u != pl->n_u || dp.q != pl->q || dp.hash != host_plan_hash(*pl, P))
    return failed(FT_EHIP, "decode graph: device and host cache decisions differ", true);
  c->cache->stats.h2d_bytes += (int64_t)pl->q * (int64_t)c->S;
  const int q = pl->q, n_c = pl->n_c;
  if (n_c == 0) return;
  c->cpu_ex.resize(n_c);
  for (int i = 0; i < n_c; ++i) {
    ft::CpuExpert& ex = c->cpu_ex[i];
    const int e = pl->M[q + i];
    ex.rec = c->record(layer, e);
    ex.n_use = 0;
    for (int pr = 0; pr < P; ++pr)
      if (c->h_idx[pr] == e && ex.n_use < 64) ex.use[ex.n_use++] = ft::CpuUse{pr / k, c->h_gates[pr]};
  }
  ft::cpu_pool_submit(c->cpu, c->h_x, T, d, c->shape.d_ff, c->shape.fmt, c->cpu_ex.data(), n_c, c->h_partial);
  ft::cpu_pool_wait(c->cpu);
}

void release_capture(ft_decode_graph* g) {
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  g->exec = nullptr;
  g->graph = nullptr;
}

// Captures the step on the graph's private streams.
int capture_decode_graph(ft_decode_graph* g) {
  ft_ctx* c = g->c;
  release_capture(g);
  const int T = g->T, k = c->shape.k, d = c->shape.d, E = c->shape.E, d_ff = c->shape.d_ff, L = c->shape.L;
  const int P = T * k;
  int32_t* d_idx = c->wsp<int32_t>(c->cv.idx);
  float* d_gates = c->wsp<float>(c->cv.gates);
  float* d_h = c->wsp<float>(c->cv.h);
  float* d_out = c->wsp<float>(c->cv.out);
  ft::DecideArgs da{};
  da.dc = c->dc;
  da.plan = c->d_plan;
  da.pub = c->h_plan;
  da.fq = c->cfg.frac_q16;
  da.min_fill = c->cfg.min_fill;
  da.max_fetch = c->cfg.max_fetch;
  FT_HIP(hipStreamBeginCapture(g->cap, hipStreamCaptureModeRelaxed));
  int rc = FT_OK;
  for (int l = 0; l < L && rc == FT_OK; ++l) {
    const uint16_t* xl = g->x + (size_t)l * T * d;
    const uint8_t* al = g->allowed ? g->allowed + (size_t)l * T * E : nullptr;
    da.layer = l;
    // sequence number 0 in the publication: the eager path never waits for it
    rc = ft::launch_router_decode(xl, g->w_router[l], al, T, d, E, k, c->wsp<float>(c->cv.logits), d_idx, d_gates,
                                  c->wsp<unsigned int>(c->cv.ticket), c->h_idx, c->h_gates, c->h_x, c->h_flag, 0u,
                                  g->cap, &da);
    if (rc) break;
    if (hipEventRecord(g->fork, g->cap) != hipSuccess) {
      rc = fail(FT_EHIP, "decode graph: capture of the fork failed");
      break;
    }
    if ((rc = ft::launch_fill(c->record(l, 0), c->S, E, c->slots, c->cache->n_slots(), c->d_plan, g->cap))) break;
    if (c->mx)
      rc = ft::launch_mx_ffn_rows(xl, d, d_ff, k, c->slots, c->d_plan->G_slot, c->d_plan->offsets, c->d_plan->perm, 0,
                                  P, T, d_h, d_out, g->cap, nullptr, nullptr, &c->d_plan->n_g, T == 1);
    else
      rc = ft::launch_ffn_rows(xl, d, d_ff, k, reinterpret_cast<const uint16_t*>(c->slots), c->d_plan->G_slot,
                               c->d_plan->offsets, c->d_plan->perm, 0, P, T, d_h, d_out, g->cap, nullptr,
                               nullptr, &c->d_plan->n_g, T == 1);
    if (rc) break;
    // the host node depends on the router alone; captured after the fills and the FFN
    // so that a runtime walking the nodes in capture order submits those first
    if (hipStreamWaitEvent(g->side, g->fork, 0) != hipSuccess ||
        hipLaunchHostFunc(g->side, decode_graph_host_node, &g->args[l]) != hipSuccess ||
        hipEventRecord(g->join, g->side) != hipSuccess || hipStreamWaitEvent(g->cap, g->join, 0) != hipSuccess) {
      rc = fail(FT_EHIP, "decode graph: capture of the host node failed");
      break;
    }
    rc = ft::launch_combine(d_out, c->d_plan->inv, d_gates, c->h_partial, T, k, d, g->y + (size_t)l * T * d, g->cap);
  }
  hipGraph_t graph = nullptr;
  const hipError_t ec = hipStreamEndCapture(g->cap, &graph);
  if (rc) {
    if (graph) (void)hipGraphDestroy(graph);
    return rc;
  }
  if (ec != hipSuccess || !graph) return fail(FT_EHIP, std::string("decode graph: end of capture: ") + hipGetErrorString(ec));
  g->graph = graph;
  const hipError_t ei = hipGraphInstantiate(&g->exec, graph, nullptr, nullptr, 0);
  if (ei != hipSuccess) {
    release_capture(g);
    return fail(FT_EHIP, std::string("decode graph: instantiate: ") + hipGetErrorString(ei));
  }
  g->slots = c->slots;
  g->n_slots = c->cache->n_slots();
  g->dc = c->dc;
  return FT_OK;
}

bool capture_stale(const ft_decode_graph* g) {
  const ft_ctx* c = g->c;
  return !g->exec || g->slots != c->slots || g->n_slots != c->cache->n_slots() || g->dc.where != c->dc.where ||
         g->dc.slot_key != c->dc.slot_key || g->dc.slot_stamp != c->dc.slot_stamp || g->dc.clock != c->dc.clock ||
         g->dc.n_slots != c->dc.n_slots;
}

}  // namespace

extern "C" {

int ft_decode_graph_create(ft_ctx_t c, int32_t T, const void* x, const void* const* w_router, const uint8_t* allowed,
                           float* y, ft_decode_graph_t* out) {
  if (!out) return fail(FT_EINVAL, "decode_graph_create: null out");
  *out = nullptr;
  if (!c || !x || !w_router || !y) return fail(FT_EINVAL, "decode_graph_create: null argument");
  if (!c->dev) return fail(FT_EINVAL, "decode_graph_create: context has no device path");
  if (T < 1 || T > c->t_dec) return fail(FT_EINVAL, "decode_graph_create: T out of range");
  for (int l = 0; l < c->shape.L; ++l)
    if (!w_router[l]) return fail(FT_EINVAL, "decode_graph_create: null router weights");
  FT_HIP(hipSetDevice(c->device));
  auto* g = new ft_decode_graph();
  g->c = c;
  g->T = T;
  g->x = static_cast<const uint16_t*>(x);
  g->allowed = allowed;
  g->y = y;
  for (int l = 0; l < c->shape.L; ++l) g->w_router.push_back(static_cast<const uint16_t*>(w_router[l]));
  g->args.resize(c->shape.L);
  for (int l = 0; l < c->shape.L; ++l) g->args[l] = ft_decode_graph::NodeArg{g, l};
  if (hipStreamCreateWithFlags(&g->cap, hipStreamNonBlocking) != hipSuccess ||
      hipStreamCreateWithFlags(&g->side, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&g->fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&g->join, hipEventDisableTiming) != hipSuccess) {
    ft_decode_graph_destroy(g);
    return fail(FT_EHIP, "decode_graph_create: stream or event creation failed");
  }
  if (c->dev_dirty) {
    if (int rc = upload_cache(c)) {
      ft_decode_graph_destroy(g);
      return rc;
    }
  }
  if (int rc = capture_decode_graph(g)) {
    ft_decode_graph_destroy(g);
    return rc;
  }
  *out = g;
  return FT_OK;
}

int ft_decode_graph_status(ft_decode_graph_t g) {
  if (!g) return fail(FT_EINVAL, "decode_graph_status: null");
  std::string msg;
  int st;
  {
    std::lock_guard<std::mutex> lk(g->error_lock);
    st = g->status.exchange(FT_OK);
    if (st != FT_OK) msg = g->error;
  }
  if (st != FT_OK) return fail(st, msg);
  return FT_OK;
}

int ft_decode_graph_launch(ft_decode_graph_t g, void* stream) {
  if (!g) return fail(FT_EINVAL, "decode_graph_launch: null");
  ft_ctx* c = g->c;
  if (int st = ft_decode_graph_status(g)) return st;
  if (c->cache->prefill_open()) return fail(FT_EBUSY, "decode_graph_launch: a prefill is open");
  FT_HIP(hipSetDevice(c->device));
  hipStream_t s = static_cast<hipStream_t>(stream);
  FT_HIP(hipStreamWaitEvent(s, c->ev_done, 0));
  if (c->dev_dirty) {
    FT_HIP(hipStreamSynchronize(s));
    if (int rc = upload_cache(c)) return rc;
  }
  if (capture_stale(g))
    if (int rc = capture_decode_graph(g)) return rc;
  FT_HIP(hipGraphLaunch(g->exec, s));
  FT_HIP(hipEventRecord(c->ev_done, s));
  return FT_OK;
}

int ft_decode_graph_destroy(ft_decode_graph_t g) {
  if (!g) return FT_OK;
  if (g->cap) (void)hipStreamSynchronize(g->cap);
  release_capture(g);
  if (g->fork) (void)hipEventDestroy(g->fork);
  if (g->join) (void)hipEventDestroy(g->join);
  if (g->cap) (void)hipStreamDestroy(g->cap);
  if (g->side) (void)hipStreamDestroy(g->side);
  delete g;
  return FT_OK;
}

// ---- prefill -----------------------------------------------------------------------

// Loads all E records of `layer` into its buffer on `ps`.  The buffer is recorded as
// holding the layer only once every copy was issued.
static int enqueue_layer_load(ft_ctx_t c, int layer, hipStream_t ps) {
  c->cache->prefill_set_buffer_layer(layer & 1, -1);
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
  c->cache->prefill_set_buffer_layer(layer & 1, layer);
  return FT_OK;
}

int ft_moe_prefill_begin(ft_ctx_t c, void* copy) {
  if (!c) return fail(FT_EINVAL, "prefill_begin: null");
  // [FT] §3.1: without two spare full layers (or with overlap off) prefill loads each
  // layer's routed experts on demand
  if (!c->overlap || c->cache->n_slots() < 2 * c->shape.E) {
    if (int rc = c->cache->prefill_begin_on_demand()) return rc;
    c->prefill_next = 0;
    return FT_OK;
  }
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

// One on-demand prefill layer ([FT] §3.1 fallback; the decisions are
// ExpertCache::prefill_on_demand): route, bring the ids to the host, decide, group
// the pairs in the plan's group order, run the hits' FFN, then per round load the
// round's misses on `copy` (after the previous round's compute, whose slots they
// may reuse) and run their FFN once the loads landed; combine.
static int prefill_layer_on_demand(ft_ctx_t c, int layer, const uint16_t* xs, int T, const uint16_t* w_router,
                                   float* y, hipStream_t cs, hipStream_t ps) {
  const int k = c->shape.k, d = c->shape.d, E = c->shape.E, d_ff = c->shape.d_ff;
  const int P = T * k;
  int32_t* d_idx = c->wsp<int32_t>(c->cv.idx);
  float* d_gates = c->wsp<float>(c->cv.gates);
  int32_t* d_key = c->wsp<int32_t>(c->cv.key);
  int32_t* d_gslot = c->wsp<int32_t>(c->cv.gslot);
  int32_t* d_rank = c->wsp<int32_t>(c->cv.bufslot);
  int32_t* d_off = c->wsp<int32_t>(c->cv.offsets);
  int32_t* d_perm = c->wsp<int32_t>(c->cv.perm);
  int32_t* d_inv = c->wsp<int32_t>(c->cv.inv);
  FT_HIP(hipStreamWaitEvent(cs, c->ev_done, 0));
  if (int rc = ft::launch_router(xs, w_router, nullptr, T, d, E, k, d_idx, d_gates, c->wsp<float>(c->cv.logits), cs))
    return rc;
  FT_HIP(hipMemcpyAsync(c->h_pf_idx, d_idx, (size_t)P * 4, hipMemcpyDeviceToHost, cs));
  FT_HIP(hipEventRecord(c->ev_route, cs));
  FT_HIP(hipEventSynchronize(c->ev_route));
  ft_prefill_plan& pl = c->pf_plan;
  if (int rc = c->cache->prefill_on_demand(layer, c->h_pf_idx, P, &pl)) return rc;
  // group of every routed expert, slot of every group (pinned staging; the previous
  // layer's copies out of it finished before this layer's router ran)
  int32_t* h_rank = c->h_gslot + c->cv.g_max;
  for (int e = 0; e < E; ++e) h_rank[e] = -1;
  for (int g = 0; g < pl.n_u; ++g) {
    h_rank[pl.group_expert[g]] = g;
    c->h_gslot[g] = pl.group_slot[g];
  }
  FT_HIP(hipMemcpyAsync(d_rank, h_rank, (size_t)E * 4, hipMemcpyHostToDevice, cs));
  FT_HIP(hipMemcpyAsync(d_gslot, c->h_gslot, (size_t)pl.n_u * 4, hipMemcpyHostToDevice, cs));
  if (int rc = ft::launch_remap(d_idx, d_rank, E, P, d_key, cs)) return rc;
  if (int rc = ft::launch_permute(d_key, P, pl.n_u, d_off, d_perm, d_inv, c->ws + c->cv.pws, c->cv.pws_bytes, cs))
    return rc;
  const bool mfma = d % 256 == 0 && d_ff % 128 == 0;
  const uint16_t* slots16 = reinterpret_cast<const uint16_t*>(c->slots);
  auto ffn = [&](int g0, int g1) -> int {
    if (g1 <= g0) return FT_OK;
    if (c->mx)
      return ft::launch_mx_ffn_mfma(xs, T, d, d_ff, k, c->slots, d_gslot, d_off, d_perm, g0, g1, P,
                                    c->wsp<uint8_t>(c->cv.xq), c->wsp<uint8_t>(c->cv.xs), c->wsp<float>(c->cv.h),
                                    c->wsp<uint8_t>(c->cv.hq), c->wsp<uint8_t>(c->cv.hs), c->wsp<float>(c->cv.out),
                                    cs, nullptr);
    if (mfma)
      return ft::launch_ffn_mfma(xs, T, d, d_ff, k, slots16, d_gslot, d_off, d_perm, g0, g1, P,
                                 c->wsp<uint16_t>(c->cv.h), c->wsp<float>(c->cv.out), cs, nullptr);
    return ft::launch_ffn_rows(xs, d, d_ff, k, slots16, d_gslot, d_off, d_perm, g0, g1, 8, c->wsp<float>(c->cv.h),
                               c->wsp<float>(c->cv.out), cs, nullptr);
  };
  // every earlier reader of a slot a round-0 load may take is before this point
  FT_HIP(hipEventRecord(c->ev_pf_comp[0], cs));
  if (int rc = ffn(0, pl.n_h)) return rc;
  for (int r = 0; r < pl.n_rounds; ++r) {
    const int g0 = std::max(r ? pl.round_end[r - 1] : 0, pl.n_h), g1 = pl.round_end[r];
    if (g1 <= g0) continue;
    FT_HIP(hipStreamWaitEvent(ps, c->ev_pf_comp[0], 0));
    for (int g = g0; g < g1; ++g)
      FT_HIP(hipMemcpyAsync(c->slot_ptr(pl.group_slot[g]), c->record(layer, pl.group_expert[g]), c->S,
                            hipMemcpyHostToDevice, ps));
    c->cache->stats.h2d_bytes += (int64_t)(g1 - g0) * (int64_t)c->S;
    FT_HIP(hipEventRecord(c->ev_pf_fill[0], ps));
    FT_HIP(hipStreamWaitEvent(cs, c->ev_pf_fill[0], 0));
    if (int rc = ffn(g0, g1)) return rc;
    FT_HIP(hipEventRecord(c->ev_pf_comp[0], cs));
  }
  if (int rc = ft::launch_combine(c->wsp<float>(c->cv.out), d_inv, d_gates, nullptr, T, k, d, y, cs)) return rc;
  FT_HIP(hipEventRecord(c->ev_done, cs));
  c->prefill_next = layer + 1;
  c->last_T = T;
  return FT_OK;
}

int ft_moe_prefill_layer(ft_ctx_t c, int32_t layer, const void* x, int32_t T, const void* w_router, float* y,
                         void* compute, void* copy) {
  if (!c || !x || !w_router || !y) return fail(FT_EINVAL, "prefill_layer: null argument");
  if (!c->cache->prefill_open()) return fail(FT_EINVAL, "prefill_layer: no open prefill");
  if (layer != c->prefill_next) return fail(FT_EINVAL, "prefill_layer: layers must come in order 0..L-1");
  if (T < 1 || T > c->cfg.T_max) return fail(FT_EINVAL, "prefill_layer: T out of range");
  if (!c->dev) return fail(FT_EINVAL, "prefill_layer: context has no device path");
  FT_HIP(hipSetDevice(c->device));
  hipStream_t cs = static_cast<hipStream_t>(compute);
  hipStream_t ps = static_cast<hipStream_t>(copy);
  if (c->cache->prefill_on_demand_mode())
    return prefill_layer_on_demand(c, layer, static_cast<const uint16_t*>(x), T,
                                   static_cast<const uint16_t*>(w_router), y, cs, ps);
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
  const bool mfma = d % 256 == 0 && d_ff % 128 == 0;
  ft_ctx::ProfRec* r = prof_begin(c);
  void* const* evs = r ? reinterpret_cast<void* const*>(r->ev) : nullptr;
  const uint16_t* slots16 = reinterpret_cast<const uint16_t*>(c->slots);
  if (c->mx) {
    // MXFP4 experts on the scaled MFMA, x and h in MXFP8
    if (int rc = ft::launch_mx_ffn_mfma(xs, T, d, d_ff, k, c->slots, d_buf, d_off, d_perm, 0, E, P,
                                        c->wsp<uint8_t>(c->cv.xq), c->wsp<uint8_t>(c->cv.xs), c->wsp<float>(c->cv.h),
                                        c->wsp<uint8_t>(c->cv.hq), c->wsp<uint8_t>(c->cv.hs),
                                        c->wsp<float>(c->cv.out), cs, evs))
      return rc;
  } else if (mfma) {
    if (int rc = ft::launch_ffn_mfma(xs, T, d, d_ff, k, slots16, d_buf, d_off, d_perm, 0, E, P,
                                     c->wsp<uint16_t>(c->cv.h), c->wsp<float>(c->cv.out), cs, evs))
      return rc;
  } else {
    if (int rc = ft::launch_ffn_rows(xs, d, d_ff, k, slots16, d_buf, d_off, d_perm, 0, E, 8,
                                     c->wsp<float>(c->cv.h), c->wsp<float>(c->cv.out), cs, evs))
      return rc;
  }
  if (r) {
    // rows per group are known on the device only: keep a copy for ft_profile_read
    if (!c->off_free.empty()) {
      r->offsets = c->off_free.back();
      c->off_free.pop_back();
    } else if (hipHostMalloc((void**)&r->offsets, (size_t)(E + 1) * 4) != hipSuccess) {
      r->offsets = nullptr;
    }
    r->n_groups = E;
    r->hb = c->mx ? 1 : (mfma ? 2 : 4);
    if (r->offsets) FT_HIP(hipMemcpyAsync(r->offsets, d_off, (size_t)(E + 1) * 4, hipMemcpyDeviceToHost, cs));
  }
  if (int rc = ft::launch_combine(c->wsp<float>(c->cv.out), d_inv, d_gates, nullptr, T, k, d, y, cs)) return rc;
  FT_HIP(hipEventRecord(c->ev_pf_comp[b], cs));
  FT_HIP(hipEventRecord(c->ev_done, cs));
  c->prefill_next = layer + 1;
  c->cache->stats.prefill_layers += 1;
  c->last_T = T;
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
  // what the two buffers hold stays resident: the last layer computed and the one
  // streamed in during its compute (L-2 and L-1 after a whole pass)
  if (c->dev)
    c->cache->prefill_end();
  else
    c->cache->prefill_end_full_pass();
  c->prefill_next = -1;
  c->dev_dirty = true;
  return FT_OK;
}

// ---- kernel timing -----------------------------------------------------------------

int ft_profile_enable(ft_ctx_t c, int32_t on) {
  if (!c) return fail(FT_EINVAL, "profile_enable: null");
  if (c->dev) {
    FT_HIP(hipSetDevice(c->device));
    for (auto& r : c->prof) {
      for (hipEvent_t e : r.ev) {
        (void)hipEventSynchronize(e);
        c->ev_free.push_back(e);
      }
      if (r.offsets) c->off_free.push_back(r.offsets);
    }
  }
  c->prof.clear();
  c->prof_on = on != 0 && c->dev;
  return FT_OK;
}

int ft_profile_read(ft_ctx_t c, ft_profile* out) {
  if (!c || !out) return fail(FT_EINVAL, "profile_read: null");
  *out = ft_profile{};
  if (!c->dev) return FT_OK;
  FT_HIP(hipSetDevice(c->device));
  for (auto& r : c->prof) {
    FT_HIP(hipEventSynchronize(r.ev[3]));
    float a = 0.f, b = 0.f;
    FT_HIP(hipEventElapsedTime(&a, r.ev[0], r.ev[1]));  // gate/up kernel, start to stop
    FT_HIP(hipEventElapsedTime(&b, r.ev[2], r.ev[3]));  // down kernel, start to stop
    if (r.offsets) {
      std::vector<int> rows(r.n_groups);
      for (int g = 0; g < r.n_groups; ++g) rows[g] = r.offsets[g + 1] - r.offsets[g];
      prof_account(c, &r, rows.data(), r.n_groups, r.hb);
    }
    if (r.bytes_up <= 0.0) continue;  // a decode launch whose plan had no group for it
    out->launches += 1;
    out->ms_gateup += a;
    out->ms_down += b;
    out->bytes_gateup += r.bytes_up;
    out->bytes_down += r.bytes_dn;
    out->flops_gateup += r.flops_up;
    out->flops_down += r.flops_dn;
  }
  return FT_OK;
}

// ---- bandwidth probe ---------------------------------------------------------------

// [AIN] "How to maintain it": the contended pair.  Record reads over PCIe are kept
// in flight (a second pass is queued whenever fewer than two are outstanding) while
// the host expert kernel runs passes over other records; the CPU rate counts the
// passes it finished, the PCIe rate the read passes finished before the CPU stopped.
int ft_bench_bw_contended(const ft_shape* shape, const void* host_pool, int32_t n_records, void* dev_scratch,
                          int32_t threads, double* pcie_ov, double* cpu_ov) {
  if (!shape_ok(shape) || !host_pool || !dev_scratch || n_records < 2 || !pcie_ov || !cpu_ov)
    return fail(FT_EINVAL, "bench_bw_contended: bad argument (n_records >= 2)");
  const size_t S = ft_record_bytes(shape);
  const int n_gpu = n_records / 2, n_cpu = n_records - n_gpu;
  const uint8_t* pool = static_cast<const uint8_t*>(host_pool);
  hipStream_t s = nullptr;
  FT_HIP(hipStreamCreateWithFlags(&s, hipStreamNonBlocking));
  std::vector<hipEvent_t> ends;
  hipEvent_t start = nullptr;
  ft::CpuPool* cpu = nullptr;
  auto cleanup = [&]() {
    (void)hipStreamSynchronize(s);
    for (hipEvent_t e : ends) (void)hipEventDestroy(e);
    if (start) (void)hipEventDestroy(start);
    (void)hipStreamDestroy(s);
    if (cpu) ft::cpu_pool_destroy(cpu);
  };
  auto enqueue_pass = [&]() -> int {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return fail(FT_EHIP, "bench_bw_contended: hipEventCreate failed");
    ends.push_back(e);
    for (int i = 0; i < n_gpu; ++i)
      if (int rc = ft::launch_h2d_copy(pool + (size_t)i * S, static_cast<uint8_t*>(dev_scratch) + (size_t)i * S, S, s))
        return rc;
    if (hipEventRecord(e, s) != hipSuccess) return fail(FT_EHIP, "bench_bw_contended: hipEventRecord failed");
    return FT_OK;
  };
  cpu = ft::cpu_pool_create(threads);
  std::vector<uint16_t> x((size_t)shape->d, 0x3c00);  // 2^-7 in bf16 words
  std::vector<float> part((size_t)shape->d);
  std::vector<ft::CpuExpert> ex(n_cpu);
  for (int i = 0; i < n_cpu; ++i) {
    ex[i].rec = pool + (size_t)(n_gpu + i) * S;
    ex[i].n_use = 1;
    ex[i].use[0] = ft::CpuUse{0, 1.0f};
  }
  if (hipEventCreate(&start) != hipSuccess || hipEventRecord(start, s) != hipSuccess) {
    cleanup();
    return fail(FT_EHIP, "bench_bw_contended: start event failed");
  }
  for (int i = 0; i < 2; ++i)
    if (int rc = enqueue_pass()) {
      cleanup();
      return rc;
    }
  size_t done_seen = 0;
  auto completed = [&]() {
    while (done_seen < ends.size() && hipEventQuery(ends[done_seen]) == hipSuccess) ++done_seen;
    return done_seen;
  };
  const double t0 = now_us();
  int passes = 0;
  while (passes < 3 || (now_us() - t0 < 150000.0 && passes < 256)) {
    ft::cpu_pool_submit(cpu, x.data(), 1, shape->d, shape->d_ff, shape->fmt, ex.data(), n_cpu, part.data());
    ft::cpu_pool_wait(cpu);
    ++passes;
    while (ends.size() - completed() < 2)
      if (int rc = enqueue_pass()) {
        cleanup();
        return rc;
      }
  }
  const double t_cpu = now_us() - t0;
  const size_t gpu_done = completed();
  if (gpu_done == 0) {
    cleanup();
    return fail(FT_EHIP, "bench_bw_contended: no PCIe pass finished while the host kernel ran");
  }
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, start, ends[gpu_done - 1]) != hipSuccess || !(ms > 0.f)) {
    cleanup();
    return fail(FT_EHIP, "bench_bw_contended: event timing failed");
  }
  *cpu_ov = (double)passes * n_cpu * S / (t_cpu * 1e-6);
  *pcie_ov = (double)gpu_done * n_gpu * S / (ms * 1e-3);
  cleanup();
  return FT_OK;
}

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
  // B_P: the rate at which the decode fills move records, read by the GPU from the
  // pinned pool over PCIe one record per launch
  float best_ms = 1e30f;
  for (int rep = 0; rep < 4; ++rep) {
    (void)hipEventRecord(e0, s);
    for (int i = 0; i < n_records; ++i)
      if (int rc = ft::launch_h2d_copy(static_cast<const uint8_t*>(host_pool) + (size_t)i * S,
                                       static_cast<uint8_t*>(dev_scratch) + (size_t)i * S, S, s)) {
        cleanup();
        return rc;
      }
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
    ex[i].rec = static_cast<const uint8_t*>(host_pool) + (size_t)i * S;
    ex[i].n_use = 1;
    ex[i].use[0] = ft::CpuUse{0, 1.0f};
  }
  // B_H: the fastest of the passes run over at least 100 ms (and 3 passes) after one
  // warm-up pass; a short pass over few records is otherwise dominated by waking the
  // workers
  double best_us = 1e30;
  const double t_start = now_us();
  for (int rep = 0; rep < 1 + 3 || (now_us() - t_start < 100000.0 && rep < 1 + 256); ++rep) {
    const double a = now_us();
    ft::cpu_pool_submit(pool, x.data(), 1, shape->d, shape->d_ff, shape->fmt, ex.data(), n_records, part.data());
    ft::cpu_pool_wait(pool);
    const double b = now_us() - a;
    if (rep > 0) best_us = std::min(best_us, b);
  }
  ft::cpu_pool_destroy(pool);
  *B_H = (double)bytes / (best_us * 1e-6);
  return FT_OK;
}

}  // extern "C"
