// Residency decisions of the elastic expert cache; see cache.h for the passages.
#include "cache.h"

#include <algorithm>
#include <cstring>

#include "internal.h"

namespace ft {

namespace {
constexpr int32_t kEmpty = -1;
constexpr int32_t kReserved = -2;
}  // namespace

ExpertCache::ExpertCache(int L, int E, int n_slots) : L_(L), E_(E), n_(0) {
  where_.assign((size_t)L * E, -1);
  resize(n_slots);
}

void ExpertCache::resize(int n_slots) {
  n_ = n_slots;
  slot_key_.assign(n_slots, kEmpty);
  slot_stamp_.assign(n_slots, -1);
  std::fill(where_.begin(), where_.end(), -1);
  buf_[0].clear();
  buf_[1].clear();
  buf_layer_[0] = buf_layer_[1] = -1;
  prefill_open_ = false;
  on_demand_ = false;
  const int64_t resizes = stats.resizes;
  stats = ft_stats{};
  stats.resizes = resizes;
}

void ExpertCache::clear_residency() {
  std::fill(slot_key_.begin(), slot_key_.end(), kEmpty);
  std::fill(slot_stamp_.begin(), slot_stamp_.end(), -1);
  std::fill(where_.begin(), where_.end(), -1);
}

int32_t ExpertCache::where(int layer, int e) const {
  if (layer < 0 || layer >= L_ || e < 0 || e >= E_) return -1;
  return where_[(size_t)layer * E_ + e];
}

void ExpertCache::select_victims(int count, const std::vector<uint8_t>& excluded,
                                 std::vector<int32_t>* out) const {
  out->clear();
  if (count <= 0) return;
  // max-heap on (stamp, slot) holding the `count` smallest seen so far
  auto less = [&](int32_t a, int32_t b) {
    return slot_stamp_[a] < slot_stamp_[b] || (slot_stamp_[a] == slot_stamp_[b] && a < b);
  };
  std::vector<int32_t>& heap = *out;
  heap.reserve(count);
  for (int s = 0; s < n_; ++s) {
    if (excluded[s] || slot_key_[s] == kReserved) continue;
    if ((int)heap.size() < count) {
      heap.push_back(s);
      std::push_heap(heap.begin(), heap.end(), less);
    } else if (less(s, heap.front())) {
      std::pop_heap(heap.begin(), heap.end(), less);
      heap.back() = s;
      std::push_heap(heap.begin(), heap.end(), less);
    }
  }
  std::sort_heap(heap.begin(), heap.end(), less);
}

int ExpertCache::lookup(int layer, const int32_t* idx, int T, int k, uint32_t fq, int min_fill,
                        int max_fetch, ft_plan* p) {
  if (layer < 0 || layer >= L_ || T < 0 || k < 1 || (int64_t)T * k > FT_PLAN_CAP || fq > 65536u)
    return fail(FT_EINVAL, "lookup: bad layer, T*k > FT_PLAN_CAP, or frac_q16 > 65536");
  if (prefill_open_) return fail(FT_EBUSY, "lookup: a prefill is open");
  const int P = T * k;
  for (int i = 0; i < P; ++i)
    if (idx[i] < 0 || idx[i] >= E_) return fail(FT_EINVAL, "lookup: routed id out of range");
  p->layer = layer;
  p->T = T;
  p->k = k;
  // dedup in first-occurrence order (E <= 1024 bound via a stamp array)
  int n_u = 0;
  thread_local std::vector<int32_t> mark;
  thread_local int32_t mark_gen = 0;
  if ((int)mark.size() < E_) mark.assign(E_, 0);
  if (++mark_gen == 0) {
    std::fill(mark.begin(), mark.end(), 0);
    mark_gen = 1;
  }
  for (int i = 0; i < P; ++i)
    if (mark[idx[i]] != mark_gen) {
      mark[idx[i]] = mark_gen;
      p->U[n_u++] = idx[i];
    }
  p->n_u = n_u;
  // classify
  int n_h = 0, n_m = 0;
  const size_t base = (size_t)layer * E_;
  for (int i = 0; i < n_u; ++i) {
    if (where_[base + p->U[i]] >= 0)
      p->H[n_h++] = p->U[i];
    else
      p->M[n_m++] = p->U[i];
  }
  p->n_h = n_h;
  p->n_m = n_m;
  // eligible victims: every slot not holding a hit of this call
  thread_local std::vector<uint8_t> excluded;
  excluded.assign(n_, 0);
  for (int i = 0; i < n_h; ++i) excluded[where_[base + p->H[i]]] = 1;
  int avail = 0;
  for (int s = 0; s < n_; ++s) avail += (!excluded[s] && slot_key_[s] != kReserved);
  p->avail = avail;
  const int q = ft_qstar_split(n_m, fq, min_fill, max_fetch, avail);
  if (q < 0) return fail(FT_EINVAL, "lookup: split failed");
  p->q = q;
  p->n_c = n_m - q;
  thread_local std::vector<int32_t> victims;
  select_victims(q, excluded, &victims);
  for (int i = 0; i < q; ++i) {
    const int s = victims[i];
    if (slot_key_[s] >= 0) where_[slot_key_[s]] = -1;
    slot_key_[s] = (int32_t)(base + p->M[i]);
    where_[base + p->M[i]] = s;
    p->F_slot[i] = s;
  }
  // touch H and F in U order; G = H then F
  for (int i = 0; i < n_u; ++i) {
    const int32_t s = where_[base + p->U[i]];
    if (s >= 0) slot_stamp_[s] = ++clock_;
  }
  for (int i = 0; i < n_h; ++i) p->G_slot[i] = where_[base + p->H[i]];
  for (int i = 0; i < q; ++i) p->G_slot[n_h + i] = p->F_slot[i];
  // slot rewrite; group index by position in G
  for (int i = 0; i < P; ++i) {
    const int e = idx[i];
    const int32_t s = where_[base + e];
    int grp = -1;
    if (s >= 0) {
      for (int g = 0; g < n_h + q; ++g)
        if (p->G_slot[g] == s) {
          grp = g;
          break;
        }
    }
    p->route_slot[i] = s;
    p->pair_group[i] = grp;
    stats.reads += 1;
    if (s < 0) {
      stats.read_cpu += 1;
    } else {
      bool is_hit = false;
      for (int h = 0; h < n_h; ++h) is_hit |= (p->H[h] == e);
      if (is_hit)
        stats.read_hits += 1;
      else
        stats.read_fills += 1;
    }
  }
  stats.calls += 1;
  stats.unique_hits += n_h;
  stats.unique_misses += n_m;
  stats.fills += q;
  stats.cpu_experts += n_m - q;
  return FT_OK;
}

int ExpertCache::prefill_begin() {
  if (prefill_open_) return fail(FT_EBUSY, "prefill already open");
  if (n_ < 2 * E_) return fail(FT_ECAP, "prefill double buffering needs n_slots >= 2E");
  std::vector<uint8_t> none(n_, 0);
  std::vector<int32_t> order;
  select_victims(2 * E_, none, &order);
  if ((int)order.size() < 2 * E_) return fail(FT_ECAP, "not enough slots for two prefill buffers");
  buf_[0].assign(order.begin(), order.begin() + E_);
  buf_[1].assign(order.begin() + E_, order.begin() + 2 * E_);
  buf_layer_[0] = buf_layer_[1] = -1;
  for (int s : order) {
    if (slot_key_[s] >= 0) where_[slot_key_[s]] = -1;
    slot_key_[s] = kReserved;
    slot_stamp_[s] = -1;
  }
  prefill_open_ = true;
  return FT_OK;
}

int ExpertCache::prefill_begin_on_demand() {
  if (prefill_open_) return fail(FT_EBUSY, "prefill already open");
  prefill_open_ = true;
  on_demand_ = true;
  return FT_OK;
}

int ExpertCache::prefill_on_demand(int layer, const int32_t* idx, int P, ft_prefill_plan* p) {
  if (!prefill_open_ || !on_demand_) return fail(FT_EINVAL, "prefill_on_demand: no open on-demand prefill");
  if (layer < 0 || layer >= L_ || P < 0 || !p || E_ > FT_E_MAX)
    return fail(FT_EINVAL, "prefill_on_demand: bad layer, pair count or plan");
  for (int i = 0; i < P; ++i)
    if (idx[i] < 0 || idx[i] >= E_) return fail(FT_EINVAL, "prefill_on_demand: routed id out of range");
  // U in first-occurrence order, then H and M in U order
  std::vector<uint8_t> seen(E_, 0);
  std::vector<int32_t> U, H, M;
  for (int i = 0; i < P; ++i)
    if (!seen[idx[i]]) {
      seen[idx[i]] = 1;
      U.push_back(idx[i]);
    }
  const size_t base = (size_t)layer * E_;
  for (int32_t e : U) (where_[base + e] >= 0 ? H : M).push_back(e);
  std::vector<uint8_t> excluded(n_, 0), in_round(E_, 0);
  for (int32_t e : H) excluded[where_[base + e]] = 1;
  p->layer = layer;
  p->n_u = (int32_t)U.size();
  p->n_h = (int32_t)H.size();
  p->n_rounds = 0;
  int g = 0;
  for (int32_t e : H) {
    p->group_expert[g] = e;
    p->group_slot[g++] = where_[base + e];
  }
  std::vector<int32_t> victims;
  size_t done = 0;
  for (int r = 0; r == 0 || done < M.size(); ++r) {
    const size_t want = M.size() - done;
    select_victims((int)want, excluded, &victims);
    if (victims.empty() && want > 0) return fail(FT_ECAP, "prefill_on_demand: no slot to load a miss into");
    const size_t n = victims.size();
    for (size_t i = 0; i < n; ++i) {
      const int s = victims[i];
      const int32_t e = M[done + i];
      if (slot_key_[s] >= 0) where_[slot_key_[s]] = -1;
      slot_key_[s] = (int32_t)(base + e);
      where_[base + e] = s;
      p->group_expert[g] = e;
      p->group_slot[g++] = s;
    }
    // touches: round 0 its hits and loads in U order, later rounds their loads in order
    if (r == 0) {
      for (int32_t e : H) in_round[e] = 1;
      for (size_t i = 0; i < n; ++i) in_round[M[done + i]] = 1;
      for (int32_t e : U)
        if (in_round[e]) slot_stamp_[where_[base + e]] = ++clock_;
    } else {
      for (size_t i = 0; i < n; ++i) slot_stamp_[where_[base + M[done + i]]] = ++clock_;
    }
    p->round_end[p->n_rounds++] = g;
    done += n;
  }
  stats.prefill_layers += 1;
  return FT_OK;
}

int32_t ExpertCache::prefill_slot(int layer, int e) const {
  if (!prefill_open_ || on_demand_ || layer < 0 || e < 0 || e >= E_) return -1;
  return buf_[layer & 1][e];
}

void ExpertCache::prefill_set_buffer_layer(int b, int layer) {
  if (b < 0 || b > 1) return;
  buf_layer_[b] = (layer >= 0 && layer < L_) ? layer : -1;
}

void ExpertCache::prefill_end_full_pass() {
  if (prefill_open_ && !on_demand_) {
    if (L_ >= 2) prefill_set_buffer_layer((L_ - 2) & 1, L_ - 2);
    prefill_set_buffer_layer((L_ - 1) & 1, L_ - 1);
  }
  prefill_end();
}

void ExpertCache::prefill_end() {
  if (!prefill_open_) return;
  if (on_demand_) {  // residency was updated layer by layer
    prefill_open_ = false;
    on_demand_ = false;
    return;
  }
  // [FT] §3.1: layer l+1 streams into the other buffer while layer l computes, so a
  // buffer may hold a layer that was loaded but never computed (a pass ended early);
  // what each buffer holds is what survives, in ascending layer order
  int order[2] = {0, 1};
  if (buf_layer_[1] >= 0 && (buf_layer_[0] < 0 || buf_layer_[1] < buf_layer_[0])) std::swap(order[0], order[1]);
  std::vector<uint8_t> used(n_, 0);
  for (int b : order) {
    const int layer = buf_layer_[b];
    if (layer < 0) continue;
    const std::vector<int32_t>& buf = buf_[b];
    for (int e = 0; e < E_; ++e) {
      const int s = buf[e];
      const size_t key = (size_t)layer * E_ + e;
      const int32_t old = where_[key];
      if (old >= 0 && old != s) {
        slot_key_[old] = kEmpty;
        slot_stamp_[old] = -1;
      }
      slot_key_[s] = (int32_t)key;
      where_[key] = s;
      slot_stamp_[s] = ++clock_;
      used[s] = 1;
    }
  }
  for (int b = 0; b < 2; ++b)
    for (int s : buf_[b])
      if (!used[s]) {
        slot_key_[s] = kEmpty;
        slot_stamp_[s] = -1;
      }
  buf_[0].clear();
  buf_[1].clear();
  buf_layer_[0] = buf_layer_[1] = -1;
  prefill_open_ = false;
}

}  // namespace ft
