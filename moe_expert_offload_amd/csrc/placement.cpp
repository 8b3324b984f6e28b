// Expert-placement replay ([FT] §5.3 "Expert locality", Fig. 4b): the decode-time
// expert reads of a routing trace replayed against one placement policy at one
// cache capacity.  The LRU policy is the engine's own residency controller
// (ExpertCache), driven as the layer entry points drive it; the two others are
// the pages' one-line descriptions of the alternatives they compare against.
#include <algorithm>
#include <vector>

#include "cache.h"
#include "ft.h"
#include "internal.h"

namespace {

// The n pairs (l*E + e) routed most often by one request's prefill tokens, ties
// to the lower l*E + e; pairs never routed fill the rest in that order.
void hot_set(const int32_t* prompt_ids, int prompt, int L, int E, int k, int n, std::vector<uint8_t>* resident) {
  const int pairs = L * E;
  std::vector<int64_t> count(pairs, 0);
  for (int s = 0; s < prompt; ++s)
    for (int l = 0; l < L; ++l)
      for (int j = 0; j < k; ++j) ++count[(size_t)l * E + prompt_ids[((size_t)s * L + l) * k + j]];
  std::vector<int32_t> order(pairs);
  for (int i = 0; i < pairs; ++i) order[i] = i;
  const int take = std::max(0, std::min(n, pairs));
  std::partial_sort(order.begin(), order.begin() + take, order.end(), [&](int32_t a, int32_t b) {
    return count[a] != count[b] ? count[a] > count[b] : a < b;
  });
  resident->assign(pairs, 0);
  for (int i = 0; i < take; ++i) (*resident)[order[i]] = 1;
}

}  // namespace

extern "C" int ft_replay_placement(int32_t policy, const ft_shape* shape, int32_t n_slots, const int32_t* ids,
                                   int32_t n_requests, int32_t prompt, int32_t decode, int64_t* reads,
                                   int64_t* misses) {
  if (!shape || shape->L <= 0 || shape->E <= 0 || shape->E > FT_E_MAX || shape->k < 1 || shape->k > 8 ||
      shape->k > shape->E || n_slots < 0 || n_requests < 0 || prompt < 0 || decode < 0 || !reads || !misses ||
      (!ids && n_requests > 0 && prompt + decode > 0))
    return ft::fail(FT_EINVAL, "replay_placement: bad argument");
  if (policy != FT_PLACE_LRU && policy != FT_PLACE_HOTSET && policy != FT_PLACE_STATIC)
    return ft::fail(FT_EINVAL, "replay_placement: unknown policy");
  const int L = shape->L, E = shape->E, k = shape->k;
  const int steps = prompt + decode;
  const size_t per_step = (size_t)L * k, per_req = (size_t)steps * per_step;
  for (size_t i = 0; i < (size_t)n_requests * per_req; ++i)
    if (ids[i] < 0 || ids[i] >= E) return ft::fail(FT_EINVAL, "replay_placement: expert id out of range");
  int64_t n_reads = 0, n_miss = 0;
  if (policy == FT_PLACE_LRU) {
    ft::ExpertCache cache(L, E, n_slots);
    ft_plan plan;
    ft_prefill_plan pplan;
    for (int r = 0; r < n_requests; ++r) {
      const int32_t* req = ids + (size_t)r * per_req;
      if (prompt > 0) {
        if (n_slots >= 2 * E) {  // two full-layer buffers, the last two layers stay
          if (int rc = cache.prefill_begin()) return rc;
          cache.prefill_end_full_pass();
        } else {  // the on-demand fallback: each layer's routed experts loaded in rounds
          if (int rc = cache.prefill_begin_on_demand()) return rc;
          std::vector<int32_t> layer_ids((size_t)prompt * k);
          for (int l = 0; l < L; ++l) {
            for (int s = 0; s < prompt; ++s)
              for (int j = 0; j < k; ++j) layer_ids[(size_t)s * k + j] = req[(size_t)s * per_step + (size_t)l * k + j];
            if (int rc = cache.prefill_on_demand(l, layer_ids.data(), prompt * k, &pplan)) {
              cache.prefill_end();
              return rc;
            }
          }
          cache.prefill_end();
        }
      }
      for (int s = prompt; s < steps; ++s)
        for (int l = 0; l < L; ++l) {
          // every miss is filled: the per-miss LRU (q = m)
          if (int rc = cache.lookup(l, req + (size_t)s * per_step + (size_t)l * k, 1, k, 65536u, 1, -1, &plan))
            return rc;
          n_reads += k;
          n_miss += plan.n_m;
        }
    }
  } else {
    std::vector<uint8_t> resident;
    if (policy == FT_PLACE_STATIC) {  // the last n_slots pairs, whatever the routing
      const int64_t first = (int64_t)L * E - std::max(0, std::min(n_slots, L * E));
      resident.assign((size_t)L * E, 0);
      for (int64_t i = first; i < (int64_t)L * E; ++i) resident[i] = 1;
    }
    for (int r = 0; r < n_requests; ++r) {
      const int32_t* req = ids + (size_t)r * per_req;
      if (policy == FT_PLACE_HOTSET) hot_set(req, prompt, L, E, k, n_slots, &resident);
      for (int s = prompt; s < steps; ++s)
        for (int l = 0; l < L; ++l)
          for (int j = 0; j < k; ++j) {
            n_reads += 1;
            n_miss += !resident[(size_t)l * E + req[(size_t)s * per_step + (size_t)l * k + j]];
          }
    }
  }
  *reads = n_reads;
  *misses = n_miss;
  return FT_OK;
}
