// Residency state of the elastic GPU expert cache (host side).
//
// [FT] = "FreeToken: Efficient Edge-Native MoE Serving with Bandwidth-Adaptive
// Execution" (arXiv 2608.16157).
//   §3    one cache shared by all MoE layers, keyed on logical (layer, expert).
//   §3.2  hits refresh recency, fills admit, eviction drops the least recently
//         demanded entry; the m misses split into F (filled) and C (host).
//   §4.1  per layer: dedup, classify, derive q, select the K least recently used
//         victims in one pass and consume the first q, rewrite ids to slots or -1.
//   §3.1  two full-layer prefill buffers are taken from the same slot pool; when
//         the pool cannot spare them (or overlap is off) prefill loads the routed
//         experts of each layer on demand.
//   §3.3  rebuild for a new budget at a safe point.
#pragma once

#include <cstdint>
#include <vector>

#include "../../include/ft.h"

namespace ft {

class ExpertCache {
 public:
  ExpertCache(int L, int E, int n_slots);

  int n_slots() const { return n_; }
  int E() const { return E_; }

  // One decode call's decisions for routed ids idx[T*k]; updates state.
  int lookup(int layer, const int32_t* idx, int T, int k, uint32_t fq, int min_fill,
             int max_fetch, ft_plan* plan);

  // Prefill buffers: reserves 2E slots (victim order), returns FT_OK or FT_ECAP.
  int prefill_begin();
  // On-demand prefill: opens a prefill with no buffers; each layer then calls
  // prefill_on_demand with the chunk's routed ids (T x k).  Its misses are loaded in
  // rounds of at most the slots not holding a hit, LRU victims per round (round 0
  // also computes the hits).  FT_ECAP when a miss has no slot at all.
  int prefill_begin_on_demand();
  int prefill_on_demand(int layer, const int32_t* idx, int P, ft_prefill_plan* plan);
  bool prefill_on_demand_mode() const { return prefill_open_ && on_demand_; }
  int32_t prefill_slot(int layer, int e) const;
  const std::vector<int32_t>& prefill_buffer(int b) const { return buf_[b]; }
  bool prefill_open() const { return prefill_open_; }
  // Which layer's records buffer b holds once its issued loads land (-1: none, or a
  // load that was not issued completely).  Set as loads are issued.
  void prefill_set_buffer_layer(int b, int layer);
  int prefill_buffer_layer(int b) const { return buf_layer_[b]; }
  // Ends the prefill.  Double-buffered: the layer each buffer holds becomes resident
  // (ascending layer order, e ascending, each touching the clock; a copy of the same
  // key elsewhere is emptied); buffer slots holding no layer become empty.
  void prefill_end();
  // A whole pass in a context that issues no loads (residency only): the buffers
  // end holding layers L-2 and L-1, as after a full pass, then prefill_end().
  void prefill_end_full_pass();

  void resize(int n_slots);  // all slots empty, counters reset, clock kept
  // All slots empty, counters and clock kept: for when the slots' contents can no
  // longer be trusted (the device acted on decisions the host did not take).
  void clear_residency();
  int32_t where(int layer, int e) const;

  // the whole state, for a copy in device memory
  const std::vector<int32_t>& slot_keys() const { return slot_key_; }
  const std::vector<int64_t>& slot_stamps() const { return slot_stamp_; }
  const std::vector<int32_t>& where_table() const { return where_; }
  int64_t clock() const { return clock_; }

  ft_stats stats{};

 private:
  // first `count` slots in (stamp, slot) order among those not excluded;
  // one pass with a bounded max-heap (ties by slot index).
  void select_victims(int count, const std::vector<uint8_t>& excluded, std::vector<int32_t>* out) const;

  int L_, E_, n_;
  int64_t clock_ = 0;
  std::vector<int32_t> slot_key_;    // -1 empty, -2 reserved for prefill, else l*E+e
  std::vector<int64_t> slot_stamp_;  // -1 for empty
  std::vector<int32_t> where_;       // [L*E] slot or -1
  std::vector<int32_t> buf_[2];
  int32_t buf_layer_[2] = {-1, -1};
  bool prefill_open_ = false;
  bool on_demand_ = false;
};

}  // namespace ft
