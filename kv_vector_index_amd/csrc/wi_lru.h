// Host-side decisions of the wave buffer's block cache (RetroInfer technical summary, section 2.B;
// Arabic summary, section 2.b: replacement runs on the CPU, off the attention's critical path).
// Plain C++ with no HIP dependency, so that the policy can be exercised on the host alone.
//
// decide() takes the access log of one decode call: (block key, code) entries in any order, code
// -1 for a hit, -2 for a block the attention read in place from host memory, else the index of
// the execution-buffer slot (of the call's parity q) where the miss was staged.  In ascending key
// order it refreshes the recency of the hits that are still cached, then admits every staged miss
// that is not cached yet, into a free slot or in place of the least recently used block (exact
// LRU: every access takes the next tick).  It returns the admissions as device work for a later
// call: block copies (pool source, cache slot), one per slot however many times the batch refilled
// it, and directory updates (key, final value), one per key the batch changed.
#pragma once

#include <algorithm>
#include <cstdint>
#include <utility>
#include <vector>

namespace wi {

class WbLru {
 public:
  int64_t stats[6] = {0, 0, 0, 0, 0, 0};   // calls, hits, staged misses, host reads, admitted, evicted

  WbLru(int cache_blocks, int exec_blocks, int64_t n_keys)
      : cache_(cache_blocks), exec_(exec_blocks), slot_tick_(cache_blocks, 0), slot_key_(cache_blocks, -1),
        slot_src_(cache_blocks, -1), dir_(n_keys, -1), key_mark_(n_keys, 0) {
    for (int i = cache_blocks - 1; i >= 0; --i) free_.push_back(i);
    key_bits_ = 1;
    while (((int64_t)1 << key_bits_) < n_keys) ++key_bits_;
  }

  // `log` holds n (key, code) pairs; cp receives n_cp (source, slot) pairs and up n_up (key,
  // value) pairs (room for min(cache, exec) and 2 exec pairs)
  void decide(const int32_t* log, int n, int q, int32_t* cp, int* n_cp, int32_t* up, int* n_up) {
    ent_.resize(n);
    for (int i = 0; i < n; ++i) ent_[i] = ((uint64_t)(uint32_t)log[2 * i] << 32) | (uint32_t)(log[2 * i + 1] + 2);
    sort_entries(n);
    for (int i = 0; i < n; ++i) {
      if (code_of(ent_[i]) != -1) continue;
      ++stats[1];
      const int s = dir_[key_of(ent_[i])];
      if (s >= 0) touch(s);                      // (a block hit then may have been evicted since)
    }
    std::vector<int32_t> touched, changed;
    ++batch_;
    auto mark = [&](int key) {
      if (key_mark_[key] != batch_) { key_mark_[key] = batch_; changed.push_back(key); }
    };
    for (int i = 0; i < n; ++i) {
      const int key = key_of(ent_[i]), code = code_of(ent_[i]);
      if (code == -1) continue;
      if (code == -2) { ++stats[3]; continue; }
      ++stats[2];
      if (cache_ == 0) continue;
      if (dir_[key] >= 0) { touch(dir_[key]); continue; }   // admitted from an earlier log
      int s;
      if (!free_.empty()) {
        s = free_.back();
        free_.pop_back();
      } else {
        s = pop_lru();
        dir_[slot_key_[s]] = -1;
        mark(slot_key_[s]);
        ++stats[5];
      }
      if (slot_src_[s] < 0) touched.push_back(s);
      slot_src_[s] = cache_ + q * exec_ + code;
      slot_key_[s] = key;
      dir_[key] = s;
      mark(key);
      touch(s);
      ++stats[4];
    }
    int m = 0;
    for (const int s : touched) {
      cp[2 * m] = slot_src_[s];
      cp[2 * m + 1] = s;
      ++m;
      slot_src_[s] = -1;
    }
    int u = 0;
    for (const int key : changed) { up[2 * u] = key; up[2 * u + 1] = dir_[key]; ++u; }
    *n_cp = m;
    *n_up = u;
    compact_queue();
  }

 private:
  int cache_, exec_, key_bits_;
  std::vector<int64_t> slot_tick_;
  std::vector<std::pair<int64_t, int32_t>> queue_;   // (tick, slot) in tick order; stale ones skipped
  size_t qhead_ = 0;
  int64_t tick_ = 0;
  std::vector<int32_t> slot_key_, slot_src_, dir_, free_, key_mark_;
  int32_t batch_ = 0;
  std::vector<uint64_t> ent_, tmp_;

  static int key_of(uint64_t e) { return (int)(e >> 32); }
  static int code_of(uint64_t e) { return (int)(e & 0xffffffffu) - 2; }
  void touch(int s) {
    slot_tick_[s] = ++tick_;
    queue_.emplace_back(tick_, s);
  }
  int pop_lru() {
    for (;;) {
      const auto x = queue_[qhead_++];
      if (slot_tick_[x.second] == x.first) return x.second;
    }
  }
  void compact_queue() {
    if (qhead_ < queue_.size() / 2 && queue_.size() < 4 * (size_t)std::max(cache_, 1024)) return;
    std::vector<std::pair<int64_t, int32_t>> q;
    for (size_t i = qhead_; i < queue_.size(); ++i)
      if (slot_tick_[queue_[i].second] == queue_[i].first) q.push_back(queue_[i]);
    queue_.swap(q);
    qhead_ = 0;
  }
  // by key: LSD radix sort, 11 bits a pass (keys are unique within a log)
  void sort_entries(int n) {
    tmp_.resize(n);
    for (int shift = 32; shift < 32 + key_bits_; shift += 11) {
      std::vector<int> cnt(2049, 0);
      for (int i = 0; i < n; ++i) ++cnt[((ent_[i] >> shift) & 2047) + 1];
      for (int b = 0; b < 2048; ++b) cnt[b + 1] += cnt[b];
      for (int i = 0; i < n; ++i) tmp_[cnt[(ent_[i] >> shift) & 2047]++] = ent_[i];
      ent_.swap(tmp_);
    }
  }
};

}  // namespace wi
