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
        slot_src_(cache_blocks, -1), dir_(n_keys, -1), key_mark_(n_keys, 0), code_at_(n_keys, 0),
        seen_((n_keys + 63) / 64, 0ull) {
    for (int i = cache_blocks - 1; i >= 0; --i) free_.push_back(i);
  }

  // `log` holds n (key, code) pairs; cp receives n_cp (source, slot) pairs and up n_up (key,
  // value) pairs (room for min(cache, exec) and 2 exec pairs)
  void decide(const int32_t* log, int n, int q, int32_t* cp, int* n_cp, int32_t* up, int* n_up) {
    // ascending key order without a sort: the logged keys (unique within a log) as a bitmap,
    // their codes in a table indexed by key
    for (int i = 0; i < n; ++i) {
      const int key = log[2 * i];
      code_at_[key] = log[2 * i + 1];
      seen_[key >> 6] |= 1ull << (key & 63);
    }
    auto for_keys = [&](auto&& fn) {
      for (size_t w = 0; w < seen_.size(); ++w)
        for (uint64_t m = seen_[w]; m; m &= m - 1) fn((int)(w * 64 + (size_t)__builtin_ctzll(m)));
    };
    for_keys([&](int key) {
      if (code_at_[key] != -1) return;
      ++stats[1];
      const int s = dir_[key];
      if (s >= 0) touch(s);                      // (a block hit then may have been evicted since)
    });
    touched_.clear();
    changed_.clear();
    ++batch_;
    auto mark = [&](int key) {
      if (key_mark_[key] != batch_) { key_mark_[key] = batch_; changed_.push_back(key); }
    };
    for_keys([&](int key) {
      const int code = code_at_[key];
      if (code == -1) return;
      if (code == -2) { ++stats[3]; return; }
      ++stats[2];
      if (cache_ == 0) return;
      if (dir_[key] >= 0) { touch(dir_[key]); return; }   // admitted from an earlier log
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
      if (slot_src_[s] < 0) touched_.push_back(s);
      slot_src_[s] = cache_ + q * exec_ + code;
      slot_key_[s] = key;
      dir_[key] = s;
      mark(key);
      touch(s);
      ++stats[4];
    });
    for (int i = 0; i < n; ++i) seen_[log[2 * i] >> 6] = 0ull;
    int m = 0;
    for (const int s : touched_) {
      cp[2 * m] = slot_src_[s];
      cp[2 * m + 1] = s;
      ++m;
      slot_src_[s] = -1;
    }
    int u = 0;
    for (const int key : changed_) { up[2 * u] = key; up[2 * u + 1] = dir_[key]; ++u; }
    *n_cp = m;
    *n_up = u;
    compact_queue();
  }

 private:
  int cache_, exec_;
  // exact LRU: every touch appends the slot to queue_; the entry at position i carries the tick
  // tick0_ + i, and it is current while the slot's own tick equals that (stale ones are skipped)
  std::vector<int64_t> slot_tick_;
  std::vector<int32_t> queue_;
  size_t qhead_ = 0;
  int64_t tick0_ = 1;
  std::vector<int32_t> slot_key_, slot_src_, dir_, free_, key_mark_, code_at_, touched_, changed_;
  std::vector<uint64_t> seen_;
  int32_t batch_ = 0;

  void touch(int s) {
    slot_tick_[s] = tick0_ + (int64_t)queue_.size();
    queue_.push_back(s);
  }
  int pop_lru() {
    for (;;) {
      const int s = queue_[qhead_];
      const int64_t t = tick0_ + (int64_t)qhead_;
      ++qhead_;
      if (slot_tick_[s] == t) return s;
    }
  }
  // drop the stale entries, giving the current ones fresh ticks in the same order
  void compact_queue() {
    if (qhead_ < queue_.size() / 2 && queue_.size() < 4 * (size_t)std::max(cache_, 1024)) return;
    const int64_t base = tick0_ + (int64_t)queue_.size();
    std::vector<int32_t> nq;
    nq.reserve((size_t)cache_ + 1024);
    for (size_t i = qhead_; i < queue_.size(); ++i) {
      const int s = queue_[i];
      if (slot_tick_[s] == tick0_ + (int64_t)i) {
        slot_tick_[s] = base + (int64_t)nq.size();
        nq.push_back(s);
      }
    }
    queue_.swap(nq);
    qhead_ = 0;
    tick0_ = base;
  }
};

}  // namespace wi
