// Host-only emulation of the wave buffer's device side around the library's own LRU policy
// (kv_vector_index_amd/csrc/wi_lru.h), for tests/test_wavebuf_host.py.  Per step t: the decisions
// from step t - 2 are applied (block copies into cache slots, directory updates), then the step's
// blocks are resolved in the given order (hit: the directory names a slot, whose content must be
// that block; miss: staged in the execution buffer of the step's parity while it has room, else
// read in place), and the step's log goes to the policy.
#include <cstdint>
#include <vector>

#include "wi_lru.h"

extern "C" int wb_protocol(int cache, int exec, int n_keys, int n_steps, const int* off, const int* keys,
                           int64_t* out) {
  wi::WbLru lru(cache, exec, n_keys);
  std::vector<int> dir(n_keys, -1), content(cache, -1);
  std::vector<int> staged[2] = {std::vector<int>(exec, -1), std::vector<int>(exec, -1)};
  std::vector<int32_t> cp[2], up[2];
  int n_cp[2] = {0, 0}, n_up[2] = {0, 0};
  const int room = exec > 0 ? exec : 1;
  for (int q = 0; q < 2; ++q) { cp[q].assign(2 * room, 0); up[q].assign(4 * room, 0); }
  int64_t prev[6] = {0, 0, 0, 0, 0, 0};
  for (int t = 0; t < n_steps; ++t) {
    const int q = t & 1;
    for (int i = 0; i < n_cp[q]; ++i) {
      const int src = cp[q][2 * i] - cache;
      content[cp[q][2 * i + 1]] = staged[src / exec][src % exec];
    }
    for (int i = 0; i < n_up[q]; ++i) dir[up[q][2 * i]] = up[q][2 * i + 1];
    n_cp[q] = n_up[q] = 0;
    std::vector<int32_t> log;
    int x = 0;
    for (int i = off[t]; i < off[t + 1]; ++i) {
      const int key = keys[i];
      int code;
      if (dir[key] >= 0) {
        if (content[dir[key]] != key) return -1 - t;        // the directory names a wrong slot
        code = -1;
      } else if (x < exec) {
        staged[q][x] = key;
        code = x++;
      } else {
        code = -2;
      }
      log.push_back(key);
      log.push_back(code);
    }
    lru.stats[0]++;
    lru.decide(log.data(), (int)log.size() / 2, q, cp[q].data(), &n_cp[q], up[q].data(), &n_up[q]);
    for (int k = 1; k < 6; ++k) { out[5 * t + k - 1] = lru.stats[k] - prev[k]; prev[k] = lru.stats[k]; }
  }
  return 0;
}
