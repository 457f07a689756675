// Longest-processing-time-first assignment of context chunks to devices with equal
// chunk counts ("Split-KV speeds diffusion drafter training...", section "Balance
// actual attention work": costly chunks first, each to the device with the least
// work among those with room left, every device ending with the same count).
//
// Chunks are visited by (cost descending, index ascending).  A min-heap keyed by
// (load, bin index) holds the bins that still have room; the chosen bin is popped,
// charged, and pushed back while it holds fewer than n_chunk / n_bin chunks.  The
// ordering makes the plan unique, so every device derives the same plan from the
// same costs.  O(n log n + n log n_bin).
#include <algorithm>
#include <cstdint>
#include <functional>
#include <queue>
#include <utility>
#include <vector>

namespace sxa {

int lpt_assign_host(const int64_t* cost, int32_t n_chunk, int32_t n_bin, int32_t* bin_of_chunk,
                    int64_t* bin_load) {
  const int32_t cap = n_chunk / n_bin;
  std::vector<int32_t> order(static_cast<size_t>(n_chunk));
  for (int32_t i = 0; i < n_chunk; ++i) order[static_cast<size_t>(i)] = i;
  std::sort(order.begin(), order.end(), [cost](int32_t a, int32_t b) {
    return cost[a] != cost[b] ? cost[a] > cost[b] : a < b;
  });
  using Entry = std::pair<int64_t, int32_t>;  // (load, bin)
  std::priority_queue<Entry, std::vector<Entry>, std::greater<Entry>> heap;
  std::vector<int32_t> count(static_cast<size_t>(n_bin), 0);
  for (int32_t b = 0; b < n_bin; ++b) {
    bin_load[b] = 0;
    heap.emplace(0, b);
  }
  for (int32_t c : order) {
    const Entry top = heap.top();
    heap.pop();
    const int32_t b = top.second;
    bin_of_chunk[c] = b;
    bin_load[b] += cost[c];
    if (++count[static_cast<size_t>(b)] < cap) heap.emplace(bin_load[b], b);
  }
  return 0;
}

}  // namespace sxa
