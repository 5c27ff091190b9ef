// Host-side check behind the choice of write form in pa_upload_and_cache:
// do a call's new tokens each land in a block of their own?  Plain C++ with
// no device code, so it is also compiled into a CPU test harness.
#pragma once

#include <algorithm>
#include <cstdint>
#include <vector>

namespace pa {

// True when no two tokens' slots inside the pool fall in one block.  Read on
// the host from the page-locked slot mapping (final at the call).  O(n) with
// a per-thread stamp per block for pools of up to stamp_blocks blocks; larger
// pools sort the call's block ids instead (no allocation that scales with the
// pool, and nothing that can throw across the C ABI).
constexpr int32_t kStampBlocks = 1 << 24;
inline bool one_token_per_block(const int32_t* slots, int32_t n, int32_t num_blocks, int32_t block_size,
                                int32_t stamp_blocks = kStampBlocks) {
  if (n <= 1) return true;
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
  thread_local std::vector<uint32_t> stamp;
  thread_local uint32_t epoch = 0;
  bool stamps = num_blocks <= stamp_blocks;
  if (stamps && stamp.size() < static_cast<size_t>(num_blocks)) {
    try {
      stamp.assign(static_cast<size_t>(num_blocks), 0u);
      epoch = 0;
    } catch (...) {
      stamp.clear();
      stamps = false;
    }
  }
  if (!stamps) {
    thread_local std::vector<int32_t> ids;
    try {
      ids.clear();
      for (int32_t i = 0; i < n; ++i)
        if (slots[i] >= 0 && slots[i] < num_slots) ids.push_back(slots[i] / block_size);
    } catch (...) {
      return false;  // the element-wise write is correct for any slots
    }
    std::sort(ids.begin(), ids.end());
    return std::adjacent_find(ids.begin(), ids.end()) == ids.end();
  }
  if (++epoch == 0) {  // wrapped: clear and start again
    std::fill(stamp.begin(), stamp.end(), 0u);
    epoch = 1;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int64_t slot = slots[i];
    if (slot < 0 || slot >= num_slots) continue;
    uint32_t& st = stamp[static_cast<size_t>(slot / block_size)];
    if (st == epoch) return false;
    st = epoch;
  }
  return true;
}

}  // namespace pa
