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
// a per-thread stamp per block when the pool is small next to the call (at
// most kStampPerToken blocks per token and stamp_blocks blocks in all, so the
// kept stamp array is at most 4 MB and scales with the calls, not with the
// pool); otherwise the call's block ids are sorted (a few hundred ids per
// decode step).  Nothing here can throw across the C ABI.
constexpr int32_t kStampBlocks = 1 << 20;
constexpr int64_t kStampPerToken = 16;
inline bool one_token_per_block(const int32_t* slots, int32_t n, int32_t num_blocks, int32_t block_size,
                                int32_t stamp_blocks = kStampBlocks) {
  if (n <= 1) return true;
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
  thread_local std::vector<uint32_t> stamp;
  thread_local uint32_t epoch = 0;
  bool stamps = num_blocks <= stamp_blocks && num_blocks <= kStampPerToken * n;
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
