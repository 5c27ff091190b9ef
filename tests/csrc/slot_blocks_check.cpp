// CPU harness for pa::one_token_per_block.  Reads cases from stdin:
//   count, then per case: num_blocks block_size stamp_blocks n slot_0 .. slot_{n-1}
// and prints one 0/1 answer per line, in order.  Cases run in one thread, so
// they share the per-thread stamp array the way successive library calls do.
#include <cstdio>
#include <vector>

#include "slot_blocks.hpp"

int main() {
  int count = 0;
  if (std::scanf("%d", &count) != 1) return 2;
  for (int c = 0; c < count; ++c) {
    int32_t nb = 0, bs = 0, limit = 0, n = 0;
    if (std::scanf("%d %d %d %d", &nb, &bs, &limit, &n) != 4) return 2;
    std::vector<int32_t> slots(static_cast<size_t>(n));
    for (auto& s : slots)
      if (std::scanf("%d", &s) != 1) return 2;
    std::printf("%d\n", pa::one_token_per_block(slots.data(), n, nb, bs, limit) ? 1 : 0);
  }
  return 0;
}
