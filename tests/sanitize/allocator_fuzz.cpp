// Random operations on the host allocator's C API, built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_allocator_sanitized.py (host
// code only: allocator.cpp and status.cpp, no device code).  Valid and invalid
// calls alike: unknown and duplicate ids, exhausted pools, out-of-range
// blocks, undersized output buffers, clones, prefixes, swaps, windows, the
// shared-prefix grouping and the launch order.  The sanitizers report memory
// and undefined-behaviour errors; this program itself checks that every block is
// either free or referenced and that no call returns an unknown status.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "pa.h"

namespace {

struct Rng {  // 64-bit linear congruential generator (Knuth's MMIX constants)
  uint64_t s;
  uint32_t next() {
    s = s * 6364136223846793005ULL + 1442695040888963407ULL;
    return static_cast<uint32_t>(s >> 33);
  }
  int32_t below(int32_t n) { return n > 0 ? static_cast<int32_t>(next() % static_cast<uint32_t>(n)) : 0; }
};

int failures = 0;

void expect(bool ok, const char* what, int seed, int step) {
  if (!ok) {
    std::fprintf(stderr, "seed %d step %d: %s\n", seed, step, what);
    ++failures;
  }
}

bool known(pa_status s) { return s >= PA_OK && s <= PA_ERR_UNKNOWN_PREFIX; }

void check_blocks(const pa_allocator* a, int32_t nb, int seed, int step) {
  int32_t used = 0;
  for (int32_t b = 0; b < nb; ++b) {
    const int32_t r = pa_ref_count(a, b);
    expect(r >= 0, "negative refcount", seed, step);
    used += r > 0;
  }
  expect(used + pa_num_free_blocks(a) == nb, "a block is neither free nor referenced", seed, step);
  expect(pa_ref_count(a, -1) == -1 && pa_ref_count(a, nb) == -1, "refcount outside the pool", seed, step);
}

void run(int seed) {
  Rng g{static_cast<uint64_t>(seed) * 7919u + 1u};
  const int32_t bs = g.below(2) ? 16 : 32;
  const int32_t nb = 24 + g.below(80);
  std::vector<int32_t> order(nb);
  for (int32_t i = 0; i < nb; ++i) order[i] = i;
  for (int32_t i = nb - 1; i > 0; --i) std::swap(order[i], order[g.below(i + 1)]);
  pa_allocator* a = nullptr;
  if (pa_allocator_create(nb, bs, g.below(2) ? order.data() : nullptr, &a) != PA_OK || !a) {
    expect(false, "create failed", seed, -1);
    return;
  }
  pa_allocator_set_host_pool(a, g.below(40));
  std::vector<int64_t> live;
  std::vector<int64_t> prefixes;
  int64_t next_id = 1;
  for (int step = 0; step < 400; ++step) {
    const int op = g.below(16);
    const int64_t some = live.empty() ? 999 : live[g.below(static_cast<int32_t>(live.size()))];
    pa_status st = PA_OK;
    switch (op) {
      case 0: {  // create (sometimes an existing id)
        const int64_t id = g.below(8) ? next_id++ : some;
        st = pa_seq_create(a, id, g.below(5 * bs));
        if (st == PA_OK) live.push_back(id);
        break;
      }
      case 1: {  // fork (sometimes more tokens than the parent, -1 for all)
        const int64_t id = next_id++;
        int32_t len = 0;
        if (pa_seq_len(a, some, &len) != PA_OK) len = 10;
        st = pa_seq_fork(a, some, id, g.below(4) ? g.below(len + 2) : -1);
        if (st == PA_OK) live.push_back(id);
        break;
      }
      case 2: {  // append one
        int32_t slot = 0, src = 0, dst = 0;
        st = pa_seq_append_slot(a, some, &slot, &src, &dst);
        break;
      }
      case 3: {  // a batch of appends, possibly with unknown ids
        std::vector<int64_t> ids;
        for (int i = g.below(6); i > 0; --i)
          ids.push_back(g.below(5) ? some : 777777);
        if (!live.empty())
          for (int i = g.below(4); i > 0; --i) ids.push_back(live[g.below(static_cast<int32_t>(live.size()))]);
        std::vector<int32_t> slots(ids.size() + 1), pairs(2 * ids.size() + 2);
        int32_t np = 0;
        st = pa_seq_append_slots(a, ids.data(), static_cast<int32_t>(ids.size()), slots.data(), pairs.data(), &np);
        break;
      }
      case 4: {  // free (sometimes twice)
        st = pa_seq_free(a, some);
        if (st == PA_OK)
          for (size_t i = 0; i < live.size(); ++i)
            if (live[i] == some) {
              live.erase(live.begin() + static_cast<long>(i));
              break;
            }
        break;
      }
      case 5: {  // tables, with a capacity that is sometimes too small
        std::vector<int64_t> ids(live.begin(), live.end());
        if (g.below(4) == 0) ids.push_back(123456);
        const int32_t mb = g.below(12);
        std::vector<int32_t> tab(ids.size() * static_cast<size_t>(mb) + 1), lens(ids.size() + 1);
        st = pa_build_block_tables(a, ids.data(), static_cast<int32_t>(ids.size()), mb, tab.data(), lens.data());
        if (st == PA_OK && mb > 0 && !ids.empty()) {
          std::vector<int32_t> gs(ids.size() + 1), pl(ids.size() + 1), ord(ids.size() + 1);
          int32_t ng = 0, mg = 0;
          expect(pa_shared_prefix_groups(tab.data(), lens.data(), static_cast<int32_t>(ids.size()), mb, bs,
                                         gs.data(), pl.data(), &ng, &mg) == PA_OK,
                 "grouping failed", seed, step);
          expect(pa_order_longest_first(lens.data(), static_cast<int32_t>(ids.size()), ord.data()) == PA_OK,
                 "order failed", seed, step);
        }
        std::vector<int32_t> lo(ids.size() + 1), hi(ids.size() + 1);
        pa_build_masks(a, ids.data(), static_cast<int32_t>(ids.size()), lo.data(), hi.data());
        break;
      }
      case 6: {  // a table into a buffer of random capacity
        std::vector<int32_t> out(static_cast<size_t>(g.below(8)) + 1);
        int32_t n = 0;
        st = pa_seq_block_table(a, some, out.data(), static_cast<int32_t>(out.size()) - g.below(2), &n);
        std::vector<int32_t> fl(static_cast<size_t>(nb));
        pa_free_list(a, fl.data(), g.below(nb + 1), &n);
        break;
      }
      case 7: {  // prefix get_or_create from a few token strings
        std::vector<int32_t> toks(static_cast<size_t>(g.below(3 * bs)));
        const int32_t base = g.below(3);
        for (size_t i = 0; i < toks.size(); ++i) toks[i] = base * 1000 + static_cast<int32_t>(i);
        int64_t pid = -1;
        int32_t hit = 0;
        st = pa_prefix_get_or_create(a, toks.data(), static_cast<int32_t>(toks.size()), &pid, &hit);
        if (st == PA_OK) prefixes.push_back(pid);
        break;
      }
      case 8: {  // a sequence on a prefix (sometimes an unknown one)
        const int64_t pid = prefixes.empty() || g.below(6) == 0 ? 424242
                                                                : prefixes[g.below(static_cast<int32_t>(prefixes.size()))];
        const int64_t id = next_id++;
        st = pa_seq_create_with_prefix(a, id, pid, g.below(2 * bs));
        if (st == PA_OK) live.push_back(id);
        int32_t blocks[8], nbk = 0, nt = 0, users = 0;
        pa_prefix_info(a, pid, blocks, g.below(9), &nbk, &nt, &users);
        break;
      }
      case 9: {  // release a prefix (sometimes twice)
        if (!prefixes.empty()) {
          const size_t i = static_cast<size_t>(g.below(static_cast<int32_t>(prefixes.size())));
          st = pa_prefix_release(a, prefixes[i]);
          if (st == PA_OK && g.below(2)) prefixes.erase(prefixes.begin() + static_cast<long>(i));
        }
        break;
      }
      case 10:
      case 11: {  // swap a group out or in
        std::vector<int64_t> ids;
        for (int i = 1 + g.below(3); i > 0; --i) ids.push_back(g.below(6) ? some : 55555);
        std::vector<int32_t> pairs(static_cast<size_t>(2 * g.below(2 * nb) + 2));
        int32_t np = 0;
        st = op == 10 ? pa_seq_swap_out(a, ids.data(), static_cast<int32_t>(ids.size()), pairs.data(),
                                        static_cast<int32_t>(pairs.size() / 2), &np)
                      : pa_seq_swap_in(a, ids.data(), static_cast<int32_t>(ids.size()), pairs.data(),
                                       static_cast<int32_t>(pairs.size() / 2), &np);
        std::vector<int32_t> hf(64);
        int32_t n = 0;
        pa_host_free_list(a, hf.data(), static_cast<int32_t>(hf.size()), &n);
        pa_host_ref_count(a, g.below(50) - 5);
        break;
      }
      case 12:  // a sliding window (sometimes invalid)
        st = pa_seq_set_window(a, some, g.below(4 * bs) - 2);
        break;
      case 13: {  // clone, use the clone, destroy it
        pa_allocator* c = nullptr;
        st = pa_allocator_clone(a, &c);
        if (st == PA_OK) {
          pa_seq_create(c, next_id + 100000, g.below(3 * bs));
          check_blocks(c, nb, seed, step);
          pa_allocator_destroy(c);
        }
        break;
      }
      case 14: {
        int32_t ok = 0;
        st = pa_can_allocate(a, g.below(2 * nb) - 3, &ok);
        pa_allocator_stats stats;
        pa_allocator_get_stats(a, &stats);
        break;
      }
      default: {  // null and negative arguments
        st = pa_seq_create(a, next_id++, -5);
        expect(st != PA_OK, "negative token count accepted", seed, step);
        st = pa_build_block_tables(a, nullptr, 3, 4, nullptr, nullptr);
        expect(st != PA_OK, "null tables accepted", seed, step);
        int32_t ng = 0, mg = 0;
        st = pa_shared_prefix_groups(nullptr, nullptr, -1, 0, bs, nullptr, nullptr, &ng, &mg);
        expect(st != PA_OK, "negative grouping size accepted", seed, step);
        break;
      }
    }
    expect(known(st), "unknown status", seed, step);
    check_blocks(a, nb, seed, step);
  }
  pa_allocator_destroy(a);
}

}  // namespace

int main(int argc, char** argv) {
  const int seeds = argc > 1 ? std::atoi(argv[1]) : 200;
  for (int s = 0; s < seeds; ++s) run(s);
  if (failures) {
    std::fprintf(stderr, "%d failed checks\n", failures);
    return 1;
  }
  std::printf("ok: %d seeds\n", seeds);
  return 0;
}
