// Stress test of the host block manager through its C ABI, meant to run under AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only). Seeded random operations -- prompts with shared prefixes, forks,
// decode appends with copy-on-write, finished sequences, swaps to a host pool and back -- are replayed on host
// stand-ins for the device and host pools, where each slot holds the identity of the token written there. After
// every operation each running sequence's block table must reproduce its logical token list, and the occupancy
// counters must add up. Exit status 0 on success.
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <map>
#include <vector>

#include "../../include/pa.h"
#include "../../include/paged_block_manager.h"

namespace {

struct Rng {  // 64-bit linear congruential generator (Knuth's MMIX constants), high bits used
  uint64_t s;
  explicit Rng(uint64_t seed) : s(seed * 2654435761u + 1) {}
  uint32_t next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(s >> 33);
  }
  int32_t below(int32_t n) { return (int32_t)(next() % (uint32_t)n); }
};

int fail(const char* what, int64_t a, int64_t b) {
  fprintf(stderr, "FAIL: %s (%lld, %lld)\n", what, (long long)a, (long long)b);
  return 1;
}

int run(uint64_t seed) {
  const int32_t nb = 48, bs = 4, mb = 24, nh = 40, reserved = nb - 1;
  pa_block_manager* bm = pa_bm_create(nb, bs, mb, reserved);
  if (!bm) return fail("create", nb, bs);
  if (pa_bm_set_host_pool(bm, nh) != PA_OK) return fail("set_host_pool", nh, 0);
  Rng rng(seed);
  std::vector<int64_t> dev((size_t)nb * bs, -1), host((size_t)nh * bs, -1);
  std::map<int64_t, std::vector<int64_t>> running, swapped;  // logical token identities per sequence
  std::vector<int32_t> system(9);
  for (auto& t : system) t = rng.below(50);
  int64_t next_id = 0, next_token = 1000000;
  std::vector<int32_t> slots(mb * bs + 8), pairs(2 * (nb + 8)), table((size_t)mb * 64), lens(64);

  auto pick = [&](const std::map<int64_t, std::vector<int64_t>>& m) {
    auto it = m.begin();
    std::advance(it, rng.below((int32_t)m.size()));
    return it->first;
  };

  for (int op = 0; op < 20000; ++op) {
    const int32_t r = rng.below(100);
    if (r < 18 || running.empty()) {  // a new prompt, often starting with the common prefix
      std::vector<int32_t> tokens;
      if (rng.below(10) < 6) tokens = system;
      const int32_t extra = 1 + rng.below(8);
      for (int32_t i = 0; i < extra; ++i) tokens.push_back(rng.below(50));
      const int32_t n = (int32_t)tokens.size();
      const int32_t rc = pa_bm_add_sequence(bm, next_id, tokens.data(), n, slots.data());
      if (rc == PA_ERR_NOMEM) continue;
      if (rc < 0) return fail("add_sequence", rc, op);
      // a token's identity depends on the prompt up to it (shared blocks hold equal identities)
      std::vector<int64_t> ident(n);
      uint64_t h = 1469598103934665603ull;
      for (int32_t t = 0; t < n; ++t) {
        h = (h ^ (uint64_t)tokens[t]) * 1099511628211ull;
        ident[t] = (int64_t)(h >> 1);
        if (slots[t] >= 0) dev[slots[t]] = ident[t];
      }
      running[next_id++] = ident;
    } else if (r < 26) {  // fork
      const int64_t parent = pick(running);
      if (pa_bm_fork(bm, parent, next_id) != PA_OK) return fail("fork", parent, op);
      running[next_id++] = running[parent];
    } else if (r < 36) {  // finish a running or swapped-out sequence
      const bool sw = !swapped.empty() && rng.below(3) == 0;
      const int64_t victim = sw ? pick(swapped) : pick(running);
      if (pa_bm_free_sequence(bm, victim) != PA_OK) return fail("free", victim, op);
      (sw ? swapped : running).erase(victim);
    } else if (r < 46) {  // swap out
      const int64_t victim = pick(running);
      const int32_t n = pa_bm_swap_out(bm, victim, pairs.data(), (int32_t)pairs.size() / 2);
      if (n == PA_ERR_NOMEM) continue;
      if (n < 0) return fail("swap_out", n, op);
      for (int32_t i = 0; i < n; ++i)
        std::copy_n(dev.begin() + (int64_t)pairs[2 * i] * bs, bs, host.begin() + (int64_t)pairs[2 * i + 1] * bs);
      swapped[victim] = running[victim];
      running.erase(victim);
      if (pa_bm_block_tables(bm, &victim, 1, table.data(), lens.data(), reserved) != PA_ERR_SEQ)
        return fail("swapped sequence listed", victim, op);
    } else if (r < 56 && !swapped.empty()) {  // swap in
      const int64_t sid = pick(swapped);
      const int32_t n = pa_bm_swap_in(bm, sid, pairs.data(), (int32_t)pairs.size() / 2);
      if (n == PA_ERR_NOMEM) continue;
      if (n < 0) return fail("swap_in", n, op);
      for (int32_t i = 0; i < n; ++i)
        std::copy_n(host.begin() + (int64_t)pairs[2 * i] * bs, bs, dev.begin() + (int64_t)pairs[2 * i + 1] * bs);
      running[sid] = swapped[sid];
      swapped.erase(sid);
    } else {  // a decode step for a random subset of the running sequences
      std::vector<int64_t> ids;
      for (const auto& kv : running)
        if (rng.below(2)) ids.push_back(kv.first);
      if (ids.empty()) continue;
      const int32_t rc = pa_bm_append_slots(bm, ids.data(), (int32_t)ids.size(), slots.data());
      if (rc == PA_ERR_NOMEM || rc == PA_ERR_SHAPE) continue;
      if (rc < 0) return fail("append", rc, op);
      const int32_t n = pa_bm_take_copies(bm, pairs.data(), (int32_t)pairs.size() / 2);
      if (n < 0) return fail("take_copies", n, op);
      for (int32_t i = 0; i < n; ++i)  // copies first, then the new tokens
        std::copy_n(dev.begin() + (int64_t)pairs[2 * i] * bs, bs, dev.begin() + (int64_t)pairs[2 * i + 1] * bs);
      for (size_t i = 0; i < ids.size(); ++i) {
        dev[slots[i]] = next_token;
        running[ids[i]].push_back(next_token++);
      }
    }
    // every running sequence reads back its logical tokens through its table
    for (const auto& kv : running) {
      const int64_t id = kv.first;
      if (pa_bm_block_tables(bm, &id, 1, table.data(), lens.data(), reserved) != PA_OK) return fail("tables", id, op);
      if (lens[0] != (int32_t)kv.second.size()) return fail("length", lens[0], (int64_t)kv.second.size());
      for (int32_t t = 0; t < lens[0]; ++t) {
        const int32_t b = table[t / bs];
        if (b < 0 || b >= nb || b == reserved) return fail("table entry", b, op);
        if (dev[(int64_t)b * bs + t % bs] != kv.second[t]) return fail("token", id, t);
      }
    }
    int64_t st[8], sw[4];
    if (pa_bm_stats(bm, st) != PA_OK || pa_bm_swap_stats(bm, sw) != PA_OK) return fail("stats", op, 0);
    if (st[0] + st[1] + 1 != nb) return fail("free + used + reserved", st[0] + st[1], nb);
    if (st[3] != (int64_t)running.size()) return fail("sequences", st[3], (int64_t)running.size());
    if (sw[0] + sw[1] != nh || sw[2] != (int64_t)swapped.size()) return fail("host pool", sw[0] + sw[1], sw[2]);
    int64_t host_used = 0;
    for (const auto& kv : swapped) host_used += ((int64_t)kv.second.size() + bs - 1) / bs;
    if (sw[1] != host_used) return fail("host blocks in use", sw[1], host_used);
  }
  // swapped-out sequences come back intact
  for (const auto& kv : swapped) {
    const int64_t id = kv.first;
    for (const auto& rkv : running) pa_bm_free_sequence(bm, rkv.first);
    running.clear();
    const int32_t n = pa_bm_swap_in(bm, id, pairs.data(), (int32_t)pairs.size() / 2);
    if (n < 0) return fail("final swap_in", n, id);
    for (int32_t i = 0; i < n; ++i)
      std::copy_n(host.begin() + (int64_t)pairs[2 * i] * bs, bs, dev.begin() + (int64_t)pairs[2 * i + 1] * bs);
    if (pa_bm_block_tables(bm, &id, 1, table.data(), lens.data(), reserved) != PA_OK) return fail("final tables", id, 0);
    for (int32_t t = 0; t < lens[0]; ++t)
      if (dev[(int64_t)table[t / bs] * bs + t % bs] != kv.second[t]) return fail("final token", id, t);
    pa_bm_free_sequence(bm, id);
  }
  pa_bm_destroy(bm);
  return 0;
}

}  // namespace

int main() {
  for (uint64_t seed = 1; seed <= 6; ++seed)
    if (run(seed)) {
      fprintf(stderr, "seed %llu\n", (unsigned long long)seed);
      return 1;
    }
  printf("block manager stress: ok\n");
  return 0;
}
