// Host thread model of the library's cross-workgroup protocols, one
// std::thread per workgroup, built with ThreadSanitizer by
// tests/test_join_model.py.  Each protocol is restated here with C++ atomics
// in the order the device code performs its steps:
//
//  gen     the generation-counted join: a member publishes its partial
//          (plain memory here, so the sanitizer checks that every read is
//          ordered after its write through the join word), arrives with one
//          fetch-add (the last arriver advances the generation and resets the
//          count in one atomic), the others poll until the generation moves,
//          then every member reads all partials;
//  split   the split-row exchange: per launch every member clears its four
//          tagged slots and arrives on the group's launch join, then for each
//          row it walks publishes two {tag, value} slots (double-buffered by
//          row parity, tag = 1 + the row's index within the launch), awaits the
//          launch join before its first take, and takes every member's slots by
//          tag;
//  ln      the GEMM + LayerNorm exchange: per launch every member clears its
//          slots, arrives after its MainLoop, publishes {1, value} slots once,
//          awaits the launch join and takes every member's slots by tag;
//  missing one member of a group never arrives or publishes (a workgroup that
//          is not resident): every wait gives up at the spin cap, sets the
//          error word, and every thread still finishes.
//
// Values encode (launch, row, member), so a stale or foreign value that a
// reader accepted shows up as a wrong merged result.  Random sleeps perturb
// the interleaving.  Exit status 0 and "OK <scenario>" on success.
#include <atomic>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <thread>
#include <vector>

namespace {

uint32_t g_cap = 1u << 22;  // spin cap (iterations), lowered for the missing-member scenario

void jitter(std::mt19937& rng) {
  const uint32_t r = rng() % 16;
  if (r < 3) std::this_thread::sleep_for(std::chrono::microseconds(rng() % 40));
  else if (r < 8) std::this_thread::yield();
}

// ---- the generation-counted join word {generation:32 | arrivals:32}
bool arrive_and_wait(std::atomic<uint64_t>& j, uint32_t members, std::atomic<uint32_t>& err) {
  const uint64_t old = j.fetch_add(1, std::memory_order_acq_rel);
  const uint32_t gen0 = (uint32_t)(old >> 32);
  if ((uint32_t)old == members - 1) {
    j.fetch_add((1ull << 32) - members, std::memory_order_acq_rel);
    return true;
  }
  for (uint32_t it = 0; it < g_cap; ++it) {
    if ((uint32_t)(j.load(std::memory_order_acquire) >> 32) != gen0) return true;
    std::this_thread::yield();
  }
  err.fetch_or(1);
  return false;
}
// split form: arrive early (the last arriver advances at once), await later
uint64_t arrive(std::atomic<uint64_t>& j, uint32_t members) {
  const uint64_t old = j.fetch_add(1, std::memory_order_acq_rel);
  if ((uint32_t)old == members - 1) j.fetch_add((1ull << 32) - members, std::memory_order_acq_rel);
  return old;
}
bool await(std::atomic<uint64_t>& j, uint64_t old, uint32_t members, std::atomic<uint32_t>& err) {
  if ((uint32_t)old == members - 1) return true;
  const uint32_t gen0 = (uint32_t)(old >> 32);
  for (uint32_t it = 0; it < g_cap; ++it) {
    if ((uint32_t)(j.load(std::memory_order_acquire) >> 32) != gen0) return true;
    std::this_thread::yield();
  }
  err.fetch_or(1);
  return false;
}

// ---- tagged slots {tag:32 | value:32}, one atomic word each
void put(std::atomic<uint64_t>& s, uint32_t tag, uint32_t v) {
  s.store(((uint64_t)tag << 32) | v, std::memory_order_relaxed);
}
bool take(std::atomic<uint64_t>& s, uint32_t tag, uint32_t* v, std::atomic<uint32_t>& err) {
  for (uint32_t it = 0; it < g_cap; ++it) {
    const uint64_t w = s.load(std::memory_order_relaxed);
    if ((uint32_t)(w >> 32) == tag) {
      *v = (uint32_t)w;
      return true;
    }
    std::this_thread::yield();
  }
  err.fetch_or(1);
  *v = 0;
  return false;
}

uint32_t code(uint32_t launch, uint32_t row, uint32_t member) { return (launch * 1000003u + row * 131u + member) & 0xFFFFFFFu; }

int fails = 0;
std::atomic<int> bad{0};
// planted mistakes (the model must catch each): read the partials without
// waiting for the join; take slots before the launch join; one slot set for
// every row (no parity double buffering)
bool m_nowait = false, m_noawait = false, m_oneparity = false;

// gen: G groups x S members, each launch R rows per group, partials per row
void scenario_gen(int G, int S, int R, int L) {
  std::vector<std::atomic<uint64_t>> joins(G);
  for (auto& j : joins) j.store(0);
  std::vector<uint32_t> partials((size_t)G * R * S);  // plain memory
  std::atomic<uint32_t> err{0};
  for (int launch = 0; launch < L; ++launch) {
    std::vector<std::thread> th;
    for (int g = 0; g < G; ++g)
      for (int s = 0; s < S; ++s)
        th.emplace_back([&, g, s, launch] {
          std::mt19937 rng(launch * 7919 + g * 131 + s);
          for (int r = 0; r < R; ++r) {
            jitter(rng);
            partials[((size_t)g * R + r) * S + s] = code(launch, r, s);
            if (!m_nowait && !arrive_and_wait(joins[g], (uint32_t)S, err)) return;
            uint64_t got = 0, want = 0;
            for (int q = 0; q < S; ++q) {
              got += partials[((size_t)g * R + r) * S + q];
              want += code(launch, r, q);
            }
            if (got != want) bad.fetch_add(1);
          }
        });
    for (auto& t : th) t.join();
  }
  if (err.load() != 0 || bad.load() != 0) ++fails;
}

// split: the tagged exchange of rows split over S members, G groups walking
// R rows each per launch, slots double-buffered by row parity
void scenario_split(int G, int S, int R, int L, int missing_group = -1) {
  std::vector<std::atomic<uint64_t>> joins(G);
  for (auto& j : joins) j.store(0);
  std::vector<std::atomic<uint64_t>> slots((size_t)G * 4 * S);
  for (auto& x : slots) x.store(0xDEADBEEF00000001ull);  // foreign data, tag-like bits included
  std::atomic<uint32_t> err{0};
  for (int launch = 0; launch < L; ++launch) {
    std::vector<std::thread> th;
    for (int g = 0; g < G; ++g)
      for (int s = 0; s < S; ++s)
        th.emplace_back([&, g, s, launch] {
          if (g == missing_group && s == 0) return;  // never resident: no clear, no arrival, no partials
          std::mt19937 rng(launch * 104729 + g * 17 + s);
          std::atomic<uint64_t>* sl = &slots[(size_t)g * 4 * S];
          jitter(rng);  // members start at different times
          for (int k = 0; k < 4; ++k) sl[k * S + s].store(0, std::memory_order_relaxed);
          const uint64_t jold = arrive(joins[g], (uint32_t)S);
          for (uint32_t it = 0; it < (uint32_t)R; ++it) {
            jitter(rng);
            const uint32_t tag = it + 1;
            std::atomic<uint64_t>* sp = sl + (m_oneparity ? 0u : (it & 1u)) * 2 * S;
            if (it == 0 && !m_noawait && !await(joins[g], jold, (uint32_t)S, err)) return;
            put(sp[s], tag, code(launch, it, s));
            put(sp[S + s], tag, code(launch, it, s) ^ 0x5555u);
            uint64_t got = 0, want = 0;
            for (int q = 0; q < S; ++q) {
              uint32_t a = 0, b = 0;
              if (!take(sp[q], tag, &a, err) || !take(sp[S + q], tag, &b, err)) return;
              got += a + (b ^ 0x5555u);
              want += 2ull * code(launch, it, q);
            }
            if (got != want) bad.fetch_add(1);
          }
        });
    for (auto& t : th) t.join();
    if (missing_group >= 0) break;
  }
  if (missing_group >= 0) {
    if (err.load() == 0) ++fails;  // the waits must have given up
  } else if (err.load() != 0 || bad.load() != 0) {
    ++fails;
  }
}

// ln: member-major tagged slots, one publication per member per launch
void scenario_ln(int B, int T, int rows, int L) {
  std::vector<std::atomic<uint64_t>> joins(B);
  for (auto& j : joins) j.store(0);
  std::vector<std::atomic<uint64_t>> slots((size_t)B * T * rows * 2);
  for (auto& x : slots) x.store(0x0000000100000000ull | 7u);  // a stale {tag 1} from before the first launch
  std::atomic<uint32_t> err{0};
  for (int launch = 0; launch < L; ++launch) {
    std::vector<std::thread> th;
    for (int b = 0; b < B; ++b)
      for (int k = 0; k < T; ++k)
        th.emplace_back([&, b, k, launch] {
          std::mt19937 rng(launch * 31337 + b * 101 + k);
          std::atomic<uint64_t>* base = &slots[(size_t)b * T * rows * 2];
          for (int i = 0; i < rows; ++i) {
            base[((size_t)k * rows + i) * 2].store(0, std::memory_order_relaxed);
            base[((size_t)k * rows + i) * 2 + 1].store(0, std::memory_order_relaxed);
          }
          jitter(rng);  // the MainLoop
          const uint64_t jold = arrive(joins[b], (uint32_t)T);
          jitter(rng);  // residual and tile statistics
          for (int i = 0; i < rows; ++i) {
            put(base[((size_t)k * rows + i) * 2], 1u, code(launch, i, k));
            put(base[((size_t)k * rows + i) * 2 + 1], 1u, code(launch, i, k) ^ 0x3333u);
          }
          if (!await(joins[b], jold, (uint32_t)T, err)) return;
          for (int i = 0; i < rows; ++i) {
            uint64_t got = 0, want = 0;
            for (int q = 0; q < T; ++q) {
              uint32_t x = 0, y = 0;
              if (!take(base[((size_t)q * rows + i) * 2], 1u, &x, err) ||
                  !take(base[((size_t)q * rows + i) * 2 + 1], 1u, &y, err))
                return;
              got += x + (y ^ 0x3333u);
              want += 2ull * code(launch, i, q);
            }
            if (got != want) bad.fetch_add(1);
          }
        });
    for (auto& t : th) t.join();
  }
  if (err.load() != 0 || bad.load() != 0) ++fails;
}

}  // namespace

int main(int argc, char** argv) {
  const std::string sc = argc > 1 ? argv[1] : "all";
  if (sc == "gen" || sc == "all") scenario_gen(3, 5, 6, 4);
  if (sc == "split" || sc == "all") scenario_split(3, 6, 7, 5);
  if (sc == "ln" || sc == "all") scenario_ln(2, 8, 16, 4);
  if (sc == "missing") {
    g_cap = 1u << 12;
    scenario_split(2, 4, 3, 1, 1);
  }
  if (sc == "mutant-nowait") {
    m_nowait = true;
    scenario_gen(3, 5, 6, 4);
  }
  if (sc == "mutant-noawait") {
    // one row per group and launch: every slot of parity 0 still holds the
    // previous launch's tag 1 until its owner clears it
    m_noawait = true;
    g_cap = 1u << 16;
    scenario_split(4, 8, 1, 60);
  }
  if (sc == "mutant-oneparity") {
    m_oneparity = true;
    g_cap = 1u << 16;
    scenario_split(3, 6, 7, 3);
  }
  if (fails != 0) {
    std::printf("FAIL %s (%d scenario(s), %d wrong merges)\n", sc.c_str(), fails, bad.load());
    return 1;
  }
  std::printf("OK %s\n", sc.c_str());
  return 0;
}
