// Host checks of the planner, built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py (CPU only): random rollout forests and packed batches through
// the trie, the minimum-call planner, the descriptor validator and the tree-attention tables;
// then single-field corruptions of valid plans, each of which the validator must reject with
// the right error code.
#include <cstdio>
#include <cstdlib>
#include <functional>
#include <vector>

#include "../../chunkwise_linear_attention_gated_amd/csrc/host/attn_tables.hpp"
#include "../../chunkwise_linear_attention_gated_amd/csrc/host/plan.hpp"
#include "../../include/harts.h"

using harts::PlanHost;

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(uint32_t n) {  // xorshift64*, uniform enough for test shapes
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return uint32_t((g_state * 2685821657736338717ull) >> 33) % n;
}

static int failures = 0;
#define CHECK(cond, ...)                   \
  do {                                     \
    if (!(cond)) {                         \
      std::fprintf(stderr, __VA_ARGS__);   \
      std::fprintf(stderr, "\n");          \
      ++failures;                          \
    }                                      \
  } while (0)

// trajectories that share random prefixes: each new one copies a prefix of an earlier one
static void random_forest(std::vector<int32_t>& tok, std::vector<int64_t>& off, int n, int maxlen) {
  std::vector<std::vector<int32_t>> tr;
  for (int i = 0; i < n; ++i) {
    std::vector<int32_t> t;
    if (!tr.empty() && rnd(4)) {
      const auto& src = tr[rnd(uint32_t(tr.size()))];
      t.assign(src.begin(), src.begin() + 1 + rnd(uint32_t(src.size())));
    }
    const int extra = 1 + int(rnd(uint32_t(maxlen)));
    for (int j = 0; j < extra; ++j) t.push_back(int32_t(rnd(50)));
    tr.push_back(t);
  }
  off.assign(1, 0);
  tok.clear();
  for (auto& t : tr) {
    tok.insert(tok.end(), t.begin(), t.end());
    off.push_back(int64_t(tok.size()));
  }
}

static int code_of(const std::function<void()>& f) {
  try {
    f();
  } catch (const harts::Error& e) {
    return e.code;
  }
  return HARTS_OK;
}

static void corruptions(const PlanHost& good) {
  using Mut = std::function<bool(PlanHost&)>;  // returns false when the plan has nothing to corrupt
  const std::vector<std::pair<int, Mut>> cases = {
      {HARTS_ERANGE, [](PlanHost& p) { if (p.vrows.empty()) return false; p.vrows[rnd(uint32_t(p.vrows.size()))] = int32_t(p.C); return true; }},
      {HARTS_ERANGE, [](PlanHost& p) { p.vrows.back() = -1; return true; }},
      {HARTS_ERANGE, [](PlanHost& p) { p.seq_desc[0].n_replay = p.B; return true; }},
      {HARTS_ERANGE, [](PlanHost& p) { p.seq_desc.back().vlen += 1; return true; }},
      {HARTS_ERANGE, [](PlanHost& p) { p.seq_desc[0].init = p.varlen ? int32_t(p.seq_desc.size()) : p.n_slots; return true; }},
      {HARTS_ERANGE, [](PlanHost& p) { p.chunk_desc.back().len = p.B + 1; return true; }},
      {HARTS_ERANGE, [](PlanHost& p) { p.chunk_desc[0].emit = p.varlen ? p.n_boundaries : p.n_slots; return true; }},
      {HARTS_ERANGE, [](PlanHost& p) { p.rounds.back().chunk1 -= 1; return true; }},
      {HARTS_ERANGE, [](PlanHost& p) { if (p.fix_rows.empty()) return false; p.fix_rows[0] = int32_t(p.C); return true; }},
      {HARTS_ERANGE, [](PlanHost& p) { if (p.fix_idx.empty()) return false; p.fix_idx.back() = int32_t(p.replay_total); return true; }},
      {HARTS_ERANGE, [](PlanHost& p) { if (p.varlen || p.slot_cons.empty()) return false; p.slot_cons[0] = int32_t(p.seq_desc.size()); return true; }},
      // a consumer reading a slot before (or in the same round as) the chunk that writes it
      {HARTS_EINVAL, [](PlanHost& p) {
         if (p.varlen) return false;
         for (auto& d : p.seq_desc)
           if (d.init >= 0) {
             for (auto& c : p.chunk_desc)
               if (c.emit == d.init) c.emit = -1;
             return true;
           }
         return false;
       }},
  };
  for (size_t i = 0; i < cases.size(); ++i) {
    PlanHost p = good;
    if (!cases[i].second(p)) continue;
    const int got = code_of([&] { harts::validate_plan(p); });
    CHECK(got == cases[i].first, "corruption %zu: expected %d, got %d", i, cases[i].first, got);
  }
}

int main() {
  int plans = 0;
  for (int it = 0; it < 300; ++it) {
    std::vector<int32_t> tok;
    std::vector<int64_t> off;
    random_forest(tok, off, 1 + int(rnd(12)), 1 + int(rnd(150)));
    const int B = 16 << rnd(3);
    const harts::TreeHost t = harts::build_tree(tok.data(), off.data(), int64_t(off.size()) - 1);
    const PlanHost p = harts::make_plan(t, B);
    const int c = code_of([&] { harts::validate_plan(p); });
    CHECK(c == HARTS_OK, "valid tree plan %d rejected (%d)", it, c);
    if (it % 10 == 0) corruptions(p);
    const harts::AttnTables at = harts::build_attn_tables(p.m.data(), off.data(), int64_t(off.size()) - 1, p.C);
    CHECK(at.C == p.C, "attention tables of plan %d", it);
    ++plans;
    // a packed batch of the same lengths
    std::vector<uint8_t> has(off.size() - 1);
    for (auto& h : has) h = uint8_t(rnd(2));
    const PlanHost v = harts::make_varlen_plan(off.data(), int64_t(off.size()) - 1, B, has.data(), rnd(2) != 0);
    const int cv = code_of([&] { harts::validate_plan(v); });
    CHECK(cv == HARTS_OK, "valid varlen plan %d rejected (%d)", it, cv);
    if (it % 10 == 0) corruptions(v);
    ++plans;
  }
  // bad inputs are refused with error codes, not undefined behaviour
  const int32_t tk[3] = {1, 2, 3};
  const int64_t o1[3] = {0, 3, 3};
  CHECK(code_of([&] { harts::build_tree(tk, o1, 2); }) == HARTS_EINVAL, "empty trajectory accepted");
  const int64_t o2[2] = {0, 3};
  CHECK(code_of([&] { harts::make_plan(harts::build_tree(tk, o2, 1), 48); }) == HARTS_EINVAL, "chunk 48 accepted");
  std::printf("%d plans checked, %d failures\n", plans, failures);
  return failures ? 1 : 0;
}
