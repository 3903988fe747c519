// Host tables of tree softmax attention (see attn_tables.hpp).  The ancestor
// view of a branch (HARTS, section 4 "MLA execution"; blog section 4.3) is
// kept as a list of row indices per fork-free segment instead of a copy of
// the ancestors' keys and values.
#include "attn_tables.hpp"

#include <algorithm>
#include <climits>
#include <numeric>
#include <string>

#include "../../../include/harts.h"
#include "plan.hpp"

namespace harts {

AttnTables build_attn_tables(const int64_t* m, const int64_t* off, int64_t n_traj, int64_t C) {
  if (n_traj < 0 || C < 0) throw Error(HARTS_EINVAL, "need n_traj >= 0, C >= 0");
  if (C > INT32_MAX) throw Error(HARTS_ERANGE, "C must fit int32 row indices");
  if (!off || off[0] != 0) throw Error(HARTS_EINVAL, "traj_offsets[0] must be 0");
  for (int64_t i = 0; i < n_traj; ++i)
    if (off[i + 1] < off[i]) throw Error(HARTS_EINVAL, "traj_offsets must be non-decreasing");
  if (off[n_traj] > 0 && !m) throw Error(HARTS_EINVAL, "m is NULL");

  AttnTables t;
  t.C = C;
  constexpr int32_t kUnset = INT32_MIN;
  std::vector<int32_t> parent(size_t(C), kUnset);
  t.pos.assign(size_t(C), 0);
  for (int64_t i = 0; i < n_traj; ++i)
    for (int64_t p = 0; p < off[i + 1] - off[i]; ++p) {
      const int64_t r = m[off[i] + p];
      if (r < 0 || r >= C) throw Error(HARTS_EINVAL, "m[" + std::to_string(off[i] + p) + "] is outside [0, C)");
      const int32_t a = p ? int32_t(m[off[i] + p - 1]) : -1;
      if (parent[size_t(r)] == kUnset) {
        parent[size_t(r)] = a;
        if (p > INT32_MAX - 1) throw Error(HARTS_ERANGE, "trajectory too long");
        t.pos[size_t(r)] = int32_t(p);
      } else if (parent[size_t(r)] != a || t.pos[size_t(r)] != p) {
        throw Error(HARTS_EINVAL, "m is not the map of a prefix tree: row " + std::to_string(r) +
                                      " has two different prefixes");
      }
    }
  std::vector<int32_t> nchild(size_t(C), 0);
  for (int64_t r = 0; r < C; ++r) {
    if (parent[size_t(r)] == kUnset) throw Error(HARTS_EINVAL, "row " + std::to_string(r) + " is on no trajectory");
    if (parent[size_t(r)] >= 0) ++nchild[size_t(parent[size_t(r)])];
    t.pairs += int64_t(t.pos[size_t(r)]) + 1;
    t.max_depth = std::max(t.max_depth, t.pos[size_t(r)] + 1);
  }

  // fork-free segments: row r continues the segment of r - 1 iff r - 1 is its parent and
  // has no other child
  std::vector<int64_t> seg_r0, seg_r1;
  std::vector<int32_t> seg_of(static_cast<size_t>(C));
  for (int64_t r = 0; r < C; ++r) {
    const int32_t p = parent[size_t(r)];
    if (r == 0 || p != r - 1 || nchild[size_t(p)] != 1) {
      seg_r0.push_back(r);
      seg_r1.push_back(r + 1);
    } else {
      seg_r1.back() = r + 1;
    }
    seg_of[size_t(r)] = int32_t(seg_r0.size() - 1);
  }
  const size_t ns = seg_r0.size();
  t.n_segments = int64_t(ns);
  // a segment's first row hangs below the last row of its parent segment: a row with a
  // child other than the next row ends its segment
  std::vector<std::vector<int32_t>> kids(ns);
  for (size_t s = 0; s < ns; ++s) {
    const int32_t p = parent[size_t(seg_r0[s])];
    if (p >= 0) kids[size_t(seg_of[size_t(p)])].push_back(int32_t(s));
  }

  auto grow = [](std::vector<int32_t>& v, int64_t extra) {
    if (int64_t(v.size()) + extra > INT32_MAX) throw Error(HARTS_ERANGE, "attention row lists exceed int32 offsets");
  };
  std::vector<int32_t> stack;
  for (size_t s = 0; s < ns; ++s) {
    const int64_t r0 = seg_r0[s], r1 = seg_r1[s], len = r1 - r0;
    const int32_t h = t.pos[size_t(r0)];
    // kv list: ancestors root first, then own rows
    grow(t.kv_list, int64_t(h) + len);
    const int64_t kv_off = int64_t(t.kv_list.size());
    t.kv_list.resize(t.kv_list.size() + size_t(h) + size_t(len));
    int32_t a = parent[size_t(r0)];
    for (int64_t i = h - 1; i >= 0; --i, a = parent[size_t(a)]) t.kv_list[size_t(kv_off + i)] = a;
    for (int64_t i = 0; i < len; ++i) t.kv_list[size_t(kv_off + h + i)] = int32_t(r0 + i);
    // q list: own rows, then every segment below (depth first)
    const int64_t q_off = int64_t(t.q_list.size());
    grow(t.q_list, len);
    for (int64_t i = 0; i < len; ++i) t.q_list.push_back(int32_t(r0 + i));
    stack.assign(kids[s].rbegin(), kids[s].rend());
    while (!stack.empty()) {
      const int32_t d = stack.back();
      stack.pop_back();
      grow(t.q_list, seg_r1[size_t(d)] - seg_r0[size_t(d)]);
      for (int64_t r = seg_r0[size_t(d)]; r < seg_r1[size_t(d)]; ++r) t.q_list.push_back(int32_t(r));
      stack.insert(stack.end(), kids[size_t(d)].rbegin(), kids[size_t(d)].rend());
    }
    const int64_t below = int64_t(t.q_list.size()) - q_off - len;
    for (int64_t a0 = r0; a0 < r1; a0 += kAttnQTile) {
      const int32_t n = int32_t(std::min<int64_t>(kAttnQTile, r1 - a0));
      t.qtiles.insert(t.qtiles.end(), {int32_t(a0), n, int32_t(kv_off), int32_t(h + (a0 - r0))});
    }
    for (int64_t a0 = r0; a0 < r1; a0 += kAttnKTile) {
      const int32_t n = int32_t(std::min<int64_t>(kAttnKTile, r1 - a0));
      t.ktiles.insert(t.ktiles.end(), {int32_t(a0), n, int32_t(q_off + (a0 - r0)), int32_t(r1 - a0 + below)});
    }
  }
  // longest list first
  auto sort_tiles = [](std::vector<int32_t>& v, auto len) {
    const size_t n = v.size() / 4;
    std::vector<size_t> idx(n);
    std::iota(idx.begin(), idx.end(), size_t(0));
    std::stable_sort(idx.begin(), idx.end(), [&](size_t x, size_t y) { return len(&v[4 * x]) > len(&v[4 * y]); });
    std::vector<int32_t> out(v.size());
    for (size_t i = 0; i < n; ++i) std::copy(&v[4 * idx[i]], &v[4 * idx[i]] + 4, &out[4 * i]);
    v.swap(out);
  };
  sort_tiles(t.qtiles, [](const int32_t* e) { return int64_t(e[3]) + e[1]; });
  sort_tiles(t.ktiles, [](const int32_t* e) { return int64_t(e[3]); });
  return t;
}

}  // namespace harts
