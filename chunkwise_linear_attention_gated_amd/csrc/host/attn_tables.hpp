// Host tables of tree softmax attention over compact rows.
//
// A compact row attends over the rows of its own root-to-row path (the
// branch's ancestor prefix plus its own earlier rows, bottom-right causal).
// The rows are cut into fork-free segments: maximal runs r0, r0+1, .., r1-1 in
// which every row is the only child of the row before it.  Each segment s
// with h ancestor rows gets two row lists:
//   kv list: its h ancestor rows (root first), then its own rows;
//   q list:  its own rows, then the rows of every segment below it.
// and is cut into query tiles of kAttnQTile rows and key tiles of kAttnKTile rows:
//   query tile {row0, n, off, base}: rows row0 .. row0+n-1; keys are
//     kv_list[off + v] for v < base + n, and query row0 + i sees key v iff
//     v <= base + i;
//   key tile {row0, n, off, nq}: keys row0 .. row0+n-1; queries are
//     q_list[off + u] for u < nq, and key row0 + j is seen by query u iff u >= j.
// Tiles are sorted by the length of their list, longest first.
#pragma once
#include <cstdint>
#include <vector>

namespace harts {

constexpr int kAttnQTile = 128;
constexpr int kAttnKTile = 128;

struct AttnTables {
  int64_t C = 0;
  int64_t n_segments = 0;
  int64_t pairs = 0;              // sum over rows of (path length): visible (query, key) pairs
  int32_t max_depth = 0;          // longest path
  std::vector<int32_t> pos;       // [C] position of the row on its trajectories (path length - 1)
  std::vector<int32_t> qtiles;    // [n][4]
  std::vector<int32_t> kv_list;
  std::vector<int32_t> ktiles;    // [n][4]
  std::vector<int32_t> q_list;
};

// m: semantic -> compact [traj_offsets[n_traj]]; throws harts::Error (EINVAL) if m is not the
// map of a prefix tree over rows 0..C-1 or a row is on no trajectory, ERANGE if a list
// outgrows int32 offsets.
AttnTables build_attn_tables(const int64_t* m, const int64_t* traj_offsets, int64_t n_traj, int64_t C);

}  // namespace harts
