// Host-side rollout-tree builder and minimum-call round planner (C++17).
//
// HARTS (arXiv 2608.28158): compact tokens and m: S -> C (close-reading blog,
// section 3.2); stable lexicographic sort + compressed trie, split cost = LCP
// of sorted neighbours (paperlayer summary, section 3); segment tree, packed
// chunkwise call model, T_pre/T_in recursion, top-down recovery, replay of
// [a(p), p) (blog, section 4.2; thelatestinai Figure 2); compact physical
// layout (blog, section 4.3); multiplicities q (blog, section 4.4).
#pragma once
#include <cstdint>
#include <stdexcept>
#include <string>
#include <vector>

#include "../desc.h"

namespace harts {

struct Error : std::runtime_error {
  int code;
  Error(int c, const std::string& m) : std::runtime_error(m), code(c) {}
};

// Compressed trie with node ids in DFS preorder (children by token id).
struct TreeHost {
  int64_t S = 0, C = 0;
  std::vector<int64_t> m_node;      // [S] semantic position -> trie node
  std::vector<int64_t> node_parent; // [C] (-1 under the empty prefix)
  std::vector<int32_t> node_depth;  // [C] absolute position
  std::vector<int32_t> node_nchild; // [C]
  // fork-free segments: consecutive node ranges [first, first + len)
  std::vector<int64_t> seg_first;
  std::vector<int32_t> seg_len;
  std::vector<int32_t> seg_parent;  // -1 for roots
  std::vector<int32_t> seg_child_off, seg_child;  // CSR, children in token order
  std::vector<int32_t> roots;       // root segments in token order
  int64_t n_forks = 0;
  int32_t start(int v) const { return node_depth[seg_first[v]]; }
  int32_t end(int v) const { return node_depth[seg_first[v]] + seg_len[v]; }
  int32_t nchild(int v) const { return seg_child_off[v + 1] - seg_child_off[v]; }
  const int32_t* children(int v) const { return seg_child.data() + seg_child_off[v]; }
};

TreeHost build_tree(const int32_t* tokens, const int64_t* offsets, int64_t n_traj);

struct SeqHost {
  int32_t round = 0;       // 1-based
  int32_t head = -1;       // head segment (-1 for varlen sequences)
  int64_t start = 0;       // a(s_head)
  int64_t row_begin = 0, row_end = 0;
  int64_t replay_off = 0;  // into PlanHost::replay_rows
  int32_t n_replay = 0;
  int32_t init = -1;       // slot / init-state index, -1 = zero
  int32_t final_idx = -1;
  int64_t emit_off = 0;
  int32_t n_emits = 0;
  int64_t vlen() const { return n_replay + (row_end - row_begin); }
};

struct RoundRange {
  int32_t seq0, seq1;       // global sequence range
  int32_t chunk0, chunk1;   // global chunk range
  int64_t vrow0, vrow1;     // global virtual-row range
  int64_t replay0, replay1; // global replay range
  int32_t max_chunks;       // longest sequence of the round, in chunks
};

struct PlanHost {
  bool varlen = false;
  int32_t B = 64;
  int64_t S = 0, C = 0;
  int32_t n_rounds = 0, min_calls = 0;
  int32_t n_slots = 0, n_boundaries = 0;
  std::vector<int64_t> m, node_to_row;
  std::vector<int32_t> q;
  std::vector<SeqHost> seqs;
  std::vector<int64_t> replay_rows;
  std::vector<int32_t> emit_boundary, emit_target;
  std::vector<int64_t> boundary_offsets;  // varlen plans
  // slot consumers (tree plans): CSR over slots of consumer sequence indices
  std::vector<int32_t> slot_cons_off, slot_cons;
  // device descriptors
  std::vector<int32_t> vrows;
  std::vector<SeqDesc> seq_desc;
  std::vector<ChunkDesc> chunk_desc;
  std::vector<RoundRange> rounds;
  // replay-gradient fixup: CSR over replayed compact rows
  std::vector<int32_t> fix_rows, fix_off, fix_idx;
  int64_t replay_total = 0;
  int32_t max_round_chunks = 0;
  int32_t max_round_seqs = 0;
};

PlanHost make_plan(const TreeHost& tree, int32_t B);
// Checks every device descriptor of a plan against the bounds the kernels index with (virtual
// rows inside [0, C); sequence and chunk ranges inside the virtual-row table; replay shorter
// than B; state indices inside the slot pool or the caller's state arrays; every handed-off
// state produced in an earlier round than each of its consumers; fixup and consumer lists in
// range).  Throws Error(HARTS_ERANGE or HARTS_EINVAL) naming the first violation.
void validate_plan(const PlanHost& p);
PlanHost make_varlen_plan(const int64_t* cu_seqlens, int64_t n_seq, int32_t B, const uint8_t* has_init,
                          bool emit_boundaries);

}  // namespace harts
