// Host-side rollout-tree builder and minimum-call round planner.
// See plan.hpp for the sources on the HARTS pages.
#include "plan.hpp"

#include <algorithm>
#include <cstring>
#include <numeric>
#include <unordered_map>

#include "../../../include/harts.h"

namespace harts {

// ---------------------------------------------------------------------------------------------
// Trie by stable lexicographic sort.  Trajectory x_i in sorted order shares its first
// LCP(x_{i-1}, x_i) nodes with its sorted predecessor (no earlier trajectory shares more,
// since LCP over a sorted range is the minimum of adjacent LCPs) and creates the rest.
// Nodes are numbered on creation, which visits the trie in DFS preorder with children in
// token order.
TreeHost build_tree(const int32_t* tokens, const int64_t* off, int64_t n) {
  if (n < 1) throw Error(HARTS_EINVAL, "n_traj must be >= 1");
  if (!tokens || !off) throw Error(HARTS_EINVAL, "tokens and traj_offsets must be non-NULL");
  if (off[0] != 0) throw Error(HARTS_EINVAL, "traj_offsets[0] must be 0");
  for (int64_t i = 0; i < n; ++i)
    if (off[i + 1] <= off[i]) throw Error(HARTS_EINVAL, "empty trajectory or decreasing offsets at " + std::to_string(i));
  TreeHost t;
  t.S = off[n];
  if (t.S >= (int64_t(1) << 31)) throw Error(HARTS_ERANGE, "more than 2^31 - 1 semantic positions");
  std::vector<int64_t> order(n);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
    return std::lexicographical_compare(tokens + off[a], tokens + off[a + 1], tokens + off[b], tokens + off[b + 1]);
  });
  t.m_node.resize(t.S);
  std::vector<int64_t> prev, cur;
  const int32_t* ptok = nullptr;
  int64_t plen = 0;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t x = order[i];
    const int32_t* tk = tokens + off[x];
    const int64_t L = off[x + 1] - off[x];
    int64_t l = 0;
    if (i > 0) {
      const int64_t lim = std::min(L, plen);
      while (l < lim && tk[l] == ptok[l]) ++l;
    }
    cur.resize(L);
    for (int64_t p = 0; p < l; ++p) cur[p] = prev[p];
    for (int64_t p = l; p < L; ++p) {
      const int64_t id = t.C++;
      const int64_t par = p == 0 ? -1 : cur[p - 1];
      t.node_parent.push_back(par);
      t.node_depth.push_back(int32_t(p));
      t.node_nchild.push_back(0);
      if (par >= 0) t.node_nchild[par]++;
      cur[p] = id;
    }
    std::memcpy(t.m_node.data() + off[x], cur.data(), sizeof(int64_t) * L);
    prev.swap(cur);
    ptok = tk;
    plen = L;
  }
  // fork-free segments: a node starts a segment unless its parent has exactly one child
  std::vector<int32_t> seg_of(t.C);
  std::vector<std::vector<int32_t>> kids;
  for (int64_t nd = 0; nd < t.C; ++nd) {
    const int64_t par = t.node_parent[nd];
    if (par < 0 || t.node_nchild[par] != 1) {
      const int32_t sid = int32_t(t.seg_first.size());
      t.seg_first.push_back(nd);
      t.seg_len.push_back(1);
      const int32_t ps = par < 0 ? -1 : seg_of[par];
      t.seg_parent.push_back(ps);
      kids.emplace_back();
      if (ps >= 0) kids[ps].push_back(sid);
      else t.roots.push_back(sid);
      seg_of[nd] = sid;
    } else {
      const int32_t sid = seg_of[par];
      t.seg_len[sid]++;
      seg_of[nd] = sid;
    }
  }
  t.seg_child_off.assign(1, 0);
  for (auto& k : kids) {
    t.seg_child.insert(t.seg_child.end(), k.begin(), k.end());
    t.seg_child_off.push_back(int32_t(t.seg_child.size()));
    if (k.size() >= 2) t.n_forks++;
  }
  return t;
}

// ---------------------------------------------------------------------------------------------
static void finish_descriptors(PlanHost& P) {
  const int32_t B = P.B;
  P.vrows.clear();
  P.seq_desc.clear();
  P.chunk_desc.clear();
  P.rounds.clear();
  std::vector<std::pair<int64_t, int64_t>> fix;  // (target row, global replay index)
  int64_t replay_g = 0;
  size_t si = 0;
  for (int32_t r = 1; r <= P.n_rounds; ++r) {
    RoundRange rr{};
    rr.seq0 = int32_t(si);
    rr.chunk0 = int32_t(P.chunk_desc.size());
    rr.vrow0 = int64_t(P.vrows.size());
    rr.replay0 = replay_g;
    rr.max_chunks = 0;
    for (; si < P.seqs.size() && P.seqs[si].round == r; ++si) {
      const SeqHost& s = P.seqs[si];
      SeqDesc d{};
      d.vbase = int32_t(P.vrows.size());
      d.vlen = int32_t(s.vlen());
      d.n_replay = s.n_replay;
      d.chunk_base = int32_t(P.chunk_desc.size()) - rr.chunk0;  // round-local
      d.n_chunks = (d.vlen + B - 1) / B;
      d.init = s.init;
      d.final_idx = s.final_idx;
      d.replay_base = int32_t(replay_g);
      for (int32_t i = 0; i < s.n_replay; ++i) {
        P.vrows.push_back(int32_t(P.replay_rows[s.replay_off + i]));
        fix.emplace_back(P.replay_rows[s.replay_off + i], replay_g + i);
      }
      for (int64_t row = s.row_begin; row < s.row_end; ++row) P.vrows.push_back(int32_t(row));
      std::vector<int32_t> emit_at(d.n_chunks + 1, -1);
      for (int32_t e = 0; e < s.n_emits; ++e) {
        const int32_t b = P.emit_boundary[s.emit_off + e];
        if (b < 1 || b > d.n_chunks) throw Error(HARTS_ERANGE, "emitted boundary outside its sequence");
        if (emit_at[b] >= 0) throw Error(HARTS_EINVAL, "two states emitted at one boundary");
        emit_at[b] = P.emit_target[s.emit_off + e];
      }
      for (int32_t c = 0; c < d.n_chunks; ++c) {
        ChunkDesc ch{};
        ch.seq = int32_t(si);
        ch.vbase = d.vbase + c * B;
        ch.len = std::min(B, d.vlen - c * B);
        ch.own_from = std::max(0, std::min(ch.len, s.n_replay - c * B));
        ch.cidx = c;
        ch.emit = emit_at[c + 1];
        ch.local = int32_t(P.chunk_desc.size()) - rr.chunk0;
        ch.replay_base = d.replay_base + c * B;
        P.chunk_desc.push_back(ch);
      }
      rr.max_chunks = std::max(rr.max_chunks, d.n_chunks);
      replay_g += s.n_replay;
      P.seq_desc.push_back(d);
    }
    rr.seq1 = int32_t(si);
    rr.chunk1 = int32_t(P.chunk_desc.size());
    rr.vrow1 = int64_t(P.vrows.size());
    rr.replay1 = replay_g;
    P.rounds.push_back(rr);
    P.max_round_chunks = std::max(P.max_round_chunks, rr.chunk1 - rr.chunk0);
    P.max_round_seqs = std::max(P.max_round_seqs, rr.seq1 - rr.seq0);
  }
  if (P.vrows.size() >= (size_t(1) << 31)) throw Error(HARTS_ERANGE, "plan too large for int32 descriptors");
  P.replay_total = replay_g;
  std::sort(fix.begin(), fix.end());
  P.fix_rows.clear();
  P.fix_off.assign(1, 0);
  P.fix_idx.clear();
  for (size_t i = 0; i < fix.size(); ++i) {
    if (i == 0 || fix[i].first != fix[i - 1].first) {
      if (i > 0) P.fix_off.push_back(int32_t(P.fix_idx.size()));
      P.fix_rows.push_back(int32_t(fix[i].first));
    }
    P.fix_idx.push_back(int32_t(fix[i].second));
  }
  if (!fix.empty()) P.fix_off.push_back(int32_t(P.fix_idx.size()));
}

// ---------------------------------------------------------------------------------------------
PlanHost make_plan(const TreeHost& t, int32_t B) {
  if (B != 16 && B != 32 && B != 64) throw Error(HARTS_EINVAL, "chunk_B must be 16, 32 or 64");
  const int32_t nseg = int32_t(t.seg_first.size());
  auto crosses = [&](int v) { return t.end(v) / B > t.start(v) / B; };
  // T_pre / T_in bottom-up: children have larger ids (preorder).  F uses the largest and
  // second-largest T_pre among the children, so each fork costs O(#children).
  std::vector<int32_t> Tpre(nseg), Tin(nseg), best(nseg, -1);
  for (int v = nseg - 1; v >= 0; --v) {
    const int nc = t.nchild(v);
    if (nc == 0) {
      Tpre[v] = Tin[v] = 1;
      continue;
    }
    const int32_t* ch = t.children(v);
    int32_t max1 = -1, max2 = -1, cnt1 = 0;
    for (int i = 0; i < nc; ++i) {
      const int32_t x = Tpre[ch[i]];
      if (x > max1) { max2 = max1; max1 = x; cnt1 = 1; }
      else if (x == max1) { cnt1++; }
      else if (x > max2) { max2 = x; }
    }
    int32_t F = INT32_MAX;
    for (int i = 0; i < nc; ++i) {
      const int32_t d = ch[i];
      const int32_t other = (Tpre[d] == max1 && cnt1 == 1) ? max2 : max1;
      const int32_t val = std::max(Tin[d], other < 0 ? Tin[d] : 1 + other);
      if (val < F) { F = val; best[v] = d; }
    }
    Tin[v] = F;
    Tpre[v] = crosses(v) ? F : max1;
  }
  PlanHost P;
  P.B = B;
  P.S = t.S;
  P.C = t.C;
  for (int32_t r : t.roots) P.min_calls = std::max(P.min_calls, Tpre[r]);
  // top-down recovery: every sequence in its earliest legal round
  std::vector<int32_t> seq_round(nseg, 0), cont(nseg, -1);
  std::vector<char> ready(nseg, 0);
  std::vector<int32_t> chain_head(nseg, -1);
  for (int32_t r : t.roots) { ready[r] = 1; chain_head[r] = r; seq_round[r] = 1; }
  for (int v = 0; v < nseg; ++v) {
    const int nc = t.nchild(v);
    if (nc == 0) continue;
    const int32_t* ch = t.children(v);
    const int32_t h = chain_head[v];
    int32_t d;
    bool d_ready;
    int32_t side_round;
    if (ready[v] && !crosses(v)) {
      d = ch[0];
      d_ready = true;
      side_round = seq_round[h];
    } else {
      d = best[v];
      d_ready = false;
      side_round = seq_round[h] + 1;
    }
    cont[v] = d;
    for (int i = 0; i < nc; ++i) {
      const int32_t c = ch[i];
      if (c == d) {
        ready[c] = d_ready;
        chain_head[c] = h;
      } else {
        ready[c] = 1;
        chain_head[c] = c;
        seq_round[c] = side_round;
      }
    }
  }
  std::vector<int32_t> heads;
  for (int v = 0; v < nseg; ++v)
    if (chain_head[v] == v) heads.push_back(v);
  std::stable_sort(heads.begin(), heads.end(), [&](int a, int b) { return seq_round[a] < seq_round[b]; });
  P.n_rounds = heads.empty() ? 0 : seq_round[heads.back()];
  // compact rows: round-major, sequence order, path order
  P.node_to_row.assign(t.C, -1);
  std::vector<int32_t> row_owner(t.C);
  int64_t row = 0;
  for (size_t i = 0; i < heads.size(); ++i) {
    SeqHost s;
    s.head = heads[i];
    s.round = seq_round[s.head];
    s.start = int64_t(B) * (t.start(s.head) / B);
    s.row_begin = row;
    for (int32_t v = s.head; v >= 0; v = cont[v])
      for (int32_t k = 0; k < t.seg_len[v]; ++k) {
        P.node_to_row[t.seg_first[v] + k] = row;
        row_owner[row] = int32_t(i);
        ++row;
      }
    s.row_end = row;
    P.seqs.push_back(s);
  }
  if (row != t.C) throw Error(HARTS_EINVAL, "internal: compact layout does not cover the trie");
  P.m.resize(t.S);
  P.q.assign(t.C, 0);
  for (int64_t s = 0; s < t.S; ++s) {
    P.m[s] = P.node_to_row[t.m_node[s]];
    P.q[P.m[s]]++;
  }
  // replay rows and slots (first-use order, keyed by the row before the anchor)
  std::unordered_map<int64_t, int32_t> slot_of_row;
  std::vector<std::vector<std::pair<int32_t, int32_t>>> emits(P.seqs.size());
  std::vector<std::vector<int32_t>> consumers;
  for (size_t i = 0; i < P.seqs.size(); ++i) {
    SeqHost& s = P.seqs[i];
    const int32_t sh = t.start(s.head);
    s.n_replay = int32_t(sh - s.start);
    s.replay_off = int64_t(P.replay_rows.size());
    int64_t nd = t.node_parent[t.seg_first[s.head]];
    std::vector<int64_t> rev;
    for (int32_t k = 0; k < s.n_replay; ++k) {
      rev.push_back(P.node_to_row[nd]);
      nd = t.node_parent[nd];
    }
    P.replay_rows.insert(P.replay_rows.end(), rev.rbegin(), rev.rend());
    if (s.start > 0) {
      const int64_t key = P.node_to_row[nd];
      auto it = slot_of_row.find(key);
      int32_t sl;
      if (it == slot_of_row.end()) {
        sl = int32_t(consumers.size());
        slot_of_row.emplace(key, sl);
        consumers.emplace_back();
        const int32_t prod = row_owner[key];
        const int64_t b = s.start - P.seqs[prod].start;
        if (b <= 0 || b % B) throw Error(HARTS_EINVAL, "internal: slot boundary not on a chunk boundary");
        emits[prod].emplace_back(int32_t(b / B), sl);
      } else {
        sl = it->second;
      }
      consumers[sl].push_back(int32_t(i));
      s.init = sl;
    }
  }
  P.n_slots = int32_t(consumers.size());
  for (size_t i = 0; i < P.seqs.size(); ++i) {
    std::sort(emits[i].begin(), emits[i].end());
    P.seqs[i].emit_off = int64_t(P.emit_boundary.size());
    P.seqs[i].n_emits = int32_t(emits[i].size());
    for (auto& e : emits[i]) {
      P.emit_boundary.push_back(e.first);
      P.emit_target.push_back(e.second);
    }
  }
  P.slot_cons_off.assign(1, 0);
  for (auto& c : consumers) {
    P.slot_cons.insert(P.slot_cons.end(), c.begin(), c.end());
    P.slot_cons_off.push_back(int32_t(P.slot_cons.size()));
  }
  finish_descriptors(P);
  return P;
}

// ---------------------------------------------------------------------------------------------
void validate_plan(const PlanHost& P) {
  auto bad = [](int code, const std::string& what) { throw Error(code, "plan descriptor check: " + what); };
  const int64_t nv = int64_t(P.vrows.size()), ns = int64_t(P.seq_desc.size()), nc = int64_t(P.chunk_desc.size());
  const int32_t B = P.B;
  if (B != 16 && B != 32 && B != 64) bad(HARTS_EINVAL, "chunk_B " + std::to_string(B));
  if (ns != int64_t(P.seqs.size())) bad(HARTS_EINVAL, "sequence tables disagree");
  for (int64_t i = 0; i < nv; ++i)
    if (P.vrows[i] < 0 || P.vrows[i] >= P.C) bad(HARTS_ERANGE, "virtual row " + std::to_string(i) + " outside [0, C)");
  // state indices: tree plans read and write the slot pool; varlen plans read init_states and
  // write final_states per sequence and boundary states in [0, n_boundaries)
  const int64_t n_init = P.varlen ? ns : P.n_slots, n_emit = P.varlen ? P.n_boundaries : P.n_slots;
  std::vector<int32_t> produced_in(size_t(std::max<int64_t>(n_emit, 0)), -1);
  if (int64_t(P.rounds.size()) != P.n_rounds) bad(HARTS_EINVAL, "round count");
  int32_t seq_expect = 0, chunk_expect = 0;
  for (int32_t r = 0; r < P.n_rounds; ++r) {
    const RoundRange& rr = P.rounds[size_t(r)];
    if (rr.seq0 != seq_expect || rr.seq1 < rr.seq0 || rr.seq1 > ns || rr.chunk0 != chunk_expect || rr.chunk1 < rr.chunk0 ||
        rr.chunk1 > nc || rr.vrow0 < 0 || rr.vrow1 < rr.vrow0 || rr.vrow1 > nv)
      bad(HARTS_ERANGE, "round " + std::to_string(r + 1) + " ranges");
    seq_expect = rr.seq1;
    chunk_expect = rr.chunk1;
    for (int32_t q = rr.seq0; q < rr.seq1; ++q) {
      const SeqDesc& d = P.seq_desc[size_t(q)];
      const std::string who = "sequence " + std::to_string(q);
      if (d.vbase < rr.vrow0 || d.vlen < 1 || int64_t(d.vbase) + d.vlen > rr.vrow1) bad(HARTS_ERANGE, who + " rows");
      if (d.n_replay < 0 || d.n_replay >= B || d.n_replay > d.vlen) bad(HARTS_ERANGE, who + " replay length");
      if (d.n_chunks != (d.vlen + B - 1) / B || d.chunk_base < 0 || rr.chunk0 + d.chunk_base + d.n_chunks > rr.chunk1)
        bad(HARTS_ERANGE, who + " chunks");
      if (d.init < -1 || d.init >= n_init) bad(HARTS_ERANGE, who + " initial state index");
      if (d.final_idx < -1 || d.final_idx >= (P.varlen ? ns : 0)) bad(HARTS_ERANGE, who + " final state index");
      if (!P.varlen && d.init >= 0 && (produced_in[size_t(d.init)] < 0 || produced_in[size_t(d.init)] >= r))
        bad(HARTS_EINVAL, who + " consumes slot " + std::to_string(d.init) + " before a round produced it");
      for (int32_t c = 0; c < d.n_chunks; ++c) {
        const ChunkDesc& ch = P.chunk_desc[size_t(rr.chunk0 + d.chunk_base + c)];
        const std::string cw = who + " chunk " + std::to_string(c);
        if (ch.seq != q || ch.cidx != c || ch.local != d.chunk_base + c || ch.vbase != d.vbase + c * B ||
            ch.len != std::min(B, d.vlen - c * B) || ch.own_from < 0 || ch.own_from > ch.len)
          bad(HARTS_ERANGE, cw + " layout");
        if (ch.emit < -1 || ch.emit >= n_emit) bad(HARTS_ERANGE, cw + " emitted state index");
        if (ch.emit >= 0) {
          if (produced_in[size_t(ch.emit)] >= 0) bad(HARTS_EINVAL, cw + " writes state " + std::to_string(ch.emit) + " twice");
          produced_in[size_t(ch.emit)] = r;
        }
        if (ch.own_from > 0 && (ch.replay_base < 0 || ch.replay_base + ch.own_from > P.replay_total))
          bad(HARTS_ERANGE, cw + " replay index");
      }
    }
  }
  if (seq_expect != ns || chunk_expect != nc) bad(HARTS_ERANGE, "rounds do not cover every sequence and chunk");
  if (!P.varlen) {
    if (int64_t(P.slot_cons_off.size()) != int64_t(P.n_slots) + 1) bad(HARTS_EINVAL, "slot consumer offsets");
    for (size_t i = 0; i < P.slot_cons.size(); ++i)
      if (P.slot_cons[i] < 0 || P.slot_cons[i] >= ns) bad(HARTS_ERANGE, "slot consumer index");
    for (int32_t sl = 0; sl < P.n_slots; ++sl)
      if (P.slot_cons_off[size_t(sl) + 1] < P.slot_cons_off[size_t(sl)] ||
          P.slot_cons_off[size_t(sl) + 1] > int64_t(P.slot_cons.size()))
        bad(HARTS_ERANGE, "slot consumer offsets");
  }
  if (P.fix_off.size() != P.fix_rows.size() + 1 || P.fix_off.back() != int32_t(P.fix_idx.size()))
    bad(HARTS_EINVAL, "replay fixup offsets");
  for (int32_t row : P.fix_rows)
    if (row < 0 || row >= P.C) bad(HARTS_ERANGE, "replay fixup row outside [0, C)");
  for (int32_t ix : P.fix_idx)
    if (ix < 0 || ix >= P.replay_total) bad(HARTS_ERANGE, "replay fixup index");
}

PlanHost make_varlen_plan(const int64_t* cu, int64_t n, int32_t B, const uint8_t* has_init, bool emit_boundaries) {
  if (B != 16 && B != 32 && B != 64) throw Error(HARTS_EINVAL, "chunk_B must be 16, 32 or 64");
  if (n < 1 || !cu) throw Error(HARTS_EINVAL, "need at least one sequence");
  if (cu[0] != 0) throw Error(HARTS_EINVAL, "cu_seqlens[0] must be 0");
  for (int64_t i = 0; i < n; ++i)
    if (cu[i + 1] <= cu[i]) throw Error(HARTS_EINVAL, "empty sequence or decreasing cu_seqlens at " + std::to_string(i));
  if (cu[n] >= (int64_t(1) << 31)) throw Error(HARTS_ERANGE, "more than 2^31 - 1 tokens");
  PlanHost P;
  P.varlen = true;
  P.B = B;
  P.S = P.C = cu[n];
  P.n_rounds = 1;
  P.min_calls = 1;
  P.m.resize(P.S);
  std::iota(P.m.begin(), P.m.end(), 0);
  P.node_to_row = P.m;
  P.q.assign(P.C, 1);
  P.boundary_offsets.assign(1, 0);
  int32_t nb = 0;
  for (int64_t i = 0; i < n; ++i) {
    SeqHost s;
    s.round = 1;
    s.start = 0;
    s.row_begin = cu[i];
    s.row_end = cu[i + 1];
    s.init = (has_init && has_init[i]) ? int32_t(i) : -1;
    s.final_idx = int32_t(i);
    s.emit_off = int64_t(P.emit_boundary.size());
    if (emit_boundaries) {
      const int64_t L = cu[i + 1] - cu[i];
      for (int64_t b = 1; b <= L / B; ++b) {
        P.emit_boundary.push_back(int32_t(b));
        P.emit_target.push_back(nb++);
      }
    }
    s.n_emits = int32_t(P.emit_boundary.size() - s.emit_off);
    P.boundary_offsets.push_back(nb);
    P.seqs.push_back(s);
  }
  P.n_boundaries = nb;
  finish_descriptors(P);
  return P;
}

}  // namespace harts
