// C ABI of the tree-packed chunkwise gated-delta path (declared in include/harts.h).
// Host calls wrap the C++ planner; device calls upload descriptors and enqueue
// the per-round HIP kernels on the caller's stream.  No exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "../../include/harts.h"
#include "host/attn_tables.hpp"
#include "host/plan.hpp"
#include "kernels/launch.h"

using harts::Error;

struct harts_attn_tables {
  harts::AttnTables t;
};
struct harts_tree {
  harts::TreeHost t;
};
struct harts_plan {
  harts::PlanHost p;
  // per-round host views (harts_plan_round), built on first use
  struct RoundStore {
    std::vector<int64_t> row_start, row_end, abs_start, replay_off, replay_rows, emit_off;
    std::vector<int32_t> init_slot, emit_chunk, emit_slot;
  };
  mutable std::mutex views_mu;
  mutable std::vector<RoundStore> views;
};
struct harts_dev_plan {
  harts::PlanHost p;
  harts::KdaDims dims{};
  int32_t* vrows = nullptr;
  harts::SeqDesc* seqs = nullptr;
  harts::ChunkDesc* chunks = nullptr;
  int32_t* crows = nullptr;
  int32_t* cons_off = nullptr;
  int32_t* cons = nullptr;
  int32_t* fix_rows = nullptr;
  int32_t* fix_off = nullptr;
  int32_t* fix_idx = nullptr;
  int32_t* rslots = nullptr;           // slots produced per round (concatenated)
  int32_t* units = nullptr;            // per round, (sequence, head) launch order of the serial passes
  std::vector<int32_t> rslot_off;      // [n_rounds + 1] offsets into rslots
  // workspace layout (byte offsets)
  size_t off_W = 0, off_Mf = 0, off_UpT = 0, off_KhT = 0, off_Qt = 0, off_Mm = 0, off_El = 0, off_Qe = 0, off_h = 0, off_dh = 0, off_hc = 0, off_dhc = 0, off_WT = 0, off_Kh = 0, off_sink = 0,
         off_dinit = 0, off_rg = 0, off_Tm = 0, off_Xm = 0, off_Am = 0, off_dslot = 0;
  size_t ws_fwd = 0, ws_bwd = 0;
  size_t off_ctr = 0;
  // the workspace whose kept operands and chunk-start states the last forward left (keep = 1);
  // a forward without keep on that workspace clears it (harts_kda_bwd with keep = 1 checks it)
  mutable std::mutex kept_mu;
  mutable const void* kept_ws = nullptr;
};

namespace {
thread_local std::string g_err;

// ---- kernel timing (harts_profile_*): HIP event pairs per launch, on the launch stream
struct ProfRec {
  const char* name;
  hipEvent_t e0, e1;
  int64_t units;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof;

struct ProfScope {
  ProfRec rec{};
  hipStream_t s;
  bool on;
  ProfScope(const char* name, hipStream_t st, int64_t units) : s(st) {
    {
      std::lock_guard<std::mutex> lk(g_prof_mu);
      on = g_prof_on;
    }
    if (!on) return;
    rec.name = name;
    rec.units = units;
    if (hipEventCreate(&rec.e0) != hipSuccess || hipEventCreate(&rec.e1) != hipSuccess) {
      on = false;
      return;
    }
    (void)hipEventRecord(rec.e0, s);
  }
  ~ProfScope() {
    if (!on) return;
    (void)hipEventRecord(rec.e1, s);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof.push_back(rec);
  }
};

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

template <typename F>
int guarded(F&& f) {
  try {
    f();
    return HARTS_OK;
  } catch (const Error& e) {
    return fail(e.code, e.what());
  } catch (const std::bad_alloc&) {
    return fail(HARTS_ENOMEM, "host allocation failed");
  } catch (const std::exception& e) {
    return fail(HARTS_EINVAL, e.what());
  }
}

void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) throw Error(HARTS_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

template <typename T>
T* upload(const std::vector<T>& v, hipStream_t s) {
  if (v.empty()) return nullptr;
  T* p = nullptr;
  hip_check(hipMalloc(reinterpret_cast<void**>(&p), v.size() * sizeof(T)), "hipMalloc");
  const hipError_t e = hipMemcpyAsync(p, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice, s);
  if (e != hipSuccess) {
    (void)hipFree(p);
    hip_check(e, "hipMemcpyAsync");
  }
  return p;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Launch order of a round's (sequence, head) pairs in the serial passes.  Workgroup b runs on
// XCD b mod 8, and the kernels map the pairs to contiguous eighths of the grid, one eighth per
// XCD, so that the workgroups of one pair share an L2.  Each chain takes its sequence's chunk
// count in steps: the pairs are dealt to the eighths longest first, each to the least loaded
// eighth with room, and each eighth lists its pairs longest first, so that every XCD starts its
// long chains early and the XCDs carry equal work.  Returns u = s * H + h per launch slot.
std::vector<int32_t> slab_unit_order(const std::vector<int32_t>& chunks, int32_t H) {
  const size_t n = chunks.size() * size_t(H);
  std::vector<int32_t> id(n);
  for (size_t u = 0; u < n; ++u) id[u] = int32_t(u);
  if (n % 8) return id;  // the eighths would split pairs: natural order
  auto wt = [&](int32_t u) { return int64_t(chunks[size_t(u / H)]) + 1; };
  std::stable_sort(id.begin(), id.end(), [&](int32_t x, int32_t y) { return wt(x) > wt(y); });
  const size_t cap = n / 8;
  std::vector<std::vector<int32_t>> bin(8);
  std::vector<int64_t> load(8, 0);
  for (int32_t u : id) {
    int best = -1;
    for (int x = 0; x < 8; ++x)
      if (bin[size_t(x)].size() < cap && (best < 0 || load[size_t(x)] < load[size_t(best)])) best = x;
    bin[size_t(best)].push_back(u);
    load[size_t(best)] += wt(u);
  }
  std::vector<int32_t> out;
  out.reserve(n);
  for (const std::vector<int32_t>& b : bin) out.insert(out.end(), b.begin(), b.end());
  return out;
}

// Write-only region of the workspace that masked-off lanes store into, so that a
// kernel's stores are unconditional (see RoundArgs::sink).
constexpr size_t kSinkBytes = 64 * 1024;

void free_dev(harts_dev_plan* d) {
  void* ptrs[] = {d->vrows, d->seqs, d->chunks, d->crows, d->cons_off, d->cons, d->fix_rows, d->fix_off, d->fix_idx,
                  d->rslots, d->units};
  for (void* p : ptrs)
    if (p) (void)hipFree(p);
}

// Auxiliary streams of the current device, created once at the default priority and kept
// for the life of the process; work is forked onto them from the caller's stream and joined
// back with events, so every entry point still only enqueues on the caller's stream.
hipStream_t aux_stream(int i) {
  static std::mutex mu;
  static std::map<int, std::pair<hipStream_t, hipStream_t>> streams;
  int dev = 0;
  hip_check(hipGetDevice(&dev), "hipGetDevice");
  std::lock_guard<std::mutex> lk(mu);
  auto it = streams.find(dev);
  if (it == streams.end()) {
    hipStream_t a = nullptr, b = nullptr;
    hip_check(hipStreamCreateWithFlags(&a, hipStreamNonBlocking), "hipStreamCreateWithFlags");
    hip_check(hipStreamCreateWithFlags(&b, hipStreamNonBlocking), "hipStreamCreateWithFlags");
    it = streams.emplace(dev, std::make_pair(a, b)).first;
  }
  return i == 0 ? it->second.first : it->second.second;
}

// Events recorded while enqueueing one call; released when the call returns (a recorded
// event's resources outlive it until the device reaches it).
struct Events {
  std::vector<hipEvent_t> ev;
  hipEvent_t record(hipStream_t s) {
    hipEvent_t e = nullptr;
    hip_check(hipEventCreateWithFlags(&e, hipEventDisableTiming), "hipEventCreateWithFlags");
    ev.push_back(e);
    hip_check(hipEventRecord(e, s), "hipEventRecord");
    return e;
  }
  ~Events() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  }
};

// stream `to` continues after the work enqueued so far on `from`
void fork(hipStream_t from, hipStream_t to, Events& ev) {
  hip_check(hipStreamWaitEvent(to, ev.record(from), 0), "hipStreamWaitEvent");
}

harts::RoundArgs round_args(const harts_dev_plan* d, const harts_kda_io* io, int r, char* ws) {
  const harts::RoundRange& rr = d->p.rounds[r];
  harts::RoundArgs a{};
  a.vrows = d->vrows;
  a.seqs = d->seqs + rr.seq0;
  a.chunks = d->chunks + rr.chunk0;
  a.crows = d->crows + size_t(rr.chunk0) * d->p.B;
  a.nseq = rr.seq1 - rr.seq0;
  a.nchunk = rr.chunk1 - rr.chunk0;
  a.seq0 = rr.seq0;
  a.units = d->units + size_t(rr.seq0) * size_t(d->dims.H);
  a.q = io->q;
  a.k = io->k;
  a.v = io->v;
  a.g = io->g;
  a.beta = io->beta;
  if (d->p.varlen) {
    a.init_pool = io->init_states;
    a.emit_pool = io->states;
    a.final_pool = io->final_states;
  } else {
    a.init_pool = io->states;
    a.emit_pool = io->states;
    a.final_pool = nullptr;
  }
  // every per-chunk workspace array holds all rounds, so rounds may run concurrently
  const size_t H = size_t(d->dims.H), BT = size_t(d->p.B), dk = size_t(d->dims.D), dv = size_t(d->dims.DV);
  const size_t es = d->dims.dtype == HARTS_DTYPE_BF16 ? 2 : 4, item0 = size_t(rr.chunk0) * H;
  auto at = [&](size_t off, size_t elems, size_t esz) { return ws + off + item0 * elems * esz; };
  a.ws.W = at(d->off_W, BT * dk, es);
  a.ws.UpT = at(d->off_UpT, dv * BT, es);
  a.ws.KhT = at(d->off_KhT, dk * BT, es);
  a.ws.Qt = at(d->off_Qt, BT * dk, es);
  a.ws.Mm = at(d->off_Mm, BT * BT, es);
  a.ws.El = reinterpret_cast<float*>(at(d->off_El, dk, 4));
  a.sink = ws + d->off_sink;
  const bool f32 = d->dims.dtype == HARTS_DTYPE_FP32;
  a.ws.QeffT = f32 ? at(d->off_Qe, dk * BT, es) : nullptr;
  a.ws.WT = f32 ? at(d->off_WT, dk * BT, es) : nullptr;
  a.ws.Kh = f32 ? at(d->off_Kh, BT * dk, es) : nullptr;
  a.ws.Tm = at(d->off_Tm, BT * BT, es);
  a.ws.Xm = at(d->off_Xm, BT * BT, es);
  a.ws.Am = at(d->off_Am, BT * BT, es);
  a.ws.Mf = at(d->off_Mf, BT * BT, es);
  a.h = at(d->off_h, dv * dk, es);
  a.hc = d->dims.dtype == HARTS_DTYPE_FP32 ? at(d->off_hc, dv * dk, es) : nullptr;
  a.ctr = nullptr;
  a.zero = nullptr;
  a.nzero = 0;
  return a;
}

void check_io(const harts_dev_plan* d, const harts_kda_io* io, bool bwd) {
  if (!io) throw Error(HARTS_EINVAL, "io is NULL");
  if (!io->q || !io->k || !io->v || !io->g || !io->beta) throw Error(HARTS_EINVAL, "q, k, v, g and beta are required");
  if (!bwd && !io->o) throw Error(HARTS_EINVAL, "o is required");
  if (io->keep != 0 && io->keep != 1) throw Error(HARTS_EINVAL, "keep must be 0 or 1");
  if (!io->workspace || io->workspace_bytes < (bwd || io->keep ? d->ws_bwd : d->ws_fwd))
    throw Error(HARTS_EINVAL, "workspace missing or smaller than harts_kda_workspace_size()");
  if (!d->p.varlen && d->p.n_slots > 0 && !io->states) throw Error(HARTS_EINVAL, "states (slot pool) is required");
  if (d->p.varlen) {
    bool any_init = false;
    for (auto& s : d->p.seqs) any_init |= s.init >= 0;
    if (any_init && !io->init_states) throw Error(HARTS_EINVAL, "init_states is required (plan has initial states)");
    if (d->p.n_boundaries > 0 && !io->states) throw Error(HARTS_EINVAL, "states is required (plan emits boundaries)");
  }
}
}  // namespace

extern "C" {

const char* harts_last_error(void) { return g_err.c_str(); }
const char* harts_version(void) { return "harts-mi355x 0.1 (gfx950)"; }

int harts_tree_build(const int32_t* tokens, const int64_t* traj_offsets, int64_t n_traj, harts_tree** out) {
  return guarded([&] {
    if (!out) throw Error(HARTS_EINVAL, "out is NULL");
    *out = nullptr;
    auto* t = new harts_tree{harts::build_tree(tokens, traj_offsets, n_traj)};
    *out = t;
  });
}

int harts_tree_stats(const harts_tree* tree, int64_t* S, int64_t* C, int64_t* n_segments, int64_t* n_forks) {
  return guarded([&] {
    if (!tree) throw Error(HARTS_EINVAL, "tree is NULL");
    if (S) *S = tree->t.S;
    if (C) *C = tree->t.C;
    if (n_segments) *n_segments = int64_t(tree->t.seg_first.size());
    if (n_forks) *n_forks = tree->t.n_forks;
  });
}

void harts_tree_free(harts_tree* tree) { delete tree; }

int harts_plan_create(const harts_tree* tree, int32_t chunk_B, harts_plan** out) {
  return guarded([&] {
    if (!tree || !out) throw Error(HARTS_EINVAL, "tree and out must be non-NULL");
    *out = nullptr;
    *out = new harts_plan{harts::make_plan(tree->t, chunk_B)};
  });
}

int harts_plan_create_varlen(const int64_t* cu_seqlens, int64_t n_seq, int32_t chunk_B, const uint8_t* has_init,
                             int32_t emit_boundaries, harts_plan** out) {
  return guarded([&] {
    if (!out) throw Error(HARTS_EINVAL, "out is NULL");
    *out = nullptr;
    *out = new harts_plan{harts::make_varlen_plan(cu_seqlens, n_seq, chunk_B, has_init, emit_boundaries != 0)};
  });
}

int harts_plan_info(const harts_plan* plan, harts_plan_info_t* o) {
  return guarded([&] {
    if (!plan || !o) throw Error(HARTS_EINVAL, "plan and out must be non-NULL");
    const harts::PlanHost& p = plan->p;
    o->S = p.S;
    o->C = p.C;
    o->chunk_B = p.B;
    o->n_rounds = p.n_rounds;
    o->min_calls = p.min_calls;
    o->n_sequences = int32_t(p.seqs.size());
    o->n_slots = p.n_slots;
    o->n_boundaries = p.n_boundaries;
    o->replay_total = p.replay_total;
    o->n_chunks = int64_t(p.chunk_desc.size());
    o->n_vrows = int64_t(p.vrows.size());
  });
}

int harts_plan_maps(const harts_plan* plan, int64_t* m, int32_t* q, int64_t* node_to_row) {
  return guarded([&] {
    if (!plan) throw Error(HARTS_EINVAL, "plan is NULL");
    const harts::PlanHost& p = plan->p;
    if (m) std::memcpy(m, p.m.data(), p.m.size() * sizeof(int64_t));
    if (q) std::memcpy(q, p.q.data(), p.q.size() * sizeof(int32_t));
    if (node_to_row) std::memcpy(node_to_row, p.node_to_row.data(), p.node_to_row.size() * sizeof(int64_t));
  });
}

int harts_plan_sequences(const harts_plan* plan, harts_seq_view* seqs) {
  return guarded([&] {
    if (!plan || !seqs) throw Error(HARTS_EINVAL, "plan and seqs must be non-NULL");
    for (size_t i = 0; i < plan->p.seqs.size(); ++i) {
      const harts::SeqHost& s = plan->p.seqs[i];
      harts_seq_view& v = seqs[i];
      v.round = s.round;
      v.init_slot = s.init;
      v.start = s.start;
      v.row_begin = s.row_begin;
      v.row_end = s.row_end;
      v.replay_off = s.replay_off;
      v.n_replay = s.n_replay;
      v.n_emits = s.n_emits;
      v.emit_off = s.emit_off;
    }
  });
}

int harts_plan_replay_rows(const harts_plan* plan, int64_t* rows) {
  return guarded([&] {
    if (!plan || (!rows && !plan->p.replay_rows.empty())) throw Error(HARTS_EINVAL, "plan and rows must be non-NULL");
    if (!plan->p.replay_rows.empty())
      std::memcpy(rows, plan->p.replay_rows.data(), plan->p.replay_rows.size() * sizeof(int64_t));
  });
}

int harts_plan_emits(const harts_plan* plan, int32_t* boundary, int32_t* target) {
  return guarded([&] {
    if (!plan) throw Error(HARTS_EINVAL, "plan is NULL");
    const size_t n = plan->p.emit_boundary.size();
    if (n && boundary) std::memcpy(boundary, plan->p.emit_boundary.data(), n * sizeof(int32_t));
    if (n && target) std::memcpy(target, plan->p.emit_target.data(), n * sizeof(int32_t));
  });
}

int harts_plan_boundary_offsets(const harts_plan* plan, int64_t* offsets) {
  return guarded([&] {
    if (!plan || !offsets) throw Error(HARTS_EINVAL, "plan and offsets must be non-NULL");
    if (!plan->p.varlen) throw Error(HARTS_ESTATE, "boundary offsets exist only for varlen plans");
    std::memcpy(offsets, plan->p.boundary_offsets.data(), plan->p.boundary_offsets.size() * sizeof(int64_t));
  });
}

int harts_plan_round(const harts_plan* plan, int32_t r, harts_round_view* out) {
  return guarded([&] {
    if (!plan || !out) throw Error(HARTS_EINVAL, "plan and out must be non-NULL");
    if (r < 0 || r >= plan->p.n_rounds)
      throw Error(HARTS_EINVAL, "round " + std::to_string(r) + " outside [0, " + std::to_string(plan->p.n_rounds) + ")");
    std::lock_guard<std::mutex> lk(plan->views_mu);
    if (plan->views.empty()) {
      std::vector<harts_plan::RoundStore> v(size_t(plan->p.n_rounds));
      for (auto& st : v) {
        st.replay_off.push_back(0);
        st.emit_off.push_back(0);
      }
      for (const harts::SeqHost& q : plan->p.seqs) {
        harts_plan::RoundStore& st = v[size_t(q.round - 1)];
        st.row_start.push_back(q.row_begin);
        st.row_end.push_back(q.row_end);
        st.abs_start.push_back(q.start);
        st.init_slot.push_back(q.init);
        for (int32_t i = 0; i < q.n_replay; ++i) st.replay_rows.push_back(plan->p.replay_rows[size_t(q.replay_off + i)]);
        st.replay_off.push_back(int64_t(st.replay_rows.size()));
        for (int32_t i = 0; i < q.n_emits; ++i) {
          st.emit_chunk.push_back(plan->p.emit_boundary[size_t(q.emit_off + i)]);
          st.emit_slot.push_back(plan->p.emit_target[size_t(q.emit_off + i)]);
        }
        st.emit_off.push_back(int64_t(st.emit_chunk.size()));
      }
      plan->views = std::move(v);
    }
    const harts_plan::RoundStore& st = plan->views[size_t(r)];
    out->n_seq = int32_t(st.row_start.size());
    out->row_start = st.row_start.data();
    out->row_end = st.row_end.data();
    out->abs_start = st.abs_start.data();
    out->replay_off = st.replay_off.data();
    out->replay_rows = st.replay_rows.data();
    out->init_slot = st.init_slot.data();
    out->emit_off = st.emit_off.data();
    out->emit_chunk = st.emit_chunk.data();
    out->emit_slot = st.emit_slot.data();
  });
}

void harts_plan_free(harts_plan* plan) { delete plan; }

int harts_plan_upload(const harts_plan* plan, int32_t H, int32_t dk, int32_t dv, int32_t dtype, void* stream,
                      harts_dev_plan** out) {
  return guarded([&] {
    if (!plan || !out) throw Error(HARTS_EINVAL, "plan and out must be non-NULL");
    *out = nullptr;
    if (H < 1) throw Error(HARTS_EINVAL, "H must be >= 1");
    if (dtype != HARTS_DTYPE_BF16 && dtype != HARTS_DTYPE_FP32) throw Error(HARTS_EINVAL, "unknown dtype");
    harts::validate_plan(plan->p);  // every index the kernels use, before anything reaches the device
    harts::KdaDims dims{H, dk, dv, plan->p.B, dtype};
    if (!harts::kda_supported(dims))
      throw Error(HARTS_EINVAL, "unsupported (dtype, chunk_B, dk, dv) = (" + std::to_string(dtype) + ", " +
                                    std::to_string(plan->p.B) + ", " + std::to_string(dk) + ", " + std::to_string(dv) +
                                    ")");
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto* d = new harts_dev_plan();
    try {
      d->p = plan->p;
      d->dims = dims;
      d->vrows = upload(d->p.vrows, s);
      d->seqs = upload(d->p.seq_desc, s);
      d->chunks = upload(d->p.chunk_desc, s);
      {
        // padded per-chunk row table: lets the per-chunk kernels fetch a chunk's rows
        // without first reading its descriptor
        const size_t BTc = size_t(d->p.B);
        std::vector<int32_t> cr(d->p.chunk_desc.size() * BTc, -1);
        for (size_t c = 0; c < d->p.chunk_desc.size(); ++c) {
          const harts::ChunkDesc& cd = d->p.chunk_desc[c];
          for (int i = 0; i < cd.len; ++i) cr[c * BTc + i] = d->p.vrows[size_t(cd.vbase) + i];
        }
        d->crows = upload(cr, s);
        hip_check(hipStreamSynchronize(s), "hipStreamSynchronize");
      }
      d->cons_off = upload(d->p.slot_cons_off, s);
      d->cons = upload(d->p.slot_cons, s);
      d->fix_rows = upload(d->p.fix_rows, s);
      d->fix_off = upload(d->p.fix_off, s);
      d->fix_idx = upload(d->p.fix_idx, s);
      std::vector<int32_t> rsl;
      d->rslot_off.assign(1, 0);
      for (const harts::RoundRange& rr : d->p.rounds) {
        if (!d->p.varlen)
          for (int32_t c = rr.chunk0; c < rr.chunk1; ++c)
            if (d->p.chunk_desc[size_t(c)].emit >= 0) rsl.push_back(d->p.chunk_desc[size_t(c)].emit);
        d->rslot_off.push_back(int32_t(rsl.size()));
      }
      d->rslots = upload(rsl, s);
      std::vector<int32_t> units;
      for (const harts::RoundRange& rr : d->p.rounds) {
        std::vector<int32_t> w;
        for (int32_t q = rr.seq0; q < rr.seq1; ++q) w.push_back(d->p.seq_desc[size_t(q)].n_chunks);
        const std::vector<int32_t> u = slab_unit_order(w, H);
        units.insert(units.end(), u.begin(), u.end());
      }
      d->units = upload(units, s);
      // the host vectors must outlive the asynchronous copies
      hip_check(hipStreamSynchronize(s), "hipStreamSynchronize");
      const size_t es = dtype == HARTS_DTYPE_BF16 ? 2 : 4;
      // per-chunk arrays are sized for every chunk of the plan (rounds may run concurrently)
      const size_t MC = d->p.chunk_desc.size() * size_t(H), BT = size_t(d->p.B);
      size_t off = 0;
      auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
      };
      d->off_W = take(MC * BT * dk * es);
      d->off_UpT = take(MC * dv * BT * es);
      d->off_KhT = take(MC * dk * BT * es);
      d->off_Mm = take(MC * BT * BT * es);
      d->off_El = take(MC * dk * 4);
      d->off_sink = take(kSinkBytes);
      // item counters of the persistent per-chunk kernels: per round, forward preparation,
      // backward preparation and the gradient kernel; zeroed at the start of every call
      d->off_ctr = take(size_t(3) * d->p.rounds.size() * sizeof(int32_t));
      d->off_Qt = take(MC * BT * dk * es);
      d->off_Mf = take(MC * BT * BT * es);
      d->ws_fwd = off;
      // the backward arrays follow the forward's, so that a forward that keeps them for the
      // backward (harts_kda_io::keep) leaves its own outputs intact
      d->off_h = take(MC * dv * dk * es);
      d->off_dh = take(MC * dv * dk * es);
      // fp32 path only: channel-major copies of the chunk-start states and their gradients, and
      // the state-gradient operands Qeff^T, W^T, K^ (the bf16 gradient kernel transposes its state
      // slices in LDS, and the bf16 state-gradient pass reads the forward's operands transposed)
      if (dtype == HARTS_DTYPE_FP32) {
        d->off_hc = take(MC * dv * dk * es);
        d->off_dhc = take(MC * dv * dk * es);
        d->off_Qe = take(MC * dk * BT * es);
        d->off_WT = take(MC * dk * BT * es);
        d->off_Kh = take(MC * BT * dk * es);
      }
      d->off_dinit = take(size_t(d->p.seqs.size()) * H * dk * dv * 4);
      d->off_rg = take(size_t(d->p.replay_total) * H * (2 * dk + dv + 1) * 4);
      d->off_Tm = take(MC * BT * BT * es);
      d->off_Xm = take(MC * BT * BT * es);
      d->off_Am = take(MC * BT * BT * es);
      d->off_dslot = take(size_t(d->p.n_slots) * H * dk * dv * 4);
      d->ws_bwd = off;
      if (d->ws_fwd == 0) d->ws_fwd = 256;
    } catch (...) {
      free_dev(d);
      delete d;
      throw;
    }
    *out = d;
  });
}

int harts_kda_workspace_size(const harts_dev_plan* dplan, int32_t backward, size_t* bytes) {
  return guarded([&] {
    if (!dplan || !bytes) throw Error(HARTS_EINVAL, "dplan and bytes must be non-NULL");
    if (backward < 0 || backward > 2) throw Error(HARTS_EINVAL, "backward must be 0, 1 or 2");
    *bytes = backward ? dplan->ws_bwd : dplan->ws_fwd;
  });
}

void harts_dev_plan_free(harts_dev_plan* dplan) {
  if (!dplan) return;
  free_dev(dplan);
  delete dplan;
}

int harts_kda_fwd(const harts_dev_plan* d, const harts_kda_io* io, void* stream) {
  return guarded([&] {
    if (!d) throw Error(HARTS_EINVAL, "dplan is NULL");
    check_io(d, io, false);
    hipStream_t s0 = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(io->workspace);
    // Preparation of every round after the first runs on an auxiliary stream (it depends on the
    // inputs only); the serial passes follow in round order on the caller's stream.
    Events ev;
    hipStream_t s1 = aux_stream(0);
    const bool slab = harts::kda_slab_supported(d->dims);
    // keep: the preparation also writes the backward's per-chunk operands and the serial pass
    // every chunk-start state, so that the backward neither prepares nor recomputes
    const bool keep = io->keep && slab;
    {
      std::lock_guard<std::mutex> lk(d->kept_mu);
      if (keep) d->kept_ws = io->workspace;
      else if (d->kept_ws == io->workspace) d->kept_ws = nullptr;
    }
    int32_t* ctr = reinterpret_cast<int32_t*>(ws + d->off_ctr);
    // The first round's preparation runs on the caller's stream in static item order and clears
    // the item counters of every later launch (no separate reset launch); round r + 1's
    // preparation is enqueued behind the start of round r's serial pass, so that the serial pass
    // takes its compute units first, and its workgroups draw items from a counter and fill the
    // rest of the chip as it frees up.
    hipEvent_t started = nullptr;
    for (int r = 0; r < d->p.n_rounds; ++r) {
      const int64_t units = int64_t(d->p.rounds[r].vrow1 - d->p.rounds[r].vrow0) * d->dims.H;
      hipStream_t sp = r == 0 ? s0 : s1;
      if (started) hip_check(hipStreamWaitEvent(s1, started, 0), "hipStreamWaitEvent");
      {
        harts::RoundArgs a = round_args(d, io, r, ws);
        if (r == 0) {
          a.zero = ctr;
          a.nzero = 3 * d->p.n_rounds;
        } else {
          a.ctr = ctr + 3 * r;
        }
        ProfScope ps("kda_prep_fwd", sp, units);
        hip_check(harts::launch_kda_prep(d->dims, a, keep ? 2 : 0, sp), "prep kernel launch");
      }
      if (r > 0) hip_check(hipStreamWaitEvent(s0, ev.record(s1), 0), "hipStreamWaitEvent");
      if (r + 1 < d->p.n_rounds) started = ev.record(s0);
      harts::RoundArgs a = round_args(d, io, r, ws);
      a.o = io->o;
      if (!keep) a.h = a.hc = nullptr;
      ProfScope ps("kda_state_fwd", s0, units);
      if (slab) {
        harts::BwdRoundArgs b{};
        b.r = a;
        hip_check(harts::launch_kda_slab(d->dims, b, keep ? 3 : 0, d->p.rounds[r].max_chunks, s0),
                  "state kernel launch");
      } else {
        hip_check(harts::launch_kda_state(d->dims, a, false, s0), "state kernel launch");
      }
    }
    // join: every preparation precedes the last serial pass on the caller's stream
  });
}

int harts_kda_fwd_varlen(const harts_varlen_args* a, void* stream) {
  harts_plan* plan = nullptr;
  harts_dev_plan* dp = nullptr;
  void* ws = nullptr;
  const int rc = guarded([&] {
    if (!a) throw Error(HARTS_EINVAL, "args is NULL");
    if (!a->cu_seqlens || a->n_seq < 1) throw Error(HARTS_EINVAL, "cu_seqlens and n_seq >= 1 are required");
    if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->o)
      throw Error(HARTS_EINVAL, "q, k, v, g, beta and o are required");
    std::vector<uint8_t> mask;
    const uint8_t* has_init = nullptr;
    if (a->init_states) {
      mask.assign(size_t(a->n_seq), 1);
      if (a->init_mask) std::copy(a->init_mask, a->init_mask + a->n_seq, mask.begin());
      has_init = mask.data();
    }
    int e = harts_plan_create_varlen(a->cu_seqlens, a->n_seq, a->chunk_B, has_init, a->boundary_states ? 1 : 0, &plan);
    if (e != HARTS_OK) throw Error(e, g_err);
    e = harts_plan_upload(plan, a->H, a->dk, a->dv, a->dtype, stream, &dp);
    if (e != HARTS_OK) throw Error(e, g_err);
    if (a->boundary_states && a->boundary_offsets) {
      e = harts_plan_boundary_offsets(plan, a->boundary_offsets);
      if (e != HARTS_OK) throw Error(e, g_err);
    }
    size_t bytes = 0;
    e = harts_kda_workspace_size(dp, 0, &bytes);
    if (e != HARTS_OK) throw Error(e, g_err);
    hip_check(hipMalloc(&ws, bytes), "hipMalloc (workspace)");
    harts_kda_io io{};
    io.q = a->q;
    io.k = a->k;
    io.v = a->v;
    io.g = a->g;
    io.beta = a->beta;
    io.o = a->o;
    io.states = a->boundary_states;
    io.init_states = a->init_states;
    io.final_states = a->final_states;
    io.workspace = ws;
    io.workspace_bytes = bytes;
    e = harts_kda_fwd(dp, &io, stream);
    if (e != HARTS_OK) throw Error(e, g_err);
    hip_check(hipStreamSynchronize(static_cast<hipStream_t>(stream)), "hipStreamSynchronize");
  });
  // every path waits for the stream before the plan's descriptors and the workspace are freed
  if (rc != HARTS_OK && (dp || ws)) (void)hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (ws) (void)hipFree(ws);
  harts_dev_plan_free(dp);
  harts_plan_free(plan);
  return rc;
}

int harts_kda_bwd(const harts_dev_plan* d, const harts_kda_io* io, const harts_kda_grad* g, void* stream) {
  return guarded([&] {
    if (!d) throw Error(HARTS_EINVAL, "dplan is NULL");
    check_io(d, io, true);
    if (!g || !g->dO || !g->dq || !g->dk || !g->dv || !g->dg || !g->dbeta)
      throw Error(HARTS_EINVAL, "dO, dq, dk, dv, dg and dbeta are required");
    hipStream_t s0 = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(io->workspace);
    const bool slab = harts::kda_slab_supported(d->dims);
    const bool keep = io->keep && slab;  // operands and chunk-start states are in the workspace
    if (keep) {
      std::lock_guard<std::mutex> lk(d->kept_mu);
      if (d->kept_ws != io->workspace)
        throw Error(HARTS_EINVAL, "keep = 1 needs this workspace as left by a forward with keep = 1 on this device plan");
    }
    const int R = d->p.n_rounds;
    // Three streams, rounds in reverse:
    //   s1: preparation and state recompute of every round (they need no gradient);
    //   s0: the state-gradient chain (each round needs the initial-state gradients of the
    //       later rounds that consume its handed-off states);
    //   s2: the per-chunk gradient kernels of a round once its recompute and state
    //       gradient are done.
    Events ev;
    hipStream_t s1 = aux_stream(0), s2 = aux_stream(1);
    int32_t* ctr = reinterpret_cast<int32_t*>(ws + d->off_ctr);
    // Recompute: the last round's preparation runs first, on the caller's stream, in static item
    // order, and clears the item counters of every later launch.  Keep: a reset launch does.
    if (keep) hip_check(harts::launch_zero_i32(ctr, 3 * int64_t(R), s0), "counter reset");
    auto round = [&](int r) {
      harts::BwdRoundArgs b{};
      b.r = round_args(d, io, r, ws);
      b.r.o = nullptr;
      b.dO = g->dO;
      b.dq = g->dq;
      b.dk = g->dk;
      b.dv = g->dv;
      b.dg = g->dg;
      b.dbeta = g->dbeta;
      const size_t item0 = size_t(d->p.rounds[r].chunk0) * d->dims.H;
      const size_t sz = size_t(d->dims.D) * d->dims.DV * (d->dims.dtype == HARTS_DTYPE_BF16 ? 2 : 4);
      b.dh = ws + d->off_dh + item0 * sz;
      b.dhc = d->dims.dtype == HARTS_DTYPE_FP32 ? ws + d->off_dhc + item0 * sz : nullptr;
      b.dinit = d->p.varlen ? g->dinit : reinterpret_cast<float*>(ws + d->off_dinit);
      b.dstates = d->p.varlen ? nullptr : g->dstates;
      b.slot_cons_off = d->p.varlen ? nullptr : d->cons_off;
      b.slot_cons = d->p.varlen ? nullptr : d->cons;
      b.replay_grad = reinterpret_cast<float*>(ws + d->off_rg);
      if (slab && !d->p.varlen) b.dslot = g->dstates ? g->dstates : reinterpret_cast<float*>(ws + d->off_dslot);
      return b;
    };
    auto units = [&](int r) { return int64_t(d->p.rounds[r].vrow1 - d->p.rounds[r].vrow0) * d->dims.H; };
    std::vector<hipEvent_t> prepped(R, nullptr), recomputed(R, nullptr);
    for (int r = R - 1; r >= 0 && !keep; --r) {
      harts::BwdRoundArgs b = round(r);
      const bool first = r == R - 1;
      {
        hipStream_t sp = first ? s0 : s1;
        ProfScope ps("kda_prep_bwd", sp, units(r));
        harts::RoundArgs a = b.r;
        if (first) {
          a.zero = ctr;
          a.nzero = 3 * R;
        } else {
          a.ctr = ctr + 3 * r + 1;
        }
        hip_check(harts::launch_kda_prep(d->dims, a, 1, sp), "prep kernel launch");
      }
      if (first) {
        fork(s0, s1, ev);
        prepped[size_t(r)] = nullptr;  // on the caller's stream already
      } else {
        prepped[size_t(r)] = ev.record(s1);
      }
      {
        ProfScope ps("kda_state_bwd", s1, units(r));
        if (slab) hip_check(harts::launch_kda_slab(d->dims, b, 1, d->p.rounds[r].max_chunks, s1), "state kernel launch");
        else hip_check(harts::launch_kda_state(d->dims, b.r, true, s1), "state kernel launch");
      }
      recomputed[size_t(r)] = ev.record(s1);
    }
    // The per-chunk gradients of round r + 1 are enqueued behind the start of round r's
    // state-gradient pass, so that the serial pass takes its compute units before the
    // gradient kernels fill the chip.
    auto grads = [&](int r) {
      harts::BwdRoundArgs b = round(r);
      if (!keep) hip_check(hipStreamWaitEvent(s2, recomputed[size_t(r)], 0), "hipStreamWaitEvent");
      {
        ProfScope ps("kda_grad", s2, units(r));
        b.r.ctr = ctr + 3 * r + 2;
        hip_check(harts::launch_kda_grad(d->dims, b, s2), "gradient kernel launch");
      }
    };
    // s2 needs no fork of its own: each gradient launch waits for an event recorded on s0 after
    // this call's first launch.  (keep: s1 runs nothing.)
    for (int r = R - 1; r >= 0; --r) {
      harts::BwdRoundArgs b = round(r);
      if (b.dslot) {
        // gradients of the states this round hands off: complete, since every consumer runs later
        const int32_t n0 = d->rslot_off[size_t(r)], n1 = d->rslot_off[size_t(r) + 1];
        ProfScope ps("kda_slot_grad", s0, int64_t(n1 - n0));
        hip_check(harts::launch_slot_grad(d->dims, d->rslots + n0, n1 - n0, d->cons_off, d->cons, b.dinit,
                                          const_cast<float*>(b.dslot), s0),
                  "slot gradient launch");
      }
      // the slot gradients above need only the later rounds; this round's preparation is awaited
      // after them
      if (prepped[size_t(r)]) hip_check(hipStreamWaitEvent(s0, prepped[size_t(r)], 0), "hipStreamWaitEvent");
      // round r + 1's state gradient (and everything before it on s0) is complete here
      hipEvent_t ready = r + 1 < R ? ev.record(s0) : nullptr;
      {
        ProfScope ps("kda_dstate", s0, units(r));
        if (slab) hip_check(harts::launch_kda_slab(d->dims, b, 2, d->p.rounds[r].max_chunks, s0), "state-gradient kernel launch");
        else hip_check(harts::launch_kda_dstate(d->dims, b, s0), "state-gradient kernel launch");
      }
      if (r + 1 < R) {
        hip_check(hipStreamWaitEvent(s2, ready, 0), "hipStreamWaitEvent");
        grads(r + 1);
      }
    }
    hip_check(hipStreamWaitEvent(s2, ev.record(s0), 0), "hipStreamWaitEvent");
    grads(0);
    // replayed rows' gradients into their own rows: every gradient launch is behind it on s2
    if (!d->p.fix_rows.empty()) {
      ProfScope ps("kda_replay_fixup", s2, int64_t(d->p.replay_total) * d->dims.H);
      hip_check(harts::launch_replay_fixup(d->dims, d->fix_rows, d->fix_off, d->fix_idx,
                                           int32_t(d->p.fix_rows.size()), reinterpret_cast<float*>(ws + d->off_rg),
                                           g->dk, g->dv, g->dg, g->dbeta, s2),
                "replay fixup launch");
    }
    // join: the caller's stream continues after every round's gradients (s1's last launch, the
    // first round's recompute, precedes the first round's gradients)
    hip_check(hipStreamWaitEvent(s0, ev.record(s2), 0), "hipStreamWaitEvent");
  });
}

size_t harts_logprob_workspace_size(int64_t C) { return C > 0 ? align256(size_t(C) * 4) : 256; }
size_t harts_logprob_workspace(int64_t C, int64_t) { return harts_logprob_workspace_size(C); }

int harts_logprob_gather(const void* logits, int64_t C, int64_t V, int32_t dtype, const int64_t* m,
                         const int32_t* labels, int64_t S, float* logp_out, int32_t* q_out, float* lse_out,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return guarded([&] {
    if (C < 0 || V < 1 || S < 0) throw Error(HARTS_EINVAL, "need C >= 0, V >= 1, S >= 0");
    if (dtype != HARTS_DTYPE_BF16 && dtype != HARTS_DTYPE_FP32) throw Error(HARTS_EINVAL, "unknown dtype");
    if (C > 0 && !logits) throw Error(HARTS_EINVAL, "logits is NULL");
    if (S > 0 && (!m || !labels || !logp_out)) throw Error(HARTS_EINVAL, "m, labels and logp_out are required");
    if (C >= (int64_t(1) << 31)) throw Error(HARTS_ERANGE, "C must be < 2^31");
    float* lse = lse_out;
    if (!lse) {
      if (!workspace || workspace_bytes < size_t(C) * 4) throw Error(HARTS_EINVAL, "workspace too small");
      lse = static_cast<float*>(workspace);
    }
    ProfScope ps("logprob_gather", static_cast<hipStream_t>(stream), C);
    hip_check(harts::launch_logprob(logits, C, V, dtype, m, labels, S, logp_out, q_out, lse,
                                    static_cast<hipStream_t>(stream)),
              "log-prob kernel launch");
  });
}

int harts_logprob_gather_noalloc(const void* logits, int64_t C, int64_t V, int32_t dtype, const int64_t* m,
                                 const int32_t* labels, int64_t S, float* logp_out, int32_t* q_out, void* stream) {
  return guarded([&] {
    if (C > HARTS_LOGPROB_NOALLOC_MAX_ROWS)
      throw Error(HARTS_EINVAL, "C = " + std::to_string(C) + " exceeds the no-allocation maximum of " +
                                    std::to_string(HARTS_LOGPROB_NOALLOC_MAX_ROWS) + " rows");
    if (C < 0 || V < 1 || S < 0) throw Error(HARTS_EINVAL, "need C >= 0, V >= 1, S >= 0");
    if (dtype != HARTS_DTYPE_BF16 && dtype != HARTS_DTYPE_FP32) throw Error(HARTS_EINVAL, "unknown dtype");
    if (C > 0 && !logits) throw Error(HARTS_EINVAL, "logits is NULL");
    if (S > 0 && (!m || !labels || !logp_out)) throw Error(HARTS_EINVAL, "m, labels and logp_out are required");
    static_assert(HARTS_LOGPROB_NOALLOC_MAX_ROWS == harts::kLogprobStaticRows, "one maximum");
    // no timing scope here: it would create events
    hip_check(harts::launch_logprob_static(logits, C, V, dtype, m, labels, S, logp_out, q_out,
                                           static_cast<hipStream_t>(stream)),
              "log-prob kernel launch");
  });
}

int harts_logprob_backward(const void* logits, int64_t C, int64_t V, int32_t dtype, const float* lse,
                           const int64_t* row_off, const int64_t* row_pos, const int32_t* labels, const float* dlogp,
                           int64_t S, void* dlogits_out, void* stream) {
  return guarded([&] {
    if (C < 0 || V < 1 || S < 0) throw Error(HARTS_EINVAL, "need C >= 0, V >= 1, S >= 0");
    if (dtype != HARTS_DTYPE_BF16 && dtype != HARTS_DTYPE_FP32) throw Error(HARTS_EINVAL, "unknown dtype");
    if (C >= (int64_t(1) << 31)) throw Error(HARTS_ERANGE, "C must be < 2^31");
    if (C == 0) return;
    if (!logits || !lse || !row_off || !dlogits_out) throw Error(HARTS_EINVAL, "logits, lse, row_off and dlogits_out are required");
    if (S > 0 && (!row_pos || !labels || !dlogp)) throw Error(HARTS_EINVAL, "row_pos, labels and dlogp are required");
    const size_t es = dtype == HARTS_DTYPE_BF16 ? 2 : 4;
    const char* a = static_cast<const char*>(logits);
    const char* b = static_cast<const char*>(dlogits_out);
    const size_t bytes = size_t(C) * size_t(V) * es;
    if (a < b + bytes && b < a + bytes) throw Error(HARTS_EINVAL, "dlogits_out overlaps logits");
    ProfScope ps("logprob_backward", static_cast<hipStream_t>(stream), C);
    hip_check(harts::launch_logprob_bwd(logits, C, V, dtype, lse, row_off, row_pos, labels, dlogp, dlogits_out,
                                        static_cast<hipStream_t>(stream)),
              "log-prob backward kernel launch");
  });
}

int harts_logprob_check_map(const int64_t* m, const int32_t* labels, int64_t S, int64_t C, int64_t V) {
  return guarded([&] {
    if (S < 0 || C < 0 || V < 1) throw Error(HARTS_EINVAL, "need S >= 0, C >= 0, V >= 1");
    if (S > 0 && !m) throw Error(HARTS_EINVAL, "m is NULL");
    for (int64_t s = 0; s < S; ++s) {
      if (m[s] < 0 || m[s] >= C) throw Error(HARTS_ERANGE, "m[" + std::to_string(s) + "] is outside [0, C)");
      if (labels && (labels[s] < 0 || labels[s] >= V))
        throw Error(HARTS_ERANGE, "labels[" + std::to_string(s) + "] is outside [0, V)");
    }
  });
}

int harts_logprob_rows(const int64_t* m, int64_t S, int64_t C, int64_t* row_off, int64_t* row_pos) {
  return guarded([&] {
    if (S < 0 || C < 0) throw Error(HARTS_EINVAL, "need S >= 0, C >= 0");
    if (!row_off || (S > 0 && (!m || !row_pos))) throw Error(HARTS_EINVAL, "m, row_off and row_pos are required");
    std::vector<int64_t> cnt(size_t(C) + 1, 0);
    for (int64_t s = 0; s < S; ++s) {
      if (m[s] < 0 || m[s] >= C) throw Error(HARTS_EINVAL, "m[" + std::to_string(s) + "] is outside [0, C)");
      ++cnt[size_t(m[s]) + 1];
    }
    for (int64_t c = 0; c < C; ++c) cnt[size_t(c) + 1] += cnt[size_t(c)];
    std::copy(cnt.begin(), cnt.end(), row_off);
    for (int64_t s = 0; s < S; ++s) row_pos[cnt[size_t(m[s])]++] = s;  // stable: positions in increasing s
  });
}

int harts_conv_tables(const int64_t* m, const int64_t* traj_offsets, int64_t n_traj, int64_t C, int32_t w,
                      int32_t* anc, int64_t* gather_off, int64_t* gather) {
  return guarded([&] {
    if (n_traj < 0 || C < 0) throw Error(HARTS_EINVAL, "need n_traj >= 0, C >= 0");
    if (w < 2 || w > 8) throw Error(HARTS_EINVAL, "w must be in [2, 8]");
    if (!traj_offsets || !gather_off || (C > 0 && (!anc || !gather))) throw Error(HARTS_EINVAL, "missing arrays");
    if (traj_offsets[0] != 0) throw Error(HARTS_EINVAL, "traj_offsets[0] must be 0");
    for (int64_t i = 0; i < n_traj; ++i)
      if (traj_offsets[i + 1] < traj_offsets[i]) throw Error(HARTS_EINVAL, "traj_offsets must be non-decreasing");
    if (traj_offsets[n_traj] > 0 && !m) throw Error(HARTS_EINVAL, "m is NULL");
    const int K = w - 1;
    constexpr int32_t kUnset = INT32_MIN;
    std::fill(anc, anc + size_t(C) * K, kUnset);
    for (int64_t i = 0; i < n_traj; ++i) {
      const int64_t o = traj_offsets[i], L = traj_offsets[i + 1] - o;
      for (int64_t p = 0; p < L; ++p) {
        const int64_t t = m[o + p];
        if (t < 0 || t >= C) throw Error(HARTS_EINVAL, "m[" + std::to_string(o + p) + "] is outside [0, C)");
        for (int j = 1; j <= K; ++j) {
          const int32_t a = p >= j ? int32_t(m[o + p - j]) : -1;
          int32_t& slot = anc[size_t(t) * K + j - 1];
          if (slot == kUnset) slot = a;
          else if (slot != a)
            throw Error(HARTS_EINVAL, "m is not the map of a prefix tree: row " + std::to_string(t) +
                                          " has two different predecessors");
        }
      }
    }
    std::vector<int64_t> cnt(size_t(C) + 1, 0);
    for (int64_t t = 0; t < C; ++t)
      for (int j = 1; j <= K; ++j) {
        const int32_t a = anc[size_t(t) * K + j - 1];
        if (a == kUnset) throw Error(HARTS_EINVAL, "row " + std::to_string(t) + " is on no trajectory");
        if (a >= 0) ++cnt[size_t(a) + 1];
      }
    for (int64_t c = 0; c < C; ++c) cnt[size_t(c) + 1] += cnt[size_t(c)];
    std::copy(cnt.begin(), cnt.end(), gather_off);
    for (int j = 1; j <= K; ++j)  // increasing (j, t) within each row's list
      for (int64_t t = 0; t < C; ++t) {
        const int32_t a = anc[size_t(t) * K + j - 1];
        if (a >= 0) gather[cnt[size_t(a)]++] = t * 8 + j;
      }
  });
}

size_t harts_conv_workspace_size(int64_t C, int32_t channels, int32_t w) {
  return C > 0 && channels > 0 && w > 0 ? align256(harts::conv_workspace_bytes(C, channels, w)) : 256;
}

namespace {
void conv_check(const void* x, int64_t C, int32_t channels, int32_t w, int32_t dtype) {
  if (C < 0) throw Error(HARTS_EINVAL, "need C >= 0");
  if (C > int64_t(65535) * 64) throw Error(HARTS_ERANGE, "C must be <= 65535 * 64 rows");
  if (channels <= 0 || channels % 8) throw Error(HARTS_EINVAL, "channels must be a positive multiple of 8");
  if (w < 2 || w > 8) throw Error(HARTS_EINVAL, "w must be in [2, 8]");
  if (dtype != HARTS_DTYPE_BF16 && dtype != HARTS_DTYPE_FP32) throw Error(HARTS_EINVAL, "unknown dtype");
  if (C > 0 && (!x || reinterpret_cast<uintptr_t>(x) % 16)) throw Error(HARTS_EINVAL, "x must be 16-byte aligned");
}
}  // namespace

int harts_conv_fwd(const void* x, const float* weight, const int32_t* anc, int64_t C, int32_t channels, int32_t w,
                   int32_t dtype, void* out, void* stream) {
  return guarded([&] {
    conv_check(x, C, channels, w, dtype);
    if (C == 0) return;
    if (!weight || !anc || !out || reinterpret_cast<uintptr_t>(out) % 16)
      throw Error(HARTS_EINVAL, "weight, anc and a 16-byte aligned out are required");
    const size_t bytes = size_t(C) * size_t(channels) * (dtype == HARTS_DTYPE_BF16 ? 2 : 4);
    const char *a = static_cast<const char*>(x), *b = static_cast<const char*>(out);
    if (a < b + bytes && b < a + bytes) throw Error(HARTS_EINVAL, "out overlaps x");
    ProfScope ps("conv_fwd", static_cast<hipStream_t>(stream), C);
    hip_check(harts::launch_conv_fwd(x, weight, anc, C, channels, w, dtype, out, static_cast<hipStream_t>(stream)),
              "convolution kernel launch");
  });
}

int harts_conv_bwd(const void* x, const float* weight, const int32_t* anc, const int64_t* gather_off,
                   const int64_t* gather, const void* dout, int64_t C, int32_t channels, int32_t w, int32_t dtype,
                   void* dx, float* dweight, void* workspace, size_t workspace_bytes, void* stream) {
  return guarded([&] {
    conv_check(x, C, channels, w, dtype);
    if (C == 0) return;
    if (!weight || !dout || reinterpret_cast<uintptr_t>(dout) % 16) throw Error(HARTS_EINVAL, "weight and a 16-byte aligned dout are required");
    if (dx && (!gather_off || !gather || reinterpret_cast<uintptr_t>(dx) % 16))
      throw Error(HARTS_EINVAL, "dx needs gather_off, gather and 16-byte alignment");
    if (dweight && (!anc || !workspace || workspace_bytes < harts::conv_workspace_bytes(C, channels, w)))
      throw Error(HARTS_EINVAL, "dweight needs anc and a workspace of harts_conv_workspace_size bytes");
    ProfScope ps("conv_bwd", static_cast<hipStream_t>(stream), C);
    hip_check(harts::launch_conv_bwd(x, weight, anc, gather_off, gather, dout, C, channels, w, dtype, dx, dweight,
                                     static_cast<float*>(workspace), static_cast<hipStream_t>(stream)),
              "convolution gradient kernel launch");
  });
}

int harts_attn_tables_build(const int64_t* m, const int64_t* traj_offsets, int64_t n_traj, int64_t C,
                            harts_attn_tables** out) {
  return guarded([&] {
    if (!out) throw Error(HARTS_EINVAL, "out is NULL");
    *out = nullptr;
    auto* t = new harts_attn_tables{harts::build_attn_tables(m, traj_offsets, n_traj, C)};
    *out = t;
  });
}

int harts_attn_info(const harts_attn_tables* t, harts_attn_info_t* info) {
  return guarded([&] {
    if (!t || !info) throw Error(HARTS_EINVAL, "NULL argument");
    info->C = t->t.C;
    info->n_segments = t->t.n_segments;
    info->n_qtiles = int64_t(t->t.qtiles.size() / 4);
    info->n_ktiles = int64_t(t->t.ktiles.size() / 4);
    info->kv_list_len = int64_t(t->t.kv_list.size());
    info->q_list_len = int64_t(t->t.q_list.size());
    info->pairs = t->t.pairs;
    info->max_depth = t->t.max_depth;
  });
}

int harts_attn_tables_copy(const harts_attn_tables* t, int32_t* qtiles, int32_t* kv_list, int32_t* ktiles,
                           int32_t* q_list, int32_t* pos) {
  return guarded([&] {
    if (!t) throw Error(HARTS_EINVAL, "NULL tables");
    auto cp = [](const std::vector<int32_t>& v, int32_t* dst) {
      if (!v.empty()) {
        if (!dst) throw Error(HARTS_EINVAL, "missing output array");
        std::memcpy(dst, v.data(), v.size() * sizeof(int32_t));
      }
    };
    cp(t->t.qtiles, qtiles);
    cp(t->t.kv_list, kv_list);
    cp(t->t.ktiles, ktiles);
    cp(t->t.q_list, q_list);
    if (pos) std::copy(t->t.pos.begin(), t->t.pos.end(), pos);
  });
}

void harts_attn_tables_free(harts_attn_tables* t) { delete t; }

size_t harts_attn_workspace_size(int64_t C, int32_t H) { return C > 0 && H > 0 ? align256(size_t(C) * H * 4) : 256; }

namespace {
void attn_check(const void* q, const void* k, const void* v, const int32_t* tiles, int64_t n_tiles,
                const int32_t* list, int64_t C, int32_t H, int32_t dqk, int32_t dv) {
  if (C < 0 || H <= 0 || n_tiles < 0) throw Error(HARTS_EINVAL, "need C >= 0, H > 0, n_tiles >= 0");
  if (C > INT32_MAX) throw Error(HARTS_ERANGE, "C must fit int32 row indices");
  if (!harts::attn_dims_supported(dqk, dv))
    throw Error(HARTS_EINVAL, "(dqk, dv) must be (192, 128), (128, 128) or (64, 64)");
  if (n_tiles * int64_t(H) > INT32_MAX) throw Error(HARTS_ERANGE, "too many tiles x heads for one grid");
  if (C > 0 && n_tiles == 0) throw Error(HARTS_EINVAL, "no tiles for a non-empty set of rows");
  for (const void* p : {q, k, v})
    if (C > 0 && (!p || reinterpret_cast<uintptr_t>(p) % 16)) throw Error(HARTS_EINVAL, "q, k, v must be 16-byte aligned");
  if (n_tiles > 0 && (!tiles || !list || reinterpret_cast<uintptr_t>(tiles) % 16))
    throw Error(HARTS_EINVAL, "tiles (16-byte aligned) and list are required");
}
void no_overlap(const void* a, size_t na, const void* b, size_t nb, const char* what) {
  const char *x = static_cast<const char*>(a), *y = static_cast<const char*>(b);
  if (x < y + nb && y < x + na) throw Error(HARTS_EINVAL, what);
}
}  // namespace

int harts_attn_fwd(const void* q, const void* k, const void* v, const int32_t* qtiles, int64_t n_qtiles,
                   const int32_t* kv_list, int64_t C, int32_t H, int32_t dqk, int32_t dv, float scale, void* o,
                   float* lse, void* stream) {
  return guarded([&] {
    attn_check(q, k, v, qtiles, n_qtiles, kv_list, C, H, dqk, dv);
    if (C == 0) return;
    if (!o || !lse || reinterpret_cast<uintptr_t>(o) % 16) throw Error(HARTS_EINVAL, "o (16-byte aligned) and lse are required");
    const size_t no = size_t(C) * H * dv * 2, nq = size_t(C) * H * dqk * 2;
    no_overlap(o, no, q, nq, "o overlaps q");
    no_overlap(o, no, k, nq, "o overlaps k");
    no_overlap(o, no, v, no, "o overlaps v");
    harts::AttnArgs a{};
    a.q = static_cast<const __bf16*>(q);
    a.k = static_cast<const __bf16*>(k);
    a.v = static_cast<const __bf16*>(v);
    a.tiles = qtiles;
    a.list = kv_list;
    a.o_out = static_cast<__bf16*>(o);
    a.lse_out = lse;
    a.C = C;
    a.H = H;
    a.scale = scale;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    ProfScope ps("attn_fwd", s, C);
    hip_check(harts::launch_attn(0, a, n_qtiles, dqk, dv, s), "attention forward launch");
  });
}

int harts_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   const int32_t* qtiles, int64_t n_qtiles, const int32_t* kv_list, const int32_t* ktiles,
                   int64_t n_ktiles, const int32_t* q_list, int64_t C, int32_t H, int32_t dqk, int32_t dv,
                   float scale, void* dq, void* dk, void* dv_out, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return guarded([&] {
    attn_check(q, k, v, qtiles, n_qtiles, kv_list, C, H, dqk, dv);
    attn_check(q, k, v, ktiles, n_ktiles, q_list, C, H, dqk, dv);
    if (C == 0) return;
    for (const void* p : {o, dout, static_cast<const void*>(dq), static_cast<const void*>(dk), static_cast<const void*>(dv_out)})
      if (!p || reinterpret_cast<uintptr_t>(p) % 16) throw Error(HARTS_EINVAL, "o, dout, dq, dk, dv must be 16-byte aligned");
    if (!lse) throw Error(HARTS_EINVAL, "lse is required");
    if (!workspace || workspace_bytes < size_t(C) * H * 4)
      throw Error(HARTS_EINVAL, "workspace must hold harts_attn_workspace_size bytes");
    const size_t nqb = size_t(C) * H * dqk * 2, nvb = size_t(C) * H * dv * 2;
    const void* ins[] = {q, k, v, o, dout};
    const size_t insz[] = {nqb, nqb, nvb, nvb, nvb};
    const void* outs[] = {dq, dk, dv_out};
    const size_t outsz[] = {nqb, nqb, nvb};
    for (int i = 0; i < 3; ++i) {
      for (int j = 0; j < 5; ++j) no_overlap(outs[i], outsz[i], ins[j], insz[j], "a gradient overlaps an input");
      for (int j = 0; j < i; ++j) no_overlap(outs[i], outsz[i], outs[j], outsz[j], "gradients overlap");
    }
    harts::AttnArgs a{};
    a.q = static_cast<const __bf16*>(q);
    a.k = static_cast<const __bf16*>(k);
    a.v = static_cast<const __bf16*>(v);
    a.o = static_cast<const __bf16*>(o);
    a.dout = static_cast<const __bf16*>(dout);
    a.lse = lse;
    a.delta = static_cast<const float*>(workspace);
    a.delta_out = static_cast<float*>(workspace);
    a.dq = static_cast<__bf16*>(dq);
    a.dk = static_cast<__bf16*>(dk);
    a.dv = static_cast<__bf16*>(dv_out);
    a.C = C;
    a.H = H;
    a.scale = scale;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    {
      ProfScope ps("attn_delta", s, C);
      hip_check(harts::launch_attn(1, a, 0, dqk, dv, s), "attention delta launch");
    }
    {
      a.tiles = qtiles;
      a.list = kv_list;
      ProfScope ps("attn_dq", s, C);
      hip_check(harts::launch_attn(2, a, n_qtiles, dqk, dv, s), "attention dq launch");
    }
    {
      a.tiles = ktiles;
      a.list = q_list;
      ProfScope ps("attn_dkv", s, C);
      hip_check(harts::launch_attn(3, a, n_ktiles, dqk, dv, s), "attention dk/dv launch");
    }
  });
}

size_t harts_moe_workspace_size(int64_t C, int32_t E) {
  return C >= 0 && E > 0 ? align256(size_t(harts::moe_partial_rows(C)) * size_t(2 * E + 1) * 4) : 256;
}

namespace {
void moe_check(int64_t C, int32_t E, int32_t k, int64_t S) {
  if (C < 0 || S < 0) throw Error(HARTS_EINVAL, "need C >= 0, S >= 0");
  if (E != 64 && E != 128 && E != 256 && E != 512) throw Error(HARTS_EINVAL, "E must be 64, 128, 256 or 512");
  if (k < 1 || k > 8 || k > E) throw Error(HARTS_EINVAL, "k must be in [1, 8]");
  if (C > 0 && S < C) throw Error(HARTS_EINVAL, "S (the sum of q) must be >= C");
  if (S > int64_t(INT32_MAX) / k) throw Error(HARTS_ERANGE, "S * k must fit int32 counts");
  if (C > int64_t(INT32_MAX) * 64) throw Error(HARTS_ERANGE, "C too large");
}
}  // namespace

int harts_moe_stats(const float* logits, const float* bias, const int32_t* q, int64_t C, int32_t E, int32_t k,
                    int64_t S, int32_t* topk, float* lse, int32_t* counts, float* mass, float* losses,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return guarded([&] {
    moe_check(C, E, k, S);
    if (!counts || !mass || !losses) throw Error(HARTS_EINVAL, "counts, mass and losses are required");
    if (C > 0 && (!logits || !q || !topk || !lse)) throw Error(HARTS_EINVAL, "logits, q, topk and lse are required");
    if (!workspace || workspace_bytes < size_t(harts::moe_partial_rows(C)) * size_t(2 * E + 1) * 4)
      throw Error(HARTS_EINVAL, "workspace must hold harts_moe_workspace_size bytes");
    harts::MoeArgs a{};
    a.z = logits;
    a.bias = bias;
    a.q = q;
    a.top = topk;
    a.lse = lse;
    a.counts = counts;
    a.part = static_cast<float*>(workspace);
    a.mass = mass;
    a.losses = losses;
    a.C = C;
    a.S = S;
    a.E = E;
    a.k = k;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    ProfScope ps("moe_stats", s, C);
    hip_check(harts::launch_moe(0, a, s), "router statistics launch");
  });
}

int harts_moe_grad(const float* logits, const int32_t* q, const int32_t* counts, int64_t C, int32_t E, int32_t k,
                   int64_t S, float z_coef, float aux_coef, float* dlogits, void* stream) {
  return guarded([&] {
    moe_check(C, E, k, S);
    if (C == 0) return;
    if (!logits || !q || !counts || !dlogits) throw Error(HARTS_EINVAL, "logits, q, counts and dlogits are required");
    const size_t nb = size_t(C) * E * 4;
    const char *x = reinterpret_cast<const char*>(logits), *y = reinterpret_cast<const char*>(dlogits);
    if (x < y + nb && y < x + nb) throw Error(HARTS_EINVAL, "dlogits overlaps logits");
    harts::MoeArgs a{};
    a.z = logits;
    a.q = q;
    a.counts = const_cast<int32_t*>(counts);
    a.dz = dlogits;
    a.C = C;
    a.S = S;
    a.E = E;
    a.k = k;
    a.z_coef = z_coef;
    a.aux_coef = aux_coef;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    ProfScope ps("moe_grad", s, C);
    hip_check(harts::launch_moe(1, a, s), "router gradient launch");
  });
}

int harts_moe_bias_update(const int32_t* counts, int32_t E, float gamma, float* bias, void* stream) {
  return guarded([&] {
    if (E <= 0) throw Error(HARTS_EINVAL, "need E > 0");
    if (!counts || !bias) throw Error(HARTS_EINVAL, "counts and bias are required");
    hip_check(harts::launch_moe_bias(counts, E, gamma, bias, static_cast<hipStream_t>(stream)), "bias update launch");
  });
}

int harts_profile_enable(int32_t on) {
  return guarded([&] {
    std::vector<ProfRec> old;
    {
      std::lock_guard<std::mutex> lk(g_prof_mu);
      g_prof_on = on != 0;
      if (on) old.swap(g_prof);
    }
    for (auto& r : old) {
      (void)hipEventDestroy(r.e0);
      (void)hipEventDestroy(r.e1);
    }
  });
}

int harts_profile_collect(harts_profile_entry* out, int32_t max_entries, int32_t* n_out) {
  return guarded([&] {
    std::vector<ProfRec> recs;
    {
      std::lock_guard<std::mutex> lk(g_prof_mu);
      recs.swap(g_prof);
    }
    std::map<std::string, harts_profile_entry> agg;
    std::vector<std::string> order;
    hipError_t err = hipSuccess;
    for (auto& r : recs) {
      float ms = 0.f;
      if (err == hipSuccess) err = hipEventSynchronize(r.e1);
      if (err == hipSuccess) err = hipEventElapsedTime(&ms, r.e0, r.e1);
      auto it = agg.find(r.name);
      if (it == agg.end()) {
        harts_profile_entry e{};
        std::strncpy(e.name, r.name, sizeof(e.name) - 1);
        it = agg.emplace(r.name, e).first;
        order.push_back(r.name);
      }
      it->second.launches += 1;
      it->second.total_ms += ms;
      it->second.units += r.units;
      (void)hipEventDestroy(r.e0);
      (void)hipEventDestroy(r.e1);
    }
    hip_check(err, "profile event timing");
    if (n_out) *n_out = int32_t(order.size());
    for (size_t i = 0; i < order.size() && out && int32_t(i) < max_entries; ++i) out[i] = agg[order[i]];
  });
}

}  // extern "C"
