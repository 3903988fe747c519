// Device descriptors of a packed chunkwise plan, shared by the host planner
// and the HIP kernels.  Plain 32-byte PODs, int32 fields.
//
// A round is one packed varlen call.  Its sequences are laid out as a
// *virtual stream*: the replayed ancestor rows (fewer than B) followed by the
// sequence's own compact rows, starting at the chunk boundary a(s_head), so
// the chunk partition of every sequence is that of trajectory-wise execution
// (HARTS close-reading blog, section 4.2, replay; section 4.3, compact layout).
// `vrows` maps every virtual position of every round to its compact row.
#pragma once
#include <stdint.h>

namespace harts {

struct SeqDesc {
  int32_t vbase;       // first virtual position (index into vrows)
  int32_t vlen;        // virtual stream length (replay + own)
  int32_t n_replay;    // replayed rows at the front of the stream (< B)
  int32_t chunk_base;  // round-local index of the sequence's first chunk
  int32_t n_chunks;    // ceil(vlen / B)
  int32_t init;        // state index of the initial state, -1 = zero state
  int32_t final_idx;   // final-state output index, -1 = none
  int32_t replay_base; // global replay index of the first replayed row
};

struct ChunkDesc {
  int32_t seq;         // global sequence index
  int32_t vbase;       // virtual position of the chunk's first token
  int32_t len;         // tokens in the chunk (1..B)
  int32_t own_from;    // positions [0, own_from) of the chunk are replayed rows
  int32_t cidx;        // chunk index within its sequence
  int32_t emit;        // state index written after this chunk, -1 = none
  int32_t local;       // chunk index within its round (workspace slot)
  int32_t replay_base; // global replay index of the chunk's first position (valid when own_from > 0)
};

static_assert(sizeof(SeqDesc) == 32, "SeqDesc layout");
static_assert(sizeof(ChunkDesc) == 32, "ChunkDesc layout");

}  // namespace harts
