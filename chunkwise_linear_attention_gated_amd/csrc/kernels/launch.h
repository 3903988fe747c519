// Host-callable launchers of the HIP kernels (one packed round at a time).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../desc.h"

namespace harts {

// Per-chunk-head workspace produced by the prep kernel and consumed by the
// serial state / state-gradient passes.  Element offsets are
// [local chunk][head][...]; every array holds the plan dtype except El.
struct ChunkWs {
  void* W;      // [BT][D]   W = T (K * e^G)                      (token-major)
  void* UpT;    // [DV][BT]  (T V)^T
  void* KhT;    // [D][BT]   (K * e^{G_last - G})^T
  void* Qt;     // [BT][D]   Q~ = Q * e^G                          (forward)
  void* Mm;     // [BT][BT]  M = lower(gated Q K^T)
  float* El;    // [D]       e^{G_last}
  void* QeffT;  // [D][BT]   (Q~ - M W)^T                          (backward, fp32 path)
  void* WT;     // [D][BT]   W^T                                   (backward, fp32 path)
  void* Kh;     // [BT][D]   K * e^{G_last - G}                    (backward, fp32 path)
  void* Tm;     // [BT][BT]  T = X diag(beta)                      (backward)
  void* Xm;     // [BT][BT]  X = (I + diag(beta) A)^{-1}           (backward)
  void* Am;     // [BT][BT]  A (strictly lower)                    (backward)
  void* Mf;     // [BT][BT]  M, permuted fragment-major             (bf16 slab passes)
};

struct KdaDims {
  int H, D, DV, BT, dtype;  // dtype: 0 bf16, 1 fp32
};

struct RoundArgs {
  const int32_t* vrows;       // global virtual-row table
  const SeqDesc* seqs;        // this round's sequences
  const ChunkDesc* chunks;    // this round's chunks
  const int32_t* crows;       // [chunk][BT] compact row of every chunk row, -1 past the chunk's end
  int32_t nseq, nchunk;
  int32_t seq0;               // global index of this round's first sequence
  const void *q, *k, *v, *g, *beta;
  void* o;                    // forward output [N][H][DV] (nullable)
  const float* init_pool;     // initial states by SeqDesc::init
  float* emit_pool;           // emitted states by ChunkDesc::emit
  float* final_pool;          // final states by SeqDesc::final_idx
  ChunkWs ws;
  void* sink;                 // >= 64 KiB that lanes with nothing to store write into: stores stay
                              // unconditional, so the wait counters see the same count on every path
  void* h;                    // backward: S_n^T per chunk [chunk][H][DV][D] (nullable)
  void* hc;                   // backward: S_n per chunk, channel-major [chunk][H][D][DV] (nullable)
  int* ctr;                   // zeroed item counter of this launch of a persistent per-chunk kernel
                              // (nullable: static item order)
  int* zero;                  // preparation kernel: item counters that its block 0 clears for the
  int32_t nzero;              // launches ordered after it (nullable)
  const int32_t* units;       // serial passes: this round's (sequence, head) pairs s * H + h in
                              // launch order (nullable: natural order)
};

struct BwdRoundArgs {
  RoundArgs r;
  const void* dO;             // [N][H][DV]
  void *dq, *dk, *dv, *dg, *dbeta;
  void* dh;                   // dS at chunk ends, [chunk][H][DV][D]
  void* dhc;                  // dS at chunk ends, channel-major [chunk][H][D][DV]
  float* dinit;               // per-sequence dL/d(initial state) [global seq][H][D][DV]
  float* dstates;             // per-slot gradient output (nullable)
  const int32_t* slot_cons_off;  // CSR of consumer sequences per slot (nullable for varlen)
  const int32_t* slot_cons;
  float* replay_grad;         // [replay_total][H][2*D + DV + 1] fp32 (dk, dv, dg, dbeta of replayed rows)
  const float* dslot;         // slab passes: gradient of every handed-off state, summed over its
                              // consumers before the producing round runs (nullable)
};

// Grid of a persistent per-chunk kernel: one workgroup per compute unit of the
// current device (at most one item per workgroup when there are fewer items).
inline unsigned persistent_grid(unsigned items) {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return items < unsigned(cus[dev]) ? items : unsigned(cus[dev]);
}

// mode 0 forward operands, 1 backward operands, 2 both (bf16)
hipError_t launch_kda_prep(const KdaDims& d, const RoundArgs& a, int mode, hipStream_t s);
hipError_t launch_kda_state(const KdaDims& d, const RoundArgs& a, bool backward, hipStream_t s);
// Slab-parallel serial passes (bf16 operands): mode 0 forward, 1 backward state recompute,
// 2 state gradient, 3 forward that also writes every chunk-start state (a.h, a.hc).  Returns hipErrorNotSupported for configurations they do not cover.
bool kda_slab_supported(const KdaDims& d);
// out[slot] = sum over the slot's consumer sequences of dinit[consumer], for the listed slots
hipError_t launch_slot_grad(const KdaDims& d, const int32_t* slots, int32_t nslots, const int32_t* cons_off,
                            const int32_t* cons, const float* dinit, float* out, hipStream_t s);
hipError_t launch_kda_slab(const KdaDims& d, const BwdRoundArgs& b, int mode, int round_max_chunks, hipStream_t s);
hipError_t launch_kda_dstate(const KdaDims& d, const BwdRoundArgs& a, hipStream_t s);
hipError_t launch_kda_grad(const KdaDims& d, const BwdRoundArgs& a, hipStream_t s);
hipError_t launch_replay_fixup(const KdaDims& d, const int32_t* fix_rows, const int32_t* fix_off,
                               const int32_t* fix_idx, int32_t nrows, const float* replay_grad, void* dk, void* dv,
                               void* dg, void* dbeta, hipStream_t s);
bool kda_supported(const KdaDims& d);

// p[0..n) = 0 on stream s
hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t s);
hipError_t launch_logprob(const void* logits, int64_t C, int64_t V, int dtype, const int64_t* m, const int32_t* labels,
                          int64_t S, float* logp, int32_t* q, float* lse, hipStream_t s);
// The same gather with lse in the library's own per-device array of kLogprobStaticRows floats
// (hipErrorInvalidValue when C exceeds it); allocates nothing.
constexpr int64_t kLogprobStaticRows = int64_t(1) << 20;
hipError_t launch_logprob_static(const void* logits, int64_t C, int64_t V, int dtype, const int64_t* m,
                                 const int32_t* labels, int64_t S, float* logp, int32_t* q, hipStream_t s);
// Tree softmax attention (attn.hip).  which: 0 forward, 1 delta = <dout, o>, 2 dq, 3 dk and dv.
struct AttnArgs {
  const __bf16 *q, *k, *v, *o, *dout;
  const float *lse, *delta;
  const int32_t *tiles, *list;  // query tiles + kv lists (0, 2) or key tiles + q lists (3)
  __bf16 *o_out, *dq, *dk, *dv;
  float *lse_out, *delta_out;
  int64_t C;
  int32_t H;
  float scale;
};
bool attn_dims_supported(int dqk, int dv);
hipError_t launch_attn(int which, const AttnArgs& a, int64_t n_tiles, int dqk, int dv, hipStream_t s);

// Multiplicity-weighted router statistics (moe.hip).  which: 0 statistics, 1 gradient.
struct MoeArgs {
  const float* z;      // [C][E] router logits
  const float* bias;   // [E] or null
  const int32_t* q;    // [C] multiplicities
  int32_t* top;        // [C][k]
  float* lse;          // [C]
  int32_t* counts;     // [E] (statistics: written; gradient: read)
  float* part;         // workspace: [moe_partial_rows(C)][E + 1] float, then [..][E] int32
  float* mass;         // [E]
  float* losses;       // [2]: L_z, L_aux
  float* dz;           // [C][E]
  int64_t C, S;
  int32_t E, k;
  float z_coef, aux_coef;
};
int64_t moe_partial_rows(int64_t C);
hipError_t launch_moe(int which, const MoeArgs& a, hipStream_t s);
hipError_t launch_moe_bias(const int32_t* counts, int E, float gamma, float* bias, hipStream_t s);

size_t conv_workspace_bytes(int64_t C, int32_t ch, int32_t w);
hipError_t launch_conv_fwd(const void* x, const float* wt, const int32_t* anc, int64_t C, int32_t ch, int32_t w,
                           int dtype, void* out, hipStream_t s);
hipError_t launch_conv_bwd(const void* x, const float* wt, const int32_t* anc, const int64_t* goff, const int64_t* gl,
                           const void* dout, int64_t C, int32_t ch, int32_t w, int dtype, void* dx, float* dw,
                           float* part, hipStream_t s);
hipError_t launch_logprob_bwd(const void* logits, int64_t C, int64_t V, int dtype, const float* lse,
                              const int64_t* row_off, const int64_t* row_pos, const int32_t* labels, const float* dlogp,
                              void* dlogits, hipStream_t s);

}  // namespace harts
