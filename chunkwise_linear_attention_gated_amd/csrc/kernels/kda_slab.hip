// Serial chunk passes with wave-owned value slabs: bf16 matrix-core operands, fp32 state,
// gfx950.
//
// The chunkwise form passes the recurrent state from chunk to chunk (HARTS close-reading
// blog, sections 1.2 and 4.2); boundary states are handed between packed calls and their
// gradients flow back through the handoff (blog, section 4.3).  Per chunk, with the chunk
// quantities of the preparation kernel (W = T (K e^G), U' = T V, K^ = K e^{G_last - G},
// Q~ = Q e^G, M = lower(gated Q K^T), Qeff = Q~ - M W, E = e^{G_last}):
//   forward:    U = U' - W S,   O = Q~ S + M U,    S <- diag(E) S + K^^T U
//   recompute:  the forward's state chain only, writing every chunk-start state
//   gradient:   Y = K^ dS + M^T dO,  dS <- diag(E) dS + Q~^T dO - W^T Y   (reverse over chunks;
//               Qeff^T dO - W^T K^ dS regrouped, Qeff = Q~ - M W)
//
// The value columns of S (and dS) evolve independently.  Each compute wave owns NS slabs of
// 16 value columns of one (sequence, head) and keeps them in accumulator registers for the
// whole sequence.  Every product is arranged so that a pair of result tiles is the next
// product's operand in registers (permuted fragment-major layout, see pf_off): neither the
// state nor U nor Y ever leaves the wave.
//
// Each workgroup has one producer wave besides its NC compute waves.  The producer issues
// every load of a chunk -- the operands shared by all slabs (W, Q~, K^^T, M; K^, Q~^T, W^T, M^T;
// E), the per-slab inputs (U'; dO) and the chunk descriptor -- as direct-to-LDS buffer
// loads into a ring of RD buffers, RD-1 chunks ahead; one workgroup barrier per chunk hands
// a buffer over.  The compute waves never wait on memory: they read LDS, run the matrix
// cores and store their outputs.
//
// W and W^T are stored negated by the preparation kernel, so U' + (-W) S and
// dS + (-W^T) Y accumulate directly on the matrix cores.
#include <stddef.h>

#include "common.h"
#include "launch.h"

namespace harts {

// SLAB_FWDS: the forward that also writes every chunk-start state (what SLAB_REC writes)
enum : int { SLAB_FWD = 0, SLAB_REC = 1, SLAB_DST = 2, SLAB_FWDS = 3 };

template <int MODE, int BT, int D, int DV, int NC, int NS, int RD>
struct SlabCfg {
  static constexpr int KBD = D / 32, KBT = BT / 32, NTT = BT / 16, NTS = D / 16;
  static constexpr int BD = BT * D / 512;                // 1 KiB operand blocks per shared array
  static constexpr bool FO = MODE == SLAB_FWD || MODE == SLAB_FWDS;  // forward outputs
  static constexpr int NARR = MODE == SLAB_REC ? 2 : 3;  // shared [BT][D] arrays
  static constexpr int MB = MODE == SLAB_REC ? 0 : BT * BT / 512;  // M ([BT][BT]) blocks after them
  static constexpr int MOFF = NARR * BD * 1024;
  static constexpr int EOFF = MOFF + MB * 1024;          // E (fp32 [D]), then the chunk descriptor
  static constexpr int SOFF = EOFF + 1024;               // per-slab inputs
  static constexpr int PA = BT * 32;                     // bytes of one per-slab array (BT x 16 x 2 B)
  static constexpr int NPA = 1;                          // per-slab arrays: U' | dO
  static constexpr int SLABS = NC * NS, NGRP = DV / (16 * SLABS);
  static constexpr int BUF = SOFF + SLABS * NPA * PA;    // bytes per ring buffer
  // producer loads per chunk: shared blocks, E, descriptor, per-slab blocks
  static constexpr int NDMA = NARR * BD + MB + 2 + SLABS * NPA * (PA / 1024);
  static constexpr int NW = NC + 1;                      // waves per workgroup
  static_assert(BT % 32 == 0 && D % 32 == 0 && D * 4 + 32 <= 1024, "slab tiling");
  static_assert(DV % (16 * SLABS) == 0 && PA % 1024 == 0, "slab split");
  static_assert(RD * BUF <= 160 * 1024, "LDS ring");
  static_assert(RD == 2 || NDMA <= 63, "loads per chunk within the vector memory counter");
};

__device__ __forceinline__ f32x4 f4_of(bf16x4 v) { return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]}; }
__device__ __forceinline__ bf16x4 b4_of(f32x4 v) { return bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]}; }
__device__ __forceinline__ bf16x4 lo4(bf16x8 v) { return bf16x4{v[0], v[1], v[2], v[3]}; }
__device__ __forceinline__ bf16x4 hi4(bf16x8 v) { return bf16x4{v[4], v[5], v[6], v[7]}; }
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// raw buffer over [p, p + bytes): out-of-range lanes read zero instead of faulting
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, size_t bytes) {
  const int n = bytes >= size_t(0x7fffffff) ? 0x7fffffff : int(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}
// 16 bytes per active lane from rsrc at voff + soff into dst + 16 * lane (LDS)
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, char* dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// s_waitcnt immediate (gfx9 encoding) that waits for vmcnt <= n only
constexpr int vmcnt_only(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

template <int MODE, int BT, int D, int DV, int NC, int NS, int RD>
struct SlabPass {
  using C = SlabCfg<MODE, BT, D, DV, NC, NS, RD>;
  static constexpr int KBD = C::KBD, KBT = C::KBT, NTT = C::NTT, NTS = C::NTS, BD = C::BD;
  static constexpr bool FO = C::FO, SAVE = MODE == SLAB_REC || MODE == SLAB_FWDS;

  const BwdRoundArgs& b;
  int H, h, si, lane, wave, g4, n16, grp;
  SeqDesc sd;
  int own0;
  size_t wbase;  // workspace item of chunk c is wbase + c * H
  int jv0[NS];
  f32x4 S[NS][NTS];  // forward/recompute: S; gradient: dS (state rows x slab columns)

  __device__ __forceinline__ SlabPass(const BwdRoundArgs& b_, int H_) : b(b_), H(H_) {}
  __device__ __forceinline__ size_t wsi(int c) const { return wbase + size_t(c) * H; }
  __device__ __forceinline__ int jv0_of(int sl) const { return 16 * (grp * C::SLABS + sl); }

  // Slot of 16-byte piece L (0..63) of a 1 KiB operand block in the gradient pass's ring: bits 2-3
  // of L flipped by bits 4-5 (an involution).  A transposing read of a fragment touches pieces
  // 16 a + 4 g + b (a, b = 0..3) for each 16-lane group g; unswizzled, the four pieces with the
  // same b share their banks.
  __device__ __forceinline__ static int swz(int L) { return L ^ ((L >> 4) << 2); }

  // ---- producer ---------------------------------------------------------------------------
  struct Src {
    __amdgpu_buffer_rsrc_t arr[3], el, up, m, dO, desc;
  };
  __device__ __forceinline__ void make_src(Src& r) const {
    const RoundArgs& a = b.r;
    const size_t items = size_t(a.nchunk) * H;
    const size_t opb = items * BT * D * 2;
    if constexpr (MODE == SLAB_DST) {
      // the forward's operand layouts, read back transposed (see read_phase)
      r.arr[0] = buf_rsrc(a.ws.KhT, opb);
      r.arr[1] = buf_rsrc(a.ws.Qt, opb);
      r.arr[2] = buf_rsrc(a.ws.W, opb);
      r.m = buf_rsrc(a.ws.Mf, items * BT * BT * 2);
      r.dO = buf_rsrc(b.dO, size_t(0x7fffffff));
    } else {
      r.arr[0] = buf_rsrc(a.ws.W, opb);
      r.arr[1] = buf_rsrc(FO ? a.ws.Qt : a.ws.KhT, opb);
      r.arr[2] = buf_rsrc(a.ws.KhT, opb);
      r.up = buf_rsrc(a.ws.UpT, items * BT * DV * 2);
      r.m = buf_rsrc(FO ? a.ws.Mf : a.ws.UpT, items * BT * BT * 2);
    }
    r.el = buf_rsrc(a.ws.El, items * D * 4);
    r.desc = buf_rsrc(a.chunks, size_t(a.nchunk) * sizeof(ChunkDesc));
  }

  // All loads of chunk c into ring buffer dst: exactly C::NDMA load instructions.
  __device__ __forceinline__ void produce(const Src& r, int c, char* dst) const {
    const size_t w = wsi(c);
    const int vo = lane * 16;
    // the gradient pass reads its operands transposed: its copies place 16-byte piece L of each
    // 1 KiB block at slot swz(L) (see read_phase), so that those reads spread over the banks
    const int vs = (MODE == SLAB_DST ? swz(lane) : lane) * 16;
#pragma unroll
    for (int ar = 0; ar < C::NARR; ++ar)
#pragma unroll
      for (int q = 0; q < BD; ++q) lds_load16(r.arr[ar], dst + (ar * BD + q) * 1024, vs, int(w * BT * D * 2) + q * 1024);
#pragma unroll
    for (int q = 0; q < C::MB; ++q) lds_load16(r.m, dst + C::MOFF + q * 1024, vs, int(w * BT * BT * 2) + q * 1024);
    // E in lanes [0, D/4), the chunk descriptor (32 bytes) in the next two lanes
    constexpr int NE = D / 4;
    if (lane < NE) lds_load16(r.el, dst + C::EOFF, vo, int(w * D * 4));
    if (lane >= NE && lane < NE + 2)
      lds_load16(r.desc, dst + C::EOFF, (lane - NE) * 16, int(size_t(sd.chunk_base + c) * sizeof(ChunkDesc)));
#pragma unroll
    for (int sl = 0; sl < C::SLABS; ++sl) {
      const int j = jv0_of(sl) / 16;
      char* sdst = dst + C::SOFF + sl * C::NPA * C::PA;
      if constexpr (MODE == SLAB_DST) {
        // dO rows of the slab, [token][16 values]; replayed and padding rows read a valid row
        // and are masked by the compute waves
#pragma unroll
        for (int x = 0; x < C::PA / 1024; ++x) {
          const int v = c * BT + 32 * x + (lane >> 1);
          const bool ok = v >= sd.n_replay && v < sd.vlen;
          const int row = ok ? own0 + v - sd.n_replay : own0;
          lds_load16(r.dO, sdst + x * 1024, ((row * H + h) * DV + j * 16 + 8 * (lane & 1)) * 2, 0);
        }
      } else {
        // U' accumulator tiles (token block i, slab j): lane pairs, tile after tile
#pragma unroll
        for (int x = 0; x < C::PA / 1024; ++x) {
          const int i = 2 * x + (lane >> 5);
          lds_load16(r.up, sdst + x * 1024, (i * (DV / 16) + j) * 512 + (lane & 31) * 16, int(w * BT * DV * 2));
        }
      }
    }
  }

  // ---- compute: LDS operand phases ------------------------------------------------------
  // A chunk's products form 2-4 phases of up to 16 operand fragments each (one product:
  // U, Q~ S, S, M U forward; Q~^T dO, M^T dO, K^ dS, W^T Y gradient).  Fragments are ordered
  // contraction slice outer, tile inner, so consecutive matrix-core operations feed independent
  // accumulators; phase p+1 is read from LDS while the matrix cores work through phase p.
  static constexpr int NFT = KBD * NTT;  // token-block products (U, O, Y)
  static constexpr int NFS = KBT * NTS;  // state-tile products (S, Qeff^T dO, W^T Y)
  static constexpr int NFQ = KBT * NTT;  // in-chunk products (M U, M^T dO)
  static constexpr int NFM = NFT > NFS ? NFT : NFS;
  static constexpr int NP = MODE == SLAB_REC ? 2 : 4;
  struct Phase {
    bf16x8 f[NFM];
    f32x4 e[NTS];
  };
  // kind of phase p: 0 token-block product, 1 state-tile product, 2 in-chunk product
  __device__ __forceinline__ static constexpr int phase_kind(int ph) {
    if (MODE == SLAB_DST) return ph == 1 ? 2 : (ph == 2 ? 0 : 1);
    if (MODE == SLAB_REC) return ph;
    return ph < 2 ? 0 : ph - 1;
  }
  __device__ __forceinline__ static constexpr int phase_mfma(int ph) {
    return (phase_kind(ph) == 2 ? NFQ : NFM) * NS;
  }
  __device__ __forceinline__ bf16x8 frag(const char* arr, int blk) const {
    return *reinterpret_cast<const bf16x8*>(arr + (size_t(blk) * 64 + lane) * 16);
  }
  __device__ __forceinline__ void read_phase(int ph, Phase& g, const char* p) const {
    const float* E = reinterpret_cast<const float*>(p + C::EOFF);
    const char* arr;
    bool with_e;
    if constexpr (MODE == SLAB_DST) {
      arr = ph == 1 ? p + C::MOFF : p + (ph == 0 ? 1 : (ph == 2 ? 0 : 2)) * BD * 1024;  // Q~^T, M^T, K^, W^T
      with_e = ph == 0;
    } else {
      arr = p + (phase_kind(ph) == 2 ? C::MOFF : ph * BD * 1024);  // W, [Q~], K^^T, [M]
      with_e = phase_kind(ph) == 1;
    }
    if constexpr (MODE == SLAB_DST) {
      // The gradient's operands are the transposes of the forward's: K^ from K^^T [D][BT], Q~^T
      // and -W^T from Q~ and -W [BT][D], M^T from M [BT][BT], all in the permuted fragment-major
      // layout.  A
      // transposed fragment (rows r0 + lane % 16, contraction k0 + pf_k(lane / 16, 0..7)) is two
      // transposing reads: lane q of a 16-lane group points at 4 consecutive columns r0 + 4 (q % 4)
      // of source row k0 + 4 (lane / 16) + q / 4 (then + 16), and receives column r0 + q of the
      // four rows the group's lanes point at.
      const int q = lane & 15, k4 = 4 * g4 + (q >> 2), r4 = 4 * (q & 3);
      auto at = [&](int k, int r, int K) {
        const int o = 2 * int(pf_off(k, r, K));  // byte offset: 1 KiB block, 16-byte piece, half
        return arr + (o & ~1023) + 16 * swz((o >> 4) & 63) + (o & 15);
      };
      auto tr = [&](int k, int r, int K) {
        const bf16x4 lo = ds_tr16(at(k, r, K)), hi = ds_tr16(at(k + 16, r, K));
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
      if (phase_kind(ph) == 0) {
#pragma unroll
        for (int kb = 0; kb < KBD; ++kb)
#pragma unroll
          for (int i = 0; i < NTT; ++i) g.f[kb * NTT + i] = tr(32 * kb + k4, 16 * i + r4, BT);
      } else if (phase_kind(ph) == 2) {
#pragma unroll
        for (int kb = 0; kb < KBT; ++kb)
#pragma unroll
          for (int i = 0; i < NTT; ++i) g.f[kb * NTT + i] = tr(32 * kb + k4, 16 * i + r4, BT);
      } else {
#pragma unroll
        for (int kb = 0; kb < KBT; ++kb)
#pragma unroll
          for (int t = 0; t < NTS; ++t) g.f[kb * NTS + t] = tr(32 * kb + k4, 16 * t + r4, D);
      }
    } else if (phase_kind(ph) == 0) {
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb)
#pragma unroll
        for (int i = 0; i < NTT; ++i) g.f[kb * NTT + i] = frag(arr, i * KBD + kb);
    } else if (phase_kind(ph) == 2) {
#pragma unroll
      for (int kb = 0; kb < KBT; ++kb)
#pragma unroll
        for (int i = 0; i < NTT; ++i) g.f[kb * NTT + i] = frag(arr, i * KBT + kb);
    } else {
#pragma unroll
      for (int kb = 0; kb < KBT; ++kb)
#pragma unroll
        for (int t = 0; t < NTS; ++t) g.f[kb * NTS + t] = frag(arr, t * KBT + kb);
    }
    if (with_e) {
#pragma unroll
      for (int t = 0; t < NTS; ++t) g.e[t] = *reinterpret_cast<const f32x4*>(E + 16 * t + 4 * g4);
    }
  }
  // prep(ph, g): the phase's elementwise work; mma(ph, g): its matrix-core operations
  template <typename FP, typename FM>
  __device__ __forceinline__ void walk(const char* p, FP&& prep, FM&& mma) {
    Phase g[2];
    read_phase(0, g[0], p);
    sched_fence();
#pragma unroll
    for (int ph = 0; ph < NP; ++ph) {
      if (ph + 1 < NP) read_phase(ph + 1, g[(ph + 1) & 1], p);
      prep(ph, g[ph & 1]);
      mma(ph, g[ph & 1]);
#pragma unroll
      for (int x = 0; x < phase_mfma(ph); ++x) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                        // one matrix-core op
        __builtin_amdgcn_sched_group_barrier(0x100, MODE == SLAB_DST ? 2 : 1, 0);  // its share of LDS reads
      }
      sched_fence();
    }
  }

  // Chunk-start state (or chunk-end state gradient) as bf16 S^T, fragment-major [DV][D], for
  // the gradient kernels; issued once the chunk's products are under way, off the serial chain.
  __device__ __forceinline__ void state_store(bf16* hT, const bf16x8 (&Sf)[NS][KBD]) const {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int t = 0; t < NTS; ++t) {
        const bf16x4 v = (t & 1) ? hi4(Sf[s][t / 2]) : lo4(Sf[s][t / 2]);
        *reinterpret_cast<bf16x4*>(hT + fm_off<bf16>(jv0[s] + n16, 16 * t + 4 * g4, D)) = v;
      }
  }

  // fp32 state slab into pool[idx][h][D][DV]
  __device__ __forceinline__ void store_f32(float* pool, int idx) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int t = 0; t < NTS; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          pool[((size_t(idx) * H + h) * D + 16 * t + 4 * g4 + r) * DV + jv0[s] + n16] = S[s][t][r];
  }

  __device__ __forceinline__ const char* slab_in(const char* p, int s) const {
    return p + C::SOFF + (wave * NS + s) * C::NPA * C::PA;
  }
  // the emitted-state index of the chunk whose loads are in ring buffer p (uniform)
  __device__ __forceinline__ int emit_of(const char* p) const {
    const int* d = reinterpret_cast<const int*>(p + C::EOFF + D * 4);
    return __builtin_amdgcn_readfirstlane(d[offsetof(ChunkDesc, emit) / 4]);
  }

  __device__ __forceinline__ void compute_fwd(int c, const char* p) {
    const RoundArgs& a = b.r;
    const int emit = FO ? emit_of(p) : -1;
    bf16x8 Sf[NS][KBD];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) Sf[s][kb] = pf_pair(S[s][2 * kb], S[s][2 * kb + 1]);
    f32x4 U[NS][NTT];
    f32x4 O[FO ? NS : 1][NTT];
    bf16x8 Uf[NS][KBT];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const char* in = slab_in(p, s);
#pragma unroll
      for (int i = 0; i < NTT; ++i) {
        U[s][i] = f4_of(*reinterpret_cast<const bf16x4*>(in + i * 512 + lane * 8));
        if constexpr (FO) O[s][i] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    walk(
        p,
        [&](int ph, const Phase& g) {
          if (phase_kind(ph) == 1) {
            // S <- diag(E) S (+ K^^T U below)
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
              for (int k2 = 0; k2 < KBT; ++k2) Uf[s][k2] = pf_pair(U[s][2 * k2], U[s][2 * k2 + 1]);
#pragma unroll
            for (int t = 0; t < NTS; ++t)
#pragma unroll
              for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int r = 0; r < 4; ++r) S[s][t][r] *= g.e[t][r];
          }
        },
        [&](int ph, const Phase& g) {
          if (phase_kind(ph) == 0 && ph == 0) {
            // U = U' + (-W) S
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb)
#pragma unroll
              for (int i = 0; i < NTT; ++i)
#pragma unroll
                for (int s = 0; s < NS; ++s) U[s][i] = mfma_bf16(g.f[kb * NTT + i], Sf[s][kb], U[s][i]);
          } else if (phase_kind(ph) == 0) {
            // O^T = S^T Q~^T
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb)
#pragma unroll
              for (int i = 0; i < NTT; ++i)
#pragma unroll
                for (int s = 0; s < NS; ++s) O[s][i] = mfma_bf16(Sf[s][kb], g.f[kb * NTT + i], O[s][i]);
          } else if (phase_kind(ph) == 2) {
            // O^T += U^T M^T: the bf16 U fragments of the state update are U^T's operand
            // registers in the same contraction order as M's fragments
#pragma unroll
            for (int kb = 0; kb < KBT; ++kb)
#pragma unroll
              for (int i = 0; i < NTT; ++i)
#pragma unroll
                for (int s = 0; s < NS; ++s) O[s][i] = mfma_bf16(Uf[s][kb], g.f[kb * NTT + i], O[s][i]);
          } else {
#pragma unroll
            for (int kb = 0; kb < KBT; ++kb)
#pragma unroll
              for (int t = 0; t < NTS; ++t)
#pragma unroll
                for (int s = 0; s < NS; ++s) S[s][t] = mfma_bf16(g.f[kb * NTS + t], Uf[s][kb], S[s][t]);
          }
        });
    if constexpr (SAVE) {
      const size_t w = wsi(c);
      state_store(static_cast<bf16*>(a.h) + w * DV * D, Sf);
    }
    if constexpr (FO) {
      // own rows only (replayed rows and padding store into the sink)
      bf16* og = static_cast<bf16*>(a.o);
#pragma unroll
      for (int i = 0; i < NTT; ++i) {
        const int v = c * BT + 16 * i + n16;
        const bool ok = og && v >= sd.n_replay && v < sd.vlen;
        const size_t row = size_t(own0 + v - sd.n_replay);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          bf16* dst = ok ? og + (row * H + h) * DV + jv0[s] + 4 * g4
                         : static_cast<bf16*>(a.sink) + ((lane + 64 * (s + NS * i)) * 4) % kSinkElems<bf16>();
          *reinterpret_cast<bf16x4*>(dst) = b4_of(O[s][i]);
        }
      }
      if (emit >= 0 && a.emit_pool) store_f32(a.emit_pool, emit);
    }
  }

  __device__ __forceinline__ void compute_dst(int c, const char* p) {
    const int emit = emit_of(p);
    // gradient of the state emitted after this chunk (summed over its consumers beforehand)
    if (emit >= 0 && b.dslot) {
      const float* sg = b.dslot + (size_t(emit) * H + h) * D * DV;
      float add[NS][NTS][4];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int t = 0; t < NTS; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) add[s][t][r] = sg[size_t(16 * t + 4 * g4 + r) * DV + jv0[s] + n16];
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int t = 0; t < NTS; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) S[s][t][r] += add[s][t][r];
    }
    bf16x8 Sf[NS][KBD];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int kb = 0; kb < KBD; ++kb) Sf[s][kb] = pf_pair(S[s][2 * kb], S[s][2 * kb + 1]);
    // dO fragments: tokens 32 kb + pf_k(g4, t) at the slab's column n16, by two transposing
    // LDS reads per 32-token block (within each 16-lane group, result element j of lane s is
    // element s % 4 of the 8 bytes that lane 4 j + s / 4 points at); replayed rows carry no
    // output gradient here, padding rows none at all
    bf16x8 dof[NS][KBT];
    const bool masked = c * BT < sd.n_replay || (c + 1) * BT > sd.vlen;  // uniform
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const char* rows = slab_in(p, s);
#pragma unroll
      for (int kb = 0; kb < KBT; ++kb) {
        const int o = kb * 1024 + (4 * g4 + (n16 >> 2)) * 32 + (n16 & 3) * 8;
        const bf16x4 lo = ds_tr16(rows + o), hi = ds_tr16(rows + o + 16 * 32);
        dof[s][kb] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if (masked) {
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int v = c * BT + 32 * kb + pf_k(g4, t);
            if (!(v >= sd.n_replay && v < sd.vlen)) dof[s][kb][t] = (bf16)0.f;
          }
        }
      }
    }
    f32x4 Y[NS][NTT];
    bf16x8 Yf[NS][KBT];
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int i = 0; i < NTT; ++i) Y[s][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    walk(
        p,
        [&](int ph, const Phase& g) {
          if (ph == 0) {
            // dS <- diag(E) dS (+ Q~^T dO below)
#pragma unroll
            for (int t = 0; t < NTS; ++t)
#pragma unroll
              for (int s = 0; s < NS; ++s)
#pragma unroll
                for (int r = 0; r < 4; ++r) S[s][t][r] *= g.e[t][r];
          } else if (ph == 3) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
#pragma unroll
              for (int k2 = 0; k2 < KBT; ++k2) Yf[s][k2] = pf_pair(Y[s][2 * k2], Y[s][2 * k2 + 1]);
          }
        },
        [&](int ph, const Phase& g) {
          if (ph == 0) {
#pragma unroll
            for (int kb = 0; kb < KBT; ++kb)
#pragma unroll
              for (int t = 0; t < NTS; ++t)
#pragma unroll
                for (int s = 0; s < NS; ++s) S[s][t] = mfma_bf16(g.f[kb * NTS + t], dof[s][kb], S[s][t]);
          } else if (ph == 1) {
            // Y = M^T dO
#pragma unroll
            for (int kb = 0; kb < KBT; ++kb)
#pragma unroll
              for (int i = 0; i < NTT; ++i)
#pragma unroll
                for (int s = 0; s < NS; ++s) Y[s][i] = mfma_bf16(g.f[kb * NTT + i], dof[s][kb], Y[s][i]);
          } else if (ph == 2) {
            // Y += K^ dS(chunk end)
#pragma unroll
            for (int kb = 0; kb < KBD; ++kb)
#pragma unroll
              for (int i = 0; i < NTT; ++i)
#pragma unroll
                for (int s = 0; s < NS; ++s) Y[s][i] = mfma_bf16(g.f[kb * NTT + i], Sf[s][kb], Y[s][i]);
          } else {
            // dS += (-W^T) Y
#pragma unroll
            for (int kb = 0; kb < KBT; ++kb)
#pragma unroll
              for (int t = 0; t < NTS; ++t)
#pragma unroll
                for (int s = 0; s < NS; ++s) S[s][t] = mfma_bf16(g.f[kb * NTS + t], Yf[s][kb], S[s][t]);
          }
        });
    const size_t w = wsi(c);
    state_store(static_cast<bf16*>(b.dh) + w * DV * D, Sf);
  }
};

template <int MODE, int BT, int D, int DV, int NC, int NS, int RD>
__global__ __launch_bounds__(64 * (NC + 1)) void kda_slab_kernel(BwdRoundArgs b, int H) {
  using P = SlabPass<MODE, BT, D, DV, NC, NS, RD>;
  using C = typename P::C;
  __shared__ __attribute__((aligned(1024))) char ring[RD * C::BUF];
  const RoundArgs& a = b.r;
  P x(b, H);
  // the workgroups of one (sequence, head) pair sit on one XCD; the pairs in the round's launch order
  const int lb = xcd_logical(blockIdx.x, gridDim.x);
  x.grp = lb % C::NGRP;
  const int us = lb / C::NGRP;
  if (us >= a.nseq * H) return;
  const int u = a.units ? a.units[us] : us;
  x.h = u % H;
  x.si = u / H;
  x.lane = threadIdx.x & 63;
  x.wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  x.g4 = x.lane >> 4;
  x.n16 = x.lane & 15;
  x.sd = a.seqs[x.si];
  const int N = x.sd.n_chunks;
  x.own0 = x.sd.vlen > x.sd.n_replay ? a.vrows[x.sd.vbase + x.sd.n_replay] : 0;
  x.wbase = size_t(x.sd.chunk_base) * H + x.h;
  // step k handles chunk c(k): forward order, or reverse for the state gradient
  auto chunk_of = [&](int k) {
    const int kk = k < N ? k : N - 1;
    return MODE == SLAB_DST ? N - 1 - kk : kk;
  };

  if (x.wave == NC) {
    // producer: the loads of chunk c(k + RD - 1) while the compute waves work on c(k)
    typename P::Src src;
    x.make_src(src);
    if (N > 0) {
#pragma unroll
      for (int k = 0; k + 1 < RD; ++k) x.produce(src, chunk_of(k), ring + k * C::BUF);
    }
    for (int k = 0; k < N; ++k) {
      // chunk c(k)'s loads have landed (only the RD-2 newer batches may be in flight)
      __builtin_amdgcn_s_waitcnt(vmcnt_only((RD - 2) * C::NDMA));
      wg_barrier();
      // every compute wave is past chunk c(k-1): its buffer takes chunk c(k + RD - 1)
      x.produce(src, chunk_of(k + RD - 1), ring + ((k + RD - 1) % RD) * C::BUF);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the workgroup's LDS outlives every load
    return;
  }

  // compute waves
#pragma unroll
  for (int s = 0; s < NS; ++s) x.jv0[s] = x.jv0_of(x.wave * NS + s);
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int t = 0; t < C::NTS; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = 0.f;
        if (MODE != SLAB_DST && x.sd.init >= 0)
          v = a.init_pool[((size_t(x.sd.init) * H + x.h) * D + 16 * t + 4 * x.g4 + r) * DV + x.jv0[s] + x.n16];
        x.S[s][t][r] = v;
      }
  for (int k = 0; k < N; ++k) {
    wg_barrier();
    const char* p = ring + (k % RD) * C::BUF;
    if constexpr (MODE == SLAB_DST) x.compute_dst(chunk_of(k), p);
    else x.compute_fwd(chunk_of(k), p);
  }
  if constexpr (P::FO) {
    if (x.sd.final_idx >= 0 && a.final_pool) x.store_f32(a.final_pool, x.sd.final_idx);
  }
  if constexpr (MODE == SLAB_DST) {
    if (b.dinit) x.store_f32(b.dinit, a.seq0 + x.si);
  }
}

// Gradient of each handed-off state produced in a round: the sum, in consumer order, of the
// initial-state gradients of the sequences that start from it (all in later rounds).
__global__ __launch_bounds__(256) void slot_grad_kernel(const int32_t* slots, const int32_t* cons_off,
                                                        const int32_t* cons, const float* dinit, float* out,
                                                        int64_t per) {
  const int slot = slots[blockIdx.y];
  const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= per) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int q = cons_off[slot]; q < cons_off[slot + 1]; ++q) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(dinit + int64_t(cons[q]) * per + i);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += v[r];
  }
  *reinterpret_cast<f32x4*>(out + int64_t(slot) * per + i) = acc;
}

hipError_t launch_slot_grad(const KdaDims& d, const int32_t* slots, int32_t nslots, const int32_t* cons_off,
                            const int32_t* cons, const float* dinit, float* out, hipStream_t s) {
  if (nslots <= 0) return hipSuccess;
  const int64_t per = int64_t(d.H) * d.D * d.DV;  // a multiple of 4 for every supported shape
  dim3 grid(unsigned((per / 4 + 255) / 256), unsigned(nslots));
  hipLaunchKernelGGL(slot_grad_kernel, grid, dim3(256), 0, s, slots, cons_off, cons, dinit, out, per);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
template <int MODE, int BT, int D, int DV, int NC, int NS, int RD>
static hipError_t slab_go(const KdaDims& d, const BwdRoundArgs& b, hipStream_t s) {
  using C = SlabCfg<MODE, BT, D, DV, NC, NS, RD>;
  unsigned n = unsigned(b.r.nseq) * d.H * C::NGRP;
  n = (n + 7) / 8 * 8;
  hipLaunchKernelGGL((kda_slab_kernel<MODE, BT, D, DV, NC, NS, RD>), dim3(n), dim3(64 * C::NW), 0, s, b, d.H);
  return hipGetLastError();
}

// Two compute waves of two slabs each per workgroup, sharing one ring: every wave has a SIMD
// (and its registers) to itself, the shared operands are read from LDS once per two slabs, and a
// (sequence, head) pair takes two compute units.  Only a round too small to matter for the rest
// of the chip (at most a quarter of the compute units' worth of slabs) runs one slab per
// workgroup, for the shortest chain latency; a larger round shares the chip with the per-chunk
// kernels of other rounds, and packing its chains onto fewer compute units leaves them more.
// A forward round of at most half the compute units' worth of slabs (a long root sequence)
// runs one compute wave of two slabs per workgroup: the same chain per wave on twice the
// compute units, each wave with its ring and LDS to itself.  The recompute pass of a round of
// many sequences (more than twice the compute units' worth of slabs) runs a whole head per
// workgroup, four compute waves of two slabs: its two shared arrays are loaded once per head
// instead of twice, and half as many workgroups take compute units from the concurrent passes
// (the forward and gradient modes, with four more operand arrays per chunk, lose more to LDS
// traffic and register spills at that size than they save).  A head of 32 value columns runs its
// two slabs on one compute wave.
template <int MODE, int BT, int D, int DV>
static hipError_t slab_pick(const KdaDims& d, const BwdRoundArgs& b, hipStream_t s) {
  const unsigned slabs = unsigned(b.r.nseq) * d.H * (DV / 16);
  constexpr bool FWD = MODE == SLAB_FWD || MODE == SLAB_FWDS;
  // (the forward's and the gradient's ring buffers also hold M: two of them fit)
  constexpr int RD1 = MODE == SLAB_REC ? 3 : 2;
  const unsigned cus = persistent_grid(1u << 30);
  if (4 * slabs <= cus) return slab_go<MODE, BT, D, DV, 1, 1, RD1>(d, b, s);
  if constexpr (DV < 64) {
    return slab_go<MODE, BT, D, DV, 1, 2, 2>(d, b, s);  // two slabs: the whole head
  } else {
    if (FWD && 2 * slabs <= cus) return slab_go<MODE, BT, D, DV, 1, 2, 2>(d, b, s);
    if constexpr (DV == 128 && MODE == SLAB_REC) {
      if (slabs > 2 * cus) return slab_go<MODE, BT, D, DV, 4, 2, 2>(d, b, s);
    }
    return slab_go<MODE, BT, D, DV, 2, 2, 2>(d, b, s);
  }
}

template <int BT, int D, int DV>
static hipError_t slab_mode(const KdaDims& d, const BwdRoundArgs& b, int mode, hipStream_t s) {
  if (b.r.nseq <= 0) return hipSuccess;
  if (mode == SLAB_FWD) return slab_pick<SLAB_FWD, BT, D, DV>(d, b, s);
  if (mode == SLAB_FWDS) return slab_pick<SLAB_FWDS, BT, D, DV>(d, b, s);
  if (mode == SLAB_REC) return slab_pick<SLAB_REC, BT, D, DV>(d, b, s);
  return slab_pick<SLAB_DST, BT, D, DV>(d, b, s);
}

#define HARTS_SLAB_CONFIGS(X) \
  X(64, 128, 128)             \
  X(64, 64, 64)               \
  X(32, 64, 64)               \
  X(32, 32, 32)

bool kda_slab_supported(const KdaDims& d) {
#define X(B_, D_, V_) \
  if (d.dtype == 0 && d.BT == B_ && d.D == D_ && d.DV == V_) return true;
  HARTS_SLAB_CONFIGS(X)
#undef X
  return false;
}

hipError_t launch_kda_slab(const KdaDims& d, const BwdRoundArgs& b, int mode, int, hipStream_t s) {
#define X(B_, D_, V_) \
  if (d.dtype == 0 && d.BT == B_ && d.D == D_ && d.DV == V_) return slab_mode<B_, D_, V_>(d, b, mode, s);
  HARTS_SLAB_CONFIGS(X)
#undef X
  return hipErrorNotSupported;
}

}  // namespace harts
