// Chunkwise gated-delta backward on gfx950, one packed round at a time, rounds
// in reverse (HARTS close-reading blog, section 4.3: differentiable state
// handoff -- initial-state gradients flow back into the call that produced the
// boundary; paperlayer summary, section 4: recomputation under the fixed plan).
//
// Per chunk with start state S0, end-state gradient dS (both known after the
// serial passes), L = <dO, O> + <dS, S_end>:
//   dU = M^T dO + K^ dS,  dR = T^T dU  (dV = dR),  dT = dU R^T,  R = V - K~ S0,
//   dX = dT diag(beta),  dL = -X^T dX X^T,  dA = strict_lower(diag(beta) dL),
//   dbeta_j = sum_i X_ij dT_ij + sum_k dL_jk A_jk,   dM = lower(dO U^T),
//   dS_start = diag(e^{G_last}) dS + Qeff^T dO - W^T (K^ dS),  Qeff = Q~ - M W,
// and the q, k, g gradients through the gated token products (e^{G_i - G_j}
// factored at 16-row sub-block references, as in the forward):
//   dq = e^L (rowgated(dM, K) + e^{F_b} dO S0^T)
//   dk = e^L (rowgated(dA, K) - e^{F_b} dR S0^T) + colgated(dM, Q) + colgated(dA, K) + K^-factor (U dS^T)
//   dG = q dq + k (row-side terms) - k (column-side terms);  dG_last += sum_i k^ (U dS^T) + e^{G_last} rowsum(dS S0)
//   dg = reverse cumulative sum of dG over the chunk.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "state_common.h"

namespace harts {

template <int DV> constexpr int dv_tile_b() { return DV; }  // one workgroup per (sequence, head)

// Replay-gradient side buffer: per (replay position, head) dk[D], dv[DV], dg[D], dbeta.
template <int D, int DV> struct RG {
  static constexpr int W = 2 * D + DV + 1, DK = 0, DVO = D, DG = D + DV, DB = 2 * D + DV;
};

// ------------------------------------------------------------------------------------------
// Serial state-gradient pass, reverse over chunks.  One workgroup of SNW waves per
// (sequence, head, value-column tile of DVT).  dS (fp32) lives in accumulator registers
// (wave w owns rows 16w..).  Per chunk:  Y = K^ dS;  dS <- diag(e^{G_last}) dS + Qeff^T dO - W^T Y.
// The left operands (K^, W^T, Qeff^T) are register fragments read from their fragment-major
// workspace layouts one chunk ahead; dO is staged transposed into LDS one chunk ahead
// (double-buffered), so Qeff^T dO is formed off the chain and a step is
// dS -> LDS -> barrier -> Y -> LDS -> barrier -> dS.
template <typename T, int BT, int D, int DV, int DVT>
struct DStateOps {
  using MM = Mma<T>;
  using F = typename MM::Frag;
  using TL = StateTiles<BT, D, DVT>;
  static constexpr int NTH = 64 * TL::NW, VN = 16 / sizeof(T);
  static constexpr int KD = D / MM::KS, KB = BT / MM::KS;
  static constexpr int NO = (BT * (DVT / VN) + NTH - 1) / NTH;  // dO pieces per thread
  F kh[KD];                // K^ (token-major) fragments of this wave's token block
  F wt[TL::MU][KB];        // W^T fragments of this wave's dS rows
  F qe[TL::MU][KB];        // Qeff^T fragments of this wave's dS rows
  float el[TL::MU][4];     // e^{G_last} of this lane's dS rows
  int emit;                // slot emitted after this chunk (-1: none)
  f32x4 dov[NO];           // dO pieces of the chunk before this one (staged one step ahead)
};
template <typename T, int BT, int D, int DV, int DVT>
struct DStateRows {
  int r[DStateOps<T, BT, D, DV, DVT>::NO];
};

template <typename T, int BT, int D, int DV, int DVT>
__device__ __forceinline__ void load_dstate_rows(DStateRows<T, BT, D, DV, DVT>& o, const RoundArgs& a, int chunk,
                                                 int tid) {
  using Ops = DStateOps<T, BT, D, DV, DVT>;
#pragma unroll
  for (int x = 0; x < Ops::NO; ++x) {
    const int i = (tid + Ops::NTH * x) / (DVT / Ops::VN);
    o.r[x] = a.crows[size_t(chunk) * BT + (i < BT ? i : BT - 1)];
  }
}

template <typename T, int BT, int D, int DV, int DVT>
__device__ __forceinline__ void load_dstate_dov(f32x4* dov, const DStateRows<T, BT, D, DV, DVT>& rw, const T* gdo,
                                                int H, int h, int tid, int jvb) {
  using Ops = DStateOps<T, BT, D, DV, DVT>;
#pragma unroll
  for (int x = 0; x < Ops::NO; ++x) {
    const int j0 = ((tid + Ops::NTH * x) % (DVT / Ops::VN)) * Ops::VN;
    const int row = rw.r[x] >= 0 ? rw.r[x] : 0;
    dov[x] = ldq(gdo + (size_t(row) * H + h) * DV + jvb + j0);
  }
}

// Unconditional loads from clamped addresses; padding and replayed rows are masked at use.
template <typename T, int BT, int D, int DV, int DVT>
__device__ __forceinline__ void load_dstate_ops(DStateOps<T, BT, D, DV, DVT>& o, const RoundArgs& a, int chunk, int H,
                                                int h, int wave, int lane, int z) {
  using Ops = DStateOps<T, BT, D, DV, DVT>;
  using TL = typename Ops::TL;
  const size_t wsi = size_t(chunk) * H + h;
  const T* khg = static_cast<const T*>(a.ws.Kh) + wsi * BT * D;
  const T* wtg = static_cast<const T*>(a.ws.WT) + wsi * D * BT;
  const T* qeg = static_cast<const T*>(a.ws.QeffT) + wsi * D * BT;
  const float* el = a.ws.El + wsi * D;
  const int mi = wave / TL::WPB;
  o.emit = a.chunks[chunk + z].emit;
#pragma unroll
  for (int kk = 0; kk < Ops::KD; ++kk) o.kh[kk] = fm_frag<T>(khg, D, mi, kk, lane);
#pragma unroll
  for (int u = 0; u < TL::MU; ++u) {
    const int mt = wave + TL::NW * u, mc = mt < TL::MT ? mt : 0;
#pragma unroll
    for (int kk = 0; kk < Ops::KB; ++kk) {
      o.wt[u][kk] = fm_frag<T>(wtg, BT, mc, kk, lane);
      o.qe[u][kk] = fm_frag<T>(qeg, BT, mc, kk, lane);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) o.el[u][r] = el[16 * mc + crow(lane, r)];
  }
}

template <typename T, int BT, int D, int DV, int DVT>
__global__ __launch_bounds__(64 * state_waves<D>()) void kda_dstate_kernel(BwdRoundArgs b, int H) {
  using MM = Mma<T>;
  using Ops = DStateOps<T, BT, D, DV, DVT>;
  using TL = typename Ops::TL;
  using Rows = DStateRows<T, BT, D, DV, DVT>;
  const RoundArgs& a = b.r;
  constexpr int NW = TL::NW, NTH = Ops::NTH, NTL = DV / DVT, PAD = 16 / sizeof(T), VN = Ops::VN;
  constexpr int LDS_S = D + PAD, LDJ = BT + PAD;
  constexpr int MT = TL::MT, NTV = TL::NTV, MU = TL::MU, NTU = TL::NTU, NO = Ops::NO;
  __shared__ __attribute__((aligned(16))) T dSt[DVT * LDS_S];
  __shared__ __attribute__((aligned(16))) T Yt[DVT * LDJ];
  __shared__ __attribute__((aligned(16))) T dOt[2][DVT * LDJ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lb = xcd_logical(blockIdx.x, gridDim.x);
  const int tile = lb % NTL, h = (lb / NTL) % H, si = lb / (NTL * H);
  if (si >= a.nseq) return;
  const SeqDesc sd = a.seqs[si];
  const int jvb = tile * DVT;
  const int mi = wave / TL::WPB, nt0 = (wave % TL::WPB) * NTU;  // this wave's token block and tile columns
  const T* gdo = static_cast<const T*>(b.dO);
  const int N = sd.n_chunks, c0 = sd.chunk_base;
  auto chunk_at = [&](int n) { return c0 + (n > 0 ? n : 0); };
  // dO of chunk m, transposed into dOt[m & 1]; replayed (and padding) rows are zero
  auto stage_dO = [&](const f32x4* dov, const Rows& rw, int m, int tid) {
    T* dst = dOt[m & 1];
    const int own = sd.n_replay - m * BT;
#pragma unroll
    for (int x = 0; x < NO; ++x) {
      const int idx = tid + NTH * x;
      if (idx < BT * (DVT / VN)) {
        const int i = idx / (DVT / VN), j0 = (idx % (DVT / VN)) * VN;
        float v[VN];
        unpack16<T>(rw.r[x] >= 0 && i >= own ? dov[x] : f32x4{0.f, 0.f, 0.f, 0.f}, v);
#pragma unroll
        for (int t = 0; t < VN; ++t) dst[(j0 + t) * LDJ + i] = from_f<T>(v[t]);
      }
    }
  };
  f32x4 dS[MU][NTV];
#pragma unroll
  for (int u = 0; u < MU; ++u)
#pragma unroll
    for (int nt = 0; nt < NTV; ++nt) dS[u][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // nxt: operands of chunk n with the dO of chunk n-1; rows_x: rows of the chunk whose
  // dO is in nxt; rows_n: rows of the chunk before that.  cur is taken from nxt at the
  // top of each step, before the next fetch is issued.
  const int z = lane_zero();
  Ops cur, nxt;
  Rows cur_rows, rows_x, rows_n;
  {
    Rows r0;
    f32x4 d0[NO];
    load_dstate_rows<T, BT, D, DV, DVT>(r0, a, chunk_at(N - 1), tid);
    load_dstate_dov<T, BT, D, DV, DVT>(d0, r0, gdo, H, h, tid, jvb);
    stage_dO(d0, r0, N - 1, tid);
    load_dstate_rows<T, BT, D, DV, DVT>(rows_x, a, chunk_at(N - 2), tid);
    load_dstate_ops<T, BT, D, DV, DVT>(nxt, a, chunk_at(N - 1), H, h, wave, lane, z);
    load_dstate_dov<T, BT, D, DV, DVT>(nxt.dov, rows_x, gdo, H, h, tid, jvb);
    load_dstate_rows<T, BT, D, DV, DVT>(rows_n, a, chunk_at(N - 3), tid);
  }
  __syncthreads();
  for (int n = N - 1; n >= 0; --n) {
    // thread-derived addresses are recomputed per step instead of being held across the loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const size_t wsi = size_t(c0 + n) * H + h;
    cur = nxt;
    cur_rows = rows_x;
    // fetch ahead: operands of chunk n-1, dO of chunk n-2 (its rows are here), rows of chunk n-3
    load_dstate_ops<T, BT, D, DV, DVT>(nxt, a, chunk_at(n - 1), H, h, wave, lane, z);
    load_dstate_dov<T, BT, D, DV, DVT>(nxt.dov, rows_n, gdo, H, h, tid, jvb);
    rows_x = rows_n;
    load_dstate_rows<T, BT, D, DV, DVT>(rows_n, a, chunk_at(n - 3), tid);
    // Qeff^T dO (independent of dS)
    f32x4 a1[MU][NTV];
    const T* dOc = dOt[n & 1];
#pragma unroll
    for (int u = 0; u < MU; ++u)
#pragma unroll
      for (int nt = 0; nt < NTV; ++nt) {
        a1[u][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < Ops::KB; ++kk)
          a1[u][nt] = MM::mma(cur.qe[u][kk], MM::kc(dOc, LDJ, 16 * nt, kk * MM::KS, lane), a1[u][nt]);
      }
    // slot gradient: sum over the consumers of the state emitted after this chunk
    if (cur.emit >= 0 && b.slot_cons_off) {
      const int q0 = b.slot_cons_off[cur.emit], q1 = b.slot_cons_off[cur.emit + 1];
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const int mt = wave + NW * u;
        if (mt < MT)
#pragma unroll
          for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int c = 16 * mt + crow(lane, r), jv = jvb + 16 * nt + ccol(lane);
              float add = 0.f;
              for (int qq = q0; qq < q1; ++qq)
                add += b.dinit[((size_t(b.slot_cons[qq]) * H + h) * D + c) * DV + jv];
              dS[u][nt][r] += add;
              if (b.dstates) b.dstates[((size_t(cur.emit) * H + h) * D + c) * DV + jv] = add;
            }
      }
    }
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int mt = wave + NW * u;
      if (mt < MT)
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt)
          store4(dSt + (16 * nt + ccol(lane)) * LDS_S + 16 * mt + crow(lane, 0), dS[u][nt][0], dS[u][nt][1],
                 dS[u][nt][2], dS[u][nt][3]);
    }
    if (n > 0) stage_dO(cur.dov, cur_rows, n - 1, tid);
    __syncthreads();
    // Y = K^ dS  (stored transposed; this wave: token block mi, value tiles nt0 ..)
#pragma unroll
    for (int j = 0; j < NTU; ++j) {
      const int nt = nt0 + j;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < Ops::KD; ++kk)
        acc = MM::mma(cur.kh[kk], MM::kc(dSt, LDS_S, 16 * nt, kk * MM::KS, lane), acc);
      store4(Yt + (16 * nt + ccol(lane)) * LDJ + 16 * mi + crow(lane, 0), acc[0], acc[1], acc[2], acc[3]);
    }
    // gradient w.r.t. the chunk-end state for the per-chunk gradient kernels (dS^T and dS,
    // fragment-major); dSt is rewritten only after the next barrier
    store_state_fm<T, D, DV, DVT, NTH>(static_cast<T*>(b.dh) + wsi * DV * D, static_cast<T*>(b.dhc) + wsi * D * DV,
                                       dSt, LDS_S, jvb, tid);
    __syncthreads();
    // dS <- diag(e^{G_last}) dS + Qeff^T dO - W^T Y
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int mt = wave + NW * u;
      if (mt < MT) {
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt) {
          f32x4 a2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < Ops::KB; ++kk)
            a2 = MM::mma(cur.wt[u][kk], MM::kc(Yt, LDJ, 16 * nt, kk * MM::KS, lane), a2);
#pragma unroll
          for (int r = 0; r < 4; ++r) dS[u][nt][r] = cur.el[u][r] * dS[u][nt][r] + a1[u][nt][r] - a2[r];
        }
      }
    }
  }
  if (b.dinit) {
    const size_t gs = size_t(a.seq0 + si);
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int mt = wave + NW * u;
      if (mt < MT)
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int c = 16 * mt + crow(lane, r), jv = jvb + 16 * nt + ccol(lane);
            b.dinit[((gs * H + h) * D + c) * DV + jv] = dS[u][nt][r];
          }
    }
  }
}

constexpr size_t al16(size_t x) { return (x + 15) / 16 * 16; }
constexpr size_t cmx(size_t a, size_t b) { return a > b ? a : b; }

// ------------------------------------------------------------------------------------------
// C[16x16] += A B over a 16-long contraction: lane l supplies A[l%16][4(l/16) + t] and
// B[4(l/16) + t][l%16], t = 0..3 (B is then a 16-token block of the accumulator layout), as four
// values of the matrix-core element type, so that staged bf16 tiles feed it without a round
// trip through fp32.
template <typename T>
using k16_t = typename std::conditional<sizeof(T) == 2, bf16x4, f32x4>::type;
template <typename T> __device__ __forceinline__ k16_t<T> k16_pack(const float* v) {
  if constexpr (sizeof(T) == 2) return bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  else return f32x4{v[0], v[1], v[2], v[3]};
}
template <typename T> __device__ __forceinline__ k16_t<T> k16_pack(f32x4 v) {
  const float a[4] = {v[0], v[1], v[2], v[3]};
  return k16_pack<T>(a);
}
// four consecutive elements p[0..3]
template <typename T> __device__ __forceinline__ k16_t<T> k16_row(const T* p) {
  return *reinterpret_cast<const k16_t<T>*>(p);
}
// column slice of a row-major LDS tile (as col4_load)
template <typename T> __device__ __forceinline__ k16_t<T> k16_col(const T* p, int ld, int r0, int c0, int lane) {
  if constexpr (sizeof(T) == 2) {
    const int q = lane & 15;
    return ds_tr16(p + (r0 + 4 * (lane >> 4) + (q >> 2)) * ld + c0 + 4 * (q & 3));
  } else {
    float v[4];
    col4_load<T>(p, ld, r0, c0, lane, v);
    return f32x4{v[0], v[1], v[2], v[3]};
  }
}
template <typename T> __device__ __forceinline__ f32x4 mma_k16r(k16_t<T> a, k16_t<T> b, f32x4 c) {
  if constexpr (sizeof(T) == 2) {
    typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s4;
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a), __builtin_bit_cast(s4, b), c, 0, 0, 0);
  } else {
    return mma16_f32(a, b, c);
  }
}

// c + a b with a right operand b given in fp32: for bf16 operands b is split into a bf16 head
// and the bf16 rounding of its remainder, two products, so b carries about 16 significant bits.
// The gated diagonal-block products need them: with steep gates dg is a small difference of
// large terms that the row side and the column side compute from differently scaled operands,
// and one bf16 rounding of each would not cancel.
template <typename T> __device__ __forceinline__ f32x4 mma_k16r_split(k16_t<T> a, const float (&b)[4], f32x4 c) {
  const k16_t<T> hi = k16_pack<T>(b);
  c = mma_k16r<T>(a, hi, c);
  if constexpr (sizeof(T) == 2) {
    const float lo[4] = {b[0] - (float)hi[0], b[1] - (float)hi[1], b[2] - (float)hi[2], b[3] - (float)hi[3]};
    c = mma_k16r<T>(a, k16_pack<T>(lo), c);
  }
  return c;
}

// Per-chunk gradients: one persistent kernel, one workgroup per compute unit walking the
// (chunk, head) items of the round, each item in two halves.
//
// Token side (configuration GACfg): dv, dbeta, and U, dR, dM, dA for the channel side.  Wave
// w owns value columns [16w, 16w + 16): R = V - K~ S0, dU = M^T dO + K^ dS, U = T R and
// dR = T^T dU are chained in the accumulator layout (lane l holds tokens 16b + 4(l/16) + r of
// column 16w + l%16), the 16-token block products taking the lane's own values as their
// right operand.  The token-token tail (dM, dT, dX, dL, dA, dbeta) runs on tiles staged in LDS.
template <typename T, int BT, int D, int DV>
struct GACfg {
  using MM = Mma<T>;
  static constexpr int NW = DV / 16, NT = 64 * NW, NB = BT / 16, VN = 16 / sizeof(T), PAD = 2 * VN;
  static constexpr int NPR = D / VN, NPK = BT * NPR, NK = (NPK + NT - 1) / NT;
  static constexpr int NPRV = DV / VN, NPV = BT * NPRV, NV = (NPV + NT - 1) / NT;
  static constexpr int NPJ = BT * BT / VN, NJ = (NPJ + NT - 1) / NT;
  static constexpr int NKS = D / MM::KS;
  static constexpr bool SAMEV = NPR == NPRV;
  static constexpr int NPART = NT / BT;  // row groups of the dbeta_1 column sums
  // rows padded by 32 bytes: measured fewer LDS bank conflicts than 16 on this kernel's mix of
  // row fragment reads, transposing column reads and 2-byte scattered stores
  static constexpr int LDK = D + PAD, LDV = DV + PAD, LDJ = BT + PAD, LDA = BT + 4;
  static constexpr size_t ES = sizeof(T);
  static constexpr size_t al(size_t x) { return (x + 15) / 16 * 16; }
  static constexpr size_t SKV = al(cmx(size_t(BT) * LDK * ES, size_t(BT) * LDV * ES));
  static constexpr size_t SJ = al(size_t(BT) * LDJ * ES);
  // R0: g -> K~ -> R -> Y1^T   R1: k -> K^ -> U -> dX   R2: v -> dU   R3: dO   R4: dR
  static constexpr size_t O_R0 = 0, O_R1 = SKV, O_R2 = 2 * SKV, O_R3 = 3 * SKV, O_R4 = 4 * SKV;
  // T, M (-> dT fp32 over both), X, A
  static constexpr size_t O_T = 5 * SKV, O_M = O_T + SJ, O_X = O_M + SJ, O_A = O_X + SJ;
  static constexpr size_t O_VEC = O_A + SJ;
  static_assert(2 * SJ >= size_t(BT) * LDA * 4, "dT fits over T and M");
  // vectors (fp32): beta[BT], block totals[NB][D], dbeta_1 parts[NPART][BT], dbeta_2 parts[NB][BT]
  static constexpr size_t V_BET = 0, V_TB = BT, V_DB1 = V_TB + NB * D, V_DB2 = V_DB1 + NPART * BT,
                          V_END = V_DB2 + NB * BT;
  static constexpr size_t TOTAL = O_VEC + V_END * 4;
  static_assert(TOTAL <= 160 * 1024, "token side LDS budget");
  static_assert(NB * D <= NT, "one (block, channel) decay item per thread");
  static_assert(NPART >= 1 && BT % NPART == 0, "dbeta_1 row groups");
};

template <typename T, int BT, int D, int DV>
struct GARows {
  using C = GACfg<T, BT, D, DV>;
  int rk[C::NK], rv_[C::SAMEV ? 1 : C::NV], rb, own, rbase;
  __device__ __forceinline__ int rv(int x) const {
    if constexpr (C::SAMEV) return rk[x];
    else return rv_[x];
  }
};

template <typename T, int BT, int D, int DV>
struct GAIn {
  using C = GACfg<T, BT, D, DV>;
  using F = typename C::MM::Frag;
  f32x4 k[C::NK], g[C::NK], v[C::NV], dO[C::NV], tm[C::NJ], mm[C::NJ], xm[C::NJ], am[C::NJ];
  T beta;
  F hf[C::NKS], dhf[C::NKS];  // this wave's rows of S_n^T and dS_n^T as matrix-core B operands
};

template <typename T, int BT, int D, int DV>
__device__ __forceinline__ void ga_rows(GARows<T, BT, D, DV>& r, const RoundArgs& a, int chunk, int tid) {
  using C = GACfg<T, BT, D, DV>;
  const int32_t* cr = a.crows + size_t(chunk) * BT;
#pragma unroll
  for (int x = 0; x < C::NK; ++x) {
    const int p = tid + C::NT * x;
    r.rk[x] = cr[(p < C::NPK ? p : C::NPK - 1) / C::NPR];
  }
  if constexpr (!C::SAMEV) {
#pragma unroll
    for (int x = 0; x < C::NV; ++x) {
      const int p = tid + C::NT * x;
      r.rv_[x] = cr[(p < C::NPV ? p : C::NPV - 1) / C::NPRV];
    }
  }
  r.rb = cr[tid < BT ? tid : BT - 1];
  r.own = a.chunks[chunk].own_from;
  r.rbase = a.chunks[chunk].replay_base;
}

// P selects a part of the fetch (-1: all): 0 k, g; 1 v, dO; 2 T, M, X, A, beta; 3 and 4 the
// state and state-gradient slices.  The persistent loop issues the parts between phases, so that a workgroup's loads
// are spread over the item instead of queueing behind each other at its top.
template <typename T, int BT, int D, int DV, int P = -1>
__device__ __forceinline__ void ga_load(GAIn<T, BT, D, DV>& o, const GARows<T, BT, D, DV>& r, const BwdRoundArgs& b,
                                        size_t wsi, int h, int H, int tid, int wave, int lane) {
  using C = GACfg<T, BT, D, DV>;
  using MM = typename C::MM;
  const RoundArgs& a = b.r;
  if constexpr (P < 0 || P == 0) {
#pragma unroll
    for (int x = 0; x < C::NK; ++x) {
      const int c0 = ((tid + C::NT * x) % C::NPR) * C::VN;
      const size_t off = (size_t(r.rk[x] >= 0 ? r.rk[x] : 0) * H + h) * D + c0;
      o.k[x] = ldq(static_cast<const T*>(a.k) + off);
      o.g[x] = ldq(static_cast<const T*>(a.g) + off);
    }
  }
  if constexpr (P < 0 || P == 1) {
#pragma unroll
    for (int x = 0; x < C::NV; ++x) {
      const int c0 = ((tid + C::NT * x) % C::NPRV) * C::VN;
      const int rr = r.rv(x);
      const size_t off = (size_t(rr >= 0 ? rr : 0) * H + h) * DV + c0;
      o.v[x] = ldq(static_cast<const T*>(a.v) + off);
      o.dO[x] = ldq(static_cast<const T*>(b.dO) + off);
    }
  }
  if constexpr (P < 0 || P == 2) {
    const size_t BB = size_t(BT) * BT;
#pragma unroll
    for (int x = 0; x < C::NJ; ++x) {
      const int p = tid + C::NT * x;
      const size_t off = wsi * BB + size_t(p < C::NPJ ? p : C::NPJ - 1) * C::VN;
      o.tm[x] = ldq(static_cast<const T*>(a.ws.Tm) + off);
      o.mm[x] = ldq(static_cast<const T*>(a.ws.Mm) + off);
      o.xm[x] = ldq(static_cast<const T*>(a.ws.Xm) + off);
      o.am[x] = ldq(static_cast<const T*>(a.ws.Am) + off);
    }
    o.beta = static_cast<const T*>(a.beta)[size_t(r.rb >= 0 ? r.rb : 0) * H + h];
  }
  if constexpr (P < 0 || P == 3) {
    const T* hg = static_cast<const T*>(a.h) + wsi * DV * D;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) o.hf[ks] = fm_frag<T>(hg, D, wave, ks, lane);
  }
  if constexpr (P < 0 || P == 4) {
    const T* dhg = static_cast<const T*>(b.dh) + wsi * DV * D;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) o.dhf[ks] = fm_frag<T>(dhg, D, wave, ks, lane);
  }
}

// ------------------------------------------------------------------------------------------
// Channel side (configuration GBCfg): dq, dk, dg.  Wave w owns channels [16w, 16w + 16) for
// every token of the chunk, with lane l holding, for each 16-token block b, tokens
// 16b + 4(l/16) + r (r = 0..3) of channel 16w + l%16 -- the accumulator layout of the matrix
// cores.  The in-chunk decay, the 16-token block products (whose right operand is the lane's
// own values), the state products and the final reverse cumulative sum of dg all stay inside
// the wave.
template <typename T, int BT, int D, int DV>
struct GBCfg {
  using MM = Mma<T>;
  static constexpr int NW = D / 16, NT = 64 * NW, NB = BT / 16, VN = 16 / sizeof(T), PAD = 2 * VN;
  static constexpr int NPR = D / VN, NPK = BT * NPR, NK = (NPK + NT - 1) / NT;
  static constexpr int NPRV = DV / VN, NPV = BT * NPRV, NV = (NPV + NT - 1) / NT;
  static constexpr int NPJ = BT * BT / VN, NJ = (NPJ + NT - 1) / NT;
  static constexpr int NKS = DV / MM::KS;
  static constexpr bool SAMEV = NPR == NPRV;
  static constexpr int LDK = D + PAD, LDV = DV + PAD, LDJ = BT + PAD, LDF = D + 4;
  static constexpr size_t ES = sizeof(T);
  static constexpr size_t al(size_t x) { return (x + 15) / 16 * 16; }
  // staged inputs (bf16/fp32): Q, K, g [BT][LDK]; dO, U, dR [BT][LDV]; dM, dA [BT][LDJ]
  static constexpr size_t SK = al(size_t(BT) * LDK * ES), SV = al(size_t(BT) * LDV * ES), SJ = al(size_t(BT) * LDJ * ES);
  static constexpr size_t O_Q = 0, O_K = SK, O_G = 2 * SK, O_DO = 3 * SK, O_U = O_DO + SV, O_DR = O_U + SV,
                          O_DM = O_DR + SV, O_DA = O_DM + SJ, IN_END = O_DA + SJ;
  // output staging (fp32 [BT][LDF] for dq, dk, dg) over the inputs once they are consumed
  static constexpr size_t SF = al(size_t(BT) * LDF * 4);
  // bf16: per wave, its 16 channels of S_n (then of dS_n) as [DV][16], read back transposed
  static constexpr size_t O_HS = cmx(IN_END, 3 * SF), HS = sizeof(T) == 2 ? al(size_t(NW) * DV * 16 * ES) : 0;
  static constexpr size_t TOTAL = O_HS + HS;
  static constexpr int NHP = DV / 32;  // 16-byte pieces per lane of one wave's slice
  static_assert(TOTAL <= 160 * 1024, "channel side LDS budget");
};

template <typename T, int BT, int D, int DV>
struct GBIn {
  using C = GBCfg<T, BT, D, DV>;
  using F = typename C::MM::Frag;
  f32x4 q[C::NK];  // k and g are the token side's own pieces (same threads, same layout)
  // bf16: this wave's channels of S_n and dS_n, read from their S_n^T fragment-major copies
  // (16-byte pieces, staged in LDS and read back as matrix-core B operands); fp32: the B
  // operands from the channel-major copies
  static constexpr bool BF = sizeof(T) == 2;
  f32x4 hp[BF ? C::NHP : 1], dp[BF ? C::NHP : 1];
  F hc[BF ? 1 : C::NKS], dhc[BF ? 1 : C::NKS];
};

// Unconditional loads from clamped addresses: padding is masked where the values are used.
// P selects a part of the fetch: 0 q; 1 the state slices.
template <typename T, int BT, int D, int DV, int P>
__device__ __forceinline__ void gb_load(GBIn<T, BT, D, DV>& o, const GARows<T, BT, D, DV>& r, const BwdRoundArgs& b,
                                        size_t wsi, int h, int H, int tid, int wave, int lane) {
  using C = GBCfg<T, BT, D, DV>;
  using MM = typename C::MM;
  const RoundArgs& a = b.r;
  if constexpr (P == 0) {
#pragma unroll
    for (int x = 0; x < C::NK; ++x) {
      const int c0 = ((tid + C::NT * x) % C::NPR) * C::VN;
      const size_t off = (size_t(r.rk[x] >= 0 ? r.rk[x] : 0) * H + h) * D + c0;
      o.q[x] = ldq(static_cast<const T*>(a.q) + off);
    }
  }
  if constexpr (P == 1) {
    if constexpr (sizeof(T) == 2) {
      // piece x of lane l: value rows 16 (2x + l/32) + l%16, channels 16 wave + 8 ((l/16)%2) + 0..7
      // of the [DV][D] fragment-major S_n^T (block (v tile, channel block wave/2), lane 32 (wave%2)
      // + l%32)
      const T* hg = static_cast<const T*>(a.h) + wsi * DV * D;
      const T* dhg = static_cast<const T*>(b.dh) + wsi * DV * D;
#pragma unroll
      for (int x = 0; x < C::NHP; ++x) {
        const size_t off = ((size_t(2 * x + (lane >> 5)) * (D / 32) + (wave >> 1)) * 64 + 32 * (wave & 1) + (lane & 31)) * 8;
        o.hp[x] = ldq(hg + off);
        o.dp[x] = ldq(dhg + off);
      }
    } else {
      const T* hcg = static_cast<const T*>(a.hc) + wsi * D * DV;
      const T* dhcg = static_cast<const T*>(b.dhc) + wsi * D * DV;
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) {
        o.hc[ks] = fm_frag<T>(hcg, DV, wave, ks, lane);
        o.dhc[ks] = fm_frag<T>(dhcg, DV, wave, ks, lane);
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// The gradient kernel: a workgroup takes each (chunk, head) item through the token side and
// then the channel side.  U, dR, dM and dA stay in LDS between the halves and dO is staged
// once for both, so the intermediates never reach HBM and the shared inputs are read once: the
// channel side stages k and g from the token side's registers (both sides give a thread the same
// pieces).  The channel side's own inputs (q and its state slices) are fetched while the token
// side computes, the next item's token-side inputs while the channel side computes.
template <typename T, int BT, int D, int DV>
struct GFCfg {
  using A = GACfg<T, BT, D, DV>;
  using B = GBCfg<T, BT, D, DV>;
  static_assert(D == DV, "one thread layout serves both halves");
  static_assert(DV >= BT, "token-token tiles fit in the token-channel regions");
  static constexpr size_t SKV = A::SKV, SJ = A::SJ;
  // dO | k -> K^ -> U | dR | dM | T (-> dT over T and M -> dA) | M | X | A |
  // R0: g -> K~ -> R -> Y1^T | R2: v -> dU -> dX | token-side vectors
  static constexpr size_t O_DO = 0, O_U = SKV, O_DR = 2 * SKV, O_DM = 3 * SKV, O_T = O_DM + SJ, O_M = O_T + SJ,
                          O_X = O_M + SJ, O_A = O_X + SJ, O_R0 = O_A + SJ, O_R2 = O_R0 + SKV, O_VEC = O_R2 + SKV;
  static constexpr size_t A_END = O_VEC + A::V_END * 4;
  // channel side: per-wave state slices over R0 and R2, then q, k, g from M on; the fp32
  // output staging over everything once the inputs are consumed
  static constexpr size_t O_HS = O_R0, O_Q = O_M, O_K = O_M + B::SK, O_G = O_M + 2 * B::SK;
  static constexpr size_t TOTAL = cmx(A_END, 3 * B::SF);
  static_assert(2 * SJ >= size_t(BT) * A::LDA * 4, "dT fits over T and M");
  static_assert(O_HS + B::HS <= O_VEC, "state slices clear of the token-side vectors");
  static_assert(O_G + B::SK <= TOTAL, "q, k, g");
  static_assert(B::SV <= SKV && B::SJ == SJ && A::LDV == B::LDV && A::LDJ == B::LDJ && A::LDK == B::LDK &&
                    A::NK == B::NK && A::NV == B::NV && A::NT == B::NT,
                "shared tiles and thread mapping");
  static_assert(TOTAL <= 160 * 1024, "fused gradient kernel LDS budget");
};

// Pairwise diagonal-block terms of block bb for a steep channel c (block gate sum below
// -kSteepGate), this lane's rows i = 16 bb + 4 g4 + r:
//   dq_i += sum_{j <= i} dM_ij k_jc e^{L_ic - L_jc},   dk_i (row) += sum_{j < i} dA_ij k_jc e^{L_ic - L_jc},
//   dk_i (col) += sum_{j >= i} (dM_ji q_jc + dA_ji k_jc) e^{L_jc - L_ic},
// L the block-local cumulative log-decays, taken from the lanes that hold them (lane cc + 16 q
// holds rows 4 q .. 4 q + 3 of channel c), so the j = i terms carry exactly e^0.  Called by the
// whole wave.
template <typename T, int LDK, int LDJ>
__device__ __forceinline__ void steep_diag_grad(const T* Qb, const T* Kb, const T* dMl, const T* dAl, int bb, int c,
                                                int cc, int g4, const float (&Li)[4], bool mine, f32x4& dq, f32x4& kr,
                                                f32x4& kc) {
  // a rolled loop over j keeps this rarely taken path from raising the register demand of the
  // kernel around it; lanes whose channel is not steep add nothing
  const float w = mine ? 1.f : 0.f;
#pragma unroll 1
  for (int j = 0; j < 16; ++j) {
    const int t = j & 3;
    const float lsrc = t == 0 ? Li[0] : t == 1 ? Li[1] : t == 2 ? Li[2] : Li[3];
    const float lj = __shfl(lsrc, cc + 16 * (j >> 2), 64);
    const int rj = 16 * bb + j;
    const float kj = w * to_f(Kb[rj * LDK + c]), qj = w * to_f(Qb[rj * LDK + c]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * g4 + r, ri = 16 * bb + i;
      if (j <= i) {
        const float e = __expf(fminf(Li[r] - lj, 0.f));
        dq[r] += to_f(dMl[ri * LDJ + rj]) * kj * e;
        if (j < i) kr[r] += to_f(dAl[ri * LDJ + rj]) * kj * e;
      }
      if (j >= i)
        kc[r] += (to_f(dMl[rj * LDJ + ri]) * qj + to_f(dAl[rj * LDJ + ri]) * kj) * __expf(fminf(lj - Li[r], 0.f));
    }
  }
}

template <typename T, int BT, int D, int DV>
__global__ __launch_bounds__(64 * (DV / 16)) void kda_grad_kernel(BwdRoundArgs b, int H) {
  using C = GFCfg<T, BT, D, DV>;
  using CA = GACfg<T, BT, D, DV>;
  using CB = GBCfg<T, BT, D, DV>;
  using MM = typename CA::MM;
  using G = RG<D, DV>;
  using In = GAIn<T, BT, D, DV>;
  using InB = GBIn<T, BT, D, DV>;
  using Rows = GARows<T, BT, D, DV>;
  constexpr int NT = CA::NT, NW = CA::NW, NB = CA::NB, VN = CA::VN, NK = CA::NK, NV = CA::NV, NJ = CA::NJ;
  constexpr int LDK = CA::LDK, LDV = CA::LDV, LDJ = CA::LDJ, LDA = CA::LDA, LDF = CB::LDF, NPR = CA::NPR,
                NPRV = CA::NPRV;
  __shared__ __attribute__((aligned(16))) char smem[C::TOTAL];
  T* dOs = reinterpret_cast<T*>(smem + C::O_DO);
  T* Ks = reinterpret_cast<T*>(smem + C::O_U);  // k, then K^ in place, then U
  T* Kh = Ks;
  T* Us = Ks;
  T* dRs = reinterpret_cast<T*>(smem + C::O_DR);
  T* dMl = reinterpret_cast<T*>(smem + C::O_DM);
  T* Tl = reinterpret_cast<T*>(smem + C::O_T);
  float* dTf = reinterpret_cast<float*>(smem + C::O_T);
  T* dAl = Tl;
  T* Ml = reinterpret_cast<T*>(smem + C::O_M);
  T* Xl = reinterpret_cast<T*>(smem + C::O_X);
  T* Al = reinterpret_cast<T*>(smem + C::O_A);
  T* Gs = reinterpret_cast<T*>(smem + C::O_R0);  // g, then K~ in place, then R, then Y1^T
  T* Kt = Gs;
  T* Rs = Gs;
  T* Y1t = Gs;
  T* Vs = reinterpret_cast<T*>(smem + C::O_R2);  // v, then dU, then dX
  T* dUs = Vs;
  T* dXs = Vs;
  float* vec = reinterpret_cast<float*>(smem + C::O_VEC);
  float* bet = vec + CA::V_BET;
  float* Tbv = vec + CA::V_TB;
  float* db1 = vec + CA::V_DB1;
  float* db2 = vec + CA::V_DB2;
  T* Qb = reinterpret_cast<T*>(smem + C::O_Q);
  T* Kb = reinterpret_cast<T*>(smem + C::O_K);
  T* Gb = reinterpret_cast<T*>(smem + C::O_G);
  float* stg = reinterpret_cast<float*>(smem);  // [3][BT][LDF] at the end of the channel side
  const RoundArgs& a = b.r;

  const int nitems = a.nchunk * H;
  int item = blockIdx.x;
  if (item >= nitems) return;
  const int tid0 = threadIdx.x;
  // rows_x: rows of the item whose token-side inputs are in nxt; rows_n: rows of the item after it
  Rows rows, rows_x, rows_n;
  In cur, nxt;
  InB cb;  // channel-side inputs of the current item
  ga_rows<T, BT, D, DV>(rows_x, a, item / H, tid0);
  ga_load<T, BT, D, DV>(nxt, rows_x, b, size_t(item), item % H, H, tid0, tid0 >> 6, tid0 & 63);
  int item_n = item + gridDim.x;
  ga_rows<T, BT, D, DV>(rows_n, a, (item_n < nitems ? item_n : item) / H, tid0);
  __shared__ int tk_slot;
  // Nothing fetched before the loop stays outstanding into it.  The compiler's wait counts at the
  // loop head take the more cautious of its two entries; the prologue issues only a few memory
  // operations after its fetches, the loop body many (the item's stores), so without this wait
  // every item would wait at its top for nearly all of the previous item's stores to complete.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  while (item < nitems) {
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    // the wave index is uniform: tile selection and addressing derived from it stay scalar
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), cc = lane & 15, g4 = lane >> 4;
    const int h = item % H;
    const size_t wsi = size_t(item);
    cur = nxt;
    rows = rows_x;
    const int itn = item_n < nitems ? item_n : item;
    rows_x = rows_n;
    int tk = 0;  // thread 0: the ticket for the item after the next one
    if (a.ctr && tid == 0) tk = draw_ticket(a.ctr);
    gb_load<T, BT, D, DV, 0>(cb, rows, b, wsi, h, H, tid, wave, lane);  // q of this item

    // ---------------- token side ----------------
    // A1. stage the inputs (padding rows zero; dO zero on replayed rows)
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < NK; ++x) {
      const int p = tid + NT * x;
      if (p < CA::NPK) {
        const int i = p / NPR, c0 = (p % NPR) * VN;
        const bool ok = rows.rk[x] >= 0;
        stq(Gs + i * LDK + c0, ok ? cur.g[x] : z4);
        stq(Ks + i * LDK + c0, ok ? cur.k[x] : z4);
      }
    }
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      const int p = tid + NT * x;
      if (p < CA::NPV) {
        const int i = p / NPRV, c0 = (p % NPRV) * VN;
        const bool ok = rows.rv(x) >= 0;
        stq(Vs + i * LDV + c0, ok ? cur.v[x] : z4);
        stq(dOs + i * LDV + c0, ok && i >= rows.own ? cur.dO[x] : z4);
      }
    }
#pragma unroll
    for (int x = 0; x < NJ; ++x) {
      const int p = tid + NT * x;
      if (p < CA::NPJ) {
        const int i = p / (BT / VN), j0 = (p % (BT / VN)) * VN;
        stq(Tl + i * LDJ + j0, cur.tm[x]);
        stq(Xl + i * LDJ + j0, cur.xm[x]);
        stq(Al + i * LDJ + j0, cur.am[x]);
        if constexpr (sizeof(T) == 2) {
          stq(Ml + i * LDJ + j0, cur.mm[x]);  // row-major from the bf16 preparation
        } else {
          // M arrives fragment-major: element o of the piece is row r, column k of M
          constexpr int LE = fm_le<T>(), KS = MM::KS;
          float mv[VN];
          unpack16<T>(cur.mm[x], mv);
#pragma unroll
          for (int e = 0; e < VN; ++e) {
            const int o = p * VN + e, li = o / LE, f = li / 64, l = li % 64;
            const int r = (f / (BT / KS)) * 16 + (l & 15), k = (f % (BT / KS)) * KS + LE * (l >> 4) + o % LE;
            Ml[r * LDJ + k] = from_f<T>(mv[e]);
          }
        }
      }
    }
    if (tid < BT) bet[tid] = rows.rb >= 0 ? to_f(cur.beta) : 0.f;
    __syncthreads();
    // A2. decay per (16-row block, channel): block totals
    HARTS_STRIDED(idx, tid, NB * D, NT) {
      const int bb = idx / D, c = idx % D;
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < 16; ++t) s += to_f(Gs[(16 * bb + t) * LDK + c]);
      Tbv[bb * D + c] = s;
    }
    __syncthreads();
    // A3. K~ = k e^{F_b + L} over g, K^ = k e^{G_last - F_b - L} over k, L the block-local
    //     cumulative log-decay (summed again rather than held across the barrier)
    HARTS_STRIDED(idx, tid, NB * D, NT) {
      const int bb = idx / D, c = idx % D;
      float fb = 0.f, fe = 0.f;
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        const float tq = Tbv[q * D + c];
        fb += q < bb ? tq : 0.f;
        fe += tq;
      }
      float Lr = 0.f;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int i = 16 * bb + t;
        Lr += to_f(Gs[i * LDK + c]);
        const float kv = to_f(Ks[i * LDK + c]);
        Kt[i * LDK + c] = from_f<T>(kv * __expf(fb + Lr));
        Kh[i * LDK + c] = from_f<T>(kv * __expf(fe - fb - Lr));
      }
    }
    if (a.ctr && tid == 0) tk_slot = tk;
    __syncthreads();
    // the item after the next one: its rows are fetched a whole item ahead of their use
    const int item_nn = a.ctr ? 2 * int(gridDim.x) + tk_slot : item_n + int(gridDim.x);
    ga_rows<T, BT, D, DV>(rows_n, a, (item_nn < nitems ? item_nn : item) / H, tid);
    // A4. R = V - K~ S0 and dU = K^ dS + M^T dO for this wave's value columns
    const int jv = 16 * wave + cc;
    f32x4 R[NB], dU[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      f32x4 r1 = z4, r2 = z4;
#pragma unroll
      for (int ks = 0; ks < CA::NKS; ++ks) {
        r1 = MM::mma(MM::kc(Kt, LDK, 16 * bb, ks * MM::KS, lane), cur.hf[ks], r1);
        r2 = MM::mma(MM::kc(Kh, LDK, 16 * bb, ks * MM::KS, lane), cur.dhf[ks], r2);
      }
      float vv[4];
      col4_load<T>(Vs, LDV, 16 * bb, 16 * wave, lane, vv);
#pragma unroll
      for (int r = 0; r < 4; ++r) R[bb][r] = vv[r] - r1[r];
      dU[bb] = r2;
    }
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int br = 0; br < NB; ++br) {
        if (br < bi) continue;
        dU[bi] = mma_k16r<T>(k16_col<T>(Ml, LDJ, 16 * br, 16 * bi, lane), k16_col<T>(dOs, LDV, 16 * br, 16 * wave, lane),
                             dU[bi]);
      }
    __syncthreads();  // K~, K^ and V consumed
    gb_load<T, BT, D, DV, 1>(cb, rows, b, wsi, h, H, tid, wave, lane);  // the channel side's state slices
    // A5. U = T R, dR = T^T dU; stage R, U, dU, dR
    f32x4 U[NB], dR[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) U[bb] = dR[bb] = z4;
    k16_t<T> Rk[NB], dUk[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      Rk[bb] = k16_pack<T>(R[bb]);
      dUk[bb] = k16_pack<T>(dU[bb]);
    }
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int bj = 0; bj <= bi; ++bj) {
        const k16_t<T> ta = k16_row<T>(Tl + (16 * bi + cc) * LDJ + 16 * bj + 4 * g4);
        const k16_t<T> tb = k16_col<T>(Tl, LDJ, 16 * bi, 16 * bj, lane);
        U[bi] = mma_k16r<T>(ta, Rk[bj], U[bi]);
        dR[bj] = mma_k16r<T>(tb, dUk[bi], dR[bj]);
      }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * bb + 4 * g4 + r;
        Rs[i * LDV + jv] = from_f<T>(R[bb][r]);
        Us[i * LDV + jv] = from_f<T>(U[bb][r]);
        dUs[i * LDV + jv] = from_f<T>(dU[bb][r]);
        dRs[i * LDV + jv] = from_f<T>(dR[bb][r]);
      }
    __syncthreads();
    // A6. dM = lower(dO U^T) (computed transposed) into LDS; dT = dU R^T (fp32) over T, M;
    //     dv of own rows to the output, of replayed rows to the side buffer
    {
      constexpr int NTRI = NB * (NB + 1) / 2;
      HARTS_STRIDED(jb, wave, 2 * NTRI, NW) {
        const int t = jb < NTRI ? jb : jb - NTRI;
        int bi = 0;
        while ((bi + 1) * (bi + 2) / 2 <= t) ++bi;
        const int bj = t - bi * (bi + 1) / 2;
        f32x4 acc = z4;
        if (jb < NTRI) {
#pragma unroll
          for (int k0 = 0; k0 < DV; k0 += MM::KS)
            acc = MM::mma(MM::kc(Us, LDV, 16 * bj, k0, lane), MM::kc(dOs, LDV, 16 * bi, k0, lane), acc);
          const int i = 16 * bi + cc, j0 = 16 * bj + 4 * g4;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = j0 + r <= i ? acc[r] : 0.f;
          store4(dMl + i * LDJ + j0, v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int k0 = 0; k0 < DV; k0 += MM::KS)
            acc = MM::mma(MM::kc(dUs, LDV, 16 * bi, k0, lane), MM::kc(Rs, LDV, 16 * bj, k0, lane), acc);
#pragma unroll
          for (int r = 0; r < 4; ++r) dTf[(16 * bi + 4 * g4 + r) * LDA + 16 * bj + cc] = acc[r];
        }
      }
#pragma unroll
      for (int x = 0; x < NV; ++x) {
        const int p = tid + NT * x;
        const int row = rows.rv(x);
        if (p < CA::NPV && row >= 0) {
          const int i = p / NPRV, c0 = (p % NPRV) * VN;
          const f32x4 drv = ldq(dRs + i * LDV + c0);
          if (i >= rows.own) {
            stq(static_cast<T*>(b.dv) + (size_t(row) * H + h) * DV + c0, drv);
          } else {
            float f[VN];
            unpack16<T>(drv, f);
            float* rg = b.replay_grad + (size_t(rows.rbase + i) * H + h) * G::W + G::DVO + c0;
#pragma unroll
            for (int t = 0; t < VN; ++t) rg[t] = f[t];
          }
        }
      }
    }
    __syncthreads();
    // A7. dX = dT diag(beta) (lower incl.) over dU; column partial sums of X .* dT for dbeta_1
    HARTS_STRIDED(idx, tid, BT * (BT / VN), NT) {
      const int i = idx / (BT / VN), j0 = (idx % (BT / VN)) * VN;
      float v[VN];
#pragma unroll
      for (int t = 0; t < VN; ++t) v[t] = j0 + t <= i ? dTf[i * LDA + j0 + t] * bet[j0 + t] : 0.f;
      stq(dXs + i * LDJ + j0, pack16<T>(v));
    }
    {
      constexpr int RPP = BT / CA::NPART;
      const int j = tid % BT, part = tid / BT;
      float s = 0.f;
#pragma unroll
      for (int u = 0; u < RPP; ++u) {
        const int i = part * RPP + u;
        s += i >= j ? to_f(Xl[i * LDJ + j]) * dTf[i * LDA + j] : 0.f;
      }
      db1[part * BT + j] = s;
    }
    __syncthreads();
    // A8. Y1 = dX X^T, stored transposed over R
    HARTS_STRIDED(jb, wave, NB * NB, NW) {
      const int mi = jb / NB, nk = jb % NB;
      f32x4 acc = z4;
#pragma unroll
      for (int k0 = 0; k0 < BT; k0 += MM::KS)
        acc = MM::mma(MM::kc(dXs, LDJ, 16 * mi, k0, lane), MM::kc(Xl, LDJ, 16 * nk, k0, lane), acc);
      store4(Y1t + (16 * nk + cc) * LDJ + 16 * mi + 4 * g4, acc[0], acc[1], acc[2], acc[3]);
    }
    __syncthreads();
    // A9. dL = -X^T Y1 (lower tiles, computed transposed): dA = strict_lower(diag(beta) dL) into
    //     LDS over T, row partial sums of dL .* A for dbeta_2
    {
      constexpr int NTRI = NB * (NB + 1) / 2;
      HARTS_STRIDED(jb, wave, NTRI, NW) {
        int bi = 0;
        while ((bi + 1) * (bi + 2) / 2 <= jb) ++bi;
        const int bj = jb - bi * (bi + 1) / 2;
        f32x4 acc = z4;
#pragma unroll
        for (int k0 = 0; k0 < BT; k0 += MM::KS)
          acc = MM::mma(MM::kc(Y1t, LDJ, 16 * bj, k0, lane), MM::rc(Xl, LDJ, 16 * bi, k0, lane), acc);
        const int i = 16 * bi + cc, j0 = 16 * bj + 4 * g4;
        const float bi_ = bet[i];
        float v[4], p2 = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + r;
          const float dl = -acc[r];
          v[r] = j < i ? bi_ * dl : 0.f;
          p2 += j < i ? dl * to_f(Al[i * LDJ + j]) : 0.f;
        }
        store4(dAl + i * LDJ + j0, v[0], v[1], v[2], v[3]);
        p2 += __shfl_xor(p2, 16, 64);
        p2 += __shfl_xor(p2, 32, 64);
        if (g4 == 0) db2[bj * BT + i] = p2;
      }
    }
    __syncthreads();
    // A10. dbeta = dbeta_1 + dbeta_2: own rows to the output, replayed rows to the side buffer
    if (tid < BT && rows.rb >= 0) {
      const int i = tid;
      float s = 0.f;
#pragma unroll
      for (int part = 0; part < CA::NPART; ++part) s += db1[part * BT + i];
#pragma unroll
      for (int bj = 0; bj < NB; ++bj) s += bj <= i / 16 ? db2[bj * BT + i] : 0.f;
      if (i >= rows.own) static_cast<T*>(b.dbeta)[size_t(rows.rb) * H + h] = from_f<T>(s);
      else b.replay_grad[(size_t(rows.rbase + i) * H + h) * G::W + G::DB] = s;
    }

    // ---------------- channel side ----------------
    const int c = 16 * wave + cc;
    // B2. state products (raw): dO S0^T, dR S0^T, U dS^T (into X23, where the column side of the
    //     block products accumulates on top of it: both take the factor e^{F_{b+1} - G_j}, B4);
    //     rowsum(dS .* S0) for dG_last
    f32x4 dqa[NB], X1[NB], X23[NB];
    float rs = 0.f;
    if constexpr (sizeof(T) == 2) {
      // this wave's channels of S_n, then of dS_n, through its LDS slice [DV][16] (over R0 and
      // R2, whose last readers passed the barrier above); B operands by two transposing reads
      T* hs = reinterpret_cast<T*>(smem + C::O_HS) + wave * (DV * 16);
      const int cl0 = 8 * ((lane >> 4) & 1), q = lane & 15;
      auto stage = [&](const f32x4 (&pc)[CB::NHP]) {
#pragma unroll
        for (int x = 0; x < CB::NHP; ++x) stq(hs + (16 * (2 * x + (lane >> 5)) + (lane & 15)) * 16 + cl0, pc[x]);
      };
      auto frag = [&](int ks) {
        const T* src = hs + (32 * ks + 8 * (lane >> 4) + (q >> 2)) * 16 + 4 * (q & 3);
        const bf16x4 lo = ds_tr16(src), hi = ds_tr16(src + 4 * 16);
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
      bf16x8 hf[CB::NKS];
      stage(cb.hp);
#pragma unroll
      for (int ks = 0; ks < CB::NKS; ++ks) hf[ks] = frag(ks);
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        dqa[bb] = X1[bb] = X23[bb] = z4;
#pragma unroll
        for (int ks = 0; ks < CB::NKS; ++ks) {
          dqa[bb] = MM::mma(MM::kc(dOs, LDV, 16 * bb, ks * MM::KS, lane), hf[ks], dqa[bb]);
          X1[bb] = MM::mma(MM::kc(dRs, LDV, 16 * bb, ks * MM::KS, lane), hf[ks], X1[bb]);
        }
      }
      stage(cb.dp);  // in order behind this wave's reads of the S_n slice
#pragma unroll
      for (int ks = 0; ks < CB::NKS; ++ks) {
        const bf16x8 df = frag(ks);
#pragma unroll
        for (int t = 0; t < 8; t += 2) {  // two bf16 products per instruction, summed in fp32
          typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
          rs = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{hf[ks][t], hf[ks][t + 1]}, bf16x2{df[t], df[t + 1]}, rs, false);
        }
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) X23[bb] = MM::mma(MM::kc(Us, LDV, 16 * bb, ks * MM::KS, lane), df, X23[bb]);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < CB::NKS; ++ks) rs += cb.hc[ks] * cb.dhc[ks];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        dqa[bb] = X1[bb] = X23[bb] = z4;
#pragma unroll
        for (int ks = 0; ks < CB::NKS; ++ks) {
          dqa[bb] = MM::mma(MM::kc(dOs, LDV, 16 * bb, ks * MM::KS, lane), cb.hc[ks], dqa[bb]);
          X1[bb] = MM::mma(MM::kc(dRs, LDV, 16 * bb, ks * MM::KS, lane), cb.hc[ks], X1[bb]);
          X23[bb] = MM::mma(MM::kc(Us, LDV, 16 * bb, ks * MM::KS, lane), cb.dhc[ks], X23[bb]);
        }
      }
    }
    rs += __shfl_xor(rs, 16, 64);
    rs += __shfl_xor(rs, 32, 64);
    ga_load<T, BT, D, DV, 0>(nxt, rows_x, b, size_t(itn), itn % H, H, tid, wave, lane);
    __syncthreads();  // state slices read: q, k, g take their place
#pragma unroll
    for (int x = 0; x < NK; ++x) {
      const int p = tid + NT * x;
      if (p < CA::NPK) {
        const int i = p / NPR, c0 = (p % NPR) * VN;
        const bool ok = rows.rk[x] >= 0;
        stq(Qb + i * LDK + c0, ok ? cb.q[x] : z4);
        stq(Kb + i * LDK + c0, ok ? cur.k[x] : z4);
        stq(Gb + i * LDK + c0, ok ? cur.g[x] : z4);
      }
    }
    __syncthreads();
    ga_load<T, BT, D, DV, 1>(nxt, rows_x, b, size_t(itn), itn % H, H, tid, wave, lane);
    // B3. in-chunk decay of channel c at this lane's tokens: L (block-local cumulative),
    //     block totals Tb and block entry values F (F[NB] = G_last)
    float L[NB][4], Tb[NB], F[NB + 1];
    F[0] = 0.f;
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      float s = 0.f, gv[4];
      col4_load<T>(Gb, LDK, 16 * bb, 16 * wave, lane, gv);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s += gv[r];
        L[bb][r] = s;
      }
      float tot[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) tot[q] = __shfl(s, cc + 16 * q, 64);
      float ex = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) ex += q < g4 ? tot[q] : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) L[bb][r] += ex;
      Tb[bb] = tot[0] + tot[1] + tot[2] + tot[3];
      F[bb + 1] = F[bb] + Tb[bb];
    }
    // gated state products; csum = sum over this lane's rows of k e^{G_last - G} (U dS^T), the
    // K^ part of dG_last.  e^{L} and e^{T_b - L} (exponents <= 0) of this lane's rows.
    rs *= __expf(F[NB]);
    float csum = 0.f, eL[NB][4], ecL[NB][4];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const float ef = __expf(F[bb]), eh = __expf(F[NB] - F[bb + 1]);
      float kvv[4];
      col4_load<T>(Kb, LDK, 16 * bb, 16 * wave, lane, kvv);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        eL[bb][r] = __expf(L[bb][r]);
        ecL[bb][r] = __expf(Tb[bb] - L[bb][r]);
        dqa[bb][r] *= ef;
        X1[bb][r] *= -ef;
        X23[bb][r] *= eh;
        csum += kvv[r] * ecL[bb][r] * X23[bb][r];
      }
    }
    ga_load<T, BT, D, DV, 2>(nxt, rows_x, b, size_t(itn), itn % H, H, tid, wave, lane);
    // B4. 16-token block products with the gated masks factored per block pair, every
    //     exponent <= 0 off the diagonal blocks (P = dM with x = q, P = dA with x = k):
    //     row side  sum_j P_ij k_j e^{F_bi - G_j},  e^{F_bi - G_j} = e^{F_bi - F_{bj+1}} e^{T_bj - L_j}
    //     col side  sum_i P_ij x_i e^{G_i - F_{bj+1}},  e^{G_i - F_{bj+1}} = e^{L_i} e^{F_bi - F_{bj+1}}
    //     and on a diagonal block e^{-L_j} = e^{T_b - L_j} e^{-T_b} and e^{L_i - T_b} = e^{L_i} e^{-T_b},
    //     both at most e^{kSteepGate}; a steep block (gate sum below -kSteepGate) takes 0 here and
    //     its diagonal terms pairwise in B5
#pragma unroll
    for (int bi = 0; bi < NB; ++bi)
#pragma unroll
      for (int bj = 0; bj <= bi; ++bj) {
        const float ep = bi == bj ? (Tb[bi] < -kSteepGate ? 0.f : __expf(-Tb[bi])) : __expf(F[bi] - F[bj + 1]);
        float bk[4];
        col4_load<T>(Kb, LDK, 16 * bj, 16 * wave, lane, bk);
#pragma unroll
        for (int t = 0; t < 4; ++t) bk[t] *= ep * ecL[bj][t];
        const k16_t<T> dMr = k16_row<T>(dMl + (16 * bi + cc) * LDJ + 16 * bj + 4 * g4);
        const k16_t<T> dAr = k16_row<T>(dAl + (16 * bi + cc) * LDJ + 16 * bj + 4 * g4);
        // the diagonal block's terms (decay near 1) are the ones that cancel in dg under steep
        // gates: their right operands carry a bf16 remainder; off the diagonal the decay factor
        // is at most e^{T_b} and one bf16 rounding is enough
        const bool dgb = bi == bj;
        dqa[bi] = dgb ? mma_k16r_split<T>(dMr, bk, dqa[bi]) : mma_k16r<T>(dMr, k16_pack<T>(bk), dqa[bi]);
        X1[bi] = dgb ? mma_k16r_split<T>(dAr, bk, X1[bi]) : mma_k16r<T>(dAr, k16_pack<T>(bk), X1[bi]);
        float bq[4], bk2[4];
        col4_load<T>(Qb, LDK, 16 * bi, 16 * wave, lane, bq);
        col4_load<T>(Kb, LDK, 16 * bi, 16 * wave, lane, bk2);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float e = eL[bi][t] * ep;
          bq[t] *= e;
          bk2[t] *= e;
        }
        const k16_t<T> dMc = k16_col<T>(dMl, LDJ, 16 * bi, 16 * bj, lane), dAc = k16_col<T>(dAl, LDJ, 16 * bi, 16 * bj, lane);
        X23[bj] = dgb ? mma_k16r_split<T>(dMc, bq, X23[bj]) : mma_k16r<T>(dMc, k16_pack<T>(bq), X23[bj]);
        X23[bj] = dgb ? mma_k16r_split<T>(dAc, bk2, X23[bj]) : mma_k16r<T>(dAc, k16_pack<T>(bk2), X23[bj]);
      }
    ga_load<T, BT, D, DV, 3>(nxt, rows_x, b, size_t(itn), itn % H, H, tid, wave, lane);
    // B5. assemble dq, dk, dG with exact q, k and fp32 factors: dq into dqa, the row and column
    //     parts of dk into X1 and X23, then the steep blocks' pairwise diagonal terms, then dk and dG
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float er = eL[bb][r];
        dqa[bb][r] *= er;
        X1[bb][r] *= er;
        X23[bb][r] *= ecL[bb][r];
      }
    }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const bool steep = Tb[bb] < -kSteepGate;
      if (__any(steep)) steep_diag_grad<T, LDK, LDJ>(Qb, Kb, dMl, dAl, bb, 16 * wave + cc, cc, g4, L[bb], steep, dqa[bb], X1[bb], X23[bb]);
    }
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      float kvv[4], qvv[4];
      col4_load<T>(Kb, LDK, 16 * bb, 16 * wave, lane, kvv);
      col4_load<T>(Qb, LDK, 16 * bb, 16 * wave, lane, qvv);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float dq = dqa[bb][r], krow = X1[bb][r], kcol = X23[bb][r];
        X1[bb][r] = krow + kcol;                            // dk
        X23[bb][r] = qvv[r] * dq + kvv[r] * (krow - kcol);  // dG
      }
    }
    csum += __shfl_xor(csum, 16, 64);
    csum += __shfl_xor(csum, 32, 64);
    ga_load<T, BT, D, DV, 4>(nxt, rows_x, b, size_t(itn), itn % H, H, tid, wave, lane);
    // B6. dg = reverse cumulative sum of dG over the chunk, dG_last added at the last row
    {
      float gt[NB], after_blk = rs + csum;
      float suf[NB][4];
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        float s = 0.f;
#pragma unroll
        for (int r = 3; r >= 0; --r) {
          s += X23[bb][r];
          suf[bb][r] = s;
        }
        gt[bb] = s;
      }
#pragma unroll
      for (int bb = NB - 1; bb >= 0; --bb) {
        float tot[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) tot[q] = __shfl(gt[bb], cc + 16 * q, 64);
        float later = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) later += q > g4 ? tot[q] : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) X23[bb][r] = suf[bb][r] + later + after_blk;
        after_blk += tot[0] + tot[1] + tot[2] + tot[3];
      }
    }
    __syncthreads();  // staged inputs consumed: the output staging takes their place
#pragma unroll
    for (int bb = 0; bb < NB; ++bb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * bb + 4 * g4 + r;
        stg[i * LDF + c] = dqa[bb][r];
        stg[BT * LDF + i * LDF + c] = X1[bb][r];
        stg[2 * BT * LDF + i * LDF + c] = X23[bb][r];
      }
    __syncthreads();
    // B7. own rows to dq, dk, dg; replayed rows (dk, dg) to the side buffer
#pragma unroll
    for (int x = 0; x < NK; ++x) {
      const int p = tid + NT * x;
      const int row = rows.rk[x];
      if (p < CA::NPK && row >= 0) {
        const int i = p / NPR, c0 = (p % NPR) * VN;
        if (i >= rows.own) {
          const size_t off = (size_t(row) * H + h) * D + c0;
          stq(static_cast<T*>(b.dq) + off, pack16<T>(stg + i * LDF + c0));
          stq(static_cast<T*>(b.dk) + off, pack16<T>(stg + BT * LDF + i * LDF + c0));
          stq(static_cast<T*>(b.dg) + off, pack16<T>(stg + 2 * BT * LDF + i * LDF + c0));
        } else {
          float* rg = b.replay_grad + (size_t(rows.rbase + i) * H + h) * G::W;  // odd row stride: scalar stores
#pragma unroll
          for (int t = 0; t < VN; ++t) {
            rg[G::DK + c0 + t] = stg[BT * LDF + i * LDF + c0 + t];
            rg[G::DG + c0 + t] = stg[2 * BT * LDF + i * LDF + c0 + t];
          }
        }
      }
    }
    __syncthreads();  // the next item restages every region
    // the ticket word is read again rather than the item held across the item's phases
    item = item_n;
    item_n = a.ctr ? 2 * int(gridDim.x) + tk_slot : item + int(gridDim.x);
  }
}

// ------------------------------------------------------------------------------------------
// Replayed rows: add every replay's gradient into the owning compact row, in a fixed order.
template <typename T, int D, int DV>
__global__ __launch_bounds__(128) void replay_fixup_kernel(const int32_t* rows, const int32_t* off, const int32_t* idx,
                                                           const float* rg, T* dk, T* dv, T* dg, T* dbeta, int H) {
  using G = RG<D, DV>;
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  const size_t row = size_t(rows[r]);
  const int q0 = off[r], q1 = off[r + 1];
  for (int e = threadIdx.x; e < G::W; e += blockDim.x) {
    float s = 0.f;
    for (int q = q0; q < q1; ++q) s += rg[(size_t(idx[q]) * H + h) * G::W + e];
    if (e < D) {
      T* p = dk + (row * H + h) * D + e;
      *p = from_f<T>(to_f(*p) + s);
    } else if (e < D + DV) {
      T* p = dv + (row * H + h) * DV + (e - D);
      *p = from_f<T>(to_f(*p) + s);
    } else if (e < 2 * D + DV) {
      T* p = dg + (row * H + h) * D + (e - D - DV);
      *p = from_f<T>(to_f(*p) + s);
    } else {
      T* p = dbeta + row * H + h;
      *p = from_f<T>(to_f(*p) + s);
    }
  }
}

// ------------------------------------------------------------------------------------------
template <typename T, int BT, int D, int DV>
static hipError_t dstate_launch(const KdaDims& d, const BwdRoundArgs& b, hipStream_t s) {
  if (b.r.nseq <= 0) return hipSuccess;
  constexpr int DVT = dv_tile_b<DV>();
  unsigned n = unsigned(b.r.nseq) * d.H * (DV / DVT);
  n = (n + 7) / 8 * 8;
  hipLaunchKernelGGL((kda_dstate_kernel<T, BT, D, DV, DVT>), dim3(n), dim3(64 * state_waves<D>()), 0, s, b, d.H);
  return hipGetLastError();
}

template <typename T, int BT, int D, int DV>
static hipError_t grad_launch(const KdaDims& d, const BwdRoundArgs& b, hipStream_t s) {
  if (b.r.nchunk <= 0) return hipSuccess;
  hipLaunchKernelGGL((kda_grad_kernel<T, BT, D, DV>), dim3(persistent_grid(unsigned(b.r.nchunk) * d.H)),
                     dim3(GACfg<T, BT, D, DV>::NT), 0, s, b, d.H);
  return hipGetLastError();
}

template <typename T, int D, int DV>
static hipError_t fixup_launch(const KdaDims& d, const int32_t* rows, const int32_t* off, const int32_t* idx,
                               int32_t n, const float* rg, void* dk, void* dv, void* dg, void* dbeta, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL((replay_fixup_kernel<T, D, DV>), dim3(unsigned(n) * d.H), dim3(128), 0, s, rows, off, idx, rg,
                     static_cast<T*>(dk), static_cast<T*>(dv), static_cast<T*>(dg), static_cast<T*>(dbeta), d.H);
  return hipGetLastError();
}

#define HARTS_KDA_BWD_CONFIGS(X) \
  X(bf16, 64, 128, 128)          \
  X(bf16, 64, 64, 64)            \
  X(bf16, 32, 64, 64)            \
  X(bf16, 32, 32, 32)            \
  X(float, 16, 16, 16)           \
  X(float, 32, 32, 32)

// fp32 configurations only: bf16 runs the slab passes (kda_slab.hip)
hipError_t launch_kda_dstate(const KdaDims& d, const BwdRoundArgs& b, hipStream_t s) {
#define X(T_, B_, D_, V_)                                                             \
  if constexpr (sizeof(T_) == 4)                                                      \
    if (d.dtype == 1 && d.BT == B_ && d.D == D_ && d.DV == V_) return dstate_launch<T_, B_, D_, V_>(d, b, s);
  HARTS_KDA_BWD_CONFIGS(X)
#undef X
  return hipErrorNotSupported;
}

hipError_t launch_kda_grad(const KdaDims& d, const BwdRoundArgs& b, hipStream_t s) {
#define X(T_, B_, D_, V_) \
  if (d.dtype == (sizeof(T_) == 2 ? 0 : 1) && d.BT == B_ && d.D == D_ && d.DV == V_) return grad_launch<T_, B_, D_, V_>(d, b, s);
  HARTS_KDA_BWD_CONFIGS(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_replay_fixup(const KdaDims& d, const int32_t* rows, const int32_t* off, const int32_t* idx,
                               int32_t n, const float* rg, void* dk, void* dv, void* dg, void* dbeta, hipStream_t s) {
#define X(T_, B_, D_, V_) \
  if (d.dtype == (sizeof(T_) == 2 ? 0 : 1) && d.D == D_ && d.DV == V_) return fixup_launch<T_, D_, V_>(d, rows, off, idx, n, rg, dk, dv, dg, dbeta, s);
  HARTS_KDA_BWD_CONFIGS(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace harts
