// Chunkwise gated-delta forward on gfx950: per-chunk preparation and the
// serial state pass, one packed round at a time.
//
// Per chunk of <= BT tokens (HARTS close-reading blog, sections 1.2 and 4.2:
// fixed chunk length, parallel inside a chunk, state passed between chunks),
// with G the in-chunk cumulative log-decay:
//   A = strict_lower(gated K K^T), M = lower(gated Q K^T),
//   T = (I + diag(beta) A)^{-1} diag(beta),
//   W = T (K e^G), U' = T V,
//   U = U' - W S0,  O = (Q e^G) S0 + M U,  S = diag(e^{G_last}) S0 + (K e^{G_last - G})^T U.
// The bf16 serial passes take Q e^G and M (both written here) and form their products with
// Qeff = Q e^G - M W through them; the fp32 state-gradient kernel reads Qeff^T.
// "gated" products use e^{G_i - G_j} factored through 16-row sub-block
// reference points: for rows i in block bi and j in block bj < bi,
// e^{G_i - G_j} = e^{G_i - F_bi} * e^{F_bi - F_{bj+1}} * e^{F_{bj+1} - G_j}, F_b the
// log-decay before block b; every factor is an exponential of a non-positive
// number, formed directly.  Within a diagonal block the pair (i, j <= i) factors
// as e^{L_i} * e^{-L_j} (L the block-local cumulative log-decay) when
// L_i >= -kSteepGate, which bounds both factors by e^{kSteepGate}; the terms of
// the "steep" (row, channel) elements with L_i < -kSteepGate are masked out of
// the matrix-core product and summed pairwise, e^{L_i - L_j} directly, in a
// separate step.  The decision depends on row i alone, so a row's results never
// depend on the rows after it (tree and expanded execution stay bitwise equal),
// and the result is exact (to fp32 rounding) for every g <= 0, including the
// g -> -inf limit.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "state_common.h"

namespace harts {

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
__host__ __device__ constexpr int pair_index(int bi, int bj) { return (bi - 2) * (bi - 1) / 2 + bj; }

template <typename T, int BT, int D, int DV>
struct PrepLayout {
  static constexpr int NB = BT / 16, VN = 16 / sizeof(T), PAD = VN;
  static constexpr int LDK = D + PAD, LDV = DV + PAD, LDJ = BT + PAD, LDF = D + 4, LDA = BT + 4;
  static constexpr int NPX = NB >= 3 ? (NB - 1) * (NB - 2) / 2 : 0;
  static constexpr size_t ES = sizeof(T);
  static constexpr size_t al(size_t x) { return (x + 15) / 16 * 16; }
  // R1: Gf (fp32 [BT][LDF]) | X (fp32 [BT][LDA]) + M ([BT][LDJ], backward)
  static constexpr size_t X_SZ = al(size_t(BT) * LDA * 4), ML_SZ = al(size_t(BT) * LDJ * ES);
  static constexpr size_t R1 = cmax(al(size_t(BT) * LDF * 4), X_SZ + ML_SZ);
  static constexpr size_t O_GF = 0, O_X = 0, O_ML = X_SZ;
  // four operand slots, reused after the A/M products:
  //   S0: Kr -> K~ (-> W, backward)   S1: Qr -> Q~ (backward)   S2: Kc0 -> V   S3: Kcd -> KhT
  static constexpr size_t SLOT = al(cmax(size_t(BT) * LDK * ES, size_t(BT) * LDV * ES));
  static constexpr size_t O_S0 = R1, O_S1 = O_S0 + SLOT, O_S2 = O_S1 + SLOT, O_S3 = O_S2 + SLOT, O_SX = O_S3 + SLOT;
  // SX: Kcx (pair-scaled column operands); afterwards the tail of KhT and T
  static constexpr size_t KHT_SZ = al(size_t(D) * LDJ * ES), TM_SZ = al(size_t(BT) * LDJ * ES);
  static constexpr size_t O_TM = O_S3 + KHT_SZ;
  static constexpr size_t SX = cmax(al(size_t(NPX) * 16 * LDK * ES), O_TM + TM_SZ > O_SX ? O_TM + TM_SZ - O_SX : 0);
  static constexpr size_t O_A = O_SX + SX;  // A (fp32 [BT][LDA])
  static constexpr size_t O_VEC = O_A + X_SZ;
  // vectors (fp32): Tv[NB][D], Fv[NB+1][D], EF[NB+1][D], EH[NB][D], Sx[NPX][D], bet[BT],
  // DA[NB][16][16] and DM[NB][16][16] (pairwise diagonal-block sums of the steep elements),
  // stf[NB + 1] (int: block b has a steep element; [NB]: any block has), then the steep mask
  // (bytes [BT][D / VN]: bit t of byte (i, g) marks element (i, VN g + t))
  static constexpr size_t TV = 0, FV = TV + NB * D, EF = FV + (NB + 1) * D, EH = EF + (NB + 1) * D,
                          SXV = EH + NB * D, BET = SXV + (NPX > 0 ? NPX : 1) * D, DAV = BET + BT,
                          DMV = DAV + NB * 256, STF = DMV + NB * 256, SMK = STF + NB + 1;
  static constexpr int MKR = D / VN;  // mask bytes per row
  // raw k and q of one 16-row block for the pairwise steep terms ([16][LDK] each): over A, which
  // is first written after that step, when it fits there
  static constexpr size_t STG_SZ = al(size_t(2) * 16 * LDK * ES);
  static constexpr bool STG_IN_A = STG_SZ <= X_SZ;
  static constexpr size_t O_STG = STG_IN_A ? O_A : O_VEC + SMK * 4 + al(size_t(BT) * MKR);
  static constexpr size_t TOTAL = O_VEC + SMK * 4 + al(size_t(BT) * MKR) + (STG_IN_A ? 0 : STG_SZ);
  static_assert(TOTAL <= 160 * 1024, "prep kernel LDS budget");
};

// Register-resident global inputs of one (chunk, head) item.  Thread tid owns the
// 16-byte pieces p = tid + CNT * x of the [BT][D] key/query/gate tiles (row p / NPR)
// and of the [BT][DV] value tile.  Gates, keys, queries and beta are fetched one item
// ahead; values are fetched at the start of their own item (first used halfway).
template <typename T, int BT, int D, int DV>
struct PrepIn {
  static constexpr int VN = 16 / sizeof(T);
  static constexpr int NPR = D / VN, NPK = BT * NPR, NK = (NPK + CNT - 1) / CNT;
  static constexpr int NPRV = DV / VN, NPV = BT * NPRV, NV = (NPV + CNT - 1) / CNT;
  static constexpr bool SAMEV = NPR == NPRV;  // value pieces sit on the key pieces' rows
  f32x4 g[NK], k[NK], q[NK];
  T beta;
};
template <typename T, int BT, int D, int DV>
struct PrepRows {
  using P = PrepIn<T, BT, D, DV>;
  int rk[P::NK], rv_[P::SAMEV ? 1 : P::NV], rb;
  __device__ __forceinline__ int rv(int x) const {
    if constexpr (P::SAMEV) return rk[x];
    else return rv_[x];
  }
};

// Loads are unconditional (clamped to a valid row) so that no register of an in-flight
// load is written on another path, which would force an early wait; padding rows
// are masked where the values are used.
template <typename T, int BT, int D, int DV>
__device__ __forceinline__ void prep_rows(PrepRows<T, BT, D, DV>& r, const int32_t* crows, int chunk, int tid) {
  using P = PrepIn<T, BT, D, DV>;
  const int32_t* cr = crows + size_t(chunk) * BT;
#pragma unroll
  for (int x = 0; x < P::NK; ++x) {
    const int p = tid + CNT * x;
    r.rk[x] = cr[(p < P::NPK ? p : P::NPK - 1) / P::NPR];
  }
  if constexpr (!P::SAMEV) {
#pragma unroll
    for (int x = 0; x < P::NV; ++x) {
      const int p = tid + CNT * x;
      r.rv_[x] = cr[(p < P::NPV ? p : P::NPV - 1) / P::NPRV];
    }
  }
  r.rb = cr[tid < BT ? tid : BT - 1];
}

// PART selects a part of the fetch (-1: all): 0 g and beta, 1 k, 2 q.  The persistent loop
// issues the parts between phases so that a workgroup's loads do not queue at its top.
template <typename T, int BT, int D, int DV, int PART = -1>
__device__ __forceinline__ void prep_load(PrepIn<T, BT, D, DV>& o, const PrepRows<T, BT, D, DV>& r, const RoundArgs& a,
                                          int h, int H, int tid) {
  using P = PrepIn<T, BT, D, DV>;
#pragma unroll
  for (int x = 0; x < P::NK; ++x) {
    const int c0 = ((tid + CNT * x) % P::NPR) * P::VN;
    const size_t off = (size_t(r.rk[x] >= 0 ? r.rk[x] : 0) * H + h) * D + c0;
    if constexpr (PART < 0 || PART == 0) o.g[x] = ldq(static_cast<const T*>(a.g) + off);
    if constexpr (PART < 0 || PART == 1) o.k[x] = ldq(static_cast<const T*>(a.k) + off);
    if constexpr (PART < 0 || PART == 2) o.q[x] = ldq(static_cast<const T*>(a.q) + off);
  }
  if constexpr (PART < 0 || PART == 0) o.beta = static_cast<const T*>(a.beta)[size_t(r.rb >= 0 ? r.rb : 0) * H + h];
}

template <typename T, int BT, int D, int DV>
__device__ __forceinline__ void prep_load_v(f32x4* v, const PrepRows<T, BT, D, DV>& r, const RoundArgs& a, int h, int H,
                                            int tid) {
  using P = PrepIn<T, BT, D, DV>;
#pragma unroll
  for (int x = 0; x < P::NV; ++x) {
    const int c0 = ((tid + CNT * x) % P::NPRV) * P::VN;
    const int rr = r.rv(x);
    v[x] = ldq(static_cast<const T*>(a.v) + (size_t(rr >= 0 ? rr : 0) * H + h) * DV + c0);
  }
}

// An operand fragment of rows r0 + lane % 16 (contraction = channels k0 + ..., as Mma<T>::kc reads
// them) with the steep elements of its row zeroed; mrow is the row's mask (bit t of byte g marks
// channel VN g + t, VN = 16 / sizeof(T)).
template <typename T>
__device__ __forceinline__ typename Mma<T>::Frag steep_masked(typename Mma<T>::Frag f, const uint8_t* mrow, int k0,
                                                              int lane) {
  if constexpr (sizeof(T) == 2) {
    const int bits = mrow[(k0 + 8 * (lane >> 4)) / 8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if ((bits >> e) & 1) f[e] = bf16(0.f);
    return f;
  } else {
    const int c = k0 + (lane >> 4);
    return ((mrow[c / 4] >> (c % 4)) & 1) ? 0.f : f;
  }
}

// Pairwise diagonal-block terms of the steep elements (row i, channel c with L_ic < -kSteepGate,
// marked in the mask), block after block for the blocks that have one: the raw k and q of the
// block's rows are staged from the registers that hold them (PrepIn, thread-owned pieces) into
// Sk, Sq ([16][LDK]), then thread tid takes entry (i, j) = (tid / 16 % 16, tid % 16) of A
// (tid < 256) or M (tid >= 256) and sums x_ic k_jc e^{L_ic - L_jc} over row i's steep channels,
// x = k for A (i > j) and q for M (i >= j), L the block-local cumulative log-decays in Gf.  No
// global memory is read, so the loads in flight for the next item are not waited for.  Called
// by the whole workgroup; ends with a barrier.
template <typename T, int BT, int D, int DV>
__device__ __forceinline__ void steep_diag_sums(float* DA, float* DM, T* Sk, T* Sq, const float* Gf,
                                                const uint8_t* smask, const int* stf,
                                                const PrepIn<T, BT, D, DV>& cur, const PrepRows<T, BT, D, DV>& rows,
                                                int tid) {
  using P = PrepIn<T, BT, D, DV>;
  constexpr int NB = BT / 16, VN = 16 / sizeof(T), LDF = D + 4, MKR = D / VN, LDK = D + VN;
  static_assert(CNT >= 512, "one thread per entry of A and of M");
  const bool isM = tid >= 256;
  const int i = (tid >> 4) & 15, j = tid & 15;
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
  // rolled loops: this step runs only for steep blocks and must not grow the kernel's code
#pragma unroll 1
  for (int b = 0; b < NB; ++b) {
    if (!stf[b]) continue;
#pragma unroll
    for (int x = 0; x < P::NK; ++x) {
      const int p = tid + CNT * x;
      const int r = p / P::NPR - 16 * b, c0 = (p % P::NPR) * VN;
      if (p < P::NPK && r >= 0 && r < 16) {
        const bool ok = rows.rk[x] >= 0;
        stq(Sk + r * LDK + c0, ok ? cur.k[x] : z4);
        stq(Sq + r * LDK + c0, ok ? cur.q[x] : z4);
      }
    }
    __syncthreads();
    if (tid < 512) {
      float acc = 0.f;
      if (isM ? i >= j : i > j) {
        const T* xp = (isM ? Sq : Sk) + i * LDK;
        const T* kp = Sk + j * LDK;
        const float* Li = Gf + (16 * b + i) * LDF;
        const float* Lj = Gf + (16 * b + j) * LDF;
        const uint8_t* mrow = smask + (16 * b + i) * MKR;
#pragma unroll 1
        for (int g = 0; g < MKR; ++g) {
          const int bits = mrow[g];
          if (!bits) continue;
#pragma unroll
          for (int t = 0; t < VN; ++t)
            if ((bits >> t) & 1)
              acc += to_f(xp[VN * g + t]) * to_f(kp[VN * g + t]) * __expf(Li[VN * g + t] - Lj[VN * g + t]);
        }
      }
      (isM ? DM : DA)[b * 256 + i * 16 + j] = acc;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------
// Per-chunk preparation.  Persistent: one workgroup of CNT threads per CU walks the
// (chunk, head) items of the round; the next item's rows and inputs are fetched into
// registers while the current item computes.
// PM: 0 forward operands, 1 backward operands, 2 both (bf16 only: a forward that keeps
// everything the backward needs).
template <typename T, int BT, int D, int DV, int PM>
__global__ __launch_bounds__(CNT) void kda_prep_kernel(RoundArgs a, int H) {
  using Ly = PrepLayout<T, BT, D, DV>;
  using In = PrepIn<T, BT, D, DV>;
  using Rows = PrepRows<T, BT, D, DV>;
  using MM = Mma<T>;
  // bf16: operands of the slab-parallel serial passes in the permuted fragment-major layout
  constexpr bool PF = sizeof(T) == 2;
  constexpr bool BWD = PM != 0, FO = PM != 1;
  static_assert(PM != 2 || PF, "kept backward operands need the fragment-major layouts");
  static_assert(!PF || size_t(BT) * Ly::LDK * sizeof(T) <= Ly::KHT_SZ, "token-major K^ fits its slot");
  constexpr int NB = Ly::NB, LDK = Ly::LDK, LDV = Ly::LDV, LDJ = Ly::LDJ, LDF = Ly::LDF, LDA = Ly::LDA;
  constexpr int VN = In::VN, NK = In::NK, NV = In::NV, NPR = In::NPR, NPRV = In::NPRV;
  __shared__ __attribute__((aligned(16))) char smem[Ly::TOTAL];
  float* Gf = reinterpret_cast<float*>(smem + Ly::O_GF);
  float* Xf = reinterpret_cast<float*>(smem + Ly::O_X);
  T* Ml = reinterpret_cast<T*>(smem + Ly::O_ML);
  T* Kr = reinterpret_cast<T*>(smem + Ly::O_S0);
  T* Kt = Kr;  // K~ after the products, then W (backward)
  T* Qr = reinterpret_cast<T*>(smem + Ly::O_S1);
  T* Kc0 = reinterpret_cast<T*>(smem + Ly::O_S2);
  T* Vl = Kc0;
  T* Kcd = reinterpret_cast<T*>(smem + Ly::O_S3);
  T* KhT = Kcd;  // fp32: K^^T [D][LDJ]; bf16: K^ token-major [BT][LDK] (read back transposed)
  T* Kcx = reinterpret_cast<T*>(smem + Ly::O_SX);
  T* Tm = reinterpret_cast<T*>(smem + Ly::O_TM);
  float* Af = reinterpret_cast<float*>(smem + Ly::O_A);
  float* vec = reinterpret_cast<float*>(smem + Ly::O_VEC);
  float* Tv = vec + Ly::TV;
  float* Fv = vec + Ly::FV;
  float* EF = vec + Ly::EF;
  float* EH = vec + Ly::EH;
  float* Sx = vec + Ly::SXV;
  float* bet = vec + Ly::BET;
  float* DA = vec + Ly::DAV;
  float* DM = vec + Ly::DMV;
  int* stf = reinterpret_cast<int*>(vec + Ly::STF);
  uint8_t* smask = reinterpret_cast<uint8_t*>(vec + Ly::SMK);

  const int tid0 = threadIdx.x;
  if (a.zero && blockIdx.x == 0)
    for (int i = tid0; i < a.nzero; i += CNT) a.zero[i] = 0;
  const int nitems = a.nchunk * H;
  int item = blockIdx.x;
  if (item >= nitems) return;
  // rows_x: rows of the item whose inputs are in nxt; rows_n: rows of the item after it.
  // cur is taken from nxt at the top of each iteration, before the next fetch is issued.
  Rows rows, rows_x, rows_n;
  In cur, nxt;
  prep_rows<T, BT, D, DV>(rows_x, a.crows, item / H, tid0);
  prep_load<T, BT, D, DV>(nxt, rows_x, a, item % H, H, tid0);
  int item_n = item + gridDim.x;
  prep_rows<T, BT, D, DV>(rows_n, a.crows, (item_n < nitems ? item_n : item) / H, tid0);
  __shared__ int tk_slot;
  // Nothing fetched before the loop stays outstanding into it.  The compiler's wait counts at the
  // loop head take the more cautious of its two entries; the prologue issues only a few memory
  // operations after its fetches, the loop body many (the item's stores), so without this wait
  // every item would wait at its top for nearly all of the previous item's stores to complete.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

  while (item < nitems) {
    // thread-derived addresses are recomputed per item instead of being held across the loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    // the wave index is uniform: tile selection and addressing derived from it stay scalar
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = item % H;
    const size_t wsi = size_t(item);  // (round-local chunk) * H + head
    cur = nxt;
    rows = rows_x;
    int tk = 0;  // thread 0: the ticket for the item after the next one
    if (a.ctr && tid == 0) tk = draw_ticket(a.ctr);
    // this item's values; fetch ahead: inputs of the next item, rows of the one after
    f32x4 vv[NV];
    prep_load_v<T, BT, D, DV>(vv, rows, a, h, H, tid);
    const int hn = (item_n < nitems ? item_n : item) % H;
    prep_load<T, BT, D, DV, 0>(nxt, rows_n, a, hn, H, tid);
    rows_x = rows_n;

    // 1. g -> Gf (fp32), beta
#pragma unroll
    for (int x = 0; x < NK; ++x) {
      const int p = tid + CNT * x;
      if (p < In::NPK) {
        const int i = p / NPR, c0 = (p % NPR) * VN;
        float gv[VN];
        unpack16<T>(rows.rk[x] >= 0 ? cur.g[x] : f32x4{0.f, 0.f, 0.f, 0.f}, gv);
#pragma unroll
        for (int t = 0; t < VN; t += 4)
          stq(Gf + i * LDF + c0 + t, f32x4{gv[t], gv[t + 1], gv[t + 2], gv[t + 3]});
      }
    }
    if (tid < BT) bet[tid] = rows.rb >= 0 ? to_f(cur.beta) : 0.f;
    if (tid <= NB) stf[tid] = 0;
    __syncthreads();
    // 2. block-local cumulative sums L and block totals
    HARTS_STRIDED(idx, tid, NB * D, CNT) {
      const int b = idx / D, c = idx % D;
      float v[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) v[t] = Gf[(16 * b + t) * LDF + c];
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        acc += v[t];
        Gf[(16 * b + t) * LDF + c] = acc;
      }
      Tv[b * D + c] = acc;
    }
    if (a.ctr && tid == 0) tk_slot = tk;
    __syncthreads();
    // the item after the next one: its rows are fetched a whole item ahead of their use
    const int item_nn = a.ctr ? 2 * int(gridDim.x) + tk_slot : item_n + int(gridDim.x);
    prep_rows<T, BT, D, DV>(rows_n, a.crows, (item_nn < nitems ? item_nn : item) / H, tid);
    prep_load<T, BT, D, DV, 1>(nxt, rows_x, a, hn, H, tid);
    // 3. per channel: block entry log-decays F_b, e^{F_b}, e^{F_end - F_{b+1}}, pair scales
    HARTS_STRIDED(c, tid, D, CNT) {
      float f = 0.f, fv[NB + 1], tb[NB];
      fv[0] = 0.f;
      Fv[c] = 0.f;
      EF[c] = 1.f;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        tb[b] = Tv[b * D + c];
        f += tb[b];
        fv[b + 1] = f;
        Fv[(b + 1) * D + c] = f;
        EF[(b + 1) * D + c] = __expf(f);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) EH[b * D + c] = __expf(f - fv[b + 1]);
#pragma unroll
      for (int bi = 2; bi < NB; ++bi)
#pragma unroll
        for (int bj = 0; bj + 2 <= bi; ++bj) Sx[pair_index(bi, bj) * D + c] = __expf(fv[bi] - fv[bj + 1]);
    }
    __syncthreads();
    // 4. operand arrays: Kr = k e^L, Qr = q e^L, Kc0 = k e^{T_b - L}, Kcd = k e^{-L} (0 on steep
    //    elements, L < -kSteepGate, which are marked in the mask), Kcx = Kc0 * pair scale.
    //    e^L and e^{T_b - L} stay in registers for step 6.
    float Er[NK][VN], En[NK][VN];  // e^{L}, e^{T_b - L} of this thread's elements
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < NK; ++x) {
      const int p = tid + CNT * x;
      if (p < In::NPK) {
        const int i = p / NPR, c0 = (p % NPR) * VN, b = i / 16;
        float kk[VN], qq[VN], kr[VN], qr[VN], kc[VN], kd[VN];
        unpack16<T>(rows.rk[x] >= 0 ? cur.k[x] : z4, kk);
        unpack16<T>(rows.rk[x] >= 0 ? cur.q[x] : z4, qq);
        int bits = 0;
#pragma unroll
        for (int t = 0; t < VN; ++t) {
          const float Lv = Gf[i * LDF + c0 + t], Tb = Gf[(16 * b + 15) * LDF + c0 + t];
          const bool st = Lv < -kSteepGate;
          const float er = __expf(Lv), ec = __expf(Tb - Lv), en = __expf(st ? 0.f : -Lv);
          Er[x][t] = er;
          En[x][t] = ec;
          kr[t] = kk[t] * er;
          qr[t] = qq[t] * er;
          kc[t] = kk[t] * ec;
          kd[t] = st ? 0.f : kk[t] * en;
          bits |= int(st) << t;
        }
        smask[i * Ly::MKR + c0 / VN] = uint8_t(bits);
        if (bits) stf[b] = stf[NB] = 1;
        stq(Kr + i * LDK + c0, pack16<T>(kr));
        stq(Qr + i * LDK + c0, pack16<T>(qr));
        stq(Kc0 + i * LDK + c0, pack16<T>(kc));
        stq(Kcd + i * LDK + c0, pack16<T>(kd));
        for (int bi = b + 2; bi < NB; ++bi) {
          const int pp = pair_index(bi, b);
          float xs[VN];
#pragma unroll
          for (int t = 0; t < VN; ++t) xs[t] = kc[t] * Sx[pp * D + c0 + t];
          stq(Kcx + (pp * 16 + i - 16 * b) * LDK + c0, pack16<T>(xs));
        }
      } else {
#pragma unroll
        for (int t = 0; t < VN; ++t) Er[x][t] = En[x][t] = 1.f;
      }
    }
    __syncthreads();
    prep_load<T, BT, D, DV, 2>(nxt, rows_x, a, hn, H, tid);
    // 4b. steep channels of a diagonal block: A_ij and M_ij terms sum_c x_ic k_jc e^{L_ic - L_jc}
    //     formed pairwise (x = k for A, q for M) from the raw inputs, one entry per thread
    if (stf[NB])
      steep_diag_sums<T, BT, D, DV>(DA, DM, reinterpret_cast<T*>(smem + Ly::O_STG),
                                    reinterpret_cast<T*>(smem + Ly::O_STG) + 16 * LDK, Gf, smask, stf, cur, rows, tid);
    // 5. A (strict lower, fp32) into Af; M (lower incl.) to the workspace (and Ml), one 16x16 tile each
    T* Mg = static_cast<T*>(a.ws.Mm) + wsi * BT * BT;
    {
      constexpr int NTA = NB * (NB + 1) / 2, NTT = NTA + NB * NB;
      HARTS_STRIDED(jb, wave, NTT, CNW) {
        if (jb < NTA) {
          int bi = 0;
          while ((bi + 1) * (bi + 2) / 2 <= jb) ++bi;
          const int bj = jb - bi * (bi + 1) / 2;
          const T* col = bi == bj ? Kcd + 16 * bj * LDK
                         : (bi - bj == 1 ? Kc0 + 16 * bj * LDK : Kcx + pair_index(bi, bj) * 16 * LDK);
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          if (bi == bj && stf[bi]) {
            // steep elements of the rows masked out, their terms summed pairwise (DA)
            const uint8_t* mrow = smask + (16 * bi + (lane & 15)) * Ly::MKR;
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += MM::KS)
              acc = MM::mma(steep_masked<T>(MM::kc(Kr + 16 * bi * LDK, LDK, 0, k0, lane), mrow, k0, lane),
                            MM::kc(col, LDK, 0, k0, lane), acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += DA[bi * 256 + crow(lane, r) * 16 + ccol(lane)];
          } else {
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += MM::KS)
              acc = MM::mma(MM::kc(Kr + 16 * bi * LDK, LDK, 0, k0, lane), MM::kc(col, LDK, 0, k0, lane), acc);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 16 * bi + crow(lane, r), j = 16 * bj + ccol(lane);
            Af[i * LDA + j] = (bi == bj && i <= j) ? 0.f : acc[r];
          }
        } else {
          const int t = jb - NTA, bi = t / NB, bj = t % NB;
          const int i = 16 * bi + ccol(lane), j0 = 16 * bj + crow(lane, 0);
          float v[4] = {0.f, 0.f, 0.f, 0.f};
          if (bj <= bi) {
            const T* col = bi == bj ? Kcd + 16 * bj * LDK
                           : (bi - bj == 1 ? Kc0 + 16 * bj * LDK : Kcx + pair_index(bi, bj) * 16 * LDK);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (bi == bj && stf[bi]) {
              const uint8_t* mrow = smask + (16 * bi + (lane & 15)) * Ly::MKR;
#pragma unroll
              for (int k0 = 0; k0 < D; k0 += MM::KS)
                acc = MM::mma(MM::kc(col, LDK, 0, k0, lane),
                              steep_masked<T>(MM::kc(Qr + 16 * bi * LDK, LDK, 0, k0, lane), mrow, k0, lane), acc);
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[r] += DM[bi * 256 + ccol(lane) * 16 + crow(lane, r)];
            } else {
#pragma unroll
              for (int k0 = 0; k0 < D; k0 += MM::KS)
                acc = MM::mma(MM::kc(col, LDK, 0, k0, lane), MM::kc(Qr + 16 * bi * LDK, LDK, 0, k0, lane), acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = (bi == bj && j0 + r > i) ? 0.f : acc[r];
          }
          // M to the workspace: row-major for the bf16 gradient kernel, permuted fragment-major
          // (rows i, contraction j) for the bf16 serial passes, fragment-major for the fp32
          // serial pass
          if constexpr (PF) {
            if constexpr (BWD) store4(Mg + i * BT + j0, v[0], v[1], v[2], v[3]);
            store4(static_cast<T*>(a.ws.Mf) + wsi * BT * BT + pf_off(i, j0, BT), v[0], v[1], v[2], v[3]);
          } else {
            fm_store<T>(Mg, BT, i, j0, v, 4);
          }
          if constexpr (BWD && !PF) store4(Ml + i * LDJ + j0, v[0], v[1], v[2], v[3]);
        }
      }
    }
    __syncthreads();
    // 6a. diagonal 16x16 blocks of X = (I + N)^{-1}, N = diag(beta) A_bb strictly lower and so
    //     nilpotent: (I + N)^{-1} = (I - N)(I + N^2)(I + N^4)(I + N^8).  fp32 matrix cores, each
    //     operand kept with its transpose in accumulator layout (mma16_f32(c(Z^T), c(Y)) = Z Y).
    if (wave < NB) {
      const int b = wave, lr = lane & 15, lg = lane >> 4;
      const float bl = bet[16 * b + lr];
      const f32x4 arow = ldq(Af + (16 * b + lr) * LDA + 16 * b + 4 * lg);
      f32x4 n, nt, q, qt;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * lg + r;
        n[r] = bet[16 * b + i] * Af[(16 * b + i) * LDA + 16 * b + lr];
        nt[r] = bl * arow[r];
        const float id = i == lr ? 1.f : 0.f;
        q[r] = id - n[r];
        qt[r] = id - nt[r];
      }
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const f32x4 n2 = mma16_f32(nt, n, z), n2t = mma16_f32(n, nt, z);
      const f32x4 n4 = mma16_f32(n2t, n2, z), n4t = mma16_f32(n2, n2t, z);
      const f32x4 n8 = mma16_f32(n4t, n4, z);
      const f32x4 p1 = mma16_f32(qt, n2, q), p1t = mma16_f32(n2, qt, qt);
      const f32x4 p2 = mma16_f32(p1t, n4, p1), p2t = mma16_f32(n4, p1t, p1t);
      const f32x4 x = mma16_f32(p2t, n8, p2);
#pragma unroll
      for (int r = 0; r < 4; ++r) Xf[(16 * b + 4 * lg + r) * LDA + 16 * b + lr] = x[r];
    }
    // 6b. K~ = k e^G, K^ = k e^{G_last - G} (transposed), Q~ = q e^G, V; e^{G_last}
#pragma unroll
    for (int x = 0; x < NK; ++x) {
      const int p = tid + CNT * x;
      if (p < In::NPK) {
        const int i = p / NPR, c0 = (p % NPR) * VN, b = i / 16;
        float kk[VN], qq[VN], kt[VN], qt[VN], kh[VN];
        unpack16<T>(rows.rk[x] >= 0 ? cur.k[x] : z4, kk);
        unpack16<T>(rows.rk[x] >= 0 ? cur.q[x] : z4, qq);
#pragma unroll
        for (int t = 0; t < VN; ++t) {
          const float er = Er[x][t], ef = EF[b * D + c0 + t];
          kt[t] = kk[t] * er * ef;
          qt[t] = qq[t] * er * ef;
          kh[t] = kk[t] * En[x][t] * EH[b * D + c0 + t];
        }
        stq(Kt + i * LDK + c0, pack16<T>(kt));
        if constexpr (BWD && !PF) fm_store<T>(static_cast<T*>(a.ws.Kh) + wsi * BT * D, D, i, c0, kh, VN);
        if (BWD || PF) stq(Qr + i * LDK + c0, pack16<T>(qt));
        else fm_store<T>(static_cast<T*>(a.ws.Qt) + wsi * BT * D, D, i, c0, qt, VN);
        if constexpr (PF) {
          stq(KhT + i * LDK + c0, pack16<T>(kh));
        } else {
#pragma unroll
          for (int t = 0; t < VN; ++t) KhT[(c0 + t) * LDJ + i] = from_f<T>(kh[t]);
        }
      }
    }
#pragma unroll
    for (int x = 0; x < NV; ++x) {
      const int p = tid + CNT * x;
      if (p < In::NPV) stq(Vl + (p / NPRV) * LDV + (p % NPRV) * VN, rows.rv(x) >= 0 ? vv[x] : z4);
    }
    HARTS_STRIDED(c, tid, D, CNT) a.ws.El[wsi * D + c] = EF[NB * D + c];
    __syncthreads();
    // 7. off-diagonal blocks of X, column block j per wave, with fp32 matrix cores:
    //    X_ij = -X_ii sum_{m=j}^{i-1} diag(beta_i) A_im X_mj; then T = X diag(beta) (bf16/fp32) into Tm.
    if (wave < NB) {
      const int j = wave, lr = lane & 15, lg = lane >> 4;
      f32x4 xb[NB];
#pragma unroll
      for (int m = 0; m < NB; ++m) xb[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) xb[j][s] = Xf[(16 * j + 4 * lg + s) * LDA + 16 * j + lr];
#pragma unroll
      for (int i = 1; i < NB; ++i) {
        if (i <= j) continue;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const float bi = bet[16 * i + lr];
#pragma unroll
        for (int m = 0; m < NB; ++m) {
          if (m < j || m >= i) continue;
          f32x4 pa = ldq(Af + (16 * i + lr) * LDA + 16 * m + 4 * lg);
#pragma unroll
          for (int s = 0; s < 4; ++s) pa[s] *= bi;
          acc = mma16_f32(pa, xb[m], acc);
        }
        const f32x4 pd = ldq(Xf + (16 * i + lr) * LDA + 16 * i + 4 * lg);
        const f32x4 r2 = mma16_f32(pd, acc, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          xb[i][s] = -r2[s];
          Xf[(16 * i + 4 * lg + s) * LDA + 16 * j + lr] = -r2[s];
        }
      }
      const float bc = bet[16 * j + lr];
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          Tm[(16 * i + 4 * lg + s) * LDJ + 16 * j + lr] = from_f<T>(i < j ? 0.f : xb[i][s] * bc);
    } else {
      // the other waves export what does not depend on T: K^^T (bf16) and A (backward)
      constexpr int HN = CNT - 64 * NB;
      const int ht = tid - 64 * NB;
      if constexpr (PF) {
        // K^^T [D][BT] permuted fragment-major from the token-major K^: block (channel block cb,
        // token block kb), lane l: channel 16 cb + l % 16, tokens 32 kb + 4 (l / 16) + {0..3} and
        // the same + 16, by two transposing reads (lane q of a 16-lane group points at 4
        // consecutive channels of token 4 (q / 4) + ...)
        T* khg = static_cast<T*>(a.ws.KhT) + wsi * D * BT;
        HARTS_STRIDED(pc, ht, D * BT / 8, HN) {
          const int blk = pc / 64, l = pc % 64, q = l & 15;
          const int cb = blk / (BT / 32), kb = blk % (BT / 32);
          const T* src = KhT + (32 * kb + 4 * (l >> 4) + (q >> 2)) * LDK + 16 * cb + 4 * (q & 3);
          const bf16x4 lo = ds_tr16(src), hi = ds_tr16(src + 16 * LDK);
          *reinterpret_cast<bf16x8*>(khg + size_t(pc) * 8) = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
      }
      if constexpr (PF) {
        // Q~ [BT][D] permuted fragment-major (rows: tokens, contraction: channels) from the
        // token-major Q~, one 16-byte operand register per piece
        T* qg = static_cast<T*>(a.ws.Qt) + wsi * BT * D;
        HARTS_STRIDED(pc, ht, BT * D / 8, HN) {
          const int blk = pc / 64, l = pc % 64;
          const int rt = blk / (D / 32), kb = blk % (D / 32);
          *reinterpret_cast<bf16x8*>(qg + size_t(pc) * 8) = pf_kc(Qr, LDK, 16 * rt, 32 * kb, l);
        }
      }
      if constexpr (BWD) {
        T* ag = static_cast<T*>(a.ws.Am) + wsi * size_t(BT) * BT;
        HARTS_STRIDED(idx, ht, BT * (BT / VN), HN) {
          const int i = idx / (BT / VN), j0 = (idx % (BT / VN)) * VN;
          float av[VN];
#pragma unroll
          for (int t = 0; t < VN; ++t) av[t] = j0 + t < i ? Af[i * LDA + j0 + t] : 0.f;
          stq(ag + i * BT + j0, pack16<T>(av));
        }
      }
    }
    __syncthreads();
    // 8. U' = T V (accumulator tiles), W = T K~; backward: T, X out.
    //    PF: W is stored negated.  fp32 backward: W stays in registers for Qeff = Q~ - M W.
    {
      T* upg = static_cast<T*>(a.ws.UpT) + wsi * DV * BT;
      T* wg = static_cast<T*>(a.ws.W) + wsi * BT * D;
      constexpr int NU = (BT / 16) * (DV / 16), NW = (D / 16) * (BT / 16);
      constexpr bool KEEPW = BWD && !PF;
      constexpr int NWW = KEEPW ? (NW + CNW - 1) / CNW : 1, NUW = (NU + CNW - 1) / CNW;
      f32x4 wacc[NWW];
#pragma unroll
      for (int u = 0; u < NUW; ++u) {
        const int jb = wave + CNW * u;
        if (jb < NU) {
          constexpr int NT = DV / 16;
          const int mt = jb / NT, nt = jb % NT;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k0 = 0; k0 < BT; k0 += MM::KS)
            acc = MM::mma(MM::kc(Tm, LDJ, 16 * mt, k0, lane), MM::rc(Vl, LDV, 16 * nt, k0, lane), acc);
          store4(upg + cm_off(16 * mt + crow(lane, 0), 16 * nt + ccol(lane), DV), acc[0], acc[1], acc[2], acc[3]);
        }
      }
      if constexpr (KEEPW) {
#pragma unroll
        for (int u = 0; u < NWW; ++u) {
          const int jb = wave + CNW * u;
          wacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (jb < NW) {
            constexpr int NT = BT / 16;
            const int mt = jb / NT, nt = jb % NT;
#pragma unroll
            for (int k0 = 0; k0 < BT; k0 += MM::KS)
              wacc[u] = MM::mma(MM::rc(Kt, LDK, 16 * mt, k0, lane), MM::kc(Tm, LDJ, 16 * nt, k0, lane), wacc[u]);
            const int i = 16 * nt + ccol(lane), c0 = 16 * mt + crow(lane, 0);
            if constexpr (PF) {
              store4(wg + pf_off(i, c0, D), -wacc[u][0], -wacc[u][1], -wacc[u][2], -wacc[u][3]);
            } else {
              const float wv[4] = {wacc[u][0], wacc[u][1], wacc[u][2], wacc[u][3]};
              fm_store<T>(wg, D, i, c0, wv, 4);
            }
            if constexpr (BWD && !PF) {
              T* wtg = static_cast<T*>(a.ws.WT) + wsi * D * BT;
#pragma unroll
              for (int r = 0; r < 4; ++r) wtg[fm_off<T>(c0 + r, i, BT)] = from_f<T>(wacc[u][r]);
            }
          }
        }
      } else {
        HARTS_STRIDED(jb, wave, NW, CNW) {
          constexpr int NT = BT / 16;
          const int mt = jb / NT, nt = jb % NT;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k0 = 0; k0 < BT; k0 += MM::KS)
            acc = MM::mma(MM::rc(Kt, LDK, 16 * mt, k0, lane), MM::kc(Tm, LDJ, 16 * nt, k0, lane), acc);
          const int i = 16 * nt + ccol(lane), c0 = 16 * mt + crow(lane, 0);
          if constexpr (PF) {
            store4(wg + pf_off(i, c0, D), -acc[0], -acc[1], -acc[2], -acc[3]);
          } else {
            const float wv[4] = {acc[0], acc[1], acc[2], acc[3]};
            fm_store<T>(wg, D, i, c0, wv, 4);
          }
        }
      }
      if constexpr (!PF) {  // (bf16: exported during step 7)
        T* khg = static_cast<T*>(a.ws.KhT) + wsi * D * BT;
        HARTS_STRIDED(idx, tid, D * (BT / VN), CNT) {
          const int c = idx / (BT / VN), i0 = (idx % (BT / VN)) * VN;
          float kv[VN];
          ld16(KhT + c * LDJ + i0, kv);
          fm_store<T>(khg, BT, c, i0, kv, VN);
        }
      }
      if constexpr (BWD) {
        const size_t BB = size_t(BT) * BT;
        T* tg = static_cast<T*>(a.ws.Tm) + wsi * BB;
        T* xg = static_cast<T*>(a.ws.Xm) + wsi * BB;
        HARTS_STRIDED(idx, tid, BT * (BT / VN), CNT) {
          const int i = idx / (BT / VN), j0 = (idx % (BT / VN)) * VN;
          copy16(tg + i * BT + j0, Tm + i * LDJ + j0);
          float xv[VN];
#pragma unroll
          for (int t = 0; t < VN; ++t) xv[t] = j0 + t <= i ? Xf[i * LDA + j0 + t] : 0.f;
          stq(xg + i * BT + j0, pack16<T>(xv));
        }
      }
      if constexpr (KEEPW) {
        __syncthreads();  // every wave is done reading K~: W takes its place
#pragma unroll
        for (int u = 0; u < NWW; ++u) {
          const int jb = wave + CNW * u;
          if (jb < NW) {
            constexpr int NT = BT / 16;
            const int mt = jb / NT, nt = jb % NT;
            const int i = 16 * nt + ccol(lane), c0 = 16 * mt + crow(lane, 0);
            store4(Kt + i * LDK + c0, wacc[u][0], wacc[u][1], wacc[u][2], wacc[u][3]);
          }
        }
        __syncthreads();
        {
          // 9. Qeff = Q~ - M W, stored as Qeff^T [D][BT]
          T* qe = static_cast<T*>(a.ws.QeffT) + wsi * D * BT;
          constexpr int MT = BT / 16, NT = D / 16;
          HARTS_STRIDED(jb, wave, MT * NT, CNW) {
            const int mt = jb / NT, nt = jb % NT;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < BT; k0 += MM::KS)
              acc = MM::mma(MM::kc(Ml, LDJ, 16 * mt, k0, lane), MM::rc(Kt, LDK, 16 * nt, k0, lane), acc);
            const int c = 16 * nt + ccol(lane), i0 = 16 * mt + crow(lane, 0);
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = to_f(Qr[(i0 + r) * LDK + c]) - acc[r];
            fm_store<T>(qe, BT, c, i0, v, 4);
          }
        }
      }
    }
    __syncthreads();  // the next item overwrites every region
    // the ticket word is read again rather than the item held across the item's phases
    item = item_n;
    item_n = a.ctr ? 2 * int(gridDim.x) + tk_slot : item + int(gridDim.x);
  }
}

// ------------------------------------------------------------------------------------------
// Serial state pass.  One workgroup of SNW waves per (sequence, head, value-column tile of
// DVT): the columns of S evolve independently.  Per chunk:
//   U = U' - W S;  [forward] O^T = S^T Q~^T + U^T M^T;  S = diag(e^{G_last}) S + KhT U.
// S lives in accumulator registers (fp32; wave w owns state rows 16w..); S^T and U^T are
// staged in LDS as matrix-core operands.  Every per-chunk operand that does not depend on S
// (W, U', Q~, M, KhT, e^{G_last}, the output rows) is read from its fragment-major
// workspace layout one chunk ahead into registers, so a step is
// S -> LDS -> barrier -> U -> LDS -> barrier -> S on the matrix cores.  Backward mode
// writes the chunk-start states (S^T and S, fragment-major) after the second barrier.
template <typename T, int BT, int D, int DV, int DVT, bool FWD>
struct StateOps {
  using MM = Mma<T>;
  using F = typename MM::Frag;
  using Raw4 = typename std::conditional<sizeof(T) == 2, bf16x4, f32x4>::type;
  using TL = StateTiles<BT, D, DVT>;
  static constexpr int KD = D / MM::KS, KB = BT / MM::KS;
  static constexpr int KQ = FWD ? KD : 1, KM = FWD ? KB : 1;
  F wa[KD];               // W fragments of this wave's token block (A operand of W S)
  Raw4 up[TL::NTU];       // U' at this lane's accumulator positions of its U tiles
  F qb[KQ];               // forward: Q~ fragments of the token block (B operand of the output)
  F mb[KM];               // forward: M fragments of the token block (B operand of the output)
  F ka[TL::MU][KB];       // KhT fragments (A operand of S += KhT U)
  float el[TL::MU][4];    // e^{G_last} of this lane's state rows
  int emit;               // emitted slot (-1: none)
  int orow;               // forward: compact row of this lane's output token (-1: padding)
};

template <typename T, int BT, int D, int DV, int DVT, bool FWD>
__device__ __forceinline__ void load_state_ops(StateOps<T, BT, D, DV, DVT, FWD>& o, const RoundArgs& a, int chunk,
                                               int h, int H, int wave, int lane, int jvb, int z) {
  using Ops = StateOps<T, BT, D, DV, DVT, FWD>;
  using TL = typename Ops::TL;
  const ChunkWs& ws = a.ws;
  const size_t wsi = size_t(chunk) * H + h;
  const int mi = wave / TL::WPB, nt0 = jvb / 16 + (wave % TL::WPB) * TL::NTU;
  const T* wg = static_cast<const T*>(ws.W) + wsi * BT * D;
  const T* upg = static_cast<const T*>(ws.UpT) + wsi * BT * DV;
  const T* khg = static_cast<const T*>(ws.KhT) + wsi * D * BT;
  const float* el = ws.El + wsi * D;
  o.emit = a.chunks[chunk + z].emit;
#pragma unroll
  for (int kk = 0; kk < Ops::KD; ++kk) o.wa[kk] = fm_frag<T>(wg, D, mi, kk, lane);
#pragma unroll
  for (int j = 0; j < TL::NTU; ++j)
    o.up[j] = *reinterpret_cast<const typename Ops::Raw4*>(upg + ((size_t(mi) * (DV / 16) + nt0 + j) * 64 + lane) * 4);
  if constexpr (FWD) {
    const T* qg = static_cast<const T*>(ws.Qt) + wsi * BT * D;
    const T* mg = static_cast<const T*>(ws.Mm) + wsi * BT * BT;
#pragma unroll
    for (int kk = 0; kk < Ops::KD; ++kk) o.qb[kk] = fm_frag<T>(qg, D, mi, kk, lane);
#pragma unroll
    for (int kk = 0; kk < Ops::KB; ++kk) o.mb[kk] = fm_frag<T>(mg, BT, mi, kk, lane);
    o.orow = a.crows[size_t(chunk) * BT + 16 * mi + ccol(lane)];
  }
#pragma unroll
  for (int u = 0; u < TL::MU; ++u) {
    const int mt = wave + TL::NW * u, mc = mt < TL::MT ? mt : 0;
#pragma unroll
    for (int kk = 0; kk < Ops::KB; ++kk) o.ka[u][kk] = fm_frag<T>(khg, BT, mc, kk, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) o.el[u][r] = el[16 * mc + crow(lane, r)];
  }
}

template <typename T, int BT, int D, int DV, int DVT, bool BWD>
__global__ __launch_bounds__(64 * state_waves<D>()) void kda_state_kernel(RoundArgs a, int H) {
  using MM = Mma<T>;
  using Ops = StateOps<T, BT, D, DV, DVT, !BWD>;
  using TL = typename Ops::TL;
  constexpr int NW = TL::NW, NTL = DV / DVT, NTV = TL::NTV, MT = TL::MT, MU = TL::MU, NTU = TL::NTU;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int LDS_S = D + PAD, LDS_U = BT + PAD;
  constexpr int NTH = 64 * NW;
  __shared__ __attribute__((aligned(16))) T St[2][DVT * LDS_S];
  __shared__ __attribute__((aligned(16))) T Ut[DVT * LDS_U];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lb = xcd_logical(blockIdx.x, gridDim.x);
  const int tile = lb % NTL, h = (lb / NTL) % H, si = lb / (NTL * H);
  if (si >= a.nseq) return;
  const SeqDesc sd = a.seqs[si];
  const int jvb = tile * DVT;
  const int mi = wave / TL::WPB, nt0 = (wave % TL::WPB) * NTU;  // this wave's token block and tile columns
  f32x4 S[MU][NTV];
#pragma unroll
  for (int u = 0; u < MU; ++u)
#pragma unroll
    for (int nt = 0; nt < NTV; ++nt) {
      const int mt = wave + NW * u;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = 0.f;
        if (mt < MT && sd.init >= 0) {
          const int c = 16 * mt + crow(lane, r), jv = jvb + 16 * nt + ccol(lane);
          v = a.init_pool[((size_t(sd.init) * H + h) * D + c) * DV + jv];
        }
        S[u][nt][r] = v;
      }
    }
  // cur is taken from nxt at the top of each step, before the next fetch is issued, so
  // no path into the loop leaves a load pending on cur's registers
  Ops cur, nxt;
  const int z = lane_zero();
  load_state_ops<T, BT, D, DV, DVT, !BWD>(nxt, a, sd.chunk_base, h, H, wave, lane, jvb, z);
  for (int n = 0; n < sd.n_chunks; ++n) {
    // thread-derived addresses are recomputed per step instead of being held across the loop
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const size_t wsi = size_t(sd.chunk_base + n) * H + h;
    const int own = sd.n_replay - n * BT;  // replayed rows sit at the front of the first chunk
    cur = nxt;
    load_state_ops<T, BT, D, DV, DVT, !BWD>(nxt, a, sd.chunk_base + (n + 1 < sd.n_chunks ? n + 1 : n), h, H, wave,
                                            lane, jvb, z);
    T* Sb = St[n & 1];
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int mt = wave + NW * u;
      if (mt < MT)
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt)
          store4(Sb + (16 * nt + ccol(lane)) * LDS_S + 16 * mt + crow(lane, 0), S[u][nt][0], S[u][nt][1],
                 S[u][nt][2], S[u][nt][3]);
    }
    __syncthreads();
    // (a) U = U' - W S  (this wave: token block mi, value tiles nt0 ..)
#pragma unroll
    for (int j = 0; j < NTU; ++j) {
      const int nt = nt0 + j;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < Ops::KD; ++kk)
        acc = MM::mma(cur.wa[kk], MM::kc(Sb, LDS_S, 16 * nt, kk * MM::KS, lane), acc);
      store4(Ut + (16 * nt + ccol(lane)) * LDS_U + 16 * mi + crow(lane, 0), to_f(cur.up[j][0]) - acc[0],
             to_f(cur.up[j][1]) - acc[1], to_f(cur.up[j][2]) - acc[2], to_f(cur.up[j][3]) - acc[3]);
    }
    __syncthreads();
    // (b) S = diag(e^{G_last}) S + KhT U   (the chain: issued before the side work below)
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int mt = wave + NW * u;
      if (mt < MT) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int nt = 0; nt < NTV; ++nt) S[u][nt][r] *= cur.el[u][r];
#pragma unroll
        for (int kk = 0; kk < Ops::KB; ++kk)
#pragma unroll
          for (int nt = 0; nt < NTV; ++nt)
            S[u][nt] = MM::mma(cur.ka[u][kk], MM::kc(Ut, LDS_U, 16 * nt, kk * MM::KS, lane), S[u][nt]);
      }
    }
    if constexpr (BWD) {
      // chunk-start state for the per-chunk gradient kernels; Sb is next written two steps on
      store_state_fm<T, D, DV, DVT, NTH>(static_cast<T*>(a.h) + wsi * DV * D, static_cast<T*>(a.hc) + wsi * D * DV,
                                         Sb, LDS_S, jvb, tid);
    } else {
      // O^T = S^T Q~^T + U^T M^T for own rows; lanes without a row store into the sink
      T* og = static_cast<T*>(a.o);
      const int i = 16 * mi + ccol(lane);
      const bool ok = og && cur.orow >= 0 && i >= own;
#pragma unroll
      for (int j = 0; j < NTU; ++j) {
        const int m = nt0 + j;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < Ops::KD; ++kk)
          acc = MM::mma(MM::kc(Sb, LDS_S, 16 * m, kk * MM::KS, lane), cur.qb[kk], acc);
#pragma unroll
        for (int kk = 0; kk < Ops::KB; ++kk)
          acc = MM::mma(MM::kc(Ut, LDS_U, 16 * m, kk * MM::KS, lane), cur.mb[kk], acc);
        T* dst = ok ? og + (size_t(cur.orow) * H + h) * DV + jvb + 16 * m + crow(lane, 0)
                    : static_cast<T*>(a.sink) + (tid * 4) % kSinkElems<T>();
        store4(dst, acc[0], acc[1], acc[2], acc[3]);
      }
    }
    if (cur.emit >= 0 && a.emit_pool) {
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const int mt = wave + NW * u;
        if (mt < MT)
#pragma unroll
          for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int c = 16 * mt + crow(lane, r), jv = jvb + 16 * nt + ccol(lane);
              a.emit_pool[((size_t(cur.emit) * H + h) * D + c) * DV + jv] = S[u][nt][r];
            }
      }
    }
  }
  if (sd.final_idx >= 0 && a.final_pool) {
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int mt = wave + NW * u;
      if (mt < MT)
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int c = 16 * mt + crow(lane, r), jv = jvb + 16 * nt + ccol(lane);
            a.final_pool[((size_t(sd.final_idx) * H + h) * D + c) * DV + jv] = S[u][nt][r];
          }
    }
  }
}

// ------------------------------------------------------------------------------------------
template <typename T, int BT, int D, int DV>
static hipError_t prep_launch(const KdaDims& d, const RoundArgs& a, int mode, hipStream_t s) {
  if (a.nchunk <= 0 && !a.zero) return hipSuccess;
  dim3 grid(a.nchunk > 0 ? persistent_grid(unsigned(a.nchunk) * d.H) : 1u), block(CNT);
  if (mode == 1) hipLaunchKernelGGL((kda_prep_kernel<T, BT, D, DV, 1>), grid, block, 0, s, a, d.H);
  else if (mode == 0) hipLaunchKernelGGL((kda_prep_kernel<T, BT, D, DV, 0>), grid, block, 0, s, a, d.H);
  else if constexpr (sizeof(T) == 2) hipLaunchKernelGGL((kda_prep_kernel<T, BT, D, DV, 2>), grid, block, 0, s, a, d.H);
  else return hipErrorNotSupported;
  return hipGetLastError();
}

template <int DV> constexpr int dv_tile() { return DV; }  // one workgroup per (sequence, head)

template <typename T, int BT, int D, int DV>
static hipError_t state_launch(const KdaDims& d, const RoundArgs& a, bool bwd, hipStream_t s) {
  if (a.nseq <= 0) return hipSuccess;
  constexpr int DVT = dv_tile<DV>();
  unsigned n = unsigned(a.nseq) * d.H * (DV / DVT);
  n = (n + 7) / 8 * 8;
  dim3 grid(n), block(64 * state_waves<D>());
  if (bwd) hipLaunchKernelGGL((kda_state_kernel<T, BT, D, DV, DVT, true>), grid, block, 0, s, a, d.H);
  else hipLaunchKernelGGL((kda_state_kernel<T, BT, D, DV, DVT, false>), grid, block, 0, s, a, d.H);
  return hipGetLastError();
}

#define HARTS_KDA_CONFIGS(X) \
  X(bf16, 64, 128, 128)      \
  X(bf16, 64, 64, 64)        \
  X(bf16, 32, 64, 64)        \
  X(bf16, 32, 32, 32)        \
  X(float, 16, 16, 16)       \
  X(float, 32, 32, 32)

bool kda_supported(const KdaDims& d) {
#define X(T_, B_, D_, V_) \
  if (d.dtype == (sizeof(T_) == 2 ? 0 : 1) && d.BT == B_ && d.D == D_ && d.DV == V_) return true;
  HARTS_KDA_CONFIGS(X)
#undef X
  return false;
}

hipError_t launch_kda_prep(const KdaDims& d, const RoundArgs& a, int mode, hipStream_t s) {
#define X(T_, B_, D_, V_) \
  if (d.dtype == (sizeof(T_) == 2 ? 0 : 1) && d.BT == B_ && d.D == D_ && d.DV == V_) return prep_launch<T_, B_, D_, V_>(d, a, mode, s);
  HARTS_KDA_CONFIGS(X)
#undef X
  return hipErrorInvalidValue;
}

// fp32 configurations only: bf16 runs the slab passes (kda_slab.hip)
hipError_t launch_kda_state(const KdaDims& d, const RoundArgs& a, bool backward, hipStream_t s) {
#define X(T_, B_, D_, V_)                                                             \
  if constexpr (sizeof(T_) == 4)                                                      \
    if (d.dtype == 1 && d.BT == B_ && d.D == D_ && d.DV == V_) return state_launch<T_, B_, D_, V_>(d, a, backward, s);
  HARTS_KDA_CONFIGS(X)
#undef X
  return hipErrorNotSupported;
}

}  // namespace harts
