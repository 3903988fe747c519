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
// "gated" products use e^{G_i - G_j} factored through 16-row sub-block
// reference points: for rows i in block bi and j in block bj <= bi,
// e^{G_i - G_j} = e^{G_i - F_bi} * e^{F_bi - G_j}, F_b the log-decay before
// block b; both factors are <= 1 off the diagonal blocks, and within a
// diagonal block the pair is bounded by one 16-row gate sum.
#include "common.h"
#include "launch.h"

namespace harts {

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
__host__ __device__ constexpr int pair_index(int bi, int bj) { return (bi - 2) * (bi - 1) / 2 + bj; }

template <typename T, int BT, int D, int DV>
struct PrepLayout {
  static constexpr int NB = BT / 16;
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int LDK = D + PAD, LDJ = BT + PAD, LDV = DV + PAD;
  static constexpr int LDF = D + 4, LDA = BT + 4;
  static constexpr int NPX = NB >= 3 ? (NB - 1) * (NB - 2) / 2 : 0;
  static constexpr size_t szK = size_t(BT) * LDK * sizeof(T);
  // R1: Gf | X, Tmp | V, W(backward)
  static constexpr size_t R1 = cmax(cmax(size_t(BT) * LDF * 4, 2 * size_t(BT) * LDA * 4),
                                    size_t(BT) * LDV * sizeof(T) + szK);
  static constexpr size_t R1_OFF = 0;
  // Am: A (fp32) | M (backward, T)
  static constexpr size_t AM_OFF = R1_OFF + R1;
  static constexpr size_t AM = cmax(size_t(BT) * LDA * 4, size_t(BT) * LDJ * sizeof(T));
  // R2: Kr->K~ | Qr->Q~ | Kc0 | Kcd,Kcx -> KhT | Tm
  static constexpr size_t R2_OFF = AM_OFF + AM;
  static constexpr size_t KR = 0, QR = KR + szK, KC0 = QR + szK, KCD = KC0 + szK, KCX = KCD + szK;
  static constexpr size_t AEND = KCX + size_t(NPX) * 16 * LDK * sizeof(T);
  static constexpr size_t KHT = KCD;
  static constexpr size_t TM = cmax(AEND, KHT + size_t(D) * LDJ * sizeof(T));
  static constexpr size_t R2 = TM + size_t(BT) * LDJ * sizeof(T);
  // vectors (fp32): Tv[NB][D], Fv[NB+1][D], EF[NB+1][D], EH[NB][D], Sx[NPX][D], bet[BT]
  static constexpr size_t VEC_OFF = R2_OFF + R2;
  static constexpr size_t TV = 0, FV = TV + NB * D, EF = FV + (NB + 1) * D, EH = EF + (NB + 1) * D,
                          SX = EH + NB * D, BET = SX + (NPX > 0 ? NPX : 1) * D;
  static constexpr size_t VEC = (BET + BT) * 4;
  static constexpr size_t TOTAL = VEC_OFF + VEC;
  static_assert(TOTAL <= 160 * 1024, "prep kernel LDS budget");
};

// ------------------------------------------------------------------------------------------
// Per-chunk preparation.  One workgroup (4 waves) per (chunk, head).
template <typename T, int BT, int D, int DV, bool BWD>
__global__ __launch_bounds__(256) void kda_prep_kernel(RoundArgs a, int H) {
  using Ly = PrepLayout<T, BT, D, DV>;
  using MM = Mma<T>;
  constexpr int NB = Ly::NB, LDK = Ly::LDK, LDJ = Ly::LDJ, LDV = Ly::LDV, LDF = Ly::LDF, LDA = Ly::LDA;
  constexpr int VN = 16 / sizeof(T);
  __shared__ __attribute__((aligned(16))) char smem[Ly::TOTAL];
  float* Gf = reinterpret_cast<float*>(smem + Ly::R1_OFF);
  float* X = Gf;
  float* Tmp = X + BT * LDA;
  T* Vl = reinterpret_cast<T*>(smem + Ly::R1_OFF);
  T* Wl = reinterpret_cast<T*>(smem + Ly::R1_OFF + size_t(BT) * LDV * sizeof(T));
  float* Am = reinterpret_cast<float*>(smem + Ly::AM_OFF);
  T* Ml = reinterpret_cast<T*>(smem + Ly::AM_OFF);
  char* r2 = smem + Ly::R2_OFF;
  T* Kr = reinterpret_cast<T*>(r2 + Ly::KR);
  T* Qr = reinterpret_cast<T*>(r2 + Ly::QR);
  T* Kc0 = reinterpret_cast<T*>(r2 + Ly::KC0);
  T* Kcd = reinterpret_cast<T*>(r2 + Ly::KCD);
  T* Kcx = reinterpret_cast<T*>(r2 + Ly::KCX);
  T* KhT = reinterpret_cast<T*>(r2 + Ly::KHT);
  T* Tm = reinterpret_cast<T*>(r2 + Ly::TM);
  float* vec = reinterpret_cast<float*>(smem + Ly::VEC_OFF);
  float* Tv = vec + Ly::TV;
  float* Fv = vec + Ly::FV;
  float* EF = vec + Ly::EF;
  float* EH = vec + Ly::EH;
  float* Sx = vec + Ly::SX;
  float* bet = vec + Ly::BET;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x / H, h = blockIdx.x % H;
  const ChunkDesc cd = a.chunks[chunk];
  const int len = cd.len;
  const size_t wsi = size_t(cd.local) * H + h;
  const T* gq = static_cast<const T*>(a.q);
  const T* gk = static_cast<const T*>(a.k);
  const T* gv = static_cast<const T*>(a.v);
  const T* gg = static_cast<const T*>(a.g);
  const T* gb = static_cast<const T*>(a.beta);
  const int32_t* vr = a.vrows + cd.vbase;

  // 1. g -> Gf (fp32), beta
  for (int idx = tid; idx < BT * (D / VN); idx += 256) {
    const int i = idx / (D / VN), c0 = (idx % (D / VN)) * VN;
    float v[VN];
    if (i < len) ld16(gg + (size_t(vr[i]) * H + h) * D + c0, v);
    else
#pragma unroll
      for (int t = 0; t < VN; ++t) v[t] = 0.f;
#pragma unroll
    for (int t = 0; t < VN; ++t) Gf[i * LDF + c0 + t] = v[t];
  }
  if (tid < BT) bet[tid] = tid < len ? to_f(gb[size_t(vr[tid]) * H + h]) : 0.f;
  __syncthreads();
  // 2. block-local cumulative sums L, block totals, entry log-decays and scale vectors
  for (int idx = tid; idx < NB * D; idx += 256) {
    const int b = idx / D, c = idx % D;
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      acc += Gf[(16 * b + t) * LDF + c];
      Gf[(16 * b + t) * LDF + c] = acc;
    }
    Tv[b * D + c] = acc;
  }
  __syncthreads();
  for (int c = tid; c < D; c += 256) {
    float f = 0.f;
    Fv[c] = 0.f;
    EF[c] = 1.f;
    for (int b = 0; b < NB; ++b) {
      f += Tv[b * D + c];
      Fv[(b + 1) * D + c] = f;
      EF[(b + 1) * D + c] = __expf(f);
    }
    for (int b = 0; b < NB; ++b) EH[b * D + c] = __expf(f - Fv[(b + 1) * D + c]);
  }
  __syncthreads();
  if constexpr (Ly::NPX > 0) {
    for (int idx = tid; idx < Ly::NPX * D; idx += 256) {
      const int p = idx / D, c = idx % D;
      int bi = 2, rem = p;
      while (rem >= bi - 1) { rem -= bi - 1; ++bi; }
      const int bj = rem;
      Sx[p * D + c] = __expf(Fv[bi * D + c] - Fv[(bj + 1) * D + c]);
    }
  }
  __syncthreads();
  // 3. operand arrays: Kr = k e^L, Qr = q e^L, Kc0 = k e^{T_b - L}, Kcd = k e^{-L}, Kcx = Kc0 * pair scale
  for (int idx = tid; idx < BT * (D / VN); idx += 256) {
    const int i = idx / (D / VN), c0 = (idx % (D / VN)) * VN, b = i / 16;
    float kk[VN], qq[VN];
    if (i < len) {
      ld16(gk + (size_t(vr[i]) * H + h) * D + c0, kk);
      ld16(gq + (size_t(vr[i]) * H + h) * D + c0, qq);
    } else {
#pragma unroll
      for (int t = 0; t < VN; ++t) kk[t] = qq[t] = 0.f;
    }
    float kr[VN], qr[VN], kc[VN], kd[VN];
#pragma unroll
    for (int t = 0; t < VN; ++t) {
      const float Lv = Gf[i * LDF + c0 + t];
      const float er = __expf(Lv);
      kr[t] = kk[t] * er;
      qr[t] = qq[t] * er;
      kc[t] = kk[t] * __expf(Tv[b * D + c0 + t] - Lv);
      kd[t] = kk[t] * __expf(-Lv);
    }
    st16(Kr + i * LDK + c0, kr);
    st16(Qr + i * LDK + c0, qr);
    st16(Kc0 + i * LDK + c0, kc);
    st16(Kcd + i * LDK + c0, kd);
    for (int bi = b + 2; bi < NB; ++bi) {
      const int p = pair_index(bi, b);
      float x[VN];
#pragma unroll
      for (int t = 0; t < VN; ++t) x[t] = kc[t] * Sx[p * D + c0 + t];
      st16(Kcx + (p * 16 + i - 16 * b) * LDK + c0, x);
    }
  }
  __syncthreads();
  // 4. A (strict lower) into Am; M (lower incl.) to global, one 16x16 tile per sub-block pair
  T* Mg = static_cast<T*>(a.ws.Mm) + wsi * BT * BT;
  {
    constexpr int NT = NB * (NB + 1) / 2;
    for (int jb = wave; jb < 2 * NT; jb += 4) {
      const bool isM = jb >= NT;
      const int t = isM ? jb - NT : jb;
      int bi = 0;
      while ((bi + 1) * (bi + 2) / 2 <= t) ++bi;
      const int bj = t - bi * (bi + 1) / 2;
      const T* col = bi == bj ? Kcd + 16 * bj * LDK
                     : (bi - bj == 1 ? Kc0 + 16 * bj * LDK : Kcx + pair_index(bi, bj) * 16 * LDK);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if (!isM) {
        for (int k0 = 0; k0 < D; k0 += MM::KS)
          acc = MM::mma(MM::kc(Kr + 16 * bi * LDK, LDK, 0, k0, lane), MM::kc(col, LDK, 0, k0, lane), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * bi + crow(lane, r), j = 16 * bj + ccol(lane);
          Am[i * LDA + j] = (bi == bj && i <= j) ? 0.f : acc[r];
        }
      } else {
        for (int k0 = 0; k0 < D; k0 += MM::KS)
          acc = MM::mma(MM::kc(col, LDK, 0, k0, lane), MM::kc(Qr + 16 * bi * LDK, LDK, 0, k0, lane), acc);
        const int i = 16 * bi + ccol(lane), j0 = 16 * bj + crow(lane, 0);
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (bi == bj && j0 + r > i) ? 0.f : acc[r];
        store4(Mg + i * BT + j0, v[0], v[1], v[2], v[3]);
      }
    }
    for (int idx = tid; idx < BT * BT; idx += 256) {
      const int i = idx / BT, j = idx % BT;
      if (j / 16 > i / 16) Mg[idx] = from_f<T>(0.f);
    }
  }
  __syncthreads();
  // 5. X = (I + diag(beta) A)^{-1}: diagonal 16x16 blocks by forward substitution,
  //    then X_{bi,bj} = -X_{bi,bi} sum_{m=bj}^{bi-1} L_{bi,m} X_{m,bj} by increasing distance.
  for (int idx = tid; idx < BT * LDA; idx += 256) X[idx] = 0.f;
  __syncthreads();
  if (tid < NB * 16) {
    const int b = tid / 16, col = tid % 16;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m)
        if (m < r) s += Am[(16 * b + r) * LDA + 16 * b + m] * x[m];
      x[r] = r < col ? 0.f : (r == col ? 1.f : -bet[16 * b + r] * s);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) X[(16 * b + r) * LDA + 16 * b + col] = x[r];
  }
  __syncthreads();
  for (int dd = 1; dd < NB; ++dd) {
    for (int idx = tid; idx < (NB - dd) * 256; idx += 256) {
      const int bj = idx / 256, e = idx % 256, bi = bj + dd;
      const int i = 16 * bi + e / 16, j = 16 * bj + e % 16;
      float s = 0.f;
      for (int mm = 16 * bj; mm < 16 * bi; ++mm) s += Am[i * LDA + mm] * X[mm * LDA + j];
      Tmp[i * LDA + j] = bet[i] * s;
    }
    __syncthreads();
    for (int idx = tid; idx < (NB - dd) * 256; idx += 256) {
      const int bj = idx / 256, e = idx % 256, bi = bj + dd;
      const int i = 16 * bi + e / 16, j = 16 * bj + e % 16;
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < 16; ++t) s += X[i * LDA + 16 * bi + t] * Tmp[(16 * bi + t) * LDA + j];
      X[i * LDA + j] = -s;
    }
    __syncthreads();
  }
  // 6. T = X diag(beta); K~ = Kr e^{F_b}, Q~ = Qr e^{F_b} in place; KhT = (Kc0 e^{F_end - F_{b+1}})^T
  for (int idx = tid; idx < BT * BT; idx += 256) {
    const int i = idx / BT, j = idx % BT;
    const float tv = j <= i ? X[i * LDA + j] * bet[j] : 0.f;
    Tm[i * LDJ + j] = from_f<T>(tv);
    if (BWD) {
      // T, X and A for the gradient kernels
      static_cast<T*>(a.ws.Tm)[wsi * BT * BT + idx] = from_f<T>(tv);
      static_cast<T*>(a.ws.Xm)[wsi * BT * BT + idx] = from_f<T>(j <= i ? X[i * LDA + j] : 0.f);
      static_cast<T*>(a.ws.Am)[wsi * BT * BT + idx] = from_f<T>(j < i ? Am[i * LDA + j] : 0.f);
    }
  }
  for (int idx = tid; idx < BT * (D / VN); idx += 256) {
    const int i = idx / (D / VN), c0 = (idx % (D / VN)) * VN, b = i / 16;
    float kr[VN], qr[VN], kc[VN];
    ld16(Kr + i * LDK + c0, kr);
    ld16(Qr + i * LDK + c0, qr);
    ld16(Kc0 + i * LDK + c0, kc);
#pragma unroll
    for (int t = 0; t < VN; ++t) {
      const float ef = EF[b * D + c0 + t];
      kr[t] *= ef;
      qr[t] *= ef;
      kc[t] *= EH[b * D + c0 + t];
    }
    st16(Kr + i * LDK + c0, kr);
    st16(Qr + i * LDK + c0, qr);
#pragma unroll
    for (int t = 0; t < VN; ++t) KhT[(c0 + t) * LDJ + i] = from_f<T>(kc[t]);
  }
  __syncthreads();
  // 7. V into R1; K~ stays in Kr, Q~ in Qr.  Copy KhT, Q~ (forward) and e^{G_last} out.
  for (int idx = tid; idx < BT * (DV / VN); idx += 256) {
    const int i = idx / (DV / VN), c0 = (idx % (DV / VN)) * VN;
    if (i < len) copy16(Vl + i * LDV + c0, gv + (size_t(vr[i]) * H + h) * DV + c0);
    else *reinterpret_cast<f32x4*>(Vl + i * LDV + c0) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  {
    T* khg = static_cast<T*>(a.ws.KhT) + wsi * D * BT;
    for (int idx = tid; idx < D * (BT / VN); idx += 256) {
      const int c = idx / (BT / VN), i0 = (idx % (BT / VN)) * VN;
      copy16(khg + c * BT + i0, KhT + c * LDJ + i0);
    }
    if (!BWD) {
      T* qg = static_cast<T*>(a.ws.Qt) + wsi * BT * D;
      for (int idx = tid; idx < BT * (D / VN); idx += 256) {
        const int i = idx / (D / VN), c0 = (idx % (D / VN)) * VN;
        copy16(qg + i * D + c0, Qr + i * LDK + c0);
      }
    }
    for (int c = tid; c < D; c += 256) a.ws.El[wsi * D + c] = EF[NB * D + c];
  }
  __syncthreads();
  // 8. U' = T V, stored transposed: UpT[jv][i]
  {
    T* upg = static_cast<T*>(a.ws.UpT) + wsi * DV * BT;
    constexpr int MT = BT / 16, NT = DV / 16;
    for (int jb = wave; jb < MT * NT; jb += 4) {
      const int mt = jb / NT, nt = jb % NT;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < BT; k0 += MM::KS)
        acc = MM::mma(MM::kc(Tm, LDJ, 16 * mt, k0, lane), MM::rc(Vl, LDV, 16 * nt, k0, lane), acc);
      store4(upg + (16 * nt + ccol(lane)) * BT + 16 * mt + crow(lane, 0), acc[0], acc[1], acc[2], acc[3]);
    }
  }
  // 9. W^T = K~^T T^T (tile rows = channels), stored token-major: W[i][c]
  {
    T* wg = static_cast<T*>(a.ws.W) + wsi * BT * D;
    constexpr int MT = D / 16, NT = BT / 16;
    for (int jb = wave; jb < MT * NT; jb += 4) {
      const int mt = jb / NT, nt = jb % NT;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < BT; k0 += MM::KS)
        acc = MM::mma(MM::rc(Kr, LDK, 16 * mt, k0, lane), MM::kc(Tm, LDJ, 16 * nt, k0, lane), acc);
      const int i = 16 * nt + ccol(lane), c0 = 16 * mt + crow(lane, 0);
      store4(wg + i * D + c0, acc[0], acc[1], acc[2], acc[3]);
      if (BWD) store4(Wl + i * LDK + c0, acc[0], acc[1], acc[2], acc[3]);
    }
  }
  if constexpr (BWD) {
    // 10. Qeff = Q~ - M W, stored transposed: QeffT[c][i]
    __syncthreads();
    for (int idx = tid; idx < BT * (BT / VN); idx += 256) {
      const int i = idx / (BT / VN), j0 = (idx % (BT / VN)) * VN;
      copy16(Ml + i * LDJ + j0, Mg + i * BT + j0);
    }
    __syncthreads();
    T* qe = static_cast<T*>(a.ws.QeffT) + wsi * D * BT;
    constexpr int MT = BT / 16, NT = D / 16;
    for (int jb = wave; jb < MT * NT; jb += 4) {
      const int mt = jb / NT, nt = jb % NT;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < BT; k0 += MM::KS)
        acc = MM::mma(MM::kc(Ml, LDJ, 16 * mt, k0, lane), MM::rc(Wl, LDK, 16 * nt, k0, lane), acc);
      const int c = 16 * nt + ccol(lane), i0 = 16 * mt + crow(lane, 0);
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = to_f(Qr[(i0 + r) * LDK + c]) - acc[r];
      store4(qe + c * BT + i0, v[0], v[1], v[2], v[3]);
    }
  }
}

// ------------------------------------------------------------------------------------------
// Serial state pass.  One workgroup (4 waves) per (sequence, head, value-column tile of DVT):
// the columns of S evolve independently.  Per chunk:
//   U = U' - W S;  [forward] O^T = S^T Q~^T + U^T M^T;  S = diag(e^{G_last}) S + KhT U.
// S lives in accumulator registers (fp32); S^T and U^T are staged in LDS as MFMA operands.
// Every per-chunk operand that does not depend on S (W, U', Q~, M, KhT, e^{G_last}) is
// loaded one chunk ahead into registers, so the chain S -> U -> S only waits on LDS and
// the matrix cores.  Backward mode writes S^T of every chunk start (the recomputed
// chunk-start states).
template <typename T, int BT, int D, int DV, int DVT, bool FWD>
struct StateOps {
  using MM = Mma<T>;
  using F = typename MM::Frag;
  static constexpr int NMI = (BT / 16 + 3) / 4, MU = (D / 16 + 3) / 4, NTV = DVT / 16;
  static constexpr int KD = D / MM::KS, KB = BT / MM::KS;
  static constexpr int NQ = FWD ? NMI : 1, KQ = FWD ? KD : 1, KM = FWD ? KB : 1;
  F wa[NMI][KD];        // W fragments (A operand of U = W S), token rows of this wave
  float up[NMI][NTV][4];  // U' at this lane's accumulator positions
  F qb[NQ][KQ];         // Q~ fragments (B operand of O^T), forward only
  F mb[NQ][KM];         // M fragments (B operand of O^T), forward only
  F ka[MU][KB];         // KhT fragments (A operand of S += KhT U)
  float el[MU][4];      // e^{G_last} of this lane's state rows
};

template <typename T, int BT, int D, int DV, int DVT, bool FWD>
__device__ __forceinline__ void load_state_ops(StateOps<T, BT, D, DV, DVT, FWD>& o, const ChunkWs& ws, size_t wsi,
                                               int wave, int lane, int jvb) {
  using Ops = StateOps<T, BT, D, DV, DVT, FWD>;
  using MM = Mma<T>;
  constexpr int MT = D / 16;
  const T* wg = static_cast<const T*>(ws.W) + wsi * BT * D;
  const T* upg = static_cast<const T*>(ws.UpT) + wsi * DV * BT;
  const T* khg = static_cast<const T*>(ws.KhT) + wsi * D * BT;
  const float* el = ws.El + wsi * D;
#pragma unroll
  for (int x = 0; x < Ops::NMI; ++x) {
    const int mi = wave + 4 * x;
    if (mi < BT / 16) {
#pragma unroll
      for (int kk = 0; kk < Ops::KD; ++kk) o.wa[x][kk] = MM::kc(wg, D, 16 * mi, kk * MM::KS, lane);
#pragma unroll
      for (int nt = 0; nt < Ops::NTV; ++nt)
        load4(upg + (jvb + 16 * nt + ccol(lane)) * BT + 16 * mi + crow(lane, 0), o.up[x][nt]);
      if constexpr (FWD) {
        const T* qg = static_cast<const T*>(ws.Qt) + wsi * BT * D;
        const T* mg = static_cast<const T*>(ws.Mm) + wsi * BT * BT;
#pragma unroll
        for (int kk = 0; kk < Ops::KD; ++kk) o.qb[x][kk] = MM::kc(qg, D, 16 * mi, kk * MM::KS, lane);
#pragma unroll
        for (int kk = 0; kk < Ops::KB; ++kk) o.mb[x][kk] = MM::kc(mg, BT, 16 * mi, kk * MM::KS, lane);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < Ops::MU; ++u) {
    const int mt = wave + 4 * u;
    if (mt < MT) {
#pragma unroll
      for (int kk = 0; kk < Ops::KB; ++kk) o.ka[u][kk] = MM::kc(khg, BT, 16 * mt, kk * MM::KS, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) o.el[u][r] = el[16 * mt + crow(lane, r)];
    }
  }
}

template <typename T, int BT, int D, int DV, int DVT, bool BWD>
__global__ __launch_bounds__(256) void kda_state_kernel(RoundArgs a, int H) {
  using MM = Mma<T>;
  using Ops = StateOps<T, BT, D, DV, DVT, !BWD>;
  constexpr int NTL = DV / DVT;
  constexpr int PAD = 16 / sizeof(T);
  constexpr int LDS_S = D + PAD, LDS_U = BT + PAD;
  constexpr int MT = D / 16, NTV = DVT / 16, MU = Ops::MU, NMI = Ops::NMI;
  __shared__ __attribute__((aligned(16))) T St[2][DVT * LDS_S];
  __shared__ __attribute__((aligned(16))) T Ut[DVT * LDS_U];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lb = xcd_logical(blockIdx.x, gridDim.x);
  const int tile = lb % NTL, h = (lb / NTL) % H, si = lb / (NTL * H);
  if (si >= a.nseq) return;
  const SeqDesc sd = a.seqs[si];
  const int jvb = tile * DVT;
  f32x4 S[MU][NTV];
#pragma unroll
  for (int u = 0; u < MU; ++u)
#pragma unroll
    for (int nt = 0; nt < NTV; ++nt) {
      const int mt = wave + 4 * u;
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
  Ops cur, nxt;
  ChunkDesc cd = a.chunks[sd.chunk_base];
  load_state_ops<T, BT, D, DV, DVT, !BWD>(cur, a.ws, size_t(cd.local) * H + h, wave, lane, jvb);
  for (int n = 0; n < sd.n_chunks; ++n) {
    const size_t wsi = size_t(cd.local) * H + h;
    const ChunkDesc cdn = a.chunks[sd.chunk_base + (n + 1 < sd.n_chunks ? n + 1 : n)];
    if (n + 1 < sd.n_chunks)
      load_state_ops<T, BT, D, DV, DVT, !BWD>(nxt, a.ws, size_t(cdn.local) * H + h, wave, lane, jvb);
    T* Sb = St[n & 1];
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int mt = wave + 4 * u;
      if (mt < MT)
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt)
          store4(Sb + (16 * nt + ccol(lane)) * LDS_S + 16 * mt + crow(lane, 0), S[u][nt][0], S[u][nt][1],
                 S[u][nt][2], S[u][nt][3]);
    }
    __syncthreads();
    if constexpr (BWD) {
      T* hg = static_cast<T*>(a.h) + wsi * DV * D;
      constexpr int VN = 16 / sizeof(T);
      for (int idx = tid; idx < DVT * (D / VN); idx += 256) {
        const int jl = idx / (D / VN), c0 = (idx % (D / VN)) * VN;
        copy16(hg + (jvb + jl) * D + c0, Sb + jl * LDS_S + c0);
      }
    }
    // (a) U = U' - W S
#pragma unroll
    for (int x = 0; x < NMI; ++x) {
      const int mi = wave + 4 * x;
      if (mi < BT / 16) {
        f32x4 acc[NTV];
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < Ops::KD; ++kk)
#pragma unroll
          for (int nt = 0; nt < NTV; ++nt)
            acc[nt] = MM::mma(cur.wa[x][kk], MM::kc(Sb, LDS_S, 16 * nt, kk * MM::KS, lane), acc[nt]);
#pragma unroll
        for (int nt = 0; nt < NTV; ++nt) {
          const int jl = 16 * nt + ccol(lane), i0 = 16 * mi + crow(lane, 0);
          store4(Ut + jl * LDS_U + i0, cur.up[x][nt][0] - acc[nt][0], cur.up[x][nt][1] - acc[nt][1],
                 cur.up[x][nt][2] - acc[nt][2], cur.up[x][nt][3] - acc[nt][3]);
        }
      }
    }
    __syncthreads();
    // (b) S = diag(e^{G_last}) S + KhT U   (the chain: issued before the output products)
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int mt = wave + 4 * u;
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
    if constexpr (!BWD) {
      // O^T = S^T Q~^T + U^T M^T for own rows
      T* og = static_cast<T*>(a.o);
#pragma unroll
      for (int x = 0; x < NMI; ++x) {
        const int ni = wave + 4 * x;
        if (ni < BT / 16) {
          f32x4 acc[NTV];
#pragma unroll
          for (int m = 0; m < NTV; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < Ops::KD; ++kk)
#pragma unroll
            for (int m = 0; m < NTV; ++m)
              acc[m] = MM::mma(MM::kc(Sb, LDS_S, 16 * m, kk * MM::KS, lane), cur.qb[x][kk], acc[m]);
#pragma unroll
          for (int kk = 0; kk < Ops::KB; ++kk)
#pragma unroll
            for (int m = 0; m < NTV; ++m)
              acc[m] = MM::mma(MM::kc(Ut, LDS_U, 16 * m, kk * MM::KS, lane), cur.mb[x][kk], acc[m]);
          const int i = 16 * ni + ccol(lane);
          if (og && i < cd.len && i >= cd.own_from) {
            const size_t row = size_t(a.vrows[cd.vbase + i]);
#pragma unroll
            for (int m = 0; m < NTV; ++m)
              store4(og + (row * H + h) * DV + jvb + 16 * m + crow(lane, 0), acc[m][0], acc[m][1], acc[m][2],
                     acc[m][3]);
          }
        }
      }
    }
    if (cd.emit >= 0 && a.emit_pool) {
#pragma unroll
      for (int u = 0; u < MU; ++u) {
        const int mt = wave + 4 * u;
        if (mt < MT)
#pragma unroll
          for (int nt = 0; nt < NTV; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int c = 16 * mt + crow(lane, r), jv = jvb + 16 * nt + ccol(lane);
              a.emit_pool[((size_t(cd.emit) * H + h) * D + c) * DV + jv] = S[u][nt][r];
            }
      }
    }
    cur = nxt;
    cd = cdn;
  }
  if (sd.final_idx >= 0 && a.final_pool) {
#pragma unroll
    for (int u = 0; u < MU; ++u) {
      const int mt = wave + 4 * u;
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
static hipError_t prep_launch(const KdaDims& d, const RoundArgs& a, bool bwd, hipStream_t s) {
  if (a.nchunk <= 0) return hipSuccess;
  dim3 grid(unsigned(a.nchunk) * d.H), block(256);
  if (bwd) hipLaunchKernelGGL((kda_prep_kernel<T, BT, D, DV, true>), grid, block, 0, s, a, d.H);
  else hipLaunchKernelGGL((kda_prep_kernel<T, BT, D, DV, false>), grid, block, 0, s, a, d.H);
  return hipGetLastError();
}

template <int D> constexpr int dv_tile() { return D >= 64 ? 32 : 16; }

template <typename T, int BT, int D, int DV>
static hipError_t state_launch(const KdaDims& d, const RoundArgs& a, bool bwd, hipStream_t s) {
  if (a.nseq <= 0) return hipSuccess;
  constexpr int DVT = dv_tile<DV>();
  unsigned n = unsigned(a.nseq) * d.H * (DV / DVT);
  n = (n + 7) / 8 * 8;
  dim3 grid(n), block(256);
  if (bwd) hipLaunchKernelGGL((kda_state_kernel<T, BT, D, DV, DVT, true>), grid, block, 0, s, a, d.H);
  else hipLaunchKernelGGL((kda_state_kernel<T, BT, D, DV, DVT, false>), grid, block, 0, s, a, d.H);
  return hipGetLastError();
}

#define HARTS_KDA_CONFIGS(X) \
  X(bf16, 64, 128, 128)      \
  X(bf16, 64, 64, 64)        \
  X(bf16, 32, 64, 64)        \
  X(float, 16, 16, 16)       \
  X(float, 32, 32, 32)

bool kda_supported(const KdaDims& d) {
#define X(T_, B_, D_, V_) \
  if (d.dtype == (sizeof(T_) == 2 ? 0 : 1) && d.BT == B_ && d.D == D_ && d.DV == V_) return true;
  HARTS_KDA_CONFIGS(X)
#undef X
  return false;
}

hipError_t launch_kda_prep(const KdaDims& d, const RoundArgs& a, bool backward, hipStream_t s) {
#define X(T_, B_, D_, V_) \
  if (d.dtype == (sizeof(T_) == 2 ? 0 : 1) && d.BT == B_ && d.D == D_ && d.DV == V_) return prep_launch<T_, B_, D_, V_>(d, a, backward, s);
  HARTS_KDA_CONFIGS(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_kda_state(const KdaDims& d, const RoundArgs& a, bool backward, hipStream_t s) {
#define X(T_, B_, D_, V_) \
  if (d.dtype == (sizeof(T_) == 2 ? 0 : 1) && d.BT == B_ && d.D == D_ && d.DV == V_) return state_launch<T_, B_, D_, V_>(d, a, backward, s);
  HARTS_KDA_CONFIGS(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace harts
