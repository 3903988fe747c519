// Tree softmax attention over compact rows (the full-attention / MLA layer of
// the hybrid model; HARTS, section 4 "MLA execution"; blog section 4.3;
// Figure C.1(c)).  A compact row attends over its own root-to-row path.  The
// ancestor view of a branch is never copied: query tiles read keys and values
// through the segment's row list (ancestors, then own rows, bottom-right causal),
// and key tiles read queries through the list of the rows below the segment.
//
// A workgroup owns one tile of one head: a 128-row query tile (forward: 4 waves of
// 32 queries, so every key/value fragment read from LDS feeds two products; dq: 8
// waves of 16) or a 128-row key tile (dk/dv: 8 waves of 16 keys).  The gathered
// operand tile (64 rows) goes through LDS with a register prefetch of the next
// tile; products run on v_mfma_f32_16x16x32_bf16.
//
//   forward / dq (query tiles): S^T = K Q^T puts the 16 queries of a wave in the
//     accumulator columns and 4 keys per lane in its rows; the online softmax is a
//     per-lane scalar per query, and two accumulator tiles converted to bf16 are the
//     B operand of O^T += V^T P (keys in the permuted contraction order, V^T read by
//     transposing LDS reads in the same order).
//   dk / dv (key tiles): S = Q K^T puts the 16 keys of a wave in the columns; P and
//     dS are then B operands of dV^T += dO^T P and dK^T += Q^T dS.
#include <cmath>

#include "common.h"
#include "launch.h"

namespace harts {
namespace {

constexpr int AT = 64;      // rows per gathered operand tile (and per key tile)
constexpr int ATHR = 256;   // 4 waves
constexpr int QT = 128;     // rows per query tile
constexpr float kLog2e = 1.4426950408889634f;

// 2^x on the hardware instruction alone: probabilities below 2^-126 of the row maximum come out as
// 0 instead of as denormals, which no bf16 product downstream could hold anyway (the library
// exp2f spends five more instructions per element on that range)
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DA, int DB> struct AttnCfg {
  static_assert(DA % 64 == 0 && DB % 64 == 0, "head dims must be multiples of 64");
  static constexpr int LA = DA + 16, LB = DB + 16;   // LDS row strides in elements (32-byte pad)
};

// A-operand fragment of M^T where M is an LDS matrix stored [k][r] (row stride ld): rows
// (M's columns) r0 + l%16, contraction k0 + pf_k(l/16, 0..7) -- two transposing reads.
__device__ __forceinline__ bf16x8 pf_rc(const bf16* p, int ld, int r0, int k0, int lane) {
  const int s = lane & 15;
  const bf16* q = p + (k0 + 4 * (lane >> 4) + (s >> 2)) * ld + r0 + 4 * (s & 3);
  const bf16x4 lo = ds_tr16(q), hi = ds_tr16(q + 16 * ld);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Tile of 64 gathered rows of two row-major arrays (widths DA and DB) loaded by 64 TPR
// threads: thread t loads row t/TPR, 16-byte chunks t%TPR + TPR i; a row index < 0 loads zeros.
template <int DA, int DB, int TPR> struct RowLoad {
  using Cf = AttnCfg<DA, DB>;
  struct N {
    static constexpr int NA = DA / (8 * TPR), NB = DB / (8 * TPR);
  };
  f32x4 a[N::NA], b[N::NB];
  __device__ __forceinline__ void issue(const bf16* A, const bf16* B, int64_t lda, int64_t ldb, int row, int p) {
    if (row >= 0) {
      const bf16* pa = A + row * lda + 8 * p;
      const bf16* pb = B + row * ldb + 8 * p;
#pragma unroll
      for (int i = 0; i < N::NA; ++i) a[i] = ldq(pa + 8 * TPR * i);
#pragma unroll
      for (int i = 0; i < N::NB; ++i) b[i] = ldq(pb + 8 * TPR * i);
    } else {
#pragma unroll
      for (int i = 0; i < N::NA; ++i) a[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < N::NB; ++i) b[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  __device__ __forceinline__ void put(bf16* sA, bf16* sB, int r, int p) const {
#pragma unroll
    for (int i = 0; i < N::NA; ++i) stq(sA + r * Cf::LA + 8 * p + 8 * TPR * i, a[i]);
#pragma unroll
    for (int i = 0; i < N::NB; ++i) stq(sB + r * Cf::LB + 8 * p + 8 * TPR * i, b[i]);
  }
};

__device__ __forceinline__ float wave_quad_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float wave_quad_sum(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

// S^T block products of a query tile: sc[kb] = K[16kb .. 16kb+15] Q^T for the wave's 16 queries
// (sK: the key tile in LDS, row stride LA)
template <int DQ, int LA>
__device__ __forceinline__ void scores_t(const bf16* sK, const bf16x8 (&qf)[DQ / 32], int lane, f32x4 (&sc)[4]) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < DQ / 32; ++s) a = Mma<bf16>::mma(Mma<bf16>::kc(sK, LA, 16 * kb, 32 * s, lane), qf[s], a);
    sc[kb] = a;
  }
}

// two waves per SIMD (<= 256 registers; one spilled): at the unconstrained 320 registers one
// wave per SIMD leaves the gathered loads' latency exposed (16.3 ms against 9.5 ms at dims
// 192/128 on the rollout tree)
template <int DQ, int DV>
__global__ __launch_bounds__(ATHR) __attribute__((amdgpu_waves_per_eu(2))) void attn_fwd_kernel(AttnArgs g) {
  using Cf = AttnCfg<DQ, DV>;
  __shared__ __align__(16) bf16 sK[AT * Cf::LA];
  __shared__ __align__(16) bf16 sV[AT * Cf::LB];
  const int H = g.H, tile = blockIdx.x / H, h = blockIdx.x % H;
  const int4 T = reinterpret_cast<const int4*>(g.tiles)[tile];
  const int row0 = T.x, nr = T.y, base = T.w, nkv = base + nr, nt = (nkv + AT - 1) / AT;
  const int32_t* lst = g.list + T.z;
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 4, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the wave's two query halves: qi[n] = 32 w + 16 n + l % 16
  int qi[2], qrow[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    qi[n] = 32 * (tid >> 6) + 16 * n + (lane & 15);
    qrow[n] = row0 + min(qi[n], nr - 1);
  }
  const int64_t ldq = int64_t(H) * DQ, ldv = int64_t(H) * DV;
  const bf16* kh = g.k + h * DQ;
  const bf16* vh = g.v + h * DV;
  bf16x8 qf[2][DQ / 32];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const bf16* qp = g.q + qrow[n] * ldq + h * DQ + 8 * gq;
#pragma unroll
    for (int s = 0; s < DQ / 32; ++s) qf[n][s] = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
  }
  // rows lr and lr + 32 of each gathered tile, 8 threads per row: every 8-lane group of a tile
  // store writes 128 contiguous bytes of one row (4 threads per row measured LDS bank conflicts)
  const int lr = tid >> 3, lp = tid & 7;
  RowLoad<DQ, DV, 8> ld0, ld1;
  ld0.issue(kh, vh, ldq, ldv, lr < nkv ? lst[lr] : -1, lp);
  ld1.issue(kh, vh, ldq, ldv, lr + 32 < nkv ? lst[lr + 32] : -1, lp);
  int nxt0 = AT + lr < nkv ? lst[AT + lr] : -1, nxt1 = AT + 32 + lr < nkv ? lst[AT + 32 + lr] : -1;
  ld0.put(sK, sV, lr, lp);
  ld1.put(sK, sV, lr + 32, lp);
  __syncthreads();

  const float c = g.scale * kLog2e;
  float mrun[2] = {-INFINITY, -INFINITY}, lsum[2] = {0.f, 0.f};
  f32x4 acc[2][DV / 16];
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) acc[n][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < nt; ++j) {
    if (j + 1 < nt) {
      ld0.issue(kh, vh, ldq, ldv, nxt0, lp);
      ld1.issue(kh, vh, ldq, ldv, nxt1, lp);
      const int u = (j + 2) * AT + lr;
      nxt0 = u < nkv ? lst[u] : -1;
      nxt1 = u + 32 < nkv ? lst[u + 32] : -1;
    }
    f32x4 sc[2][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DQ / 32; ++s) {
        const bf16x8 kf = Mma<bf16>::kc(sK, Cf::LA, 16 * kb, 32 * s, lane);
        a0 = Mma<bf16>::mma(kf, qf[0][s], a0);
        a1 = Mma<bf16>::mma(kf, qf[1][s], a1);
      }
      sc[0][kb] = a0;
      sc[1][kb] = a1;
    }
    bf16x8 pb[2][2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int lim = base + qi[n] - j * AT;  // keys of this tile with index <= lim are visible
      float mx = -INFINITY;
      // hidden keys to -inf, only where the tile is not wholly visible to the half's first query
      // (so to all of its queries)
      if (base + 32 * wv + 16 * n - j * AT < AT - 1) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[n][kb][i] = 16 * kb + 4 * gq + i <= lim ? sc[n][kb][i] : -INFINITY;
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[n][kb][i]);
      mx = wave_quad_max(mx) * c;  // the scale is positive: the maximum of the scaled scores
      // The reference m of the exponentials moves only when some query's maximum passes it by
      // more than 8 (base 2): otherwise the probabilities stay below 2^8 and neither the
      // accumulators nor l need rescaling.  o = acc / l and lse = m + log2 l hold for any m
      // the whole sum shares.  The first tile always moves it (m starts at -inf, and key 0 of
      // the first tile is visible to every query).
      if (__any(mx > mrun[n] + 8.f)) {
        const float mnew = fmaxf(mrun[n], mx);
        const float alpha = exp2_hw(mrun[n] - mnew);
        mrun[n] = mnew;
        lsum[n] *= alpha;
#pragma unroll
        for (int d = 0; d < DV / 16; ++d) acc[n][d] *= alpha;
      }
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2_hw(fmaf(sc[n][kb][i], c, -mrun[n]));
          sc[n][kb][i] = p;
          ps += p;
        }
      lsum[n] += ps;
      pb[n][0] = pf_pair(sc[n][0], sc[n][1]);
      pb[n][1] = pf_pair(sc[n][2], sc[n][3]);
    }
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) {
      const bf16x8 v0 = pf_rc(sV, Cf::LB, 16 * d, 0, lane), v1 = pf_rc(sV, Cf::LB, 16 * d, 32, lane);
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        acc[n][d] = Mma<bf16>::mma(v0, pb[n][0], acc[n][d]);
        acc[n][d] = Mma<bf16>::mma(v1, pb[n][1], acc[n][d]);
      }
    }
    if (j + 1 < nt) {
      __syncthreads();
      ld0.put(sK, sV, lr, lp);
      ld1.put(sK, sV, lr + 32, lp);
      __syncthreads();
    }
  }
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const float l = wave_quad_sum(lsum[n]);
    if (qi[n] < nr) {
      const float inv = 1.f / l;
      bf16* op = g.o_out + qrow[n] * ldv + h * DV + 4 * gq;
#pragma unroll
      for (int d = 0; d < DV / 16; ++d)
        store4<bf16>(op + 16 * d, acc[n][d][0] * inv, acc[n][d][1] * inv, acc[n][d][2] * inv, acc[n][d][3] * inv);
      if (gq == 0) g.lse_out[int64_t(qrow[n]) * H + h] = (mrun[n] + log2f(l)) * (1.f / kLog2e);
    }
  }
}

// delta[t, h] = <dout[t, h], o[t, h]> over the value dimension (fp32)
template <int DV>
__global__ __launch_bounds__(256) void attn_delta_kernel(const bf16* o, const bf16* dout, float* delta, int64_t n) {
  constexpr int L = DV / 8;  // lanes per (row, head)
  const int64_t pair = (int64_t(blockIdx.x) * 256 + threadIdx.x) / L;
  const int sub = threadIdx.x % L;
  float acc = 0.f;
  if (pair < n) {
    float a[8], b[8];
    ld16<bf16>(o + pair * DV + 8 * sub, a);
    ld16<bf16>(dout + pair * DV + 8 * sub, b);
#pragma unroll
    for (int t = 0; t < 8; ++t) acc += a[t] * b[t];
  }
#pragma unroll
  for (int m = L / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (pair < n && sub == 0) delta[pair] = acc;
}

template <int DQ, int DV>
__global__ __launch_bounds__(2 * ATHR) void attn_dq_kernel(AttnArgs g) {
  using Cf = AttnCfg<DQ, DV>;
  __shared__ __align__(16) bf16 sK[AT * Cf::LA];
  __shared__ __align__(16) bf16 sV[AT * Cf::LB];
  const int H = g.H, tile = blockIdx.x / H, h = blockIdx.x % H;
  const int4 T = reinterpret_cast<const int4*>(g.tiles)[tile];
  const int row0 = T.x, nr = T.y, base = T.w, nkv = base + nr, nt = (nkv + AT - 1) / AT;
  const int32_t* lst = g.list + T.z;
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 4, qi = 16 * (tid >> 6) + (lane & 15);
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qrow = row0 + min(qi, nr - 1);
  const int64_t ldq = int64_t(H) * DQ, ldv = int64_t(H) * DV;
  const bf16* kh = g.k + h * DQ;
  const bf16* vh = g.v + h * DV;
  bf16x8 qf[DQ / 32], df[DV / 32];
  {
    const bf16* qp = g.q + qrow * ldq + h * DQ + 8 * gq;
#pragma unroll
    for (int s = 0; s < DQ / 32; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + 32 * s);
    const bf16* dp = g.dout + qrow * ldv + h * DV + 8 * gq;
#pragma unroll
    for (int s = 0; s < DV / 32; ++s) df[s] = *reinterpret_cast<const bf16x8*>(dp + 32 * s);
  }
  const float lse2 = g.lse[int64_t(qrow) * H + h] * kLog2e, dlt = g.delta[int64_t(qrow) * H + h];
  const int lr = tid >> 3, lp = tid & 7;
  RowLoad<DQ, DV, 8> ld;
  ld.issue(kh, vh, ldq, ldv, lr < nkv ? lst[lr] : -1, lp);
  int nxt = AT + lr < nkv ? lst[AT + lr] : -1;
  ld.put(sK, sV, lr, lp);
  __syncthreads();

  const float c = g.scale * kLog2e;
  f32x4 acc[DQ / 16];
#pragma unroll
  for (int d = 0; d < DQ / 16; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < nt; ++j) {
    if (j + 1 < nt) {
      ld.issue(kh, vh, ldq, ldv, nxt, lp);
      const int u = (j + 2) * AT + lr;
      nxt = u < nkv ? lst[u] : -1;
    }
    f32x4 sc[4], dp[4];
    scores_t<DQ, Cf::LA>(sK, qf, lane, sc);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DV / 32; ++s) a = Mma<bf16>::mma(Mma<bf16>::kc(sV, Cf::LB, 16 * kb, 32 * s, lane), df[s], a);
      dp[kb] = a;
    }
    const int lim = base + qi - j * AT;
    // hidden keys to -inf (probability 0), only where the tile is not wholly visible to the
    // wave's first query
    if (base + 16 * wv - j * AT < AT - 1) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[kb][i] = 16 * kb + 4 * gq + i <= lim ? sc[kb][i] : -INFINITY;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[kb][i] = exp2_hw(sc[kb][i] * c - lse2) * (dp[kb][i] - dlt);
    const bf16x8 s0 = pf_pair(sc[0], sc[1]), s1 = pf_pair(sc[2], sc[3]);
#pragma unroll
    for (int d = 0; d < DQ / 16; ++d) {
      acc[d] = Mma<bf16>::mma(pf_rc(sK, Cf::LA, 16 * d, 0, lane), s0, acc[d]);
      acc[d] = Mma<bf16>::mma(pf_rc(sK, Cf::LA, 16 * d, 32, lane), s1, acc[d]);
    }
    if (j + 1 < nt) {
      __syncthreads();
      ld.put(sK, sV, lr, lp);
      __syncthreads();
    }
  }
  if (qi < nr) {
    const float sc = g.scale;
    bf16* op = g.dq + qrow * ldq + h * DQ + 4 * gq;
#pragma unroll
    for (int d = 0; d < DQ / 16; ++d)
      store4<bf16>(op + 16 * d, acc[d][0] * sc, acc[d][1] * sc, acc[d][2] * sc, acc[d][3] * sc);
  }
}

// dk / dv over a 128-row key tile: 8 waves of 16 keys, so that each gathered query tile serves
// 128 keys and two waves share a SIMD (the accumulators and the operands of 16 keys, and half of
// the register prefetch of a 64-row tile, fit in 256 registers)
template <int DQ, int DV>
__global__ __launch_bounds__(2 * ATHR) void attn_dkv_kernel(AttnArgs g) {
  using Cf = AttnCfg<DQ, DV>;
  __shared__ __align__(16) bf16 sQ[AT * Cf::LA];
  __shared__ __align__(16) bf16 sO[AT * Cf::LB];  // dout rows
  __shared__ __align__(16) float sL[AT], sD[AT];
  const int H = g.H, tile = blockIdx.x / H, h = blockIdx.x % H;
  const int4 T = reinterpret_cast<const int4*>(g.tiles)[tile];
  const int row0 = T.x, nk = T.y, nq = T.w, nt = (nq + AT - 1) / AT;
  const int32_t* lst = g.list + T.z;
  const int tid = threadIdx.x, lane = tid & 63, gq = lane >> 4, kk = 16 * (tid >> 6) + (lane & 15);
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int krow = row0 + min(kk, nk - 1);
  const int64_t ldq = int64_t(H) * DQ, ldv = int64_t(H) * DV;
  const bf16* qh = g.q + h * DQ;
  const bf16* oh = g.dout + h * DV;
  bf16x8 kf[DQ / 32], vf[DV / 32];
  {
    const bf16* kp = g.k + krow * ldq + h * DQ + 8 * gq;
#pragma unroll
    for (int s = 0; s < DQ / 32; ++s) kf[s] = *reinterpret_cast<const bf16x8*>(kp + 32 * s);
    const bf16* vp = g.v + krow * ldv + h * DV + 8 * gq;
#pragma unroll
    for (int s = 0; s < DV / 32; ++s) vf[s] = *reinterpret_cast<const bf16x8*>(vp + 32 * s);
  }
  const int lr = tid >> 3, lp = tid & 7;
  RowLoad<DQ, DV, 8> ld;
  float xl = 0.f, xd = 0.f;
  auto issue = [&](int row) {
    ld.issue(qh, oh, ldq, ldv, row, lp);
    if (lp == 0) {
      xl = row >= 0 ? g.lse[int64_t(row) * H + h] * kLog2e : 0.f;
      xd = row >= 0 ? g.delta[int64_t(row) * H + h] : 0.f;
    }
  };
  auto put = [&]() {
    ld.put(sQ, sO, lr, lp);
    if (lp == 0) {
      sL[lr] = xl;
      sD[lr] = xd;
    }
  };
  issue(lr < nq ? lst[lr] : -1);
  int nxt = AT + lr < nq ? lst[AT + lr] : -1;
  put();
  __syncthreads();

  const float c = g.scale * kLog2e;
  f32x4 av[DV / 16], ak[DQ / 16];
#pragma unroll
  for (int d = 0; d < DV / 16; ++d) av[d] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int d = 0; d < DQ / 16; ++d) ak[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < nt; ++j) {
    if (j + 1 < nt) {
      issue(nxt);
      const int u = (j + 2) * AT + lr;
      nxt = u < nq ? lst[u] : -1;
    }
    f32x4 sp[4], sd[4];
    // every query of the tile sees every key of the wave: below the wave's last key, inside nq
    const bool open = j * AT >= 16 * wv + 15 && (j + 1) * AT <= nq;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < DQ / 32; ++s) a = Mma<bf16>::mma(Mma<bf16>::kc(sQ, Cf::LA, 16 * qb, 32 * s, lane), kf[s], a);
#pragma unroll
      for (int s = 0; s < DV / 32; ++s) b = Mma<bf16>::mma(Mma<bf16>::kc(sO, Cf::LB, 16 * qb, 32 * s, lane), vf[s], b);
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(sL + 16 * qb + 4 * gq);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(sD + 16 * qb + 4 * gq);
      if (!open) {  // hidden pairs to -inf (probability 0)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int u = j * AT + 16 * qb + 4 * gq + i;
          a[i] = (u >= kk && u < nq) ? a[i] : -INFINITY;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2_hw(a[i] * c - l4[i]);
        sp[qb][i] = p;
        sd[qb][i] = p * (b[i] - d4[i]);
      }
    }
    const bf16x8 p0 = pf_pair(sp[0], sp[1]), p1 = pf_pair(sp[2], sp[3]);
    const bf16x8 s0 = pf_pair(sd[0], sd[1]), s1 = pf_pair(sd[2], sd[3]);
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) {
      av[d] = Mma<bf16>::mma(pf_rc(sO, Cf::LB, 16 * d, 0, lane), p0, av[d]);
      av[d] = Mma<bf16>::mma(pf_rc(sO, Cf::LB, 16 * d, 32, lane), p1, av[d]);
    }
#pragma unroll
    for (int d = 0; d < DQ / 16; ++d) {
      ak[d] = Mma<bf16>::mma(pf_rc(sQ, Cf::LA, 16 * d, 0, lane), s0, ak[d]);
      ak[d] = Mma<bf16>::mma(pf_rc(sQ, Cf::LA, 16 * d, 32, lane), s1, ak[d]);
    }
    if (j + 1 < nt) {
      __syncthreads();
      put();
      __syncthreads();
    }
  }
  if (kk < nk) {
    bf16* vp = g.dv + krow * ldv + h * DV + 4 * gq;
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) store4<bf16>(vp + 16 * d, av[d][0], av[d][1], av[d][2], av[d][3]);
    const float sc = g.scale;
    bf16* kp = g.dk + krow * ldq + h * DQ + 4 * gq;
#pragma unroll
    for (int d = 0; d < DQ / 16; ++d)
      store4<bf16>(kp + 16 * d, ak[d][0] * sc, ak[d][1] * sc, ak[d][2] * sc, ak[d][3] * sc);
  }
}

template <int DQ, int DV>
hipError_t attn_dispatch(int which, const AttnArgs& a, int64_t n_tiles, hipStream_t s) {
  if (which == 1) {
    const int64_t n = a.C * a.H;
    constexpr int L = DV / 8;
    const int64_t blocks = (n * L + 255) / 256;
    hipLaunchKernelGGL(attn_delta_kernel<DV>, dim3(unsigned(blocks)), dim3(256), 0, s, a.dout, a.o, a.delta_out, n);
    return hipGetLastError();
  }
  const dim3 grid(unsigned(n_tiles * a.H)), block(ATHR);
  if (which == 0) hipLaunchKernelGGL((attn_fwd_kernel<DQ, DV>), grid, block, 0, s, a);
  else if (which == 2) hipLaunchKernelGGL((attn_dq_kernel<DQ, DV>), grid, dim3(2 * ATHR), 0, s, a);
  else hipLaunchKernelGGL((attn_dkv_kernel<DQ, DV>), grid, dim3(2 * ATHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool attn_dims_supported(int dqk, int dv) {
  return (dqk == 192 && dv == 128) || (dqk == 128 && dv == 128) || (dqk == 64 && dv == 64);
}

hipError_t launch_attn(int which, const AttnArgs& a, int64_t n_tiles, int dqk, int dv, hipStream_t s) {
  if (dqk == 192 && dv == 128) return attn_dispatch<192, 128>(which, a, n_tiles, s);
  if (dqk == 128 && dv == 128) return attn_dispatch<128, 128>(which, a, n_tiles, s);
  if (dqk == 64 && dv == 64) return attn_dispatch<64, 64>(which, a, n_tiles, s);
  return hipErrorInvalidValue;
}

}  // namespace harts
