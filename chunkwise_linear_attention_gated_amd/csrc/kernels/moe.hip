// Router statistics of compact rows weighted by their multiplicities (HARTS
// blog sections 4.3 and 4.4; arXiv summary, section 4 "MoE execution"; Figure
// C.1(d)).  A compact row is routed once; q_c, the number of semantic positions
// that read row c, weights its z-loss term, its probability mass and its top-k
// assignment counts, so the statistics equal those of the expanded positions
// while routing decisions stay those of the row.
//
//   route:  one 16-lane group per row (E / 16 logits per lane, four rows per
//           wave at once): softmax, lse, top-k of p + bias by k arg-max rounds
//           over the group (ties: lower expert); per workgroup: q-weighted
//           counts by LDS integer adds (exact), mass and z-loss summed over its
//           rows in row order, written as one partial row
//   reduce: two fixed-order levels: whole rows of the partials in 64 row chunks,
//           then one workgroup per column of the chunk sums
//   aux:    E / (k S^2) sum_e n_e P_e
//   grad:   dz = z_coef 2 q lse p / S + aux_coef E / (k S^2) q p (n - <n, p>),
//           a row per 16-lane group
//   bias:   b_e += gamma sign(mean n - n_e)
#include <cmath>

#include "common.h"
#include "launch.h"

namespace harts {
namespace {

constexpr int MR = 16;   // rows per workgroup: a row per 16-lane group
constexpr int MT = 256;  // 4 waves

constexpr int MR1 = 64;  // row chunks of the first reduction level
// partial rows: [rows][E + 1] float (mass, z-loss sum), then [rows][E] int32 (counts); rows = one
// per route workgroup, then MR1 rows of first-level sums
__host__ __device__ inline int64_t moe_blocks(int64_t C) { return (C + MR - 1) / MR; }
__host__ __device__ inline int64_t moe_partial_rows_dev(int64_t C) { return moe_blocks(C) + MR1; }

// Exchanges within a row group of 16 lanes by data-parallel-primitive moves (vector ALU, no LDS
// round trip): swap adjacent lanes, swap lane pairs, mirror each half row, mirror the row.  After
// the four steps of a reduction every lane of the group holds the group's result.
constexpr int kDppSwap1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kDppSwap2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141; // row_half_mirror
constexpr int kDppMirror = 0x140;     // row_mirror
template <int CTRL> __device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xF, 0xF, false);
}
template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, x)));
}
__device__ __forceinline__ float gsum(float x) {
  x += dpp_f<kDppSwap1>(x);
  x += dpp_f<kDppSwap2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  return x + dpp_f<kDppMirror>(x);
}
__device__ __forceinline__ float gmax(float x) {
  x = fmaxf(x, dpp_f<kDppSwap1>(x));
  x = fmaxf(x, dpp_f<kDppSwap2>(x));
  x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  return fmaxf(x, dpp_f<kDppMirror>(x));
}
// (value, expert) of the larger score, the lower expert on a tie
template <int CTRL> __device__ __forceinline__ void gargmax_step(float& bv, int& bi) {
  const float ov = dpp_f<CTRL>(bv);
  const int oi = dpp_i<CTRL>(bi);
  if (ov > bv || (ov == bv && oi < bi)) {
    bv = ov;
    bi = oi;
  }
}

// Route: a row per 16-lane group (4 rows per wave at once), lane i of the group holding experts
// NL i .. NL i + NL - 1 (NL = E / 16, contiguous: two or more 16-byte loads).  The top-k rounds
// are butterflies over the group's 16 lanes, four rows' chains interleaved in each wave.
template <int NE>
__global__ __launch_bounds__(MT) void moe_route_kernel(MoeArgs a) {
  constexpr int E = NE * 64, NL = E / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, gl = lane & 15, grp = lane >> 4;
  const int e0 = NL * gl;
  float b[NL], mass[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    b[j] = a.bias ? a.bias[e0 + j] : 0.f;
    mass[j] = 0.f;
  }
  float zs = 0.f;
  __shared__ int32_t cnt[E];
  for (int e = threadIdx.x; e < E; e += MT) cnt[e] = 0;
  __syncthreads();
  const int64_t c = int64_t(blockIdx.x) * MR + 4 * wave + grp;  // MR == 4 rows x 4 waves
  if (c < a.C) {
    float p[NL];
    const float* zr = a.z + c * E + e0;
#pragma unroll
    for (int j = 0; j < NL; j += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(zr + j);
      p[j] = v[0];
      p[j + 1] = v[1];
      p[j + 2] = v[2];
      p[j + 3] = v[3];
    }
    float m = p[0];
#pragma unroll
    for (int j = 1; j < NL; ++j) m = fmaxf(m, p[j]);
    m = gmax(m);
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      p[j] = __expf(p[j] - m);  // exponent <= 0: the hardware 2^x after one multiply
      sum += p[j];
    }
    sum = gsum(sum);
    const float inv = 1.f / sum, lse = m + logf(sum);
    const int qc = a.q[c];
    const float qf = float(qc);
    float sc[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      p[j] *= inv;
      mass[j] = qf * p[j];
      sc[j] = p[j] + b[j];
    }
    zs = qf * lse * lse;
    for (int t = 0; t < a.k; ++t) {
      float bv = sc[0];
      int bi = e0;
#pragma unroll
      for (int j = 1; j < NL; ++j)
        if (sc[j] > bv) {  // strict: the lower expert of a tie stays
          bv = sc[j];
          bi = e0 + j;
        }
      gargmax_step<kDppSwap1>(bv, bi);
      gargmax_step<kDppSwap2>(bv, bi);
      gargmax_step<kDppHalfMirror>(bv, bi);
      gargmax_step<kDppMirror>(bv, bi);
#pragma unroll
      for (int j = 0; j < NL; ++j)
        if (bi == e0 + j) sc[j] = -INFINITY;
      if (gl == 0) {
        a.top[c * a.k + t] = bi;
        atomicAdd(cnt + bi, qc);  // LDS
      }
    }
    if (gl == 0) a.lse[c] = lse;
  }
  // this workgroup's mass and z-loss sums over its 16 rows, in row order
  __shared__ float sm[MR][E];
  __shared__ float sz[MR];
#pragma unroll
  for (int j = 0; j < NL; ++j) sm[4 * wave + grp][e0 + j] = mass[j];
  if (gl == 0) sz[4 * wave + grp] = zs;
  __syncthreads();
  float* part = a.part + int64_t(blockIdx.x) * (E + 1);
  int32_t* ipart = reinterpret_cast<int32_t*>(a.part + moe_partial_rows_dev(a.C) * (E + 1)) + int64_t(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += MT) {
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < MR; ++r) acc += sm[r][e];
    part[e] = acc;
    ipart[e] = cnt[e];
  }
  if (threadIdx.x == 0) {
    float acc = 0.f;
#pragma unroll
    for (int r = 0; r < MR; ++r) acc += sz[r];
    part[E] = acc;
  }
}

// First level: chunk rc of the route partials' rows, 64 columns per workgroup (e == E: the
// z-loss sums), four row phases summed in row order each, then in phase order; reads whole rows
__global__ __launch_bounds__(256) void moe_reduce1_kernel(MoeArgs a) {
  const int E = a.E;
  const int64_t nblk = moe_blocks(a.C), rows = moe_partial_rows_dev(a.C), per = (nblk + MR1 - 1) / MR1;
  const int l = threadIdx.x & 63, ph = threadIdx.x >> 6, col = 64 * blockIdx.x + l;
  const int64_t rc = blockIdx.y, r0 = rc * per, r1 = r0 + per < nblk ? r0 + per : nblk;
  int32_t* ipart = reinterpret_cast<int32_t*>(a.part + rows * (E + 1));
  float acc = 0.f;
  int32_t iacc = 0;
  if (col <= E)
    for (int64_t i = r0 + ph; i < r1; i += 4) {
      acc += a.part[i * (E + 1) + col];
      if (col < E) iacc += ipart[i * E + col];
    }
  __shared__ float red[4][64];
  __shared__ int32_t ired[4][64];
  red[ph][l] = acc;
  ired[ph][l] = iacc;
  __syncthreads();
  if (ph == 0 && col <= E) {
    a.part[(nblk + rc) * (E + 1) + col] = ((red[0][l] + red[1][l]) + red[2][l]) + red[3][l];
    if (col < E) ipart[(nblk + rc) * E + col] = ((ired[0][l] + ired[1][l]) + ired[2][l]) + ired[3][l];
  }
}

// column e of the first-level sums (e == E: the z-loss sums), fixed order: strided per thread,
// then a tree
__global__ __launch_bounds__(256) void moe_reduce_kernel(MoeArgs a) {
  const int E = a.E, e = blockIdx.x;
  const int64_t nblk = moe_blocks(a.C), rows = moe_partial_rows_dev(a.C);
  const int32_t* ipart = reinterpret_cast<const int32_t*>(a.part + rows * (E + 1));
  float acc = 0.f;
  int64_t iacc = 0;
  for (int64_t i = nblk + threadIdx.x; i < rows; i += 256) {
    acc += a.part[i * (E + 1) + e];
    if (e < E) iacc += ipart[i * E + e];
  }
  __shared__ float red[256];
  __shared__ long long ired[256];
  red[threadIdx.x] = acc;
  ired[threadIdx.x] = iacc;
  __syncthreads();
  for (int h = 128; h >= 1; h >>= 1) {
    if (int(threadIdx.x) < h) {
      red[threadIdx.x] += red[threadIdx.x + h];
      ired[threadIdx.x] += ired[threadIdx.x + h];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (e < E) {
      a.mass[e] = red[0];
      a.counts[e] = int32_t(ired[0]);
    } else {
      a.losses[0] = a.S > 0 ? red[0] / float(a.S) : 0.f;
    }
  }
}

// L_aux = E / (k S^2) sum_e n_e P_e (one workgroup)
__global__ __launch_bounds__(256) void moe_aux_kernel(MoeArgs a) {
  float acc = 0.f;
  for (int e = threadIdx.x; e < a.E; e += 256) acc += float(a.counts[e]) * a.mass[e];
  __shared__ float red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int h = 128; h >= 1; h >>= 1) {
    if (int(threadIdx.x) < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double S = double(a.S);
    a.losses[1] = a.S > 0 ? float(double(a.E) / (double(a.k) * S * S) * double(red[0])) : 0.f;
  }
}

// Gradient: a row per 16-lane group as in the route, NL contiguous experts per lane.
template <int NE>
__global__ __launch_bounds__(MT) void moe_grad_kernel(MoeArgs a) {
  constexpr int E = NE * 64, NL = E / 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, gl = lane & 15, grp = lane >> 4;
  const int e0 = NL * gl;
  const int64_t c = int64_t(blockIdx.x) * MR + 4 * wave + grp;
  if (c >= a.C) return;
  float n[NL];
#pragma unroll
  for (int j = 0; j < NL; ++j) n[j] = float(a.counts[e0 + j]);
  const double S = double(a.S);
  const float cz = float(2.0 * double(a.z_coef) / S);
  const float ca = float(double(a.aux_coef) * double(E) / (double(a.k) * S * S));
  float p[NL];
  const float* zr = a.z + c * E + e0;
#pragma unroll
  for (int j = 0; j < NL; j += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(zr + j);
    p[j] = v[0];
    p[j + 1] = v[1];
    p[j + 2] = v[2];
    p[j + 3] = v[3];
  }
  float m = p[0];
#pragma unroll
  for (int j = 1; j < NL; ++j) m = fmaxf(m, p[j]);
  m = gmax(m);
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    p[j] = __expf(p[j] - m);  // as in the route kernel
    sum += p[j];
  }
  sum = gsum(sum);
  const float inv = 1.f / sum, lse = m + logf(sum);
  float nb = 0.f;
#pragma unroll
  for (int j = 0; j < NL; ++j) {
    p[j] *= inv;
    nb += p[j] * n[j];
  }
  nb = gsum(nb);
  const float qf = float(a.q[c]);
  float* dr = a.dz + c * E + e0;
#pragma unroll
  for (int j = 0; j < NL; j += 4) {
    f32x4 v;
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = qf * p[j + t] * (cz * lse + ca * (n[j + t] - nb));
    *reinterpret_cast<f32x4*>(dr + j) = v;
  }
}

// b_e += gamma sign(mean_j n_j - n_e) (one workgroup)
__global__ __launch_bounds__(256) void moe_bias_kernel(const int32_t* counts, int E, float gamma, float* bias) {
  int64_t acc = 0;
  for (int e = threadIdx.x; e < E; e += 256) acc += counts[e];
  __shared__ long long red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int h = 128; h >= 1; h >>= 1) {
    if (int(threadIdx.x) < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  const double mean = double(red[0]) / double(E);
  for (int e = threadIdx.x; e < E; e += 256) {
    const double d = mean - double(counts[e]);
    bias[e] += d > 0 ? gamma : (d < 0 ? -gamma : 0.f);
  }
}

template <int NE>
hipError_t moe_run(int which, const MoeArgs& a, hipStream_t s) {
  const int64_t nblk = moe_blocks(a.C);
  if (which == 0) {
    if (a.C > 0) hipLaunchKernelGGL(moe_route_kernel<NE>, dim3(unsigned(nblk)), dim3(MT), 0, s, a);
    hipLaunchKernelGGL(moe_reduce1_kernel, dim3(unsigned((a.E + 1 + 63) / 64), unsigned(MR1)), dim3(256), 0, s, a);
    hipLaunchKernelGGL(moe_reduce_kernel, dim3(unsigned(a.E + 1)), dim3(256), 0, s, a);
    hipLaunchKernelGGL(moe_aux_kernel, dim3(1), dim3(256), 0, s, a);
  } else if (a.C > 0) {
    hipLaunchKernelGGL(moe_grad_kernel<NE>, dim3(unsigned(nblk)), dim3(MT), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

int64_t moe_partial_rows(int64_t C) { return moe_partial_rows_dev(C); }

hipError_t launch_moe(int which, const MoeArgs& a, hipStream_t s) {
  switch (a.E) {
    case 64: return moe_run<1>(which, a, s);
    case 128: return moe_run<2>(which, a, s);
    case 256: return moe_run<4>(which, a, s);
    case 512: return moe_run<8>(which, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_moe_bias(const int32_t* counts, int E, float gamma, float* bias, hipStream_t s) {
  hipLaunchKernelGGL(moe_bias_kernel, dim3(1), dim3(256), 0, s, counts, E, gamma, bias);
  return hipGetLastError();
}

}  // namespace harts
