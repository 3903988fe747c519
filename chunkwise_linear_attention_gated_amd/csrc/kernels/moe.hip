// Router statistics of compact rows weighted by their multiplicities (HARTS
// blog sections 4.3 and 4.4; arXiv summary, section 4 "MoE execution"; Figure
// C.1(d)).  A compact row is routed once; q_c, the number of semantic positions
// that read row c, weights its z-loss term, its probability mass and its top-k
// assignment counts, so the statistics equal those of the expanded positions
// while routing decisions stay those of the row.
//
//   route:  one wave per row (E / 64 logits per lane): softmax, lse, top-k of
//           p + bias by k wave-wide arg-max rounds (ties: lower expert); per
//           workgroup: q-weighted counts by LDS integer adds (exact), mass and
//           z-loss in a fixed order, written as one partial row
//   reduce: one workgroup per column of the partials, fixed-order sum
//   aux:    E / (k S^2) sum_e n_e P_e
//   grad:   dz = z_coef 2 q lse p / S + aux_coef E / (k S^2) q p (n - <n, p>)
//   bias:   b_e += gamma sign(mean n - n_e)
#include <cmath>

#include "common.h"
#include "launch.h"

namespace harts {
namespace {

constexpr int MR = 16;   // rows per workgroup (4 per wave: latency-bound shuffle chains want many waves)
constexpr int MT = 256;  // 4 waves, one row at a time each

// partial rows: [nblk][E + 1] float (mass, z-loss sum), then [nblk][E] int32 (counts)
__host__ __device__ inline int64_t moe_partial_rows_dev(int64_t C) { return (C + MR - 1) / MR; }

__device__ __forceinline__ float wsum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wmax(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// softmax of one row held as NE values per lane (expert lane + 64 j)
template <int NE>
__device__ __forceinline__ float row_softmax(float (&x)[NE]) {
  float m = x[0];
#pragma unroll
  for (int j = 1; j < NE; ++j) m = fmaxf(m, x[j]);
  m = wmax(m);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    x[j] = expf(x[j] - m);
    s += x[j];
  }
  s = wsum(s);
  const float inv = 1.f / s;
#pragma unroll
  for (int j = 0; j < NE; ++j) x[j] *= inv;
  return m + logf(s);
}

template <int NE>
__global__ __launch_bounds__(MT) void moe_route_kernel(MoeArgs a) {
  constexpr int E = NE * 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float b[NE], mass[NE];
#pragma unroll
  for (int j = 0; j < NE; ++j) {
    b[j] = a.bias ? a.bias[lane + 64 * j] : 0.f;
    mass[j] = 0.f;
  }
  float zs = 0.f;
  __shared__ int32_t cnt[E];
  for (int e = threadIdx.x; e < E; e += MT) cnt[e] = 0;
  __syncthreads();
  for (int r = wave; r < MR; r += MT / 64) {
    const int64_t c = int64_t(blockIdx.x) * MR + r;
    if (c >= a.C) break;
    float p[NE];
#pragma unroll
    for (int j = 0; j < NE; ++j) p[j] = a.z[c * E + lane + 64 * j];
    const float lse = row_softmax<NE>(p);
    const int qc = a.q[c];
    const float qf = float(qc);
    float sc[NE];
#pragma unroll
    for (int j = 0; j < NE; ++j) {
      mass[j] += qf * p[j];
      sc[j] = p[j] + b[j];
    }
    zs += qf * lse * lse;
    for (int t = 0; t < a.k; ++t) {
      float bv = sc[0];
      int bi = lane;
#pragma unroll
      for (int j = 1; j < NE; ++j)
        if (sc[j] > bv) {  // strict: the lower expert of a tie stays
          bv = sc[j];
          bi = lane + 64 * j;
        }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
#pragma unroll
      for (int j = 0; j < NE; ++j)
        if (bi == lane + 64 * j) sc[j] = -INFINITY;
      if (lane == 0) {
        a.top[c * a.k + t] = bi;
        atomicAdd(cnt + bi, qc);  // LDS
      }
    }
    if (lane == 0) a.lse[c] = lse;
  }
  __shared__ float sm[MT / 64][E];
  __shared__ float sz[MT / 64];
#pragma unroll
  for (int j = 0; j < NE; ++j) sm[wave][lane + 64 * j] = mass[j];
  if (lane == 0) sz[wave] = zs;
  __syncthreads();
  float* part = a.part + int64_t(blockIdx.x) * (E + 1);
  int32_t* ipart = reinterpret_cast<int32_t*>(a.part + moe_partial_rows_dev(a.C) * (E + 1)) + int64_t(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += MT) {
    part[e] = ((sm[0][e] + sm[1][e]) + sm[2][e]) + sm[3][e];
    ipart[e] = cnt[e];
  }
  if (threadIdx.x == 0) part[E] = ((sz[0] + sz[1]) + sz[2]) + sz[3];
}

// column e of the partials (e == E: the z-loss sums), fixed order: strided per thread, then a tree
__global__ __launch_bounds__(256) void moe_reduce_kernel(MoeArgs a, int64_t nblk) {
  const int E = a.E, e = blockIdx.x;
  const int32_t* ipart = reinterpret_cast<const int32_t*>(a.part + nblk * (E + 1));
  float acc = 0.f;
  int64_t iacc = 0;
  for (int64_t i = threadIdx.x; i < nblk; i += 256) {
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

template <int NE>
__global__ __launch_bounds__(MT) void moe_grad_kernel(MoeArgs a) {
  constexpr int E = NE * 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float n[NE];
#pragma unroll
  for (int j = 0; j < NE; ++j) n[j] = float(a.counts[lane + 64 * j]);
  const double S = double(a.S);
  const float cz = float(2.0 * double(a.z_coef) / S);
  const float ca = float(double(a.aux_coef) * double(E) / (double(a.k) * S * S));
  for (int r = wave; r < MR; r += MT / 64) {
    const int64_t c = int64_t(blockIdx.x) * MR + r;
    if (c >= a.C) break;
    float p[NE];
#pragma unroll
    for (int j = 0; j < NE; ++j) p[j] = a.z[c * E + lane + 64 * j];
    const float lse = row_softmax<NE>(p);
    float nb = 0.f;
#pragma unroll
    for (int j = 0; j < NE; ++j) nb += p[j] * n[j];
    nb = wsum(nb);
    const float qf = float(a.q[c]);
#pragma unroll
    for (int j = 0; j < NE; ++j) a.dz[c * E + lane + 64 * j] = qf * p[j] * (cz * lse + ca * (n[j] - nb));
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
  const int64_t nblk = (a.C + MR - 1) / MR;
  if (which == 0) {
    if (a.C > 0) hipLaunchKernelGGL(moe_route_kernel<NE>, dim3(unsigned(nblk)), dim3(MT), 0, s, a);
    hipLaunchKernelGGL(moe_reduce_kernel, dim3(unsigned(a.E + 1)), dim3(256), 0, s, a, nblk);
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
