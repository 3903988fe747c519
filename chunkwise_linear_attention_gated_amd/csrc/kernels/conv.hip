// Depthwise causal convolution over the compact rows of a rollout tree on gfx950 (HARTS
// close-reading blog, section 4.3: the convolution's context for a branch is built from its real
// ancestors' last w - 1 projected activations, and windows never cross into another
// trajectory).  Each row's window is read through a per-row ancestor table (row of the token j
// places earlier on the row's trajectories, -1 before the first token), so a fork's branches
// all see their common prefix and no row is expanded:
//
//   out[t, c] = sum_{j<w} weight[c, j] x[anc_j(t), c]                         (anc_0(t) = t)
//   dx[s, c]  = weight[c, 0] dout[s, c] + sum_{(t, j): anc_j(t) = s} weight[c, j] dout[t, c]
//   dweight[c, j] = sum_t dout[t, c] x[anc_j(t), c]
//
// Every pass moves 16-byte pieces of 8 channels, a thread keeping its channels' weights in
// registers over a block of rows; dx gathers over a per-row list of (t, j) in a fixed order and
// dweight sums fixed row blocks, then the blocks in order, so the results do not depend on
// scheduling.  The windows' reads of earlier rows mostly hit the L2 (rows of one
// branch are contiguous).
#include "common.h"
#include "launch.h"

namespace harts {

constexpr int kConvRowBlock = 256;  // rows per partial sum of dweight

template <typename T>
__device__ __forceinline__ void ld8(const T* p, float* v) {
  if constexpr (sizeof(T) == 2) {
    unpack16<T>(*reinterpret_cast<const f32x4*>(p), v);
  } else {
    unpack16<T>(*reinterpret_cast<const f32x4*>(p), v);
    unpack16<T>(*reinterpret_cast<const f32x4*>(p + 4), v + 4);
  }
}
template <typename T>
__device__ __forceinline__ void st8(T* p, const float* v) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<f32x4*>(p) = pack16<T>(v);
  } else {
    *reinterpret_cast<f32x4*>(p) = pack16<T>(v);
    *reinterpret_cast<f32x4*>(p + 4) = pack16<T>(v + 4);
  }
}

// Forward and dx: grid (channel pieces / 256, row blocks of kConvRows); a thread keeps its 8
// channels' weights in registers and walks the block's rows, whose ancestor rows and gather
// lists are uniform over the workgroup (scalar loads).
constexpr int kConvRows = 64;

template <typename T, int W>
__device__ __forceinline__ void conv_weights(const float* __restrict__ wt, int c0, float (&wv)[W][8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int j = 0; j < W; ++j) wv[j][e] = wt[(c0 + e) * W + j];
}

template <typename T, int W>
__global__ __launch_bounds__(256) void conv_fwd_kernel(const T* __restrict__ x, const float* __restrict__ wt,
                                                       const int32_t* __restrict__ anc, int64_t C, int32_t ch,
                                                       T* __restrict__ out) {
  const int c0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  float wv[W][8];
  conv_weights<T, W>(wt, c0 < ch ? c0 : 0, wv);
  const int64_t t0 = int64_t(blockIdx.y) * kConvRows, t1 = t0 + kConvRows < C ? t0 + kConvRows : C;
  // the block's ancestor rows, staged once
  __shared__ int32_t sa[kConvRows * (W - 1)];
  for (int i = threadIdx.x; i < int(t1 - t0) * (W - 1); i += 256) sa[i] = anc[t0 * (W - 1) + i];
  __syncthreads();
  if (c0 >= ch) return;
  // hist[j - 1]: this thread's channels of row t - j, read in an earlier iteration (a branch's
  // rows are contiguous, so most windows are the previous rows)
  float hist[W - 1][8];
  for (int64_t t = t0; t < t1; ++t) {
    float acc[8], cur[8];
    ld8<T>(x + t * ch + c0, cur);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = wv[0][e] * cur[e];
#pragma unroll
    for (int j = 1; j < W; ++j) {
      const int64_t r = sa[(t - t0) * (W - 1) + j - 1];
      if (r < 0) continue;
      float v[8];
      if (r == t - j && t - j >= t0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = hist[j - 1][e];
      } else {
        ld8<T>(x + r * ch + c0, v);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wv[j][e] * v[e];
    }
    st8<T>(out + t * ch + c0, acc);
#pragma unroll
    for (int j = W - 2; j > 0; --j)
#pragma unroll
      for (int e = 0; e < 8; ++e) hist[j][e] = hist[j - 1][e];
#pragma unroll
    for (int e = 0; e < 8; ++e) hist[0][e] = cur[e];
  }
}

template <typename T, int W>
__global__ __launch_bounds__(256) void conv_dx_kernel(const T* __restrict__ dout, const float* __restrict__ wt,
                                                      const int64_t* __restrict__ goff, const int64_t* __restrict__ gl,
                                                      int64_t C, int32_t ch, T* __restrict__ dx) {
  constexpr int KG = 4 * kConvRows;  // gather entries staged per block (the rest read from memory)
  const int c0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  float wv[W][8];
  conv_weights<T, W>(wt, c0 < ch ? c0 : 0, wv);
  const int64_t s0 = int64_t(blockIdx.y) * kConvRows, s1 = s0 + kConvRows < C ? s0 + kConvRows : C;
  __shared__ int64_t so[kConvRows + 1], sg[KG];
  for (int i = threadIdx.x; i <= int(s1 - s0); i += 256) so[i] = goff[s0 + i];
  __syncthreads();
  const int64_t g0 = so[0], ng = so[s1 - s0] - g0;
  for (int i = threadIdx.x; i < (ng < KG ? ng : KG); i += 256) sg[i] = gl[g0 + i];
  __syncthreads();
  if (c0 >= ch) return;
  // rows in reverse; next[j - 1]: this thread's channels of dout[s + j], read in an earlier
  // iteration (most gather entries of a row are the rows just after it)
  float next[W - 1][8];
  for (int64_t s = s1 - 1; s >= s0; --s) {
    float acc[8], cur[8], v[8];
    ld8<T>(dout + s * ch + c0, cur);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = wv[0][e] * cur[e];
    // Inside a branch the list is exactly (s + 1, 1) .. (s + W - 1, W - 1), rows this thread
    // already holds: the window's weights then apply at fixed places.  Rows near a fork, a leaf
    // end or the block's end take the general walk.  The test is the same for the block's threads.
    const int64_t ia = so[s - s0], ib = so[s - s0 + 1];
    bool inner = ib - ia == W - 1 && s + W - 1 < s1;
#pragma unroll
    for (int q = 1; q < W; ++q) {
      const int64_t i = ia + q - 1;
      const int64_t ge = !inner ? -1 : i - g0 < KG ? sg[i - g0] : gl[i];
      inner = inner && ge == (((s + q) << 3) | q);
    }
    if (inner) {
#pragma unroll
      for (int q = 1; q < W; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += wv[q][e] * next[q - 1][e];
    } else for (int64_t i = ia; i < ib; ++i) {
      const int64_t ge = i - g0 < KG ? sg[i - g0] : gl[i];
      const int64_t t = ge >> 3;
      const int j = int(ge & 7);
      const int64_t k = t - s;  // in 1 .. W - 1 when t is one of the rows held
      bool held = false;
#pragma unroll
      for (int q = 1; q < W; ++q)
        if (k == q && s + q < s1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = next[q - 1][e];
          held = true;
        }
      if (!held) ld8<T>(dout + t * ch + c0, v);
      float wj[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        wj[e] = wv[1][e];
#pragma unroll
        for (int q = 2; q < W; ++q) wj[e] = j == q ? wv[q][e] : wj[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += wj[e] * v[e];
    }
    st8<T>(dx + s * ch + c0, acc);
#pragma unroll
    for (int q = W - 2; q > 0; --q)
#pragma unroll
      for (int e = 0; e < 8; ++e) next[q][e] = next[q - 1][e];
#pragma unroll
    for (int e = 0; e < 8; ++e) next[0][e] = cur[e];
  }
}

// partial[b][c][j] = sum over rows t of block b of dout[t, c] x[anc_j(t), c]; grid (channel
// pieces / 256, row blocks)
template <typename T, int W>
__global__ __launch_bounds__(256) void conv_dw_partial_kernel(const T* __restrict__ x, const T* __restrict__ dout,
                                                              const int32_t* __restrict__ anc, int64_t C, int32_t ch,
                                                              float* __restrict__ part) {
  const int c0 = (blockIdx.x * 256 + threadIdx.x) * 8;
  const int64_t t0 = int64_t(blockIdx.y) * kConvRowBlock, t1 = t0 + kConvRowBlock < C ? t0 + kConvRowBlock : C;
  __shared__ int32_t sa[kConvRowBlock * (W - 1)];
  for (int i = threadIdx.x; i < int(t1 - t0) * (W - 1); i += 256) sa[i] = anc[t0 * (W - 1) + i];
  __syncthreads();
  if (c0 >= ch) return;
  float acc[W][8];
#pragma unroll
  for (int j = 0; j < W; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;
  float hist[W - 1][8];  // x of rows t - j read in earlier iterations (as in the forward)
  for (int64_t t = t0; t < t1; ++t) {
    float g[8], cur[8];
    ld8<T>(dout + t * ch + c0, g);
    ld8<T>(x + t * ch + c0, cur);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[0][e] += g[e] * cur[e];
#pragma unroll
    for (int j = 1; j < W; ++j) {
      const int64_t r = sa[(t - t0) * (W - 1) + j - 1];
      if (r < 0) continue;
      float v[8];
      if (r == t - j && t - j >= t0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = hist[j - 1][e];
      } else {
        ld8<T>(x + r * ch + c0, v);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] += g[e] * v[e];
    }
#pragma unroll
    for (int j = W - 2; j > 0; --j)
#pragma unroll
      for (int e = 0; e < 8; ++e) hist[j][e] = hist[j - 1][e];
#pragma unroll
    for (int e = 0; e < 8; ++e) hist[0][e] = cur[e];
  }
  float* pb = part + (size_t(blockIdx.y) * ch + c0) * W;
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int j = 0; j < W; ++j) pb[e * W + j] = acc[j][e];
}

// dweight[i] = sum over the row blocks b of part[b][i]: 32 outputs per workgroup, eight phases
// of blocks (b = ph, ph + 8, ..) summed in order each, then the phases in order
__global__ __launch_bounds__(256) void conv_dw_sum_kernel(const float* __restrict__ part, int64_t nblk, int64_t n,
                                                          float* __restrict__ dw) {
  const int l = threadIdx.x & 31, ph = threadIdx.x >> 5;
  const int64_t i = blockIdx.x * int64_t(32) + l;
  float s = 0.f;
  if (i < n)
    for (int64_t b = ph; b < nblk; b += 8) s += part[b * n + i];
  __shared__ float red[8][32];
  red[ph][l] = s;
  __syncthreads();
  if (ph == 0 && i < n) {
    float t = red[0][l];
#pragma unroll
    for (int q = 1; q < 8; ++q) t += red[q][l];
    dw[i] = t;
  }
}

size_t conv_workspace_bytes(int64_t C, int32_t ch, int32_t w) {
  const int64_t nblk = (C + kConvRowBlock - 1) / kConvRowBlock;
  return size_t(nblk > 0 ? nblk : 1) * size_t(ch) * size_t(w) * 4;
}

static dim3 conv_grid(int64_t C, int32_t ch) {
  return dim3(unsigned((ch / 8 + 255) / 256), unsigned((C + kConvRows - 1) / kConvRows));
}

template <typename T, int W>
static hipError_t conv_fwd_t(const void* x, const float* wt, const int32_t* anc, int64_t C, int32_t ch, void* out,
                             hipStream_t s) {
  hipLaunchKernelGGL((conv_fwd_kernel<T, W>), conv_grid(C, ch), dim3(256), 0, s, static_cast<const T*>(x),
                     wt, anc, C, ch, static_cast<T*>(out));
  return hipGetLastError();
}

template <typename T, int W>
static hipError_t conv_bwd_t(const void* x, const float* wt, const int32_t* anc, const int64_t* goff, const int64_t* gl,
                             const void* dout, int64_t C, int32_t ch, void* dx, float* dw, float* part, hipStream_t s) {
  if (dx)
    hipLaunchKernelGGL((conv_dx_kernel<T, W>), conv_grid(C, ch), dim3(256), 0, s,
                       static_cast<const T*>(dout), wt, goff, gl, C, ch, static_cast<T*>(dx));
  if (dw) {
    const int64_t nblk = (C + kConvRowBlock - 1) / kConvRowBlock;
    hipLaunchKernelGGL((conv_dw_partial_kernel<T, W>), dim3(unsigned((ch / 8 + 255) / 256), unsigned(nblk)), dim3(256), 0,
                       s, static_cast<const T*>(x), static_cast<const T*>(dout), anc, C, ch, part);
    const int64_t n = int64_t(ch) * W;
    hipLaunchKernelGGL(conv_dw_sum_kernel, dim3(unsigned((n + 31) / 32)), dim3(256), 0, s, part, nblk, n, dw);
  }
  return hipGetLastError();
}

#define HARTS_CONV_W(X) X(2) X(3) X(4) X(5) X(6) X(7) X(8)

hipError_t launch_conv_fwd(const void* x, const float* wt, const int32_t* anc, int64_t C, int32_t ch, int32_t w,
                           int dtype, void* out, hipStream_t s) {
  if (C <= 0) return hipSuccess;
#define X(W_)                                                                                   \
  if (w == W_) return dtype == 0 ? conv_fwd_t<bf16, W_>(x, wt, anc, C, ch, out, s)             \
                                 : conv_fwd_t<float, W_>(x, wt, anc, C, ch, out, s);
  HARTS_CONV_W(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t launch_conv_bwd(const void* x, const float* wt, const int32_t* anc, const int64_t* goff, const int64_t* gl,
                           const void* dout, int64_t C, int32_t ch, int32_t w, int dtype, void* dx, float* dw,
                           float* part, hipStream_t s) {
  if (C <= 0) return hipSuccess;
#define X(W_)                                                                                        \
  if (w == W_) return dtype == 0 ? conv_bwd_t<bf16, W_>(x, wt, anc, goff, gl, dout, C, ch, dx, dw, part, s) \
                                 : conv_bwd_t<float, W_>(x, wt, anc, goff, gl, dout, C, ch, dx, dw, part, s);
  HARTS_CONV_W(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace harts
