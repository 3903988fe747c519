// Compact -> semantic log-probabilities on gfx950 (HARTS close-reading blog,
// section 4.4; paperlayer summary, section 3 "Semantic Preservation"): the
// vocabulary-wide max and sum-exp are computed once per compact logit row,
// then every semantic position reads its own target logit in the original
// order, so vocabulary work is O(C V) + O(S), never O(S V).
//
//   row pass:    lse[c] = log sum_v exp(x[c, v])   (one streaming read of each row)
//   gather pass: logp[s] = x[m[s], label[s]] - lse[m[s]];  q[m[s]] += 1
//
// Backward (equation 19 of the same section): for L = sum_s g_s logp[s], each compact row
// takes the sum of its semantic positions' own gradients g_s (onehot(label_s) - softmax(x[c])):
//   dx[c, v] = sum_{s in c, label_s = v} g_s - (sum_{s in c} g_s) softmax(x[c])[v]
// in one streaming read and write of the row; the positions of a row come from the CSR inverse
// of m and are summed in increasing s, so the result does not depend on scheduling.
//
// The row pass is a pure HBM stream: 16-byte loads, eight in flight per
// thread, online max / sum-exp in base 2 (one exp2 per element).
#include <mutex>

#include "common.h"
#include "launch.h"

namespace harts {
namespace {
// 2^x on the hardware instruction alone, for the row log-sum-exp (exponents <= 0 up to
// rounding): terms below 2^-126 of the row maximum come out as 0 rather than denormal, which the
// fp32 row sum could not tell apart.  (The backward keeps the library exp2f: measured faster there.)
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
}  // namespace


constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ void online_add(float& m, float& s, float v2) {
  // v2 is in base-2 units; (m, s) represents s * 2^m
  if (v2 > m) {
    s = s * exp2_hw(m - v2) + 1.f;
    m = v2;
  } else {
    s += exp2_hw(v2 - m);
  }
}

__device__ __forceinline__ void online_merge(float& m, float& s, float m2, float s2) {
  if (m2 > m) {
    s = s * exp2_hw(m - m2) + s2;
    m = m2;
  } else if (s2 > 0.f) {
    s += s2 * exp2_hw(m2 - m);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void row_lse_kernel(const T* __restrict__ x, int64_t V, float* __restrict__ lse,
                                                      bool vec_ok) {
  constexpr int VN = 16 / sizeof(T);
  const int64_t c = blockIdx.x;
  const T* row = x + c * V;
  float m = -INFINITY, s = 0.f;
  const int64_t nvec = vec_ok ? V / VN : 0;
  const f32x4* rv = reinterpret_cast<const f32x4*>(row);
  int64_t i = threadIdx.x;
  // eight 16-byte loads in flight per thread; the maximum is taken on the raw values, so each
  // element costs one fused multiply-add into base 2 and one exp2
  for (; i + 7 * 256 < nvec; i += 8 * 256) {
    f32x4 raw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) raw[u] = __builtin_nontemporal_load(rv + i + u * 256);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float v[VN];
      if constexpr (sizeof(T) == 2) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, raw[u]);
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = (float)b[t];
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = raw[u][t];
      }
      float vm = v[0];
#pragma unroll
      for (int t = 1; t < VN; ++t) vm = fmaxf(vm, v[t]);
      vm *= kLog2e;
      if (vm > m) {
        s *= exp2_hw(m - vm);
        m = vm;
      }
#pragma unroll
      for (int t = 0; t < VN; ++t) s += exp2_hw(fmaf(v[t], kLog2e, -m));
    }
  }
  for (; i < nvec; i += 256) {
    float v[VN];
    ld16(row + i * VN, v);
#pragma unroll
    for (int t = 0; t < VN; ++t) online_add(m, s, v[t] * kLog2e);
  }
  for (int64_t j = nvec * VN + threadIdx.x; j < V; j += 256) online_add(m, s, to_f(row[j]) * kLog2e);
  // wave reduction, then across the 4 waves
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const float s2 = __shfl_xor(s, off, 64);
    online_merge(m, s, m2, s2);
  }
  __shared__ float sm[4], ss[4];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm[wave] = m;
    ss[wave] = s;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = sm[0], Sx = ss[0];
    for (int w = 1; w < 4; ++w) online_merge(M, Sx, sm[w], ss[w]);
    lse[c] = (M + log2f(Sx)) * kLn2;
  }
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; i < n; i += int64_t(gridDim.x) * blockDim.x) p[i] = 0;
}

hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(unsigned((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

// A position whose row is outside [0, C) or whose label is outside [0, V) reads nothing, gets
// NaN and is not counted.
template <typename T>
__global__ __launch_bounds__(256) void gather_kernel(const T* __restrict__ x, int64_t C, int64_t V,
                                                     const int64_t* __restrict__ m, const int32_t* __restrict__ labels,
                                                     int64_t S, const float* __restrict__ lse, float* __restrict__ logp,
                                                     int32_t* __restrict__ q) {
  for (int64_t s = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; s < S; s += int64_t(gridDim.x) * blockDim.x) {
    const int64_t c = m[s];
    const int32_t y = labels[s];
    if (c < 0 || c >= C || y < 0 || y >= V) {
      logp[s] = __builtin_nanf("");
      continue;
    }
    logp[s] = to_f(x[c * V + y]) - lse[c];
    if (q) atomicAdd(q + c, 1);
  }
}

// One workgroup per compact row: the row's positions (label, weight) staged in LDS, their weight
// sum G, a streaming pass writing -G softmax(x[c]), then the label entries rewritten with their
// positions' weights added (a wait for the streamed stores and a barrier order them after).
// Rows with more than KPOS positions read their lists from global memory instead.
constexpr int KPOS = 512;

template <typename T>
__global__ __launch_bounds__(256) void logprob_bwd_kernel(const T* __restrict__ x, int64_t V, const float* __restrict__ lse,
                                                          const int64_t* __restrict__ row_off,
                                                          const int64_t* __restrict__ row_pos,
                                                          const int32_t* __restrict__ labels,
                                                          const float* __restrict__ dlogp, T* __restrict__ dx,
                                                          bool vec_ok) {
  constexpr int VN = 16 / sizeof(T);
  const int64_t c = blockIdx.x;
  const int64_t b = row_off[c], n = row_off[c + 1] - b;
  __shared__ int32_t plab[KPOS];
  __shared__ float pw[KPOS];
  __shared__ float wsum;
  const bool staged = n <= KPOS;
  if (staged)
    for (int64_t t = threadIdx.x; t < n; t += 256) {
      const int64_t s = row_pos[b + t];
      plab[t] = labels[s];
      pw[t] = dlogp[s];
    }
  auto lab_of = [&](int64_t t) { return staged ? plab[t] : labels[row_pos[b + t]]; };
  auto w_of = [&](int64_t t) { return staged ? pw[t] : dlogp[row_pos[b + t]]; };
  __syncthreads();
  if (threadIdx.x == 0) {
    float g = 0.f;
    for (int64_t t = 0; t < n; ++t) g += w_of(t);
    wsum = g;
  }
  __syncthreads();
  const float ng = 0.f - wsum;  // +0 for a row no position reads
  const float l2 = lse[c] * kLog2e;
  const T* row = x + c * V;
  T* out = dx + c * V;
  const int64_t nvec = vec_ok ? V / VN : 0;
  const f32x4* rv = reinterpret_cast<const f32x4*>(row);
  int64_t i = threadIdx.x;
  for (; i + 7 * 256 < nvec; i += 8 * 256) {
    f32x4 raw[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) raw[u] = __builtin_nontemporal_load(rv + i + u * 256);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float v[VN];
      unpack16<T>(raw[u], v);
#pragma unroll
      for (int t = 0; t < VN; ++t) v[t] = ng * exp2f(fmaf(v[t], kLog2e, -l2));
      __builtin_nontemporal_store(pack16<T>(v), reinterpret_cast<f32x4*>(out) + i + u * 256);
    }
  }
  for (; i < nvec; i += 256) {
    float v[VN];
    unpack16<T>(rv[i], v);
#pragma unroll
    for (int t = 0; t < VN; ++t) v[t] = ng * exp2f(v[t] * kLog2e - l2);
    st16<T>(out + i * VN, v);
  }
  for (int64_t j = nvec * VN + threadIdx.x; j < V; j += 256) out[j] = from_f<T>(ng * exp2f(to_f(row[j]) * kLog2e - l2));
  // every streamed store has completed (acknowledged by the L2 that holds its line) before any
  // label entry is rewritten: a plain wait, where a device-scope fence would write the L2 back
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // label entries: the first position of each distinct label in the row writes the sum of the
  // weights of all its positions with that label, in increasing s
  for (int64_t k = threadIdx.x; k < n; k += 256) {
    const int32_t y = lab_of(k);
    if (y < 0 || y >= V) continue;  // a label outside the vocabulary writes nothing
    bool first = true;
    for (int64_t j = 0; j < k && first; ++j) first = lab_of(j) != y;
    if (!first) continue;
    float g = 0.f;
    for (int64_t j = k; j < n; ++j)
      if (lab_of(j) == y) g += w_of(j);
    out[y] = from_f<T>(g + ng * exp2f(to_f(row[y]) * kLog2e - l2));
  }
}

hipError_t launch_logprob_bwd(const void* logits, int64_t C, int64_t V, int dtype, const float* lse,
                              const int64_t* row_off, const int64_t* row_pos, const int32_t* labels, const float* dlogp,
                              void* dlogits, hipStream_t s) {
  if (C <= 0) return hipSuccess;
  const int vn = dtype == 0 ? 8 : 4;
  const bool vec_ok = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) && (reinterpret_cast<uintptr_t>(dlogits) % 16 == 0) &&
                      (V % vn == 0);
  if (dtype == 0)
    hipLaunchKernelGGL(logprob_bwd_kernel<bf16>, dim3(unsigned(C)), dim3(256), 0, s, static_cast<const bf16*>(logits), V,
                       lse, row_off, row_pos, labels, dlogp, static_cast<bf16*>(dlogits), vec_ok);
  else
    hipLaunchKernelGGL(logprob_bwd_kernel<float>, dim3(unsigned(C)), dim3(256), 0, s, static_cast<const float*>(logits),
                       V, lse, row_off, row_pos, labels, dlogp, static_cast<float*>(dlogits), vec_ok);
  return hipGetLastError();
}

hipError_t launch_logprob(const void* logits, int64_t C, int64_t V, int dtype, const int64_t* m, const int32_t* labels,
                          int64_t S, float* logp, int32_t* q, float* lse, hipStream_t s) {
  if (C <= 0) return hipSuccess;
  if (q) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3(unsigned((C + 255) / 256 < 4096 ? (C + 255) / 256 : 4096)), dim3(256), 0, s,
                       q, C);
  }
  // rows are read with 16-byte vectors only when every row start is 16-byte aligned
  const int vn = dtype == 0 ? 8 : 4;
  const bool vec_ok = (reinterpret_cast<uintptr_t>(logits) % 16 == 0) && (V % vn == 0);
  if (dtype == 0)
    hipLaunchKernelGGL(row_lse_kernel<bf16>, dim3(unsigned(C)), dim3(256), 0, s, static_cast<const bf16*>(logits), V, lse,
                       vec_ok);
  else
    hipLaunchKernelGGL(row_lse_kernel<float>, dim3(unsigned(C)), dim3(256), 0, s, static_cast<const float*>(logits), V,
                       lse, vec_ok);
  if (S > 0) {
    const unsigned nb = unsigned((S + 255) / 256 < 8192 ? (S + 255) / 256 : 8192);
    if (dtype == 0)
      hipLaunchKernelGGL(gather_kernel<bf16>, dim3(nb), dim3(256), 0, s, static_cast<const bf16*>(logits), C, V, m,
                         labels, S, lse, logp, q);
    else
      hipLaunchKernelGGL(gather_kernel<float>, dim3(nb), dim3(256), 0, s, static_cast<const float*>(logits), C, V, m,
                         labels, S, lse, logp, q);
  }
  return hipGetLastError();
}


// ---- the gather without allocation: the per-row log-sum-exp in a file-scope device array, one
// copy per GPU, held until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in); it resolves each device's address once, with that
// device current, and passes that.
static __device__ __align__(256) float scratch[kLogprobStaticRows];

namespace {
std::mutex g_scratch_mu;
float* g_scratch_dev[64] = {};
}  // namespace

static hipError_t scratch_for_current_device(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

hipError_t launch_logprob_static(const void* logits, int64_t C, int64_t V, int dtype, const int64_t* m,
                                 const int32_t* labels, int64_t S, float* logp, int32_t* q, hipStream_t s) {
  if (C > kLogprobStaticRows) return hipErrorInvalidValue;
  float* lse = nullptr;
  const hipError_t e = scratch_for_current_device(&lse);
  if (e != hipSuccess) return e;
  return launch_logprob(logits, C, V, dtype, m, labels, S, logp, q, lse, s);
}

}  // namespace harts
