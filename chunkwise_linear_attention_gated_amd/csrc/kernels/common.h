// Device helpers for gfx950 (CDNA4): MFMA fragment loads and tile layouts.
//
// Matrix-core layouts (16x16 output tiles, 64-lane wavefront):
//   bf16: v_mfma_f32_16x16x32_bf16 -- lane l holds A[l%16][8*(l/16) .. +8) and
//         B[8*(l/16) .. +8)[l%16]; K step 32.
//   fp32: v_mfma_f32_16x16x4f32    -- lane l holds A[l%16][l/16] and
//         B[l/16][l%16]; K step 4.
//   Both: lane l holds C[4*(l/16) + r][l%16], r = 0..3.
//
// An operand is read either from a matrix whose K dimension is contiguous
// (one 16-byte read per bf16 fragment) or from one stored K-major (the
// fragment is gathered element by element).  The same helpers serve LDS and
// global memory.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace harts {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

// transposing LDS read of four 16-bit values (gfx950 ds_read_b64_tr_b16); p is an LDS
// address, 8-byte aligned
__device__ __forceinline__ bf16x4 ds_tr16(const void* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) const char*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

template <typename T> struct Mma;

template <> struct Mma<bf16> {
  static constexpr int KS = 32;
  using Frag = bf16x8;
  // element (r, k) at p[r * ld + k]: K contiguous
  __device__ static __forceinline__ Frag kc(const bf16* p, int ld, int r0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8*>(p + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
  }
  // element (r, k) at p[k * ld + r], p in LDS, ld and r0 multiples of 4: two transposing
  // reads (in each 16-lane group, result element j of lane s is element s % 4 of the four
  // that lane 4 j + s / 4 points at), each lane pointing at 4 consecutive r of one k
  __device__ static __forceinline__ Frag rc(const bf16* p, int ld, int r0, int k0, int lane) {
    const int s = lane & 15;
    const bf16* q = p + (k0 + 8 * (lane >> 4) + (s >> 2)) * ld + r0 + 4 * (s & 3);
    const bf16x4 lo = ds_tr16(q), hi = ds_tr16(q + 4 * ld);
    return Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ static __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int KS = 4;
  using Frag = float;
  __device__ static __forceinline__ Frag kc(const float* p, int ld, int r0, int k0, int lane) {
    return p[(r0 + (lane & 15)) * ld + k0 + (lane >> 4)];
  }
  __device__ static __forceinline__ Frag rc(const float* p, int ld, int r0, int k0, int lane) {
    return p[(k0 + (lane >> 4)) * ld + r0 + (lane & 15)];
  }
  __device__ static __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// C-layout coordinates of accumulator element r for this lane
__device__ __forceinline__ int crow(int lane, int r) { return 4 * (lane >> 4) + r; }
__device__ __forceinline__ int ccol(int lane) { return lane & 15; }

// Store 4 consecutive values (the 4 accumulator rows of one lane) at p[0..3].
template <typename T> __device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}
template <> __device__ __forceinline__ void store4<bf16>(bf16* p, float a, float b, float c, float d) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)a, (bf16)b, (bf16)c, (bf16)d};
}
template <typename T> __device__ __forceinline__ void load4(const T* p, float* v) {
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = to_f(p[r]);
}

// 16-byte vector of T (8 bf16 or 4 fp32) converted to floats
template <typename T> struct Vec16 {
  static constexpr int N = 16 / sizeof(T);
};

template <typename T> __device__ __forceinline__ void ld16(const T* p, float* out) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int t = 0; t < 8; ++t) out[t] = (float)v[t];
  } else {
    f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int t = 0; t < 4; ++t) out[t] = v[t];
  }
}
template <typename T> __device__ __forceinline__ void st16(T* p, const float* in) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 v;
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = (bf16)in[t];
    *reinterpret_cast<bf16x8*>(p) = v;
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{in[0], in[1], in[2], in[3]};
  }
}
template <typename T> __device__ __forceinline__ void copy16(T* dst, const T* src) {
  *reinterpret_cast<f32x4*>(dst) = *reinterpret_cast<const f32x4*>(src);
}

// 16 bytes of T held in a register quad (8 bf16 or 4 fp32), converted to and from floats
template <typename T> __device__ __forceinline__ void unpack16(f32x4 v, float* out) {
  if constexpr (sizeof(T) == 2) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, v);
#pragma unroll
    for (int t = 0; t < 8; ++t) out[t] = (float)b[t];
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) out[t] = v[t];
  }
}
template <typename T> __device__ __forceinline__ f32x4 pack16(const float* in) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 b;
#pragma unroll
    for (int t = 0; t < 8; ++t) b[t] = (bf16)in[t];
    return __builtin_bit_cast(f32x4, b);
  } else {
    return f32x4{in[0], in[1], in[2], in[3]};
  }
}
__device__ __forceinline__ f32x4 ldq(const void* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ void stq(void* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// fp32 16x16 product step with a permuted contraction index: at step s lane l
// supplies A[l%16][4*(l/16) + s] and B[4*(l/16) + s][l%16].  Over s = 0..3 every
// k in 0..15 is covered once, the A values of a lane are 4 consecutive row
// elements (one 16-byte read) and the B values of a lane are exactly the C
// layout of an earlier product, so results chain without leaving registers.
__device__ __forceinline__ f32x4 mma16_f32(f32x4 a, f32x4 b, f32x4 c) {
#pragma unroll
  for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
  return c;
}

// for (var = start; var < n; var += step) with a compile-time trip count, fully
// unrolled: inside the persistent kernels a runtime-bounded loop makes the compiler
// drain every outstanding load (the fetch-ahead included) before entering it.
#define HARTS_STRIDED(var, start, n, step)                                              \
  _Pragma("unroll") for (int var##_u = 0; var##_u < ((n) + (step) - 1) / (step); ++var##_u) \
    if (const int var = (start) + (step) * var##_u; var < (n))

// Item order of a persistent per-chunk kernel.  Workgroup b takes items b and b + G (G = grid
// size) statically, then items 2G + t for tickets t drawn from a per-launch counter that starts
// at zero.  Thread 0 draws a ticket at the top of each item, before that item's fetches, and
// publishes it through one LDS word just before one of the item's early barriers; the workgroup
// reads it after that barrier and fetches the rows of the ticket's item, which it processes two
// items later.  A workgroup that starts late (its compute unit was busy with another kernel)
// simply draws fewer tickets.  Each workgroup's draws increase, so once its item is past the
// end so are all its later draws, and every ticket below the end is processed by the workgroup
// that drew it.

// A zero the compiler cannot see through.  Loads of per-chunk descriptor fields are
// indexed with it so their values stay per-lane: a value the compiler knows to be
// uniform is moved to a scalar register right where it is loaded, which waits for
// that load (and, counters being in order, for every fetch issued before it).
__device__ __forceinline__ int lane_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// One lane draws.  The counter's address goes through lane_zero(): for an address it knows to
// be uniform the compiler rewrites the atomic for the whole wave and reads the returned value
// at once, which waits for every fetch issued before it; here the ticket is read only where it
// is consumed, a phase or two later.
__device__ __forceinline__ int draw_ticket(int* ctr) { return atomicAdd(ctr + lane_zero(), 1); }

// ---- workspace layouts read by the matrix cores -------------------------------------------
// Fragment-major ("FM") layout of an [R][K] matrix used as a matrix-core operand with rows R
// (the A operand's m or the B operand's n) and contraction K: every 16 x KS block is stored
// as the 64 lanes' register contents, lane after lane, so loading an operand fragment is one
// contiguous read per wavefront.  Lane l holds row l%16, contraction indices
// LE*(l/16) .. LE*(l/16) + LE - 1 of its block, LE = KS/4.
template <typename T> __host__ __device__ constexpr int fm_le() { return Mma<T>::KS / 4; }
template <typename T> __device__ __forceinline__ size_t fm_off(int r, int k, int K) {
  constexpr int KS = Mma<T>::KS, LE = KS / 4;
  return ((size_t(r >> 4) * (K / KS) + k / KS) * 64 + (r & 15) + 16 * ((k % KS) / LE)) * LE + (k % LE);
}
template <typename T>
__device__ __forceinline__ typename Mma<T>::Frag fm_frag(const T* p, int K, int rt, int kt, int lane) {
  constexpr int KS = Mma<T>::KS, LE = KS / 4;
  const T* q = p + ((size_t(rt) * (K / KS) + kt) * 64 + lane) * LE;
  if constexpr (sizeof(T) == 2) return *reinterpret_cast<const bf16x8*>(q);
  else return *q;
}
// store n consecutive contraction entries k0 .. k0+n-1 of row r (n = 4 or 16/sizeof(T))
template <typename T> __device__ __forceinline__ void fm_store(T* p, int K, int r, int k0, const float* v, int n) {
  constexpr int LE = fm_le<T>();
  if (LE >= 4 && n <= LE) {  // the n entries are contiguous in one lane's run
    if (n == 8) stq(p + fm_off<T>(r, k0, K), pack16<T>(v));
    else store4(p + fm_off<T>(r, k0, K), v[0], v[1], v[2], v[3]);
  } else {
    for (int t = 0; t < n; ++t) p[fm_off<T>(r, k0 + t, K)] = from_f<T>(v[t]);
  }
}
// Accumulator-major ("CM") layout of an [R][C] matrix of 16 x 16 result tiles: tile after
// tile, each as the 64 lanes' four accumulator values (rows 4(l/16)..+3 of column l%16).
__device__ __forceinline__ size_t cm_off(int r, int c, int C) {
  return ((size_t(r >> 4) * (C / 16) + (c >> 4)) * 64 + (c & 15) + 16 * ((r & 15) >> 2)) * 4 + (r & 3);
}

// Permuted fragment-major ("PF") layout of a bf16 [R][K] matrix-core operand (K a multiple
// of 32).  Every 16 x 32 block is stored as the 64 lanes' 16-byte operand registers, lane
// after lane (1 KiB per block, blocks row-tile-major).  Lane l holds row l%16 and the
// contraction indices 4(l/16) + {0..3} and 16 + 4(l/16) + {0..3} of its block.  Those are
// exactly the rows at which a lane holds the accumulators of two stacked 16 x 16 result
// tiles, so a pair of result tiles is, converted in registers, the other operand of the next
// product over that contraction; the matrix core sums over the contraction in any order as
// long as both operands use the same one.
__host__ __device__ constexpr size_t pf_off(int r, int k, int K) {
  return ((size_t(r >> 4) * (K >> 5) + (k >> 5)) * 64 + (((k & 15) >> 2) << 4) + (r & 15)) * 8 +
         (((k >> 4) & 1) << 2) + (k & 3);
}
// The 8 contraction indices lane-group gq (= lane/16) holds in a PF block, slot order.
__host__ __device__ constexpr int pf_k(int gq, int s) { return s < 4 ? 4 * gq + s : 16 + 4 * gq + (s - 4); }
// Operand fragment from a pair of accumulator tiles (rows 0-15 and 16-31 of a contraction block).
__device__ __forceinline__ bf16x8 pf_pair(f32x4 lo, f32x4 hi) {
  return bf16x8{(bf16)lo[0], (bf16)lo[1], (bf16)lo[2], (bf16)lo[3], (bf16)hi[0], (bf16)hi[1], (bf16)hi[2], (bf16)hi[3]};
}

// A-operand fragment of an [R][K] bf16 matrix with K contiguous (row stride ld), in the PF
// contraction order: rows r0 + l%16, contraction k0 + pf_k(l/16, 0..7).
__device__ __forceinline__ bf16x8 pf_kc(const bf16* p, int ld, int r0, int k0, int lane) {
  const bf16* q = p + (r0 + (lane & 15)) * ld + k0 + 4 * (lane >> 4);
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(q), hi = *reinterpret_cast<const bf16x4*>(q + 16);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// 4 x 4 transpose across each group of 4 consecutive lanes (DPP quad permutes): lane q of a
// group holds x[r] = M[r][q] on entry and M[q][r] on return.
__device__ __forceinline__ float dpp_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ f32x4 quad_transpose(f32x4 x, int lane) {
  const bool lo = (lane & 2) == 0, ev = (lane & 1) == 0;
  float r0 = dpp_xor2(lo ? x[2] : x[0]), r1 = dpp_xor2(lo ? x[3] : x[1]);
  const f32x4 y = lo ? f32x4{x[0], x[1], r0, r1} : f32x4{r0, r1, x[2], x[3]};
  r0 = dpp_xor1(ev ? y[1] : y[0]);
  r1 = dpp_xor1(ev ? y[3] : y[2]);
  return ev ? f32x4{y[0], r0, y[2], r1} : f32x4{r0, y[1], r1, y[3]};
}

// Column slice of a row-major LDS tile in the accumulator layout: lane l reads column
// c0 + l % 16, rows r0 + 4 (l / 16) + t, t = 0..3 (ld and c0 multiples of 4, bf16 tiles 8-byte
// aligned); bf16 by one transposing read.
template <typename T>
__device__ __forceinline__ void col4_load(const T* p, int ld, int r0, int c0, int lane, float (&v)[4]) {
  if constexpr (sizeof(T) == 2) {
    const int q = lane & 15;
    const bf16x4 x = ds_tr16(p + (r0 + 4 * (lane >> 4) + (q >> 2)) * ld + c0 + 4 * (q & 3));
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = (float)x[t];
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t) v[t] = p[(r0 + 4 * (lane >> 4) + t) * ld + c0 + (lane & 15)];
  }
}
// Elements of T in the store sink (RoundArgs::sink, 64 KiB)
template <typename T> __host__ __device__ constexpr int kSinkElems() { return 64 * 1024 / sizeof(T); }

// In-chunk decay products e^{L_i - L_j} inside a 16-token block factor as e^{L_i} e^{-L_j} (L the
// block-local cumulative log-decay) only for channels whose block gate sum is at least
// -kSteepGate: then no factor exceeds e^{kSteepGate}, far inside fp32 and bf16 range, and none
// underflows to a subnormal for unit-scale keys.  Steeper channels take the pairwise form.
constexpr float kSteepGate = 60.f;

// Waves of a serial state-pass workgroup: one per 16 state rows, at most 8.
template <int D> constexpr int state_waves() { return D / 16 < 8 ? D / 16 : 8; }

// Workgroup size of the persistent preparation kernel: 16 waves, four per SIMD (at most 128
// registers each).  One workgroup fills a compute unit (its LDS), so the waves of one item are
// all the latency hiding there is: at 8 waves the kernel took 8-17 % longer.
constexpr int CNT = 1024;
constexpr int CNW = CNT / 64;

// Blocks of a grid are dealt round-robin to the 8 XCDs; remap so that runs of
// consecutive logical ids (e.g. the value-column tiles of one sequence-head,
// which read the same per-chunk operands) land on one XCD and share its L2.
__device__ __forceinline__ int xcd_logical(int b, int nblocks) {
  if (nblocks % 8) return b;
  return (b % 8) * (nblocks / 8) + b / 8;
}

}  // namespace harts
