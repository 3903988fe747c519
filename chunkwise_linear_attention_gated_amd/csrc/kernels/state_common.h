// Pieces shared by the serial state pass and the serial state-gradient pass.
#pragma once
#include "common.h"

namespace harts {

// Tiling of one (sequence, head, value-column tile) workgroup over its SNW waves.
template <int BT, int D, int DVT>
struct StateTiles {
  static constexpr int NW = state_waves<D>(), NTV = DVT / 16, MT = D / 16, NB = BT / 16;
  static constexpr int MU = (MT + NW - 1) / NW;  // state row tiles per wave
  static constexpr int WPB = NW / NB;            // waves per 16-token block (U, Y and output tiles)
  static constexpr int NTU = NTV / WPB;          // value-column tiles per wave in those
  static_assert(NW % NB == 0 && NTV % WPB == 0, "token-block tiles split evenly over the waves");
};

// S^T (value-major, [DV][D]) and S (channel-major, [D][DV]) of one value-column tile, both
// fragment-major, from the tile's S^T staged in LDS ([DVT][lds]).
template <typename T, int D, int DV, int DVT, int NTH>
__device__ __forceinline__ void store_state_fm(T* sT, T* s, const T* St, int lds, int jvb, int tid) {
  constexpr int LE = fm_le<T>(), KS = Mma<T>::KS;
  // S^T: rows jv (this tile's), contraction c
  HARTS_STRIDED(p, tid, DVT * D / LE, NTH) {
    const int f = p / 64, l = p % 64;
    const int r = (f / (D / KS)) * 16 + (l & 15), k0 = (f % (D / KS)) * KS + LE * (l >> 4);
    T* dst = sT + fm_off<T>(jvb + r, k0, D);
    if constexpr (LE == 8) copy16(dst, St + r * lds + k0);
    else
#pragma unroll
      for (int t = 0; t < LE; ++t) dst[t] = St[r * lds + k0 + t];
  }
  // S: rows c, contraction jv (this tile's KS-blocks of it)
  HARTS_STRIDED(p, tid, D * DVT / LE, NTH) {
    const int f = p / 64, l = p % 64;
    const int rt = f / (DVT / KS), kt = f % (DVT / KS);
    const int c = rt * 16 + (l & 15), j0 = kt * KS + LE * (l >> 4);
    float v[LE];
#pragma unroll
    for (int t = 0; t < LE; ++t) v[t] = to_f(St[(j0 + t) * lds + c]);
    T* dst = s + fm_off<T>(c, jvb + j0, DV);
    if constexpr (LE == 8) stq(dst, pack16<T>(v));
    else
#pragma unroll
      for (int t = 0; t < LE; ++t) dst[t] = from_f<T>(v[t]);
  }
}

}  // namespace harts
