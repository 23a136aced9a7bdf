// Matrix-core main loop shared by the dense, expert and LM-head kernels.
//
// Computes, for one wave, MT x NS output tiles of 16x16: acc[mt][ns] +=
// A[rows of m-tile mt] . W[rows of n-tile ns]^T over nk k-chunks of 64 bytes.
// Both operands are row-major with the reduction dimension contiguous (weights
// are [out, in], activations [rows, in]), so every lane issues 16-byte loads:
// lane l reads row (l % 16) of each tile at byte offset 16 * (l / 16) of each
// 64-byte chunk.  The caller passes per-lane row pointers that already include
// that lane offset.  Loads for chunk k+1 are issued before the MFMAs of chunk k
// (register double buffering).  m-tiles at index >= mt_active are skipped.
#pragma once
#include "dg_common.h"

template <typename T, int MT, int NS>
__device__ __forceinline__ void mma_loop(const char* (&ap)[MT], const char* (&wp)[NS], int nk, int mt_active,
                                         v4f (&acc)[MT][NS]) {
  typedef typename MF<T>::frag F;
  F a0[MT], a1[MT], w0[NS], w1[NS];
#pragma unroll
  for (int ns = 0; ns < NS; ++ns) w0[ns] = load_frag<F>(wp[ns]);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    if (mt < mt_active) a0[mt] = load_frag<F>(ap[mt]);
  int ks = 0;
  for (; ks + 1 < nk; ks += 2) {
    const int o1 = (ks + 1) * 64;
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) w1[ns] = load_frag<F>(wp[ns] + o1);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      if (mt < mt_active) a1[mt] = load_frag<F>(ap[mt] + o1);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      if (mt < mt_active) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) MF<T>::mma(acc[mt][ns], a0[mt], w0[ns]);
      }
    if (ks + 2 < nk) {
      const int o2 = (ks + 2) * 64;
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) w0[ns] = load_frag<F>(wp[ns] + o2);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (mt < mt_active) a0[mt] = load_frag<F>(ap[mt] + o2);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      if (mt < mt_active) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) MF<T>::mma(acc[mt][ns], a1[mt], w1[ns]);
      }
  }
  if (ks < nk) {  // odd number of chunks: the last one is in a0/w0
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      if (mt < mt_active) {
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) MF<T>::mma(acc[mt][ns], a0[mt], w0[ns]);
      }
  }
}

template <int MT, int NS>
__device__ __forceinline__ void zero_acc(v4f (&acc)[MT][NS]) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) acc[mt][ns] = v4f{0.f, 0.f, 0.f, 0.f};
}
