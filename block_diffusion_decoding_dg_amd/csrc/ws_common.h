// Device helpers shared by the weight-streaming GEMM kernels (k_ws, k_wsd): the
// weight rows of an n-block per epilogue and the epilogue of one 16-row m-tile.
#pragma once
#include "dg_common.h"
#include "dg_kernels.h"

// Eight E4M3 codes (little-endian bytes, in reduction order) widened to eight
// bf16 values: exact, since an E4M3 value has a 4-bit significand and an
// exponent inside bf16's range.  The conversion reads the OCP E4M3 encoding.
__device__ __forceinline__ uint4 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                    __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
}

// Eight MXFP4 (E2M1) codes, two per byte with the lower reduction index in the
// low nibble, widened to bf16 and multiplied by their block's E8M0 scale
// 2^(sb - 127), passed to the conversion as the float with that exponent field.
// A two-bit significand times a power of two: exact for scale bytes 1 .. 252
// (a GPU check over every code byte and byte select matched the exact value
// rounded to bf16, subnormals included, at scale bytes 1, 2, 120, 127 and 252;
// from 253 the largest codes overflow bf16; byte 0 reads as a zero scale and
// 255 as infinity).
__device__ __forceinline__ uint4 mxfp4x8_to_bf16(uint32_t codes, uint32_t sb) {
  const float sc = __uint_as_float(sb << 23);
  const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0);
  const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1);
  const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2);
  const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3);
  return make_uint4(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                    __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3));
}

// Weight row `r` (0 .. BN-1) of n-block nb of group g, per epilogue, as a byte
// address; EB = bits per weight (16: bf16, 8: E4M3 codes, 4: MXFP4 codes).
template <int EPI, int NTN, int EB = 16>
__device__ __forceinline__ const char* weight_row(const WsArgs& a, int g, int nb, int r) {
  if constexpr (EPI == WS_EPI_SWIGLU) {
    // rows 0 .. 8 NTN - 1: W1 rows, rows 8 NTN .. 16 NTN - 1: W3 rows, of the same
    // 8 NTN hidden columns
    constexpr int HALF = 8 * NTN;
    const char* W = (const char*)(r < HALF ? a.W0 : a.W1) + (size_t)g * a.wgs * EB / 8;
    const int n = nb * HALF + (r % HALF);
    return W + (size_t)min(n, a.N - 1) * a.K * EB / 8;
  } else if constexpr (EPI == WS_EPI_ROPE_QKV) {
    // rows 0..31: columns j0 .. j0+31 of one head's first half, rows 32..63: the
    // matching columns of its second half (RoPE pairs j, j + hd/2)
    const int half = a.hd / 2, per_head = half / 32;
    const int head = nb / per_head, j = (nb - head * per_head) * 32 + (r & 31) + (r < 32 ? 0 : half);
    const bf16_t* W;
    int hl;
    if (head < a.hq) { W = (const bf16_t*)a.W0; hl = head; }
    else if (head < a.hq + a.hkv) { W = (const bf16_t*)a.W1; hl = head - a.hq; }
    else { W = (const bf16_t*)a.W2; hl = head - a.hq - a.hkv; }
    return (const char*)(W + (size_t)(hl * a.hd + j) * a.K);
  } else {
    const char* W = (const char*)a.W0 + (size_t)g * a.wgs * EB / 8;
    const int n = nb * (16 * NTN) + r;
    return W + (size_t)min(n, a.N - 1) * a.K * EB / 8;
  }
}

// E8M0 block scales (K / 32 bytes per weight row) of the MXFP4 weight row that
// weight_row names, for the grouped epilogues.
template <int EPI, int NTN>
__device__ __forceinline__ const uint8_t* scale_row(const WsArgs& a, int g, int nb, int r) {
  static_assert(EPI == WS_EPI_SWIGLU || EPI == WS_EPI_STORE_F32, "MXFP4 weights: routed experts only");
  if constexpr (EPI == WS_EPI_SWIGLU) {
    constexpr int HALF = 8 * NTN;
    const int n = nb * HALF + (r % HALF);
    return (r < HALF ? a.wbs0 : a.wbs1) + (size_t)g * (a.wgs / 32) + (size_t)min(n, a.N - 1) * (a.K / 32);
  } else {
    const int n = nb * (16 * NTN) + r;
    return a.wbs0 + (size_t)g * (a.wgs / 32) + (size_t)min(n, a.N - 1) * (a.K / 32);
  }
}

__device__ __forceinline__ int seg_index(const DgSegs& sg, int r) {
  int s = 0;
  for (int i = 1; i < sg.count; ++i)
    if (r >= sg.s[i].row0) s = i;
  return s;
}

// Epilogue of one 16-row m-tile for every epilogue but the LM head's
// statistics (v_mfma_f32_16x16x32_bf16 result layout): lane holds columns
// nb * BN + n * 16 + lane % 16 (n < NTN, BN = 16 NTN; SwiGLU: W1 columns in the
// first NTN / 2 tiles, the matching W3 columns in the rest; q/k/v: a head's
// RoPE pairs in tiles n and n + 2) of the tile's rows 4 (lane / 16) + i, which
// are rows rl0 + 4 (lane / 16) + i of a part of cnt rows (row row0 + rl of the
// group; rows rl >= cnt are not stored).  g, off, arow0: the group and its
// first positions in perm and in the expert-sorted rows (grouped launches);
// ks: the reduction range of a split add launch.
template <int EPI, int NTN, int WF>
__device__ __forceinline__ void ws_tile_epilogue(const WsArgs& a, const v4f (&acc)[NTN], int g, int nb, int row0,
                                                 int rl0, int cnt, int off, int arow0, int ks, int lane) {
  constexpr int BN = 16 * NTN;
  if constexpr (EPI == WS_EPI_ROPE_QKV) {
    // V into the transposed cache: a lane holds 4 consecutive rows (cache
    // positions) of one column, so when they are valid, of one request
    // and start at a position divisible by 4 the lane writes them as one
    // 8-byte run (4 lanes: 32 contiguous bytes per column); else per row
    const int per_head = a.hd / 64, head = nb / per_head;
    if (head >= a.hq + a.hkv) {
      const int rl4 = rl0 + (lane >> 4) * 4, r0 = row0 + rl4;
      bool run = rl4 + 3 < cnt;
      int si = 0, pos = 0;
      if (run) {
        si = seg_index(a.segs, r0);
        pos = a.segs.s[si].pos0 + (r0 - a.segs.s[si].row0);
        run = seg_index(a.segs, r0 + 3) == si && (pos & 3) == 0;
      }
      if (run) {
        const int half = a.hd / 2, hl = head - a.hq - a.hkv;
        bf16_t* vt = (bf16_t*)a.segs.s[si].vt + (size_t)hl * a.hd * a.max_ctx;
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const int jj = (nb - head * per_head) * 32 + n * 16 + (lane & 15);
          const uint2 lo = make_uint2((uint32_t)f2bf(acc[n][0]) | ((uint32_t)f2bf(acc[n][1]) << 16),
                                      (uint32_t)f2bf(acc[n][2]) | ((uint32_t)f2bf(acc[n][3]) << 16));
          const uint2 hi =
              make_uint2((uint32_t)f2bf(acc[n + 2][0]) | ((uint32_t)f2bf(acc[n + 2][1]) << 16),
                         (uint32_t)f2bf(acc[n + 2][2]) | ((uint32_t)f2bf(acc[n + 2][3]) << 16));
          *(uint2*)(vt + (size_t)jj * a.max_ctx + pos) = lo;
          *(uint2*)(vt + (size_t)(jj + half) * a.max_ctx + pos) = hi;
        }
        return;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = rl0 + (lane >> 4) * 4 + i;
    if (rl >= cnt) continue;
    const int r = row0 + rl;
    if constexpr (EPI == WS_EPI_SWIGLU) {
      // fragment-major output with N columns, at the input's row (the
      // expert-sorted row for a grouped launch)
      const int frow = arow0 + r;
#pragma unroll
      for (int n = 0; n < NTN / 2; ++n) {
        const int col = nb * (8 * NTN) + n * 16 + (lane & 15);
        if (col >= a.N) continue;
        float u = acc[n][i], v = acc[n + NTN / 2][i];
        if constexpr (WF == DG_WS_W_E4M3) {  // row scales of the W1 and W3 codes
          u *= a.wsc0[(size_t)g * a.N + col];
          v *= a.wsc1[(size_t)g * a.N + col];
        }
        ((bf16_t*)a.out)[fm_index(frow, col, a.N)] = f2bf(silu_f(u) * v);
      }
    } else if constexpr (EPI == WS_EPI_ROPE_QKV) {
      const int half = a.hd / 2, per_head = half / 32;
      const int head = nb / per_head;
      const int si = seg_index(a.segs, r);
      const int pos = a.segs.s[si].pos0 + (r - a.segs.s[si].row0);
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int jj = (nb - head * per_head) * 32 + n * 16 + (lane & 15);
        float x1 = acc[n][i], x2 = acc[n + 2][i];
        if (head < a.hq + a.hkv) {
          double ang = (double)pos * a.inv_freq[jj];
          const double two_pi = 6.283185307179586476925286766559;
          ang -= two_pi * rint(ang / two_pi);
          float sn, cs;
          sincosf((float)ang, &sn, &cs);
          const float y1 = x1 * cs - x2 * sn, y2 = x2 * cs + x1 * sn;
          x1 = y1;
          x2 = y2;
        }
        if (head < a.hq) {
          bf16_t* qd = (bf16_t*)a.out + (size_t)r * a.ldo + head * a.hd;
          qd[jj] = f2bf(x1);
          qd[jj + half] = f2bf(x2);
        } else if (head < a.hq + a.hkv) {
          const int hl = head - a.hq;
          bf16_t* k = (bf16_t*)a.segs.s[si].k + ((size_t)hl * a.max_ctx + pos) * a.hd;
          k[jj] = f2bf(x1);
          k[jj + half] = f2bf(x2);
        } else {
          const int hl = head - a.hq - a.hkv;
          bf16_t* vt = (bf16_t*)a.segs.s[si].vt + (size_t)hl * a.hd * a.max_ctx;
          vt[(size_t)jj * a.max_ctx + pos] = f2bf(x1);
          vt[(size_t)(jj + half) * a.max_ctx + pos] = f2bf(x2);
        }
      }
    } else {
      const int orow = a.counts ? a.perm[off + r] : r;
#pragma unroll
      for (int n = 0; n < NTN; ++n) {
        const int col = nb * BN + n * 16 + (lane & 15);
        if (col >= a.N) continue;
        const size_t o = (size_t)orow * a.ldo + col;
        if constexpr (EPI == WS_EPI_STORE_BF16) ((bf16_t*)a.out)[o] = f2bf(acc[n][i]);
        else if constexpr (EPI == WS_EPI_STORE_F32)
          ((float*)a.out)[o] =
              WF == DG_WS_W_E4M3 ? acc[n][i] * a.wsc0[(size_t)g * a.N + col] : acc[n][i];
        else if (a.ksplit > 1) a.part_out[(size_t)ks * a.part_stride + o] = acc[n][i];  // partial sum
        else ((float*)a.out)[o] += acc[n][i];
      }
    }
  }
}
