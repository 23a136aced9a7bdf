// Routed-expert projections (bf16 weights) with the weight tiles copied straight
// from HBM into LDS: the same work units, tiles and epilogues as the grouped
// launches of k_ws, with the weight stream moved out of registers.
//
// A block owns 64 weight rows of one expert (an n-block) and one part of that
// expert's rows (at most DG_WS_GROUP_ROWS = 128, one 16-row m-tile per consumer
// wave).  Its ten waves split the work by role:
//   * two producer waves copy each 8 KB weight chunk (64 rows x 64 reduction
//     elements) into an LDS ring of NST stages with global_load_lds_dwordx4 --
//     four copies per wave per chunk, NST - 1 chunks ahead of the consumers --
//     and, since the compiler does not track these copies, wait for them
//     themselves (DG_WAIT_VMCNT) before the chunk's barrier;
//   * eight consumer waves load their m-tile's activation fragments with
//     ordinary loads three chunks ahead (so the compiler's own waits for them
//     stay exact: a consumer issues no copies), read the weight fragments of
//     the chunk from LDS and run the matrix cores.  The activations are the
//     expert-sorted rows in the fragment-major layout (fm_index), gathered once
//     after routing, so each fragment is one contiguous 1 KB load.
// One barrier per chunk, passed by all ten waves: it publishes chunk c (every
// producer has waited for its copies of c) and frees the stage that chunk c - 1
// used (every consumer has read it), which the producers refill at once.  The
// ring holds NST stages, so the bytes in flight per block are (NST - 1) x 8 KB
// instead of the four register slots of k_ws, and no register holds weights.
//
// LDS rows are XOR-swizzled in 16-byte units exactly as in k_ws, so the
// fragment reads are free of bank conflicts; the copies write each stage in
// lane order, and each lane picks the global segment that belongs at its slot.
// Copies of chunks past the end reload the last chunk into a free stage, so
// every iteration issues the same copies and the waits stay constant.
#include "dg_common.h"
#include "dg_kernels.h"

namespace {

constexpr int WSD_NCW = 8;                           // consumer waves (m-tile = wave)
constexpr int WSD_NPW = 2;                           // producer waves
constexpr int WSD_NT = 64 * (WSD_NCW + WSD_NPW);     // 640 threads
constexpr int WSD_BN = 64;                           // weight rows per block
constexpr int WSD_SLOTS = WSD_BN * 8;                // 16-byte LDS slots per stage (8 KB)
constexpr int WSD_INS = WSD_SLOTS / 64 / WSD_NPW;    // copies per producer wave per chunk
static_assert(WSD_NCW * 16 == DG_WS_GROUP_ROWS, "one m-tile per consumer wave covers a part");

// LDS slot of 16-byte segment seg (0..7) of weight row `row` of a stage.
__device__ __forceinline__ int wsd_slot(int row, int seg) { return row * 8 + (seg ^ (row & 7)); }

// Byte address of weight row r (0..63) of n-block nb of expert g.  SwiGLU: rows
// 0..31 are W1 rows and 32..63 the W3 rows of the same 32 hidden columns.
template <int EPI>
__device__ __forceinline__ const char* wsd_row(const WsArgs& a, int g, int nb, int r) {
  if constexpr (EPI == WS_EPI_SWIGLU) {
    const char* W = (const char*)(r < 32 ? a.W0 : a.W1) + (size_t)g * a.wgs * 2;
    const int n = nb * 32 + (r & 31);
    return W + (size_t)min(n, a.N - 1) * a.K * 2;
  } else {
    const char* W = (const char*)a.W0 + (size_t)g * a.wgs * 2;
    const int n = nb * WSD_BN + r;
    return W + (size_t)min(n, a.N - 1) * a.K * 2;
  }
}

// A consumer wave's chunk loop: fragments of chunk c + 3 loaded while chunk c
// is computed (ACT; an idle wave only meets the barriers), one barrier per
// chunk, the weight fragments read from stage c % NST.  The loop body covers
// whole groups of 4 chunks with no branch (so the compiler keeps exact waits
// for the activation loads); the last nk % 4 chunks follow it.
template <bool ACT, int NST>
__device__ __forceinline__ void wsd_consume(uint4 (*sW)[WSD_SLOTS], const char* ap, int nk, int lane, v4f (&acc)[4]) {
  auto fetch_a = [&](v8s (&A)[2], int c) __attribute__((always_inline)) {
    if constexpr (ACT) {
      const int cc = min(c, nk - 1);
#pragma unroll
      for (int q = 0; q < 2; ++q) A[q] = *(const v8s*)(ap + (size_t)(2 * cc + q) * 1024);
    }
  };
  v8s A0[2], A1[2], A2[2], A3[2];
  fetch_a(A0, 0);
  fetch_a(A1, 1);
  fetch_a(A2, 2);
  auto step = [&](v8s (&Acur)[2], v8s (&Anext)[2], int c) __attribute__((always_inline)) {
    fetch_a(Anext, c + 3);
    __builtin_amdgcn_s_barrier();  // chunk c is in its stage
    asm volatile("" ::: "memory");
    if constexpr (ACT) {
      const uint4* st = sW[c % NST];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const v8s am = Acur[q];
        v8s wf[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const uint4 u = st[wsd_slot(n * 16 + (lane & 15), q * 4 + (lane >> 4))];
          wf[n] = *reinterpret_cast<const v8s*>(&u);
        }
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, wf[n], acc[n], 0, 0, 0);
      }
    }
  };
  int c = 0;
  for (; c + 4 <= nk; c += 4) {  // whole groups of 4, branch-free
    step(A0, A3, c);
    step(A1, A0, c + 1);
    step(A2, A1, c + 2);
    step(A3, A2, c + 3);
  }
  if (c < nk) step(A0, A3, c);  // the last nk % 4 chunks
  if (c + 1 < nk) step(A1, A0, c + 1);
  if (c + 2 < nk) step(A2, A1, c + 2);
}

template <int EPI, int NST>
__global__ void __launch_bounds__(WSD_NT) k_wsd(WsArgs a) {
  static_assert(NST >= 3 && (NST - 2) * WSD_INS <= 63, "ring depth within the vmcnt range");
  __shared__ uint4 sW[NST][WSD_SLOTS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if ((int)blockIdx.x >= *a.n_units) return;
  const uint32_t code = (uint32_t)a.units[blockIdx.x];
  if (code == DG_WS_UNIT_NONE) return;  // padding of the work list
  const int g = (int)(code >> 24), part = (int)((code >> 16) & 0xff), nb = (int)(code & 0xffff);
  const int row0 = part * DG_WS_GROUP_ROWS;
  const int cnt = min(a.counts[g] - row0, DG_WS_GROUP_ROWS);
  if (cnt <= 0) return;  // uniform over the block
  const int nk = a.K / 64;

  if (wave >= WSD_NCW) {
    // ---- producer: copies of the weight chunks into the LDS ring
    const int p = wave - WSD_NCW;
    const char* src[WSD_INS];
#pragma unroll
    for (int i = 0; i < WSD_INS; ++i) {
      const int s = (p * WSD_INS + i) * 64 + lane, row = s >> 3, seg = (s & 7) ^ (row & 7);
      src[i] = wsd_row<EPI>(a, g, nb, row) + seg * 16;
    }
    auto issue = [&](int c, int st) __attribute__((always_inline)) {
      const size_t kb = (size_t)min(c, nk - 1) * 128;
#pragma unroll
      for (int i = 0; i < WSD_INS; ++i) lds_dma16(src[i] + kb, &sW[st][(p * WSD_INS + i) * 64]);
    };
    DG_WAIT_VMCNT(0);  // nothing of the compiler's own is outstanding from here on
#pragma unroll
    for (int c = 0; c < NST - 1; ++c) issue(c, c);
    for (int c = 0; c < nk; ++c) {
      DG_WAIT_VMCNT((NST - 2) * WSD_INS);  // this wave's copies of chunk c have landed
      __builtin_amdgcn_s_barrier();        // ... and every wave's; stage (c - 1) % NST is free
      asm volatile("" ::: "memory");
      issue(c + NST - 1, (c + NST - 1) % NST);
    }
    DG_WAIT_VMCNT(0);  // no copy may land after the block has ended
    return;
  }

  // ---- consumer: this wave's m-tile (rows t0 .. t0 + 15 of the part)
  const int t0 = wave * 16;
  const bool act = t0 < cnt;  // uniform over the wave
  const int off = a.offsets[g], arow0 = a.offsets16[g];
  // fragment-major rows (fm_index): one contiguous 1 KB block per 32 elements;
  // a tile past the part's rows reads the last one, which holds valid rows
  const int tr = arow0 + row0 + min(t0, (cnt - 1) & ~15);
  const char* ap = (const char*)a.A + (size_t)(tr >> 4) * (a.K >> 5) * 1024 + lane * 16;
  v4f acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};
  // The active and the idle waves run separate branch-free loops (same
  // barriers): a conditional load inside the loop makes the compiler's wait
  // bookkeeping give up the three-chunk lead of the activation loads.
  if (act) wsd_consume<true, NST>(sW, ap, nk, lane, acc);
  else wsd_consume<false, NST>(sW, ap, nk, lane, acc);
  if (!act) return;

  // ---- epilogue: lane holds columns n * 16 + lane % 16 of rows 4 (lane / 16) + i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = t0 + (lane >> 4) * 4 + i;
    if (rl >= cnt) continue;
    const int r = row0 + rl;
    if constexpr (EPI == WS_EPI_SWIGLU) {
      // fragment-major hidden rows at the expert-sorted row
      const int frow = arow0 + r;
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int col = nb * 32 + n * 16 + (lane & 15);
        if (col >= a.N) continue;
        ((bf16_t*)a.out)[fm_index(frow, col, a.N)] = f2bf(silu_f(acc[n][i]) * acc[n + 2][i]);
      }
    } else {
      const int orow = a.perm[off + r];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int col = nb * WSD_BN + n * 16 + (lane & 15);
        if (col >= a.N) continue;
        ((float*)a.out)[(size_t)orow * a.ldo + col] = acc[n][i];
      }
    }
  }
}

}  // namespace

// LDS ring depth (stages of 8 KB; two blocks per CU fit up to 10).
#ifndef DG_WSD_NST
#define DG_WSD_NST 8
#endif

int dg_launch_wsd(int epi, const WsArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return 0;
  if (!a.counts || !a.units || !a.n_units || a.rowsrc || a.wfmt != DG_WS_W_BF16 || a.K % 64 || a.K < 64) return -1;
  if (epi == WS_EPI_SWIGLU) k_wsd<WS_EPI_SWIGLU, DG_WSD_NST><<<grid, WSD_NT, 0, s>>>(a);
  else if (epi == WS_EPI_STORE_F32) k_wsd<WS_EPI_STORE_F32, DG_WSD_NST><<<grid, WSD_NT, 0, s>>>(a);
  else return -1;
  return 0;
}
