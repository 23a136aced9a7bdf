// Routed-expert projections (bf16 weights) with the weight tiles copied straight
// from HBM into LDS: the same work units, tiles and epilogues as the grouped
// launches of k_ws, with the weight stream moved out of registers.
//
// A block owns one part of an expert's rows (at most DG_WS_GROUP_ROWS = 128, one
// 16-row m-tile per consumer wave) and a span of S consecutive n-blocks of 64
// weight rows, which it sweeps one after the other: the weight stream runs on
// from one n-block into the next (the ring does not drain between them), and
// the consumers store each n-block's results as it ends.  Its ten waves split
// the work by role:
//   * two producer waves copy each 8 KB weight chunk (64 rows x 64 reduction
//     elements) into an LDS ring of NST stages with global_load_lds_dwordx4 --
//     four copies per wave per chunk, NST - 1 chunks ahead of the consumers --
//     and, since the compiler does not track these copies, wait for them
//     themselves (DG_WAIT_VMCNT) before the chunk's barrier;
//   * eight consumer waves load their m-tile's activation fragments with
//     ordinary loads three chunks ahead (so the compiler's own waits for them
//     stay exact: a consumer issues no copies), read the weight fragments of
//     the chunk from LDS and run the matrix cores.  The activations are
//     row-major rows: for W1/W3 the normalised token rows themselves, each
//     sorted row read through rowsrc (no sorted copy is made: the few token
//     rows stay in L2), for W2 the SwiGLU output, stored row-major at the
//     expert-sorted rows.  Lane l holds row l % 16 and loads, for matrix-core
//     step q of a chunk, the 16 bytes of reduction elements 32 q + 8 g .. + 7
//     (g = l / 16): 64 contiguous bytes of each of 16 rows per load.
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
//
// The work list (built with the routing) is cut into 8 contiguous slices in
// the order expert, span, part, and slice x is laid out at list positions x,
// x + 8, x + 16, ...: work-groups are dealt to the XCDs in turn, so XCD x runs
// slice x in order.  An XCD then works on few experts at a time -- their rows
// are fetched into its L2 once, not by all eight XCDs -- and the parts of one
// span run side by side and share its weight tiles in that L2.
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

// A consumer wave's chunk loop over a span of nsub n-blocks (nsub x nk chunks):
// fragments of the chunk three ahead loaded while a chunk is computed (ACT; an
// idle wave only meets the barriers), one barrier per chunk, the weight
// fragments read from stage c % NST.  The activation rows are the same for
// every n-block of the span, so the fetch index wraps at nk; after the last
// chunk of each n-block its results go to epi(acc, n-block of the span).  The
// loop body covers whole groups of 4 chunks with no branch around a load (so
// the compiler keeps exact waits for the activation loads); the last
// (nsub nk) % 4 chunks follow it.
template <bool ACT, int NST, typename Epi>
__device__ __forceinline__ void wsd_consume(uint4 (*sW)[WSD_SLOTS], const char* ap, int nk, int nsub, int lane,
                                            Epi&& epi) {
  int fk = 0;  // chunk of the next activation fetch
  auto fetch_a = [&](v8s (&A)[2]) __attribute__((always_inline)) {
    if constexpr (ACT) {
#pragma unroll
      for (int q = 0; q < 2; ++q) A[q] = *(const v8s*)(ap + (size_t)fk * 128 + q * 64);
      fk = fk + 1 == nk ? 0 : fk + 1;
    }
  };
  v4f acc[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};
  v8s A0[2], A1[2], A2[2], A3[2];
  fetch_a(A0);
  fetch_a(A1);
  fetch_a(A2);
  int kc = 0, sub = 0;  // chunk within the n-block, n-block of the span
  auto step = [&](v8s (&Acur)[2], v8s (&Anext)[2], int c) __attribute__((always_inline)) {
    fetch_a(Anext);                // chunk c + 3 (past the end: the first chunks again)
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
      if (++kc == nk) {  // the n-block is done (uniform)
        epi(acc, sub);
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};
        kc = 0;
        ++sub;
      }
    }
  };
  const int total = nsub * nk;
  int c = 0;
  for (; c + 4 <= total; c += 4) {
    step(A0, A3, c);
    step(A1, A0, c + 1);
    step(A2, A1, c + 2);
    step(A3, A2, c + 3);
  }
  if (c < total) step(A0, A3, c);  // the last total % 4 chunks
  if (c + 1 < total) step(A1, A0, c + 1);
  if (c + 2 < total) step(A2, A1, c + 2);
}

// A consumer wave's results for rows t0 .. t0 + 15 of a part (rows row0 .. of
// group g, cnt of them) and the 64 weight rows of n-block nb: lane holds
// columns n * 16 + lane % 16 of rows 4 (lane / 16) + i.
template <int EPI>
__device__ __forceinline__ void wsd_epilogue(const WsArgs& a, const v4f (&acc)[4], int g, int nb, int row0, int cnt,
                                             int t0, int lane) {
  const int off = a.offsets[g], arow0 = a.offsets16[g];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = t0 + (lane >> 4) * 4 + i;
    if (rl >= cnt) continue;
    const int r = row0 + rl;
    if constexpr (EPI == WS_EPI_SWIGLU) {
      // row-major hidden rows at the expert-sorted row
      bf16_t* hrow = (bf16_t*)a.out + (size_t)(arow0 + r) * a.N;
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int col = nb * 32 + n * 16 + (lane & 15);
        if (col >= a.N) continue;
        hrow[col] = f2bf(silu_f(acc[n][i]) * acc[n + 2][i]);
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

template <int EPI, int NST>
__global__ void __launch_bounds__(WSD_NT) k_wsd(WsArgs a) {
  static_assert(NST >= 3 && (NST - 2) * WSD_INS <= 63, "ring depth within the vmcnt range");
  __shared__ uint4 sW[NST][WSD_SLOTS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if ((int)blockIdx.x >= *a.n_units) return;
  const uint32_t code = (uint32_t)a.units[blockIdx.x];
  if (code == DG_WS_UNIT_NONE) return;  // padding of the work list
  const int g = (int)(code >> 24), part = (int)((code >> 16) & 0xff);
  const int span = max(a.span, 1), nb0 = (int)(code & 0xffff) * span, nsub = min(span, a.nblk - nb0);
  const int row0 = part * DG_WS_GROUP_ROWS;
  const int cnt = min(a.counts[g] - row0, DG_WS_GROUP_ROWS);
  if (cnt <= 0 || nsub <= 0) return;  // uniform over the block
  const int nk = a.K / 64;

  if (wave >= WSD_NCW) {
    // ---- producer: copies of the span's weight chunks into the LDS ring
    const int p = wave - WSD_NCW;
    const char* src[WSD_INS];
    auto rows_of = [&](int nb) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < WSD_INS; ++i) {
        const int s = (p * WSD_INS + i) * 64 + lane, row = s >> 3, seg = (s & 7) ^ (row & 7);
        src[i] = wsd_row<EPI>(a, g, nb, row) + seg * 16;
      }
    };
    rows_of(nb0);
    int pk = -1, ps = 0;  // chunk and n-block of the last copy issued
    auto issue = [&](int st) __attribute__((always_inline)) {
      if (pk + 1 < nk) ++pk;
      else if (ps + 1 < nsub) {  // the next n-block of the span (uniform)
        ++ps;
        pk = 0;
        rows_of(nb0 + ps);
      }  // past the end: the last chunk again
      const size_t kb = (size_t)pk * 128;
#pragma unroll
      for (int i = 0; i < WSD_INS; ++i) lds_dma16(src[i] + kb, &sW[st][(p * WSD_INS + i) * 64]);
    };
    DG_WAIT_VMCNT(0);  // nothing of the compiler's own is outstanding from here on
#pragma unroll
    for (int c = 0; c < NST - 1; ++c) issue(c);
    const int total = nsub * nk;
    for (int c = 0; c < total; ++c) {
      DG_WAIT_VMCNT((NST - 2) * WSD_INS);  // this wave's copies of chunk c have landed
      __builtin_amdgcn_s_barrier();        // ... and every wave's; stage (c - 1) % NST is free
      asm volatile("" ::: "memory");
      issue((c + NST - 1) % NST);
    }
    DG_WAIT_VMCNT(0);  // no copy may land after the block has ended
    return;
  }

  // ---- consumer: this wave's m-tile (rows t0 .. t0 + 15 of the part)
  const int t0 = wave * 16;
  // lane's row (a row past the part's end reads its last row; only active
  // waves load), through rowsrc when set, and its bytes of each 128-byte chunk
  const int srow = a.offsets16[g] + row0 + min(t0 + (lane & 15), cnt - 1);
  const int row = a.rowsrc ? a.rowsrc[srow] : srow;
  const char* ap = (const char*)a.A + (size_t)row * a.K * 2 + (lane >> 4) * 16;
  auto epi = [&](const v4f (&acc)[4], int sub) __attribute__((always_inline)) {
    wsd_epilogue<EPI>(a, acc, g, nb0 + sub, row0, cnt, t0, lane);
  };
  // The active and the idle waves run separate loops (same barriers): a
  // conditional load inside the loop makes the compiler's wait bookkeeping give
  // up the three-chunk lead of the activation loads.
  if (t0 < cnt) wsd_consume<true, NST>(sW, ap, nk, nsub, lane, epi);  // uniform over the wave
  else wsd_consume<false, NST>(sW, ap, nk, nsub, lane, epi);
}

}  // namespace

// LDS ring depth (stages of 8 KB; two blocks per CU fit up to 10).
#ifndef DG_WSD_NST
#define DG_WSD_NST 8
#endif

int dg_launch_wsd(int epi, const WsArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return 0;
  if (!a.counts || !a.units || !a.n_units || a.wfmt != DG_WS_W_BF16 || a.K % 64 || a.K < 64) return -1;
  if (a.nblk <= 0 || a.span > 0xffff || (a.rowsrc && epi != WS_EPI_SWIGLU)) return -1;
  if (epi == WS_EPI_SWIGLU) k_wsd<WS_EPI_SWIGLU, DG_WSD_NST><<<grid, WSD_NT, 0, s>>>(a);
  else if (epi == WS_EPI_STORE_F32) k_wsd<WS_EPI_STORE_F32, DG_WSD_NST><<<grid, WSD_NT, 0, s>>>(a);
  else return -1;
  return 0;
}
