// Routed-expert projections (bf16 weights) with the weight tiles copied straight
// from HBM into LDS: the same work units, tiles and epilogues as the grouped
// launches of k_ws, with the weight stream moved out of registers.
//
// A block owns one part of an expert's rows (at most DG_WSD_PART_ROWS = 256:
// consumer wave w takes m-tiles w and w + 8, the second only where the part
// has more than 128 rows, so an expert's weights stream once for up to 256
// rows) and a span of S consecutive n-blocks of BN (64 or 128) weight rows,
// which it sweeps one after the other: the weight stream runs on from one
// n-block into the next (the ring does not drain between them), and the
// consumers store each n-block's results as it ends.  Dense launches use
// n-blocks of 64.  Its ten waves split the work by role:
//   * two producer waves copy each weight chunk (BN rows x 64 reduction
//     elements, 8 or 16 KB) into a 64 KB LDS ring of NST = 8 or 4 stages with
//     global_load_lds_dwordx4 -- BN / 16 copies per wave per chunk, NST - 1
//     chunks ahead of the consumers -- and, since the compiler does not track
//     these copies, wait for them themselves (DG_WAIT_VMCNT) before the
//     chunk's barrier;
//   * eight consumer waves load their m-tiles' activation fragments with
//     ordinary loads three chunks ahead (two for 16 KB chunks; so the
//     compiler's own waits for them
//     stay exact: a consumer issues no copies), read the weight fragments of
//     the chunk from LDS and run the matrix cores.  For W1/W3 the activations
//     are the normalised token rows themselves (row-major), each sorted row
//     read through rowsrc (no sorted copy is made: the few token rows stay in
//     L2): lane l holds row l % 16 and loads, for matrix-core step q of a
//     chunk, the 16 bytes of reduction elements 32 q + 8 g .. + 7 (g = l / 16),
//     64 contiguous bytes of each of 16 rows per load.  For W2 they are the
//     SwiGLU output, which W1/W3 store fragment-major at the expert-sorted
//     rows: one contiguous 1 KB load per step (whole cache lines, which the
//     many-row parts, bound by their activation loads, read about twice as
//     fast).
// One barrier per chunk, passed by all ten waves: it publishes chunk c (every
// producer has waited for its copies of c) and frees the stage that chunk c - 1
// used (every consumer has read it), which the producers refill at once.  The
// ring holds NST stages, so 56 or 48 KB are in flight per block instead of the
// four register slots of k_ws, and no register holds weights.
//
// LDS rows are XOR-swizzled in 16-byte units exactly as in k_ws, so the
// fragment reads are free of bank conflicts; the copies write each stage in
// lane order, and each lane picks the global segment that belongs at its slot.
// Copies of chunks past the end reload the last chunk into a free stage, so
// every iteration issues the same copies and the waits stay constant.
//
// The work list (built with the routing) is longest first: the parts in
// decreasing order of their 16-row tiles, each part's spans side by side, so
// the blocks that start last are the shortest and the launch ends with few CUs
// idle.  (A list cut into one slice per XCD, to keep each expert's rows in one
// L2, measured no faster: the token rows are 1.4 MB and stay in every L2.)
#include "dg_common.h"
#include "dg_kernels.h"
#include "ws_common.h"

// Weight rows per n-block of the routed launches (64 or 128; the 64 KB ring,
// which allows one block per CU, holds 8 or 4 chunks).  128: the many-row
// parts are bound by their activation loads, which every n-block repeats, so
// twice the weight rows per n-block halves them (measured 10.38 -> 10.01 ms
// per step, W1/W3 122 -> 116 us).
// The weight copies of the routed bf16 launches carry the non-temporal hint (1;
// 0: never).  Those weights are read once per launch in whole 128-byte lines
// (64 bf16 per row per chunk), and the hint lets the L2 evict them before the
// activation rows that every block re-reads: routed W1/W3 117 -> 104 us per
// launch, 9.92 -> 9.43 ms per step, measured side by side.  FP8 and MXFP4
// chunks read 64 or 32 bytes of each weight line, the rest of the line in the
// next chunks, and with the hint the line is gone by then (W1/W3 86 -> 92 us);
// the dense launches' row parts share each weight tile through the L2.  Both
// stay plain.
#ifndef DG_WSD_W_NT
#define DG_WSD_W_NT 1
#endif

#ifndef DG_WSD_BN_UP
#define DG_WSD_BN_UP 128
#endif
#ifndef DG_WSD_BN_DN
#define DG_WSD_BN_DN 128
#endif
static_assert((DG_WSD_BN_UP == 64 || DG_WSD_BN_UP == 128) && (DG_WSD_BN_DN == 64 || DG_WSD_BN_DN == 128),
              "n-blocks of 64 or 128 weight rows");

// n-blocks per unit of the routed launches (a span: the unit sweeps them with
// the ring running on from one into the next).
#ifndef DG_WSD_SPAN_UP
#define DG_WSD_SPAN_UP 1
#endif
#ifndef DG_WSD_SPAN_DN
#define DG_WSD_SPAN_DN 1
#endif

namespace {

constexpr int WSD_NCW = 8;                           // consumer waves (m-tile = wave)
constexpr int WSD_NPW = 2;                           // producer waves
constexpr int WSD_NT = 64 * (WSD_NCW + WSD_NPW);     // 640 threads
constexpr int WSD_LDS_SLOTS = 4096;                 // 16-byte LDS slots of the ring (64 KB)
// A block's n-block is BN weight rows (64 or 128: NT = BN / 16 n-tiles per
// consumer wave); a chunk is BN rows x 64 reduction elements: SEG 16-byte
// segments per row (8 for bf16 weights, 4 for E4M3 codes, 2 for MXFP4 codes),
// SLOTS = BN SEG 16-byte slots, and the ring holds WSD_LDS_SLOTS / SLOTS
// chunks.  INS: copies per producer wave per chunk.
template <int BN, int WF = DG_WS_W_BF16>
struct WsdShape {
  static constexpr int NT = BN / 16, SEG = WF == DG_WS_W_E4M3 ? 4 : WF == DG_WS_W_MXFP4 ? 2 : 8,
                       SLOTS = BN * SEG, NST = WSD_LDS_SLOTS / SLOTS, INS = SLOTS / 64 / WSD_NPW;
};
// MXFP4: LDS bytes for the block scales of a unit's weight rows (BN x K / 32),
// copied once per unit.
constexpr int WSD_MX_SCALE_BYTES = 16384;
static_assert(WSD_NCW * 16 == DG_WS_GROUP_ROWS, "one m-tile per consumer wave covers a dense part");
static_assert(2 * DG_WS_GROUP_ROWS == DG_WSD_PART_ROWS, "two m-tiles per consumer wave cover a routed part");

// LDS slot of 16-byte segment seg of weight row `row` of a stage: bf16 rows of
// 8 segments XOR-swizzled by the row's low 3 bits, E4M3 rows of 4 segments by
// bits 1-2 (eight consecutive lanes reading one segment of eight consecutive
// rows then touch eight distinct 16-byte bank groups).
// MXFP4 rows of 2 segments, the lanes reading 8 bytes (one half of a segment)
// each: the segments of rows 8..15 of every 16 are swapped, so that 16 lanes
// reading one half of 16 rows touch 16 distinct 8-byte bank groups of a 256-byte
// bank row.
template <int WF = DG_WS_W_BF16>
__device__ __forceinline__ int wsd_slot(int row, int seg) {
  if constexpr (WF == DG_WS_W_E4M3) return row * 4 + (seg ^ ((row >> 1) & 3));
  else if constexpr (WF == DG_WS_W_MXFP4) return row * 2 + (seg ^ ((row >> 3) & 1));
  else return row * 8 + (seg ^ (row & 7));
}

// A consumer wave's chunk loop over a span of nsub n-blocks (nsub x nk chunks),
// one barrier per chunk, the weight fragments read from stage c % NST and used
// for each of the wave's MT m-tiles; an idle wave (ACT false) only meets the
// barriers.  The activation fragments of the chunk PD ahead are loaded
// while a chunk is computed (PD + 1 register buffers): from row-major rows
// (ap[m]: the lane's row of m-tile m; step q of chunk c at bytes 128 c + 64 q)
// or, AFM, from the fragment-major layout (ap[m]: the m-tile's first 1 KB block
// plus 16 bytes per lane; step q of chunk c is block 2 c + q).
// The activation rows are the same for every n-block of the span, so the fetch
// index wraps at nk; after the last chunk of each n-block its results go to
// epi(acc, n-block of the span) -- inside the loop for spans (SPAN), else once
// after it, so that a large epilogue is not repeated in the unrolled body
// (epi(acc of m-tile m, n-block, m) for each m-tile).  The
// loop body covers whole groups of PD + 1 chunks with no branch around a load
// (so the compiler keeps exact waits for them); the remaining chunks follow it.
template <int MT, int BN, bool ACT, bool AFM, bool SPAN, int WF = DG_WS_W_BF16, typename Epi>
__device__ __forceinline__ void wsd_consume(const uint4* sW, const char* const (&ap)[MT], int nk, int nsub,
                                            int lane, Epi&& epi, const uint8_t* sS = nullptr) {
  using S = WsdShape<BN, WF>;
  constexpr int NT = S::NT;
  constexpr bool MX = WF == DG_WS_W_MXFP4;
  // E4M3 and MXFP4 codes take the reduction order below (E8: permuted)
  constexpr bool E8 = WF == DG_WS_W_E4M3 || MX;
  // Activation step q of chunk fk: bf16 weights take reduction elements
  // 32 q + 8 g .. + 7 of the chunk in lane group g; E4M3 weights 16 g + 8 q ..
  // + 7, so that a lane's codes for both steps are one 16-byte segment (ap then
  // already holds the lane group's offset of the permuted order).
  auto a_off = [&](int f, int q) __attribute__((always_inline)) -> size_t {
    if constexpr (AFM) return E8 ? (size_t)f * 2048 + q * 256 : (size_t)(2 * f + q) * 1024;
    else return (size_t)f * 128 + q * (E8 ? 16 : 64);
  };
  int fk = 0;  // chunk of the next activation fetch
  auto fetch_a = [&](v8s (&A)[MT][2]) __attribute__((always_inline)) {
    if constexpr (ACT) {
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int q = 0; q < 2; ++q) A[m][q] = *(const v8s*)(ap[m] + a_off(fk, q));
      fk = fk + 1 == nk ? 0 : fk + 1;
    }
  };
  v4f acc[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int n = 0; n < NT; ++n) acc[m][n] = v4f{0.f, 0.f, 0.f, 0.f};
  // activation prefetch depth in chunks: 3, or 2 for the twice as long chunks of
  // 128-row n-blocks (fewer registers for their twice as many accumulators)
  constexpr int PD = BN == 128 ? 2 : 3;
  v8s A0[MT][2], A1[MT][2], A2[MT][2], A3[MT][2];
  fetch_a(A0);
  fetch_a(A1);
  if constexpr (PD == 3) fetch_a(A2);
  int kc = 0, sub = 0;  // chunk within the n-block, n-block of the span
  auto step = [&](v8s (&Acur)[MT][2], v8s (&Anext)[MT][2], int c) __attribute__((always_inline)) {
    fetch_a(Anext);                // chunk c + PD (past the end: the first chunks again)
    __builtin_amdgcn_s_barrier();  // chunk c is in its stage
    asm volatile("" ::: "memory");
    if constexpr (ACT) {
      const uint4* st = sW + (c % S::NST) * S::SLOTS;
      if constexpr (MX) {
        // lane group u takes reduction elements 16 u .. 16 u + 15 of the chunk
        // (the activations were loaded in the same order): 8 bytes of codes per
        // n-tile, inside one MX block, whose scale byte the unit's copy holds
        const int u = lane >> 4, kb32 = (nk * 64) >> 5;
#pragma unroll
        for (int n0 = 0; n0 < NT; n0 += 2) {
          uint2 raw[2];
          uint32_t sb[2];
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            const int row = (n0 + n) * 16 + (lane & 15);
            raw[n] = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(st) +
                                                     wsd_slot<WF>(row, u >> 1) * 16 + (u & 1) * 8);
            sb[n] = sS[row * kb32 + 2 * (c % nk) + (u >> 1)];
          }
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            v8s wf[2];
#pragma unroll
            for (int n = 0; n < 2; ++n) {
              const uint4 w4 = mxfp4x8_to_bf16(q ? raw[n].y : raw[n].x, sb[n]);
              wf[n] = *reinterpret_cast<const v8s*>(&w4);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
              for (int n = 0; n < 2; ++n)
                acc[m][n0 + n] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(Acur[m][q], wf[n], acc[m][n0 + n], 0, 0, 0);
          }
        }
      } else if constexpr (E8) {
        // two n-tiles at a time (registers): one segment of 16 codes per lane
        // and n-tile, widened to bf16 half by half (step 0: codes 0..7, step 1:
        // codes 8..15)
#pragma unroll
        for (int n0 = 0; n0 < NT; n0 += 2) {
          uint4 raw[2];
#pragma unroll
          for (int n = 0; n < 2; ++n) raw[n] = st[wsd_slot<WF>((n0 + n) * 16 + (lane & 15), lane >> 4)];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            v8s wf[2];
#pragma unroll
            for (int n = 0; n < 2; ++n) {
              const uint4 u = q ? e4m3x8_to_bf16(raw[n].z, raw[n].w) : e4m3x8_to_bf16(raw[n].x, raw[n].y);
              wf[n] = *reinterpret_cast<const v8s*>(&u);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
              for (int n = 0; n < 2; ++n)
                acc[m][n0 + n] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(Acur[m][q], wf[n], acc[m][n0 + n], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
#pragma unroll
          for (int n0 = 0; n0 < NT; n0 += 4) {  // weight fragments four n-tiles at a time
            v8s wf[4];
#pragma unroll
            for (int n = 0; n < 4; ++n) {
              const uint4 u = st[wsd_slot((n0 + n) * 16 + (lane & 15), q * 4 + (lane >> 4))];
              wf[n] = *reinterpret_cast<const v8s*>(&u);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
              for (int n = 0; n < 4; ++n)
                acc[m][n0 + n] =
                    __builtin_amdgcn_mfma_f32_16x16x32_bf16(Acur[m][q], wf[n], acc[m][n0 + n], 0, 0, 0);
          }
        }
      }
      if (SPAN && ++kc == nk) {  // the n-block is done (uniform)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          epi(acc[m], sub, m);
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[m][n] = v4f{0.f, 0.f, 0.f, 0.f};
        }
        kc = 0;
        ++sub;
      }
    }
  };
  const int total = nsub * nk;
  int c = 0;
  if constexpr (PD == 3) {
    for (; c + 4 <= total; c += 4) {
      step(A0, A3, c);
      step(A1, A0, c + 1);
      step(A2, A1, c + 2);
      step(A3, A2, c + 3);
    }
    if (c < total) step(A0, A3, c);  // the last total % 4 chunks
    if (c + 1 < total) step(A1, A0, c + 1);
    if (c + 2 < total) step(A2, A1, c + 2);
  } else {
    for (; c + 3 <= total; c += 3) {
      step(A0, A2, c);
      step(A1, A0, c + 1);
      step(A2, A1, c + 2);
    }
    if (c < total) step(A0, A2, c);  // the last total % 3 chunks
    if (c + 1 < total) step(A1, A0, c + 1);
  }
  if constexpr (ACT && !SPAN) {
#pragma unroll
    for (int m = 0; m < MT; ++m) epi(acc[m], 0, m);
  }
}

// A consumer wave's results for its m-tile (rows t0 .. t0 + 15 of a part with
// cnt rows) and the 16 NT weight rows of n-block nb (SwiGLU: NT / 2 n-tiles of
// W1 rows, then the matching NT / 2 of W3): lane holds columns n * 16 +
// lane % 16 of rows 4 (lane / 16) + i.  orow[i]: where the lane's row i goes
// -- the fragment-major offset of the expert-sorted row (SwiGLU) or the pair
// index (fp32 store) -- looked up before the chunk loop, so the epilogue
// issues stores only.
template <int EPI, int NT, int WF = DG_WS_W_BF16>
__device__ __forceinline__ void wsd_epilogue(const WsArgs& a, const v4f (&acc)[NT], int g, int nb, int cnt, int t0,
                                             int lane, const int (&orow)[4]) {
  // E4M3 weights: each weight row's scale multiplies its fp32 sum (SwiGLU: the
  // W1 and W3 sums before the activation)
  constexpr bool E8 = WF == DG_WS_W_E4M3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rl = t0 + (lane >> 4) * 4 + i;
    if (rl >= cnt) continue;
    if constexpr (EPI == WS_EPI_SWIGLU) {
      // hidden rows at the expert-sorted row, fragment-major: each 32 columns
      // of an m-tile are one 1 KB block, orow[i] the row's element offset in
      // its tile's first block (fm_index of column 0)
#pragma unroll
      for (int n = 0; n < NT / 2; ++n) {
        const int col = nb * 8 * NT + n * 16 + (lane & 15);
        if (col >= a.N) continue;
        const float u = E8 ? acc[n][i] * a.wsc0[(size_t)g * a.N + col] : acc[n][i];
        const float v = E8 ? acc[n + NT / 2][i] * a.wsc1[(size_t)g * a.N + col] : acc[n + NT / 2][i];
        ((bf16_t*)a.out)[(size_t)orow[i] + (col >> 5) * 512 + ((col & 31) >> 3) * 128 + (lane & 7)] =
            f2bf(silu_f(u) * v);
      }
    } else {
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int col = nb * 16 * NT + n * 16 + (lane & 15);
        if (col >= a.N) continue;
        ((float*)a.out)[(size_t)orow[i] * a.ldo + col] = E8 ? acc[n][i] * a.wsc0[(size_t)g * a.N + col] : acc[n][i];
      }
    }
  }
}

// One kernel for both kinds of launch:
//   * grouped (DENSE false): routed experts on a work list, units (expert,
//     row part, span of n-blocks); activations row-major through rowsrc
//     (W1/W3) or fragment-major (W2), wsd_epilogue;
//   * dense (DENSE true): one weight matrix on M rows, units (n-block, row part
//     of 128, reduction range) dealt as in k_ws: work-groups go to the 8 XCDs in
//     turn (block b to XCD b % 8), so n-block nb goes to XCD nb % 8 and its
//     parts x ranges to consecutive slots of that XCD -- the parts of one
//     n-block run together and read its weight tile from that XCD's L2; the
//     grid is 8 ceil(nblk / 8) x parts x ranges, padding blocks exit at once.
//     Activations fragment-major; the epilogues of k_ws (ws_tile_epilogue).
template <int EPI, bool DENSE, int BN, int WF = DG_WS_W_BF16>
__global__ void __launch_bounds__(WSD_NT) k_wsd(WsArgs a) {
  using S = WsdShape<BN, WF>;
  constexpr bool MX = WF == DG_WS_W_MXFP4;
  // E4M3 or MXFP4 codes: the permuted reduction order, 128-row parts
  constexpr bool E8 = WF == DG_WS_W_E4M3 || MX;
  static_assert(!E8 || !DENSE, "E4M3 / MXFP4 weights: routed experts only");
  constexpr int NST = S::NST, INS = S::INS;
  static_assert(NST >= 3 && (NST - 2) * INS <= 63, "ring depth within the vmcnt range");
  __shared__ uint4 sW[WSD_LDS_SLOTS];
  __shared__ uint4 sS4[MX ? WSD_MX_SCALE_BYTES / 16 : 1];  // MXFP4: the unit's block scales
  const uint8_t* sS = reinterpret_cast<const uint8_t*>(sS4);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int g = 0, row0, cnt, nb0, nsub = 1, ks = 0, kc0 = 0, nk = a.K / 64;
  bool wnt = false;  // weight copies with the non-temporal hint
  if constexpr (DENSE) {
    const int msp = max(a.msplit, 1), ksp = max(a.ksplit, 1);
    const int b = blockIdx.x, x = b % 8, j = b / 8, nsubblk = msp * ksp, sub = j % nsubblk;
    ks = sub / msp;
    nb0 = x + 8 * (j / nsubblk);
    if (nb0 >= a.nblk) return;  // padding of the grid
    const int M = a.M_dev ? *a.M_dev : a.M;
    row0 = (sub % msp) * DG_WS_GROUP_ROWS;
    cnt = min(M - row0, DG_WS_GROUP_ROWS);
    if (ksp > 1) {
      kc0 = ks * a.kchunks;
      nk = min(nk - kc0, a.kchunks);
    }
    if (cnt <= 0 || nk <= 0) return;  // uniform over the block
  } else {
    if ((int)blockIdx.x >= *a.n_units) return;
    const uint32_t code = (uint32_t)a.units[blockIdx.x];
    if (code == DG_WS_UNIT_NONE) return;  // padding of the work list
    g = (int)(code >> 24);
    const int part = (int)((code >> 16) & 0xff), span = max(a.span, 1);
    nb0 = (int)(code & 0xffff) * span;
    nsub = min(span, a.nblk - nb0);
    // parts of DG_WSD_PART_ROWS rows (E4M3: DG_WS_GROUP_ROWS, one m-tile per
    // wave, which leaves registers for the code widening)
    constexpr int PR = E8 ? DG_WS_GROUP_ROWS : DG_WSD_PART_ROWS;
    row0 = part * PR;
    cnt = min(a.counts[g] - row0, PR);
    if (cnt <= 0 || nsub <= 0) return;  // uniform over the block
    wnt = DG_WSD_W_NT && WF == DG_WS_W_BF16;
  }

  if (wave >= WSD_NCW) {
    // ---- producer: copies of the weight chunks (a span's n-blocks in turn) into the LDS ring
    const int p = wave - WSD_NCW;
    const char* src[INS];
    auto rows_of = [&](int nb) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < INS; ++i) {
        // slot s of the stage holds the global segment of its row that
        // wsd_slot puts there
        const int s = (p * INS + i) * 64 + lane;
        int row, seg;
        if constexpr (MX) {  // the inverse of wsd_slot<MXFP4>
          row = s >> 1;
          seg = (s & 1) ^ ((row >> 3) & 1);
        } else {
          row = s / S::SEG;
          seg = WF == DG_WS_W_E4M3 ? (s & 3) ^ ((row >> 1) & 3) : (s & 7) ^ (row & 7);
        }
        src[i] = weight_row<EPI, S::NT, MX ? 4 : E8 ? 8 : 16>(a, g, nb, row) + (size_t)kc0 * S::SEG * 16 + seg * 16;
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
      const size_t kb = (size_t)pk * S::SEG * 16;
#pragma unroll
      for (int i = 0; i < INS; ++i) {
        if (wnt) lds_dma16_nt(src[i] + kb, &sW[st * S::SLOTS + (p * INS + i) * 64]);
        else lds_dma16(src[i] + kb, &sW[st * S::SLOTS + (p * INS + i) * 64]);
      }
    };
    DG_WAIT_VMCNT(0);  // nothing of the compiler's own is outstanding from here on
    if constexpr (MX) {
      // The unit's block scales (one n-block: span 1), K / 32 bytes per weight
      // row, copied once before the ring starts (SwiGLU: the W1 rows, then the
      // W3 rows); rows past N are not copied.  The first chunk's wait below
      // covers these copies too (loads complete in order).
      const int kb32 = a.K >> 5;
      auto copy_rows = [&](const uint8_t* base, int n0, int nrows, int lrow0) __attribute__((always_inline)) {
        nrows = min(nrows, a.N - n0);
        const int pieces = nrows > 0 ? nrows * kb32 / 16 : 0;
        const uint8_t* src0 = base + (size_t)g * (a.wgs / 32) + (size_t)n0 * kb32;
        for (int j = 0; j * 128 < pieces; ++j) {
          const int q = j * 128 + p * 64 + lane;
          uint4* dst = sS4 + lrow0 * kb32 / 16 + j * 128 + p * 64;  // wave-uniform: lane l writes dst[l]
          if (q < pieces) lds_dma16(src0 + (size_t)q * 16, dst);
        }
      };
      if constexpr (EPI == WS_EPI_SWIGLU) {
        copy_rows(a.wbs0, nb0 * (BN / 2), BN / 2, 0);
        copy_rows(a.wbs1, nb0 * (BN / 2), BN / 2, BN / 2);
      } else {
        copy_rows(a.wbs0, nb0 * BN, BN, 0);
      }
    }
#pragma unroll
    for (int c = 0; c < NST - 1; ++c) issue(c);
    const int total = nsub * nk;
    for (int c = 0; c < total; ++c) {
      DG_WAIT_VMCNT((NST - 2) * INS);  // this wave's copies of chunk c have landed
      __builtin_amdgcn_s_barrier();        // ... and every wave's; stage (c - 1) % NST is free
      asm volatile("" ::: "memory");
      issue((c + NST - 1) % NST);
    }
    DG_WAIT_VMCNT(0);  // no copy may land after the block has ended
    return;
  }

  // ---- consumer: this wave's m-tile (rows t0 .. t0 + 15 of the part)
  const int t0 = wave * 16;
  if constexpr (DENSE) {
    // fragment-major rows: a tile past the part's rows reads the last one, which
    // holds valid rows (only active waves load)
    const int tr = row0 + min(t0, (cnt - 1) & ~15);
    const char* const ap[1] = {(const char*)a.A + ((size_t)(tr >> 4) * (a.K >> 5) + 2 * kc0) * 1024 + lane * 16};
    auto epi = [&](const v4f (&acc)[S::NT], int sub, int) __attribute__((always_inline)) {
      ws_tile_epilogue<EPI, S::NT, DG_WS_W_BF16>(a, acc, 0, nb0 + sub, row0, t0, cnt, 0, 0, ks, lane);
    };
    if (t0 < cnt) wsd_consume<1, BN, true, true, false>(sW, ap, nk, 1, lane, epi);  // uniform over the wave
    else wsd_consume<1, BN, false, true, false>(sW, ap, nk, 1, lane, epi);
  } else {
    // m-tiles t0 and t0 + 128 of the part.  W1/W3 (row-major token rows):
    // lane's row of each (a row past the part's end reads its last row; only
    // active waves load) through rowsrc, and its bytes of each 128-byte chunk;
    // W2 (AFM: the fragment-major hidden rows at the expert-sorted rows): the
    // m-tile's first 1 KB block.  The output rows of its results (orow[m][i])
    // are looked up before the loop.
    constexpr bool AFM = EPI != WS_EPI_SWIGLU;
    const char* ap[2];
    int orow[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int tm = t0 + m * DG_WS_GROUP_ROWS;
      if constexpr (AFM) {
        const int tile = (a.offsets16[g] + row0 + min(tm, (cnt - 1) & ~15)) >> 4;
        const int gq = lane >> 4;  // E4M3, MXFP4: the permuted reduction order of wsd_consume
        ap[m] = (const char*)a.A + (size_t)tile * (a.K >> 5) * 1024 +
                (E8 ? (gq >> 1) * 1024 + (32 * (gq & 1) + (lane & 15)) * 16 : lane * 16);
      } else {
        const int srow = a.offsets16[g] + row0 + min(tm + (lane & 15), cnt - 1);
        const int row = a.rowsrc ? a.rowsrc[srow] : srow;
        ap[m] = (const char*)a.A + (size_t)row * a.K * 2 + (lane >> 4) * (E8 ? 32 : 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = min(tm + (lane >> 4) * 4 + i, cnt - 1);
        if constexpr (EPI == WS_EPI_SWIGLU) orow[m][i] = (int)fm_index(a.offsets16[g] + row0 + rl, 0, a.N);
        else orow[m][i] = tm < cnt ? a.perm[a.offsets[g] + row0 + rl] : 0;
      }
    }
    auto epi = [&](const v4f (&acc)[S::NT], int sub, int m) __attribute__((always_inline)) {
      wsd_epilogue<EPI, S::NT, WF>(a, acc, g, nb0 + sub, cnt, t0 + m * DG_WS_GROUP_ROWS, lane, orow[m]);
    };
    // The waves with two, one or no m-tiles run separate loops (same barriers):
    // a conditional load inside the loop makes the compiler's wait bookkeeping
    // give up the three-chunk lead of the activation loads.
    // units of one n-block run the epilogue once after the loop
    constexpr bool SP = (EPI == WS_EPI_SWIGLU ? DG_WSD_SPAN_UP : DG_WSD_SPAN_DN) > 1;
    if (!E8 && t0 + DG_WS_GROUP_ROWS < cnt) {  // uniform over the wave
      if constexpr (!E8) {
        const char* const ap2[2] = {ap[0], ap[1]};
        wsd_consume<2, BN, true, AFM, SP, WF>(sW, ap2, nk, nsub, lane, epi);
      }
    } else {
      const char* const ap1[1] = {ap[0]};
      if (t0 < cnt) wsd_consume<1, BN, true, AFM, SP, WF>(sW, ap1, nk, nsub, lane, epi, sS);
      else wsd_consume<1, BN, false, AFM, SP, WF>(sW, ap1, nk, nsub, lane, epi, sS);
    }
  }
}

}  // namespace

int dg_wsd_bn(int epi) { return epi == WS_EPI_SWIGLU ? DG_WSD_BN_UP : DG_WSD_BN_DN; }
int dg_wsd_span(int epi) { return epi == WS_EPI_SWIGLU ? DG_WSD_SPAN_UP : DG_WSD_SPAN_DN; }

int dg_launch_wsd(int epi, const WsArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return 0;
  if (!a.counts || !a.units || !a.n_units || a.K % 64 || a.K < 64) return -1;
  if (a.wfmt == DG_WS_W_E4M3 && (!a.wsc0 || (epi == WS_EPI_SWIGLU && !a.wsc1))) return -1;
  if (a.wfmt == DG_WS_W_MXFP4) {  // scales of a unit in LDS: one n-block, whole 16-byte pieces
    if (!a.wbs0 || (epi == WS_EPI_SWIGLU && !a.wbs1) || a.span > 1 || a.N % 8) return -1;
    if ((size_t)(epi == WS_EPI_SWIGLU ? DG_WSD_BN_UP : DG_WSD_BN_DN) * (a.K / 32) > WSD_MX_SCALE_BYTES) return -1;
  }
  if (a.wfmt != DG_WS_W_BF16 && a.wfmt != DG_WS_W_E4M3 && a.wfmt != DG_WS_W_MXFP4) return -1;
  if (a.nblk <= 0 || a.span > 0xffff || (a.rowsrc && epi != WS_EPI_SWIGLU)) return -1;
  if (a.span > 1 && dg_wsd_span(epi) <= 1) return -1;  // that kernel stores one n-block per unit
  const int f = a.wfmt;
  constexpr int B = DG_WS_W_BF16, E8 = DG_WS_W_E4M3, F4 = DG_WS_W_MXFP4;
  if (epi == WS_EPI_SWIGLU) {
    if (f == B) k_wsd<WS_EPI_SWIGLU, false, DG_WSD_BN_UP><<<grid, WSD_NT, 0, s>>>(a);
    else if (f == E8) k_wsd<WS_EPI_SWIGLU, false, DG_WSD_BN_UP, E8><<<grid, WSD_NT, 0, s>>>(a);
    else k_wsd<WS_EPI_SWIGLU, false, DG_WSD_BN_UP, F4><<<grid, WSD_NT, 0, s>>>(a);
  } else if (epi == WS_EPI_STORE_F32) {
    if (f == B) k_wsd<WS_EPI_STORE_F32, false, DG_WSD_BN_DN><<<grid, WSD_NT, 0, s>>>(a);
    else if (f == E8) k_wsd<WS_EPI_STORE_F32, false, DG_WSD_BN_DN, E8><<<grid, WSD_NT, 0, s>>>(a);
    else k_wsd<WS_EPI_STORE_F32, false, DG_WSD_BN_DN, F4><<<grid, WSD_NT, 0, s>>>(a);
  } else {
    return -1;
  }
  return 0;
}

int dg_launch_wsd_dense(int epi, const WsArgs& a, hipStream_t s) {
  if (a.counts || a.wfmt != DG_WS_W_BF16 || a.K % 64 || a.K < 64 || a.nblk <= 0 || a.span > 1) return -1;
  if (a.ksplit > 1 && (epi != WS_EPI_ADD_F32 || !a.part_out || a.kchunks <= 0)) return -1;
  const int M = a.M;  // with M_dev: the most rows the device count can hold
  const int grid = (a.nblk + 7) / 8 * 8 * max(a.msplit, 1) * max(a.ksplit, 1);
  if (M <= 0 || max(a.msplit, 1) * DG_WS_GROUP_ROWS < M) return -1;  // every row in a part
  if (a.wide) {  // n-blocks of 128 weight rows: the fp32 add only
    if (epi != WS_EPI_ADD_F32) return -1;
    k_wsd<WS_EPI_ADD_F32, true, 128><<<grid, WSD_NT, 0, s>>>(a);
    return 0;
  }
  switch (epi) {
    case WS_EPI_STORE_BF16: k_wsd<WS_EPI_STORE_BF16, true, 64><<<grid, WSD_NT, 0, s>>>(a); break;
    case WS_EPI_STORE_F32: k_wsd<WS_EPI_STORE_F32, true, 64><<<grid, WSD_NT, 0, s>>>(a); break;
    case WS_EPI_ADD_F32: k_wsd<WS_EPI_ADD_F32, true, 64><<<grid, WSD_NT, 0, s>>>(a); break;
    case WS_EPI_SWIGLU: k_wsd<WS_EPI_SWIGLU, true, 64><<<grid, WSD_NT, 0, s>>>(a); break;
    case WS_EPI_ROPE_QKV: k_wsd<WS_EPI_ROPE_QKV, true, 64><<<grid, WSD_NT, 0, s>>>(a); break;
    default: return -1;
  }
  return 0;
}
