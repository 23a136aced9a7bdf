// Weight-streaming GEMM on the bf16 matrix cores, for the shapes of the denoising
// step: a few hundred activation rows against large weight matrices, so that the
// step's time is set by how fast the weights stream from HBM.  Used for the routed
// experts (grouped by expert, rows gathered through the token permutation), the
// shared expert, the dense projections and the LM head.
//
// A block owns BN = 16 * NTN consecutive weight rows ("n-block") of one group and
// a range of that group's activation rows: a grouped launch cuts each group into
// parts of at most DG_WS_GROUP_ROWS rows, one unit of work per (group, part,
// n-block), so that an expert that receives most of the rows does not serialise
// the launch; a dense launch splits its rows over msplit blocks per n-block.  The
// blocks that share a weight tile run on the same XCD at the same time, so the
// tile crosses HBM once and the others read it from that XCD's L2.  The weight tile streams through four
// LDS stages in chunks of KSUB x 64 reduction elements (128 bytes per row per
// sub-chunk), fed by a four-slot register ring; each chunk is stored two
// iterations before it is used (see ws_stream).  The eight waves split the
// activation rows (m-tile i goes to wave i % 8) and read their own activation
// fragments straight from global memory three chunks ahead.  Activations are in
// the fragment-major layout (fm_index), so each fragment is one contiguous 1 KB
// load; the routed down projection reads them in an expert-sorted layout in
// which every expert's rows start on a 16-row tile.  The routed W1/W3 launch
// instead gathers its rows from the row-major normalised rows through the
// sorted-row -> token map (a sorted copy would cost more than it saves).  The LDS rows are
// XOR-swizzled in 16-byte units so that both the cooperative stores and the
// fragment reads are free of bank conflicts.
//
// Matrix-core layout (v_mfma_f32_16x16x32_bf16): lane l supplies activation row
// l % 16 and weight row l % 16, each with reduction elements 8 (l / 16) .. +7 of a
// 32-element step, and receives D[4 (l / 16) + i][l % 16], i = 0..3.
#include "dg_common.h"
#include "dg_kernels.h"
#include "ws_common.h"

#include <type_traits>

namespace {

#ifndef DG_WS_KSUB
#define DG_WS_KSUB 1
#endif
constexpr int NWAVE = 8;  // waves per block
constexpr int NT = 64 * NWAVE;
// MT (template parameter): m-tiles per wave per pass, so a pass covers
// NWAVE * MT * 16 activation rows.
// A chunk is KSUB sub-chunks of 64 reduction elements (128 bytes of each weight
// row per sub-chunk); one barrier per chunk (see ws_stream for the pipeline).
constexpr int KSUB_PROJ = DG_WS_KSUB;  // projections and experts
constexpr int KSUB_LM = DG_WS_KSUB < 2 ? DG_WS_KSUB : 2;  // LM head (128 weight rows per block)


// LDS slot (16-byte units) of segment `seg` (0 .. 8 KSUB - 1) of weight row `row`:
// XOR swizzle of the segment within each 128-byte sub-row.
template <int KSUB>
__device__ __forceinline__ int lds_slot(int row, int seg) {
  return row * (8 * KSUB) + (seg & ~7) + ((seg & 7) ^ (row & 7));
}

// A thread's share of one weight chunk: N segments of 16 bytes of bf16 (T = uint4),
// or the codes they are widened from (T = uint2): 8 bytes of E4M3 codes, or 4
// bytes of MXFP4 codes (.x) and their E8M0 scale byte (.y).
template <int N, typename T>
struct Segs {
  T v[N];
};

// Register ring of up to eight weight chunks, selected by a compile-time index
// (a runtime index would put the ring in scratch memory).
template <int N, typename T>
struct Ring8 {
  Segs<N, T> r0, r1, r2, r3, r4, r5, r6, r7;
};
template <int I, int N, typename T>
__device__ __forceinline__ Segs<N, T>& ring(Ring8<N, T>& R) {
  if constexpr (I == 0) return R.r0;
  else if constexpr (I == 1) return R.r1;
  else if constexpr (I == 2) return R.r2;
  else if constexpr (I == 3) return R.r3;
  else if constexpr (I == 4) return R.r4;
  else if constexpr (I == 5) return R.r5;
  else if constexpr (I == 6) return R.r6;
  else return R.r7;
}

// Activation fragments of four consecutive chunks (chunk c in buffer c % 4),
// selected by a compile-time index.
template <int MT, int KSUB>
struct AFrags {
  v8s b0[MT][2 * KSUB], b1[MT][2 * KSUB], b2[MT][2 * KSUB], b3[MT][2 * KSUB];
};
template <int I, int MT, int KSUB>
__device__ __forceinline__ v8s (&abuf(AFrags<MT, KSUB>& F))[MT][2 * KSUB] {
  if constexpr (I == 0) return F.b0;
  else if constexpr (I == 1) return F.b1;
  else if constexpr (I == 2) return F.b2;
  else return F.b3;
}



// Streams the weight tile of one pass through LDS and accumulates this wave's MA
// active m-tiles (0 .. MT).
//
// Pipeline, with NSTAGE = 4 LDS stages and a ring of 4 register slots.  In
// iteration c the wave
//   1. fetches its activation fragments of chunk c + 3 (into buffer (c + 3) % 4),
//   2. stores weight chunk c + 2 (fetched four iterations earlier) into stage
//      (c + 2) % 4 and refills that ring slot with chunk c + 6,
//   3. computes chunk c from stage c % 4 (stored two iterations earlier) and
//      activation buffer c % 4,
//   4. meets the block at one barrier.
// The hardware retires vector loads in issue order, so a wait for one load is a
// wait for every older load.  Fetching the activations three chunks ahead, before
// the weight refill of the same iteration, means that the wait for chunk c's
// activations only covers weight loads that were already needed by earlier
// stores, and the four-chunk weight prefetch stays four chunks deep.  A stage is
// rewritten two barriers after its last reader.
//
// The loop body is branch-free: the chunk count is padded to a multiple of 4,
// chunks past the end are stored as zeros (their products add nothing) and every
// load address is clamped to valid memory, so the number of loads in flight is
// the same in every iteration and the compiler can wait for exactly the load it
// needs.  All variants execute the same barriers.
template <int NTN, int KSUB, int MT, int MA, bool GATHER, int RING, int WF>
__device__ __forceinline__ void ws_stream(uint4 (*sW)[16 * NTN * 8 * KSUB], const char* const (&gsrc)[NTN * KSUB / 4],
                                          const uint8_t* const (&gsc)[NTN * KSUB / 4],
                                          const int (&slot)[NTN * KSUB / 4], const int (&sub)[NTN * KSUB / 4],
                                          const char* const (&ap)[MT], int nk64, int lane, v4f (&acc)[MT][NTN]) {
  constexpr int NSEG = NTN * KSUB / 4;  // 16-byte LDS segments (8 weights) per thread per chunk
  using SegT = std::conditional_t<WF == DG_WS_W_BF16, uint4, uint2>;
  // bytes of a weight row per 64-element sub-chunk
  constexpr int SUBB = WF == DG_WS_W_BF16 ? 128 : WF == DG_WS_W_E4M3 ? 64 : 32;
  static_assert(RING == 4 || RING == 8, "ring of 4 or 8 chunks");
  const int nchunk = (nk64 + KSUB - 1) / KSUB;
  Ring8<NSEG, SegT> R;
  auto fetch = [&](Segs<NSEG, SegT>& S, int c) {
#pragma unroll
    for (int i = 0; i < NSEG; ++i) {
      const int kc = min(c * KSUB + sub[i], nk64 - 1);
      if constexpr (WF == DG_WS_W_MXFP4)
        S.v[i] = make_uint2(*(const uint32_t*)(gsrc[i] + kc * SUBB), *(const uint8_t*)(gsc[i] + kc * 2));
      else S.v[i] = *(const SegT*)(gsrc[i] + kc * SUBB);
    }
  };
  // Stores chunk c from S into its stage (E4M3 or MXFP4 codes widened to bf16 on
  // the way; zero codes widen to zeros);
  // sub-chunks past the end store zeros (a mask on the values: a conditional
  // between two lvalues would make the compiler select between their addresses
  // and keep the ring in scratch memory).
  auto store = [&](uint4* stage, const Segs<NSEG, SegT>& S, int c) {
#pragma unroll
    for (int i = 0; i < NSEG; ++i) {
      const uint32_t live = c * KSUB + sub[i] < nk64 ? 0xffffffffu : 0u;
      if constexpr (WF == DG_WS_W_E4M3) stage[slot[i]] = e4m3x8_to_bf16(S.v[i].x & live, S.v[i].y & live);
      else if constexpr (WF == DG_WS_W_MXFP4) stage[slot[i]] = mxfp4x8_to_bf16(S.v[i].x & live, S.v[i].y);
      else stage[slot[i]] = make_uint4(S.v[i].x & live, S.v[i].y & live, S.v[i].z & live, S.v[i].w & live);
    }
  };
  AFrags<MT, KSUB> F;
  auto fetch_a = [&](v8s (&A)[MT][2 * KSUB], int c) {
#pragma unroll
    for (int j = 0; j < MA; ++j)
#pragma unroll
      for (int q = 0; q < 2 * KSUB; ++q) {
        const int kc = min(c * KSUB + q / 2, nk64 - 1);
        if constexpr (GATHER) A[j][q] = *(const v8s*)(ap[j] + kc * 128 + (q & 1) * 64);  // row-major source row
        else A[j][q] = *(const v8s*)(ap[j] + (2 * kc + (q & 1)) * 1024);               // fragment-major block
      }
  };
  fetch(ring<0>(R), 0);
  fetch(ring<1>(R), 1);
  fetch(ring<2>(R), 2);
  fetch(ring<3>(R), 3);
  if constexpr (RING == 8) {
    fetch(ring<4>(R), 4);
    fetch(ring<5>(R), 5);
    fetch(ring<6>(R), 6);
    fetch(ring<7>(R), 7);
  }
  fetch_a(abuf<0>(F), 0);
  fetch_a(abuf<1>(F), 1);
  fetch_a(abuf<2>(F), 2);
  store(sW[0], ring<0>(R), 0);
  store(sW[1], ring<1>(R), 1);
  fetch(ring<0>(R), RING);
  fetch(ring<1>(R), RING + 1);
  __syncthreads();
  // Chunk c at position J = c % RING of the unrolled loop (c0 a multiple of RING).
  auto chunk = [&](auto JJ, int c) {
    constexpr int J = decltype(JJ)::value;
    constexpr int jr = J & 3;                  // LDS stage of chunk c (and its activation buffer)
    constexpr int ahead = (jr + 2) & 3;        // stage of chunk c + 2
    constexpr int rs = (J + 2) % RING;         // ring slot holding chunk c + 2
    fetch_a(abuf<(jr + 3) & 3>(F), c + 3);
    store(sW[ahead], ring<rs>(R), c + 2);
    fetch(ring<rs>(R), c + 2 + RING);
    if constexpr (MA > 0) {
      v8s(&acur)[MT][2 * KSUB] = abuf<jr>(F);
#pragma unroll
      for (int q = 0; q < 2 * KSUB; ++q) {
        v8s wf[NTN];
#pragma unroll
        for (int n = 0; n < NTN; ++n) {
          const uint4 u = sW[jr][lds_slot<KSUB>(n * 16 + (lane & 15), q * 4 + (lane >> 4))];
          wf[n] = *reinterpret_cast<const v8s*>(&u);
        }
#pragma unroll
        for (int j = 0; j < MA; ++j)
#pragma unroll
          for (int n = 0; n < NTN; ++n)
            acc[j][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(acur[j][q], wf[n], acc[j][n], 0, 0, 0);
      }
    }
    __syncthreads();
  };
  for (int c0 = 0; c0 < nchunk; c0 += RING) {
    chunk(std::integral_constant<int, 0>{}, c0);
    chunk(std::integral_constant<int, 1>{}, c0 + 1);
    chunk(std::integral_constant<int, 2>{}, c0 + 2);
    chunk(std::integral_constant<int, 3>{}, c0 + 3);
    if constexpr (RING == 8) {
      if (c0 + 4 >= nchunk) break;  // uniform; saves up to four padded chunks
      chunk(std::integral_constant<int, 4>{}, c0 + 4);
      chunk(std::integral_constant<int, 5>{}, c0 + 5);
      chunk(std::integral_constant<int, 6>{}, c0 + 6);
      chunk(std::integral_constant<int, 7>{}, c0 + 7);
    }
  }
}

template <int EPI, int NTN, int KSUB, int MT, bool GATHER, int RING, int WF = DG_WS_W_BF16>
__global__ void __launch_bounds__(NT) k_ws(WsArgs a) {
  static_assert(WF == DG_WS_W_BF16 || EPI == WS_EPI_SWIGLU || EPI == WS_EPI_STORE_F32,
                "E4M3 / MXFP4 weights: routed experts only");
  constexpr int BN = 16 * NTN;
  constexpr int PASS_ROWS = NWAVE * MT * 16;
  constexpr int NSEG = NTN * KSUB / 4;  // 16-byte segments per thread per chunk
  __shared__ uint4 sW[4][BN * 8 * KSUB];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int g = 0, nb = blockIdx.x, ms = 0, ks = 0;
  int part = -1;
  if (a.units) {
    if ((int)blockIdx.x >= *a.n_units) return;
    const uint32_t code = (uint32_t)a.units[blockIdx.x];
    if (code == DG_WS_UNIT_NONE) return;  // padding of the work list
    g = (int)(code >> 24);
    part = (int)((code >> 16) & 0xff);
    nb = (int)(code & 0xffff);
  } else if (a.msplit > 1 || a.ksplit > 1) {
    // Row and reduction split of a dense launch.  Work-groups are dealt to the 8
    // XCDs in turn (block b runs on XCD b % 8), so tile nb is given to XCD nb % 8
    // and its msplit x ksplit parts to consecutive slots of that XCD: the row
    // parts of one reduction range start together and share that XCD's L2, and
    // the tile crosses HBM once.  The grid is padded to 8 * ceil(nblk / 8) *
    // msplit * ksplit; padding blocks exit at once.
    // (an unset split count, 0, means 1)
    const int msp = max(a.msplit, 1), ksp = max(a.ksplit, 1);
    const int b = blockIdx.x, x = b % 8, j = b / 8, nsub = msp * ksp;
    const int sub = j % nsub;
    ks = sub / msp;
    ms = sub % msp;
    nb = x + 8 * (j / nsub);
    if (nb >= a.nblk) return;
  }
  int cnt = a.counts ? a.counts[g] : (a.M_dev ? *a.M_dev : a.M);
  int row0 = 0;
  if (part >= 0) {
    // Grouped launch: rows part * DG_WS_GROUP_ROWS .. + DG_WS_GROUP_ROWS - 1 of the group.
    row0 = part * DG_WS_GROUP_ROWS;
    cnt = min(cnt - row0, DG_WS_GROUP_ROWS);
  } else if (a.msplit > 1) {
    const int per = ((cnt + a.msplit - 1) / a.msplit + 15) / 16 * 16;
    row0 = ms * per;
    cnt = min(cnt - row0, per);
  }
  if (cnt <= 0) return;  // uniform over the block
  const int off = a.counts ? a.offsets[g] : 0;
  const int arow0 = a.counts ? a.offsets16[g] : 0;  // group's first row in the A matrix
  // 64-element sub-chunks of the reduction: this block's range of them
  const int kc0 = ks * a.kchunks;
  const int nk64 = a.ksplit > 1 ? min(a.K / 64 - kc0, a.kchunks) : a.K / 64;
  if (nk64 <= 0) return;  // uniform over the block

  // This thread's 16-byte segments of every weight chunk: segment id
  // tid + NT i -> weight row id / (8 KSUB), segment id % (8 KSUB) within the
  // chunk's KSUB * 128 bytes of that row (sub-chunk segment / 8).
  const char* gsrc[NSEG];
  const uint8_t* gsc[NSEG];  // MXFP4: the segment's scale byte (a segment is 8 weights of one 32-block)
  int slot[NSEG], sub[NSEG];
#pragma unroll
  for (int i = 0; i < NSEG; ++i) {
    const int sid = tid + NT * i, wr = sid / (8 * KSUB), sg = sid % (8 * KSUB);
    if constexpr (WF == DG_WS_W_E4M3) gsrc[i] = weight_row<EPI, NTN, 8>(a, g, nb, wr) + kc0 * 64 + (sg & 7) * 8;
    else if constexpr (WF == DG_WS_W_MXFP4) gsrc[i] = weight_row<EPI, NTN, 4>(a, g, nb, wr) + kc0 * 32 + (sg & 7) * 4;
    else gsrc[i] = weight_row<EPI, NTN>(a, g, nb, wr) + kc0 * 128 + (sg & 7) * 16;
    if constexpr (WF == DG_WS_W_MXFP4) gsc[i] = scale_row<EPI, NTN>(a, g, nb, wr) + kc0 * 2 + (sg & 7) / 4;
    else gsc[i] = nullptr;
    slot[i] = lds_slot<KSUB>(wr, sg);
    sub[i] = sg >> 3;
  }

  const int npass = (cnt + PASS_ROWS - 1) / PASS_ROWS;
  for (int pass = 0; pass < npass; ++pass) {
    const int pbase = pass * PASS_ROWS;
    // Activation rows of this wave's m-tiles (rows row0 + pbase + ... of the group).
    int mt_act = 0;
    const char* ap[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int t0 = pbase + (wave + NWAVE * j) * 16;
      if (t0 < cnt) mt_act = j + 1;
      if constexpr (GATHER) {
        // row-major source rows: lane l reads the token of sorted row (clamped to
        // the group's rows) l % 16 of the m-tile
        const int r = arow0 + row0 + min(t0 + (lane & 15), cnt - 1);
        ap[j] = (const char*)((const bf16_t*)a.A + (size_t)a.rowsrc[r] * a.K + kc0 * 64) + (lane >> 4) * 16;
      } else {
        // first row of this m-tile in the A matrix (a multiple of 16); a tile past
        // the end is read from the last one, which holds valid rows
        const int tr = arow0 + row0 + min(t0, (cnt - 1) & ~15);
        ap[j] = (const char*)a.A + ((size_t)(tr >> 4) * (a.K >> 5) + 2 * kc0) * 1024 + lane * 16;
      }
    }

    v4f acc[MT][NTN];
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
      for (int n = 0; n < NTN; ++n) acc[j][n] = v4f{0.f, 0.f, 0.f, 0.f};

    if (mt_act == 0) ws_stream<NTN, KSUB, MT, 0, GATHER, RING, WF>(sW, gsrc, gsc, slot, sub, ap, nk64, lane, acc);
    else if (MT == 1 || mt_act == 1)
      ws_stream<NTN, KSUB, MT, 1, GATHER, RING, WF>(sW, gsrc, gsc, slot, sub, ap, nk64, lane, acc);
    else ws_stream<NTN, KSUB, MT, MT, GATHER, RING, WF>(sW, gsrc, gsc, slot, sub, ap, nk64, lane, acc);

    // Epilogue.
    if constexpr (EPI == WS_EPI_LM_STATS) {
      // Per row over this block's BN vocabulary columns: max, sum exp(z - max),
      // sum exp(z - max) (z - max), and the argmax (lowest column among equal
      // maxima).  Lane holds columns n * 16 + lane % 16 of rows 4 (lane / 16) + i.
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        if (j >= mt_act) break;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float m = acc[j][0][i];
          int am = nb * BN + (lane & 15);
#pragma unroll
          for (int n = 1; n < NTN; ++n)
            if (acc[j][n][i] > m) {
              m = acc[j][n][i];
              am = nb * BN + n * 16 + (lane & 15);
            }
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) {
            const float om = __shfl_xor(m, o, 64);
            const int oa = __shfl_xor(am, o, 64);
            if (om > m || (om == m && oa < am)) { m = om; am = oa; }
          }
          float s = 0.f, t = 0.f;
#pragma unroll
          for (int n = 0; n < NTN; ++n) {
            const float z = acc[j][n][i] - m;
            const float e = __expf(z);
            s += e;
            t += e * z;
          }
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) {
            s += __shfl_xor(s, o, 64);
            t += __shfl_xor(t, o, 64);
          }
          const int rl = pbase + (wave + NWAVE * j) * 16 + (lane >> 4) * 4 + i;
          const int r = row0 + rl;
          if (a.zout && rl < cnt) {  // the logits themselves (self-conditioning)
            float* zr = a.zout + (size_t)r * a.N + nb * BN + (lane & 15);
#pragma unroll
            for (int n = 0; n < NTN; ++n) zr[n * 16] = acc[j][n][i];
          }
          if ((lane & 15) == 0 && rl < cnt) {
            const size_t pi = (size_t)r * a.ldo + nb;  // ldo = number of vocabulary tiles
            float* pp = (float*)a.out + pi * 3;
            pp[0] = m;
            pp[1] = s;
            pp[2] = t;
            a.part_arg[pi] = am;
          }
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        if (j >= mt_act) break;
        ws_tile_epilogue<EPI, NTN, WF>(a, acc[j], g, nb, row0, pbase + (wave + NWAVE * j) * 16, cnt, off, arow0, ks,
                                       lane);
      }
    }
    __syncthreads();  // the next pass reuses the LDS stages
  }
}

// Work lists of two grouped launches over the same groups.  A group with c rows
// is cut into ceil(c / DG_WS_GROUP_ROWS) row parts (one pass of the kernel each),
// and every (group, part, n-block) is one unit: group << 24 | part << 16 | n-block.
// Longest-first lists (k_wsd) are described with dg_sort_parts.  Else the list holds, for each part in group order, ceil8(nblk) slots, n-blocks in
// order and DG_WS_UNIT_NONE in the padding.  Work-groups are dealt to the 8 XCDs
// in turn (block u runs on XCD u % 8), so every part of n-block b of a group runs
// on XCD b % 8 and the parts after the first find that weight tile in its L2.
// One block; E <= 256.
__global__ void __launch_bounds__(256) k_ws_units(const int32_t* __restrict__ counts, int E, int part_rows,
                                                  int nblk_a,
                                                  int32_t* __restrict__ units_a, int32_t* __restrict__ n_a,
                                                  int nblk_b, int32_t* __restrict__ units_b,
                                                  int32_t* __restrict__ n_b, int lpt) {
  const int e = threadIdx.x;
  dg_build_lists(e, e < E ? counts[e] : 0, part_rows, nblk_a, units_a, n_a, nblk_b, units_b, n_b, lpt);
}

}  // namespace

// Register ring depth (chunks in flight per block).  Eight measured slower than
// four for every launch of the denoising step: the blocks are bound by the
// L2-to-CU traffic of their tiles, not by memory latency.
#ifndef DG_WS_RING_DENSE
#define DG_WS_RING_DENSE 4
#endif
#ifndef DG_WS_RING_ROUTED
#define DG_WS_RING_ROUTED 4
#endif
// E4M3 weights: a ring of 8 (the same bytes in flight as bf16's 4) needs more
// registers than two blocks per CU allow and measured slower.  MXFP4 keeps 4 too.
#ifndef DG_WS_RING_FP8
#define DG_WS_RING_FP8 4
#endif
#ifndef DG_WS_RING_FP4
#define DG_WS_RING_FP4 4
#endif
int dg_launch_ws(int epi, const WsArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return 0;
  constexpr int RD = DG_WS_RING_DENSE, RR = DG_WS_RING_ROUTED, R8 = DG_WS_RING_FP8, R4 = DG_WS_RING_FP4;
  constexpr int E8 = DG_WS_W_E4M3, F4 = DG_WS_W_MXFP4;
  if (a.counts) {  // grouped (routed experts)
    if (a.wfmt != DG_WS_W_BF16 && a.wfmt != E8 && a.wfmt != F4) return -1;
    if (a.wfmt == F4 && a.K % 64) return -1;  // whole 32-blocks per 64-element sub-chunk
    if (a.rowsrc && epi == WS_EPI_SWIGLU) {
      if (a.wfmt == E8) k_ws<WS_EPI_SWIGLU, 4, KSUB_PROJ, 1, true, R8, E8><<<grid, NT, 0, s>>>(a);
      else if (a.wfmt == F4) k_ws<WS_EPI_SWIGLU, 4, KSUB_PROJ, 1, true, R4, F4><<<grid, NT, 0, s>>>(a);
      else k_ws<WS_EPI_SWIGLU, 4, KSUB_PROJ, 1, true, RR><<<grid, NT, 0, s>>>(a);
    } else if (!a.rowsrc && epi == WS_EPI_STORE_F32) {
      if (a.wfmt == E8) k_ws<WS_EPI_STORE_F32, 4, KSUB_PROJ, 1, false, R8, E8><<<grid, NT, 0, s>>>(a);
      else if (a.wfmt == F4) k_ws<WS_EPI_STORE_F32, 4, KSUB_PROJ, 1, false, R4, F4><<<grid, NT, 0, s>>>(a);
      else k_ws<WS_EPI_STORE_F32, 4, KSUB_PROJ, 1, false, RR><<<grid, NT, 0, s>>>(a);
    } else return -1;
    return 0;
  }
  if (a.wfmt != DG_WS_W_BF16) return -1;  // E4M3 / MXFP4 weights: routed experts only
  switch (epi) {
    case WS_EPI_STORE_BF16: k_ws<WS_EPI_STORE_BF16, 4, KSUB_PROJ, 1, false, RD><<<grid, NT, 0, s>>>(a); break;
    case WS_EPI_STORE_F32: k_ws<WS_EPI_STORE_F32, 4, KSUB_PROJ, 1, false, RD><<<grid, NT, 0, s>>>(a); break;
    case WS_EPI_ADD_F32:
      // 128 output columns per block (half the activation re-reads of 64)
      if (a.wide && a.mt2) k_ws<WS_EPI_ADD_F32, 8, KSUB_PROJ, 2, false, RD><<<grid, NT, 0, s>>>(a);
      else if (a.wide) k_ws<WS_EPI_ADD_F32, 8, KSUB_PROJ, 1, false, RD><<<grid, NT, 0, s>>>(a);
      else k_ws<WS_EPI_ADD_F32, 4, KSUB_PROJ, 1, false, RD><<<grid, NT, 0, s>>>(a);
      break;
    // mt2: two m-tiles per wave (256 rows per pass) for launches with many rows
    case WS_EPI_SWIGLU:
      if (a.mt2) k_ws<WS_EPI_SWIGLU, 4, KSUB_PROJ, 2, false, RD><<<grid, NT, 0, s>>>(a);
      else k_ws<WS_EPI_SWIGLU, 4, KSUB_PROJ, 1, false, RD><<<grid, NT, 0, s>>>(a);
      break;
    case WS_EPI_ROPE_QKV:
      if (a.mt2) k_ws<WS_EPI_ROPE_QKV, 4, KSUB_PROJ, 2, false, RD><<<grid, NT, 0, s>>>(a);
      else k_ws<WS_EPI_ROPE_QKV, 4, KSUB_PROJ, 1, false, RD><<<grid, NT, 0, s>>>(a);
      break;
    // The LM head keeps two m-tiles per wave: up to 256 rows in one pass, so the
    // embedding crosses HBM once per step.
    case WS_EPI_LM_STATS: k_ws<WS_EPI_LM_STATS, 8, KSUB_LM, 2, false, 4><<<grid, NT, 0, s>>>(a); break;
    default: return -1;
  }
  return 0;
}

void dg_launch_ws_units(const int32_t* counts, int E, int part_rows, int nblk_a, int32_t* units_a, int32_t* n_a,
                        int nblk_b, int32_t* units_b, int32_t* n_b, hipStream_t s, int lpt) {
  k_ws_units<<<1, 256, 0, s>>>(counts, E, part_rows, nblk_a, units_a, n_a, nblk_b, units_b, n_b, lpt);
}
