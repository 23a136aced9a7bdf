// Mixture-of-experts kernels: top-k routing, token permutation, and the grouped
// expert projections on the matrix cores.
//
// The pages fix 128 experts with 8 routed plus 1 shared active per token
// ("DiffusionGemma Hits 1,000 Tokens per Second", section "The speed numbers and
// the hardware they require"; "Google open-sources DiffusionGemma", section "26B
// MoE Architecture, but Only 3.8B Activated").  At one 256-token canvas every
// expert receives ~16 rows per step, so each expert's weights are streamed from
// HBM exactly once per step and applied to all of its rows at once.
#include "dg_common.h"
#include "dg_kernels.h"
#include "gemm_core.h"

// ---------------------------------------------------------------------------
// Top-k: one block per row.  The k largest logits, ties to the lower expert id (a
// NaN logit ranks lowest): the rank of logit e is the number of logits that beat
// it under that order, and the entries of rank < k are the selection, in rank
// order.  The E x E comparisons are spread over the block as (logit, slice of 32
// logits) items and the partial ranks are summed in LDS.  gates = softmax over the k kept logits, summed in
// rank order (lanes 0 .. k - 1 of the first wave take one exponential each).
__global__ void __launch_bounds__(256) k_topk(float* __restrict__ logits, int rows, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ gates, int parts) {
  __shared__ __align__(16) float s_v[256];
  __shared__ int s_rank[256];
  __shared__ float s_sel[DG_MAX_TOPK];
  const int r = blockIdx.x, tid = threadIdx.x;
  float* lrow = logits + (size_t)r * E;
  if (tid < E) {
    // the router's partial sums over its reduction ranges, added in range
    // order (the first four loaded together); the total replaces the first
    // range's (what readers of the logits see)
    float v[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) v[p] = p < parts ? lrow[(size_t)p * rows * E + tid] : 0.f;
    float x = v[0];
#pragma unroll
    for (int p = 1; p < 4; ++p)
      if (p < parts) x += v[p];
    for (int p = 4; p < parts; ++p) x += lrow[(size_t)p * rows * E + tid];
    if (parts > 1) lrow[tid] = x;
    s_v[tid] = x == x ? x : -INFINITY;
  }
  s_rank[tid] = 0;
  __syncthreads();
  // work items (e, slice): E logits x ceil(E / 32) slices of 32 comparisons
  const int nsl = (E + 31) / 32;
  for (int it = tid; it < E * nsl; it += 256) {
    const int e = it % E, sl = it / E;
    const float v = s_v[e];
    const int j0 = sl * 32, j1 = min(j0 + 32, E);
    int cnt = 0;
    if (j1 - j0 == 32) {  // a whole slice: its 32 logits read as eight 16-byte loads before the comparisons
      float4 w4[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w4[u] = reinterpret_cast<const float4*>(s_v + j0)[u];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float ww[4] = {w4[u].x, w4[u].y, w4[u].z, w4[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int j = j0 + 4 * u + q;
          cnt += (int)(ww[q] > v) | ((int)(ww[q] == v) & (int)(j < e));  // bitwise: no short-circuit branches
        }
      }
    } else {
      for (int j = j0; j < j1; ++j) {
        const float w = s_v[j];
        cnt += (int)(w > v) | ((int)(w == v) & (int)(j < e));
      }
    }
    if (cnt) atomicAdd(&s_rank[e], cnt);
  }
  __syncthreads();
  if (tid < E && s_rank[tid] < k) {
    ids[(size_t)r * k + s_rank[tid]] = tid;
    s_sel[s_rank[tid]] = s_v[tid];
  }
  __syncthreads();
  if (tid < 64) {  // lane j < k: selected logit j's exponential; lane 0's order of the sum
    const float m = s_sel[0];
    const float ej = tid < k ? __expf(s_sel[tid] - m) : 0.f;
    float s = 0.f;
    for (int j = 0; j < k; ++j) s += __shfl(ej, j, 64);
    if (tid < k) gates[(size_t)r * k + tid] = ej / s;
  }
}

void dg_launch_topk(float* logits, int rows, int E, int k, int32_t* ids, float* gates, hipStream_t s, int parts) {
  if (rows <= 0) return;
  k_topk<<<rows, 256, 0, s>>>(logits, rows, E, k, ids, gates, parts < 1 ? 1 : parts);
}

// ---------------------------------------------------------------------------
// Router logits of the bf16 model: logits[r][e] = b[r] . Wg[e] in fp32 on the
// matrix cores.  A block computes one 16-row x 16-expert tile; its eight waves
// take an eighth of the reduction each, issue the loads of up to eight steps
// before their products (the steps are few, so their latency is what counts),
// alternate two accumulators, and the partial tiles are summed in LDS in wave
// order.  b is fragment-major (fm_index), Wg row-major [E][d]; d is a multiple
// of 64.
__global__ void __launch_bounds__(512) k_router(const bf16_t* __restrict__ b, int rows, int d,
                                                const bf16_t* __restrict__ wg, int E, float* __restrict__ logits,
                                                int ksplit) {
  __shared__ v4f s_part[8][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int net = (E + 15) >> 4, ntile = ((rows + 15) >> 4) * net;
  const int ks = blockIdx.x / ntile, tile = blockIdx.x % ntile;
  const int rt = tile / net, et = tile % net;
  const int nk = d >> 5;  // 32-element reduction steps
  // this block's reduction range (of ksplit), an eighth of it per wave; the
  // range's partial sums go to slab ks of logits
  const int r0 = ks * nk / ksplit, r1 = (ks + 1) * nk / ksplit;
  const int k0 = r0 + wave * (r1 - r0) / 8, k1 = r0 + (wave + 1) * (r1 - r0) / 8;
  logits += (size_t)ks * rows * E;
  const char* ap = (const char*)b + (size_t)rt * nk * 1024 + lane * 16;
  const int e = min(et * 16 + (lane & 15), E - 1);
  const char* bp = (const char*)(wg + (size_t)e * d) + (lane >> 4) * 16;
  v4f acc[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
  for (int kg = k0; kg < k1; kg += 8) {
    v8s a[8], w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kc = min(kg + j, k1 - 1);  // steps past the range are loaded but not used
      a[j] = *(const v8s*)(ap + (size_t)kc * 1024);
      w[j] = *(const v8s*)(bp + kc * 64);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (kg + j < k1) acc[j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], w[j], acc[j & 1], 0, 0, 0);
  }
  s_part[wave][lane] = acc[0] + acc[1];
  __syncthreads();
  if (wave == 0) {
    v4f t = s_part[0][lane];
#pragma unroll
    for (int q = 1; q < 8; ++q) t += s_part[q][lane];
    // lane holds rows 4 (lane / 16) + i, expert et * 16 + lane % 16
    const int col = et * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = rt * 16 + (lane >> 4) * 4 + i;
      if (row < rows && col < E) logits[(size_t)row * E + col] = t[i];
    }
  }
}

void dg_launch_router(const void* b_fm, int rows, int d, const void* wg, int E, float* logits, hipStream_t s,
                      int ksplit) {
  if (rows <= 0) return;
  ksplit = ksplit < 1 ? 1 : ksplit;
  k_router<<<((rows + 15) / 16) * ((E + 15) / 16) * ksplit, 512, 0, s>>>((const bf16_t*)b_fm, rows, d,
                                                                         (const bf16_t*)wg, E, logits, ksplit);
}

// ---------------------------------------------------------------------------
// Permutation: block e lists the pairs p = t*k + j routed to expert e in
// increasing p (token order), at perm[offsets[e] ...]; offsets[e] = number of
// pairs routed to experts < e.  Integer counting only: deterministic.
__global__ void __launch_bounds__(256) k_permute(const int32_t* __restrict__ ids, int npairs,
                                                 int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ perm) {
  const int e = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __shared__ int s_w[4];
  __shared__ int s_tot[2];
  int less = 0, mine = 0;
  for (int p = threadIdx.x; p < npairs; p += 256) {
    const int id = ids[p];
    less += id < e;
    mine += id == e;
  }
  // block sums of both counters
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    less += __shfl_xor(less, o, 64);
    mine += __shfl_xor(mine, o, 64);
  }
  __shared__ int s_less[4], s_mine[4];
  if (lane == 0) { s_less[wave] = less; s_mine[wave] = mine; }
  __syncthreads();
  if (threadIdx.x == 0) {
    s_tot[0] = s_less[0] + s_less[1] + s_less[2] + s_less[3];
    s_tot[1] = s_mine[0] + s_mine[1] + s_mine[2] + s_mine[3];
    counts[e] = s_tot[1];
    offsets[e] = s_tot[0];
  }
  __syncthreads();
  const int off = s_tot[0];
  int base = 0;
  for (int p0 = 0; p0 < npairs; p0 += 256) {
    const int p = p0 + threadIdx.x;
    const bool hit = p < npairs && ids[p] == e;
    const unsigned long long bal = __ballot(hit);
    const int rank = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_w[wave] = __popcll(bal);
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += s_w[w];
    if (hit) perm[off + base + wbase + rank] = p;
    base += s_w[0] + s_w[1] + s_w[2] + s_w[3];
    __syncthreads();
  }
}

void dg_launch_permute(const int32_t* ids, int rows, int E, int k, int32_t* counts, int32_t* offsets, int32_t* perm,
                       hipStream_t s) {
  if (rows <= 0) return;
  k_permute<<<E, 256, 0, s>>>(ids, rows * k, counts, offsets, perm);
}

// ---------------------------------------------------------------------------
// Everything after the top-k in one block of 16 waves: the expert histogram and
// offsets, the token permutation (as k_permute: the pairs of an expert in
// increasing pair index) and the two grouped work lists (dg_build_lists).  Expert
// e's rows are a bitmap over tokens; a token picks an expert at most once, so the
// rank of pair (t, e) among e's pairs is the number of e's tokens below t.  Also
// the expert-sorted row layout of the grouped launches: expert e's rows start at
// offsets16[e] (its predecessors' counts rounded up to 16); rowsrc[r] is the token
// of sorted row r (-1 on the padding rows), r < *n_srows.  rows <=
// DG_ROUTE_MAX_ROWS, E <= 256.
__global__ void __launch_bounds__(1024) k_route_tail(const int32_t* __restrict__ ids, int rows, int E, int k,
                                                     int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm, int32_t* __restrict__ offsets16,
                                                     int32_t* __restrict__ rowsrc, int32_t* __restrict__ n_srows,
                                                     int part_rows, int nblk_a,
                                                     int32_t* __restrict__ units_a, int32_t* __restrict__ n_a,
                                                     int nblk_b, int32_t* __restrict__ units_b,
                                                     int32_t* __restrict__ n_b, int lpt) {
  constexpr int WPE = DG_ROUTE_MAX_ROWS / 32;  // bitmap words per expert
  __shared__ uint32_t s_bits[256][WPE];
  __shared__ int s_off[256], s_off16[256];
  const int tid = threadIdx.x;
  const int nw = (rows + 31) / 32;
  for (int i = tid; i < 256 * nw; i += 1024) s_bits[i / nw][i % nw] = 0u;
  __syncthreads();
  const int npairs = rows * k;
  for (int p = tid; p < npairs; p += 1024) {
    const int t = p / k;
    atomicOr(&s_bits[ids[p]][t >> 5], 1u << (t & 31));
  }
  __syncthreads();
  int cnt = 0;
  if (tid < 256) {
    if (tid < E)
      for (int w = 0; w < nw; ++w) cnt += __popc(s_bits[tid][w]);
    s_off[tid] = cnt;
    s_off16[tid] = (cnt + 15) & ~15;
  }
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {  // inclusive scans over the experts
    int a = 0, c = 0;
    if (tid < 256 && tid >= o) {
      a = s_off[tid - o];
      c = s_off16[tid - o];
    }
    __syncthreads();
    if (tid < 256) {
      s_off[tid] += a;
      s_off16[tid] += c;
    }
    __syncthreads();
  }
  const int tot_rows16 = s_off16[255];
  __syncthreads();
  if (tid < 256) {  // exclusive: first position of expert tid
    s_off[tid] -= cnt;
    s_off16[tid] -= (cnt + 15) & ~15;
  }
  __syncthreads();
  if (tid < E) {
    counts[tid] = cnt;
    offsets[tid] = s_off[tid];
    offsets16[tid] = s_off16[tid];
    for (int r = cnt; r < ((cnt + 15) & ~15); ++r) rowsrc[s_off16[tid] + r] = -1;  // padding rows
  }
  if (tid == 0) *n_srows = tot_rows16;
  // work lists (longest first for k_wsd, else in expert order, padded)
  dg_build_lists(tid, cnt, part_rows, nblk_a, units_a, n_a, nblk_b, units_b, n_b, lpt);
  for (int p = tid; p < npairs; p += 1024) {
    const int e = ids[p], t = p / k, tw = t >> 5;
    int rank = __popc(s_bits[e][tw] & ((1u << (t & 31)) - 1u));
    for (int w = 0; w < tw; ++w) rank += __popc(s_bits[e][w]);
    perm[s_off[e] + rank] = p;
    rowsrc[s_off16[e] + rank] = t;
  }
}

// The expert-sorted row layout for the multi-kernel routing path (more rows than
// k_route_tail takes), from counts, offsets and perm: one block, E <= 256.
__global__ void __launch_bounds__(256) k_sorted_layout(const int32_t* __restrict__ counts,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ perm, int E, int k,
                                                       int32_t* __restrict__ offsets16, int32_t* __restrict__ rowsrc,
                                                       int32_t* __restrict__ n_srows) {
  __shared__ int s_off16[256];
  const int e = threadIdx.x;
  const int cnt = e < E ? counts[e] : 0, pad = (cnt + 15) & ~15;
  s_off16[e] = pad;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = e >= o ? s_off16[e - o] : 0;
    __syncthreads();
    s_off16[e] += v;
    __syncthreads();
  }
  if (e == 255) *n_srows = s_off16[255];
  if (e < E) {
    const int first = s_off16[e] - pad, off = offsets[e];
    offsets16[e] = first;
    for (int r = 0; r < pad; ++r) rowsrc[first + r] = r < cnt ? perm[off + r] / k : -1;
  }
}

void dg_launch_route(float* logits, int rows, int E, int k, int32_t* ids, float* gates, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* offsets16, int32_t* rowsrc, int32_t* n_srows,
                     int part_rows, int nblk_a, int32_t* units_a, int32_t* n_a, int nblk_b, int32_t* units_b,
                     int32_t* n_b, hipStream_t s, int lpt, int parts) {
  dg_launch_topk(logits, rows, E, k, ids, gates, s, parts);
  if (E + (rows * k + part_rows - 1) / part_rows > DG_WS_MAX_PARTS) lpt = 0;  // list order only
  if (rows <= DG_ROUTE_MAX_ROWS && E <= 256) {
    k_route_tail<<<1, 1024, 0, s>>>(ids, rows, E, k, counts, offsets, perm, offsets16, rowsrc, n_srows, part_rows,
                                    nblk_a, units_a, n_a, nblk_b, units_b, n_b, lpt);
    return;
  }
  dg_launch_permute(ids, rows, E, k, counts, offsets, perm, s);
  k_sorted_layout<<<1, 256, 0, s>>>(counts, offsets, perm, E, k, offsets16, rowsrc, n_srows);
  dg_launch_ws_units(counts, E, part_rows, nblk_a, units_a, n_a, nblk_b, units_b, n_b, s, lpt);
}

// The routing after the top-k, for rows <= DG_ROUTE_MAX_ROWS and E <= 256, in
// one launch with no global synchronisation (the one-block k_route_tail does
// the same work in sequence): every block rebuilds the expert histogram from
// all rows' expert ids (a bitmap over tokens per expert in LDS; the rank of
// pair (t, e) among e's pairs is the number of e's tokens below t), so each
// computes the same offsets on its own.  Block i < ceil(rows / 16) writes perm
// and rowsrc for the pairs of rows 16 i .. 16 i + 15; the last block writes
// counts, offsets, offsets16, rowsrc on the padding rows, *n_srows and both
// work lists (dg_build_lists).  The bitmap is in dynamic LDS: E x ceil(rows /
// 32) words.
__global__ void __launch_bounds__(256) k_route_perm(const int32_t* __restrict__ ids, int rows, int E, int k,
                                                    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ perm, int32_t* __restrict__ offsets16,
                                                    int32_t* __restrict__ rowsrc, int32_t* __restrict__ n_srows,
                                                    int part_rows, int nblk_a, int32_t* __restrict__ units_a,
                                                    int32_t* __restrict__ n_a, int nblk_b,
                                                    int32_t* __restrict__ units_b, int32_t* __restrict__ n_b,
                                                    int lpt) {
  extern __shared__ uint32_t s_bits[];  // [E][nw]
  __shared__ int s_cnt[256], s_off[256], s_off16[256], s_tot16;
  const int tid = threadIdx.x;
  const int nw = (rows + 31) / 32;
  for (int i = tid; i < E * nw; i += 256) s_bits[i] = 0u;
  __syncthreads();
  const int npairs = rows * k;
  // eight ids per thread loaded before their bits are set (one memory round
  // trip per eight pairs)
  for (int p0 = 0; p0 < npairs; p0 += 8 * 256) {
    int ev[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + u * 256 + tid;
      ev[u] = p < npairs ? ids[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + u * 256 + tid, t = p / k;
      if (ev[u] >= 0) atomicOr(&s_bits[ev[u] * nw + (t >> 5)], 1u << (t & 31));
    }
  }
  __syncthreads();
  int cnt = 0;
  if (tid < E)
    for (int w = 0; w < nw; ++w) cnt += __popc(s_bits[tid * nw + w]);
  s_cnt[tid] = cnt;
  __syncthreads();
  if (tid < 64) {
    // the first wave scans the experts, four per lane: exclusive offsets by
    // pairs and by 16-row tiles
    int c[4], a = 0, a16 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c[j] = s_cnt[4 * tid + j];
      a += c[j];
      a16 += (c[j] + 15) & ~15;
    }
    int ia = a, ia16 = a16;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int xa = __shfl_up(ia, o, 64), x16 = __shfl_up(ia16, o, 64);
      if (tid >= o) {
        ia += xa;
        ia16 += x16;
      }
    }
    int ea = ia - a, e16 = ia16 - a16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s_off[4 * tid + j] = ea;
      s_off16[4 * tid + j] = e16;
      ea += c[j];
      e16 += (c[j] + 15) & ~15;
    }
    if (tid == 63) s_tot16 = ia16;
  }
  __syncthreads();
  const int tot16 = s_tot16;

  if ((int)blockIdx.x < (rows + 15) / 16) {
    if (tid < 16 * k) {
      const int i = tid / k, j = tid - i * k, t = blockIdx.x * 16 + i;
      if (t < rows) {
        const int e = ids[t * k + j], tw = t >> 5;
        int rank = __popc(s_bits[e * nw + tw] & ((1u << (t & 31)) - 1u));
        for (int w = 0; w < tw; ++w) rank += __popc(s_bits[e * nw + w]);
        perm[s_off[e] + rank] = t * k + j;
        rowsrc[s_off16[e] + rank] = t;
      }
    }
    return;
  }
  // ---- the last block: counts, offsets, padding rows, work lists
  if (tid < E) {
    counts[tid] = cnt;
    offsets[tid] = s_off[tid];
    offsets16[tid] = s_off16[tid];
    for (int r = cnt; r < ((cnt + 15) & ~15); ++r) rowsrc[s_off16[tid] + r] = -1;  // padding rows
  }
  if (tid == 0) *n_srows = tot16;
  dg_build_lists(tid, tid < E ? cnt : 0, part_rows, nblk_a, units_a, n_a, nblk_b, units_b, n_b, lpt);
}

int dg_launch_route_perm(const int32_t* ids, int rows, int E, int k, int32_t* counts, int32_t* offsets, int32_t* perm,
                         int32_t* offsets16, int32_t* rowsrc, int32_t* n_srows, int part_rows, int nblk_a,
                         int32_t* units_a, int32_t* n_a, int nblk_b, int32_t* units_b, int32_t* n_b, int lpt,
                         hipStream_t s) {
  if (rows <= 0) return 0;
  if (rows > DG_ROUTE_MAX_ROWS || E > 256 || k > DG_MAX_TOPK || 16 * k > 256) return -1;
  if (E + (rows * k + part_rows - 1) / part_rows > DG_WS_MAX_PARTS) lpt = 0;  // list order only
  const size_t lds = (size_t)E * ((rows + 31) / 32) * 4;
  k_route_perm<<<(rows + 15) / 16 + 1, 256, lds, s>>>(ids, rows, E, k, counts, offsets, perm, offsets16, rowsrc,
                                                      n_srows, part_rows, nblk_a, units_a, n_a, nblk_b, units_b, n_b,
                                                      lpt);
  return 0;
}


// ---------------------------------------------------------------------------
// Expert up-projection with SwiGLU: for expert e's rows (pairs p, token t = p / k),
// h[p] = silu(W1_e b[t]) * (W3_e b[t]).  Block = (expert, 64 output columns); each
// of the 4 waves owns 16 columns (n-tile 0 from W1, n-tile 1 from W3) and all of
// the expert's rows, MT*16 rows per pass over the weights.
template <typename T, int MT>
__global__ void __launch_bounds__(256) k_expert_up(const T* __restrict__ b, int d, int k, int eh,
                                                   const T* __restrict__ w1, const T* __restrict__ w3,
                                                   const int32_t* __restrict__ counts,
                                                   const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ perm, T* __restrict__ h) {
  const int ntiles = eh / 64;
  const int e = blockIdx.x / ntiles, nt = blockIdx.x % ntiles;
  const int cnt = counts[e];
  if (cnt == 0) return;
  const int off = offsets[e];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = nt * 64 + wave * 16 + (lane & 15);
  const size_t wrow = (size_t)e * eh + c;
  const char* wp[2];
  for (int m0 = 0; m0 < cnt; m0 += MT * 16) {
    const int mt_active = min(MT, (cnt - m0 + 15) / 16);
    const char* ap[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = min(m0 + mt * 16 + (lane & 15), cnt - 1);
      const int t = perm[off + m] / k;
      ap[mt] = (const char*)(b + (size_t)t * d) + (lane >> 4) * 16;
    }
    wp[0] = (const char*)(w1 + wrow * d) + (lane >> 4) * 16;
    wp[1] = (const char*)(w3 + wrow * d) + (lane >> 4) * 16;
    v4f acc[MT][2];
    zero_acc(acc);
    mma_loop<T, MT, 2>(ap, wp, d / MF<T>::KC, mt_active, acc);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt >= mt_active) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + mt * 16 + (lane >> 4) * 4 + i;
        if (m < cnt) {
          const int p = perm[off + m];
          h[(size_t)p * eh + c] = from_f<T>(silu_f(acc[mt][0][i]) * acc[mt][1][i]);
        }
      }
    }
  }
}

// Expert down-projection: y[p] = W2_e h[p] (fp32), block = (expert, 64 columns of d).
template <typename T, int MT>
__global__ void __launch_bounds__(256) k_expert_down(const T* __restrict__ h, int d, int eh,
                                                     const T* __restrict__ w2, const int32_t* __restrict__ counts,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ perm, float* __restrict__ y) {
  const int ntiles = d / 64;
  const int e = blockIdx.x / ntiles, nt = blockIdx.x % ntiles;
  const int cnt = counts[e];
  if (cnt == 0) return;
  const int off = offsets[e];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = nt * 64 + wave * 16 + (lane & 15);
  const char* wp[1];
  for (int m0 = 0; m0 < cnt; m0 += MT * 16) {
    const int mt_active = min(MT, (cnt - m0 + 15) / 16);
    const char* ap[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = min(m0 + mt * 16 + (lane & 15), cnt - 1);
      const int p = perm[off + m];
      ap[mt] = (const char*)(h + (size_t)p * eh) + (lane >> 4) * 16;
    }
    wp[0] = (const char*)(w2 + ((size_t)e * d + c) * eh) + (lane >> 4) * 16;
    v4f acc[MT][1];
    zero_acc(acc);
    mma_loop<T, MT, 1>(ap, wp, eh / MF<T>::KC, mt_active, acc);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt >= mt_active) break;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + mt * 16 + (lane >> 4) * 4 + i;
        if (m < cnt) y[(size_t)perm[off + m] * d + c] = acc[mt][0][i];
      }
    }
  }
}

void dg_launch_expert_up(int dtype, const void* b, int rows, int d, int E, int k, int eh, const void* w1,
                         const void* w3, const int32_t* counts, const int32_t* offsets, const int32_t* perm, void* h,
                         hipStream_t s) {
  if (rows <= 0) return;
  const int blocks = E * (eh / 64);
  if (dtype == 1)
    k_expert_up<bf16_t, 2><<<blocks, 256, 0, s>>>((const bf16_t*)b, d, k, eh, (const bf16_t*)w1, (const bf16_t*)w3,
                                                  counts, offsets, perm, (bf16_t*)h);
  else
    k_expert_up<float, 2><<<blocks, 256, 0, s>>>((const float*)b, d, k, eh, (const float*)w1, (const float*)w3,
                                                 counts, offsets, perm, (float*)h);
}

void dg_launch_expert_down(int dtype, const void* h, int rows, int d, int E, int k, int eh, const void* w2,
                           const int32_t* counts, const int32_t* offsets, const int32_t* perm, float* y,
                           hipStream_t s) {
  if (rows <= 0) return;
  (void)k;
  const int blocks = E * (d / 64);
  if (dtype == 1)
    k_expert_down<bf16_t, 2><<<blocks, 256, 0, s>>>((const bf16_t*)h, d, eh, (const bf16_t*)w2, counts, offsets,
                                                    perm, y);
  else
    k_expert_down<float, 2><<<blocks, 256, 0, s>>>((const float*)h, d, eh, (const float*)w2, counts, offsets, perm,
                                                   y);
}
