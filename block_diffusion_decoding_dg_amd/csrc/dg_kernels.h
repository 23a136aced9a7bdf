// Host-side launchers of the libdg kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define DG_MAX_SEGS 16

// One request's share of a batch of rows: rows [row0, row0 + n) of the batch sit at
// absolute positions pos0 .. pos0 + n - 1 and attend to keys [0, nkeys) of the
// request's cache of the current layer (K: [Hkv][max_ctx][hd], V: [Hkv][hd][max_ctx]).
struct DgSeg {
  void* k;
  void* vt;
  int32_t row0, n, pos0, nkeys;
};
struct DgSegs {
  DgSeg s[DG_MAX_SEGS];
  int32_t count;
  int32_t causal;
};

struct DgShape {
  int32_t d, hq, hkv, hd, max_ctx, vocab;
};

#define DG_MAX_TOPK 16  // routed experts per token, at most
#define DG_ROUTE_MAX_ROWS 2048  // rows of the one-block routing tail and of the routing scatter, at most

// dtype: 0 = f32, 1 = bf16 (weights, activations and cache).
void dg_launch_embed(int dtype, const int32_t* ids, int rows, const void* embed, int d, int vocab, float* x,
                     hipStream_t s);
struct DgSampleArgs;
void dg_launch_embed_slots(int dtype, const DgSampleArgs& a, const void* embed, int d, float* x, hipStream_t s);
// Pending partial sums of a split-reduction add projection: n ranges of
// [rows][d] fp32, range k at p + k * stride; folded into x by the next row kernel.
struct DgParts {
  const float* p = nullptr;
  int n = 0;
  size_t stride = 0;
};
// fm: bf16 output in the fragment-major layout (fm_index) instead of row-major;
// out_rm (optional, bf16): a second, row-major copy; parts: folded into x first
// (x is then written back).  Returns -1 (nothing launched) for partial sums
// without the bf16 fragment-major output, else 0.
int dg_launch_rmsnorm(int dtype, const float* x, const int32_t* row_idx, const int32_t* n_dev, int rows, int d,
                      const void* gain, float eps, void* out, bool fm, hipStream_t s, void* out_rm = nullptr,
                      const DgParts& parts = DgParts{});

// y = A W^T; mode 0: store in dtype, 1: store fp32, 2: add into fp32 out.
void dg_launch_gemm(int dtype, int mode, const void* A, int M, int K, const void* W, int N, void* out, int ldo,
                    hipStream_t s);
void dg_launch_qkv(int dtype, const void* A, int M, const DgShape& sh, const void* wq, const void* wk, const void* wv,
                   const DgSegs& segs, const double* inv_freq, void* q_out, hipStream_t s);
void dg_launch_swiglu(int dtype, const void* A, int M, int K, const void* w1, const void* w3, int N, void* h_out,
                      hipStream_t s);
// Attention: q [rows][hq*hd] (dtype), output o [rows][hq*hd] (dtype).  Uses the
// split-KV partial buffers (fp32): opart [nsplit][rows*hq][hd], mlpart [nsplit][rows*hq][2].
// Query rows per block of the attention kernel (dtype 1: bf16), and the key
// splits for a launch (about one block per CU, at least 8 key tiles per split).
int dg_attn_qrows(int dtype, int hd);
int dg_attn_splits(const DgSegs& segs, const DgShape& sh, int max_splits, int qrows);
void dg_launch_attention(int dtype, const void* q, const DgShape& sh, const DgSegs& segs, int nsplit, float* opart,
                         float* mlpart, void* o, int rows, hipStream_t s);
// Router top-k: logits [rows][E] fp32 -> ids [rows][k], gates [rows][k].
// parts > 1: logits holds that many slabs [parts][rows][E] of partial sums,
// added in slab order; their total is written over slab 0.
void dg_launch_topk(float* logits, int rows, int E, int k, int32_t* ids, float* gates, hipStream_t s, int parts = 1);
// bf16 router logits [rows][E] fp32 from the fragment-major normalised rows (d a multiple of 64); with
// ksplit > 1 the reduction is split into that many ranges, slab ks of logits ([ksplit][rows][E]) holding
// range ks's partial sums (dg_launch_topk adds them).
void dg_launch_router(const void* b_fm, int rows, int d, const void* wg, int E, float* logits, hipStream_t s,
                      int ksplit = 1);
// Permutation: counts[E], offsets[E], perm[rows*k] (pair index t*k + j, token order per expert).
void dg_launch_permute(const int32_t* ids, int rows, int E, int k, int32_t* counts, int32_t* offsets, int32_t* perm,
                       hipStream_t s);
// Router top-k, histogram, offsets, permutation, the expert-sorted row layout
// (offsets16[e]: first row of expert e, 16-aligned; rowsrc[r]: token of sorted row
// r, -1 on padding rows, for r < *n_srows) and both grouped work lists
// (dg_launch_ws_units; lpt: longest-first lists for k_wsd); everything after
// the top-k in one block for rows <= 2048.
void dg_launch_route(float* logits, int rows, int E, int k, int32_t* ids, float* gates, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* offsets16, int32_t* rowsrc, int32_t* n_srows,
                     int part_rows, int nblk_a, int32_t* units_a, int32_t* n_a, int nblk_b, int32_t* units_b,
                     int32_t* n_b, hipStream_t s, int lpt = 0, int parts = 1);
// The routing after the top-k in one launch of parallel blocks (rows <= 2048,
// E <= 256; as k_route_tail): counts, offsets, perm, the expert-sorted layout
// (offsets16, rowsrc) and both work lists (lpt: longest first).  Returns -1
// (nothing launched) outside those limits.
int dg_launch_route_perm(const int32_t* ids, int rows, int E, int k, int32_t* counts, int32_t* offsets, int32_t* perm,
                         int32_t* offsets16, int32_t* rowsrc, int32_t* n_srows, int part_rows, int nblk_a,
                         int32_t* units_a, int32_t* n_a, int nblk_b, int32_t* units_b, int32_t* n_b, int lpt,
                         hipStream_t s);
// Rows of the expert-sorted layout: pairs + 16 per expert.
inline int dg_sorted_rows(int E, int pairs) { return pairs + 16 * E; }
// Routed experts: up (SwiGLU) into h [rows*k][eh] (dtype), down into y [rows*k][d] fp32.
void dg_launch_expert_up(int dtype, const void* b, int rows, int d, int E, int k, int eh, const void* w1,
                         const void* w3, const int32_t* counts, const int32_t* offsets, const int32_t* perm, void* h,
                         hipStream_t s);
void dg_launch_expert_down(int dtype, const void* h, int rows, int d, int E, int k, int eh, const void* w2,
                           const int32_t* counts, const int32_t* offsets, const int32_t* perm, float* y,
                           hipStream_t s);
// x[t] += sum_j gates[t][j] * y[t*k + j]
// x[t] += sum_j gates[t][j] y[t k + j] for every row, then (gain given) the
// RMSNorm of the updated rows into out (model dtype).  d <= 16384, k <= 16.
// Returns -1 (nothing launched) for partial sums without the bf16
// fragment-major output, else 0.
int dg_launch_combine_norm(int dtype, float* x, const float* y, const float* gates, int rows, int d, int k,
                           const void* gain, float eps, void* out, bool fm, hipStream_t s,
                           const DgParts& parts = DgParts{});
// LM head over rows of hn [n][d] (dtype), n from n_dev (<= max_rows): partials then merge.
void dg_launch_lm_head(int dtype, const void* hn, const int32_t* n_dev, int max_rows, int d, const void* embed,
                       int vocab, float* part, int32_t* part_arg, float* ent, float* lse, int32_t* amax,
                       const int32_t* row_idx, hipStream_t s);
int dg_lm_head_tiles(int vocab);
// Tile merge of the LM-head partials alone (part [rows][n_tiles][3], part_arg [rows][n_tiles]).
void dg_launch_lm_merge(const float* part, const int32_t* part_arg, const int32_t* n_dev, int max_rows, int n_tiles,
                        const int32_t* row_idx, float* ent, float* lse, int32_t* amax, hipStream_t s);
// Sampler over a batch of canvases (one per slot).
struct DgSampleSlot {
  int32_t* ids;       // canvas ids [C]
  uint8_t* accepted;  // [C]
  int32_t* prev;      // argmax canvas of the block's previous step [C]; -1 = none
  uint64_t seed;
  int32_t block, step, row0;
};
struct DgSampleArgs {
  DgSampleSlot s[DG_MAX_SEGS];
  int32_t count, C, vocab, max_steps;
  float tau;
  int32_t mode;               // DG_SAMPLER_THRESHOLD / DG_SAMPLER_BUDGET
  uint64_t budget_q, stop_q;  // fixed-point budget and stop threshold (2^-40 nat units)
};
// ent/amax indexed by batch row (slot * C + pos).  info [count][4]: accepted, forced, open, done.
// open_rows/n_open_rows: compacted list of batch rows still open after the step.
void dg_launch_sample(const DgSampleArgs& a, const float* ent, const int32_t* amax, int32_t* info,
                      int32_t* open_rows, int32_t* n_open_rows, hipStream_t s);
// Canvas start: draw every position at step 0, clear accepted; also builds the open-row list.
void dg_launch_canvas_init(const DgSampleArgs& a, int32_t* open_rows, int32_t* n_open_rows, hipStream_t s);
// Open-row list from the accepted flags (used after state injection).
void dg_launch_open_rows(const DgSampleArgs& a, int32_t* open_rows, int32_t* n_open_rows, hipStream_t s);
void dg_launch_philox_tokens(uint64_t seed, int block, int step, int n, int vocab, int32_t* out, hipStream_t s);
// Gather rows by index list into a compact fp32 buffer (used by the logits tap).
void dg_launch_gather_rows(const float* x, const int32_t* idx, int n, int d, float* out, hipStream_t s);

// ---------------------------------------------------------------------------
// Self-conditioning (bf16 models).  DgScSlots: the state rows ([C][d] fp32) of
// the request in each slot of the step.
struct DgScSlots {
  float* state[DG_MAX_SEGS];
};
// ET [d][V] = E^T for E [V][d] bf16 (V, d multiples of 64).
// Returns -1 (nothing launched) unless V and d are multiples of 64.
int dg_launch_transpose_bf16(const void* E, int V, int d, void* ET, hipStream_t s);
// P (bf16, fragment-major [rows][V]) = exp(z - lse[row_idx[r]]) for rows r < *n_dev of z (fp32 [rows][V]).
void dg_launch_sc_probs(const float* z, const float* lse, const int32_t* row_idx, const int32_t* n_dev,
                        int max_rows, int V, void* P, hipStream_t s);
// State rows of compacted rows r < *n_dev (canvas row row_idx[r]) = sum over the nks
// ranges of parts ([nks][rows][d] fp32, range k at parts + k * stride).
// Returns -1 (nothing launched) unless d is a multiple of 4.
int dg_launch_sc_fold(const float* parts, int nks, size_t stride, int d, const int32_t* row_idx,
                      const int32_t* n_dev, int max_rows, const DgScSlots& sl, int C, hipStream_t s);
// b (bf16, fragment-major [rows][d]) = the state of canvas row t = slot * C + position.
void dg_launch_sc_gather(const DgScSlots& sl, int rows, int C, int d, void* b, hipStream_t s);
// b (bf16, fragment-major [n][d]) = u (fp32 row-major [n][d]).
void dg_launch_rows_to_fm(const float* u, int n, int d, void* b, hipStream_t s);
void dg_launch_fill_zero(float* p, size_t n, hipStream_t s);
// *p = v, written by a kernel on the stream.
void dg_launch_set_i32(int32_t* p, int32_t v, hipStream_t s);

// ---------------------------------------------------------------------------
// Weight-streaming GEMM (bf16 only): out = A W^T per group, 64 weight rows per
// block and every activation row of the group (256 per pass over the weights).
enum {
  WS_EPI_STORE_BF16 = 0,  // out bf16 [rows][ldo]
  WS_EPI_STORE_F32 = 1,   // out fp32 [rows][ldo]
  WS_EPI_ADD_F32 = 2,     // out fp32 [rows][ldo] +=
  WS_EPI_SWIGLU = 3,      // W0 = W1, W1 = W3; 32 hidden columns per block; out bf16 silu(x W1^T) * (x W3^T)
  WS_EPI_ROPE_QKV = 4,    // W0/W1/W2 = wq/wk/wv; RoPE on q and k; q to out, k and v to the cache of segs
  WS_EPI_LM_STATS = 5     // 128 vocabulary rows per block; per (row, block): (max, sum exp, sum exp * z) to out
                          // fp32 [rows][ldo][3] and the argmax to part_arg [rows][ldo] (ldo = vocab / 128)
};

// Storage of grouped (routed-expert) weights.
enum {
  DG_WS_W_BF16 = 0,   // bf16, two bytes per weight
  DG_WS_W_E4M3 = 1,   // OCP E4M3 codes, one byte per weight, with a float32 scale per weight row
  DG_WS_W_MXFP4 = 2   // OCP MX FP4 (E2M1) codes, two per byte (lower k in the low nibble), with an
                      // E8M0 scale per 32 consecutive weights of a row
};

struct WsArgs {
  const void* A;          // activation rows, bf16, fragment-major with K columns (fm_index)
  const void* W0;         // weight matrices, row-major [rows][K]
  const void* W1;
  const void* W2;
  int wfmt;               // grouped launches: DG_WS_W_* storage of W0 / W1
  const float* wsc0;      // DG_WS_W_E4M3: float32 scales per weight row, [groups][N], of W0
  const float* wsc1;      // and of W1
  const uint8_t* wbs0;    // DG_WS_W_MXFP4: E8M0 scales per 32 weights, [groups][N][K / 32], of W0
  const uint8_t* wbs1;    // and of W1
  size_t wgs;             // elements between the matrices of consecutive groups
  int K;                  // reduction length, multiple of 64
  int N;                  // weight rows per group (SwiGLU: hidden width); stores are masked to it
  int M;                  // rows of the single group when counts is null
  const int32_t* M_dev;   // if set (and counts null): the row count, read on the device
  int span;               // k_wsd: n-blocks per unit of the work list (0 = 1), swept in turn
  int msplit;             // dense launches: row ranges per n-block; 0 or 1 = none
  int ksplit;             // dense add launches: reduction ranges per n-block (partial sums); 0 or 1 = none
  int kchunks;            // with ksplit: 64-element chunks of the reduction per range
  float* part_out;        // with ksplit: partial sums [ksplit][rows][ldo] (fp32), range k at part_out + k * part_stride
  size_t part_stride;
  int wide;               // add launches: 128 output columns per block instead of 64
  int mt2;                // dense launches (wide add, SwiGLU, q/k/v): two m-tiles per wave (256 rows per pass)
  int nblk;               // dense launches: number of n-blocks
  const int32_t* counts;  // grouped: rows per group
  const int32_t* offsets; // grouped: first position of each group in perm
  const int32_t* perm;    // grouped: pair index of each sorted row (the output row of a fp32 store)
  const int32_t* offsets16;  // grouped: first row of each group in A (and a SwiGLU output), 16-aligned
  const int32_t* rowsrc;  // grouped, optional: A is row-major and sorted row r reads A row rowsrc[r]
  const int32_t* units;   // grouped: work list (group << 24 | part << 16 | n-block), length *n_units
  const int32_t* n_units;
  void* out;
  int ldo;
  int32_t* part_arg;      // LM-head argmax partials
  float* zout;            // LM head, optional: the logits, fp32 [rows][N] (compacted rows)
  // q/k/v epilogue
  int hd, hq, hkv, max_ctx;
  const double* inv_freq;
  DgSegs segs;
};

// Grouped launches: rows per unit of work (one pass of the kernel), and the
// code of an empty slot of a work list.
#ifndef DG_WS_GROUP_ROWS
#define DG_WS_GROUP_ROWS 128
#endif
#define DG_WS_UNIT_NONE 0xffffffffu
// Rows per part of the routed k_wsd launches (two m-tiles per consumer wave).
#define DG_WSD_PART_ROWS 256

// Writes the work-list entries of group e's `parts` row parts, starting at part
// slot `first`: ceil8(nblk) entries per part, n-blocks in order, then padding.
__device__ __forceinline__ void dg_fill_units(int32_t* __restrict__ units, int first, int parts, int e, int nblk) {
  const int stride = (nblk + 7) & ~7;
  for (int p = 0; p < parts; ++p)
    for (int b = 0; b < stride; ++b)
      units[(first + p) * stride + b] = b < nblk ? (int32_t)(((uint32_t)e << 24) | ((uint32_t)p << 16) | (uint32_t)b)
                                                 : (int32_t)DG_WS_UNIT_NONE;
}

// Longest-first work lists (k_wsd).  A block's time grows with the rows of its
// part (more consumer waves load activations and run the matrix cores), and
// blocks start in list order, so the list holds the parts in decreasing order
// of their tile class -- 16-row tiles, counted in pairs for parts of more than
// 128 rows, so that 8 classes cover a part -- (ties: expert order, then part
// order) and each part's
// n-blocks (or spans of n-blocks) side by side: the last blocks to start are
// the shortest, and the launch ends with fewer CUs idle.
//
// dg_sort_parts: called by every thread of a block of at least 256 threads;
// thread e < 256 passes expert e's row count (0 for e >= E).  Writes part q of
// the order to plist[q] as expert << 8 | part and returns the number of parts.
// s_scan: 256 entries of LDS scratch; plist: LDS, room for E + pairs / part_rows.
#define DG_WS_MAX_PARTS 512  // parts a longest-first list can hold (E + pairs / part_rows)
__device__ __forceinline__ int dg_sort_parts(int e, int cnt, int part_rows, ulonglong2* s_scan, int32_t* plist) {
  // per expert: full parts and a shorter last part, as 16-bit counts per tile
  // class (classes 1..4 in x, 5..8 in y; tpc tiles per class)
  const int tiles_full = (part_rows + 15) / 16, tpc = (tiles_full + 7) / 8;
  const int parts = cnt > 0 ? (cnt + part_rows - 1) / part_rows : 0;
  const int rlast = cnt - (parts - 1) * part_rows, wl = min(((rlast + 15) / 16 + tpc - 1) / tpc, 8);
  const int full = parts > 0 ? parts - 1 + (rlast == part_rows) : 0;
  auto add = [](ulonglong2& v, int cls, unsigned long long n) {
    if (cls <= 4) v.x += n << (16 * (cls - 1));
    else v.y += n << (16 * (cls - 5));
  };
  auto get = [](const ulonglong2& v, int cls) -> int {
    return (int)((cls <= 4 ? v.x >> (16 * (cls - 1)) : v.y >> (16 * (cls - 5))) & 0xffff);
  };
  ulonglong2 own = make_ulonglong2(0ull, 0ull);
  if (e < 256) {
    if (full) add(own, min((tiles_full + tpc - 1) / tpc, 8), (unsigned long long)full);
    if (parts > 0 && rlast != part_rows) add(own, wl, 1ull);
    s_scan[e] = own;
  }
  __syncthreads();
  if (e < 64) {
    // inclusive scan over the experts, field by field (no field carries into
    // the next: each is at most the part count), by the first wave, four
    // experts per lane
    ulonglong2 v[4];
    unsigned long long ax = 0ull, ay = 0ull;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = s_scan[4 * e + j];
      ax += v[j].x;
      ay += v[j].y;
    }
    unsigned long long ix = ax, iy = ay;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const unsigned long long xx = __shfl_up(ix, o, 64), yy = __shfl_up(iy, o, 64);
      if (e >= o) {
        ix += xx;
        iy += yy;
      }
    }
    unsigned long long ex = ix - ax, ey = iy - ay;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ex += v[j].x;
      ey += v[j].y;
      s_scan[4 * e + j] = make_ulonglong2(ex, ey);
    }
  }
  __syncthreads();
  const ulonglong2 tot = s_scan[255];
  if (e < 256 && parts > 0) {
    const ulonglong2 inc = s_scan[e];
    const ulonglong2 exc = make_ulonglong2(inc.x - own.x, inc.y - own.y);
    auto first_of = [&](int cls) {  // classes in decreasing order
      int f = 0;
      for (int k = 8; k > cls; --k) f += get(tot, k);
      return f;
    };
    const int cf = min((tiles_full + tpc - 1) / tpc, 8);
    for (int p = 0; p < full; ++p) plist[first_of(cf) + get(exc, cf) + p] = (e << 8) | p;
    if (rlast != part_rows) plist[first_of(wl) + get(exc, wl) + (wl == cf ? full : 0)] = (e << 8) | (parts - 1);
  }
  int n = 0;
  for (int k = 1; k <= 8; ++k) n += get(tot, k);
  __syncthreads();
  return n;
}

// Both grouped work lists from the experts' row counts, in one block of at least
// 256 threads (thread e < 256 passes expert e's count, 0 for e >= E): longest first
// (lpt, dg_sort_parts; unit u is n-block u % nblk of part u / nblk, no padding)
// or in expert order with each part's units padded to ceil8(nblk)
// (dg_fill_units).  Writes the list lengths to *n_a, *n_b.
__device__ __forceinline__ void dg_build_lists(int e, int cnt, int part_rows, int nblk_a, int32_t* __restrict__ units_a,
                                               int32_t* __restrict__ n_a, int nblk_b,
                                               int32_t* __restrict__ units_b, int32_t* __restrict__ n_b, int lpt) {
  __shared__ ulonglong2 s_sc[256];
  __shared__ int32_t s_plist[DG_WS_MAX_PARTS];
  if (lpt) {
    const int np = dg_sort_parts(e, cnt, part_rows, s_sc, s_plist);
    for (int q = e; q < np; q += blockDim.x) {  // a thread per part: its n-blocks in both lists
      const int ep = s_plist[q];
      const uint32_t code = ((uint32_t)(ep >> 8) << 24) | ((uint32_t)(ep & 0xff) << 16);
      for (int b = 0; b < nblk_a; ++b) units_a[q * nblk_a + b] = (int32_t)(code | (uint32_t)b);
      for (int b = 0; b < nblk_b; ++b) units_b[q * nblk_b + b] = (int32_t)(code | (uint32_t)b);
    }
    if (e == 0) {
      *n_a = np * nblk_a;
      *n_b = np * nblk_b;
    }
    return;
  }
  int* s_scan = (int*)s_sc;  // 256 ints
  const int parts = cnt > 0 ? (cnt + part_rows - 1) / part_rows : 0;
  if (e < 256) s_scan[e] = parts;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    const int v = e < 256 && e >= o ? s_scan[e - o] : 0;
    __syncthreads();
    if (e < 256) s_scan[e] += v;
    __syncthreads();
  }
  if (e < 256) {
    const int before = s_scan[e] - parts;  // exclusive prefix
    dg_fill_units(units_a, before, parts, e, nblk_a);
    dg_fill_units(units_b, before, parts, e, nblk_b);
  }
  if (e == 255) {
    *n_a = s_scan[255] * ((nblk_a + 7) & ~7);
    *n_b = s_scan[255] * ((nblk_b + 7) & ~7);
  }
}

// Returns 0, or -1 for a configuration the kernels do not implement (nothing launched).
int dg_launch_ws(int epi, const WsArgs& a, int grid, hipStream_t s);

// Slots of a grouped work list: parts * ceil8(nblk), where parts <= E +
// pairs / part_rows bounds the number of (group, row part) pairs.
inline int dg_unit_slots(int E, int pairs, int part_rows, int nblk) {
  return (E + (pairs + part_rows - 1) / part_rows) * ((nblk + 7) & ~7);
}
// Grouped launch of bf16 routed-expert weights with producer waves copying the
// weight tiles straight into LDS and consumer waves on the matrix cores (k_wsd):
// SwiGLU (W1 / W3; A row-major, its sorted rows read through rowsrc when set)
// or an fp32 store (W2; A fragment-major at the expert-sorted rows), on the work list
// of a.units (DG_WSD_PART_ROWS rows per part, a.span n-blocks per unit).  The
// SwiGLU output is fragment-major at the expert-sorted rows.  Returns -1 (nothing
// launched) for any other combination.
int dg_launch_wsd(int epi, const WsArgs& a, int grid, hipStream_t s);
// Weight rows per n-block of dg_launch_wsd for epilogue epi (64 or 128).
int dg_wsd_bn(int epi);
// n-blocks per unit of dg_launch_wsd for epilogue epi (a.span must not exceed it).
int dg_wsd_span(int epi);
// Dense launch of k_wsd: one bf16 weight matrix (a.W0, q/k/v: a.W0..W2; SwiGLU:
// W1 = a.W0, W3 = a.W1) on a.M fragment-major rows, a.nblk n-blocks of 64
// weight rows, a.msplit parts of DG_WS_GROUP_ROWS rows (covering a.M), and for
// WS_EPI_ADD_F32 optionally a.ksplit reduction ranges of a.kchunks chunks
// (partial sums into a.part_out); the epilogues of k_ws.  Returns -1 (nothing
// launched) for any other combination.
int dg_launch_wsd_dense(int epi, const WsArgs& a, hipStream_t s);

// Work lists of two grouped launches over the same groups (n-blocks per group nblk_a / nblk_b;
// lpt: longest-first lists for k_wsd, nblk then counting spans); each list needs
// dg_unit_slots(E, rows * k, part_rows, nblk) entries.
void dg_launch_ws_units(const int32_t* counts, int E, int part_rows, int nblk_a, int32_t* units_a, int32_t* n_a,
                        int nblk_b, int32_t* units_b, int32_t* n_b, hipStream_t s, int lpt = 0);
