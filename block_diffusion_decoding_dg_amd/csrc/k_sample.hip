// Entropy-bound sampler, canvas start and the open-row list.
//
// "DiffusionGemma hits ~1,500 TPS on one H100", section "How the sampler
// actually works": each step picks a candidate at every position, accepts the
// confident positions, re-randomizes the rest and stops when the canvas has
// converged or at the step cap.  Candidate = argmax token in both modes; at the
// step cap every open position is accepted with its argmax; the rest are
// re-drawn from Philox.  Two accept rules:
//  * threshold (a stated reading where the pages leave the rule open): open
//    positions with entropy < tau (fp32) plus the single open position of
//    lowest entropy (ties to the lower position);
//  * budget (the pages' default sampler, as read here): open positions in
//    order of rising entropy while the running entropy sum, own term included,
//    stays within the budget, the first always; early stop when the argmax
//    canvas repeats the block's previous one and the open positions' mean
//    entropy is below the stop threshold.  Entropies enter as 64-bit fixed
//    point (2^-40 nat units), so every sum is exact and independent of order:
//    each thread sums the terms of the positions ranked at or before its own.
#include "dg_common.h"
#include "dg_kernels.h"

// Order-preserving key of a float (any sign) in the high word, position in the low word.
__device__ __forceinline__ uint64_t ent_key(float h, int pos) {
  uint32_t b = __float_as_uint(h);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint32_t)pos;
}

__device__ __forceinline__ uint64_t block_min_u64(uint64_t v, uint64_t* s_red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t w = __shfl_xor(v, o, 64);
    v = w < v ? w : v;
  }
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  uint64_t r = s_red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = s_red[i] < r ? s_red[i] : r;
  __syncthreads();
  return r;
}

__device__ __forceinline__ int block_sum_i(int v, int* s_red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  int r = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r += s_red[i];
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, uint64_t* s_red) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  uint64_t r = 0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r += s_red[i];
  __syncthreads();
  return r;
}

// floor(clamp(h, 0, 64) * 2^40), NaN as 64: exact in double, truncation = floor.
__device__ __forceinline__ uint64_t ent_fixed(float h) {
  h = h >= 0.f ? fminf(h, 64.f) : (h < 0.f ? 0.f : 64.f);
  return (uint64_t)((double)h * 1099511627776.0);
}

// One block of C threads; slots processed in order.  info[slot] = {accepted by the
// entropy rule, forced at the cap or by the early stop, still open, done}.
__global__ void __launch_bounds__(256) k_sample(DgSampleArgs a, const float* __restrict__ ent,
                                                const int32_t* __restrict__ amax, int32_t* __restrict__ info) {
  __shared__ uint64_t s_red64[4];
  __shared__ int s_red[4];
  __shared__ uint64_t s_key[256], s_q[256];
  const int pos = threadIdx.x;
  const bool budget = a.mode == 1;
  for (int si = 0; si < a.count; ++si) {
    const DgSampleSlot sl = a.s[si];
    const int row = sl.row0 + pos;
    const bool was_acc = sl.accepted[pos] != 0;
    const bool open = !was_acc;
    const float H = open ? ent[row] : INFINITY;
    const int cand = open ? amax[row] : sl.ids[pos];  // this step's argmax canvas
    bool by_entropy, stop = false;
    if (!budget) {
      const uint64_t key = open ? ent_key(H, pos) : ~0ull;
      const uint64_t kmin = block_min_u64(key, s_red64);
      by_entropy = open && (H < a.tau || key == kmin);
    } else {
      const uint64_t q = open ? ent_fixed(H) : 0ull;
      const uint64_t key = open ? (q << 8) | (uint64_t)pos : ~0ull;  // q < 2^47, pos < 256
      s_key[pos] = key;
      s_q[pos] = q;
      __syncthreads();
      uint64_t run = 0;  // entropy of the open positions ranked at or before this one
      for (int j = 0; j < a.C; ++j) run += s_key[j] <= key ? s_q[j] : 0ull;
      const uint64_t kmin = block_min_u64(key, s_red64);
      by_entropy = open && (run <= a.budget_q || key == kmin);
      const int n_open0 = block_sum_i(open ? 1 : 0, s_red);
      const int n_diff = block_sum_i(cand != sl.prev[pos] ? 1 : 0, s_red);
      const uint64_t sum_q = block_sum_u64(q, s_red64);
      stop = n_diff == 0 && n_open0 > 0 && sum_q < (uint64_t)n_open0 * a.stop_q;
    }
    sl.prev[pos] = cand;
    const bool forced = open && !by_entropy && (sl.step >= a.max_steps || stop);
    const bool take = by_entropy || forced;
    if (take) {
      sl.ids[pos] = cand;
      sl.accepted[pos] = 1;
    } else if (open) {
      sl.ids[pos] = draw_token(sl.seed, (uint32_t)sl.block, (uint32_t)sl.step, (uint32_t)pos, (uint32_t)a.vocab);
    }
    const int n_ent = block_sum_i(by_entropy ? 1 : 0, s_red);
    const int n_forced = block_sum_i(forced ? 1 : 0, s_red);
    const int n_open = block_sum_i((open && !take) ? 1 : 0, s_red);
    if (pos == 0) {
      info[si * 4 + 0] = n_ent;
      info[si * 4 + 1] = n_forced;
      info[si * 4 + 2] = n_open;
      info[si * 4 + 3] = n_open == 0;
    }
  }
}

void dg_launch_sample(const DgSampleArgs& a, const float* ent, const int32_t* amax, int32_t* info,
                      int32_t* open_rows, int32_t* n_open_rows, hipStream_t s) {
  (void)open_rows;
  (void)n_open_rows;
  if (a.count <= 0) return;
  k_sample<<<1, a.C, 0, s>>>(a, ent, amax, info);
}

// Canvas start: every position drawn at step index 0, nothing accepted.
__global__ void __launch_bounds__(256) k_canvas_init(DgSampleArgs a) {
  const DgSampleSlot sl = a.s[blockIdx.x];
  const int pos = threadIdx.x;
  sl.ids[pos] = draw_token(sl.seed, (uint32_t)sl.block, 0u, (uint32_t)pos, (uint32_t)a.vocab);
  sl.accepted[pos] = 0;
  sl.prev[pos] = -1;
}

void dg_launch_canvas_init(const DgSampleArgs& a, int32_t* open_rows, int32_t* n_open_rows, hipStream_t s) {
  (void)open_rows;
  (void)n_open_rows;
  if (a.count <= 0) return;
  k_canvas_init<<<a.count, a.C, 0, s>>>(a);
}

// Compacted list of batch rows whose position is still open, slots in order,
// positions ascending; *n_open_rows = its length.
__global__ void __launch_bounds__(256) k_open_rows(DgSampleArgs a, int32_t* __restrict__ open_rows,
                                                   int32_t* __restrict__ n_open_rows) {
  __shared__ int s_w[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int base = 0;
  for (int si = 0; si < a.count; ++si) {
    const DgSampleSlot sl = a.s[si];
    const int pos = threadIdx.x;
    const bool open = sl.accepted[pos] == 0;
    const unsigned long long bal = __ballot(open);
    const int rank = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_w[wave] = __popcll(bal);
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += s_w[w];
    if (open) open_rows[base + wbase + rank] = sl.row0 + pos;
    base += s_w[0] + s_w[1] + s_w[2] + s_w[3];
    __syncthreads();
  }
  if (threadIdx.x == 0) *n_open_rows = base;
}

void dg_launch_open_rows(const DgSampleArgs& a, int32_t* open_rows, int32_t* n_open_rows, hipStream_t s) {
  k_open_rows<<<1, a.C, 0, s>>>(a, open_rows, n_open_rows);
}

__global__ void k_philox_tokens(uint64_t seed, int block, int step, int n, int vocab, int32_t* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = draw_token(seed, (uint32_t)block, (uint32_t)step, (uint32_t)i, (uint32_t)vocab);
}

void dg_launch_philox_tokens(uint64_t seed, int block, int step, int n, int vocab, int32_t* out, hipStream_t s) {
  if (n <= 0) return;
  k_philox_tokens<<<(n + 255) / 256, 256, 0, s>>>(seed, block, step, n, vocab, out);
}
