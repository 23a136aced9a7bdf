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
// Top-k: one wave per row.  The k largest logits (ties to the lower expert id),
// gates = softmax over the k kept logits.
__global__ void __launch_bounds__(256) k_topk(const float* __restrict__ logits, int rows, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ gates) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  if (r >= rows) return;
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    const float x = e < E ? logits[(size_t)r * E + e] : -INFINITY;
    v[i] = x == x ? x : -INFINITY;  // a NaN logit ranks lowest
  }
  float sel[16];
  int sid[16];
  unsigned taken = 0;  // entries of this lane already selected
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (e < E && !(taken >> i & 1u) && (v[i] > bv || (v[i] == bv && e < bi))) { bv = v[i]; bi = e; }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    sel[j] = bv;
    sid[j] = bi;  // k <= E: some untaken entry always exists, so bi is a real expert
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (lane + 64 * i == bi) taken |= 1u << i;
  }
  if (lane == 0) {
    float s = 0.f;
    for (int j = 0; j < k; ++j) s += __expf(sel[j] - sel[0]);
    for (int j = 0; j < k; ++j) {
      ids[(size_t)r * k + j] = sid[j];
      gates[(size_t)r * k + j] = __expf(sel[j] - sel[0]) / s;
    }
  }
}

void dg_launch_topk(const float* logits, int rows, int E, int k, int32_t* ids, float* gates, hipStream_t s) {
  if (rows <= 0) return;
  k_topk<<<(rows + 3) / 4, 256, 0, s>>>(logits, rows, E, k, ids, gates);
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
