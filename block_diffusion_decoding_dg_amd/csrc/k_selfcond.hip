// Self-conditioning: the previous step's softmax fed back into the next forward
// through a small gated MLP ("DiffusionGemma hits ~1,500 TPS on one H100",
// section "How the sampler actually works"; the pages give no structure).  The
// structure taken: each canvas position keeps u = sum_v softmax(z)_v E[v], the
// expectation of the tied embedding under the logits z of the last step at which
// the position was open (zero when the canvas starts), and every forward over the
// canvas adds W2 (silu(W1 u) * (W3 u)) to the token embedding.
//
// The expectation is a product of the [open rows, V] probability matrix with the
// [V, d] embedding, a reduction over the vocabulary.  The streaming GEMM wants its
// weight operand with the reduction index contiguous, so the embedding is kept a
// second time transposed ([d, V], built once per context); the LM head writes the
// open rows' logits, this file turns them into bf16 probabilities in the
// fragment-major layout, the streaming GEMM reduces them against the transposed
// embedding in split vocabulary ranges, and the fold sums the ranges in order
// into the per-request state.
#include "dg_common.h"
#include "dg_kernels.h"

#include <algorithm>
#include <cstdlib>

// ET[c][v] = E[v][c] for E [V][d] bf16: 64 x 64 tiles through LDS (one padding
// column keeps the transposed reads free of bank conflicts).  V and d are
// multiples of 64.
__global__ void __launch_bounds__(256) k_transpose_bf16(const bf16_t* __restrict__ E, int V, int d,
                                                        bf16_t* __restrict__ ET) {
  __shared__ bf16_t s[64][65];
  const int tv = blockIdx.x % (V / 64), tc = blockIdx.x / (V / 64);
  const int v0 = tv * 64, c0 = tc * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i >> 6, cc = i & 63;
    s[r][cc] = E[(size_t)(v0 + r) * d + c0 + cc];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i >> 6, vv = i & 63;
    ET[(size_t)(c0 + r) * V + v0 + vv] = s[vv][r];
  }
}

int dg_launch_transpose_bf16(const void* E, int V, int d, void* ET, hipStream_t s) {
  if (V % 64 || d % 64) return -1;  // whole tiles only
  k_transpose_bf16<<<(V / 64) * (d / 64), 256, 0, s>>>((const bf16_t*)E, V, d, (bf16_t*)ET);
  return 0;
}

// Probabilities of the open rows: P[r][v] = bf16(exp(z[r][v] - lse[row_idx[r]]))
// for r < *n_dev, z fp32 [rows][V] row-major (row r of the LM head's compacted
// rows), P bf16 fragment-major [rows][V].  A thread converts 8 consecutive
// vocabulary entries, one 16-byte unit of the fragment-major layout.
__global__ void __launch_bounds__(256) k_sc_probs(const float* __restrict__ z, const float* __restrict__ lse,
                                                  const int32_t* __restrict__ row_idx,
                                                  const int32_t* __restrict__ n_dev, int V,
                                                  bf16_t* __restrict__ P) {
  const size_t u = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = V / 8;
  const int r = (int)(u / per_row), v = (int)(u % per_row) * 8;
  if (r >= *n_dev) return;
  const float l = lse[row_idx[r]];
  const float4* zp = (const float4*)(z + (size_t)r * V + v);
  const float4 a = zp[0], b = zp[1];
  const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w[j] = (uint32_t)f2bf(__expf(x[2 * j] - l)) | ((uint32_t)f2bf(__expf(x[2 * j + 1] - l)) << 16);
  *(uint4*)(P + fm_index(r, v, V)) = make_uint4(w[0], w[1], w[2], w[3]);
}

void dg_launch_sc_probs(const float* z, const float* lse, const int32_t* row_idx, const int32_t* n_dev,
                        int max_rows, int V, void* P, hipStream_t s) {
  if (max_rows <= 0) return;
  const size_t units = (size_t)max_rows * (V / 8);
  k_sc_probs<<<(unsigned)((units + 255) / 256), 256, 0, s>>>(z, lse, row_idx, n_dev, V, (bf16_t*)P);
}

// State update: for compacted row r < *n_dev (canvas row row_idx[r] = slot * C +
// position), u = the sum of the nks partial ranges (in range order, so the result
// is deterministic) written to the slot's state row.
__global__ void __launch_bounds__(256) k_sc_fold(const float* __restrict__ parts, int nks, size_t stride, int d,
                                                 const int32_t* __restrict__ row_idx,
                                                 const int32_t* __restrict__ n_dev, DgScSlots sl, int C) {
  const int r = blockIdx.x;
  if (r >= *n_dev) return;
  const int row = row_idx[r], slot = row / C, pos = row % C;
  float* dst = sl.state[slot] + (size_t)pos * d;
  for (int c = threadIdx.x * 4; c < d; c += 256 * 4) {
    float4 acc = *(const float4*)(parts + (size_t)r * d + c);
    for (int k = 1; k < nks; ++k) {
      const float4 p = *(const float4*)(parts + k * stride + (size_t)r * d + c);
      acc.x += p.x;
      acc.y += p.y;
      acc.z += p.z;
      acc.w += p.w;
    }
    *(float4*)(dst + c) = acc;
  }
}

int dg_launch_sc_fold(const float* parts, int nks, size_t stride, int d, const int32_t* row_idx,
                      const int32_t* n_dev, int max_rows, const DgScSlots& sl, int C, hipStream_t s) {
  if (max_rows <= 0) return 0;
  if (d % 4) return -1;  // float4 rows
  k_sc_fold<<<max_rows, 256, 0, s>>>(parts, nks, stride, d, row_idx, n_dev, sl, C);
  return 0;
}

// MLP input of the canvas rows: row t = slot * C + position (t < rows) of the
// fragment-major bf16 matrix b [rows][d] = bf16(state of that slot and position).
__global__ void __launch_bounds__(256) k_sc_gather(DgScSlots sl, int rows, int C, int d, bf16_t* __restrict__ b) {
  const size_t u = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = d / 8;
  const int t = (int)(u / per_row), c = (int)(u % per_row) * 8;
  if (t >= rows) return;
  const float* src = sl.state[t / C] + (size_t)(t % C) * d + c;
  const float4 a = ((const float4*)src)[0], e = ((const float4*)src)[1];
  const uint4 w = make_uint4((uint32_t)f2bf(a.x) | ((uint32_t)f2bf(a.y) << 16),
                             (uint32_t)f2bf(a.z) | ((uint32_t)f2bf(a.w) << 16),
                             (uint32_t)f2bf(e.x) | ((uint32_t)f2bf(e.y) << 16),
                             (uint32_t)f2bf(e.z) | ((uint32_t)f2bf(e.w) << 16));
  *(uint4*)(b + fm_index(t, c, d)) = w;
}

void dg_launch_sc_gather(const DgScSlots& sl, int rows, int C, int d, void* b, hipStream_t s) {
  if (rows <= 0) return;
  const size_t units = (size_t)rows * (d / 8);
  k_sc_gather<<<(unsigned)((units + 255) / 256), 256, 0, s>>>(sl, rows, C, d, (bf16_t*)b);
}

// Rows of fp32 u (row-major [n][d]) to the fragment-major bf16 MLP input.
__global__ void __launch_bounds__(256) k_rows_to_fm(const float* __restrict__ u, int n, int d,
                                                    bf16_t* __restrict__ b) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  const int per_row = d / 8;
  const int t = (int)(i / per_row), c = (int)(i % per_row) * 8;
  if (t >= n) return;
  const float4 a = *(const float4*)(u + (size_t)t * d + c), e = *(const float4*)(u + (size_t)t * d + c + 4);
  *(uint4*)(b + fm_index(t, c, d)) = make_uint4((uint32_t)f2bf(a.x) | ((uint32_t)f2bf(a.y) << 16),
                                                (uint32_t)f2bf(a.z) | ((uint32_t)f2bf(a.w) << 16),
                                                (uint32_t)f2bf(e.x) | ((uint32_t)f2bf(e.y) << 16),
                                                (uint32_t)f2bf(e.z) | ((uint32_t)f2bf(e.w) << 16));
}

void dg_launch_rows_to_fm(const float* u, int n, int d, void* b, hipStream_t s) {
  if (n <= 0) return;
  const size_t units = (size_t)n * (d / 8);
  k_rows_to_fm<<<(unsigned)((units + 255) / 256), 256, 0, s>>>(u, n, d, (bf16_t*)b);
}

// Zero n floats (a fill kernel rather than a memset node, so that the calls
// that use it stay safe to capture in a graph).
__global__ void __launch_bounds__(256) k_fill_zero(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0.f;
}

// One int32 set to v on the stream (no host copy).
__global__ void k_set_i32(int32_t* __restrict__ p, int32_t v) {
  if (threadIdx.x == 0) p[0] = v;
}

void dg_launch_set_i32(int32_t* p, int32_t v, hipStream_t s) { k_set_i32<<<1, 64, 0, s>>>(p, v); }

void dg_launch_fill_zero(float* p, size_t n, hipStream_t s) {
  if (n == 0) return;
  const size_t blocks = std::min<size_t>((n + 255) / 256, 4096);
  k_fill_zero<<<(unsigned)blocks, 256, 0, s>>>(p, n);
}
