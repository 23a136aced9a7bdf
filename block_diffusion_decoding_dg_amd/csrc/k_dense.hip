// Dense kernels of the denoising step: embedding gather, RMSNorm, the matrix-core
// projections (q/k/v with RoPE and K/V cache write, output projection with the
// residual add, shared SwiGLU expert, router logits), the MoE combine and the
// LM head fused with the per-row softmax statistics.
#include "dg_common.h"
#include "dg_kernels.h"
#include "gemm_core.h"

// ---------------------------------------------------------------------------
// Embedding: x[r] = E[ids[r]] (no scaling), fp32 residual stream.
template <typename T>
__global__ void __launch_bounds__(256) k_embed(const int32_t* __restrict__ ids, const T* __restrict__ E, int d,
                                               int vocab, float* __restrict__ x) {
  const int r = blockIdx.x;
  // Ids are validated where they enter (host prompts, the sampler's argmax and
  // Philox draws); the clamp only keeps a corrupted id from reading outside the table.
  const int id = min(max(ids[r], 0), vocab - 1);
  const T* src = E + (size_t)id * d;
  float* dst = x + (size_t)r * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) dst[c] = to_f(src[c]);
}

void dg_launch_embed(int dtype, const int32_t* ids, int rows, const void* embed, int d, int vocab, float* x,
                     hipStream_t s) {
  if (rows <= 0) return;
  if (dtype == 1)
    k_embed<bf16_t><<<rows, 256, 0, s>>>(ids, (const bf16_t*)embed, d, vocab, x);
  else
    k_embed<float><<<rows, 256, 0, s>>>(ids, (const float*)embed, d, vocab, x);
}

// Same, reading the ids of batch row r from canvas slot r / C, position r % C.
template <typename T>
__global__ void __launch_bounds__(256) k_embed_slots(DgSampleArgs a, const T* __restrict__ E, int d,
                                                     float* __restrict__ x) {
  const int r = blockIdx.x;
  const int id = min(max(a.s[r / a.C].ids[r % a.C], 0), a.vocab - 1);  // see k_embed
  const T* src = E + (size_t)id * d;
  float* dst = x + (size_t)r * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) dst[c] = to_f(src[c]);
}

void dg_launch_embed_slots(int dtype, const DgSampleArgs& a, const void* embed, int d, float* x, hipStream_t s) {
  const int rows = a.count * a.C;
  if (rows <= 0) return;
  if (dtype == 1)
    k_embed_slots<bf16_t><<<rows, 256, 0, s>>>(a, (const bf16_t*)embed, d, x);
  else
    k_embed_slots<float><<<rows, 256, 0, s>>>(a, (const float*)embed, d, x);
}

// ---------------------------------------------------------------------------
// Row kernel over the fp32 residual stream: one block of 256 threads per row, the
// row held in registers as float4 (NV per thread, d <= 1024 NV).
//   partials (nparts > 0): x[t] += sum_s parts[s][t], the partial sums of a
//     projection whose reduction was split, in range order, written back;
//   combine (y given): x[t] += sum_j gates[t][j] y[t k + j], written back (the
//     gate-weighted sum of the routed experts' outputs, j in increasing order);
//   RMSNorm (g given): out[i] = x[t] / sqrt(mean(x[t]^2) + eps) * g in the model
//     dtype, row-major or (FM) fragment-major (fm_index).
// t = row_idx[i] if given, else i; rows with i >= *n_dev (if given) are skipped.
// out_rm (optional): a second, row-major copy of the normalised rows.
template <typename T>
__device__ __forceinline__ void store4(T* p, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, float4 v) {
  *reinterpret_cast<float4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float4 v) {
  const uint32_t lo = (uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16);
  const uint32_t hi = (uint32_t)f2bf(v.z) | ((uint32_t)f2bf(v.w) << 16);
  *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
}
template <typename T>
__device__ __forceinline__ float4 load4(const T* p);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
template <>
__device__ __forceinline__ float4 load4<bf16_t>(const bf16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xffff0000u));
}

// NTH threads per row (a multiple of 64): enough that a full-width row takes
// one float4 per thread, so that every load of the row is in flight at once
// (one block per row and a few hundred rows leave one block per CU).
template <typename T, int NV, bool FM, int NTH>
__global__ void __launch_bounds__(NTH) k_row_norm(float* __restrict__ x, const int32_t* __restrict__ row_idx,
                                                  const int32_t* __restrict__ n_dev, int d,
                                                  const float* __restrict__ parts, int nparts, size_t part_stride,
                                                  const float* __restrict__ y, const float* __restrict__ gates, int k,
                                                  const T* __restrict__ g, float eps, T* __restrict__ out,
                                                  T* __restrict__ out_rm) {
  const int i = blockIdx.x;
  if (n_dev && i >= *n_dev) return;
  const int t = row_idx ? row_idx[i] : i;
  float4* xr = reinterpret_cast<float4*>(x + (size_t)t * d);
  const int nv = d >> 2;
  float4 v[NV];
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int c = threadIdx.x + NTH * u;
    v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < nv) {
      float4 a = xr[c];
      // pending partial sums of a split-reduction projection, in range order
      for (int sp = 0; sp < nparts; ++sp) {
        const float4 pp = reinterpret_cast<const float4*>(parts + sp * part_stride + (size_t)t * d)[c];
        a.x += pp.x;
        a.y += pp.y;
        a.z += pp.z;
        a.w += pp.w;
      }
      if (y) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j0 = 0; j0 < k; j0 += 8) {
          // the (up to) eight expert rows' loads first, then their sum in order
          float4 yy[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj)
            if (j0 + jj < k) yy[jj] = reinterpret_cast<const float4*>(y + ((size_t)t * k + j0 + jj) * d)[c];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            if (j0 + jj < k) {
              const float gj = gates[(size_t)t * k + j0 + jj];
              acc.x += gj * yy[jj].x;
              acc.y += gj * yy[jj].y;
              acc.z += gj * yy[jj].z;
              acc.w += gj * yy[jj].w;
            }
          }
        }
        a.x += acc.x;
        a.y += acc.y;
        a.z += acc.z;
        a.w += acc.w;
      }
      if (y || nparts) xr[c] = a;
      v[u] = a;
      ss += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
    }
  }
  if (!g) return;  // uniform over the block
  ss = wave_sum(ss);
  __shared__ float red[NTH / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < NTH / 64; ++w) tot += red[w];
  const float inv = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int c = threadIdx.x + NTH * u;
    if (c < nv) {
      const float4 gg = load4<T>(g + 4 * c);
      const float4 r = make_float4(v[u].x * inv * gg.x, v[u].y * inv * gg.y, v[u].z * inv * gg.z, v[u].w * inv * gg.w);
      store4<T>(out + (FM ? fm_index(i, 4 * c, d) : (size_t)i * d + 4 * c), r);
      if (out_rm) store4<T>(out_rm + (size_t)i * d + 4 * c, r);
    }
  }
}

template <typename T, bool FM>
void launch_row_norm(float* x, const int32_t* row_idx, const int32_t* n_dev, int rows, int d, const float* y,
                     const float* gates, int k, const T* g, float eps, T* out, hipStream_t s, T* out_rm = nullptr,
                     const DgParts& pp = DgParts{}) {
  const int nv4 = d / 4;  // float4s per row
#define DG_ROW_NORM(NVV, NTHR)                                                                                    \
  k_row_norm<T, NVV, FM, NTHR><<<rows, NTHR, 0, s>>>(x, row_idx, n_dev, d, pp.p, pp.n, pp.stride, y, gates, k, g, \
                                                     eps, out, out_rm)
  if (nv4 <= 256) DG_ROW_NORM(1, 256);
  else if (nv4 <= 768) DG_ROW_NORM(1, 768);
  else if (nv4 <= 1024) DG_ROW_NORM(1, 1024);
  else if (nv4 <= 2048) DG_ROW_NORM(2, 1024);
  else DG_ROW_NORM(4, 1024);  // d <= 16384 (checked at creation)
#undef DG_ROW_NORM
}

int dg_launch_rmsnorm(int dtype, const float* x, const int32_t* row_idx, const int32_t* n_dev, int rows, int d,
                      const void* gain, float eps, void* out, bool fm, hipStream_t s, void* out_rm,
                      const DgParts& parts) {
  if (rows <= 0) return 0;
  if (parts.n > 0 && !(dtype == 1 && fm)) return -1;  // partial sums come only from the bf16 streaming kernel
  // x is only read unless partial sums are folded in (the combine part is off)
  float* xm = const_cast<float*>(x);
  if (dtype == 1 && fm)
    launch_row_norm<bf16_t, true>(xm, row_idx, n_dev, rows, d, nullptr, nullptr, 0, (const bf16_t*)gain, eps,
                                  (bf16_t*)out, s, (bf16_t*)out_rm, parts);
  else if (dtype == 1)
    launch_row_norm<bf16_t, false>(xm, row_idx, n_dev, rows, d, nullptr, nullptr, 0, (const bf16_t*)gain, eps,
                                   (bf16_t*)out, s);
  else
    launch_row_norm<float, false>(xm, row_idx, n_dev, rows, d, nullptr, nullptr, 0, (const float*)gain, eps,
                                  (float*)out, s);
  return 0;
}

int dg_launch_combine_norm(int dtype, float* x, const float* y, const float* gates, int rows, int d, int k,
                           const void* gain, float eps, void* out, bool fm, hipStream_t s, const DgParts& parts) {
  if (rows <= 0) return 0;
  if (parts.n > 0 && !(dtype == 1 && fm)) return -1;  // partial sums come only from the bf16 streaming kernel
  if (dtype == 1 && fm)
    launch_row_norm<bf16_t, true>(x, nullptr, nullptr, rows, d, y, gates, k, (const bf16_t*)gain, eps,
                                  (bf16_t*)out, s, nullptr, parts);
  else if (dtype == 1)
    launch_row_norm<bf16_t, false>(x, nullptr, nullptr, rows, d, y, gates, k, (const bf16_t*)gain, eps,
                                   (bf16_t*)out, s);
  else
    launch_row_norm<float, false>(x, nullptr, nullptr, rows, d, y, gates, k, (const float*)gain, eps, (float*)out,
                                  s);
  return 0;
}


// ---------------------------------------------------------------------------
// Plain projection out = A W^T.  Block = WM waves stacked along rows, each wave
// MT m-tiles x NS n-tiles; grid.x over column tiles of NS*16, grid.y over row
// blocks of WM*MT*16.  mode 0: store (model dtype), 1: store fp32, 2: add to fp32.
template <typename T, int MT, int NS, int WM, int MODE>
__global__ void __launch_bounds__(64 * WM) k_gemm(const T* __restrict__ A, int M, int K, const T* __restrict__ W,
                                                  int N, void* __restrict__ out, int ldo) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col0 = blockIdx.x * (NS * 16);
  const int row_base = blockIdx.y * (WM * MT * 16) + wave * (MT * 16);
  if (row_base >= M) return;
  const int mt_active = min(MT, (M - row_base + 15) / 16);
  const char* ap[MT];
  const char* wp[NS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = min(row_base + mt * 16 + (lane & 15), M - 1);
    ap[mt] = (const char*)(A + (size_t)r * K) + (lane >> 4) * 16;
  }
#pragma unroll
  for (int ns = 0; ns < NS; ++ns) {
    int n = min(col0 + ns * 16 + (lane & 15), N - 1);
    wp[ns] = (const char*)(W + (size_t)n * K) + (lane >> 4) * 16;
  }
  v4f acc[MT][NS];
  zero_acc(acc);
  mma_loop<T, MT, NS>(ap, wp, K / MF<T>::KC, mt_active, acc);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt >= mt_active) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row_base + mt * 16 + (lane >> 4) * 4 + i;
      if (r >= M) continue;
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const int c = col0 + ns * 16 + (lane & 15);
        if (c >= N) continue;
        const size_t o = (size_t)r * ldo + c;
        if (MODE == 0) ((T*)out)[o] = from_f<T>(acc[mt][ns][i]);
        else if (MODE == 1) ((float*)out)[o] = acc[mt][ns][i];
        else ((float*)out)[o] += acc[mt][ns][i];
      }
    }
  }
}

template <typename T, int MODE>
static void gemm_dispatch(const void* A, int M, int K, const void* W, int N, void* out, int ldo, hipStream_t s) {
  constexpr int MT = 4, WM = 4;
  if (N % 32 == 0 && N >= 8192) {
    dim3 grid(N / 32, (M + WM * MT * 16 - 1) / (WM * MT * 16));
    k_gemm<T, MT, 2, WM, MODE><<<grid, 64 * WM, 0, s>>>((const T*)A, M, K, (const T*)W, N, out, ldo);
  } else {
    dim3 grid((N + 15) / 16, (M + WM * MT * 16 - 1) / (WM * MT * 16));
    k_gemm<T, MT, 1, WM, MODE><<<grid, 64 * WM, 0, s>>>((const T*)A, M, K, (const T*)W, N, out, ldo);
  }
}

void dg_launch_gemm(int dtype, int mode, const void* A, int M, int K, const void* W, int N, void* out, int ldo,
                    hipStream_t s) {
  if (M <= 0) return;
  if (dtype == 1) {
    if (mode == 0) gemm_dispatch<bf16_t, 0>(A, M, K, W, N, out, ldo, s);
    else if (mode == 1) gemm_dispatch<bf16_t, 1>(A, M, K, W, N, out, ldo, s);
    else gemm_dispatch<bf16_t, 2>(A, M, K, W, N, out, ldo, s);
  } else {
    if (mode == 0) gemm_dispatch<float, 0>(A, M, K, W, N, out, ldo, s);
    else if (mode == 1) gemm_dispatch<float, 1>(A, M, K, W, N, out, ldo, s);
    else gemm_dispatch<float, 2>(A, M, K, W, N, out, ldo, s);
  }
}

// ---------------------------------------------------------------------------
// q/k/v projection with RoPE and the K/V cache write.
//
// The output columns are taken as RoPE pairs (j, j + hd/2) of each head, heads
// ordered q (Hq), k (Hkv), v (Hkv).  A wave computes 16 pairs: n-tile 0 holds
// column j, n-tile 1 column j + hd/2 of the same rows, so each lane owns both
// halves of its pairs and rotates them in registers:
//   y_j = x_j cos(a) - x_{j+hd/2} sin(a),  y_{j+hd/2} = x_{j+hd/2} cos(a) + x_j sin(a),
// a = pos * theta^(-2j/hd) (the angle is formed and reduced mod 2 pi in fp64,
// inv_freq[j] = theta^(-2j/hd) is precomputed in fp64).  q goes to q_out
// [rows][Hq*hd]; k to K[h][pos][:]; v (not rotated) to Vt[h][:][pos].
__device__ __forceinline__ int seg_of(const DgSegs& sg, int r) {
  int s = 0;
  for (int i = 1; i < sg.count; ++i)
    if (r >= sg.s[i].row0) s = i;
  return s;
}

template <typename T, int MT, int WM>
__global__ void __launch_bounds__(64 * WM) k_qkv(const T* __restrict__ A, int M, DgShape sh, const T* __restrict__ wq,
                                                 const T* __restrict__ wk, const T* __restrict__ wv, DgSegs sg,
                                                 const double* __restrict__ inv_freq, T* __restrict__ q_out) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int K = sh.d, hd = sh.hd, half = hd / 2;
  const int row_base = blockIdx.y * (WM * MT * 16) + wave * (MT * 16);
  if (row_base >= M) return;
  const int mt_active = min(MT, (M - row_base + 15) / 16);
  const int jp = blockIdx.x * 16 + (lane & 15);  // global pair index of this lane's column
  const int head = jp / half, j = jp - head * half;
  const T* wbase;
  int kind, hloc;  // 0 q, 1 k, 2 v
  if (head < sh.hq) { kind = 0; hloc = head; wbase = wq; }
  else if (head < sh.hq + sh.hkv) { kind = 1; hloc = head - sh.hq; wbase = wk; }
  else { kind = 2; hloc = head - sh.hq - sh.hkv; wbase = wv; }
  const char* ap[MT];
  const char* wp[2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = min(row_base + mt * 16 + (lane & 15), M - 1);
    ap[mt] = (const char*)(A + (size_t)r * K) + (lane >> 4) * 16;
  }
  wp[0] = (const char*)(wbase + (size_t)(hloc * hd + j) * K) + (lane >> 4) * 16;
  wp[1] = (const char*)(wbase + (size_t)(hloc * hd + half + j) * K) + (lane >> 4) * 16;
  v4f acc[MT][2];
  zero_acc(acc);
  mma_loop<T, MT, 2>(ap, wp, K / MF<T>::KC, mt_active, acc);

  // The lanes of one 16-lane group may straddle two heads (hd/2 < 16); each lane
  // uses its own (kind, hloc, j).
  const double f = inv_freq[j];
  const double two_pi = 6.283185307179586476925286766559;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt >= mt_active) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row_base + mt * 16 + (lane >> 4) * 4 + i;
      if (r >= M) continue;
      const int si = seg_of(sg, r);
      const int pos = sg.s[si].pos0 + (r - sg.s[si].row0);
      float x1 = acc[mt][0][i], x2 = acc[mt][1][i];
      if (kind < 2) {
        double a = (double)pos * f;
        a -= two_pi * rint(a / two_pi);
        float sn, cs;
        sincosf((float)a, &sn, &cs);
        const float y1 = x1 * cs - x2 * sn;
        const float y2 = x2 * cs + x1 * sn;
        x1 = y1;
        x2 = y2;
      }
      if (kind == 0) {
        T* qr = q_out + (size_t)r * (sh.hq * hd) + hloc * hd;
        qr[j] = from_f<T>(x1);
        qr[j + half] = from_f<T>(x2);
      } else if (kind == 1) {
        T* kr = (T*)sg.s[si].k + ((size_t)hloc * sh.max_ctx + pos) * hd;
        kr[j] = from_f<T>(x1);
        kr[j + half] = from_f<T>(x2);
      } else {
        T* vb = (T*)sg.s[si].vt + (size_t)hloc * hd * sh.max_ctx;
        vb[(size_t)j * sh.max_ctx + pos] = from_f<T>(x1);
        vb[(size_t)(j + half) * sh.max_ctx + pos] = from_f<T>(x2);
      }
    }
  }
}

void dg_launch_qkv(int dtype, const void* A, int M, const DgShape& sh, const void* wq, const void* wk, const void* wv,
                   const DgSegs& segs, const double* inv_freq, void* q_out, hipStream_t s) {
  if (M <= 0) return;
  constexpr int MT = 4, WM = 4;
  const int pairs = (sh.hq + 2 * sh.hkv) * sh.hd / 2;
  dim3 grid(pairs / 16, (M + WM * MT * 16 - 1) / (WM * MT * 16));
  if (dtype == 1)
    k_qkv<bf16_t, MT, WM><<<grid, 64 * WM, 0, s>>>((const bf16_t*)A, M, sh, (const bf16_t*)wq, (const bf16_t*)wk,
                                                   (const bf16_t*)wv, segs, inv_freq, (bf16_t*)q_out);
  else
    k_qkv<float, MT, WM><<<grid, 64 * WM, 0, s>>>((const float*)A, M, sh, (const float*)wq, (const float*)wk,
                                                  (const float*)wv, segs, inv_freq, (float*)q_out);
}

// ---------------------------------------------------------------------------
// Shared expert up-projection with SwiGLU: h = silu(A W1^T) * (A W3^T).
// n-tile 0 reads W1, n-tile 1 reads W3 for the same 16 output columns.
template <typename T, int MT, int WM>
__global__ void __launch_bounds__(64 * WM) k_swiglu(const T* __restrict__ A, int M, int K, const T* __restrict__ w1,
                                                    const T* __restrict__ w3, int N, T* __restrict__ h) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row_base = blockIdx.y * (WM * MT * 16) + wave * (MT * 16);
  if (row_base >= M) return;
  const int mt_active = min(MT, (M - row_base + 15) / 16);
  const int c = blockIdx.x * 16 + (lane & 15);
  const char* ap[MT];
  const char* wp[2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = min(row_base + mt * 16 + (lane & 15), M - 1);
    ap[mt] = (const char*)(A + (size_t)r * K) + (lane >> 4) * 16;
  }
  wp[0] = (const char*)(w1 + (size_t)c * K) + (lane >> 4) * 16;
  wp[1] = (const char*)(w3 + (size_t)c * K) + (lane >> 4) * 16;
  v4f acc[MT][2];
  zero_acc(acc);
  mma_loop<T, MT, 2>(ap, wp, K / MF<T>::KC, mt_active, acc);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt >= mt_active) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row_base + mt * 16 + (lane >> 4) * 4 + i;
      if (r < M) h[(size_t)r * N + c] = from_f<T>(silu_f(acc[mt][0][i]) * acc[mt][1][i]);
    }
  }
}

void dg_launch_swiglu(int dtype, const void* A, int M, int K, const void* w1, const void* w3, int N, void* h_out,
                      hipStream_t s) {
  if (M <= 0) return;
  constexpr int MT = 4, WM = 4;
  dim3 grid(N / 16, (M + WM * MT * 16 - 1) / (WM * MT * 16));
  if (dtype == 1)
    k_swiglu<bf16_t, MT, WM><<<grid, 64 * WM, 0, s>>>((const bf16_t*)A, M, K, (const bf16_t*)w1, (const bf16_t*)w3, N,
                                                      (bf16_t*)h_out);
  else
    k_swiglu<float, MT, WM><<<grid, 64 * WM, 0, s>>>((const float*)A, M, K, (const float*)w1, (const float*)w3, N,
                                                     (float*)h_out);
}

// ---------------------------------------------------------------------------
// MoE combine: x[t] += sum_j gates[t][j] * y[t*k + j], slots in fixed order.
__global__ void k_gather_rows(const float* __restrict__ x, const int32_t* __restrict__ idx, int d,
                              float* __restrict__ out) {
  const int i = blockIdx.x;
  const float* src = x + (size_t)idx[i] * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) out[(size_t)i * d + c] = src[c];
}

void dg_launch_gather_rows(const float* x, const int32_t* idx, int n, int d, float* out, hipStream_t s) {
  if (n <= 0) return;
  k_gather_rows<<<n, 256, 0, s>>>(x, idx, d, out);
}

// ---------------------------------------------------------------------------
// LM head fused with the softmax statistics.  Rows hn [n][d] (already normalised),
// tied head E [V][d].  Block = WM x WN waves; a block covers BM = WM*MT*16 rows and
// BN = WN*NS*16 vocabulary columns (one "tile").  For each row the block writes the
// tile's (m, s, t) and the tile's argmax (lowest column among the maxima); the
// logits never leave registers.  A second kernel merges the tiles of a row in
// tile order.
template <typename T, int MT, int NS, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN) k_lm_head(const T* __restrict__ hn, const int32_t* __restrict__ n_dev,
                                                          int d, const T* __restrict__ E, int n_tiles,
                                                          float* __restrict__ part, int32_t* __restrict__ part_arg) {
  constexpr int BM = WM * MT * 16, BN = WN * NS * 16;
  __shared__ float s_st[WN][BM][3];
  __shared__ int32_t s_arg[WN][BM];
  const int n = *n_dev;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave % WM, wn = wave / WM;
  const int blk_row0 = blockIdx.y * BM;
  if (blk_row0 >= n) return;  // uniform over the block
  const int row_base = blk_row0 + wm * (MT * 16);
  const int mt_active = row_base >= n ? 0 : min(MT, (n - row_base + 15) / 16);
  const int col0 = blockIdx.x * BN + wn * (NS * 16);
  const char* ap[MT];
  const char* wp[NS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    int r = min(row_base + mt * 16 + (lane & 15), n - 1);
    ap[mt] = (const char*)(hn + (size_t)r * d) + (lane >> 4) * 16;
  }
#pragma unroll
  for (int ns = 0; ns < NS; ++ns) wp[ns] = (const char*)(E + (size_t)(col0 + ns * 16 + (lane & 15)) * d) + (lane >> 4) * 16;
  v4f acc[MT][NS];
  zero_acc(acc);
  if (mt_active > 0) mma_loop<T, MT, NS>(ap, wp, d / MF<T>::KC, mt_active, acc);

  // Per row over this wave's NS*16 columns: lane holds column (ns*16 + lane%16).
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float m = acc[mt][0][i];
      int am = col0 + (lane & 15);
#pragma unroll
      for (int ns = 1; ns < NS; ++ns) {
        const float v = acc[mt][ns][i];
        if (v > m) { m = v; am = col0 + ns * 16 + (lane & 15); }
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float om = __shfl_xor(m, o, 64);
        const int oa = __shfl_xor(am, o, 64);
        if (om > m || (om == m && oa < am)) { m = om; am = oa; }
      }
      float s = 0.f, t = 0.f;
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const float z = acc[mt][ns][i] - m;
        const float e = __expf(z);
        s += e;
        t += e * z;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        s += __shfl_xor(s, o, 64);
        t += __shfl_xor(t, o, 64);
      }
      if ((lane & 15) == 0) {
        const int rl = wm * (MT * 16) + mt * 16 + (lane >> 4) * 4 + i;
        s_st[wn][rl][0] = m;
        s_st[wn][rl][1] = s;
        s_st[wn][rl][2] = t;
        s_arg[wn][rl] = am;
      }
    }
  }
  __syncthreads();
  for (int rl = threadIdx.x; rl < BM; rl += blockDim.x) {
    const int r = blk_row0 + rl;
    if (r >= n) continue;
    SoftStats acc_s{s_st[0][rl][0], s_st[0][rl][1], s_st[0][rl][2]};
    float best = s_st[0][rl][0];
    int barg = s_arg[0][rl];
#pragma unroll
    for (int w = 1; w < WN; ++w) {
      SoftStats o{s_st[w][rl][0], s_st[w][rl][1], s_st[w][rl][2]};
      acc_s = soft_merge(acc_s, o);
      if (o.m > best) { best = o.m; barg = s_arg[w][rl]; }  // later waves hold higher columns
    }
    const size_t pi = (size_t)r * n_tiles + blockIdx.x;
    part[pi * 3 + 0] = acc_s.m;
    part[pi * 3 + 1] = acc_s.s;
    part[pi * 3 + 2] = acc_s.t;
    part_arg[pi] = barg;
  }
}

// One wave per row: lanes merge tiles lane, lane+64, ... in order, then a fixed
// butterfly across lanes; argmax keeps the larger value, ties to the lower column.
__global__ void __launch_bounds__(64) k_lm_merge(const float* __restrict__ part, const int32_t* __restrict__ part_arg,
                                                 const int32_t* __restrict__ n_dev, int n_tiles,
                                                 const int32_t* __restrict__ row_idx, float* __restrict__ ent,
                                                 float* __restrict__ lse, int32_t* __restrict__ amax) {
  const int r = blockIdx.x;
  if (r >= *n_dev) return;
  const int lane = threadIdx.x;
  SoftStats st{0.f, 0.f, 0.f};
  float best = -INFINITY;
  int barg = 0x7fffffff;
  for (int t = lane; t < n_tiles; t += 64) {
    const size_t pi = (size_t)r * n_tiles + t;
    SoftStats o{part[pi * 3], part[pi * 3 + 1], part[pi * 3 + 2]};
    st = soft_merge(st, o);
    const int a = part_arg[pi];
    // A NaN maximum ranks lowest, so the winner is always a real column.
    const float om = o.m == o.m ? o.m : -INFINITY;
    if (om > best || (om == best && a < barg)) { best = om; barg = a; }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    SoftStats x{__shfl_xor(st.m, o, 64), __shfl_xor(st.s, o, 64), __shfl_xor(st.t, o, 64)};
    // merge in a lane-independent order so both partners compute the same value
    SoftStats lo = (lane & o) ? x : st, hi = (lane & o) ? st : x;
    st = soft_merge(lo, hi);
    const float ob = __shfl_xor(best, o, 64);
    const int oa = __shfl_xor(barg, o, 64);
    if (ob > best || (ob == best && oa < barg)) { best = ob; barg = oa; }
  }
  if (lane == 0) {
    const int dst = row_idx ? row_idx[r] : r;
    ent[dst] = logf(st.s) - st.t / st.s;
    lse[dst] = st.m + logf(st.s);
    amax[dst] = barg;
  }
}

int dg_lm_head_tiles(int vocab) { return vocab / 128; }

void dg_launch_lm_head(int dtype, const void* hn, const int32_t* n_dev, int max_rows, int d, const void* embed,
                       int vocab, float* part, int32_t* part_arg, float* ent, float* lse, int32_t* amax,
                       const int32_t* row_idx, hipStream_t s) {
  if (max_rows <= 0) return;
  constexpr int MT = 8, NS = 4, WM = 2, WN = 2;
  constexpr int BM = WM * MT * 16;
  const int n_tiles = dg_lm_head_tiles(vocab);
  dim3 grid(n_tiles, (max_rows + BM - 1) / BM);
  if (dtype == 1)
    k_lm_head<bf16_t, MT, NS, WM, WN><<<grid, 64 * WM * WN, 0, s>>>((const bf16_t*)hn, n_dev, d, (const bf16_t*)embed,
                                                                   n_tiles, part, part_arg);
  else
    k_lm_head<float, MT, NS, WM, WN><<<grid, 64 * WM * WN, 0, s>>>((const float*)hn, n_dev, d, (const float*)embed,
                                                                  n_tiles, part, part_arg);
  k_lm_merge<<<max_rows, 64, 0, s>>>(part, part_arg, n_dev, n_tiles, row_idx, ent, lse, amax);
}

void dg_launch_lm_merge(const float* part, const int32_t* part_arg, const int32_t* n_dev, int max_rows, int n_tiles,
                        const int32_t* row_idx, float* ent, float* lse, int32_t* amax, hipStream_t s) {
  if (max_rows <= 0) return;
  k_lm_merge<<<max_rows, 64, 0, s>>>(part, part_arg, n_dev, n_tiles, row_idx, ent, lse, amax);
}
