// Device-side building blocks shared by the kernels of libdg (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // raw bf16 bits

typedef short v8s __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Fragment-major ("FM") layout of a bf16 activation matrix with K columns (K a
// multiple of 64) and rows padded to a multiple of 16: the 16-row x 32-column
// blocks are stored one after another, row tiles outer, and inside a block lane
// L = 16 g + i of the matrix core's operand layout owns the 16 bytes of row i,
// columns 8 g .. 8 g + 7.  A wave's operand fragment is then one contiguous 1 KB
// load.  Element index of (r, k):
__device__ __forceinline__ size_t fm_index(int r, int k, int K) {
  return ((size_t)(r >> 4) * (K >> 5) + (k >> 5)) * 512 + (((k & 31) >> 3) * 16 + (r & 15)) * 8 + (k & 7);
}

#define DG_WAVE 64

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest even (finite inputs).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }

// Matrix-core step on 16-byte per-lane fragments.
//
// A 16x16 output tile with a "k-chunk" of 64 bytes per row: bf16 -> 32 k values
// (one v_mfma_f32_16x16x32_bf16), f32 -> 16 k values (four v_mfma_f32_16x16x4f32).
// Lane l supplies row (l % 16) of A and column (l % 16) of B, taking the 16 bytes
// at byte offset 16 * (l / 16) of the 64-byte chunk.  For f32 the four MFMAs use
// element j of every lane, i.e. k = 4 * (l / 16) + j: the same permutation of k on
// both operands, so the sum over the chunk is unchanged.
// Output: lane l holds D[4 * (l / 16) + i][l % 16], i = 0..3.
template <typename T> struct MF;

template <> struct MF<bf16_t> {
  typedef v8s frag;
  static constexpr int KC = 32;
  static __device__ __forceinline__ void mma(v4f& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
};

template <> struct MF<float> {
  typedef v4f frag;
  static constexpr int KC = 16;
  static __device__ __forceinline__ void mma(v4f& acc, const frag& a, const frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
  }
};

template <typename F> __device__ __forceinline__ F load_frag(const char* p) {
  return *reinterpret_cast<const F*>(p);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float silu_f(float x) { return x / (1.0f + __expf(-x)); }

// Softmax-statistics triple over a set of logits z: m = max z,
// s = sum exp(z - m), t = sum exp(z - m) * (z - m).  Entropy = log s - t / s,
// log-sum-exp = m + log s.  Two triples merge exactly (up to rounding):
// with M = max(m1, m2), s = s1 e^(m1-M) + s2 e^(m2-M) and
// t = e^(m1-M) (t1 + (m1 - M) s1) + e^(m2-M) (t2 + (m2 - M) s2).
struct SoftStats {
  float m, s, t;
};
__device__ __forceinline__ SoftStats soft_merge(SoftStats a, SoftStats b) {
  if (a.s == 0.f) return b;
  if (b.s == 0.f) return a;
  float M = fmaxf(a.m, b.m);
  float ea = __expf(a.m - M), eb = __expf(b.m - M);
  SoftStats r;
  r.m = M;
  r.s = a.s * ea + b.s * eb;
  r.t = ea * (a.t + (a.m - M) * a.s) + eb * (b.t + (b.m - M) * b.s);
  return r;
}

// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11): 10 rounds of
// (c0, c1, c2, c3) -> (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)),
// key advanced by the Weyl increments before every round after the first.
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { k0 += W0; k1 += W1; }
    uint64_t lo0 = M0 * c[0], hi0 = __umul64hi(M0, c[0]);
    uint64_t lo1 = M1 * c[2], hi1 = __umul64hi(M1, c[2]);
    uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
  }
}

// Uniform token in [0, vocab): high 64 bits of r0 * vocab, r0 the first Philox word of
// counter (position, step, block, 0) under key (seed, 0).
__device__ __forceinline__ int32_t draw_token(uint64_t seed, uint32_t block, uint32_t step, uint32_t pos,
                                              uint32_t vocab) {
  uint64_t c[4] = {(uint64_t)pos, (uint64_t)step, (uint64_t)block, 0ull};
  philox4x64_10(c, seed, 0ull);
  return (int32_t)__umul64hi(c[0], (uint64_t)vocab);
}

// Wait until at most n of this wave's vector memory loads are outstanding
// (vmcnt only; the lgkm and export counters are left at their maxima).
#define DG_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

// One global_load_lds_dwordx4: lane l copies 16 bytes from g (its own address)
// to lds + 16 l (lds wave-uniform).  Issued from an asm statement with inputs
// only (the LDS base goes to M0), so that the compiler adds no wait of its own
// for it: the kernel's explicit vmcnt waits and barriers order these copies
// against the LDS reads.  The statement writes no register.
__device__ __forceinline__ void lds_dma16(const void* g, const uint4* lds) {
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint4*)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(__builtin_amdgcn_readfirstlane(a)), "v"(g)
               : "memory", "m0");
}

// The same copy with the non-temporal hint (nt): for data read once per launch
// (streamed weights), which the L2 may then evict before the lines that many
// blocks re-read (activation rows).
__device__ __forceinline__ void lds_dma16_nt(const void* g, const uint4* lds) {
  const uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint4*)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :
               : "s"(__builtin_amdgcn_readfirstlane(a)), "v"(g)
               : "memory", "m0");
}
