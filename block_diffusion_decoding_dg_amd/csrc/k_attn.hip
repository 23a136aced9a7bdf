// Bidirectional (or causal, for the prompt) grouped-query attention of a batch of
// rows over their request's KV cache, split over keys (flash-decoding style) and
// merged with the log-sum-exp rule.
//
// Every canvas position sees the whole committed prefix and the whole canvas
// ("Google open-sources DiffusionGemma", section "26B MoE Architecture, but Only
// 3.8B Activated": bidirectional attention, every token sees all others in its
// context; "DiffusionGemma hits ~1,500 TPS on one H100", section "How the sampler
// actually works": the decoder runs bidirectionally over the full canvas).
//
// Layout of the work: a block takes one kv-head h of one request, 128 "query
// rows" (pairs of (q-head of h's group, canvas row), head-major) and one key
// range.  Each wave owns 32 query rows.  Scores are formed transposed,
// S^T = K Q^T, so that lane l holds, for query column l % 16, keys 4*(l/16)+i:
// exactly the B-operand layout of O^T = V^T P^T on the matrix cores.  With V
// stored transposed in the cache ([hd][position]) both operands of both
// products are plain row loads; P never leaves registers.
#include "dg_common.h"
#include "dg_kernels.h"

#include <type_traits>

#define ATTN_QROWS 128  // query rows per block (4 waves x 32)

template <typename T, int HD>
__global__ void __launch_bounds__(256) k_attn(const T* __restrict__ q, DgShape sh, DgSegs sg, int nqb, int nsplit,
                                              float* __restrict__ opart, float* __restrict__ mlpart, int rows_total) {
  typedef typename MF<T>::frag F;
  constexpr int KC = MF<T>::KC;
  constexpr int NKK = HD / KC;  // k-chunks over the head dimension
  constexpr int NHT = HD / 16;  // 16-row tiles of O^T
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g4 = lane >> 4, c16 = lane & 15;

  int bid = blockIdx.x;
  const int split = bid % nsplit;
  bid /= nsplit;
  const int qb = bid % nqb;
  bid /= nqb;
  const int h = bid % sh.hkv;
  const int si = bid / sh.hkv;
  if (si >= sg.count) return;
  const DgSeg seg = sg.s[si];
  const int G = sh.hq / sh.hkv;
  const int nq = G * seg.n;
  const int qr0 = qb * ATTN_QROWS + wave * 32;
  if (qb * ATTN_QROWS >= nq) return;  // uniform over the block

  // This lane's two query rows (one per 16-wide query tile).
  int qrow[2], qhead[2], trow[2], qpos[2];
  bool qvalid[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qr = qr0 + qt * 16 + c16;
    qvalid[qt] = qr < nq;
    const int qrc = qvalid[qt] ? qr : nq - 1;
    const int hg = qrc / seg.n, i = qrc - hg * seg.n;
    qrow[qt] = qrc;
    qhead[qt] = h * G + hg;
    trow[qt] = seg.row0 + i;
    qpos[qt] = seg.pos0 + i;
  }
  // Key range of this split; causal rows see keys <= their own position.
  const int nkeys = seg.nkeys;
  const int chunk = ((nkeys + nsplit - 1) / nsplit + 31) / 32 * 32;
  const int k_lo = split * chunk;
  int k_hi = min(nkeys, k_lo + chunk);
  if (sg.causal) {
    int mp = max(qvalid[0] ? qpos[0] : -1, qvalid[1] ? qpos[1] : -1);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) mp = max(mp, __shfl_xor(mp, o, 64));
    k_hi = min(k_hi, mp + 1);
  }

  F qf[2][NKK];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const char* qp = (const char*)(q + (size_t)trow[qt] * (sh.hq * HD) + qhead[qt] * HD) + g4 * 16;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qf[qt][kk] = load_frag<F>(qp + kk * 64);
  }

  const T* kbase = (const T*)seg.k + (size_t)h * sh.max_ctx * HD;
  const T* vbase = (const T*)seg.vt + (size_t)h * HD * sh.max_ctx;
  const float scale = 1.4426950408889634f / sqrtf((float)HD);  // log2(e) / sqrt(hd)

  v4f oacc[NHT][2];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht) oacc[ht][0] = oacc[ht][1] = v4f{0.f, 0.f, 0.f, 0.f};
  float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};

  for (int kb = k_lo; kb < k_hi; kb += 32) {
    v4f st[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      st[kt][0] = st[kt][1] = v4f{0.f, 0.f, 0.f, 0.f};
      const int key = min(kb + kt * 16 + c16, nkeys - 1);
      const char* kp = (const char*)(kbase + (size_t)key * HD) + g4 * 16;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const F kf = load_frag<F>(kp + kk * 64);
        MF<T>::mma(st[kt][0], kf, qf[0][kk]);
        MF<T>::mma(st[kt][1], kf, qf[1][kk]);
      }
    }
    // Scale, mask, online softmax per query column.
    float p[2][2][4];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + kt * 16 + g4 * 4 + i;
          float s = st[kt][qt][i] * scale;
          if (key >= k_hi || (sg.causal && key > qpos[qt])) s = -INFINITY;
          p[kt][qt][i] = s;
          tmax = fmaxf(tmax, s);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float mnew = fmaxf(mrun[qt], tmax);
      const float alpha = (mnew == -INFINITY) ? 1.f : exp2f(mrun[qt] - mnew);
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = (mnew == -INFINITY) ? 0.f : exp2f(p[kt][qt][i] - mnew);
          p[kt][qt][i] = e;
          psum += e;
        }
      lrun[qt] = lrun[qt] * alpha + psum;
      mrun[qt] = mnew;
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) oacc[ht][qt] *= alpha;
    }
    // O^T += V^T P^T over the 32 keys of this tile.  In bf16, P enters the matrix
    // cores as a high and a low bf16 part (p = hi + lo to ~2^-16 relative), two
    // products against the same V tile: a single bf16 P would carry a relative
    // error of ~2^-9 into the output, which for nearly uniform weights averaging
    // over many keys does not shrink.
    if constexpr (sizeof(T) == 2) {
      F pf[2], pl[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            const float v = p[kt][qt][i];
            const bf16_t h = f2bf(v);
            pf[qt][kt * 4 + i] = (short)h;
            pl[qt][kt * 4 + i] = (short)f2bf(v - bf2f(h));
          }
        }
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht) {
        const T* vr = vbase + (size_t)(ht * 16 + c16) * sh.max_ctx + kb + g4 * 4;
        const uint2 lo = *(const uint2*)vr;
        const uint2 hi = *(const uint2*)(vr + 16);
        F vf;
        vf[0] = (short)(lo.x & 0xffff); vf[1] = (short)(lo.x >> 16);
        vf[2] = (short)(lo.y & 0xffff); vf[3] = (short)(lo.y >> 16);
        vf[4] = (short)(hi.x & 0xffff); vf[5] = (short)(hi.x >> 16);
        vf[6] = (short)(hi.y & 0xffff); vf[7] = (short)(hi.y >> 16);
        MF<T>::mma(oacc[ht][0], vf, pf[0]);
        MF<T>::mma(oacc[ht][1], vf, pf[1]);
        MF<T>::mma(oacc[ht][0], vf, pl[0]);
        MF<T>::mma(oacc[ht][1], vf, pl[1]);
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        F pf0 = {p[kt][0][0], p[kt][0][1], p[kt][0][2], p[kt][0][3]};
        F pf1 = {p[kt][1][0], p[kt][1][1], p[kt][1][2], p[kt][1][3]};
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
          const T* vr = vbase + (size_t)(ht * 16 + c16) * sh.max_ctx + kb + kt * 16 + g4 * 4;
          const F vf = *(const F*)vr;
          MF<T>::mma(oacc[ht][0], vf, pf0);
          MF<T>::mma(oacc[ht][1], vf, pf1);
        }
      }
    }
  }
  // Row sums across the four lane groups, then the partial results of this split.
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    lrun[qt] += __shfl_xor(lrun[qt], 16, 64);
    lrun[qt] += __shfl_xor(lrun[qt], 32, 64);
    if (!qvalid[qt]) continue;
    const size_t qi = (size_t)trow[qt] * sh.hq + qhead[qt];
    float* op = opart + ((size_t)split * rows_total * sh.hq + qi) * HD;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) *(v4f*)(op + ht * 16 + g4 * 4) = oacc[ht][qt];
    if (g4 == 0) {
      float* ml = mlpart + ((size_t)split * rows_total * sh.hq + qi) * 2;
      ml[0] = mrun[qt];
      ml[1] = lrun[qt];
    }
  }
}

// bf16 attention with the K and V^T tiles of 32 keys brought from HBM straight
// into LDS by the load unit (global_load_lds: lane l of a load instruction
// writes its 16 bytes at offset 16 l of the instruction's 1 KB destination), in
// a ring of NST stages, so that NST - 1 tiles are in flight while one is
// computed and no register holds a tile on its way.  The loads bypass the
// compiler's wait bookkeeping (lds_dma16), so the loop waits for them itself: every
// thread issues the same LT loads per tile, so "tile t has landed" is "at most
// (NST - 2) LT of this thread's loads are outstanding" followed by one barrier,
// which also tells every wave that the stage about to be refilled (read in the
// previous iteration) is free.  Tiles past the end of the key range reload the
// last tile into the free stage, so every iteration issues the same loads.
//
// Layouts, chosen on the load side (a lane picks the source of the LDS slot it
// writes): a K row (one key, head_dim values) holds its 16-byte segments in the
// order s ^ kswz(key); a V^T row (one dimension, 32 keys) its four 16-byte
// segments in the order s ^ ((d >> 2) & 3).  Both make every fragment read one
// conflict-free 16-byte LDS load.  The score tile kt (16 keys) takes keys
// 8 (r >> 2) + 4 kt + (r & 3) for its row r, so that lane group g of the
// matrix core ends up holding keys 8 g .. 8 g + 7 of P: the natural order of a
// V^T row, read as one fragment.
//
// P enters the P V product as a bf16 high part and a bf16 remainder (p = hi + lo
// to 2^-18 relative), two products against the bf16 V tile: a single bf16 P
// would carry a relative error of up to 2^-9 into the output, enough to flip the
// output's bf16 rounding in a large share of its elements, and those flips then
// move everything downstream of the layer.  A row's reference maximum moves only
// when a tile's maximum exceeds it by more than 2^8 (so P <= 256), which keeps
// the rescaling of the running output rare.
// Two floats rounded to bf16 (nearest even) and packed, a in the low half: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}

template <int HD>
__device__ __forceinline__ int kswz(int key) {
  // 16 distinct values over the 16 keys of a score tile (4 bits, or 3 bits plus
  // the key's row parity at head_dim 64, where two key rows share 256 bytes)
  if constexpr (HD >= 128) return (key & 3) | (((key >> 3) & 3) << 2);
  else return ((key >> 1) & 1) | (((key >> 3) & 3) << 1);
}

template <int HD, int QT, int NST, int QR>
__global__ void __launch_bounds__(QR * 4 / QT, 1) k_attn_lds(const bf16_t* __restrict__ q, DgShape sh, DgSegs sg, int nqb,
                                                     int nsplit, float* __restrict__ opart, float* __restrict__ mlpart,
                                                     int rows_total) {
  typedef v8s F;
  constexpr int NKK = HD / 32;
  constexpr int NHT = HD / 16;
  constexpr int KSEG = HD / 8;            // 16-byte segments per key row
  constexpr int NTHR = QR * 4 / QT;       // QR query rows per block, QT m-tiles (16 rows) per wave
  constexpr int NW = NTHR / 64;
  constexpr int KB = 32 * HD * 2;         // bytes of a K tile (= bytes of a V^T tile)
  constexpr int KI = KB / 1024;           // 1 KB load instructions per tile and matrix
  static_assert(KI % NW == 0, "tile loads: whole instructions per wave");
  constexpr int LK = KI / NW;             // per wave (and thread) and matrix
  constexpr int LT = 2 * LK;              // loads per thread per tile
  static_assert((NST - 2) * LT <= 63, "vmcnt range");
  // One array per stage, every stage index a compile-time constant.
  static_assert(NST == 4, "four stages");
  __shared__ uint4 sK0[KB / 16], sK1[KB / 16], sK2[KB / 16], sK3[KB / 16];
  __shared__ uint4 sV0[KB / 16], sV1[KB / 16], sV2[KB / 16], sV3[KB / 16];
  auto stK = [&](auto J) __attribute__((always_inline)) -> uint4* {
    constexpr int j = decltype(J)::value;
    if constexpr (j == 0) return sK0; else if constexpr (j == 1) return sK1; else if constexpr (j == 2) return sK2;
    else return sK3;
  };
  auto stV = [&](auto J) __attribute__((always_inline)) -> uint4* {
    constexpr int j = decltype(J)::value;
    if constexpr (j == 0) return sV0; else if constexpr (j == 1) return sV1; else if constexpr (j == 2) return sV2;
    else return sV3;
  };
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g4 = lane >> 4, c16 = lane & 15;

  int bid = blockIdx.x;
  const int split = bid % nsplit;
  bid /= nsplit;
  const int qb = bid % nqb;
  bid /= nqb;
  const int h = bid % sh.hkv;
  const int si = bid / sh.hkv;
  if (si >= sg.count) return;
  const DgSeg seg = sg.s[si];
  const int G = sh.hq / sh.hkv;
  const int nq = G * seg.n;
  if (qb * QR >= nq) return;  // uniform over the block
  const int qr0 = qb * QR + wave * 16 * QT;
  const bool wave_active = qr0 < nq;

  int qhead[QT], trow[QT], qpos[QT];
  bool qvalid[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int qr = qr0 + qt * 16 + c16;
    qvalid[qt] = qr < nq;
    const int qrc = qvalid[qt] ? qr : nq - 1;
    const int hg = qrc / seg.n, i = qrc - hg * seg.n;
    qhead[qt] = h * G + hg;
    trow[qt] = seg.row0 + i;
    qpos[qt] = seg.pos0 + i;
  }
  const int nkeys = seg.nkeys;
  const int chunk = ((nkeys + nsplit - 1) / nsplit + 31) / 32 * 32;
  const int k_lo = split * chunk;
  int k_hi = min(nkeys, k_lo + chunk);
  if (sg.causal) {
    // largest position among the block's rows (block-uniform)
    const int first = qb * QR, last = min(first + QR, nq) - 1;
    const int max_i = (first / seg.n == last / seg.n) ? last % seg.n : seg.n - 1;
    k_hi = min(k_hi, seg.pos0 + max_i + 1);
  }
  const int ntiles = k_hi > k_lo ? (k_hi - k_lo + 31) / 32 : 0;

  F qf[QT][NKK];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const char* qp = (const char*)(q + (size_t)trow[qt] * (sh.hq * HD) + qhead[qt] * HD) + g4 * 16;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qf[qt][kk] = *(const F*)(qp + kk * 64);
  }

  const bf16_t* kbase = (const bf16_t*)seg.k + (size_t)h * sh.max_ctx * HD;
  const bf16_t* vbase = (const bf16_t*)seg.vt + (size_t)h * HD * sh.max_ctx;
  const float scale = 1.4426950408889634f / sqrtf((float)HD);

  // This thread's sources for tile t (clamped to the last tile of the range;
  // keys past the last key re-read it), written to stage (sk, sv).
  auto issue = [&](int t, uint4* sk, uint4* sv) __attribute__((always_inline)) {
    const int kb = k_lo + 32 * min(t, ntiles - 1);
#pragma unroll
    for (int i = 0; i < LK; ++i) {
      const int ins = wave * LK + i;                 // 1 KB instruction within the tile
      const int slot = ins * 64 + lane;              // 16-byte slot of the tile in LDS
      const int key = slot / KSEG, ps = slot % KSEG;  // physical segment of that key row
      const int sgi = ps ^ kswz<HD>(key);
      const int gk = min(kb + key, nkeys - 1);
      lds_dma16(kbase + (size_t)gk * HD + sgi * 8, sk + ins * 64);
    }
#pragma unroll
    for (int i = 0; i < LK; ++i) {
      const int ins = wave * LK + i;
      const int slot = ins * 64 + lane;
      const int d = slot >> 2, ps = slot & 3;
      const int s4 = ps ^ ((d >> 2) & 3);
      lds_dma16(vbase + (size_t)d * sh.max_ctx + kb + s4 * 8, sv + ins * 64);
    }
  };

  v4f oacc[NHT][QT];
  float mrun[QT], lrun[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) oacc[ht][qt] = v4f{0.f, 0.f, 0.f, 0.f};
    mrun[qt] = -INFINITY;
    lrun[qt] = 0.f;
  }
  constexpr float RESCALE_TH = 8.f;
  int klim[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) klim[qt] = sg.causal ? min(k_hi, qpos[qt] + 1) : k_hi;

  // One tile from stage (sk, sv): scores, softmax update, P V.
  auto tile = [&](int kb, const uint4* sk, const uint4* sv) __attribute__((always_inline)) {
    v4f sc4[2][QT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) sc4[kt][qt] = v4f{0.f, 0.f, 0.f, 0.f};
      const int key = 8 * (c16 >> 2) + 4 * kt + (c16 & 3);  // this lane's key row of score tile kt
      const int sw = kswz<HD>(key);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const uint4 u = sk[key * KSEG + ((kk * 4 + g4) ^ sw)];
        const F kf = *reinterpret_cast<const F*>(&u);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          sc4[kt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qt][kk], sc4[kt][qt], 0, 0, 0);
      }
    }
    // lane (g4, c16) holds, for query column c16, keys 8 g4 + 4 kt + i.  The
    // maximum is taken on the raw scores (scale > 0, so it is the scaled
    // maximum exactly once scaled) and the scale goes into the exponent's fma;
    // tiles that lie below every row's key limit skip the mask.
    float p[2][QT][4];
    bool grow = false;
    float alpha[QT];
    bool below = true;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) below &= kb + 32 <= klim[qt];
    float tmx[QT];
    auto scan = [&](auto MASK) __attribute__((always_inline)) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        float tmax = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float sv = sc4[kt][qt][i];
            if constexpr (decltype(MASK)::value) p[kt][qt][i] = kb + 8 * g4 + 4 * kt + i < klim[qt] ? sv : -INFINITY;
            else p[kt][qt][i] = sv;
            tmax = fmaxf(tmax, p[kt][qt][i]);
          }
        tmx[qt] = tmax;
      }
    };
    if (__all(below)) scan(std::false_type{});  // wave-uniform
    else scan(std::true_type{});
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float tmax = tmx[qt];
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * scale;
      const bool move = tmax > mrun[qt] + RESCALE_TH;
      const float mnew = move ? tmax : mrun[qt];
      alpha[qt] = move ? __builtin_amdgcn_exp2f(mrun[qt] - mnew) : 1.f;  // 2^-inf = 0 on the first move
      grow |= move;
      mrun[qt] = mnew;
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(p[kt][qt][i], scale, -mref));
          p[kt][qt][i] = e;
          psum += e;
        }
      lrun[qt] = lrun[qt] * alpha[qt] + psum;
    }
    if (__any(grow)) {  // wave-uniform; rare after the first tile
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) oacc[ht][qt] *= alpha[qt];
    }
    // P = hi + lo, both bf16 (round to nearest even, two values per
    // conversion instruction)
    F pf[QT], pl[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v0 = p[j >> 1][qt][2 * (j & 1)], v1 = p[j >> 1][qt][2 * (j & 1) + 1];
        const uint32_t h = bf16x2_rne(v0, v1);
        hw[j] = h;
        lw[j] = bf16x2_rne(v0 - __uint_as_float(h << 16), v1 - __uint_as_float(h & 0xffff0000u));
      }
      const uint4 hu = make_uint4(hw[0], hw[1], hw[2], hw[3]), lu = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      pf[qt] = *reinterpret_cast<const F*>(&hu);
      pl[qt] = *reinterpret_cast<const F*>(&lu);
    }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int d = ht * 16 + c16;
      const uint4 u = sv[d * 4 + (g4 ^ ((d >> 2) & 3))];
      const F vf = *reinterpret_cast<const F*>(&u);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        oacc[ht][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[qt], oacc[ht][qt], 0, 0, 0);
        oacc[ht][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pl[qt], oacc[ht][qt], 0, 0, 0);
      }
    }
  };

  if (ntiles > 0) {
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    issue(0, stK(I0{}), stV(I0{}));
    issue(1, stK(I1{}), stV(I1{}));
    issue(2, stK(I2{}), stV(I2{}));
    // The query fragments must have landed before the loop: the compiler's
    // own wait for them would otherwise sit inside it, where (not knowing of
    // the ring's loads) it would drain the ring every tile.  Waiting here, after
    // the first three tiles' copies are issued, overlaps the two latencies
    // (the wait covers those copies too).
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) asm volatile("" ::"v"(qf[qt][kk]));
    // Tile t sits in stage t % 4; its step refills stage (t + 3) % 4, read by
    // the step before (every wave has passed the barrier since).
    auto step = [&](int t, auto J, auto JN) __attribute__((always_inline)) {
      if (t >= ntiles) return;        // block-uniform
      DG_WAIT_VMCNT((NST - 2) * LT);  // this thread's loads of tile t have landed
      __builtin_amdgcn_s_barrier();   // ... everyone's, and stage (t + 3) % 4 is free
      issue(t + NST - 1, stK(JN), stV(JN));
      if (wave_active) tile(k_lo + 32 * t, stK(J), stV(J));
    };
    for (int t0 = 0; t0 < ntiles; t0 += 4) {
      step(t0, I0{}, I3{});
      step(t0 + 1, I1{}, I0{});
      step(t0 + 2, I2{}, I1{});
      step(t0 + 3, I3{}, I2{});
    }
    DG_WAIT_VMCNT(0);  // the tail reloads have landed before the block leaves
  }
  if (!wave_active) return;
  // The split's output leaves normalised (O / l, at most max |v| in size) in
  // fp32; the merge weighs it by l 2^(m - M).
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    lrun[qt] += __shfl_xor(lrun[qt], 16, 64);
    lrun[qt] += __shfl_xor(lrun[qt], 32, 64);
    if (!qvalid[qt]) continue;
    const size_t qi = (size_t)trow[qt] * sh.hq + qhead[qt];
    const float inv = lrun[qt] > 0.f ? 1.f / lrun[qt] : 0.f;
    float* op = opart + ((size_t)split * rows_total * sh.hq + qi) * HD;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) *(v4f*)(op + ht * 16 + g4 * 4) = oacc[ht][qt] * inv;
    if (g4 == 0) {
      float* ml = mlpart + ((size_t)split * rows_total * sh.hq + qi) * 2;
      ml[0] = mrun[qt];
      ml[1] = lrun[qt];
    }
  }
}

// Merge the splits of each (row, q-head): O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,
// written row-major or (FM, bf16) fragment-major with hq * hd columns (fm_index).
// P: element type of the split outputs; NORM: they hold O_s / l_s (weighed by l_s).
template <typename T, bool FM, typename P = float, bool NORM = false>
__global__ void __launch_bounds__(64) k_attn_merge(const float* __restrict__ opart_f, const float* __restrict__ mlpart,
                                                   int nsplit, int rows_total, int hq, int hd, T* __restrict__ o) {
  // One wave per (row, q-head).  Lane s reads split s's (m, l) (nsplit <= 64),
  // the wave reduces M and L, and each lane keeps its split's weight; then
  // every lane merges four columns, the loads of all splits in flight at once.
  const P* opart = reinterpret_cast<const P*>(opart_f);
  const size_t qi = blockIdx.x;  // row * hq + qhead
  const int lane = threadIdx.x;
  const size_t sstride = (size_t)rows_total * hq;
  float m = -INFINITY, l = 0.f;
  if (lane < nsplit) {
    const float2 ml = *reinterpret_cast<const float2*>(mlpart + ((size_t)lane * sstride + qi) * 2);
    m = ml.x;
    l = ml.y;
  }
  float M = m;
#pragma unroll
  for (int o2 = 32; o2 > 0; o2 >>= 1) M = fmaxf(M, __shfl_xor(M, o2, 64));
  const float e = l > 0.f ? exp2f(m - M) : 0.f;
  const float w_own = NORM ? e * l : e;
  float L = e * l;
#pragma unroll
  for (int o2 = 32; o2 > 0; o2 >>= 1) L += __shfl_xor(L, o2, 64);
  const float invL = 1.f / L;
  const int row = (int)(qi / hq), col0 = (int)(qi % hq) * hd;
  for (int c = 4 * lane; c < hd; c += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int sp = 0; sp < nsplit; ++sp) {
      const float w = __shfl(w_own, sp, 64);
      const P* src = opart + ((size_t)sp * sstride + qi) * hd + c;
      float4 v;
      if constexpr (sizeof(P) == 2) {
        typedef _Float16 v4h __attribute__((ext_vector_type(4)));
        const v4h h = *reinterpret_cast<const v4h*>(src);
        v = make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
      } else {
        v = *reinterpret_cast<const float4*>(src);
      }
      acc.x += w * v.x;
      acc.y += w * v.y;
      acc.z += w * v.z;
      acc.w += w * v.w;
    }
    T* dst = o + (FM ? fm_index(row, col0 + c, hq * hd) : qi * hd + c);
    dst[0] = from_f<T>(acc.x * invL);
    dst[1] = from_f<T>(acc.y * invL);
    dst[2] = from_f<T>(acc.z * invL);
    dst[3] = from_f<T>(acc.w * invL);
  }
}

// Query rows per block of the attention kernels (k_attn_lds for bf16).
int dg_attn_qrows(int dtype, int hd) { return ATTN_QROWS; }
// m-tiles per wave of k_attn_lds at head_dim 256: 1 (eight waves, two per SIMD)
// or 2 (four waves, one per SIMD with its whole register file, every K and V^T
// fragment read from LDS serving two m-tiles; measured slower: with one wave per
// SIMD nothing hides the latencies -- 72 against 54 us per layer with the merge).
// Two m-tiles with eight waves do not fit the 256 registers a wave then has.
#ifndef DG_ATTN_QT256
#define DG_ATTN_QT256 1
#endif

int dg_attn_splits(const DgSegs& segs, const DgShape& sh, int max_splits, int qrows) {
  int base = 0, maxkeys = 0;
  const int G = sh.hq / sh.hkv;
  for (int i = 0; i < segs.count; ++i) {
    base += sh.hkv * ((G * segs.s[i].n + qrows - 1) / qrows);
    maxkeys = maxkeys > segs.s[i].nkeys ? maxkeys : segs.s[i].nkeys;
  }
  // One block per CU at the full head size: aim at 256 blocks, each split at
  // least 8 key tiles long (fewer splits also means fewer partials to merge).
  int ns = (256 + base - 1) / (base > 0 ? base : 1);
  const int by_keys = (maxkeys + 255) / 256;
  if (ns > by_keys) ns = by_keys;
  if (ns > max_splits) ns = max_splits;
  if (ns < 1) ns = 1;
  return ns;
}

void dg_launch_attention(int dtype, const void* q, const DgShape& sh, const DgSegs& segs, int nsplit, float* opart,
                         float* mlpart, void* o, int rows, hipStream_t s) {
  if (rows <= 0) return;
  const int G = sh.hq / sh.hkv;
  int nmax = 0;
  for (int i = 0; i < segs.count; ++i) nmax = nmax > segs.s[i].n ? nmax : segs.s[i].n;
  const int qrows = dg_attn_qrows(dtype, sh.hd);
  const int nqb = (G * nmax + qrows - 1) / qrows;
  const int blocks = segs.count * sh.hkv * nqb * nsplit;
#define DG_ATTN(TT, HDV)                                                                                     \
  k_attn<TT, HDV><<<blocks, 256, 0, s>>>((const TT*)q, sh, segs, nqb, nsplit, opart, mlpart, rows);         \
  k_attn_merge<TT, sizeof(TT) == 2><<<rows * sh.hq, 64, 0, s>>>(opart, mlpart, nsplit, rows, sh.hq, HDV, (TT*)o)
// LDS stages of the tile ring (NST - 1 tiles in flight): 4 x 32 KB at head_dim 256.
#ifndef DG_ATTN_NST
#define DG_ATTN_NST 4
#endif
// m-tiles (16 query rows) per wave: one at head_dim 128 (eight waves, two per
// SIMD, half the registers each), two at 64 (the tile staging needs 256
// threads), DG_ATTN_QT256 at 256
#define DG_ATTN_QT(HDV) ((HDV) == 128 ? 1 : (HDV) == 256 ? DG_ATTN_QT256 : 2)
#define DG_ATTN_QRT(HDV) ATTN_QROWS
#define DG_ATTN_LDS(HDV)                                                                                    \
  k_attn_lds<HDV, DG_ATTN_QT(HDV), DG_ATTN_NST, DG_ATTN_QRT(HDV)>                                                   \
      <<<blocks, DG_ATTN_QRT(HDV) * 4 / DG_ATTN_QT(HDV), 0, s>>>((const bf16_t*)q, sh, segs, nqb, nsplit, opart,    \
                                                                  mlpart, rows);                                    \
  k_attn_merge<bf16_t, true, float, true><<<rows * sh.hq, 64, 0, s>>>(opart, mlpart, nsplit, rows, sh.hq, HDV,     \
                                                                       (bf16_t*)o)
  if (dtype == 1) {
    if (sh.hd == 256) { DG_ATTN_LDS(256); }
    else if (sh.hd == 128) { DG_ATTN_LDS(128); }
    else if (sh.hd == 64) { DG_ATTN_LDS(64); }
    else { DG_ATTN(bf16_t, 32); }
  } else {
    if (sh.hd == 256) { DG_ATTN(float, 256); }
    else if (sh.hd == 128) { DG_ATTN(float, 128); }
    else if (sh.hd == 64) { DG_ATTN(float, 64); }
    else if (sh.hd == 32) { DG_ATTN(float, 32); }
    else { DG_ATTN(float, 16); }
  }
#undef DG_ATTN
#undef DG_ATTN_LDS
#undef DG_ATTN_QT
#undef DG_ATTN_QRT
}
