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

// Two bf16 values (low half first) to two fp16 values: exact over fp16's normal
// range (bf16 has 8 significant bits); the conversion rounds toward zero, which
// only touches magnitudes below that range and clamps those above it to 65504.
__device__ __forceinline__ uint32_t bf2_to_h2(uint32_t u) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
  return *reinterpret_cast<const uint32_t*>(&h);
}

// bf16 attention with the K and V^T tiles of 32 keys staged in LDS once per
// block and shared by its four waves (the kernel above reads them once per wave).
// The next tile is prefetched into registers while the current one is used, and
// written to the other of two LDS stages.  K rows are XOR-swizzled in 16-byte
// units (key & 15, or key & 7 at head_dim 64); each V^T row holds its 32 keys in the order the score tiles
// deliver them (lane group g of the matrix core covers keys 4g..4g+3 and
// 16+4g..16+4g+3) and is swizzled by ((row >> 1) & 3), so every fragment read
// is one conflict-free 16-byte LDS load.  All waves of a block walk the same
// key tiles; the key range is cut at the largest position among the block's
// rows when the mask is causal.
//
// The probabilities P enter the P V product as an fp16 high part plus an fp16
// remainder (two products) against V converted to fp16 when its tile is staged:
// a bf16 value has 8 significant bits, so the conversion is exact over fp16's
// normal range; magnitudes below it keep an absolute error under 2^-25 and
// magnitudes above 65504 are clamped to it.  A row's reference maximum moves
// only when a tile's maximum exceeds it by more than 2^8 (so P <= 256), which
// keeps the rescaling of the running output rare.
template <int HD, int QT>
__global__ void __launch_bounds__(512 / QT, 1) k_attn_lds(const bf16_t* __restrict__ q, DgShape sh, DgSegs sg, int nqb,
                                                     int nsplit, float* __restrict__ opart, float* __restrict__ mlpart,
                                                     int rows_total) {
  typedef v8s F;
  constexpr int NKK = HD / 32;
  constexpr int NHT = HD / 16;
  constexpr int KSEG = HD / 8;            // 16-byte segments per key row
  constexpr int KSW = KSEG >= 16 ? 15 : 7;  // K-row swizzle: XOR of the segment with the key's low bits
  constexpr int SEGS_K = 32 * KSEG;       // per tile
  constexpr int SEGS_V = HD * 4;          // per tile (HD rows of 32 keys)
  constexpr int NTHR = 512 / QT;         // 128 query rows per block, QT m-tiles per wave
  constexpr int LK = SEGS_K / NTHR, LV = SEGS_V / NTHR;
  static_assert(LK >= 1 && LV >= 1, "tile staging: head_dim too small for this wave count");
  __shared__ uint4 sK[2][SEGS_K];
  __shared__ uint4 sV[2][SEGS_V];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
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
  if (qb * ATTN_QROWS >= nq) return;  // uniform over the block
  const int qr0 = qb * ATTN_QROWS + wave * 16 * QT;
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
    const int first = qb * ATTN_QROWS, last = min(first + ATTN_QROWS, nq) - 1;
    const int max_i = (first / seg.n == last / seg.n) ? last % seg.n : seg.n - 1;
    k_hi = min(k_hi, seg.pos0 + max_i + 1);
  }

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

  // This thread's segments of a tile.
  auto load_tile = [&](int kb, uint4 (&rk)[LK], uint4 (&rv)[LV]) {
#pragma unroll
    for (int i = 0; i < LK; ++i) {
      const int sid = tid + NTHR * i, key = sid / KSEG, sgi = sid % KSEG;
      const int gk = min(kb + key, nkeys - 1);
      rk[i] = *(const uint4*)(kbase + (size_t)gk * HD + sgi * 8);
    }
#pragma unroll
    for (int i = 0; i < LV; ++i) {
      const int sid = tid + NTHR * i, d = sid >> 2, s4 = sid & 3;
      rv[i] = *(const uint4*)(vbase + (size_t)d * sh.max_ctx + kb + s4 * 8);
    }
  };
  auto store_tile = [&](int stg, const uint4 (&rk)[LK], const uint4 (&rv)[LV]) {
#pragma unroll
    for (int i = 0; i < LK; ++i) {
      const int sid = tid + NTHR * i, key = sid / KSEG, sgi = sid % KSEG;
      sK[stg][key * KSEG + (sgi ^ (key & KSW))] = rk[i];
    }
    uint2* v8 = reinterpret_cast<uint2*>(sV[stg]);
#pragma unroll
    for (int i = 0; i < LV; ++i) {
      const int sid = tid + NTHR * i, d = sid >> 2, s4 = sid & 3;
      const int kt = s4 >> 1, g0 = (s4 & 1) * 2, sw = (d >> 1) & 3;
      v8[d * 8 + (g0 ^ sw) * 2 + kt] = make_uint2(bf2_to_h2(rv[i].x), bf2_to_h2(rv[i].y));        // keys 8 s4 .. +3
      v8[d * 8 + ((g0 + 1) ^ sw) * 2 + kt] = make_uint2(bf2_to_h2(rv[i].z), bf2_to_h2(rv[i].w));  // keys 8 s4 + 4 .. +7
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

  uint4 rk[LK], rv[LV];
  if (k_lo < k_hi) {
    load_tile(k_lo, rk, rv);
    store_tile(0, rk, rv);
  }
  __syncthreads();
  int stg = 0;
  // The reference maximum of a row (mrun) moves only when a tile's maximum
  // exceeds it by more than RESCALE_TH (log2 units): P = 2^(s - mrun) then stays
  // at most 2^RESCALE_TH, well inside fp16, and the running output and sum are
  // rescaled rarely instead of on almost every tile.  The split's (mrun, lrun)
  // pair is reported with its output, so the merge stays exact.
  constexpr float RESCALE_TH = 8.f;
  // Keys at or beyond klim[qt] are masked for row qt: the end of the range, and
  // with a causal mask the row's own position + 1.
  int klim[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) klim[qt] = sg.causal ? min(k_hi, qpos[qt] + 1) : k_hi;
  // One tile: scores, softmax update, P V.
  auto tile = [&](int kb) {
    v4f st[2][QT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) st[kt][qt] = v4f{0.f, 0.f, 0.f, 0.f};
      const int key = kt * 16 + c16;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const uint4 u = sK[stg][key * KSEG + ((kk * 4 + g4) ^ (key & KSW))];
        const F kf = *reinterpret_cast<const F*>(&u);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
          st[kt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qt][kk], st[kt][qt], 0, 0, 0);
      }
    }
    float p[2][QT][4];
    bool grow = false;
    float alpha[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float tmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kb + kt * 16 + g4 * 4 + i;
          const float sc = key < klim[qt] ? st[kt][qt][i] * scale : -INFINITY;
          p[kt][qt][i] = sc;
          tmax = fmaxf(tmax, sc);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      // a row's reference moves to its tile maximum when that exceeds it by more
      // than the threshold (always on the row's first unmasked tile)
      const bool move = tmax > mrun[qt] + RESCALE_TH;
      const float mnew = move ? tmax : mrun[qt];
      alpha[qt] = move ? __builtin_amdgcn_exp2f(mrun[qt] - mnew) : 1.f;  // 2^-inf = 0 on the first move
      grow |= move;
      mrun[qt] = mnew;
      // rows with every score masked so far keep mrun = -inf: their P is 0
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(p[kt][qt][i] - mref);
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
    // P enters the matrix cores as an fp16 high part and an fp16 remainder
    // (p = hi + lo to about 2^-22 relative), two products against the same V
    // tile: one fp16 P would carry a relative error of up to 2^-12 into the
    // output, enough to flip the output's bf16 rounding in about one element in
    // eight, and those flips then move everything downstream of the layer.
    v8h pf[QT], pl[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = p[kt][qt][i];
          const _Float16 hi = (_Float16)v;
          pf[qt][kt * 4 + i] = hi;
          pl[qt][kt * 4 + i] = (_Float16)(v - (float)hi);
        }
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int d = ht * 16 + c16;
      const uint4 u = sV[stg][d * 4 + (g4 ^ ((d >> 1) & 3))];
      const v8h vf = *reinterpret_cast<const v8h*>(&u);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        oacc[ht][qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[qt], oacc[ht][qt], 0, 0, 0);
        oacc[ht][qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pl[qt], oacc[ht][qt], 0, 0, 0);
      }
    }
  };
  for (int kb = k_lo; kb < k_hi; kb += 32) {
    const bool more = kb + 32 < k_hi;
    load_tile(more ? kb + 32 : kb, rk, rv);
    if (wave_active) tile(kb);
    store_tile(stg ^ 1, rk, rv);
    __syncthreads();
    stg ^= 1;
  }
  if (!wave_active) return;
  // The split's output leaves normalised (O / l, at most max |v| in size) in
  // fp32: an fp16 copy would add a 2^-12 relative error ahead of the output's
  // bf16 rounding (see the P product above).  The merge weighs it by
  // l 2^(m - M).
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

int dg_attn_splits(const DgSegs& segs, const DgShape& sh, int max_splits) {
  int base = 0, maxkeys = 0;
  const int G = sh.hq / sh.hkv;
  for (int i = 0; i < segs.count; ++i) {
    base += sh.hkv * ((G * segs.s[i].n + ATTN_QROWS - 1) / ATTN_QROWS);
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
  const int nqb = (G * nmax + ATTN_QROWS - 1) / ATTN_QROWS;
  const int blocks = segs.count * sh.hkv * nqb * nsplit;
#define DG_ATTN(TT, HDV)                                                                                     \
  k_attn<TT, HDV><<<blocks, 256, 0, s>>>((const TT*)q, sh, segs, nqb, nsplit, opart, mlpart, rows);         \
  k_attn_merge<TT, sizeof(TT) == 2><<<rows * sh.hq, 64, 0, s>>>(opart, mlpart, nsplit, rows, sh.hq, HDV, (TT*)o)
// m-tiles (16 query rows) per wave: one at head_dim >= 128 (eight waves, two per
// SIMD, half the registers each), two at 64 (the tile staging needs 256 threads)
#define DG_ATTN_QT(HDV) ((HDV) >= 128 ? 1 : 2)
#define DG_ATTN_LDS(HDV)                                                                                    \
  k_attn_lds<HDV, DG_ATTN_QT(HDV)><<<blocks, 512 / DG_ATTN_QT(HDV), 0, s>>>((const bf16_t*)q, sh, segs, nqb, nsplit,    \
                                                                           opart, mlpart, rows);                   \
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
}
