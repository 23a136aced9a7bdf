// Plain C++17 / OpenMP CPU oracle of one block-diffusion denoising step.
//
// TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
// CPU-baseline leg of the bench; the GPU library neither links nor includes it.
// A second, independent implementation of what the numpy oracle (oracle/*.py)
// computes, written for clarity, not speed: double precision throughout, one
// output element per loop body, OpenMP across rows or output columns only.
//
// What it computes (each part cites the passage it follows):
//  * the decoder ("Google open-sources DiffusionGemma: H100 reaches 1000 TPS",
//    section "26B MoE Architecture, but Only 3.8B Activated"; "DiffusionGemma
//    Hits 1,000 Tokens per Second", section "The speed numbers and the hardware
//    they require"): pre-norm blocks, grouped-query attention that every canvas
//    token runs over its whole context (no mask), a mixture of experts with
//    top-k routing plus one shared expert, the tied LM head;
//  * the denoising step ("DiffusionGemma hits ~1,500 TPS on one H100",
//    sections "What DiffusionGemma is" and "How the sampler actually works"):
//    candidate = argmax per position, entropy-bound acceptance (the threshold
//    reading: entropy strictly below tau, plus the lowest-entropy open
//    position), re-randomisation of the rest, step cap;
//  * the block commit ("DiffusionGemma Hits 1,000 Tokens per Second", section
//    "How diffusion text generation changes the bottleneck"): the final
//    canvas's K/V enter the cache and the committed length grows by a canvas.
//  Readings where the pages are silent (RMSNorm, rotate-half RoPE, causal
//  prompt mask, softmax over the kept router logits, unscaled embedding,
//  Philox4x64-10 counter layout, token = high 64 bits of r0 * V) are those of
//  the numpy oracle.  With bf16_points set, the operands a bf16 model stores in
//  bf16 (normalised rows, q / k after RoPE, v, the attention output, the SwiGLU
//  hidden rows, the final normalised rows) are rounded to bf16 (nearest, ties to
//  even) there; everything else stays double.
//
// Parity pins: tests/test_oracle_cxx.py checks it against the numpy oracle
// (tiny model: a whole generation, mid shape: a step through all layers) and
// against closed forms.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

struct Cfg {
  int vocab, d, L, hq, hkv, hd, E, k, eh, sh, C;
  double theta, eps;
  int bf16_points;
  int wdtype;  // 0: weights float32, 1: weights bf16
};

// Weight element i of a float32 or bf16 array, as double (bf16: exact).
inline double wget(const void* p, size_t i, int wdtype) {
  if (wdtype == 0) return (double)((const float*)p)[i];
  uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return (double)f;
}

// Round to float32, then to the nearest bf16 (ties to even), returned as double.
inline double rbf16(double x) {
  float f = (float)x;
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) != 0x7f800000u) u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
  std::memcpy(&f, &u, 4);
  return (double)f;
}
inline double rp(double x, const Cfg& c) { return c.bf16_points ? rbf16(x) : x; }

struct Layer {
  const void *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm, *router, *w1, *w3, *w2, *sw1, *sw3, *sw2;
};

// y = x / sqrt(mean(x^2) + eps) * g
void rmsnorm(const double* x, int d, const void* g, int wdtype, double eps, double* y) {
  double ms = 0;
  for (int i = 0; i < d; ++i) ms += x[i] * x[i];
  ms /= d;
  const double inv = 1.0 / std::sqrt(ms + eps);
  for (int i = 0; i < d; ++i) y[i] = x[i] * inv * wget(g, i, wdtype);
}

// out[t][n] = sum_k a[t][k] W[n][k], W row-major [N][K] starting at element w0.
void matmul(const double* a, int T, int K, const void* W, size_t w0, int N, int wdtype, double* out) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int t = 0; t < T; ++t)
    for (int n = 0; n < N; ++n) {
      double s = 0;
      const size_t row = w0 + (size_t)n * K;
      for (int kk = 0; kk < K; ++kk) s += a[(size_t)t * K + kk] * wget(W, row + kk, wdtype);
      out[(size_t)t * N + n] = s;
    }
}

// Rotate-half RoPE of one head vector at absolute position pos.
void rope(double* v, int hd, double pos, double theta) {
  const int half = hd / 2;
  for (int j = 0; j < half; ++j) {
    const double ang = pos * std::pow(theta, -2.0 * j / hd);
    const double c = std::cos(ang), s = std::sin(ang);
    const double x1 = v[j], x2 = v[j + half];
    v[j] = x1 * c - x2 * s;
    v[j + half] = x2 * c + x1 * s;
  }
}

double silu(double x) { return x / (1.0 + std::exp(-x)); }

// Indices of the k largest of r (as float32 values), largest first, ties to the
// lower index: repeated selection of the first maximum.
void topk(const double* r, int E, int k, int* ids) {
  std::vector<float> w(E);
  for (int e = 0; e < E; ++e) w[e] = (float)r[e];
  for (int j = 0; j < k; ++j) {
    int best = -1;
    for (int e = 0; e < E; ++e)
      if (w[e] == w[e] && (best < 0 || w[e] > w[best])) best = e;
    if (best < 0) best = 0;
    ids[j] = best;
    w[best] = -INFINITY;
  }
}

// SwiGLU expert over rows b [T][d]: out[t] = W2 (silu(W1 b) * (W3 b)), with
// stacked weights at element offsets o1 / o3 ([eh][d]) and o2 ([d][eh]).
void swiglu(const double* b, int T, const Cfg& c, int hidden, const void* w1, size_t o1, const void* w3, size_t o3,
            const void* w2, size_t o2, double* out) {
  std::vector<double> u((size_t)T * hidden), v((size_t)T * hidden);
  matmul(b, T, c.d, w1, o1, hidden, c.wdtype, u.data());
  matmul(b, T, c.d, w3, o3, hidden, c.wdtype, v.data());
  for (size_t i = 0; i < u.size(); ++i) u[i] = rp(silu(u[i]) * v[i], c);
  matmul(u.data(), T, hidden, w2, o2, c.d, c.wdtype, out);
}

// One decoder layer over T rows x [T][d] at positions pos, attending to the
// prefix kp / vp ([P][hkv][hd]) and to its own rows (causal: row i sees prefix
// keys and own rows j <= i).  Writes the post-RoPE k / v of its rows
// ([T][hkv][hd]) and, unless skip_ffn, the router logits [T][E], ids and gates
// [T][k].  x is updated in place.
void layer(const Cfg& c, const Layer& w, double* x, int T, const int* pos, const double* kp, const double* vp,
           int P, int causal, int skip_ffn, double* kout, double* vout, double* rlog, int* ids, double* gates) {
  const int d = c.d, hq = c.hq, hkv = c.hkv, hd = c.hd, qd = hq * hd, kvd = hkv * hd;
  std::vector<double> a((size_t)T * d), q((size_t)T * qd), kk((size_t)T * kvd), vv((size_t)T * kvd);
  for (int t = 0; t < T; ++t) {
    rmsnorm(x + (size_t)t * d, d, w.attn_norm, c.wdtype, c.eps, &a[(size_t)t * d]);
    for (int i = 0; i < d; ++i) a[(size_t)t * d + i] = rp(a[(size_t)t * d + i], c);
  }
  matmul(a.data(), T, d, w.wq, 0, qd, c.wdtype, q.data());
  matmul(a.data(), T, d, w.wk, 0, kvd, c.wdtype, kk.data());
  matmul(a.data(), T, d, w.wv, 0, kvd, c.wdtype, vv.data());
  for (int t = 0; t < T; ++t) {
    for (int h = 0; h < hq; ++h) {
      rope(&q[(size_t)t * qd + h * hd], hd, pos[t], c.theta);
      for (int j = 0; j < hd; ++j) q[(size_t)t * qd + h * hd + j] = rp(q[(size_t)t * qd + h * hd + j], c);
    }
    for (int h = 0; h < hkv; ++h) {
      rope(&kk[(size_t)t * kvd + h * hd], hd, pos[t], c.theta);
      for (int j = 0; j < hd; ++j) {
        kk[(size_t)t * kvd + h * hd + j] = rp(kk[(size_t)t * kvd + h * hd + j], c);
        vv[(size_t)t * kvd + h * hd + j] = rp(vv[(size_t)t * kvd + h * hd + j], c);
      }
    }
  }
  std::memcpy(kout, kk.data(), kk.size() * 8);
  std::memcpy(vout, vv.data(), vv.size() * 8);
  // attention: softmax(q k^T / sqrt(hd)) v per query head, kv-head h / (hq / hkv)
  std::vector<double> o((size_t)T * qd);
  const int group = hq / hkv;
  const double scale = 1.0 / std::sqrt((double)hd);
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int t = 0; t < T; ++t)
    for (int h = 0; h < hq; ++h) {
      const int g = h / group;
      const int nvis = causal ? P + t + 1 : P + T;
      std::vector<double> sc(nvis);
      const double* qv = &q[(size_t)t * qd + h * hd];
      double m = -INFINITY;
      for (int j = 0; j < nvis; ++j) {
        const double* kv = j < P ? kp + ((size_t)j * hkv + g) * hd : &kk[(size_t)(j - P) * kvd + g * hd];
        double s = 0;
        for (int e = 0; e < hd; ++e) s += qv[e] * kv[e];
        sc[j] = s * scale;
        m = std::max(m, sc[j]);
      }
      double den = 0;
      for (int j = 0; j < nvis; ++j) {
        sc[j] = std::exp(sc[j] - m);
        den += sc[j];
      }
      double* ov = &o[(size_t)t * qd + h * hd];
      for (int e = 0; e < hd; ++e) ov[e] = 0;
      for (int j = 0; j < nvis; ++j) {
        const double* vr = j < P ? vp + ((size_t)j * hkv + g) * hd : &vv[(size_t)(j - P) * kvd + g * hd];
        const double p = sc[j] / den;
        for (int e = 0; e < hd; ++e) ov[e] += p * vr[e];
      }
    }
  for (auto& e : o) e = rp(e, c);
  std::vector<double> ao((size_t)T * d);
  matmul(o.data(), T, qd, w.wo, 0, d, c.wdtype, ao.data());
  for (size_t i = 0; i < ao.size(); ++i) x[i] += ao[i];
  if (skip_ffn) return;
  // mixture of experts
  std::vector<double> b((size_t)T * d);
  for (int t = 0; t < T; ++t) {
    rmsnorm(x + (size_t)t * d, d, w.ffn_norm, c.wdtype, c.eps, &b[(size_t)t * d]);
    for (int i = 0; i < d; ++i) b[(size_t)t * d + i] = rp(b[(size_t)t * d + i], c);
  }
  std::vector<double> r((size_t)T * c.E);
  matmul(b.data(), T, d, w.router, 0, c.E, c.wdtype, r.data());
  std::memcpy(rlog, r.data(), r.size() * 8);
  std::vector<double> f((size_t)T * d, 0.0);
  for (int t = 0; t < T; ++t) {
    int* id = ids + (size_t)t * c.k;
    topk(&r[(size_t)t * c.E], c.E, c.k, id);
    double m = -INFINITY;
    for (int j = 0; j < c.k; ++j) m = std::max(m, r[(size_t)t * c.E + id[j]]);
    double s = 0;
    for (int j = 0; j < c.k; ++j) s += std::exp(r[(size_t)t * c.E + id[j]] - m);
    for (int j = 0; j < c.k; ++j) gates[(size_t)t * c.k + j] = std::exp(r[(size_t)t * c.E + id[j]] - m) / s;
  }
  // routed experts: each expert over the rows routed to it
  for (int e = 0; e < c.E; ++e) {
    std::vector<int> rows, slots;
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < c.k; ++j)
        if (ids[(size_t)t * c.k + j] == e) {
          rows.push_back(t);
          slots.push_back(j);
        }
    if (rows.empty()) continue;
    const int n = (int)rows.size();
    std::vector<double> be((size_t)n * d), ye((size_t)n * d);
    for (int i = 0; i < n; ++i) std::memcpy(&be[(size_t)i * d], &b[(size_t)rows[i] * d], d * 8);
    const size_t o13 = (size_t)e * c.eh * d, o2 = (size_t)e * d * c.eh;
    swiglu(be.data(), n, c, c.eh, w.w1, o13, w.w3, o13, w.w2, o2, ye.data());
    for (int i = 0; i < n; ++i) {
      const double gte = gates[(size_t)rows[i] * c.k + slots[i]];
      for (int j = 0; j < d; ++j) f[(size_t)rows[i] * d + j] += gte * ye[(size_t)i * d + j];
    }
  }
  std::vector<double> ys((size_t)T * d);
  swiglu(b.data(), T, c, c.sh, w.sw1, 0, w.sw3, 0, w.sw2, 0, ys.data());
  for (size_t i = 0; i < f.size(); ++i) x[i] += f[i] + ys[i];
}

// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11, section 4): ten rounds of multiply-high / multiply-low
// and xor, the key advanced by the Weyl constants between rounds.
void philox(uint64_t c[4], uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += W0;
      k1 += W1;
    }
    const unsigned __int128 p0 = (unsigned __int128)M0 * c[0], p1 = (unsigned __int128)M1 * c[2];
    const uint64_t hi0 = (uint64_t)(p0 >> 64), lo0 = (uint64_t)p0, hi1 = (uint64_t)(p1 >> 64), lo1 = (uint64_t)p1;
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}
int32_t draw(uint64_t seed, int block, int step, int pos, int vocab) {
  uint64_t c[4] = {(uint64_t)pos, (uint64_t)step, (uint64_t)block, 0};
  philox(c, seed, 0);
  return (int32_t)(uint64_t)(((unsigned __int128)c[0] * (uint64_t)vocab) >> 64);
}

}  // namespace

extern "C" {

// Configuration as plain integers / doubles (see Cfg).
struct dgo_config {
  int32_t vocab, d, L, hq, hkv, hd, E, k, eh, sh, C;
  double theta, eps;
  int32_t bf16_points, wdtype;
};

// Per-layer weight pointers (host, row-major [out][in], experts stacked).
struct dgo_layer {
  const void *attn_norm, *wq, *wk, *wv, *wo, *ffn_norm, *router, *w1, *w3, *w2, *sw1, *sw3, *sw2;
};

static Cfg to_cfg(const dgo_config* p) {
  return Cfg{p->vocab, p->d, p->L, p->hq, p->hkv, p->hd, p->E, p->k, p->eh, p->sh, p->C,
             p->theta, p->eps, p->bf16_points, p->wdtype};
}

// n uniform tokens for positions pos[0..n) of (seed, block, step).
void dgo_philox_tokens(uint64_t seed, int32_t block, int32_t step, const int32_t* pos, int32_t n, int32_t vocab,
                       int32_t* out) {
  for (int i = 0; i < n; ++i) out[i] = draw(seed, block, step, pos[i], vocab);
}

// One layer (see layer()): x [T][d] in place; kout / vout [T][hkv][hd];
// rlog [T][E], ids [T][k], gates [T][k] (untouched with skip_ffn).
void dgo_layer(const dgo_config* cp, const dgo_layer* wp, double* x, int32_t T, const int32_t* pos,
               const double* kp, const double* vp, int32_t P, int32_t causal, int32_t skip_ffn, double* kout,
               double* vout, double* rlog, int32_t* ids, double* gates) {
  const Cfg c = to_cfg(cp);
  const Layer w{wp->attn_norm, wp->wq,  wp->wk,  wp->wv,  wp->wo,  wp->ffn_norm, wp->router,
                wp->w1,        wp->w3,  wp->w2,  wp->sw1, wp->sw3, wp->sw2};
  std::vector<int> id((size_t)T * c.k);
  layer(c, w, x, T, pos, kp, vp, P, causal, skip_ffn, kout, vout, rlog, id.data(), gates);
  for (size_t i = 0; i < id.size(); ++i) ids[i] = id[i];
}

// Final RMSNorm and tied LM head over n rows h [n][d]: per row the entropy
// (nats), log-sum-exp and argmax (first maximum of the float32-rounded logits);
// logits [n][vocab] if not null.
void dgo_lm_head(const dgo_config* cp, const void* embed, const void* final_norm, const double* h, int32_t n,
                 double* entropy, double* lse, int32_t* argmax, double* logits) {
  const Cfg c = to_cfg(cp);
  const int d = c.d, V = c.vocab;
  std::vector<double> y((size_t)n * d);
  for (int t = 0; t < n; ++t) {
    rmsnorm(h + (size_t)t * d, d, final_norm, c.wdtype, c.eps, &y[(size_t)t * d]);
    for (int i = 0; i < d; ++i) y[(size_t)t * d + i] = rp(y[(size_t)t * d + i], c);
  }
  std::vector<double> z((size_t)V);
  for (int t = 0; t < n; ++t) {
    matmul(&y[(size_t)t * d], 1, d, embed, 0, V, c.wdtype, z.data());
    double m = -INFINITY;
    int am = 0;
    float best = -INFINITY;
    for (int v = 0; v < V; ++v) {
      m = std::max(m, z[v]);
      if ((float)z[v] > best) {
        best = (float)z[v];
        am = v;
      }
    }
    double s = 0;
    for (int v = 0; v < V; ++v) s += std::exp(z[v] - m);
    const double ls = m + std::log(s);
    double ent = 0;
    for (int v = 0; v < V; ++v) {
      const double lp = z[v] - ls;
      ent -= std::exp(lp) * lp;
    }
    entropy[t] = ent;
    lse[t] = ls;
    argmax[t] = am;
    if (logits) std::memcpy(logits + (size_t)t * V, z.data(), (size_t)V * 8);
  }
}

// Threshold sampler on one canvas (float32 entropies): accepts the open
// positions with entropy < tau and the open position of lowest entropy (first
// on ties); at step >= max_steps forces every other open position.  Accepted
// positions take their argmax, the rest are re-drawn at (seed, block, step).
// ids / accepted are updated in place; returns the number still open.
int32_t dgo_sample(const float* entropy, const int32_t* argmax, int32_t* ids, uint8_t* accepted, int32_t C, float tau,
                   int32_t step, int32_t max_steps, uint64_t seed, int32_t block, int32_t vocab, uint8_t* take_out) {
  std::vector<uint8_t> take(C, 0);
  int lowest = -1;
  for (int i = 0; i < C; ++i) {
    if (accepted[i]) continue;
    if (entropy[i] < tau) take[i] = 1;
    if (lowest < 0 || entropy[i] < entropy[lowest]) lowest = i;
  }
  if (lowest >= 0) take[lowest] = 1;
  if (step >= max_steps)
    for (int i = 0; i < C; ++i)
      if (!accepted[i]) take[i] = 1;
  int open = 0;
  for (int i = 0; i < C; ++i) {
    if (take[i]) {
      ids[i] = argmax[i];
      accepted[i] = 1;
    } else if (!accepted[i]) {
      ids[i] = draw(seed, block, step, i, vocab);
      ++open;
    }
    if (take_out) take_out[i] = take[i];
  }
  return open;
}

}  // extern "C"
