// libdg runtime: the C ABI of include/dg.h on top of the kernels.
//
// The context borrows caller-owned device memory (weights, KV cache, scratch) and
// a HIP stream, keeps the per-request state machine on the host, and queues the
// kernels of prefill, denoising step and block commit.  The only host<->device
// traffic per denoising step is the queue of launches and one small read-back of
// the per-request step counters.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "dg.h"
#include "dg_kernels.h"

// Reduction ranges of a split-reduction add projection, at most (partial-sum
// buffer: DG_MAX_KSPLIT x max_requests x canvas_len rows of d_model fp32).
// Reduction ranges of the router logits (bf16 model): each a slab of partial
// sums, added in range order by the top-k (twice the blocks for a 0.7 MB
// weight that 128 blocks read at the per-CU L2 rate).
#ifndef DG_ROUTER_KSPLIT
#define DG_ROUTER_KSPLIT 2
#endif
#ifndef DG_MAX_KSPLIT
#define DG_MAX_KSPLIT 8
#endif
// Kernel of the bf16 routed experts: 1 producer / consumer waves with the
// weight tiles copied straight into LDS (k_wsd, on longest-first work lists),
// 0 the register-staged k_ws.  Both read the normalised rows through the
// sorted-row -> token map.
#ifndef DG_ROUTED_KERNEL
#define DG_ROUTED_KERNEL 1
#endif
// n-blocks per k_wsd unit: W1/W3 (64 rows: 32 hidden columns of each) and W2
// (64 output columns).  W2's reduction is the expert's hidden width, 11
// chunks at the full size: a span of several keeps its weight stream from
// ramping up and draining every 11 chunks.
// Kernel of the dense bf16 projections (q/k/v, output projection, shared
// expert, self-conditioning MLP): 1 k_wsd's dense form (weight tiles copied
// straight into LDS by producer waves), 0 the register-staged k_ws.
#ifndef DG_DENSE_KERNEL
#define DG_DENSE_KERNEL 1
#endif
// Longest-first work lists for k_wsd (1) or lists in expert order (0).
#ifndef DG_ROUTE_LPT
#define DG_ROUTE_LPT 1
#endif
// Vocabulary ranges of the self-conditioning product, at most.
#ifndef DG_SC_KSPLIT
#define DG_SC_KSPLIT 16
#endif

// Static scratch of the allocation-free LM head (dg_op_lm_head_noalloc): every
// GPU the library runs on holds one copy until the process ends.  Host code
// never passes its name to a kernel; it uses the device address that
// noalloc_scratch_ptr resolves for the current device.
#define DG_NOALLOC_SCRATCH_BYTES (16u << 20)
static __device__ __align__(256) unsigned char scratch[DG_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_create_error;

struct Request {
  bool prefilled = false;
  bool active = false;
  bool done = false;
  int32_t P = 0;
  int32_t block = 0;
  int32_t step = 0;
  uint64_t seed = 0;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Device address of `scratch` on the current device, resolved once per device
// (each GPU holds its own copy at its own address).
constexpr int DG_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[DG_MAX_DEVICES];

hipError_t noalloc_scratch_ptr(void** p) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= DG_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_dev[dev] = q;
  }
  *p = g_scratch_dev[dev];
  return hipSuccess;
}

struct Carve {
  char* base;
  size_t off = 0;
  template <typename P> P* take(size_t bytes) {
    off = align_up(off, 256);
    P* p = base ? reinterpret_cast<P*>(base + off) : nullptr;
    off += bytes;
    return p;
  }
};

}  // namespace

struct dg_ctx {
  dg_model_config cfg;
  dg_sampler_config scfg;
  int dtype = 0;
  size_t esz = 4;
  const void* embed = nullptr;
  const void* final_norm = nullptr;
  std::vector<dg_layer_weights> layers;
  bool mx_wsd = false;  // MXFP4 experts fit k_wsd (16-byte aligned scale rows, their unit copy in LDS)
  char* kv = nullptr;
  hipStream_t stream = nullptr;
  hipStream_t side = nullptr;              // second stream: the shared expert overlaps the routed ones
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
  hipError_t sticky = hipSuccess;          // first failed stream call of a void helper
  const char* refused = nullptr;           // first launch a helper refused (shape outside the kernels)
  int C = 256;
  int rows_step = 0;   // max_requests * C
  int rows_max = 0;    // max(rows_step, prefill_chunk)
  int prefill_chunk = 2048;
  int lm_tiles = 0;
  size_t attn_cap = 0;  // partial rows (split x row x q-head) the attention buffers hold, / hq

  // scratch
  float* x = nullptr;
  void* xn = nullptr;
  void* xr = nullptr;  // bf16: row-major copy of the FFN-normalised rows
  float* parts = nullptr;  // partial sums of split-reduction add projections [ksplit][parts_rows][d]
  float* parts2 = nullptr;  // the same for the shared expert's W2 (side stream)
  int parts_rows = 0;
  void* q = nullptr;
  void* ao = nullptr;
  float* opart = nullptr;
  float* mlpart = nullptr;
  float* rlogits = nullptr;
  int32_t* rids = nullptr;
  float* rgates = nullptr;
  int32_t* counts = nullptr;
  int32_t* offsets = nullptr;
  int32_t* perm = nullptr;
  int32_t* offsets16 = nullptr;  // expert-sorted layout: first row of each expert (16-aligned)
  int32_t* rowsrc = nullptr;     // expert-sorted layout: token of each row (-1: padding)
  int32_t* units_up = nullptr;   // routed work lists (group << 24 | part << 16 | n-block)
  int32_t* units_dn = nullptr;
  int32_t* n_units = nullptr;    // [3]: lengths of the two lists, rows of the expert-sorted layout
  int rows_cap = 0;              // rows of the largest forward pass (sizes the work lists)
  void* hbuf = nullptr;
  void* hs = nullptr;
  float* ybuf = nullptr;
  void* hn = nullptr;
  float* lpart = nullptr;
  int32_t* lpart_arg = nullptr;
  float* ent = nullptr;
  float* lse = nullptr;
  int32_t* amax = nullptr;
  int32_t* open_rows = nullptr;
  int32_t* n_open_rows = nullptr;
  int32_t* canvas_ids = nullptr;
  uint8_t* canvas_acc = nullptr;
  int32_t* canvas_prev = nullptr;  // argmax canvas of each request's previous step (-1: none)
  int32_t* info_dev = nullptr;
  int32_t* tap_ids = nullptr;
  float* tap_gates = nullptr;
  float* tap_logits = nullptr;  // router logits of every layer of the last step [L][rows_step][E]
  double* inv_freq = nullptr;
  int32_t* ids_stage = nullptr;
  float* xg = nullptr;  // gathered rows for the logits tap [rows_step][d]
  // Debug taps of the denoising step (caller-owned device buffer, fp32):
  // [2 n_layers + 1][rows_step][d]: slot 2 l = input of layer l, slot 2 l + 1 =
  // the rows after layer l's attention half, slot 2 n_layers = the final rows.
  float* tap_buf = nullptr;
  bool tap_on = false;  // the current forward is a denoising step with taps
  bool tap_valid = false;  // the last denoising step filled the tap buffer

  int32_t* info_host = nullptr;  // pinned [max_requests][4]

  // Self-conditioning (cfg.self_cond_hidden > 0)
  const void *sc_w1 = nullptr, *sc_w3 = nullptr, *sc_w2 = nullptr;
  void* embed_t = nullptr;   // the embedding transposed, [d][V] bf16
  float* sc_z = nullptr;     // logits of the LM head's open rows [rows_step][V]
  void* sc_p = nullptr;      // their softmax, bf16 fragment-major [rows_step][V]
  float* sc_parts = nullptr; // split-vocabulary partial sums [DG_SC_KSPLIT][rows_step][d]
  float* sc_state = nullptr; // per request and position [max_requests][C][d]
  void* sc_b = nullptr;      // MLP input, bf16 fragment-major [rows_step][d]
  void* sc_h = nullptr;      // MLP hidden, bf16 fragment-major [rows_step][m]

  // Kernel timer: HIP event pairs around every launch of one kernel family.
  int kt_family = 0;
  int kt_every = 1;       // time every kt_every-th step or commit
  int64_t kt_calls = 0;   // steps and commits since dg_kernel_timer_every
  bool kt_on = true;      // the current step or commit is timed
  std::vector<hipEvent_t> kt_ev;  // 2 per recorded launch
  size_t kt_used = 0;
  double kt_ms = 0.0;
  int64_t kt_launches = 0;

  std::vector<Request> req;
  void* noalloc_scratch = nullptr;  // this device's copy of `scratch` (dg_op_lm_head_noalloc)
  std::string noalloc_err;          // why it could not be resolved
  std::vector<int> last_slots;  // request of each slot in the last step
  int last_rows = 0;
  std::string err;
};

namespace {

dg_status fail(dg_ctx* c, dg_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (c) c->err = buf;
  else g_create_error = buf;
  return st;
}

#define HIPCK(ctx, call)                                                                              \
  do {                                                                                                \
    hipError_t e_ = (call);                                                                           \
    if (e_ != hipSuccess) return fail((ctx), DG_ERR_HIP, "%s: %s", #call, hipGetErrorString(e_));     \
  } while (0)

// Launch errors, and the first error of a stream call inside a void helper
// (recorded by HIPCK_V), are reported by the next LAUNCHCK of the entry point.
#define LAUNCHCK(ctx)                                                                                  \
  do {                                                                                                 \
    hipError_t e_ = (ctx)->sticky != hipSuccess ? (ctx)->sticky : hipGetLastError();                  \
    (ctx)->sticky = hipSuccess;                                                                        \
    if (e_ != hipSuccess) {                                                                            \
      (ctx)->refused = nullptr;                                                                        \
      return fail((ctx), DG_ERR_HIP, "kernel launch: %s", hipGetErrorString(e_));                     \
    }                                                                                                  \
    const dg_status r_ = take_refusal(ctx);                                                            \
    if (r_ != DG_OK) return r_;                                                                        \
  } while (0)
// The refusal half of LAUNCHCK (host only): a launcher's -1, recorded by
// REFUSE_IF, becomes DG_ERR_UNSUPPORTED with the launch's name.
dg_status take_refusal(dg_ctx* c) {
  const char* r = c->refused;
  c->refused = nullptr;
  return r ? fail(c, DG_ERR_UNSUPPORTED, "launch refused: %s", r) : DG_OK;
}
// A launcher that returned -1 queued nothing: the entry point reports
// DG_ERR_UNSUPPORTED at its next LAUNCHCK (later launches of the same call may
// still be queued; their results are not used).
#define REFUSE_IF(ctx, cond, what)                     \
  do {                                                 \
    if ((cond) && !(ctx)->refused) (ctx)->refused = (what); \
  } while (0)
#define HIPCK_V(call)                                              \
  do {                                                             \
    hipError_t e_ = (call);                                        \
    if (e_ != hipSuccess && c->sticky == hipSuccess) c->sticky = e_; \
  } while (0)

// Kernel timer.  kt_begin/kt_end bracket one launch of family f; the events are
// read back (and the pairs reused) by kt_collect after the stream has synchronised.
void kt_begin(dg_ctx* c, int f, hipStream_t s) {
  if (c->kt_family != f || !c->kt_on) return;
  while (c->kt_ev.size() < c->kt_used + 2) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) { c->kt_family = 0; return; }
    c->kt_ev.push_back(e);
  }
  hipEventRecord(c->kt_ev[c->kt_used], s);
}
void kt_end(dg_ctx* c, int f, hipStream_t s) {
  if (c->kt_family != f || !c->kt_on) return;
  hipEventRecord(c->kt_ev[c->kt_used + 1], s);
  c->kt_used += 2;
}
void kt_collect(dg_ctx* c) {
  for (size_t i = 0; i + 1 < c->kt_used; i += 2) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, c->kt_ev[i], c->kt_ev[i + 1]) == hipSuccess) {
      c->kt_ms += ms;
      c->kt_launches += 1;
    }
  }
  c->kt_used = 0;
}
#define KT(c, fam, launch)           \
  do {                               \
    kt_begin((c), (fam), (c)->stream); \
    launch;                          \
    kt_end((c), (fam), (c)->stream);   \
  } while (0)
// The same for a launch on stream st.
#define KTS(c, fam, st, launch) \
  do {                          \
    kt_begin((c), (fam), (st)); \
    launch;                     \
    kt_end((c), (fam), (st));   \
  } while (0)

int kc_of(int dtype) { return dtype == DG_BF16 ? 32 : 16; }

// Validation of shapes against what the kernels implement.  Returns a message or null.
const char* check_config(const dg_model_config* c) {
  if (!c) return "null config";
  if (c->dtype != DG_F32 && c->dtype != DG_BF16) return "dtype must be DG_F32 or DG_BF16";
  if (c->expert_format != DG_EXPERTS_NATIVE && c->expert_format != DG_EXPERTS_FP8 &&
      c->expert_format != DG_EXPERTS_MXFP4)
    return "expert_format must be DG_EXPERTS_NATIVE, DG_EXPERTS_FP8 or DG_EXPERTS_MXFP4";
  if (c->expert_format == DG_EXPERTS_FP8 && c->dtype != DG_BF16) return "FP8 experts need a bf16 model";
  if (c->expert_format == DG_EXPERTS_MXFP4 && c->dtype != DG_BF16) return "MXFP4 experts need a bf16 model";
  if (c->vocab <= 0 || c->d_model <= 0 || c->n_layers <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
      c->head_dim <= 0 || c->n_experts <= 0 || c->top_k <= 0 || c->expert_hidden <= 0 || c->shared_hidden <= 0 ||
      c->max_ctx <= 0 || c->max_requests <= 0)
    return "every size must be positive";
  if (c->canvas_len != 256) return "canvas_len must be 256";
  if (c->max_requests > DG_MAX_SEGS) return "max_requests must be <= 16";
  if (c->n_q_heads % c->n_kv_heads) return "n_q_heads must be a multiple of n_kv_heads";
  const int kc = kc_of(c->dtype);
  const int hd = c->head_dim;
  if (!(hd == 16 || hd == 32 || hd == 64 || hd == 128 || hd == 256)) return "head_dim must be 16, 32, 64, 128 or 256";
  if (c->dtype == DG_BF16 && hd < 64) return "bf16 head_dim must be >= 64";
  if (c->dtype == DG_BF16 && ((c->n_q_heads * hd) % 64 || c->shared_hidden % 64))
    return "bf16: n_q_heads * head_dim and shared_hidden must be multiples of 64";
  if (((c->n_q_heads + 2 * c->n_kv_heads) * hd / 2) % 16) return "(Hq + 2 Hkv) * head_dim / 2 must be a multiple of 16";
  if (c->d_model % 64 || c->d_model % kc) return "d_model must be a multiple of 64";
  if (c->d_model > 16384) return "d_model must be <= 16384";
  if ((c->n_q_heads * hd) % kc) return "n_q_heads * head_dim must be a multiple of the k-chunk";
  if (c->expert_hidden % 64) return "expert_hidden must be a multiple of 64";
  if (c->shared_hidden % 16 || c->shared_hidden % kc) return "shared_hidden must be a multiple of 16 and the k-chunk";
  if (c->vocab % 128) return "vocab must be a multiple of 128";
  if (c->n_experts > 256) return "n_experts must be <= 256";
  if (c->top_k > 16 || c->top_k > c->n_experts) return "top_k must be <= 16 and <= n_experts";
  if (c->max_ctx % 64) return "max_ctx must be a multiple of 64";
  if (c->max_ctx < c->canvas_len) return "max_ctx must hold at least one canvas";
  if (c->prefill_chunk < 0) return "prefill_chunk must be >= 0";
  // a routed work unit names its row part of an expert in 8 bits (128 rows each)
  if (c->prefill_chunk > 32768) return "prefill_chunk must be <= 32768";
  if (c->self_cond_hidden < 0 || c->self_cond_hidden % 64 || c->self_cond_hidden > 4096)
    return "self_cond_hidden must be a multiple of 64 in [0, 4096]";
  if (c->self_cond_hidden > 0 && c->dtype != DG_BF16) return "self-conditioning needs a bf16 model";
  return nullptr;
}

struct Plan {
  size_t kv_bytes = 0, scratch_bytes = 0;
};

// Carves the scratch (base may be null to only size it).
size_t carve(dg_ctx* c, const dg_model_config& m, char* base) {
  Carve cv{base};
  const size_t es = m.dtype == DG_BF16 ? 2 : 4;
  const int C = m.canvas_len;
  const int Rs = m.max_requests * C;
  const int pc = m.prefill_chunk > 0 ? m.prefill_chunk : 2048;
  const int Tm = (std::max(Rs, pc) + 15) / 16 * 16;  // fragment-major buffers hold whole 16-row tiles
  const size_t d = m.d_model, qd = (size_t)m.n_q_heads * m.head_dim;
  const size_t k = m.top_k, E = m.n_experts;
  const size_t attn_cap = std::max((size_t)32 * Rs, (size_t)4 * Tm);
  const int tiles = dg_lm_head_tiles(m.vocab);
  c->x = cv.take<float>(Tm * d * 4);
  c->xn = cv.take<void>(Tm * d * es);
  c->xr = cv.take<void>(Tm * d * es);
  c->parts = cv.take<float>((size_t)DG_MAX_KSPLIT * Rs * d * 4);
  c->parts2 = cv.take<float>((size_t)DG_MAX_KSPLIT * Rs * d * 4);
  c->parts_rows = Rs;
  c->q = cv.take<void>(Tm * qd * es);
  c->ao = cv.take<void>(Tm * qd * es);
  c->opart = cv.take<float>(attn_cap * m.n_q_heads * m.head_dim * 4);
  c->mlpart = cv.take<float>(attn_cap * m.n_q_heads * 2 * 4);
  c->rlogits = cv.take<float>(Tm * E * 4 * DG_ROUTER_KSPLIT);  // a slab per router reduction range
  c->rids = cv.take<int32_t>(Tm * k * 4);
  c->rgates = cv.take<float>(Tm * k * 4);
  c->counts = cv.take<int32_t>(E * 4);
  c->offsets = cv.take<int32_t>(E * 4);
  c->perm = cv.take<int32_t>(Tm * k * 4);
  c->offsets16 = cv.take<int32_t>(E * 4);
  const size_t srows = (size_t)dg_sorted_rows((int)E, (int)(Tm * k));  // expert-sorted rows
  c->rowsrc = cv.take<int32_t>(srows * 4);
  c->units_up = cv.take<int32_t>((size_t)dg_unit_slots(E, Tm * k, DG_WS_GROUP_ROWS, (m.expert_hidden + 31) / 32) * 4);
  c->units_dn = cv.take<int32_t>((size_t)dg_unit_slots(E, Tm * k, DG_WS_GROUP_ROWS, (m.d_model + 63) / 64) * 4);
  c->rows_cap = Tm;
  c->n_units = cv.take<int32_t>(3 * 4);  // up list, down list, expert-sorted rows
  c->hbuf = cv.take<void>(srows * m.expert_hidden * es);
  c->hs = cv.take<void>(Tm * (size_t)m.shared_hidden * es);
  c->ybuf = cv.take<float>(Tm * k * d * 4);
  c->hn = cv.take<void>(Rs * d * es);
  c->lpart = cv.take<float>((size_t)Rs * tiles * 3 * 4);
  c->lpart_arg = cv.take<int32_t>((size_t)Rs * tiles * 4);
  c->ent = cv.take<float>(Rs * 4);
  c->lse = cv.take<float>(Rs * 4);
  c->amax = cv.take<int32_t>(Rs * 4);
  c->open_rows = cv.take<int32_t>(Rs * 4);
  c->n_open_rows = cv.take<int32_t>(4);
  c->canvas_ids = cv.take<int32_t>(Rs * 4);
  c->canvas_acc = cv.take<uint8_t>(Rs);
  c->canvas_prev = cv.take<int32_t>(Rs * 4);
  c->info_dev = cv.take<int32_t>(m.max_requests * 4 * 4);
  c->tap_ids = cv.take<int32_t>((size_t)m.n_layers * Rs * k * 4);
  c->tap_gates = cv.take<float>((size_t)m.n_layers * Rs * k * 4);
  c->tap_logits = cv.take<float>((size_t)m.n_layers * Rs * E * 4 * DG_ROUTER_KSPLIT);
  c->inv_freq = cv.take<double>(m.head_dim / 2 * 8);
  c->ids_stage = cv.take<int32_t>(Tm * 4);
  c->xg = cv.take<float>(Rs * d * 4);
  c->attn_cap = attn_cap;
  if (m.self_cond_hidden > 0) {
    const size_t V = m.vocab;
    c->embed_t = cv.take<void>(V * d * es);
    c->sc_z = cv.take<float>((size_t)Rs * V * 4);
    c->sc_p = cv.take<void>((size_t)Rs * V * es);
    c->sc_parts = cv.take<float>((size_t)DG_SC_KSPLIT * Rs * d * 4);
    c->sc_state = cv.take<float>((size_t)Rs * d * 4);
    c->sc_b = cv.take<void>((size_t)Rs * d * es);
    c->sc_h = cv.take<void>((size_t)Rs * m.self_cond_hidden * es);
  }
  return align_up(cv.off, 256);
}

size_t kv_size(const dg_model_config& m) {
  const size_t es = m.dtype == DG_BF16 ? 2 : 4;
  return (size_t)m.max_requests * m.n_layers * 2 * m.n_kv_heads * (size_t)m.max_ctx * m.head_dim * es;
}

DgShape shape_of(const dg_ctx* c) {
  DgShape s;
  s.d = c->cfg.d_model;
  s.hq = c->cfg.n_q_heads;
  s.hkv = c->cfg.n_kv_heads;
  s.hd = c->cfg.head_dim;
  s.max_ctx = c->cfg.max_ctx;
  s.vocab = c->cfg.vocab;
  return s;
}

void* kv_ptr(const dg_ctx* c, int r, int l, int which) {
  const size_t per = (size_t)c->cfg.n_kv_heads * c->cfg.max_ctx * c->cfg.head_dim * c->esz;
  return c->kv + (((size_t)r * c->cfg.n_layers + l) * 2 + which) * per;
}

// Copies the rows of c->x into tap slot `slot` (denoising steps with a tap buffer).
void tap_rows(dg_ctx* c, int slot, int rows) {
  if (!c->tap_on) return;
  const size_t per = (size_t)c->rows_step * c->cfg.d_model;
  HIPCK_V(hipMemcpyAsync(c->tap_buf + slot * per, c->x, (size_t)rows * c->cfg.d_model * 4, hipMemcpyDeviceToDevice,
                         c->stream));
}

// Segments (one per slot) for layer l.  rows of slot s: [s*n, (s+1)*n).
struct SlotRow {
  int req, pos0, n;
};

DgSegs make_segs(const dg_ctx* c, const std::vector<SlotRow>& slots, int l, bool causal) {
  DgSegs sg;
  memset(&sg, 0, sizeof sg);
  int row = 0;
  for (size_t i = 0; i < slots.size(); ++i) {
    sg.s[i].k = kv_ptr(c, slots[i].req, l, 0);
    sg.s[i].vt = kv_ptr(c, slots[i].req, l, 1);
    sg.s[i].row0 = row;
    sg.s[i].n = slots[i].n;
    sg.s[i].pos0 = slots[i].pos0;
    sg.s[i].nkeys = slots[i].pos0 + slots[i].n;
    row += slots[i].n;
  }
  sg.count = (int)slots.size();
  sg.causal = causal ? 1 : 0;
  return sg;
}

// Launch helpers.  bf16 models run the weight-streaming kernel (k_ws.hip); the
// fp32 model keeps the plain matrix-core kernels.

// Row ranges per weight tile for a dense launch with nblk tiles over M rows: as
// many blocks as fit one per CU (256), at least 16 rows per block.  The extra
// reads of a tile come from L2 (see the row split in k_ws).
// Output columns per n-block of the output projection (64 or 128: 128 halves
// the activation reads per weight byte, and more reduction ranges keep the
// grid near one block per CU).
#ifndef DG_OUTPROJ_BN
#define DG_OUTPROJ_BN 128
#endif
#ifndef DG_DENSE_BLOCKS
#define DG_DENSE_BLOCKS 256
#endif
// Rows per block of the shared expert's W2 (no split reduction).  It overlaps
// the routed W1/W3 launch; few large blocks slow that launch least (measured:
// 128-row parts 11.02 ms/step, 32-row 11.17, 16-row 11.44).
#ifndef DG_SHARED_W2_ROWS
#define DG_SHARED_W2_ROWS 128
#endif
int dense_msplit(int nblk, int M) {
  // At most DG_DENSE_BLOCKS (one per CU) in all: a block streams its tile at a
  // rate set by memory latency, and a CU that receives two blocks finishes last.
  const int padded = (nblk + 7) / 8 * 8;
  int ms = DG_DENSE_BLOCKS / padded;
  ms = std::min(ms, std::max(1, M / 16));
  return std::max(ms, 1);
}

// Grid of a dense launch: with a row split, tiles are dealt to XCDs in groups of
// 8 (see k_ws), so the tile count is padded to a multiple of 8.
int dense_grid(int nblk, int msplit) { return msplit > 1 ? (nblk + 7) / 8 * 8 * msplit : nblk; }
void launch_dense(dg_ctx* c, int epi, const void* A, int M, int K, const void* W0, const void* W1, int N, void* out,
                  int ldo, hipStream_t st = nullptr) {
  if (c->dtype != DG_BF16) {  // bf16-only kernel; the fp32 model has its own launches
    REFUSE_IF(c, true, "bf16 streaming projection on a non-bf16 model");
    return;
  }
  WsArgs a;
  memset(&a, 0, sizeof a);
  a.A = A;
  a.W0 = W0;
  a.W1 = W1;
  a.K = K;
  a.N = N;
  a.M = M;
  a.out = out;
  a.ldo = ldo;
  const int nblk = epi == WS_EPI_SWIGLU ? (N + 31) / 32 : (N + 63) / 64;
  if (DG_DENSE_KERNEL == 1) {  // 64 weight rows per n-block (SwiGLU: 32 W1 + 32 W3), 128-row parts
    a.nblk = nblk;
    a.msplit = (M + DG_WS_GROUP_ROWS - 1) / DG_WS_GROUP_ROWS;
    REFUSE_IF(c, dg_launch_wsd_dense(epi, a, st ? st : c->stream) != 0, "dense projection");
    return;
  }
  a.nblk = nblk;
  a.msplit = dense_msplit(nblk, M);
  a.mt2 = epi == WS_EPI_SWIGLU && M > 256;  // 256 rows per pass for prefill chunks and eight canvases
  REFUSE_IF(c, dg_launch_ws(epi, a, dense_grid(nblk, a.msplit), st ? st : c->stream) != 0, "dense projection");
}

// Grouped launch over the expert-sorted rows: A is fragment-major in the
// expert-sorted layout (c->offsets16), or row-major with rowsrc mapping each
// sorted row to its row of A.
// Output projection / shared-expert W2: out (fp32 [M][N], row-major) += A W^T.
// 128 output columns per block and at most 128 rows (one pass; 256 rows with two
// m-tiles per wave when there are more than 256 rows), and when that
// leaves CUs idle the reduction is split too: each range then stores its partial
// sums into c->parts, and the returned DgParts must be folded into out by the
// next row kernel (in range order, so the result is deterministic).
DgParts launch_dense_add(dg_ctx* c, const void* A, int M, int K, const void* W, int N, float* out,
                         hipStream_t st = nullptr, float* parts = nullptr, int max_ksplit = DG_MAX_KSPLIT,
                         int part_rows = 128, int bn = 64) {
  if (!parts) parts = c->parts;
  if (c->dtype != DG_BF16) {  // bf16-only kernel; the fp32 model has its own launches
    REFUSE_IF(c, true, "bf16 streaming add projection on a non-bf16 model");
    return DgParts{};
  }
  WsArgs a;
  memset(&a, 0, sizeof a);
  a.A = A;
  a.W0 = W;
  a.K = K;
  a.N = N;
  a.M = M;
  a.out = out;
  a.ldo = N;
  if (DG_DENSE_KERNEL == 1) {
    // k_wsd: bn (64 or 128) output columns per n-block, 128-row parts; the
    // reduction split into ranges (partial sums folded by the next row kernel)
    // while that keeps the grid within one block per CU
    const int nblk = (N + bn - 1) / bn, padded = (nblk + 7) / 8 * 8;
    a.nblk = nblk;
    a.wide = bn == 128;
    a.msplit = (M + DG_WS_GROUP_ROWS - 1) / DG_WS_GROUP_ROWS;
    int ks = 1;
    if (M <= c->parts_rows && N == c->cfg.d_model)
      ks = std::min(max_ksplit, std::max(1, DG_DENSE_BLOCKS / (padded * a.msplit)));
    const int nk = K / 64, kchunks = (nk + ks - 1) / ks;
    ks = (nk + kchunks - 1) / kchunks;  // every range non-empty
    DgParts pend;
    if (ks > 1) {
      a.ksplit = ks;
      a.kchunks = kchunks;
      a.part_out = parts;
      a.part_stride = (size_t)c->parts_rows * N;
      pend.p = parts;
      pend.n = ks;
      pend.stride = a.part_stride;
    }
    REFUSE_IF(c, dg_launch_wsd_dense(WS_EPI_ADD_F32, a, st ? st : c->stream) != 0, "add projection");
    return pend;
  }
  a.wide = 1;
  // More than 256 rows (prefill chunks, eight canvases): two m-tiles per wave and
  // 256-row parts, so each weight tile is read by half as many blocks.
  if (M > 256) {
    a.mt2 = 1;
    part_rows = std::max(part_rows, 256);
  }
  const int nblk = (N + 127) / 128, padded = (nblk + 7) / 8 * 8;
  a.nblk = nblk;
  a.msplit = std::max(1, (M + part_rows - 1) / part_rows);
  int ks = 1;
  if (M <= c->parts_rows && N == c->cfg.d_model)
    ks = std::min(max_ksplit, std::max(1, DG_DENSE_BLOCKS / (padded * a.msplit)));
  const int nk = K / 64;
  const int kchunks = (nk + ks - 1) / ks;
  ks = (nk + kchunks - 1) / kchunks;  // every range non-empty
  DgParts pend;
  if (ks > 1) {
    a.ksplit = ks;
    a.kchunks = kchunks;
    a.part_out = parts;
    a.part_stride = (size_t)c->parts_rows * N;
    pend.p = parts;
    pend.n = ks;
    pend.stride = a.part_stride;
  }
  const int grid = (a.msplit > 1 || ks > 1) ? padded * a.msplit * ks : nblk;
  REFUSE_IF(c, dg_launch_ws(WS_EPI_ADD_F32, a, grid, st ? st : c->stream) != 0, "add projection");
  return pend;
}

// Floats per layer of the router-logit taps: room for every reduction range's
// slab (the top-k writes their total over the first).
size_t tap_logit_stride(const dg_ctx* c) { return (size_t)DG_ROUTER_KSPLIT * c->rows_step * c->cfg.n_experts; }

// Kernel of the routed launches: DG_ROUTED_KERNEL (k_wsd) for bf16 experts, and
// for E4M3 and MXFP4 codes (copied into LDS as codes, widened to bf16 in
// registers); k_ws (widening on the way into LDS) for MXFP4 scale arrays that
// k_wsd cannot copy (misaligned).
#ifndef DG_ROUTED_FP8_KERNEL
#define DG_ROUTED_FP8_KERNEL 1
#endif
#ifndef DG_ROUTED_MX_KERNEL
#define DG_ROUTED_MX_KERNEL 1
#endif
int routed_kernel(const dg_ctx* c) {
  if (c->dtype != DG_BF16) return 0;
  if (c->cfg.expert_format == DG_EXPERTS_NATIVE) return DG_ROUTED_KERNEL;
  if (c->cfg.expert_format == DG_EXPERTS_FP8) return DG_ROUTED_FP8_KERNEL;
  if (c->cfg.expert_format == DG_EXPERTS_MXFP4 && c->mx_wsd) return DG_ROUTED_MX_KERNEL;
  return 0;
}
// Rows per part of a routed work list: k_wsd takes up to 256 for bf16 weights
// (two m-tiles per consumer wave), so an expert's weights stream once for up to
// 256 rows; 128 for E4M3 and MXFP4 codes (registers for their widening).
int routed_part_rows(const dg_ctx* c) {
  if (routed_kernel(c) != 1) return DG_WS_GROUP_ROWS;
  return c->cfg.expert_format == DG_EXPERTS_NATIVE ? DG_WSD_PART_ROWS : DG_WS_GROUP_ROWS;
}
// n-blocks per unit of a k_wsd work list, and the units per row part.
int wsd_span(int epi) { return dg_wsd_span(epi); }
int list_blocks(const dg_ctx* c, int epi, int nblk) {
  return routed_kernel(c) == 1 ? (nblk + wsd_span(epi) - 1) / wsd_span(epi) : nblk;
}

// Routed launch over the expert work list; with FP8 experts W0 / W1 hold E4M3
// codes and s0 / s1 their per-row scales ([E][N] each), with MXFP4 experts
// packed E2M1 codes and b0 / b1 their E8M0 block scales ([E][N][K / 32] each).
void launch_routed(dg_ctx* c, int epi, const void* A, const void* W0, const void* W1, const float* s0,
                   const float* s1, const uint8_t* b0, const uint8_t* b1, size_t wgs, int K, int N,
                   const int32_t* units, const int32_t* n_units, int nblk, void* out, int ldo,
                   const int32_t* rowsrc = nullptr) {
  if (c->dtype != DG_BF16) {  // bf16-only kernels
    REFUSE_IF(c, true, "routed streaming projection on a non-bf16 model");
    return;
  }
  WsArgs a;
  memset(&a, 0, sizeof a);
  a.A = A;
  a.W0 = W0;
  a.W1 = W1;
  a.wfmt = c->cfg.expert_format == DG_EXPERTS_FP8     ? DG_WS_W_E4M3
           : c->cfg.expert_format == DG_EXPERTS_MXFP4 ? DG_WS_W_MXFP4
                                                      : DG_WS_W_BF16;
  a.wsc0 = s0;
  a.wsc1 = s1;
  a.wbs0 = b0;
  a.wbs1 = b1;
  a.wgs = wgs;
  a.K = K;
  a.N = N;
  a.counts = c->counts;
  a.offsets = c->offsets;
  a.perm = c->perm;
  a.offsets16 = c->offsets16;
  a.rowsrc = rowsrc;
  a.units = units;
  a.n_units = n_units;
  a.out = out;
  a.ldo = ldo;
  // bf16 experts: k_wsd; codes that are widened on the way (E4M3, MXFP4) keep k_ws
  const int grid = dg_unit_slots(c->cfg.n_experts, c->rows_cap * c->cfg.top_k, routed_part_rows(c),
                                 list_blocks(c, epi, nblk));
  if (routed_kernel(c) == 1) {
    a.nblk = nblk;
    a.span = wsd_span(epi);
    REFUSE_IF(c, dg_launch_wsd(epi, a, grid, c->stream) != 0, "routed projection");
  } else {
    REFUSE_IF(c, dg_launch_ws(epi, a, grid, c->stream) != 0, "routed projection");
  }
}

void launch_qkv(dg_ctx* c, const dg_layer_weights& w, int rows, const DgSegs& sg) {
  const dg_model_config& m = c->cfg;
  if (c->dtype == DG_F32) {
    dg_launch_qkv(c->dtype, c->xn, rows, shape_of(c), w.wq, w.wk, w.wv, sg, c->inv_freq, c->q, c->stream);
    return;
  }
  WsArgs a;
  memset(&a, 0, sizeof a);
  a.A = c->xn;
  a.W0 = w.wq;
  a.W1 = w.wk;
  a.W2 = w.wv;
  a.K = m.d_model;
  a.N = (m.n_q_heads + 2 * m.n_kv_heads) * m.head_dim;
  a.M = rows;
  a.out = c->q;
  a.ldo = m.n_q_heads * m.head_dim;
  a.hd = m.head_dim;
  a.hq = m.n_q_heads;
  a.hkv = m.n_kv_heads;
  a.max_ctx = m.max_ctx;
  a.inv_freq = c->inv_freq;
  a.segs = sg;
  const int nblk = (m.n_q_heads + 2 * m.n_kv_heads) * m.head_dim / 64;
  a.nblk = nblk;
  if (DG_DENSE_KERNEL == 1) {
    a.msplit = (rows + DG_WS_GROUP_ROWS - 1) / DG_WS_GROUP_ROWS;
    REFUSE_IF(c, dg_launch_wsd_dense(WS_EPI_ROPE_QKV, a, c->stream) != 0, "q/k/v projection");
    return;
  }
  a.msplit = dense_msplit(nblk, rows);
  a.mt2 = rows > 256;  // 256 rows per pass for prefill chunks and eight canvases
  REFUSE_IF(c, dg_launch_ws(WS_EPI_ROPE_QKV, a, dense_grid(nblk, a.msplit), c->stream) != 0, "q/k/v projection");
}

// Fused LM head over the rows of c->hn (count *n_dev <= max_rows): per-row
// softmax statistics and argmax written at row_idx[row] (or row).
// hn, lpart, lpart_arg: the normalised rows and the per-tile partial statistics
// (default: the context's scratch).
void launch_lm_head(dg_ctx* c, const int32_t* n_dev, int max_rows, const int32_t* row_idx, float* ent, float* lse,
                    int32_t* amax, float* zout = nullptr, const void* hn = nullptr, float* lpart = nullptr,
                    int32_t* lpart_arg = nullptr) {
  const dg_model_config& m = c->cfg;
  if (!hn) hn = c->hn;
  if (!lpart) lpart = c->lpart;
  if (!lpart_arg) lpart_arg = c->lpart_arg;
  if (c->dtype == DG_F32) {
    dg_launch_lm_head(c->dtype, hn, n_dev, max_rows, m.d_model, c->embed, m.vocab, lpart, lpart_arg, ent, lse, amax,
                      row_idx, c->stream);
    return;
  }
  WsArgs a;
  memset(&a, 0, sizeof a);
  a.A = hn;
  a.W0 = c->embed;
  a.K = m.d_model;
  a.N = m.vocab;
  a.M = max_rows;
  a.M_dev = n_dev;
  a.out = lpart;
  a.ldo = c->lm_tiles;
  a.part_arg = lpart_arg;
  a.zout = zout;
  // k_ws: all (up to 256) rows in one pass, so the embedding crosses HBM once
  // per step; k_wsd's 128-row parts stream it twice (measured: 647 against 444 us)
  REFUSE_IF(c, dg_launch_ws(WS_EPI_LM_STATS, a, c->lm_tiles, c->stream) != 0, "LM head");
  dg_launch_lm_merge(lpart, lpart_arg, n_dev, max_rows, c->lm_tiles, row_idx, ent, lse, amax, c->stream);
}

// The static scratch of the allocation-free LM head for n rows: the row count,
// the normalised rows (whole 16-row tiles) and the per-tile partial statistics.
// Returns the bytes needed; with base, also the carved pointers.
size_t noalloc_lm_carve(const dg_model_config& m, int n, char* base, int32_t** n_dev, void** hn, float** lpart,
                        int32_t** lpart_arg) {
  Carve cv{base};
  const size_t n16 = (size_t)(n + 15) / 16 * 16, tiles = (size_t)dg_lm_head_tiles(m.vocab);
  int32_t* nd = cv.take<int32_t>(4);
  void* h = cv.take<void>(n16 * m.d_model * (m.dtype == DG_BF16 ? 2 : 4));
  float* lp = cv.take<float>(n16 * tiles * 3 * 4);
  int32_t* la = cv.take<int32_t>(n16 * tiles * 4);
  if (n_dev) *n_dev = nd;
  if (hn) *hn = h;
  if (lpart) *lpart = lp;
  if (lpart_arg) *lpart_arg = la;
  return cv.off;
}

// Self-conditioning state rows of the requests in the step's slots.
DgScSlots sc_slots(const dg_ctx* c, const std::vector<int>& slot_req) {
  DgScSlots sl;
  memset(&sl, 0, sizeof sl);
  for (size_t i = 0; i < slot_req.size(); ++i)
    sl.state[i] = c->sc_state + (size_t)slot_req[i] * c->C * c->cfg.d_model;
  return sl;
}

// The MLP term of the state rows in c->sc_b (bf16, fragment-major, `rows` rows)
// added to x: W2 (silu(W1 b) * (W3 b)).  K of the W2 product is the MLP width,
// a few 64-element chunks, so it is not split.
void sc_mlp_add(dg_ctx* c, int rows, float* x) {
  const dg_model_config& m = c->cfg;
  launch_dense(c, WS_EPI_SWIGLU, c->sc_b, rows, m.d_model, c->sc_w1, c->sc_w3, m.self_cond_hidden, c->sc_h,
               m.self_cond_hidden);
  launch_dense_add(c, c->sc_h, rows, m.self_cond_hidden, c->sc_w2, m.d_model, x, nullptr, nullptr, 1);
}

// Embedding term of the canvas rows of the step's slots (rows = slots x C).
void sc_embed(dg_ctx* c, const std::vector<int>& slot_req, int rows) {
  if (c->cfg.self_cond_hidden <= 0) return;
  KT(c, DG_KF_SELF_COND, dg_launch_sc_gather(sc_slots(c, slot_req), rows, c->C, c->cfg.d_model, c->sc_b, c->stream);
                         sc_mlp_add(c, rows, c->x));
}

// State update after the LM head, whose logits of the open rows (compacted,
// count *c->n_open_rows, canvas rows c->open_rows) are in c->sc_z and
// log-sum-exp in c->lse: softmax in bf16, its product with the embedding over
// vocabulary ranges (streaming GEMM against the transposed embedding, partial
// sums per range), and the fold into the state rows.
void sc_update(dg_ctx* c, const std::vector<int>& slot_req, int max_rows) {
  const dg_model_config& m = c->cfg;
  hipStream_t s = c->stream;
  dg_launch_sc_probs(c->sc_z, c->lse, c->open_rows, c->n_open_rows, max_rows, m.vocab, c->sc_p, s);
  WsArgs a;
  memset(&a, 0, sizeof a);
  a.A = c->sc_p;
  a.W0 = c->embed_t;
  a.K = m.vocab;
  a.N = m.d_model;
  a.M = max_rows;
  a.M_dev = c->n_open_rows;
  a.ldo = m.d_model;
  a.wide = 1;  // 128 output columns per block
  a.mt2 = 1;   // 256 rows per pass: each block reads its tile of the transposed embedding once
  const int nblk = (m.d_model + 127) / 128, padded = (nblk + 7) / 8 * 8;
  a.nblk = nblk;
  a.msplit = std::max(1, (max_rows + 255) / 256);
  // Vocabulary ranges: about one block per CU (the two-m-tile variant holds one
  // block per CU), at least two ranges (the partial-sum path), every range non-empty.
  const int nk = m.vocab / 64;
  int ks = std::min(DG_SC_KSPLIT, std::max(2, DG_DENSE_BLOCKS / (padded * a.msplit)));
  const int kchunks = (nk + ks - 1) / ks;
  ks = (nk + kchunks - 1) / kchunks;
  a.ksplit = ks;
  a.kchunks = kchunks;
  a.part_out = c->sc_parts;
  a.part_stride = (size_t)c->rows_step * m.d_model;
  REFUSE_IF(c, dg_launch_ws(WS_EPI_ADD_F32, a, padded * a.msplit * ks, s) != 0, "self-conditioning product");
  REFUSE_IF(c, dg_launch_sc_fold(c->sc_parts, ks, a.part_stride, m.d_model, c->open_rows, c->n_open_rows, max_rows,
                                 sc_slots(c, slot_req), c->C, s) != 0, "self-conditioning fold");
}

// Attention half of layer l over `rows` rows in c->x.
// norm_done: c->xn already holds the normalised rows (fused into the previous
// layer's combine).
// Returns the output projection's pending partial sums (bf16 model), which the
// caller folds into c->x with its next row kernel.
DgParts attn_half(dg_ctx* c, int l, const std::vector<SlotRow>& slots, int rows, bool causal, bool norm_done = false) {
  const dg_model_config& m = c->cfg;
  const dg_layer_weights& w = c->layers[l];
  hipStream_t s = c->stream;
  const DgShape sh = shape_of(c);
  const DgSegs sg = make_segs(c, slots, l, causal);
  if (!norm_done)
    KT(c, DG_KF_RMSNORM, dg_launch_rmsnorm(c->dtype, c->x, nullptr, nullptr, rows, m.d_model, w.attn_norm, m.rms_eps,
                                           c->xn, c->dtype == DG_BF16, s));
  KT(c, DG_KF_QKV, launch_qkv(c, w, rows, sg));
  const int max_splits = std::max(1, (int)(c->attn_cap / (size_t)rows));
  const int ns = dg_attn_splits(sg, sh, std::min(max_splits, 64), dg_attn_qrows(c->dtype, sh.hd));
  KT(c, DG_KF_ATTENTION, dg_launch_attention(c->dtype, c->q, sh, sg, ns, c->opart, c->mlpart, c->ao, rows, s));
  DgParts pend;
  if (c->dtype == DG_F32)
    KT(c, DG_KF_OUT_PROJ, dg_launch_gemm(c->dtype, 2, c->ao, rows, m.n_q_heads * m.head_dim, w.wo, m.d_model, c->x,
                                         m.d_model, s));
  else
    KT(c, DG_KF_OUT_PROJ, pend = launch_dense_add(c, c->ao, rows, m.n_q_heads * m.head_dim, w.wo, m.d_model, c->x,
                                                  nullptr, nullptr, DG_MAX_KSPLIT, 128, DG_OUTPROJ_BN));
  return pend;
}

// FFN half of layer l over `rows` rows in c->x; routing written to ids/gates,
// router logits to rlog ([rows][E] fp32).  next_gain: the RMSNorm gain of the
// next layer's attention, applied to the updated rows into c->xn by the combine.
// pend: the output projection's partial sums, folded into c->x by the FFN norm.
void ffn_half(dg_ctx* c, int l, int rows, int32_t* ids, float* gates, float* rlog, const void* next_gain = nullptr,
              const DgParts& pend = DgParts{}) {
  const dg_model_config& m = c->cfg;
  const dg_layer_weights& w = c->layers[l];
  hipStream_t s = c->stream;
  // bf16: fragment-major for the dense projections, and a row-major copy that the
  // routed launches read through the sorted-row -> token map
  KT(c, DG_KF_RMSNORM,
     REFUSE_IF(c, dg_launch_rmsnorm(c->dtype, c->x, nullptr, nullptr, rows, m.d_model, w.ffn_norm, m.rms_eps, c->xn,
                                    c->dtype == DG_BF16, s, c->dtype == DG_BF16 ? c->xr : nullptr, pend) != 0,
               "FFN norm"));
  tap_rows(c, 2 * l + 1, rows);  // x after the attention half (its partial sums are folded now)
  DgParts pend2;  // the shared expert's W2 partial sums, folded by the combine
  if (c->dtype == DG_F32) {
    KT(c, DG_KF_ROUTER, dg_launch_gemm(c->dtype, 1, c->xn, rows, m.d_model, w.router, m.n_experts, rlog, m.n_experts, s);
                            dg_launch_topk(rlog, rows, m.n_experts, m.top_k, ids, gates, s));
    KT(c, DG_KF_PERMUTE, dg_launch_permute(ids, rows, m.n_experts, m.top_k, c->counts, c->offsets, c->perm, s));
    KT(c, DG_KF_EXPERT_UP, dg_launch_expert_up(c->dtype, c->xn, rows, m.d_model, m.n_experts, m.top_k, m.expert_hidden, w.w1, w.w3,
                                               c->counts, c->offsets, c->perm, c->hbuf, s));
    KT(c, DG_KF_EXPERT_DOWN, dg_launch_expert_down(c->dtype, c->hbuf, rows, m.d_model, m.n_experts, m.top_k, m.expert_hidden, w.w2,
                                                   c->counts, c->offsets, c->perm, c->ybuf, s));
    KT(c, DG_KF_SHARED_UP, dg_launch_swiglu(c->dtype, c->xn, rows, m.d_model, w.sw1, w.sw3, m.shared_hidden, c->hs, s));
    KT(c, DG_KF_SHARED_DOWN, dg_launch_gemm(c->dtype, 2, c->hs, rows, m.shared_hidden, w.sw2, m.d_model, c->x, m.d_model, s));
  } else {
    // The shared expert depends only on the normalised rows: it runs on the side
    // stream beside the router, the routing and the routed launches, filling the
    // GPU while those small or draining launches leave it idle.  (Forking later,
    // beside the routed launches alone, measured slower: they then share HBM.)
    HIPCK_V(hipEventRecord(c->ev_fork, s));
    HIPCK_V(hipStreamWaitEvent(c->side, c->ev_fork, 0));
    KTS(c, DG_KF_SHARED_UP, c->side, launch_dense(c, WS_EPI_SWIGLU, c->xn, rows, m.d_model, w.sw1, w.sw3, m.shared_hidden,
                                                  c->hs, m.shared_hidden, c->side));
    // W2 adds straight into the residual: off the critical path, a split
    // reduction would only add its partial sums to the combine's reads.  Nothing
    // on the main stream touches c->x between the fork and the join.
    KTS(c, DG_KF_SHARED_DOWN, c->side, pend2 = launch_dense_add(c, c->hs, rows, m.shared_hidden, w.sw2, m.d_model, c->x,
                                                                c->side, c->parts2, 1, DG_SHARED_W2_ROWS));
    HIPCK_V(hipEventRecord(c->ev_join, c->side));
    KT(c, DG_KF_ROUTER, dg_launch_router(c->xn, rows, m.d_model, w.router, m.n_experts, rlog, s, DG_ROUTER_KSPLIT));
    // n-blocks: k_wsd's width (dg_wsd_bn weight rows; SwiGLU: half of them W1),
    // k_ws's 64 weight rows
    const int bn_up = routed_kernel(c) == 1 ? dg_wsd_bn(WS_EPI_SWIGLU) : 64;
    const int bn_dn = routed_kernel(c) == 1 ? dg_wsd_bn(WS_EPI_STORE_F32) : 64;
    const int nb_up = (m.expert_hidden + bn_up / 2 - 1) / (bn_up / 2), nb_dn = (m.d_model + bn_dn - 1) / bn_dn;
    // routed experts over the expert-sorted rows: W1/W3 + SwiGLU into c->hbuf,
    // W2 from there into c->ybuf at each row's pair index.  Both kernels read
    // the normalised rows (row-major c->xr) through rowsrc; c->hbuf is
    // fragment-major.
    const bool wsd = routed_kernel(c) == 1;
    const int la = list_blocks(c, WS_EPI_SWIGLU, nb_up), lb = list_blocks(c, WS_EPI_STORE_F32, nb_dn);
    if (wsd && rows <= DG_ROUTE_MAX_ROWS && m.n_experts <= 256 && 16 * m.top_k <= 256) {
      // the permutation and the work lists in one launch of parallel blocks
      KT(c, DG_KF_PERMUTE, dg_launch_topk(rlog, rows, m.n_experts, m.top_k, ids, gates, s, DG_ROUTER_KSPLIT);
         REFUSE_IF(c, dg_launch_route_perm(ids, rows, m.n_experts, m.top_k, c->counts, c->offsets, c->perm,
                                           c->offsets16, c->rowsrc, c->n_units + 2, routed_part_rows(c), la,
                                           c->units_up, c->n_units, lb, c->units_dn, c->n_units + 1,
                                           DG_ROUTE_LPT, s) != 0,
                   "routing"));
    } else {
      KT(c, DG_KF_PERMUTE, dg_launch_route(rlog, rows, m.n_experts, m.top_k, ids, gates, c->counts, c->offsets,
                                           c->perm, c->offsets16, c->rowsrc, c->n_units + 2, routed_part_rows(c), la,
                                           c->units_up, c->n_units, lb, c->units_dn, c->n_units + 1, s, wsd,
                                           DG_ROUTER_KSPLIT));
    }
    KT(c, DG_KF_EXPERT_UP, launch_routed(c, WS_EPI_SWIGLU, c->xr, w.w1, w.w3, w.w1_scale, w.w3_scale, w.w1_mx_scale,
                                         w.w3_mx_scale, (size_t)m.expert_hidden * m.d_model, m.d_model,
                                         m.expert_hidden, c->units_up, c->n_units, nb_up, c->hbuf, m.expert_hidden,
                                         c->rowsrc));
    KT(c, DG_KF_EXPERT_DOWN, launch_routed(c, WS_EPI_STORE_F32, c->hbuf, w.w2, nullptr, w.w2_scale, nullptr,
                                           w.w2_mx_scale, nullptr, (size_t)m.d_model * m.expert_hidden,
                                           m.expert_hidden, m.d_model, c->units_dn, c->n_units + 1, nb_dn, c->ybuf,
                                           m.d_model));
  }
  if (c->dtype == DG_BF16) HIPCK_V(hipStreamWaitEvent(s, c->ev_join, 0));  // the shared expert is done
  KT(c, DG_KF_COMBINE,
     REFUSE_IF(c, dg_launch_combine_norm(c->dtype, c->x, c->ybuf, gates, rows, m.d_model, m.top_k, next_gain,
                                         m.rms_eps, c->xn, c->dtype == DG_BF16, s, pend2) != 0,
               "MoE combine"));
}

// Forward of the rows in c->x through all layers.  kv_only: the last layer only
// writes its K/V (commit and prefill need nothing else from it).
void forward_layers(dg_ctx* c, const std::vector<SlotRow>& slots, int rows, bool causal, bool kv_only, bool tap) {
  const dg_model_config& m = c->cfg;
  bool xn_ready = false;  // c->xn holds layer l's attention-normalised rows
  for (int l = 0; l < m.n_layers; ++l) {
    const bool last = l == m.n_layers - 1;
    if (last && kv_only) {
      const DgSegs sg = make_segs(c, slots, l, causal);
      const dg_layer_weights& w = c->layers[l];
      if (!xn_ready)
        KT(c, DG_KF_RMSNORM, dg_launch_rmsnorm(c->dtype, c->x, nullptr, nullptr, rows, m.d_model, w.attn_norm,
                                               m.rms_eps, c->xn, c->dtype == DG_BF16, c->stream));
      KT(c, DG_KF_QKV, launch_qkv(c, w, rows, sg));
      break;
    }
    tap_rows(c, 2 * l, rows);
    const DgParts pend = attn_half(c, l, slots, rows, causal, xn_ready);
    int32_t* ids = tap ? c->tap_ids + (size_t)l * c->rows_step * m.top_k : c->rids;
    float* gates = tap ? c->tap_gates + (size_t)l * c->rows_step * m.top_k : c->rgates;
    float* rlog = tap ? c->tap_logits + (size_t)l * tap_logit_stride(c) : c->rlogits;
    const void* next_gain = last ? nullptr : c->layers[l + 1].attn_norm;
    ffn_half(c, l, rows, ids, gates, rlog, next_gain, pend);
    xn_ready = next_gain != nullptr;
  }
  if (!kv_only) tap_rows(c, 2 * m.n_layers, rows);
}

// Sampler threshold in fixed point: floor(clamp(h, 0, 64) * 2^40), NaN as 64
// (the kernel converts entropies the same way; every product is exact in double).
uint64_t entropy_fixed(float h) {
  h = h >= 0.f ? std::min(h, 64.f) : (h < 0.f ? 0.f : 64.f);
  return (uint64_t)((double)h * 1099511627776.0);
}

DgSampleArgs sample_args(const dg_ctx* c, const std::vector<int>& slot_req) {
  DgSampleArgs a;
  memset(&a, 0, sizeof a);
  for (size_t i = 0; i < slot_req.size(); ++i) {
    const int r = slot_req[i];
    a.s[i].ids = c->canvas_ids + (size_t)r * c->C;
    a.s[i].accepted = c->canvas_acc + (size_t)r * c->C;
    a.s[i].prev = c->canvas_prev + (size_t)r * c->C;
    a.s[i].seed = c->req[r].seed;
    a.s[i].block = c->req[r].block;
    a.s[i].step = c->req[r].step + 1;
    a.s[i].row0 = (int)i * c->C;
  }
  a.count = (int)slot_req.size();
  a.C = c->C;
  a.vocab = c->cfg.vocab;
  a.max_steps = c->scfg.max_steps > 0 ? c->scfg.max_steps : c->C;
  a.tau = c->scfg.tau;
  a.mode = c->scfg.mode;
  a.budget_q = entropy_fixed(c->scfg.budget);
  a.stop_q = entropy_fixed(c->scfg.stop_entropy);
  return a;
}

dg_status check_req(dg_ctx* c, int32_t req) {
  if (!c) return DG_ERR_INVALID_ARG;
  if (req < 0 || req >= c->cfg.max_requests)
    return fail(c, DG_ERR_CAPACITY, "request %d outside [0, %d)", req, c->cfg.max_requests);
  return DG_OK;
}

double now_ms() {
  return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now().time_since_epoch()).count();
}


}  // namespace

extern "C" {

dg_status dg_workspace_size(const dg_model_config* cfg, size_t* kv_bytes, size_t* scratch_bytes) {
  const char* msg = check_config(cfg);
  if (msg) return fail(nullptr, DG_ERR_INVALID_ARG, "%s", msg);
  if (!kv_bytes || !scratch_bytes) return fail(nullptr, DG_ERR_INVALID_ARG, "null output pointer");
  dg_ctx tmp;
  *kv_bytes = kv_size(*cfg);
  *scratch_bytes = carve(&tmp, *cfg, nullptr);
  return DG_OK;
}

dg_status dg_create(const dg_model_config* cfg, const dg_sampler_config* scfg, const dg_weights* weights,
                    void* kv_dev, size_t kv_bytes, void* scratch_dev, size_t scratch_bytes, void* stream,
                    dg_ctx** out) {
  if (out) *out = nullptr;
  if (!out) return fail(nullptr, DG_ERR_INVALID_ARG, "null output pointer");
  const char* msg = check_config(cfg);
  if (msg) return fail(nullptr, DG_ERR_INVALID_ARG, "%s", msg);
  if (!scfg) return fail(nullptr, DG_ERR_INVALID_ARG, "null sampler config");
  if (!(scfg->tau >= 0.f)) return fail(nullptr, DG_ERR_INVALID_ARG, "tau must be >= 0");
  if (scfg->mode != DG_SAMPLER_THRESHOLD && scfg->mode != DG_SAMPLER_BUDGET)
    return fail(nullptr, DG_ERR_INVALID_ARG, "unknown sampler mode %d", scfg->mode);
  if (scfg->mode == DG_SAMPLER_BUDGET &&
      !(scfg->budget >= 0.f && scfg->budget <= 64.f && scfg->stop_entropy >= 0.f && scfg->stop_entropy <= 64.f))
    return fail(nullptr, DG_ERR_INVALID_ARG, "budget and stop_entropy must lie in [0, 64]");
  if (!weights || !weights->embed || !weights->final_norm || !weights->layers)
    return fail(nullptr, DG_ERR_INVALID_ARG, "null weights");
  for (int l = 0; l < cfg->n_layers; ++l) {
    const dg_layer_weights& w = weights->layers[l];
    const void* ps[] = {w.attn_norm, w.wq, w.wk, w.wv, w.wo, w.ffn_norm, w.router, w.w1, w.w3, w.w2, w.sw1, w.sw3, w.sw2};
    for (const void* p : ps)
      if (!p) return fail(nullptr, DG_ERR_INVALID_ARG, "null weight pointer in layer %d", l);
    if (cfg->expert_format == DG_EXPERTS_FP8 && (!w.w1_scale || !w.w3_scale || !w.w2_scale))
      return fail(nullptr, DG_ERR_INVALID_ARG, "null expert scale pointer in layer %d", l);
    if (cfg->expert_format == DG_EXPERTS_MXFP4 && (!w.w1_mx_scale || !w.w3_mx_scale || !w.w2_mx_scale))
      return fail(nullptr, DG_ERR_INVALID_ARG, "null expert block-scale pointer in layer %d", l);
  }
  if (cfg->self_cond_hidden > 0 && (!weights->sc_w1 || !weights->sc_w3 || !weights->sc_w2))
    return fail(nullptr, DG_ERR_INVALID_ARG, "null self-conditioning weight pointer");
  if (!kv_dev || !scratch_dev) return fail(nullptr, DG_ERR_INVALID_ARG, "null kv or scratch buffer");
  dg_model_config m = *cfg;
  if (m.prefill_chunk == 0) m.prefill_chunk = 2048;
  size_t need_kv = 0, need_scratch = 0;
  dg_workspace_size(&m, &need_kv, &need_scratch);
  if (kv_bytes < need_kv || scratch_bytes < need_scratch)
    return fail(nullptr, DG_ERR_WORKSPACE, "workspace too small: kv %zu < %zu or scratch %zu < %zu", kv_bytes,
                need_kv, scratch_bytes, need_scratch);

  dg_ctx* c = new dg_ctx();
  c->cfg = m;
  c->scfg = *scfg;
  c->dtype = m.dtype;
  c->esz = m.dtype == DG_BF16 ? 2 : 4;
  c->embed = weights->embed;
  c->final_norm = weights->final_norm;
  c->layers.assign(weights->layers, weights->layers + m.n_layers);
  if (m.expert_format == DG_EXPERTS_MXFP4) {
    // k_wsd copies a unit's block scales into LDS in 16-byte pieces: every scale
    // array 16-byte aligned, whole pieces per 64 rows, and 128 rows of K / 32
    // bytes within its LDS copy
    bool ok = m.expert_hidden % 8 == 0 && m.d_model % 8 == 0 && 128 * (m.d_model / 32) <= 16384 &&
              128 * (m.expert_hidden / 32) <= 16384;
    for (const dg_layer_weights& w : c->layers)
      for (const void* p : {w.w1_mx_scale, w.w3_mx_scale, w.w2_mx_scale}) ok = ok && (uintptr_t)p % 16 == 0;
    c->mx_wsd = ok;
  }
  if (m.self_cond_hidden > 0) {
    c->sc_w1 = weights->sc_w1;
    c->sc_w3 = weights->sc_w3;
    c->sc_w2 = weights->sc_w2;
  }
  c->kv = (char*)kv_dev;
  c->stream = (hipStream_t)stream;
  c->C = m.canvas_len;
  c->rows_step = m.max_requests * m.canvas_len;
  c->prefill_chunk = m.prefill_chunk;
  c->rows_max = std::max(c->rows_step, c->prefill_chunk);
  c->lm_tiles = dg_lm_head_tiles(m.vocab);
  c->req.resize(m.max_requests);
  carve(c, m, (char*)scratch_dev);
  {  // the static scratch of dg_op_lm_head_noalloc on this device; only that call needs it
    const hipError_t es = noalloc_scratch_ptr(&c->noalloc_scratch);
    if (es != hipSuccess) {
      c->noalloc_scratch = nullptr;
      c->noalloc_err = hipGetErrorString(es);
      (void)hipGetLastError();
    }
  }

  std::vector<double> inv(m.head_dim / 2);
  for (int j = 0; j < m.head_dim / 2; ++j) inv[j] = std::pow((double)m.rope_theta, -2.0 * j / m.head_dim);
  hipError_t e = hipMemcpyAsync(c->inv_freq, inv.data(), inv.size() * 8, hipMemcpyHostToDevice, c->stream);
  // Keys past a request's length are read (with zero weight) by the attention
  // tiles; zeroing the cache once keeps those reads finite.
  if (e == hipSuccess) e = hipMemsetAsync(c->kv, 0, need_kv, c->stream);
  if (e == hipSuccess) e = hipMemsetAsync(c->canvas_acc, 1, c->rows_step, c->stream);
  if (e == hipSuccess && m.self_cond_hidden > 0) {
    if (dg_launch_transpose_bf16(c->embed, m.vocab, m.d_model, c->embed_t, c->stream) != 0) e = hipErrorInvalidValue;
    dg_launch_fill_zero(c->sc_state, (size_t)c->rows_step * m.d_model, c->stream);
    if (e == hipSuccess) e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipHostMalloc((void**)&c->info_host, m.max_requests * 4 * sizeof(int32_t));
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking);  // default priority
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_fork, hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&c->ev_join, hipEventDisableTiming);
  if (e == hipSuccess) e = hipStreamSynchronize(c->stream);
  if (e != hipSuccess) {
    fail(nullptr, DG_ERR_HIP, "create: %s", hipGetErrorString(e));
    if (c->info_host) hipHostFree(c->info_host);
    if (c->ev_fork) hipEventDestroy(c->ev_fork);
    if (c->ev_join) hipEventDestroy(c->ev_join);
    if (c->side) hipStreamDestroy(c->side);
    delete c;
    return DG_ERR_HIP;
  }
  *out = c;
  return DG_OK;
}

void dg_destroy(dg_ctx* ctx) {
  if (!ctx) return;
  hipStreamSynchronize(ctx->stream);
  if (ctx->side) hipStreamSynchronize(ctx->side);
  for (hipEvent_t e : ctx->kt_ev) hipEventDestroy(e);
  if (ctx->ev_fork) hipEventDestroy(ctx->ev_fork);
  if (ctx->ev_join) hipEventDestroy(ctx->ev_join);
  if (ctx->side) hipStreamDestroy(ctx->side);
  if (ctx->info_host) hipHostFree(ctx->info_host);
  delete ctx;
}

const char* dg_last_error(const dg_ctx* ctx) { return ctx ? ctx->err.c_str() : g_create_error.c_str(); }

dg_status dg_prefill(dg_ctx* c, int32_t req, const int32_t* prompt_ids, int32_t n, uint64_t seed) {
  dg_status st = check_req(c, req);
  if (st != DG_OK) return st;
  if (n < 0 || (n > 0 && !prompt_ids)) return fail(c, DG_ERR_INVALID_ARG, "bad prompt");
  if (n + c->C > c->cfg.max_ctx)
    return fail(c, DG_ERR_CAPACITY, "prompt of %d tokens plus one canvas exceeds max_ctx %d", n, c->cfg.max_ctx);
  for (int i = 0; i < n; ++i)
    if (prompt_ids[i] < 0 || prompt_ids[i] >= c->cfg.vocab)
      return fail(c, DG_ERR_INVALID_ARG, "prompt id %d at %d out of range", prompt_ids[i], i);
  for (int c0 = 0; c0 < n; c0 += c->prefill_chunk) {
    const int cn = std::min(c->prefill_chunk, n - c0);
    HIPCK(c, hipMemcpyAsync(c->ids_stage, prompt_ids + c0, cn * 4, hipMemcpyHostToDevice, c->stream));
    dg_launch_embed(c->dtype, c->ids_stage, cn, c->embed, c->cfg.d_model, c->cfg.vocab, c->x, c->stream);
    std::vector<SlotRow> slots{{req, c0, cn}};
    forward_layers(c, slots, cn, true, true, false);
    LAUNCHCK(c);
    // the staging buffer is reused by the next chunk
    HIPCK(c, hipStreamSynchronize(c->stream));
  }
  HIPCK(c, hipStreamSynchronize(c->stream));
  Request& r = c->req[req];
  r = Request();
  r.prefilled = true;
  r.P = n;
  r.seed = seed;
  return DG_OK;
}

dg_status dg_denoise_step(dg_ctx* c, dg_step_info* info) {
  if (!c || !info) return fail(c, DG_ERR_INVALID_ARG, "null argument");
  const int R = c->cfg.max_requests;
  std::vector<int> slot_req, fresh;
  for (int r = 0; r < R; ++r) {
    Request& q = c->req[r];
    info[r] = dg_step_info{0, q.block, q.step, 0, 0, 0, q.done ? 1 : 0};
    if (!q.prefilled) continue;
    if (q.active && q.done) continue;
    if (!q.active && q.P + c->C > c->cfg.max_ctx) continue;
    slot_req.push_back(r);
    if (!q.active) fresh.push_back(r);
  }
  if (slot_req.empty()) return fail(c, DG_ERR_STATE, "no request can take a denoising step");
  c->kt_on = c->kt_calls++ % c->kt_every == 0;
  hipStream_t s = c->stream;
  if (!fresh.empty()) {
    for (int r : fresh) {
      c->req[r].active = true;
      c->req[r].done = false;
      c->req[r].step = 0;
    }
    DgSampleArgs ia = sample_args(c, fresh);
    dg_launch_canvas_init(ia, c->open_rows, c->n_open_rows, s);
    if (c->cfg.self_cond_hidden > 0)  // a new canvas starts with a zero state
      for (int r : fresh)
        dg_launch_fill_zero(c->sc_state + (size_t)r * c->C * c->cfg.d_model, (size_t)c->C * c->cfg.d_model, s);
  }
  const DgSampleArgs a = sample_args(c, slot_req);
  const int rows = a.count * c->C;
  std::vector<SlotRow> slots;
  for (int r : slot_req) slots.push_back({r, c->req[r].P, c->C});
  dg_launch_open_rows(a, c->open_rows, c->n_open_rows, s);
  KT(c, DG_KF_EMBED, dg_launch_embed_slots(c->dtype, a, c->embed, c->cfg.d_model, c->x, s));
  sc_embed(c, slot_req, rows);
  c->tap_on = c->tap_buf != nullptr;
  c->tap_valid = c->tap_on;
  forward_layers(c, slots, rows, false, false, true);
  c->tap_on = false;
  KT(c, DG_KF_RMSNORM, dg_launch_rmsnorm(c->dtype, c->x, c->open_rows, c->n_open_rows, rows, c->cfg.d_model, c->final_norm,
                                         c->cfg.rms_eps, c->hn, c->dtype == DG_BF16, s));
  const bool sc = c->cfg.self_cond_hidden > 0;
  KT(c, DG_KF_LM_HEAD, launch_lm_head(c, c->n_open_rows, rows, c->open_rows, c->ent, c->lse, c->amax,
                                      sc ? c->sc_z : nullptr));
  // the positions open at the start of the step take this step's softmax
  if (sc) KT(c, DG_KF_SELF_COND, sc_update(c, slot_req, rows));
  KT(c, DG_KF_SAMPLE, dg_launch_sample(a, c->ent, c->amax, c->info_dev, nullptr, nullptr, s));
  LAUNCHCK(c);
  HIPCK(c, hipMemcpyAsync(c->info_host, c->info_dev, a.count * 4 * sizeof(int32_t), hipMemcpyDeviceToHost, s));
  HIPCK(c, hipStreamSynchronize(s));
  kt_collect(c);
  for (size_t i = 0; i < slot_req.size(); ++i) {
    const int r = slot_req[i];
    Request& q = c->req[r];
    q.step += 1;
    q.done = c->info_host[i * 4 + 3] != 0;
    info[r] = dg_step_info{1, q.block, q.step, c->info_host[i * 4 + 0], c->info_host[i * 4 + 1],
                           c->info_host[i * 4 + 2], q.done ? 1 : 0};
  }
  c->last_slots = slot_req;
  c->last_rows = rows;
  return DG_OK;
}

dg_status dg_commit_block(dg_ctx* c, int32_t req, int32_t* out_ids) {
  dg_status st = check_req(c, req);
  if (st != DG_OK) return st;
  Request& q = c->req[req];
  if (!q.active || !q.done) return fail(c, DG_ERR_STATE, "request %d has no finished canvas", req);
  c->kt_on = c->kt_calls++ % c->kt_every == 0;
  hipStream_t s = c->stream;
  std::vector<int> one{req};
  const DgSampleArgs a = sample_args(c, one);
  dg_launch_embed_slots(c->dtype, a, c->embed, c->cfg.d_model, c->x, s);
  sc_embed(c, one, c->C);
  std::vector<SlotRow> slots{{req, q.P, c->C}};
  forward_layers(c, slots, c->C, false, true, false);
  LAUNCHCK(c);
  if (out_ids)
    HIPCK(c, hipMemcpyAsync(out_ids, c->canvas_ids + (size_t)req * c->C, c->C * 4, hipMemcpyDeviceToHost, s));
  HIPCK(c, hipStreamSynchronize(s));
  kt_collect(c);
  q.P += c->C;
  q.block += 1;
  q.step = 0;
  q.active = false;
  q.done = false;
  return DG_OK;
}

dg_status dg_generate(dg_ctx* c, int32_t n_req, const int32_t* const* prompts, const int32_t* n_prompt,
                      int32_t n_out, const uint64_t* seeds, int32_t* const* out_ids, dg_stats* stats) {
  if (!c) return DG_ERR_INVALID_ARG;
  if (n_req <= 0 || n_req > c->cfg.max_requests)
    return fail(c, DG_ERR_CAPACITY, "n_req %d outside [1, %d]", n_req, c->cfg.max_requests);
  if (!prompts || !n_prompt || !seeds || !out_ids || n_out <= 0) return fail(c, DG_ERR_INVALID_ARG, "bad argument");
  const int C = c->C;
  const int n_blocks = (n_out + C - 1) / C;
  for (int r = 0; r < n_req; ++r) {
    if (!out_ids[r]) return fail(c, DG_ERR_INVALID_ARG, "null output of request %d", r);
    if (n_prompt[r] + (int64_t)n_blocks * C > c->cfg.max_ctx)
      return fail(c, DG_ERR_CAPACITY, "request %d: prompt %d + %d blocks exceeds max_ctx", r, n_prompt[r], n_blocks);
  }
  dg_stats stt{};
  // requests beyond n_req take no part
  for (int r = n_req; r < c->cfg.max_requests; ++r) c->req[r] = Request();
  double t0 = now_ms();
  for (int r = 0; r < n_req; ++r) {
    dg_status st = dg_prefill(c, r, prompts[r], n_prompt[r], seeds[r]);
    if (st != DG_OK) return st;
  }
  stt.prefill_ms = now_ms() - t0;
  std::vector<dg_step_info> info(c->cfg.max_requests);
  std::vector<int32_t> blk(C);
  for (int b = 0; b < n_blocks; ++b) {
    while (true) {
      t0 = now_ms();
      dg_status st = dg_denoise_step(c, info.data());
      if (st != DG_OK) return st;
      stt.decode_ms += now_ms() - t0;
      stt.steps += 1;
      bool all_done = true;
      for (int r = 0; r < n_req; ++r) {
        if (info[r].active) stt.tokens += info[r].n_accepted + info[r].n_forced;
        all_done = all_done && c->req[r].done;
      }
      if (all_done) break;
    }
    t0 = now_ms();
    for (int r = 0; r < n_req; ++r) {
      dg_status st = dg_commit_block(c, r, blk.data());
      if (st != DG_OK) return st;
      const int take = std::min(C, n_out - b * C);
      memcpy(out_ids[r] + b * C, blk.data(), take * sizeof(int32_t));
    }
    stt.commit_ms += now_ms() - t0;
  }
  if (stats) *stats = stt;
  return DG_OK;
}

dg_status dg_get_request(dg_ctx* c, int32_t req, dg_request_state* st) {
  dg_status s = check_req(c, req);
  if (s != DG_OK) return s;
  if (!st) return fail(c, DG_ERR_INVALID_ARG, "null output");
  const Request& q = c->req[req];
  *st = dg_request_state{q.prefilled, q.P, q.block, q.step, q.active, q.done, q.seed};
  return DG_OK;
}

dg_status dg_get_canvas(dg_ctx* c, int32_t req, int32_t* ids, uint8_t* accepted) {
  dg_status s = check_req(c, req);
  if (s != DG_OK) return s;
  if (!c->req[req].active) return fail(c, DG_ERR_STATE, "request %d has no canvas", req);
  if (ids) HIPCK(c, hipMemcpyAsync(ids, c->canvas_ids + (size_t)req * c->C, c->C * 4, hipMemcpyDeviceToHost, c->stream));
  if (accepted)
    HIPCK(c, hipMemcpyAsync(accepted, c->canvas_acc + (size_t)req * c->C, c->C, hipMemcpyDeviceToHost, c->stream));
  HIPCK(c, hipStreamSynchronize(c->stream));
  return DG_OK;
}

dg_status dg_set_canvas(dg_ctx* c, int32_t req, const int32_t* ids, const uint8_t* accepted, int32_t step,
                        int32_t block) {
  dg_status s = check_req(c, req);
  if (s != DG_OK) return s;
  Request& q = c->req[req];
  if (!q.prefilled) return fail(c, DG_ERR_STATE, "request %d is not prefilled", req);
  if (!ids || !accepted || step < 0 || block < 0) return fail(c, DG_ERR_INVALID_ARG, "bad canvas state");
  if (q.P + c->C > c->cfg.max_ctx) return fail(c, DG_ERR_CAPACITY, "no room for a canvas");
  int open = 0;
  for (int i = 0; i < c->C; ++i) {
    if (ids[i] < 0 || ids[i] >= c->cfg.vocab) return fail(c, DG_ERR_INVALID_ARG, "canvas id out of range");
    if (accepted[i] > 1) return fail(c, DG_ERR_INVALID_ARG, "accepted flags must be 0 or 1");
    open += accepted[i] == 0;
  }
  HIPCK(c, hipMemcpyAsync(c->canvas_ids + (size_t)req * c->C, ids, c->C * 4, hipMemcpyHostToDevice, c->stream));
  HIPCK(c, hipMemcpyAsync(c->canvas_acc + (size_t)req * c->C, accepted, c->C, hipMemcpyHostToDevice, c->stream));
  HIPCK(c, hipMemsetAsync(c->canvas_prev + (size_t)req * c->C, 0xff, c->C * 4, c->stream));  // -1: no previous step
  if (!q.active && c->cfg.self_cond_hidden > 0) {  // a new canvas starts from a zero self-conditioning state
    dg_launch_fill_zero(c->sc_state + (size_t)req * c->C * c->cfg.d_model, (size_t)c->C * c->cfg.d_model, c->stream);
    LAUNCHCK(c);
  }
  HIPCK(c, hipStreamSynchronize(c->stream));
  q.active = true;
  q.done = open == 0;
  q.step = step;
  q.block = block;
  return DG_OK;
}

dg_status dg_set_committed(dg_ctx* c, int32_t req, int32_t committed, uint64_t seed) {
  dg_status s = check_req(c, req);
  if (s != DG_OK) return s;
  if (committed < 0 || committed + c->C > c->cfg.max_ctx)
    return fail(c, DG_ERR_CAPACITY, "committed length %d leaves no room for a canvas", committed);
  Request& q = c->req[req];
  q = Request();
  q.prefilled = true;
  q.P = committed;
  q.seed = seed;
  return DG_OK;
}

dg_status dg_last_step_rows(dg_ctx* c, int32_t* n_rows, float* entropy, float* lse, int32_t* argmax,
                            int32_t* router_ids, float* router_gates) {
  if (!c) return DG_ERR_INVALID_ARG;
  if (c->last_rows == 0) return fail(c, DG_ERR_STATE, "no step has run");
  const int rows = c->last_rows;
  const int k = c->cfg.top_k;
  if (n_rows) *n_rows = rows;
  hipStream_t s = c->stream;
  if (entropy) HIPCK(c, hipMemcpyAsync(entropy, c->ent, rows * 4, hipMemcpyDeviceToHost, s));
  if (lse) HIPCK(c, hipMemcpyAsync(lse, c->lse, rows * 4, hipMemcpyDeviceToHost, s));
  if (argmax) HIPCK(c, hipMemcpyAsync(argmax, c->amax, rows * 4, hipMemcpyDeviceToHost, s));
  for (int l = 0; l < c->cfg.n_layers; ++l) {
    const size_t src = (size_t)l * c->rows_step * k, dst = (size_t)l * rows * k;
    if (router_ids)
      HIPCK(c, hipMemcpyAsync(router_ids + dst, c->tap_ids + src, (size_t)rows * k * 4, hipMemcpyDeviceToHost, s));
    if (router_gates)
      HIPCK(c, hipMemcpyAsync(router_gates + dst, c->tap_gates + src, (size_t)rows * k * 4, hipMemcpyDeviceToHost, s));
  }
  HIPCK(c, hipStreamSynchronize(s));
  return DG_OK;
}

dg_status dg_last_step_router_logits(dg_ctx* c, float* logits) {
  if (!c || !logits) return fail(c, DG_ERR_INVALID_ARG, "null argument");
  if (c->last_rows == 0) return fail(c, DG_ERR_STATE, "no step has run");
  const size_t per = (size_t)c->last_rows * c->cfg.n_experts;
  for (int l = 0; l < c->cfg.n_layers; ++l)
    HIPCK(c, hipMemcpyAsync(logits + l * per, c->tap_logits + (size_t)l * tap_logit_stride(c), per * 4,
                            hipMemcpyDeviceToHost, c->stream));
  HIPCK(c, hipStreamSynchronize(c->stream));
  return DG_OK;
}

// Each launcher's refusal path, reached on the host alone: the launcher is
// called with arguments it must refuse, which it does before any HIP call, and
// its -1 goes through REFUSE_IF and the refusal half of LAUNCHCK.
int32_t dg_debug_refusal_count(void) { return 11; }

dg_status dg_debug_refusal_case(int32_t i, char* msg, size_t msg_bytes) {
  if (i < 0 || i >= dg_debug_refusal_count()) return DG_ERR_INVALID_ARG;
  dg_ctx c;  // host-only stub: no stream, no device buffers
  memset(&c.cfg, 0, sizeof c.cfg);  // bf16 experts in native format, every size zero but those below
  c.cfg.d_model = 64;
  c.cfg.n_experts = 8;
  c.cfg.top_k = 2;
  c.rows_cap = 16;
  c.dtype = (i < 3) ? DG_F32 : DG_BF16;
  static int32_t dummy;  // a non-null work-list pointer the host never dereferences
  WsArgs a;
  memset(&a, 0, sizeof a);
  a.K = 96;
  a.N = 64;
  a.M = 16;
  DgParts parts;
  parts.n = 2;
  switch (i) {
    case 0: launch_dense(&c, WS_EPI_STORE_BF16, nullptr, 16, 64, nullptr, nullptr, 64, nullptr, 64); break;
    case 1: launch_dense_add(&c, nullptr, 16, 64, nullptr, 64, nullptr); break;
    case 2:
      launch_routed(&c, WS_EPI_SWIGLU, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 64, 64,
                    nullptr, nullptr, 2, nullptr, 64);
      break;
    case 3:  // an epilogue the dense kernel does not have
      launch_dense(&c, 99, nullptr, 16, 64, nullptr, nullptr, 64, nullptr, 64);
      break;
    case 4:  // a routed launch that neither gathers for SwiGLU nor stores fp32 rows
      c.counts = &dummy;
      launch_routed(&c, WS_EPI_ROPE_QKV, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, 64, 64,
                    &dummy, &dummy, 2, nullptr, 64, &dummy);
      break;
    case 5:  // MXFP4 weights with K not a multiple of 64
      a.counts = &dummy;
      a.wfmt = DG_WS_W_MXFP4;
      REFUSE_IF(&c, dg_launch_ws(WS_EPI_STORE_F32, a, 1, nullptr) != 0, "routed projection");
      break;
    case 6:  // FP8 weights on a dense launch
      a.wfmt = DG_WS_W_E4M3;
      REFUSE_IF(&c, dg_launch_ws(WS_EPI_STORE_F32, a, 1, nullptr) != 0, "dense projection");
      break;
    case 7:  // partial sums without the bf16 fragment-major output
      REFUSE_IF(&c, dg_launch_rmsnorm(DG_F32, nullptr, nullptr, nullptr, 16, 64, nullptr, 1e-6f, nullptr, false,
                                      nullptr, nullptr, parts) != 0,
                "FFN norm");
      break;
    case 8:
      REFUSE_IF(&c, dg_launch_combine_norm(DG_F32, nullptr, nullptr, nullptr, 16, 64, 2, nullptr, 1e-6f, nullptr,
                                           false, nullptr, parts) != 0,
                "combine and norm");
      break;
    case 9:  // a vocabulary that is not whole 64-row tiles
      REFUSE_IF(&c, dg_launch_transpose_bf16(nullptr, 100, 64, nullptr, nullptr) != 0, "embedding transpose");
      break;
    case 10: {  // rows that are not whole float4s
      DgScSlots sl;
      memset(&sl, 0, sizeof sl);
      REFUSE_IF(&c, dg_launch_sc_fold(nullptr, 2, 0, 6, nullptr, nullptr, 16, sl, 256, nullptr) != 0,
                "self-conditioning fold");
      break;
    }
  }
  const dg_status st = take_refusal(&c);
  if (msg && msg_bytes) snprintf(msg, msg_bytes, "%s", c.err.c_str());
  return st;
}

dg_status dg_debug_tap_size(const dg_model_config* cfg, size_t* bytes) {
  const char* msg = check_config(cfg);
  if (msg) return fail(nullptr, DG_ERR_INVALID_ARG, "%s", msg);
  if (!bytes) return fail(nullptr, DG_ERR_INVALID_ARG, "null output pointer");
  *bytes = (size_t)(2 * cfg->n_layers + 1) * cfg->max_requests * cfg->canvas_len * cfg->d_model * 4;
  return DG_OK;
}

dg_status dg_debug_set_tap_buffer(dg_ctx* c, void* tap_dev, size_t bytes) {
  if (!c) return DG_ERR_INVALID_ARG;
  if (!tap_dev) {
    c->tap_buf = nullptr;
    return DG_OK;
  }
  size_t need = 0;
  dg_debug_tap_size(&c->cfg, &need);
  if (bytes < need) return fail(c, DG_ERR_WORKSPACE, "tap buffer of %zu bytes < %zu", bytes, need);
  c->tap_buf = (float*)tap_dev;
  c->last_rows = 0;  // taps of earlier steps (if any) are not in the buffer
  return DG_OK;
}

dg_status dg_debug_tap(dg_ctx* c, int32_t which, int32_t layer, float* host_dst, size_t bytes) {
  if (!c) return DG_ERR_INVALID_ARG;
  if (!host_dst) return fail(c, DG_ERR_INVALID_ARG, "null destination");
  if (c->last_rows == 0) return fail(c, DG_ERR_STATE, "no step has run");
  const int L = c->cfg.n_layers;
  const size_t rows = c->last_rows, d = c->cfg.d_model;
  hipStream_t s = c->stream;
  if (which == DG_TAP_ROUTER_LOGITS) {
    if (layer < 0 || layer >= L) return fail(c, DG_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, L);
    const size_t n = rows * c->cfg.n_experts * 4;
    if (bytes < n) return fail(c, DG_ERR_INVALID_ARG, "destination of %zu bytes < %zu", bytes, n);
    HIPCK(c, hipMemcpyAsync(host_dst, c->tap_logits + (size_t)layer * tap_logit_stride(c), n,
                            hipMemcpyDeviceToHost, s));
    HIPCK(c, hipStreamSynchronize(s));
    return DG_OK;
  }
  int slot;
  if (which == DG_TAP_LAYER_INPUT) {
    if (layer < 0 || layer > L) return fail(c, DG_ERR_INVALID_ARG, "layer %d outside [0, %d]", layer, L);
    slot = 2 * layer;
  } else if (which == DG_TAP_AFTER_ATTENTION) {
    if (layer < 0 || layer >= L) return fail(c, DG_ERR_INVALID_ARG, "layer %d outside [0, %d)", layer, L);
    slot = 2 * layer + 1;
  } else {
    return fail(c, DG_ERR_INVALID_ARG, "unknown tap %d", which);
  }
  if (!c->tap_buf || !c->tap_valid) return fail(c, DG_ERR_STATE, "the last step ran without a tap buffer");
  const size_t n = rows * d * 4;
  if (bytes < n) return fail(c, DG_ERR_INVALID_ARG, "destination of %zu bytes < %zu", bytes, n);
  HIPCK(c, hipMemcpyAsync(host_dst, c->tap_buf + (size_t)slot * c->rows_step * d, n, hipMemcpyDeviceToHost, s));
  HIPCK(c, hipStreamSynchronize(s));
  return DG_OK;
}

dg_status dg_last_step_logits(dg_ctx* c, const int32_t* rows_list, int32_t n, float* logits_dev) {
  if (!c) return DG_ERR_INVALID_ARG;
  if (c->last_rows == 0) return fail(c, DG_ERR_STATE, "no step has run");
  if (n <= 0 || n > c->rows_step || !rows_list || !logits_dev) return fail(c, DG_ERR_INVALID_ARG, "bad row list");
  for (int i = 0; i < n; ++i)
    if (rows_list[i] < 0 || rows_list[i] >= c->last_rows) return fail(c, DG_ERR_INVALID_ARG, "row out of range");
  hipStream_t s = c->stream;
  HIPCK(c, hipMemcpyAsync(c->ids_stage, rows_list, n * 4, hipMemcpyHostToDevice, s));
  dg_launch_rmsnorm(c->dtype, c->x, c->ids_stage, nullptr, n, c->cfg.d_model, c->final_norm, c->cfg.rms_eps, c->hn, false, s);
  dg_launch_gemm(c->dtype, 1, c->hn, n, c->cfg.d_model, c->embed, c->cfg.vocab, logits_dev, c->cfg.vocab, s);
  LAUNCHCK(c);
  HIPCK(c, hipStreamSynchronize(s));
  return DG_OK;
}

dg_status dg_op_attention(dg_ctx* c, int32_t req, int32_t layer, float* x_dev, int32_t t, int32_t pos0,
                          int32_t causal) {
  dg_status st = check_req(c, req);
  if (st != DG_OK) return st;
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(c, DG_ERR_INVALID_ARG, "bad layer");
  if (!x_dev || t <= 0 || t > c->rows_max || pos0 < 0 || pos0 + t > c->cfg.max_ctx)
    return fail(c, DG_ERR_INVALID_ARG, "bad rows");
  const size_t bytes = (size_t)t * c->cfg.d_model * 4;
  HIPCK(c, hipMemcpyAsync(c->x, x_dev, bytes, hipMemcpyDeviceToDevice, c->stream));
  std::vector<SlotRow> slots{{req, pos0, t}};
  const DgParts pend = attn_half(c, layer, slots, t, causal != 0);
  // fold the output projection's partial sums into x (no norm follows here)
  if (pend.n > 0)
    REFUSE_IF(c, dg_launch_combine_norm(c->dtype, c->x, nullptr, nullptr, t, c->cfg.d_model, 0, nullptr,
                                        c->cfg.rms_eps, nullptr, true, c->stream, pend) != 0,
              "partial-sum fold");
  LAUNCHCK(c);
  HIPCK(c, hipMemcpyAsync(x_dev, c->x, bytes, hipMemcpyDeviceToDevice, c->stream));
  HIPCK(c, hipStreamSynchronize(c->stream));
  return DG_OK;
}

dg_status dg_op_moe(dg_ctx* c, int32_t layer, float* x_dev, int32_t t, int32_t* ids_dev, float* gates_dev) {
  if (!c) return DG_ERR_INVALID_ARG;
  if (layer < 0 || layer >= c->cfg.n_layers) return fail(c, DG_ERR_INVALID_ARG, "bad layer");
  if (!x_dev || t <= 0 || t > c->rows_max) return fail(c, DG_ERR_INVALID_ARG, "bad rows");
  const size_t bytes = (size_t)t * c->cfg.d_model * 4;
  HIPCK(c, hipMemcpyAsync(c->x, x_dev, bytes, hipMemcpyDeviceToDevice, c->stream));
  ffn_half(c, layer, t, c->rids, c->rgates, c->rlogits);
  LAUNCHCK(c);
  HIPCK(c, hipMemcpyAsync(x_dev, c->x, bytes, hipMemcpyDeviceToDevice, c->stream));
  const size_t kb = (size_t)t * c->cfg.top_k * 4;
  if (ids_dev) HIPCK(c, hipMemcpyAsync(ids_dev, c->rids, kb, hipMemcpyDeviceToDevice, c->stream));
  if (gates_dev) HIPCK(c, hipMemcpyAsync(gates_dev, c->rgates, kb, hipMemcpyDeviceToDevice, c->stream));
  HIPCK(c, hipStreamSynchronize(c->stream));
  return DG_OK;
}

dg_status dg_op_lm_head(dg_ctx* c, const float* h_dev, int32_t n, float* entropy_dev, float* lse_dev,
                        int32_t* argmax_dev) {
  if (!c) return DG_ERR_INVALID_ARG;
  if (!h_dev || n <= 0 || n > c->rows_step || !entropy_dev || !lse_dev || !argmax_dev)
    return fail(c, DG_ERR_INVALID_ARG, "bad arguments");
  hipStream_t s = c->stream;
  HIPCK(c, hipMemcpyAsync(c->n_open_rows, &n, 4, hipMemcpyHostToDevice, s));
  dg_launch_rmsnorm(c->dtype, h_dev, nullptr, c->n_open_rows, n, c->cfg.d_model, c->final_norm, c->cfg.rms_eps, c->hn, c->dtype == DG_BF16,
                    s);
  launch_lm_head(c, c->n_open_rows, n, nullptr, entropy_dev, lse_dev, argmax_dev);
  LAUNCHCK(c);
  HIPCK(c, hipStreamSynchronize(s));
  return DG_OK;
}

dg_status dg_op_lm_head_noalloc(dg_ctx* c, const float* h_dev, int32_t n, float* entropy_dev, float* lse_dev,
                                int32_t* argmax_dev) {
  if (!c) return DG_ERR_INVALID_ARG;
  if (!h_dev || n <= 0 || !entropy_dev || !lse_dev || !argmax_dev) return fail(c, DG_ERR_INVALID_ARG, "bad arguments");
  if (!c->noalloc_scratch)
    return fail(c, DG_ERR_HIP, "the static scratch has no device address: %s", c->noalloc_err.c_str());
  const size_t need = noalloc_lm_carve(c->cfg, n, nullptr, nullptr, nullptr, nullptr, nullptr);
  if (need > DG_NOALLOC_SCRATCH_BYTES) {
    int most = n;
    while (most > 1 && noalloc_lm_carve(c->cfg, most, nullptr, nullptr, nullptr, nullptr, nullptr) >
                           DG_NOALLOC_SCRATCH_BYTES)
      most = most * 7 / 8;
    return fail(c, DG_ERR_INVALID_ARG,
                "%d rows need %zu bytes of static scratch, more than its %u (about %d rows fit this model)", n, need,
                (unsigned)DG_NOALLOC_SCRATCH_BYTES, most);
  }
  int32_t* n_dev;
  void* hn;
  float* lpart;
  int32_t* lpart_arg;
  noalloc_lm_carve(c->cfg, n, (char*)c->noalloc_scratch, &n_dev, &hn, &lpart, &lpart_arg);
  hipStream_t s = c->stream;
  dg_launch_set_i32(n_dev, n, s);
  REFUSE_IF(c, dg_launch_rmsnorm(c->dtype, h_dev, nullptr, n_dev, n, c->cfg.d_model, c->final_norm, c->cfg.rms_eps,
                                 hn, c->dtype == DG_BF16, s) != 0,
            "final norm");
  launch_lm_head(c, n_dev, n, nullptr, entropy_dev, lse_dev, argmax_dev, nullptr, hn, lpart, lpart_arg);
  LAUNCHCK(c);
  return DG_OK;
}

dg_status dg_op_self_cond(dg_ctx* c, const float* u_dev, int32_t n, float* out_dev) {
  if (!c) return DG_ERR_INVALID_ARG;
  if (c->cfg.self_cond_hidden <= 0) return fail(c, DG_ERR_UNSUPPORTED, "the model has no self-conditioning");
  if (!u_dev || !out_dev || n <= 0 || n > c->rows_step) return fail(c, DG_ERR_INVALID_ARG, "bad arguments");
  hipStream_t s = c->stream;
  dg_launch_fill_zero(out_dev, (size_t)n * c->cfg.d_model, s);
  dg_launch_rows_to_fm(u_dev, n, c->cfg.d_model, c->sc_b, s);
  sc_mlp_add(c, n, out_dev);
  LAUNCHCK(c);
  HIPCK(c, hipStreamSynchronize(s));
  return DG_OK;
}

namespace {
dg_status sc_state_check(dg_ctx* c, int32_t req, const void* state) {
  dg_status st = check_req(c, req);
  if (st != DG_OK) return st;
  if (c->cfg.self_cond_hidden <= 0) return fail(c, DG_ERR_UNSUPPORTED, "the model has no self-conditioning");
  if (!state) return fail(c, DG_ERR_INVALID_ARG, "null state");
  if (!c->req[req].active) return fail(c, DG_ERR_STATE, "request %d has no canvas", req);
  return DG_OK;
}
}  // namespace

dg_status dg_get_self_cond(dg_ctx* c, int32_t req, float* state) {
  dg_status st = sc_state_check(c, req, state);
  if (st != DG_OK) return st;
  const size_t n = (size_t)c->C * c->cfg.d_model;
  HIPCK(c, hipMemcpyAsync(state, c->sc_state + (size_t)req * n, n * 4, hipMemcpyDeviceToHost, c->stream));
  HIPCK(c, hipStreamSynchronize(c->stream));
  return DG_OK;
}

dg_status dg_set_self_cond(dg_ctx* c, int32_t req, const float* state) {
  dg_status st = sc_state_check(c, req, state);
  if (st != DG_OK) return st;
  const size_t n = (size_t)c->C * c->cfg.d_model;
  HIPCK(c, hipMemcpyAsync(c->sc_state + (size_t)req * n, state, n * 4, hipMemcpyHostToDevice, c->stream));
  HIPCK(c, hipStreamSynchronize(c->stream));
  return DG_OK;
}

dg_status dg_op_sample(dg_ctx* c, int32_t req, const float* entropy_dev, const int32_t* argmax_dev, int32_t step,
                       dg_step_info* info) {
  dg_status st = check_req(c, req);
  if (st != DG_OK) return st;
  Request& q = c->req[req];
  if (!q.active) return fail(c, DG_ERR_STATE, "request %d has no canvas", req);
  if (!entropy_dev || !argmax_dev || !info || step < 1) return fail(c, DG_ERR_INVALID_ARG, "bad arguments");
  std::vector<int> one{req};
  DgSampleArgs a = sample_args(c, one);
  a.s[0].step = step;
  dg_launch_sample(a, entropy_dev, argmax_dev, c->info_dev, nullptr, nullptr, c->stream);
  LAUNCHCK(c);
  HIPCK(c, hipMemcpyAsync(c->info_host, c->info_dev, 4 * sizeof(int32_t), hipMemcpyDeviceToHost, c->stream));
  HIPCK(c, hipStreamSynchronize(c->stream));
  q.step = step;
  q.done = c->info_host[3] != 0;
  *info = dg_step_info{1, q.block, step, c->info_host[0], c->info_host[1], c->info_host[2], q.done ? 1 : 0};
  return DG_OK;
}

dg_status dg_philox_tokens(uint64_t seed, int32_t block, int32_t step, int32_t n, int32_t vocab, int32_t* out_dev,
                           void* stream) {
  if (n < 0 || vocab <= 0 || block < 0 || step < 0 || (n > 0 && !out_dev))
    return fail(nullptr, DG_ERR_INVALID_ARG, "bad arguments");
  hipStream_t s = (hipStream_t)stream;
  dg_launch_philox_tokens(seed, block, step, n, vocab, out_dev, s);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(nullptr, DG_ERR_HIP, "philox: %s", hipGetErrorString(e));
  return DG_OK;
}

dg_status dg_kernel_timer(dg_ctx* c, int32_t family) {
  if (!c) return DG_ERR_INVALID_ARG;
  if (family < 0 || family >= DG_KF_COUNT) return fail(c, DG_ERR_INVALID_ARG, "unknown kernel family %d", family);
  HIPCK(c, hipStreamSynchronize(c->stream));
  kt_collect(c);
  c->kt_family = family;
  c->kt_ms = 0.0;
  c->kt_launches = 0;
  return DG_OK;
}

dg_status dg_kernel_timer_every(dg_ctx* c, int32_t every) {
  if (!c) return DG_ERR_INVALID_ARG;
  if (every < 1) return fail(c, DG_ERR_INVALID_ARG, "every must be >= 1");
  c->kt_every = every;
  c->kt_calls = 0;
  return DG_OK;
}

dg_status dg_kernel_timer_read(dg_ctx* c, double* total_ms, int64_t* launches) {
  if (!c || !total_ms || !launches) return fail(c, DG_ERR_INVALID_ARG, "null argument");
  HIPCK(c, hipStreamSynchronize(c->stream));
  kt_collect(c);
  *total_ms = c->kt_ms;
  *launches = c->kt_launches;
  return DG_OK;
}

}  // extern "C"
