// Host side of the C ABI declared in include/dualar.h: validation, workspace
// carve-up, per-sequence state and the launch order of one decode frame.
//
// One frame ([P2] "Two autoregressions, because ten codebooks is ten times
// the sequence", the decode_one_token_ar order):
//   fusion of the previous frame -> n_layer x {QKV(+RMSNorm), attention
//   (+QK-norm, RoPE, cache append), O(+residual), W1|W3(+RMSNorm, SwiGLU),
//   W2(+residual)} -> tied head (+final RMSNorm) -> biased slow sample ->
//   fast pass 0 on the slow hidden state (slot 0) -> for k = 1..N-1:
//   fast pass k on E_fast[q^(k-1)] (slot k), fast head, unmasked sample.
// [P2] = "Fish Audio S2: a Qwen3-4B on the time axis, four layers on the
// codebook axis, and tags that are only text".
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "../../include/dualar.h"
#include "common.h"
#include "internal.h"

namespace {

// A host-side marker range around the enqueue of one part of the path
// (dualar.prefill, dualar.frame, dualar.slow, dualar.head, dualar.fast,
// dualar.fast_tf): rocprofv3 --marker-trace records it beside the kernels
// launched inside it.  Without a profiler attached a push or pop is a call
// that returns at once.
struct MarkerRange {
  explicit MarkerRange(const char* name) { roctxRangePush(name); }
  ~MarkerRange() { roctxRangePop(); }
  MarkerRange(const MarkerRange&) = delete;
  MarkerRange& operator=(const MarkerRange&) = delete;
};

thread_local std::string g_create_err;

constexpr size_t ALIGN = 256;
inline size_t up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Resolved {  // config with the inherit-on-unset fallback applied
  int n_layer, dim, H, KV, hd, ffn, V;
  int fn_layer, fdim, fH, fKV, fhd, fffn;
  int slow_qk, fast_qk, N, C, sb, se, end_id, scale;
  float base, eps;
  int dtype, kvdtype, max_batch, max_seq;
  size_t esz, kvesz;
  int pc;   // prefill: positions per sequence per step (rows = max_batch * pc)
  int semantic_head;
};

struct Layout {
  size_t kslow, vslow, kfast, vfast, rope_s, rope_f, x_slow, x_fast, qkv, att, ffn, logits, flog, part,
      xn, xn2, gpart, gpart_elems, x_pre, ppos, qbuf,
      counters, st_pos, st_done, st_frames, st_cur, st_plen, st_fidx, st_status, st_ras, total;
  size_t slow_layer_stride, fast_layer_stride;  // elements per layer of a cache
  int max_splits, qkv_ld, att_ld, ffn_ld;
  int rows;     // activation rows the buffers hold: max(max_batch, max_batch * pc)
};

bool resolve(const dualar_config* c, Resolved* r, std::string* err) {
  if (!c) { *err = "config is NULL"; return false; }
  auto inh = [](int v, int s) { return v > 0 ? v : s; };
  r->n_layer = c->n_layer; r->dim = c->dim; r->H = c->n_head; r->KV = c->n_kv_head;
  r->hd = c->head_dim; r->ffn = c->ffn_dim; r->V = c->vocab_size;
  r->fn_layer = c->n_fast_layer;
  r->fdim = inh(c->fast_dim, c->dim); r->fH = inh(c->fast_n_head, c->n_head);
  r->fKV = inh(c->fast_n_kv_head, c->n_kv_head); r->fhd = inh(c->fast_head_dim, c->head_dim);
  r->fffn = inh(c->fast_ffn_dim, c->ffn_dim);
  r->slow_qk = c->slow_qk_norm != 0;
  r->fast_qk = c->fast_qk_norm < 0 ? r->slow_qk : (c->fast_qk_norm != 0);
  r->N = c->num_codebooks; r->C = c->codebook_size;
  r->sb = c->semantic_begin_id; r->se = c->semantic_end_id; r->end_id = c->end_id;
  r->scale = c->scale_codebook_embeddings != 0;
  r->base = c->rope_base; r->eps = c->norm_eps;
  r->dtype = c->weight_dtype; r->max_batch = c->max_batch; r->max_seq = c->max_seq_len;
  r->kvdtype = c->kv_dtype < 0 ? c->weight_dtype : c->kv_dtype;
  char buf[256];
#define REQ(cond, msg)                       \
  if (!(cond)) {                             \
    snprintf(buf, sizeof buf, "%s", msg);    \
    *err = buf;                              \
    return false;                            \
  }
  REQ(c->fast_dim >= 0 && c->fast_n_head >= 0 && c->fast_n_kv_head >= 0 && c->fast_head_dim >= 0 &&
          c->fast_ffn_dim >= 0, "fast_* sizes must be >= 0 (0 = inherit)");
  REQ(c->slow_qk_norm == 0 || c->slow_qk_norm == 1, "slow_qk_norm must be 0 or 1");
  REQ(c->fast_qk_norm >= -1 && c->fast_qk_norm <= 1, "fast_qk_norm must be 1, 0 or -1 (inherit)");
  REQ(c->scale_codebook_embeddings == 0 || c->scale_codebook_embeddings == 1,
      "scale_codebook_embeddings must be 0 or 1");
  REQ(r->dtype == DUALAR_F32 || r->dtype == DUALAR_BF16, "weight_dtype must be DUALAR_F32 or DUALAR_BF16");
  REQ(r->kvdtype == DUALAR_F32 || r->kvdtype == DUALAR_BF16, "kv_dtype must be -1, DUALAR_F32 or DUALAR_BF16");
  r->esz = r->dtype == DUALAR_BF16 ? 2 : 4;
  r->kvesz = r->kvdtype == DUALAR_BF16 ? 2 : 4;
  const int unit = r->dtype == DUALAR_BF16 ? 512 : 256;  // one wave load of a row
  REQ(r->n_layer >= 1 && r->n_layer <= 256, "n_layer out of range [1, 256]");
  REQ(r->fn_layer >= 1 && r->fn_layer <= 256, "n_fast_layer out of range [1, 256]");
  REQ(r->dim > 0 && r->dim % unit == 0 && r->dim <= 12288, "dim must be a multiple of 512 (bf16) / 256 (f32), <= 12288");
  REQ(r->fdim == r->dim, "fast_dim must equal dim (no fast project_in)");
  REQ(r->ffn > 0 && r->ffn % unit == 0 && r->ffn <= 12288, "ffn_dim must be a multiple of 512 (bf16) / 256 (f32), <= 12288");
  REQ(r->fffn > 0 && r->fffn % unit == 0 && r->fffn <= 12288, "fast_ffn_dim must be a multiple of 512 (bf16) / 256 (f32), <= 12288");
  REQ(r->hd == 64 || r->hd == 128, "head_dim must be 64 or 128");
  REQ(r->fhd == 64 || r->fhd == 128, "fast_head_dim must be 64 or 128");
  auto rep_ok = [](int h, int kv) {
    return h > 0 && kv > 0 && h % kv == 0 && (h / kv == 1 || h / kv == 2 || h / kv == 4 || h / kv == 8);
  };
  REQ(rep_ok(r->H, r->KV), "n_head must be 1, 2, 4 or 8 times n_kv_head");
  REQ(rep_ok(r->fH, r->fKV), "fast_n_head must be 1, 2, 4 or 8 times fast_n_kv_head");
  REQ((r->H * r->hd) % unit == 0 && (r->fH * r->fhd) % unit == 0, "n_head*head_dim must be a multiple of the row unit");
  REQ(r->V > 0 && r->V < (1 << 30), "vocab_size out of range");
  REQ(r->N >= 2 && r->N <= 32, "num_codebooks out of range [2, 32]");
  REQ(r->C >= 2 && r->C <= 4096, "codebook_size out of range [2, 4096]");
  REQ(r->sb >= 0 && r->se == r->sb + r->C - 1 && r->se < r->V, "semantic ids must be [sb, sb+C-1] inside the vocabulary");
  REQ(r->end_id >= 0 && r->end_id < r->V && (r->end_id < r->sb || r->end_id > r->se), "end_id must be a vocabulary id outside the semantic range");
  REQ(r->base > 1.0f && isfinite(r->base), "rope_base must be > 1");
  REQ(r->eps >= 0.0f && isfinite(r->eps), "norm_eps must be >= 0");
  REQ(r->max_batch >= 1 && r->max_batch <= 256, "max_batch out of range [1, 256]");
  REQ(c->prefill_chunk >= 0 && c->prefill_chunk <= 4096, "prefill_chunk out of range [0, 4096]");
  r->pc = c->prefill_chunk > 0 ? c->prefill_chunk : std::min(4096, std::max(1, 8192 / r->max_batch));
  REQ(c->semantic_head == 0 || c->semantic_head == 1, "semantic_head must be 0 or 1");
  r->semantic_head = c->semantic_head;
  REQ(r->max_seq >= 2 && r->max_seq <= 65536, "max_seq_len out of range [2, 65536]");
#undef REQ
  return true;
}

Layout layout(const Resolved& r) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += up(bytes); return o; };
  L.max_splits = (r.max_seq + 15) / 16;   // smallest attention chunk is 16 positions
  L.slow_layer_stride = (size_t)r.max_batch * r.KV * r.max_seq * r.hd;
  L.fast_layer_stride = (size_t)r.max_batch * r.fKV * r.N * r.fhd;
  L.kslow = take(L.slow_layer_stride * r.n_layer * r.kvesz);
  L.vslow = take(L.slow_layer_stride * r.n_layer * r.kvesz);
  L.kfast = take(L.fast_layer_stride * r.fn_layer * r.kvesz);
  L.vfast = take(L.fast_layer_stride * r.fn_layer * r.kvesz);
  L.rope_s = take((size_t)r.max_seq * (r.hd / 2) * sizeof(float2));
  L.rope_f = take((size_t)r.N * (r.fhd / 2) * sizeof(float2));
  L.x_slow = take((size_t)r.max_batch * r.dim * 4);
  L.x_fast = take((size_t)r.max_batch * r.dim * 4);
  L.qkv_ld = std::max((r.H + 2 * r.KV) * r.hd, (r.fH + 2 * r.fKV) * r.fhd);
  L.att_ld = std::max(r.H * r.hd, r.fH * r.fhd);
  L.ffn_ld = std::max(r.ffn, r.fffn);
  L.rows = r.max_batch * r.pc;
  L.qkv = take((size_t)L.rows * L.qkv_ld * 4);
  L.att = take((size_t)L.rows * L.att_ld * 4);
  L.ffn = take((size_t)L.rows * L.ffn_ld * 4);
  // prefill chunk: activations, positions, rotated q of every row
  L.x_pre = take((size_t)L.rows * r.dim * 4);
  L.ppos = take((size_t)L.rows * 4);
  // prefill: q rows (fp32); decode: the query planes of the batched
  // attention ([3][max_batch][att_ld] bf16)
  L.qbuf = take(std::max((size_t)L.rows * L.att_ld * 4, (size_t)r.max_batch * L.att_ld * 6));
  L.logits = take((size_t)r.max_batch * r.V * 4);
  L.flog = take((size_t)r.max_batch * r.C * 4);
  const int maxH = std::max(r.H, r.fH), maxhd = std::max(r.hd, r.fhd);
  L.part = take((size_t)r.max_batch * maxH * L.max_splits * (maxhd + 2) * 4);
  L.counters = take((size_t)r.max_batch * std::max(r.KV, r.fKV) * 4);
  // matrix-core GEMM scratch: the activations as three bf16 planes (6 bytes
  // per element) and split-K partials (up to 32 splits)
  L.xn = take((size_t)L.rows * std::max(std::max(r.dim, r.ffn), std::max(r.fffn, L.att_ld)) * 6);
  // planes written by a producer (attention output, SwiGLU output) for the
  // next product, while xn may still be read
  L.xn2 = take((size_t)L.rows * std::max(std::max(r.dim, r.ffn), std::max(r.fffn, L.att_ld)) * 6);
  L.gpart_elems = r.max_batch >= 2 ? (size_t)32 * std::max(r.max_batch, 32) *
                                         std::max(std::max(2 * r.ffn, 2 * r.fffn), std::max(L.qkv_ld, r.dim))
                                   : 0;
  L.gpart = take(L.gpart_elems * 4);
  L.st_pos = take(r.max_batch * 4);
  L.st_done = take(r.max_batch * 4);
  L.st_frames = take(r.max_batch * 4);
  L.st_cur = take((size_t)r.max_batch * (r.N + 1) * 4);
  L.st_plen = take(r.max_batch * 4);
  L.st_fidx = take(4);
  L.st_status = take(4);
  L.st_ras = take((size_t)r.max_batch * DUALAR_RAS_MAX_WINDOW * 4);   // loop-breaker windows
  L.total = off;
  return L;
}

struct Stack {
  int n_layer, dim, H, KV, hd, ffn, qk;
  std::vector<dualar_layer_weights> lw;
  std::vector<dualar_layer_w4> l4;   // 4-bit forms (all NULL without them)
  char* k; char* v;        // cache bases
  size_t layer_stride;     // elements
  int max_pos;
  const float2* rope;
  bool any_w4() const {
    for (const dualar_layer_w4& l : l4)
      for (const void* q : l.q4)
        if (q) return true;
    return false;
  }
};

}  // namespace

struct dualar_ctx {
  Resolved r;
  Layout L;
  dualar_weights w;
  Stack slow, fast;
  char* ws;
  hipStream_t stream;
  int device;
  std::string err;
  // host mirror of the sequence state
  int batch = 0;
  bool ready = false;
  std::vector<int> plen;
  int frames_done = 0;   // decode frames since prefill (same for every sequence)
  std::vector<int> step_pos;  // host mirror of the positions of the current slow step
  // prefill step: activation tiles (GEMM_TILE_BROWS rows) that hold prompt rows
  uint64_t pf_live[2] = {0, 0};
  int pf_masked = 0;
  SeqState st;
  // measurement (dualar_profile_begin/end)
  int prof_cls = -1;
  std::vector<hipEvent_t> ev;
  size_t ev_used = 0;
  long long prof_launches = 0;
  double prof_bytes = 0.0;
  ~dualar_ctx() {
    for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  }
};

namespace {

dualar_status fail(dualar_ctx* c, dualar_status s, const std::string& m) {
  if (c) c->err = m; else g_create_err = m;
  return s;
}

// Bracket one launch of kernel class `cls` with events when it is profiled.
// A launch of class `cls` is profiled when that class is selected; the
// SwiGLU GEMVs are also profiled under DUALAR_K_GEMV_SWIGLU.
bool prof_on(dualar_ctx* c, int cls, bool swiglu = false) {
  return c->prof_cls == cls || (swiglu && c->prof_cls == DUALAR_K_GEMV_SWIGLU);
}
// The start event is recorded on the stream; a launcher of one kernel then
// re-records both events at that kernel's own start and end (launch_timed),
// otherwise prof_post records the stop event after the launches.
hipError_t prof_pre(dualar_ctx* c, int cls, bool swiglu = false) {
  g_launch_ev = LaunchEvents{nullptr, nullptr};   // never left armed by a failed launch
  if (!prof_on(c, cls, swiglu)) return hipSuccess;
  while (c->ev.size() < c->ev_used + 2) {
    hipEvent_t e;
    hipError_t er = hipEventCreate(&e);
    if (er != hipSuccess) return er;
    c->ev.push_back(e);
  }
  g_launch_ev = LaunchEvents{c->ev[c->ev_used], c->ev[c->ev_used + 1]};
  return hipEventRecord(c->ev[c->ev_used], c->stream);
}
hipError_t prof_post(dualar_ctx* c, int cls, double bytes, bool swiglu = false) {
  if (!prof_on(c, cls, swiglu)) return hipSuccess;
  const bool taken = g_launch_ev.start == nullptr;   // recorded by the kernel launch itself
  g_launch_ev = LaunchEvents{nullptr, nullptr};
  hipError_t er = taken ? hipSuccess : hipEventRecord(c->ev[c->ev_used + 1], c->stream);
  c->ev_used += 2;
  c->prof_launches += 1;
  c->prof_bytes += bytes;
  return er;
}

template <typename T>
hipError_t gemv(dualar_ctx* c, const GemvParams& g0) {
  GemvParams g = g0;
  g.xn = (void*)(c->ws + c->L.xn);
  g.part = c->L.gpart_elems ? (float*)(c->ws + c->L.gpart) : nullptr;
  g.part_elems = c->L.gpart_elems;
  g.status = c->st.status;
  g.prep.status = c->st.status;
  const bool sw = g.mode == GEMV_SWIGLU;
  hipError_t e = prof_pre(c, DUALAR_K_GEMV, sw);
  if (e != hipSuccess) return e;
  e = launch_gemv<T>(g, c->stream);
  if (e != hipSuccess) return e;
  const double wbytes = g.q4[0] ? (double)g.n_out * (sw ? 2 : 1) * (g.K / 2 + g.K / 128 * 2)
                               : (double)g.n_out * (sw ? 2 : 1) * g.K * c->r.esz;
  const double act = 4.0 * g.B * ((double)g.K + g.n_out * (g.mode == GEMV_ADD ? 2 : 1));
  return prof_post(c, DUALAR_K_GEMV, wbytes + act, sw);
}

#define HIPCHK(expr)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(c, DUALAR_ERR_HIP, std::string(#expr) + ": " + \
                                                              hipGetErrorString(e_));  \
  } while (0)

// Positions attended by the rows of the current slow step (host mirror).
double attn_positions(dualar_ctx* c, int B) {
  double s = 0;
  for (int b = 0; b < B; ++b) {
    const int p = c->step_pos.empty() ? 0 : c->step_pos[b];
    if (p >= 0) s += p + 1;
  }
  return s;
}

// Prefill steps: only the activation tiles that hold prompt rows go to the
// products' 2-D tile form.
void live_tiles(const dualar_ctx* c, GemvParams& g, int rows_per_seq) {
  if (rows_per_seq <= 0 || !c->pf_masked) return;
  g.live_bt[0] = c->pf_live[0];
  g.live_bt[1] = c->pf_live[1];
  g.bt_masked = 1;
}

// One transformer layer over B activation rows.  Decode: row b is sequence
// b at position pos_dev[b] (or pos_const).  Prefill (rows_per_seq > 0): row r
// is position pos_dev[r] of sequence r / rows_per_seq (-1 = padding).
//
// in_planes: on entry, the previous layer already wrote RMSNorm(x) with this
// layer's attention gain as planes (xn), so the QKV product reads them; on
// exit, whether this layer did the same for layer l + 1 (for the last layer:
// with out_gain, the gain of the norm in front of the head, when given).
template <typename T, typename KT>
dualar_status run_layer(dualar_ctx* c, Stack& S, int l, float* x, int B, const int* pos_dev,
                        int pos_const, int Lmax, bool& in_planes, int rows_per_seq = 0, bool depth_tf = false,
                        const void* out_gain = nullptr) {
  const Resolved& r = c->r;
  const Layout& L = c->L;
  const dualar_layer_weights& w = S.lw[l];
  const dualar_layer_w4& w4 = S.l4[l];      // 4-bit forms (NULL: bf16)
  float* qkv = (float*)(c->ws + L.qkv);
  float* att = (float*)(c->ws + L.att);
  float* ffn = (float*)(c->ws + L.ffn);
  // With 8+ rows and bf16 weights the products run on the matrix cores, which
  // read their input as bf16 planes: the attention and SwiGLU outputs are then
  // written as planes (xn2) and the next product reads them directly.
  uint16_t* planes = (sizeof(T) == 2 && B >= 2) ? (uint16_t*)(c->ws + L.xn2) : nullptr;
  // The residual products (O, W2) split K over workgroups at these sizes; their
  // finish then also writes the next product's normalised input planes (xn).
  void* const xn = c->ws + L.xn;
  int fused = 0;
  bool o_done = false;
  GemvParams g{};
  // q | k | v = W_qkv . RMSNorm(x)
  g.w[0] = w.wq; g.w[1] = w.wk; g.w[2] = w.wv;
  for (int j = 0; j < 3; ++j) { g.q4[j] = w4.q4[j]; g.s4[j] = w4.s4[j]; }
  g.rows[0] = S.H * S.hd; g.rows[1] = S.KV * S.hd; g.rows[2] = S.KV * S.hd; g.n_seg = 3;
  g.K = S.dim; g.n_out = (S.H + 2 * S.KV) * S.hd;
  g.x = x; g.ldx = S.dim; g.gain = w.attention_norm; g.eps = r.eps;
  g.y = qkv; g.ldy = L.qkv_ld; g.B = B; g.mode = GEMV_STORE;
  live_tiles(c, g, rows_per_seq);
  if (planes && in_planes) g.xplanes = xn;
  in_planes = false;
  // batched decode with a bf16 cache: the QKV finish also prepares the
  // attention (QK-norm, RoPE, q terms, k/v append) when it can
  int prepped = 0;
  if (planes && rows_per_seq == 0 && sizeof(KT) == 2) {
    g.prep.rope = S.rope; g.prep.pos = pos_dev; g.prep.pos_const = pos_const;
    g.prep.q_norm = S.qk ? w.q_norm : nullptr; g.prep.k_norm = S.qk ? w.k_norm : nullptr;
    g.prep.H = S.H; g.prep.KV = S.KV; g.prep.hd = S.hd; g.prep.max_pos = S.max_pos;
    g.prep.kcache = S.k + (size_t)l * S.layer_stride * r.kvesz;
    g.prep.vcache = S.v + (size_t)l * S.layer_stride * r.kvesz;
    g.prep.q_planes = (uint16_t*)(c->ws + L.qbuf);
    g.prep_done = &prepped;
  }
  HIPCHK(gemv<T>(c, g));
  if (depth_tf) {
    // teacher-forced fast AR: groups of rows_per_seq rows, causal along depth
    PrefillParams a{};
    a.qkv = qkv; a.ld_qkv = L.qkv_ld; a.C = rows_per_seq; a.rope = S.rope;
    a.q_norm = S.qk ? w.q_norm : nullptr; a.k_norm = S.qk ? w.k_norm : nullptr; a.eps = r.eps;
    a.H = S.H; a.KV = S.KV; a.hd = S.hd;
    a.out = att; a.ld_out = L.att_ld; a.out_planes = planes; a.R = B; a.B = B / rows_per_seq;
    a.status = c->st.status;
    HIPCHK((launch_depth_attn<T, KT>(a, c->stream)));
  } else if (rows_per_seq > 0) {
    // prefill chunk: QK-norm, RoPE, append for every row, then causal attention
    PrefillParams a{};
    a.qkv = qkv; a.ld_qkv = L.qkv_ld;
    a.qbuf = (float*)(c->ws + L.qbuf); a.ld_q = L.att_ld;
    a.kcache = S.k + (size_t)l * S.layer_stride * r.kvesz;
    a.vcache = S.v + (size_t)l * S.layer_stride * r.kvesz;
    a.max_pos = S.max_pos; a.pos = pos_dev; a.C = rows_per_seq; a.rope = S.rope;
    a.q_norm = S.qk ? w.q_norm : nullptr; a.k_norm = S.qk ? w.k_norm : nullptr; a.eps = r.eps;
    a.H = S.H; a.KV = S.KV; a.hd = S.hd;
    a.out = att; a.ld_out = L.att_ld; a.out_planes = planes; a.R = B; a.B = B / rows_per_seq;
    a.status = c->st.status;
    HIPCHK((launch_prefill_attn<T, KT>(a, c->stream)));
  } else if (B == 1 && !pos_dev && sizeof(T) == 2 && sizeof(KT) == 2 && !w4.q4[3] &&
             attn_o_b1_fits(S.H, S.KV, S.hd, S.dim, pos_const + 1)) {
    // fast AR at batch 1: the depth attention runs inside the O product
    AttnOParams a{};
    a.qkv = qkv;
    a.kcache = S.k + (size_t)l * S.layer_stride * r.kvesz;
    a.vcache = S.v + (size_t)l * S.layer_stride * r.kvesz;
    a.max_pos = S.max_pos; a.pos = pos_const; a.rope = S.rope;
    a.q_norm = S.qk ? w.q_norm : nullptr; a.k_norm = S.qk ? w.k_norm : nullptr; a.eps = r.eps;
    a.H = S.H; a.KV = S.KV; a.hd = S.hd;
    a.wo = w.wo; a.x = x; a.dim = S.dim;
    a.status = c->st.status;
    HIPCHK(prof_pre(c, DUALAR_K_GEMV));
    HIPCHK(launch_attn_o_b1(a, c->stream));
    HIPCHK(prof_post(c, DUALAR_K_GEMV, (double)S.dim * S.H * S.hd * r.esz +
                                           (double)(pos_const + 1) * 2.0 * S.KV * S.hd * r.kvesz));
    o_done = true;
  } else {
  // attention over the cache (+QK-norm, RoPE, append)
  AttnParams a{};
  a.qkv = qkv; a.ld_qkv = L.qkv_ld;
  a.kcache = S.k + (size_t)l * S.layer_stride * r.kvesz;
  a.vcache = S.v + (size_t)l * S.layer_stride * r.kvesz;
  a.max_pos = S.max_pos; a.pos = pos_dev; a.pos_const = pos_const; a.rope = S.rope;
  a.q_norm = S.qk ? w.q_norm : nullptr; a.k_norm = S.qk ? w.k_norm : nullptr; a.eps = r.eps;
  a.H = S.H; a.KV = S.KV; a.hd = S.hd;
  a.status = c->st.status;
  // Up to batch 4 with contexts of at most 2,048 positions: the split form
  // with 4 loads per lane (batch 1, 1k context: 12.0 us per layer against 14.7
  // with 2).  Otherwise the balanced flash-decoding form (it = 8): at batch 4
  // and 16k positions the split form needs 256 splits per head and a merge.
  // The fast layers' depth cache (at most 16 positions) takes it = 8 from
  // batch 2 on, which selects the one-wave depth form where it applies.
  a.it = (B <= 4 && Lmax <= 2048 && !(B >= 2 && !pos_dev && Lmax <= 16)) ? 4 : 8;
  // Batch 1, bf16 weights, the S2 head shape: the split form with at most
  // merge_o_b1_max_splits() chunks of 128 or 256 positions, its merge done by
  // the O product (each lane merges the eight values it multiplies).
  int mo_chunk = 0;
  if (B == 1 && pos_dev && sizeof(T) == 2 && !w4.q4[3] && attn_o_b1_fits(S.H, S.KV, S.hd, S.dim, 1)) {
    for (int it : {8, 16}) {   // 128-position chunks, else 256
      const int ch = attn_chunk((int)r.kvesz, S.hd, it);
      if ((Lmax + ch - 1) / ch <= merge_o_b1_max_splits()) { a.it = it; mo_chunk = ch; break; }
    }
  }
  // Batch 1 with a 4-bit O matrix: the same 8-wave split kernel in chunks of
  // 128 positions, then the plain merge writes o for the 4-bit O product.
  const int w4_chunk = (B == 1 && sizeof(T) == 2 && sizeof(KT) == 2 && w4.q4[3])
                           ? attn_chunk((int)r.kvesz, S.hd, 8) : 0;
  a.no_merge = mo_chunk > 0;
  a.lmax = Lmax;
  a.part = (float*)(c->ws + L.part);
  a.counters = (unsigned*)(c->ws + L.counters);
  a.out = att; a.ld_out = L.att_ld; a.out_planes = planes; a.B = B;
  a.q_planes = (uint16_t*)(c->ws + L.qbuf);   // the prefill q buffer is free while decoding
  a.prepped = prepped;
  HIPCHK(prof_pre(c, DUALAR_K_ATTN));
  bool split8 = false;
  if ((mo_chunk || w4_chunk) && sizeof(KT) == 2) {
    // batch 1, bf16 cache: the 8-wave split kernel (same partial layout)
    AttnParams b = a;
    b.chunk = mo_chunk ? mo_chunk : w4_chunk; b.max_splits = (Lmax + b.chunk - 1) / b.chunk;
    split8 = launch_attn_split_b1(b, c->stream);
    if (split8) HIPCHK(hipGetLastError());
    if (split8 && !mo_chunk) HIPCHK(launch_attn_merge(b, c->stream));
  }
  if (!split8) HIPCHK((launch_attn<T, KT>(a, c->stream)));
  if (c->prof_cls == DUALAR_K_ATTN) {
    // cache bytes: every attended position of every row, K and V, plus the append
    double pos_sum = pos_dev ? attn_positions(c, B) : (double)B * (pos_const + 1);
    HIPCHK(prof_post(c, DUALAR_K_ATTN, pos_sum * 2.0 * S.KV * S.hd * r.kvesz +
                                           4.0 * B * ((S.H + 2 * S.KV) * S.hd + S.H * S.hd)));
  }
  if (mo_chunk) {
    // x += Wo . merge(partials)
    MergeOParams mo{};
    mo.part = a.part; mo.chunk = mo_chunk; mo.max_splits = (Lmax + mo_chunk - 1) / mo_chunk;
    mo.att = att; mo.pos = pos_dev; mo.H = S.H; mo.hd = S.hd;
    mo.wo = w.wo; mo.x = x; mo.dim = S.dim;
    mo.status = c->st.status;
    HIPCHK(prof_pre(c, DUALAR_K_GEMV));
    HIPCHK(launch_merge_o_b1(mo, c->stream));
    HIPCHK(prof_post(c, DUALAR_K_GEMV, (double)S.dim * S.H * S.hd * r.esz +
                                           (double)mo.max_splits * S.H * (S.hd + 2) * 4.0));
    o_done = true;
  }
  }
  // x += Wo . o
  if (!o_done) {
  g = GemvParams{};
  g.w[0] = w.wo; g.q4[0] = w4.q4[3]; g.s4[0] = w4.s4[3];
  g.rows[0] = S.dim; g.n_seg = 1; g.K = S.H * S.hd; g.n_out = S.dim;
  g.x = att; g.ldx = L.att_ld; g.y = x; g.ldy = S.dim; g.res = x; g.ldres = S.dim; g.B = B; g.mode = GEMV_ADD;
  live_tiles(c, g, rows_per_seq);
  g.xplanes = planes;
  if (planes) { g.next_gain = w.ffn_norm; g.next_planes = xn; g.next_done = &fused; g.eps = r.eps; }
  HIPCHK(gemv<T>(c, g));
  }
  // h = silu(W1 n) * (W3 n), n = RMSNorm(x)
  g = GemvParams{};
  g.w[0] = w.w1; g.w[1] = w.w3; g.rows[0] = S.ffn; g.rows[1] = S.ffn; g.n_seg = 2;
  g.q4[0] = w4.q4[4]; g.q4[1] = w4.q4[5]; g.s4[0] = w4.s4[4]; g.s4[1] = w4.s4[5];
  g.K = S.dim; g.n_out = S.ffn; g.x = x; g.ldx = S.dim; g.gain = w.ffn_norm; g.eps = r.eps;
  g.y = ffn; g.ldy = L.ffn_ld; g.B = B; g.mode = GEMV_SWIGLU;
  live_tiles(c, g, rows_per_seq);
  g.yplanes = planes;
  if (fused) g.xplanes = xn;
  HIPCHK(gemv<T>(c, g));
  // x += W2 . h
  g = GemvParams{};
  g.w[0] = w.w2; g.q4[0] = w4.q4[6]; g.s4[0] = w4.s4[6];
  g.rows[0] = S.dim; g.n_seg = 1; g.K = S.ffn; g.n_out = S.dim;
  g.x = ffn; g.ldx = L.ffn_ld; g.y = x; g.ldy = S.dim; g.res = x; g.ldres = S.dim; g.B = B; g.mode = GEMV_ADD;
  live_tiles(c, g, rows_per_seq);
  g.xplanes = planes;
  fused = 0;
  if (planes && (l + 1 < S.n_layer || out_gain)) {
    g.next_gain = l + 1 < S.n_layer ? S.lw[l + 1].attention_norm : out_gain;
    g.next_planes = xn; g.next_done = &fused; g.eps = r.eps;
  }
  HIPCHK(gemv<T>(c, g));
  in_planes = fused != 0;
  return DUALAR_OK;
}

// Fast pass 0 through the last fast layer: its attention output, O and FFN
// feed only pass 0's logits, which are never used, so only the K/V rows of
// the QKV product run and k, v (QK-norm, RoPE at position 0) are appended to
// cache slot 0 -- the entries the later passes read.
template <typename T, typename KT>
dualar_status run_layer_kv_only(dualar_ctx* c, Stack& S, int l, float* x, int B, bool in_planes) {
  const Resolved& r = c->r;
  const Layout& L = c->L;
  const dualar_layer_weights& w = S.lw[l];
  const dualar_layer_w4& w4 = S.l4[l];
  float* qkv = (float*)(c->ws + L.qkv);
  GemvParams g{};
  g.w[0] = w.wk; g.w[1] = w.wv;
  g.q4[0] = w4.q4[1]; g.q4[1] = w4.q4[2]; g.s4[0] = w4.s4[1]; g.s4[1] = w4.s4[2];
  g.rows[0] = S.KV * S.hd; g.rows[1] = S.KV * S.hd; g.n_seg = 2;
  g.K = S.dim; g.n_out = 2 * S.KV * S.hd;
  g.x = x; g.ldx = S.dim; g.gain = w.attention_norm; g.eps = r.eps;
  g.y = qkv + (size_t)S.H * S.hd; g.ldy = L.qkv_ld; g.B = B; g.mode = GEMV_STORE;
  if (sizeof(T) == 2 && B >= 2 && in_planes) g.xplanes = c->ws + L.xn;
  HIPCHK(gemv<T>(c, g));
  PrefillParams a{};
  a.qkv = qkv; a.ld_qkv = L.qkv_ld;
  a.kcache = S.k + (size_t)l * S.layer_stride * r.kvesz;
  a.vcache = S.v + (size_t)l * S.layer_stride * r.kvesz;
  a.max_pos = S.max_pos; a.pos = nullptr; a.pos_const = 0; a.C = 1; a.rope = S.rope;
  a.k_norm = S.qk ? w.k_norm : nullptr; a.eps = r.eps;
  a.H = S.H; a.KV = S.KV; a.hd = S.hd; a.R = B; a.B = B;
  a.status = c->st.status;
  HIPCHK((launch_kv_append<T, KT>(a, c->stream)));
  return DUALAR_OK;
}

struct FrameIO {
  const dualar_sampling* s;
  const float* uniforms; int u_fs, u_rs;
  int* codes; long long c_rs; int c_fs;
  const dualar_taps* taps;
  bool fast_only;
};

template <typename T>
SampleParams sample_params(dualar_ctx* c, const FrameIO& io, int B, int slow, int k, float* x_next) {
  const Resolved& r = c->r;
  SampleParams sp{};
  sp.logits = (const float*)(c->ws + (slow ? c->L.logits : c->L.flog));
  sp.ld = slow ? r.V : r.C;
  sp.B = B; sp.slow = slow; sp.sb = r.sb; sp.se = r.se; sp.end_id = r.end_id; sp.C = r.C; sp.N = r.N;
  sp.k = k; sp.greedy = io.s->greedy || !io.uniforms; sp.temperature = io.s->temperature;
  sp.top_p = io.s->top_p; sp.min_frames = io.s->min_frames;
  sp.ras_window = io.fast_only ? 0 : io.s->ras_window;
  sp.ras_temperature = io.s->ras_temperature; sp.ras_top_p = io.s->ras_top_p;
  sp.uniforms = io.uniforms; sp.u_frame_stride = io.u_fs; sp.u_row_stride = io.u_rs;
  sp.codes = io.codes; sp.c_row_stride = io.c_rs; sp.c_frame_stride = io.c_fs;
  sp.c_col = io.fast_only ? k : (slow ? 0 : 1 + k);
  sp.fast_emb = c->w.fast_embeddings; sp.fast_dim = r.dim; sp.x_next = x_next;
  sp.fast_only = io.fast_only;
  sp.st = c->st;
  return sp;
}

template <typename T>
hipError_t sample(dualar_ctx* c, const SampleParams& sp) {
  hipError_t e = prof_pre(c, DUALAR_K_SAMPLE);
  if (e != hipSuccess) return e;
  e = launch_sample<T>(sp, c->stream);
  if (e != hipSuccess) return e;
  const double cand = sp.slow ? sp.C + 1 : sp.C;
  const double nxt = sp.x_next ? (double)sp.fast_dim * (4 + c->r.esz) : 0.0;
  return prof_post(c, DUALAR_K_SAMPLE, sp.B * (cand * 4 + nxt));
}

// Everything after the slow pass: head, slow sample, N fast passes.  With
// fast_only, x_slow/x_fast/q0 were set by fast_begin and there is no slow head.
template <typename T, typename KT>
// head_planes: the last slow layer already wrote RMSNorm(x_slow) with the
// final norm's gain as planes (xn) for the tied head.
dualar_status frame_tail(dualar_ctx* c, int B, const FrameIO& io, bool head_planes = false) {
  const Resolved& r = c->r;
  const Layout& L = c->L;
  float* xs = (float*)(c->ws + L.x_slow);
  float* xf = (float*)(c->ws + L.x_fast);
  if (!io.fast_only) {
    MarkerRange mr("dualar.head");
    if (io.taps && io.taps->slow_hidden)
      HIPCHK(hipMemcpyAsync(io.taps->slow_hidden, xs, (size_t)B * r.dim * 4, hipMemcpyDeviceToDevice, c->stream));
    // The tied head over the whole vocabulary, or (semantic_head, unless the
    // caller asks for the full logits) over the only rows the biased sample
    // can pick: the C semantic ids and the end id, in id order.
    const bool restricted = r.semantic_head && !(io.taps && io.taps->slow_logits);
    GemvParams g{};
    if (restricted) {
      const char* emb = (const char*)c->w.tok_embedding;
      const void* sem = emb + (size_t)r.sb * r.dim * r.esz;
      const void* end = emb + (size_t)r.end_id * r.dim * r.esz;
      const bool end_first = r.end_id < r.sb;
      g.w[0] = end_first ? end : sem; g.rows[0] = end_first ? 1 : r.C;
      g.w[1] = end_first ? sem : end; g.rows[1] = end_first ? r.C : 1;
      g.n_seg = 2; g.n_out = r.C + 1;
    } else {
      g.w[0] = c->w.tok_embedding; g.rows[0] = r.V; g.n_seg = 1; g.n_out = r.V;
    }
    g.K = r.dim;
    g.x = xs; g.ldx = r.dim; g.gain = c->w.norm; g.eps = r.eps;
    g.y = (float*)(c->ws + L.logits); g.ldy = g.n_out; g.B = B; g.mode = GEMV_STORE;
    if (head_planes) g.xplanes = c->ws + L.xn;
    HIPCHK(gemv<T>(c, g));
    if (io.taps && io.taps->slow_logits)
      HIPCHK(hipMemcpyAsync(io.taps->slow_logits, c->ws + L.logits, (size_t)B * r.V * 4, hipMemcpyDeviceToDevice,
                            c->stream));
    SampleParams sp = sample_params<T>(c, io, B, 1, 0, xf);
    if (restricted) { sp.restricted = 1; sp.ld = r.C + 1; }
    HIPCHK(sample<T>(c, sp));
  }
  MarkerRange mr("dualar.fast");
  // fast pass 0: the slow hidden state at depth position 0
  bool pl = false;
  for (int l = 0; l + 1 < r.fn_layer; ++l) {
    dualar_status st = run_layer<T, KT>(c, c->fast, l, xs, B, nullptr, 0, 1, pl);
    if (st) return st;
  }
  {
    dualar_status st = run_layer_kv_only<T, KT>(c, c->fast, r.fn_layer - 1, xs, B, pl);
    if (st) return st;
  }
  for (int k = 1; k < r.N; ++k) {
    pl = false;
    for (int l = 0; l < r.fn_layer; ++l) {
      // the last layer also writes the fast head's normalised input planes
      dualar_status st = run_layer<T, KT>(c, c->fast, l, xf, B, nullptr, k, k + 1, pl, 0, false,
                                          l + 1 == r.fn_layer ? c->w.fast_norm : nullptr);
      if (st) return st;
    }
    GemvParams g{};
    g.w[0] = c->w.fast_output; g.rows[0] = r.C; g.n_seg = 1; g.K = r.dim; g.n_out = r.C;
    g.x = xf; g.ldx = r.dim; g.gain = c->w.fast_norm; g.eps = r.eps;
    g.y = (float*)(c->ws + L.flog); g.ldy = r.C; g.B = B; g.mode = GEMV_STORE;
    if (pl) g.xplanes = c->ws + L.xn;
    HIPCHK(gemv<T>(c, g));
    if (io.taps && io.taps->fast_logits)
      HIPCHK(hipMemcpy2DAsync(io.taps->fast_logits + (size_t)(k - 1) * r.C, (size_t)(r.N - 1) * r.C * 4,
                              c->ws + L.flog, (size_t)r.C * 4, (size_t)r.C * 4, B, hipMemcpyDeviceToDevice,
                              c->stream));
    HIPCHK(sample<T>(c, sample_params<T>(c, io, B, 0, k, k < r.N - 1 ? xf : nullptr)));
  }
  HIPCHK(launch_frame_end(c->st, B, io.fast_only ? 0 : 1, c->stream));
  return DUALAR_OK;
}

// Fused embedding of the slow input.  Decode: one row per sequence into
// x_slow.  Prefill: rows_per_seq rows per sequence (positions step + i -
// (t_max - plen[b])) into x_pre, with their positions in ppos.
template <typename T>
dualar_status embed(dualar_ctx* c, int B, const int* tokens, int t_max, int step, int prefill,
                    int rows_per_seq = 1) {
  const Resolved& r = c->r;
  EmbedParams e{};
  e.tokens = tokens; e.t_max = t_max; e.step = step; e.prefill = prefill;
  e.rows_per_seq = rows_per_seq;
  e.pos_out = prefill ? (int*)(c->ws + c->L.ppos) : nullptr;
  e.tok_emb = c->w.tok_embedding; e.cb_emb = c->w.codebook_embedding;
  e.dim = r.dim; e.V = r.V; e.N = r.N; e.C = r.C; e.sb = r.sb; e.se = r.se; e.scale = r.scale;
  e.x = (float*)(c->ws + (prefill ? c->L.x_pre : c->L.x_slow)); e.B = B; e.st = c->st;
  HIPCHK(prof_pre(c, DUALAR_K_EMBED));
  HIPCHK(launch_embed<T>(e, c->stream));
  HIPCHK(prof_post(c, DUALAR_K_EMBED, (double)B * rows_per_seq * r.dim * ((r.N + 1) * r.esz + 4)));
  return DUALAR_OK;
}

// Prefill: the prompts are right-aligned (sequence b's position t is global
// step t + t_max - plen[b]) and walked in steps of pc positions, every
// sequence's pc rows at once, so every prompt ends in the last step.  Its
// last row per sequence then feeds frame 0.
// Teacher-forced fast AR over n (hidden state, codes) pairs: n*N rows through
// the fast layers at once (causal along depth inside each pair), then
// fast_norm and the fast head for every row.
template <typename T, typename KT>
dualar_status do_fast_tf(dualar_ctx* c, int n, const float* hidden, const int32_t* codes, float* logits) {
  const Resolved& r = c->r;
  const int M = n * r.N;
  float* x = (float*)(c->ws + c->L.x_pre);
  TfParams e{};
  e.hidden = hidden; e.codes = codes; e.fast_emb = c->w.fast_embeddings; e.x = x;
  e.n = n; e.N = r.N; e.C = r.C; e.dim = r.dim; e.status = c->st.status;
  HIPCHK(launch_tf_embed<T>(e, c->stream));
  bool pl = false;
  for (int l = 0; l < r.fn_layer; ++l) {
    dualar_status st = run_layer<T, KT>(c, c->fast, l, x, M, nullptr, 0, r.N, pl, r.N, true);
    if (st) return st;
  }
  GemvParams g{};
  g.w[0] = c->w.fast_output; g.rows[0] = r.C; g.n_seg = 1; g.K = r.dim; g.n_out = r.C;
  g.x = x; g.ldx = r.dim; g.gain = c->w.fast_norm; g.eps = r.eps;
  g.y = logits; g.ldy = r.C; g.B = M; g.mode = GEMV_STORE;
  HIPCHK(gemv<T>(c, g));
  return DUALAR_OK;
}

template <typename T, typename KT>
dualar_status do_prefill(dualar_ctx* c, int B, const int* tokens, int t_max, const FrameIO& io) {
  const Resolved& r = c->r;
  HIPCHK(launch_prefill_begin(c->st, c->plen.data(), B, r.N, c->stream));
  int C = std::min(r.pc, t_max);
  // 4-bit products over several rows run only on the 2-D tiles: a short
  // prompt is then prefilled in one step of GEMM_TILE_MIN_ROWS rows (left
  // padding; create guarantees prefill_chunk 1 or at least that many)
  if (C > 1 && C < GEMM_TILE_MIN_ROWS && c->slow.any_w4()) C = GEMM_TILE_MIN_ROWS;
  const int n_steps = (t_max + C - 1) / C;
  float* xp = (float*)(c->ws + c->L.x_pre);
  const int* ppos = (const int*)(c->ws + c->L.ppos);
  c->step_pos.assign(B, -1);
  for (int k = 0; k < n_steps; ++k) {
    const int s0 = t_max - (n_steps - k) * C;     // global step of row i = 0
    for (int b = 0; b < B; ++b) c->step_pos[b] = s0 + C - 1 - (t_max - c->plen[b]);
    // row b*C + i is position s0 + i - (t_max - plen[b]), a prompt row when >= 0
    const int nbt = (B * C + GEMM_TILE_BROWS - 1) / GEMM_TILE_BROWS;
    c->pf_masked = nbt <= 128;
    c->pf_live[0] = c->pf_live[1] = 0;
    if (c->pf_masked) {
      for (int b = 0; b < B; ++b) {
        const int first = std::max(0, (t_max - c->plen[b]) - s0);
        if (first >= C) continue;
        for (int j = (b * C + first) / GEMM_TILE_BROWS; j <= (b * C + C - 1) / GEMM_TILE_BROWS; ++j)
          c->pf_live[j >> 6] |= 1ull << (j & 63);
      }
    }
    dualar_status st = embed<T>(c, B, tokens, t_max, s0, 1, C);
    if (st) return st;
    bool pl = false;
    for (int l = 0; l < r.n_layer; ++l) {
      st = run_layer<T, KT>(c, c->slow, l, xp, B * C, ppos, 0, s0 + C, pl, C);
      if (st) return st;
    }
  }
  c->pf_masked = 0;
  // the last row of every sequence is its position plen - 1
  HIPCHK(hipMemcpy2DAsync(c->ws + c->L.x_slow, (size_t)r.dim * 4, xp + (size_t)(C - 1) * r.dim, (size_t)C * r.dim * 4,
                          (size_t)r.dim * 4, B, hipMemcpyDeviceToDevice, c->stream));
  return frame_tail<T, KT>(c, B, io);
}

template <typename T, typename KT>
dualar_status do_decode(dualar_ctx* c, int n_frames, const FrameIO& io) {
  const int B = c->batch;
  HIPCHK(launch_frame_reset(c->st, c->stream));
  int maxp = 0;
  for (int b = 0; b < B; ++b) maxp = std::max(maxp, c->plen[b]);
  float* xs = (float*)(c->ws + c->L.x_slow);
  for (int f = 0; f < n_frames; ++f) {
    MarkerRange mr("dualar.frame");
    dualar_status st = embed<T>(c, B, nullptr, 0, 0, 0);
    if (st) return st;
    const bool last = f == n_frames - 1;
    if (last && io.taps && io.taps->fused_x)
      HIPCHK(hipMemcpyAsync(io.taps->fused_x, xs, (size_t)B * c->r.dim * 4, hipMemcpyDeviceToDevice, c->stream));
    const int Lmax = maxp + c->frames_done + f + 1;
    c->step_pos.resize(B);
    for (int b = 0; b < B; ++b) c->step_pos[b] = c->plen[b] + c->frames_done + f;
    bool pl = false;   // after the loop: the tied head's input planes are written
    {
      MarkerRange ms("dualar.slow");
      for (int l = 0; l < c->r.n_layer; ++l) {
        st = run_layer<T, KT>(c, c->slow, l, xs, B, c->st.pos, 0, Lmax, pl, 0, false,
                              l + 1 == c->r.n_layer ? c->w.norm : nullptr);
        if (st) return st;
      }
    }
    FrameIO fio = io;
    if (!last) fio.taps = nullptr;
    st = frame_tail<T, KT>(c, B, fio, pl);
    if (st) return st;
  }
  return DUALAR_OK;
}

template <typename T, typename KT>
dualar_status do_fast(dualar_ctx* c, int B, int n_frames, const float* hidden, const int* q0, const FrameIO& io) {
  HIPCHK(launch_frame_reset(c->st, c->stream));
  for (int f = 0; f < n_frames; ++f) {
    MarkerRange mr("dualar.frame");
    FastBeginParams fb{};
    fb.hidden = hidden; fb.q0 = q0; fb.fast_emb = c->w.fast_embeddings; fb.dim = c->r.dim; fb.C = c->r.C;
    fb.N = c->r.N; fb.x_slow = (float*)(c->ws + c->L.x_slow); fb.x_fast = (float*)(c->ws + c->L.x_fast);
    fb.codes = io.codes; fb.c_row_stride = io.c_rs; fb.c_frame_stride = io.c_fs; fb.B = B; fb.st = c->st;
    HIPCHK(launch_fast_begin<T>(fb, c->stream));
    FrameIO fio = io;
    if (f != n_frames - 1) fio.taps = nullptr;
    dualar_status st = frame_tail<T, KT>(c, B, fio);
    if (st) return st;
  }
  return DUALAR_OK;
}

// Call f(weight type, cache type) with the context's element types.
template <typename F>
dualar_status dispatch(dualar_ctx* c, F&& f) {
  const bool wb = c->r.dtype == DUALAR_BF16, kb = c->r.kvdtype == DUALAR_BF16;
  if (wb && kb) return f(bf16_t{}, bf16_t{});
  if (wb) return f(bf16_t{}, float{});
  if (kb) return f(float{}, bf16_t{});
  return f(float{}, float{});
}

static_assert(RAS_HIST_STRIDE == DUALAR_RAS_MAX_WINDOW, "loop-breaker window stride");
static_assert(GEMM_TILE_MIN_ROWS == 256 && GEMV_W4_MAX_ROWS == 8, "the 4-bit error messages name 256 and 8 rows");

dualar_status check_sampling(dualar_ctx* c, const dualar_sampling* s, const float* uniforms) {
  if (!s) return fail(c, DUALAR_ERR_INVALID_ARG, "sampling is NULL");
  if (!s->greedy) {
    if (!uniforms) return fail(c, DUALAR_ERR_INVALID_ARG, "top-p sampling needs uniforms");
    if (!(s->temperature > 0.0f) || !isfinite(s->temperature))
      return fail(c, DUALAR_ERR_INVALID_ARG, "temperature must be > 0");
    if (!(s->top_p > 0.0f && s->top_p <= 1.0f)) return fail(c, DUALAR_ERR_INVALID_ARG, "top_p must be in (0, 1]");
  }
  if (s->min_frames < 0) return fail(c, DUALAR_ERR_INVALID_ARG, "min_frames must be >= 0");
  if (s->ras_window < 0 || s->ras_window > DUALAR_RAS_MAX_WINDOW)
    return fail(c, DUALAR_ERR_INVALID_ARG, "ras_window must be in [0, DUALAR_RAS_MAX_WINDOW]");
  if (s->ras_window > 0) {
    if (!uniforms) return fail(c, DUALAR_ERR_INVALID_ARG, "the loop breaker needs uniforms (slot N)");
    if (!(s->ras_temperature > 0.0f) || !isfinite(s->ras_temperature))
      return fail(c, DUALAR_ERR_INVALID_ARG, "ras_temperature must be > 0");
    if (!(s->ras_top_p > 0.0f && s->ras_top_p <= 1.0f))
      return fail(c, DUALAR_ERR_INVALID_ARG, "ras_top_p must be in (0, 1]");
  }
  return DUALAR_OK;
}

dualar_status create_ctx(const dualar_config* cfg, const dualar_weights* w, void* workspace,
                         size_t workspace_bytes, void* hip_stream, dualar_ctx_t** out);

}  // namespace

// The workspace of dualar_create_static: a static device array that every GPU
// the library runs on holds until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: only the address returned
// by hipGetSymbolAddress for the current device may reach a kernel or a
// copy.
static __device__ __align__(256) char scratch[DUALAR_STATIC_WORKSPACE_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];   // device address of `scratch` per device (nullptr: not looked up yet)

// Device address of `scratch` on the current device, looked up once per
// device (with that device current).
dualar_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= MAX_DEVICES)
    return fail(nullptr, DUALAR_ERR_NO_DEVICE, "no current HIP device for the static workspace");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(nullptr, DUALAR_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DUALAR_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

size_t dualar_workspace_bytes(const dualar_config* cfg) {
  Resolved r;
  std::string err;
  if (!resolve(cfg, &r, &err)) return 0;
  return layout(r).total;
}

dualar_status dualar_create(const dualar_config* cfg, const dualar_weights* w, void* workspace,
                            size_t workspace_bytes, void* hip_stream, dualar_ctx_t** out) {
  return create_ctx(cfg, w, workspace, workspace_bytes, hip_stream, out);
}

dualar_status dualar_create_static(const dualar_config* cfg, const dualar_weights* w, void* hip_stream,
                                   dualar_ctx_t** out) {
  Resolved r;
  std::string err;
  if (!out) return fail(nullptr, DUALAR_ERR_INVALID_ARG, "out is NULL");
  if (!resolve(cfg, &r, &err)) return fail(nullptr, DUALAR_ERR_INVALID_ARG, err);
  const size_t need = layout(r).total;
  if (need > sizeof(scratch)) {
    char buf[160];
    snprintf(buf, sizeof buf, "the config needs a %zu-byte workspace; the static workspace holds %zu bytes", need,
             sizeof(scratch));
    return fail(nullptr, DUALAR_ERR_WORKSPACE, buf);
  }
  void* ws = nullptr;
  if (dualar_status st = scratch_address(&ws)) return st;
  return create_ctx(cfg, w, ws, sizeof(scratch), hip_stream, out);
}

}  // extern "C"

namespace {

dualar_status create_ctx(const dualar_config* cfg, const dualar_weights* w, void* workspace,
                         size_t workspace_bytes, void* hip_stream, dualar_ctx_t** out) {
  dualar_ctx* c = nullptr;
  Resolved r;
  std::string err;
  if (!out) return fail(c, DUALAR_ERR_INVALID_ARG, "out is NULL");
  if (!resolve(cfg, &r, &err)) return fail(c, DUALAR_ERR_INVALID_ARG, err);
  if (!w) return fail(c, DUALAR_ERR_INVALID_ARG, "weights is NULL");
  // every tensor is read with 16-byte vector loads
  auto P = [](const void* q) { return q && ((uintptr_t)q % 16) == 0; };
  if (!w->layers || !w->fast_layers) return fail(c, DUALAR_ERR_INVALID_ARG, "a layer array is NULL");
  if (!P(w->tok_embedding) || !P(w->codebook_embedding) || !P(w->norm) || !P(w->fast_embeddings) ||
      !P(w->fast_norm) || !P(w->fast_output))
    return fail(c, DUALAR_ERR_INVALID_ARG, "a weight pointer is NULL or not 16-byte aligned");
  // a matrix may be absent from dualar_layer_weights when its 4-bit form is given
  auto has4 = [&](const dualar_layer_w4* a, int i, int j) { return a && a[i].q4[j]; };
  auto layer_ok = [&](const dualar_layer_weights& l, int qk, const dualar_layer_w4* a, int i) {
    const void* m[7] = {l.wq, l.wk, l.wv, l.wo, l.w1, l.w3, l.w2};
    for (int j = 0; j < 7; ++j)
      if (!P(m[j]) && !has4(a, i, j)) return false;
    return P(l.attention_norm) && P(l.ffn_norm) && (!qk || (P(l.q_norm) && P(l.k_norm)));
  };
  for (int i = 0; i < r.n_layer; ++i)
    if (!layer_ok(w->layers[i], r.slow_qk, w->layers_w4, i))
      return fail(c, DUALAR_ERR_INVALID_ARG, "a slow layer weight is NULL or not 16-byte aligned");
  for (int i = 0; i < r.fn_layer; ++i)
    if (!layer_ok(w->fast_layers[i], r.fast_qk, w->fast_layers_w4, i))
      return fail(c, DUALAR_ERR_INVALID_ARG, "a fast layer weight is NULL or not 16-byte aligned");
  // 4-bit matrices: batches of 1 to GEMV_W4_MAX_ROWS (the 4-bit GEMVs);
  // prefill steps of one position per sequence (the same GEMVs) or of
  // GEMM_TILE_MIN_ROWS+ positions (the 2-D tiles)
  auto w4_check = [&](const dualar_layer_w4* a, int n, int dim, int H, int KV, int hd, int ffn) -> const char* {
    if (!a) return nullptr;
    const int in[7] = {dim, dim, dim, H * hd, dim, dim, ffn};
    for (int i = 0; i < n; ++i) {
      for (int j = 0; j < 7; ++j) {
        if (!a[i].q4[j]) continue;
        if (!P(a[i].q4[j]) || !P(a[i].s4[j])) return "a 4-bit matrix or its scales is NULL or not 16-byte aligned";
        if (in[j] % 512 || in[j] > 10240) return "a 4-bit matrix's rows must be a multiple of 512 inputs, at most 10,240";
      }
      if ((!a[i].q4[0]) != (!a[i].q4[1]) || (!a[i].q4[0]) != (!a[i].q4[2])) return "wq, wk, wv must be all 4-bit or all bf16";
      if ((!a[i].q4[4]) != (!a[i].q4[5])) return "w1 and w3 must both be 4-bit or both bf16";
    }
    return nullptr;
  };
  if (w->layers_w4 || w->fast_layers_w4) {
    if (r.esz != 2 || r.max_batch > GEMV_W4_MAX_ROWS || (r.pc != 1 && r.pc < GEMM_TILE_MIN_ROWS))
      return fail(c, DUALAR_ERR_INVALID_ARG,
                  "4-bit matrices need bf16 weights, max_batch at most 8 and prefill_chunk 1 or at least 256");
    const char* e = w4_check(w->layers_w4, r.n_layer, r.dim, r.H, r.KV, r.hd, r.ffn);
    if (!e) e = w4_check(w->fast_layers_w4, r.fn_layer, r.dim, r.fH, r.fKV, r.fhd, r.fffn);
    if (e) return fail(c, DUALAR_ERR_INVALID_ARG, e);
  }
  const Layout L = layout(r);
  if (!workspace) return fail(c, DUALAR_ERR_INVALID_ARG, "workspace is NULL");
  if (((uintptr_t)workspace) % ALIGN) return fail(c, DUALAR_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (workspace_bytes < L.total) return fail(c, DUALAR_ERR_WORKSPACE, "workspace smaller than dualar_workspace_bytes()");
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return fail(c, DUALAR_ERR_NO_DEVICE, "no HIP device");

  c = new dualar_ctx();
  c->r = r; c->L = L; c->w = *w; c->ws = (char*)workspace; c->stream = (hipStream_t)hip_stream;
  if (hipGetDevice(&c->device) != hipSuccess) { delete c; return fail(nullptr, DUALAR_ERR_HIP, "hipGetDevice failed"); }
  auto mk = [&](Stack& S, const dualar_layer_weights* lw, const dualar_layer_w4* l4, int n, int dim, int H, int KV,
                int hd, int ffn, int qk, size_t k, size_t v, size_t stride, int max_pos, size_t rope) {
    S.n_layer = n; S.dim = dim; S.H = H; S.KV = KV; S.hd = hd; S.ffn = ffn; S.qk = qk;
    S.lw.assign(lw, lw + n);
    if (l4) S.l4.assign(l4, l4 + n);
    else S.l4.assign(n, dualar_layer_w4{});
    S.k = c->ws + k; S.v = c->ws + v; S.layer_stride = stride; S.max_pos = max_pos;
    S.rope = (const float2*)(c->ws + rope);
  };
  mk(c->slow, w->layers, w->layers_w4, r.n_layer, r.dim, r.H, r.KV, r.hd, r.ffn, r.slow_qk, L.kslow, L.vslow,
     L.slow_layer_stride, r.max_seq, L.rope_s);
  mk(c->fast, w->fast_layers, w->fast_layers_w4, r.fn_layer, r.dim, r.fH, r.fKV, r.fhd, r.fffn, r.fast_qk, L.kfast,
     L.vfast, L.fast_layer_stride, r.N, L.rope_f);
  c->w.layers = c->slow.lw.data();
  c->w.fast_layers = c->fast.lw.data();
  c->w.layers_w4 = nullptr;          // kept per stack (S.l4)
  c->w.fast_layers_w4 = nullptr;
  c->st.pos = (int*)(c->ws + L.st_pos); c->st.done = (int*)(c->ws + L.st_done);
  c->st.frames = (int*)(c->ws + L.st_frames); c->st.cur = (int*)(c->ws + L.st_cur);
  c->st.plen = (int*)(c->ws + L.st_plen); c->st.frame_idx = (int*)(c->ws + L.st_fidx);
  c->st.status = (int*)(c->ws + L.st_status);
  c->st.ras_hist = (int*)(c->ws + L.st_ras);

  // RoPE tables: theta_i = base^(-2i/hd), angle p*theta_i in double, cos/sin
  // rounded to bf16 (the bf16 table of the pages).  Stored as (cos, sin) fp32.
  auto table = [&](int n_pos, int hd) {
    std::vector<float2> t((size_t)n_pos * (hd / 2));
    for (int p = 0; p < n_pos; ++p)
      for (int i = 0; i < hd / 2; ++i) {
        const double theta = 1.0 / pow((double)r.base, 2.0 * i / hd);
        const double a = (double)p * theta;
        auto bf = [](double x) {  // nearest bf16, ties to even
          int e;
          const double m = frexp(x, &e);
          return ldexp(nearbyint(m * 256.0), e - 8);
        };
        t[(size_t)p * (hd / 2) + i] = make_float2((float)bf(cos(a)), (float)bf(sin(a)));
      }
    return t;
  };
  std::vector<float2> ts = table(r.max_seq, r.hd), tf = table(r.N, r.fhd);
  hipError_t e1 = hipMemsetAsync(c->ws + L.counters, 0, L.total - L.counters, c->stream);
  hipError_t e2 = hipMemcpyAsync(c->ws + L.rope_s, ts.data(), ts.size() * sizeof(float2), hipMemcpyHostToDevice, c->stream);
  hipError_t e3 = hipMemcpyAsync(c->ws + L.rope_f, tf.data(), tf.size() * sizeof(float2), hipMemcpyHostToDevice, c->stream);
  hipError_t e4 = hipStreamSynchronize(c->stream);   // host tables go out of scope
  if (e1 || e2 || e3 || e4) {
    delete c;
    return fail(nullptr, DUALAR_ERR_HIP, "workspace initialisation failed");
  }
  *out = c;
  return DUALAR_OK;
}

}  // namespace

extern "C" {

dualar_status dualar_prefill(dualar_ctx_t* c, int32_t batch, const int32_t* tokens, int32_t t_max,
                             const int32_t* prompt_len, const dualar_sampling* s, const float* uniforms,
                             int32_t* frame0, const dualar_taps* taps) {
  if (!c) return fail(c, DUALAR_ERR_INVALID_ARG, "ctx is NULL");
  if (batch < 1 || batch > c->r.max_batch) return fail(c, DUALAR_ERR_INVALID_ARG, "batch out of range [1, max_batch]");
  if (!tokens || !prompt_len || !frame0) return fail(c, DUALAR_ERR_INVALID_ARG, "tokens/prompt_len/frame0 is NULL");
  if (t_max < 1) return fail(c, DUALAR_ERR_INVALID_ARG, "t_max must be >= 1");
  for (int b = 0; b < batch; ++b) {
    if (prompt_len[b] < 1 || prompt_len[b] > t_max) return fail(c, DUALAR_ERR_INVALID_ARG, "prompt_len out of [1, t_max]");
    if (prompt_len[b] >= c->r.max_seq) return fail(c, DUALAR_ERR_CONTEXT_FULL, "prompt does not fit max_seq_len");
  }
  if (dualar_status st = check_sampling(c, s, uniforms)) return st;
  c->plen.assign(prompt_len, prompt_len + batch);
  c->batch = batch;
  c->frames_done = 0;
  c->ready = false;
  const int urs = c->r.N + (s->ras_window > 0 ? 1 : 0);   // draws per sequence (slot N: the loop breaker's)
  FrameIO io{s, uniforms, 0, urs, frame0, c->r.N + 1, 0, taps, false};
  MarkerRange mr("dualar.prefill");
  dualar_status st = dispatch(c, [&](auto wt, auto kt) {
    return do_prefill<decltype(wt), decltype(kt)>(c, batch, tokens, t_max, io);
  });
  if (st == DUALAR_OK) c->ready = true;
  return st;
}

dualar_status dualar_decode_frames(dualar_ctx_t* c, int32_t n_frames, const dualar_sampling* s,
                                   const float* uniforms, int32_t* codes, int32_t* n_emitted,
                                   const dualar_taps* taps) {
  if (!c) return fail(c, DUALAR_ERR_INVALID_ARG, "ctx is NULL");
  if (!c->ready) return fail(c, DUALAR_ERR_STATE, "decode_frames before a successful prefill");
  if (n_frames < 1) return fail(c, DUALAR_ERR_INVALID_ARG, "n_frames must be >= 1");
  if (!codes) return fail(c, DUALAR_ERR_INVALID_ARG, "codes is NULL");
  if (dualar_status st = check_sampling(c, s, uniforms)) return st;
  for (int b = 0; b < c->batch; ++b)
    if ((long long)c->plen[b] + c->frames_done + n_frames > c->r.max_seq)
      return fail(c, DUALAR_ERR_CONTEXT_FULL, "decode would pass max_seq_len");
  const int N = c->r.N;
  const int urs = N + (s->ras_window > 0 ? 1 : 0);   // draws per sequence (slot N: the loop breaker's)
  FrameIO io{s, uniforms, c->batch * urs, urs, codes, (long long)n_frames * (N + 1), N + 1, taps, false};
  dualar_status st = dispatch(c, [&](auto wt, auto kt) {
    return do_decode<decltype(wt), decltype(kt)>(c, n_frames, io);
  });
  if (st) return st;
  c->frames_done += n_frames;
  if (n_emitted) HIPCHK(hipMemcpyAsync(n_emitted, c->st.frames, c->batch * 4, hipMemcpyDeviceToDevice, c->stream));
  return DUALAR_OK;
}

dualar_status dualar_fast_frames(dualar_ctx_t* c, int32_t batch, int32_t n_frames, const float* hidden,
                                 const int32_t* q0, const dualar_sampling* s, const float* uniforms,
                                 int32_t* codes, const dualar_taps* taps) {
  if (!c) return fail(c, DUALAR_ERR_INVALID_ARG, "ctx is NULL");
  if (batch < 1 || batch > c->r.max_batch) return fail(c, DUALAR_ERR_INVALID_ARG, "batch out of range [1, max_batch]");
  if (n_frames < 1) return fail(c, DUALAR_ERR_INVALID_ARG, "n_frames must be >= 1");
  if (!hidden || !q0 || !codes) return fail(c, DUALAR_ERR_INVALID_ARG, "hidden/q0/codes is NULL");
  if (dualar_status st = check_sampling(c, s, uniforms)) return st;
  const int N = c->r.N;
  // the slow-AR sequence state is not touched by a fast-only call, except
  // that the per-sequence done flags are used as scratch: a later decode
  // needs a fresh prefill.
  c->ready = false;
  FrameIO io{s, uniforms, batch * N, N, codes, (long long)n_frames * N, N, taps, true};
  return dispatch(c, [&](auto wt, auto kt) {
    return do_fast<decltype(wt), decltype(kt)>(c, batch, n_frames, hidden, q0, io);
  });
}

dualar_status dualar_fast_teacher_forced(dualar_ctx_t* c, int32_t n, const float* hidden, const int32_t* codes,
                                        float* logits) {
  if (!c) return fail(c, DUALAR_ERR_INVALID_ARG, "ctx is NULL");
  if (!hidden || !codes || !logits) return fail(c, DUALAR_ERR_INVALID_ARG, "hidden/codes/logits is NULL");
  const int N = c->r.N;
  if (n < 1 || (long long)n * N > c->L.rows)
    return fail(c, DUALAR_ERR_INVALID_ARG, "n out of range [1, max_batch * prefill_chunk / num_codebooks]");
  if (N > 11 || c->fast.hd > 128 || c->fast.hd % 4 || c->fast.H / c->fast.KV > 8 ||
      (c->fast.H / c->fast.KV) & (c->fast.H / c->fast.KV - 1))
    return fail(c, DUALAR_ERR_INVALID_ARG, "teacher-forced form needs N <= 11, fast head_dim <= 128 (a multiple "
                                           "of 4), 1, 2, 4 or 8 query heads per KV head");
  if (c->fast.any_w4() && (long long)n * N > GEMV_W4_MAX_ROWS && (long long)n * N < GEMM_TILE_MIN_ROWS)
    return fail(c, DUALAR_ERR_INVALID_ARG, "with 4-bit fast layers the teacher-forced form needs n * num_codebooks "
                                           "<= 8 or >= 256 rows");
  // the activation buffers are scratch between calls: the decode state is untouched
  MarkerRange mr("dualar.fast_tf");
  return dispatch(c, [&](auto wt, auto kt) {
    return do_fast_tf<decltype(wt), decltype(kt)>(c, n, hidden, codes, logits);
  });
}

dualar_status dualar_sync(dualar_ctx_t* c, int32_t* device_status) {
  if (!c) return fail(c, DUALAR_ERR_INVALID_ARG, "ctx is NULL");
  HIPCHK(hipStreamSynchronize(c->stream));
  int st = 0;
  HIPCHK(hipMemcpy(&st, c->st.status, 4, hipMemcpyDeviceToHost));
  if (device_status) *device_status = st;
  if (st) {
    HIPCHK(hipMemset(c->st.status, 0, 4));
    if (st & ST_BAD_TOKEN) return fail(c, DUALAR_ERR_BAD_TOKEN, "an id outside its range reached the device");
    if (st & ST_NONFINITE) return fail(c, DUALAR_ERR_DEVICE_FAULT, "a non-finite logit reached the sampler");
    return fail(c, DUALAR_ERR_DEVICE_INDEX, "a device index check failed (checked build)");
  }
  return DUALAR_OK;
}

dualar_status dualar_reset(dualar_ctx_t* c, const int32_t* seq_ids, int32_t n) {
  if (!c) return fail(c, DUALAR_ERR_INVALID_ARG, "ctx is NULL");
  if (!c->ready) return fail(c, DUALAR_ERR_STATE, "reset before a successful prefill");
  if (n < 0 || n > c->batch) return fail(c, DUALAR_ERR_INVALID_ARG, "n out of range [0, batch]");
  if (n == 0) return DUALAR_OK;
  if (!seq_ids) return fail(c, DUALAR_ERR_INVALID_ARG, "seq_ids is NULL");
  for (int i = 0; i < n; ++i)
    if (seq_ids[i] < 0 || seq_ids[i] >= c->batch)
      return fail(c, DUALAR_ERR_INVALID_ARG, "a sequence id is outside [0, batch)");
  HIPCHK(launch_seq_reset(c->st, seq_ids, n, c->batch, c->r.N, c->stream));
  return DUALAR_OK;
}

dualar_status dualar_profile_begin(dualar_ctx_t* c, int32_t kernel_class) {
  if (!c) return fail(c, DUALAR_ERR_INVALID_ARG, "ctx is NULL");
  if (kernel_class < DUALAR_K_GEMV || kernel_class > DUALAR_K_GEMV_SWIGLU)
    return fail(c, DUALAR_ERR_INVALID_ARG, "unknown kernel class");
  c->prof_cls = kernel_class;
  c->ev_used = 0;
  c->prof_launches = 0;
  c->prof_bytes = 0.0;
  return DUALAR_OK;
}

dualar_status dualar_profile_end(dualar_ctx_t* c, int64_t* launches, double* total_ms, double* bytes) {
  if (!c) return fail(c, DUALAR_ERR_INVALID_ARG, "ctx is NULL");
  if (c->prof_cls < 0) return fail(c, DUALAR_ERR_STATE, "profiling was not begun");
  HIPCHK(hipStreamSynchronize(c->stream));
  double ms = 0.0;
  for (size_t i = 0; i + 1 < c->ev_used; i += 2) {
    float t = 0.f;
    HIPCHK(hipEventElapsedTime(&t, c->ev[i], c->ev[i + 1]));
    ms += t;
  }
  if (launches) *launches = c->prof_launches;
  if (total_ms) *total_ms = ms;
  if (bytes) *bytes = c->prof_bytes;
  c->prof_cls = -1;
  c->ev_used = 0;
  return DUALAR_OK;
}

void dualar_destroy(dualar_ctx_t* c) { delete c; }

const char* dualar_status_string(dualar_status s) {
  switch (s) {
    case DUALAR_OK: return "ok";
    case DUALAR_ERR_INVALID_ARG: return "invalid argument";
    case DUALAR_ERR_NO_DEVICE: return "no device";
    case DUALAR_ERR_WORKSPACE: return "workspace too small";
    case DUALAR_ERR_CONTEXT_FULL: return "context full";
    case DUALAR_ERR_BAD_TOKEN: return "bad token";
    case DUALAR_ERR_STATE: return "bad state";
    case DUALAR_ERR_HIP: return "HIP error";
    case DUALAR_ERR_DEVICE_FAULT: return "device fault";
    case DUALAR_ERR_DEVICE_INDEX: return "device index check failed";
  }
  return "unknown status";
}

const char* dualar_last_error(const dualar_ctx_t* c) { return c ? c->err.c_str() : g_create_err.c_str(); }

}  // extern "C"
