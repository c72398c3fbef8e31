// Internal launch interface between the C-ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

// Kernel-timing events for the next single-kernel launch (profiling only).
// When set, the launch hands them to hipExtLaunchKernel, which records them
// at the kernel's own start and end (no marker packets around it), and
// clears them; launchers of several kernels leave them untouched.
struct LaunchEvents { hipEvent_t start, stop; };
extern thread_local LaunchEvents g_launch_ev;

template <typename K, typename... A>
inline void launch_timed(K kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s, A... args) {
  if (g_launch_ev.start) {
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, g_launch_ev.start, g_launch_ev.stop, 0u, args...);
    g_launch_ev = LaunchEvents{nullptr, nullptr};
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  }
}

enum GemvMode { GEMV_STORE = 0, GEMV_ADD = 1, GEMV_SWIGLU = 2 };

// Attention preparation that a QKV product's finish can apply to its output
// (bf16 weights and cache, head_dim = the product's row tile): QK-norm, RoPE
// and the score scale on q, written as three bf16 terms; QK-norm and RoPE on
// k, and k and v appended to the cache at the row's position.
struct QkPrep {
  const float2* rope;                 // [max_pos][hd/2] (cos, sin)
  const int* pos; int pos_const;      // row b's position (pos == NULL: pos_const)
  const void* q_norm; const void* k_norm;
  int H, KV, hd, max_pos;
  void* kcache; void* vcache;         // this layer: [max_batch][KV][max_pos][hd] bf16
  uint16_t* q_planes;                 // [3][B][H*hd]; NULL = no preparation
  int* status;                        // checked build: index failures latch ST_INDEX
};

// y[b, :] = W . f(x[b, :]) for b < B, where f is RMSNorm-with-gain when
// `gain` is set and the identity otherwise.  W is up to three [rows_i, K]
// segments whose outputs are concatenated (STORE/ADD), or the gate/up pair
// (w[0], w[1]) of a SwiGLU FFN whose output is silu(W1 h) * (W3 h).
struct GemvParams {
  const void* w[3];
  // 4-bit form of the segments (1 to GEMV_W4_MAX_ROWS rows, or
  // GEMM_TILE_MIN_ROWS+ rows on the 2-D tiles): q4[i] = packed [rows_i][K/2]
  // bytes, s4[i] = bf16 scales [rows_i][K/128]; q4[0] == NULL: bf16 w[]
  const void* q4[3]; const void* s4[3];
  int rows[3];
  int n_seg;
  int K;
  int n_out;
  const float* x; int ldx;
  const void* gain; float eps;
  float* y; int ldy;
  const float* res; int ldres;   // GEMV_ADD: y = res + W.x (res may alias y)
  int B;
  int mode;
  // scratch for the matrix-core path (B >= 2): the (normalised)
  // activations as three bf16 planes [3][B][K] (6*B*K bytes) and split-K
  // partial sums (part_elems floats)
  void* xn;
  float* part; size_t part_elems;
  // matrix-core path only: xplanes = the input already as planes [3][B][K]
  // (no RMSNorm; x and xn unused); yplanes = write the output as planes
  // [3][B][n_out] instead of y (GEMV_STORE / GEMV_SWIGLU)
  const void* xplanes;
  void* yplanes;
  // GEMV_ADD with split-K partials only: also RMS-normalise each output row
  // with next_gain and write it as planes [3][B][n_out] for the next
  // product; *next_done is set to 1 when this happened (else 0)
  const void* next_gain; void* next_planes; int* next_done;
  int ksw, ldp;                  // set by the launcher
  int zswz;                      // set by the launcher: activation tiles of a swizzled 1-D grid (0 = 3-D grid)
  // set by the launcher for the stream-K form: U = tiles * chunks-per-tile
  // work units dealt to the grid, workgroup g taking sk_q (+1 if g < sk_r)
  // consecutive units; partial tiles at part + (tile * sk_smax + slot) * TE
  int sk_q, sk_r, sk_smax, sk_nch;
  // QKV product only: prepare the attention in the finish when the stream-K
  // form runs (*prep_done = 1; y is written as well)
  QkPrep prep; int* prep_done;
  // prefill steps: bit j of live_bt set = activation rows [GEMM_TILE_BROWS j,
  // GEMM_TILE_BROWS (j + 1)) hold at least one prompt position; the 2-D tile
  // form deals out only those tiles (the outputs of padding rows are never
  // read).  bt_masked = 0: every row is live.
  uint64_t live_bt[2]; int bt_masked;
  int* status;                   // checked build: index failures latch ST_INDEX
};
#define GEMM_TILE_BROWS 128   // activation rows per tile of the 2-D tile form
#define GEMM_TILE_MIN_ROWS 256   // from this many activation rows the products use the 2-D tile form

// Decode attention for one new position per sequence, split along the
// context; also applies QK-norm + RoPE to the new q and k and appends the
// new k, v to the cache.
struct AttnParams {
  const float* qkv; int ld_qkv;       // [B][ld]: q | k | v
  void* kcache; void* vcache;         // this layer: [max_batch][KV][max_pos][hd]
  int max_pos;
  const int* pos;                     // device [B] (slow), or NULL -> pos_const
  int pos_const;
  const float2* rope;                 // [max_pos][hd/2] (cos, sin), bf16 values
  const void* q_norm; const void* k_norm; float eps;
  int H, KV, hd;
  int it;                             // K/V loads per lane (2, 4 or 8): sets the chunk
  int lmax;                           // max over rows of pos + 1
  int chunk, max_splits;              // set by the launcher
  float* part;                        // [B][H][max_splits][hd + 2]
  unsigned* counters;                 // [B][KV], zero between launches
  float* out; int ld_out;             // [B][H*hd]
  uint16_t* out_planes;               // if set: o as planes [3][B][H*hd] instead of out
  uint16_t* q_planes;                 // scratch [3][B][H*hd] (flash-decoding form)
  int prepped;                        // q_planes and the appended k/v are already written
  int no_merge;                       // split form: leave the partials for a fused merge
  int B;
  int* status;                        // checked build: index failures latch ST_INDEX
};

// Batch-1 attention over a short cache (at most 16 positions: the fast AR's
// depth cache) fused with the O product and its residual: x += W_o . attn.
// Also applies QK-norm + RoPE to the new q and k and appends k, v at pos.
struct AttnOParams {
  const float* qkv;                   // q | k | v of the one row
  void* kcache; void* vcache;         // this layer, sequence 0: [KV][max_pos][hd] bf16
  int max_pos, pos;                   // attends to positions 0..pos
  const float2* rope;                 // [max_pos][hd/2] (cos, sin)
  const void* q_norm; const void* k_norm; float eps;
  int H, KV, hd;
  const void* wo;                     // [dim][H*hd] bf16
  float* x; int dim;                  // residual row, updated in place
  int* status;                        // checked build: index failures latch ST_INDEX
};
bool attn_o_b1_fits(int H, int KV, int hd, int dim, int L);
hipError_t launch_attn_o_b1(const AttnOParams& p, hipStream_t s);

// Batch-1 merge of the split attention partials (AttnParams::part of the
// split form, run with no_merge) fused with the O product and its residual.
// Same head shape as attn_o_b1 (H = 32, KV = 8, hd = 128, bf16 weights).
struct MergeOParams {
  const float* part; int max_splits, chunk;   // [H][max_splits][hd + 2] (o, m, l); the split form's chunk
  const float* att;                   // o when the context fits one chunk
  const int* pos;                     // device [1]: the row's position (context pos + 1)
  int H, hd;
  const void* wo;                     // [dim][H*hd] bf16
  float* x; int dim;                  // residual row, updated in place
  int* status;                        // checked build: index failures latch ST_INDEX
};
int merge_o_b1_max_splits();
// batch-1 split attention (bf16 cache, S2 head shape) for chunks of 128 or 256
// positions, writing the split form's partials; false if the shape does not fit
bool launch_attn_split_b1(const AttnParams& p, hipStream_t s);
hipError_t launch_merge_o_b1(const MergeOParams& p, hipStream_t s);
int attn_chunk(int kv_esz, int hd, int it);
hipError_t launch_attn_merge(const AttnParams& p, hipStream_t s);

// Prefill of a chunk of positions: rows r = b*C + i hold position pos[r] of
// sequence b (-1 = padding).  prefill_append_kernel applies QK-norm and RoPE
// to every row's q and k, writes q (scaled by 1/sqrt(hd)) to qbuf and
// appends k, v to the cache; prefill_attn_kernel then attends each row to
// positions 0..pos[r] of its sequence.
struct PrefillParams {
  const float* qkv; int ld_qkv;       // [R][ld]: q | k | v
  float* qbuf; int ld_q;              // [R][H*hd]
  void* kcache; void* vcache;         // this layer: [max_batch][KV][max_pos][hd]
  int max_pos;
  const int* pos;                     // [R], or NULL: every row at pos_const
  int pos_const;
  int C;                              // rows per sequence
  const float2* rope;                 // [max_pos][hd/2] (cos, sin)
  const void* q_norm; const void* k_norm; float eps;
  int H, KV, hd;
  float* out; int ld_out;             // [R][H*hd]
  uint16_t* out_planes;               // if set: o as planes [3][R][H*hd] instead of out
  int R, B;
  int* status;                        // checked build: index failures latch ST_INDEX
};

// Per-sequence decode state kept in the workspace.
struct SeqState {
  int* pos;        // [max_batch] next slow position (prefill: position of this step)
  int* done;       // [max_batch]
  int* frames;     // [max_batch] frames emitted
  int* cur;        // [max_batch][N+1] codes of the last frame
  int* plen;       // [max_batch] prompt lengths
  int* frame_idx;  // [1] frame index inside the current call
  int* status;     // [1] latched device faults
  int* ras_hist;   // [max_batch][RAS_HIST_STRIDE] ring of emitted slow ids: slot f % RAS_HIST_STRIDE = frame f's
};
#define RAS_HIST_STRIDE 16   // = DUALAR_RAS_MAX_WINDOW, a power of two

// Candidate set / bookkeeping for the sampler.
struct SampleParams {
  const float* logits; int ld;
  int restricted;               // slow: logits hold the C+1 candidates in id order (else the vocabulary)
  int B;
  int slow;                     // 1: semantic ids + end id, 0: all C fast codes
  int sb, se, end_id, C, N;
  int k;                        // codebook index written (0 = slow sample)
  int greedy; float temperature, top_p; int min_frames;
  int ras_window; float ras_temperature, ras_top_p;   // slow loop breaker (0 = off); its draw is slot N
  const float* uniforms; int u_frame_stride; int u_row_stride;   // uniforms[f*fs + b*rs + slot]
  int* codes; long long c_row_stride; int c_frame_stride; int c_col;   // codes out (NULL = none)
  const void* fast_emb; int fast_dim; float* x_next;   // x_next[b] = E_fast[q] (NULL = none)
  int last;                     // 1: end of frame bookkeeping
  int fast_only;
  SeqState st;
};

struct EmbedParams {
  // source of the token column: prompt tokens (prefill) or the state's last frame
  const int* tokens; int t_max; int step;   // prefill: row r = b*rows_per_seq + i uses
  int prefill;                              //   t = step + i - (t_max - plen[b])
  int rows_per_seq;                         // prefill rows per sequence (decode: 1)
  int* pos_out;                             // prefill: [B*rows_per_seq] t or -1
  const void* tok_emb; const void* cb_emb;
  int dim, V, N, C, sb, se, scale;
  float* x;
  int B;
  SeqState st;
};

// Teacher-forced fast AR rows: row i*N + k is the slow hidden state of
// pair i (k = 0) or E_F[codes[i][k - 1]] (k >= 1).
struct TfParams {
  const float* hidden;     // [n][dim]
  const int* codes;        // [n][N]
  const void* fast_emb;    // [C][dim]
  float* x;                // [n*N][dim]
  int n, N, C, dim;
  int* status;             // out-of-range codes latch ST_BAD_TOKEN
};

struct FastBeginParams {
  const float* hidden; const int* q0;   // [n_frames][B][dim], [n_frames][B]
  const void* fast_emb; int dim, C, N;
  float* x_slow; float* x_fast;
  int* codes; long long c_row_stride; int c_frame_stride;
  int B;
  SeqState st;
};

template <typename T> hipError_t launch_gemv(const GemvParams& p, hipStream_t s);
bool launch_gemm_mfma(const GemvParams& p, hipStream_t s, hipError_t* err);
// tiled matrix-core product for hundreds of activation rows (input planes at p.xn)
bool launch_gemm_tile(const GemvParams& p, bool wide, hipStream_t s);
// the same with 4-bit weights (p.q4, p.s4; K a multiple of 128, at most 10,240)
bool launch_gemm_tile_w4(const GemvParams& p, hipStream_t s);
// 4-bit weights with 2..GEMV_W4_MAX_ROWS activation rows, input planes at p.xn
#define GEMV_W4_MAX_ROWS 8
bool launch_gemv_w4_rows(const GemvParams& p, hipStream_t s, hipError_t* e);
// whether that form splits (and normalises) its fp32 input itself (no planes given)
bool gemv_w4_rows_normalises(const GemvParams& p);
bool gemm_tile_wide(const GemvParams& p);
template <typename T, typename KT> hipError_t launch_attn(const AttnParams& p, hipStream_t s);
template <typename T, typename KT> hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t s);
// k/v append only (no q, no attention): rows are sequences, grid (R, KV)
template <typename T, typename KT> hipError_t launch_kv_append(const PrefillParams& p, hipStream_t s);
template <typename T> hipError_t launch_sample(const SampleParams& p, hipStream_t s);
template <typename T> hipError_t launch_embed(const EmbedParams& p, hipStream_t s);
template <typename T> hipError_t launch_fast_begin(const FastBeginParams& p, hipStream_t s);
template <typename T> hipError_t launch_tf_embed(const TfParams& p, hipStream_t s);
// causal attention along depth inside each group of C rows (grid (B, KV)), with
// the decode arithmetic for QK-norm, RoPE at position row % C and the cache rounding
template <typename T, typename KT> hipError_t launch_depth_attn(const PrefillParams& p, hipStream_t s);
hipError_t launch_frame_reset(SeqState st, hipStream_t s);
hipError_t launch_frame_end(SeqState st, int B, int advance_pos, hipStream_t s);
hipError_t launch_prefill_begin(SeqState st, const int* plen_host, int B, int N, hipStream_t s);
hipError_t launch_seq_reset(SeqState st, const int* ids, int n, int B, int N, hipStream_t s);
