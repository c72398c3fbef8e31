// Token-level kernels of the decode step: multi-codebook fusion (the slow-AR
// input), the semantic-logit-biased slow sampler, the unmasked fast sampler,
// and per-frame bookkeeping.
//
// Fusion (Fish Audio S2 report Eq. 1, with the sqrt(N+1) divide applied when
// scale_codebook_embeddings is on): for a semantic id the input is
//   (E_tok[id] + E_F[0*C + q0] + ... + E_F[(N-1)*C + q_{N-1}]) / sqrt(N+1),
// summed in fp32 in that order; a text id takes E_tok[id] alone.
//
// Sampler: one workgroup of 1024 threads per sequence.  The slow candidates
// are the semantic ids and <|im_end|> (every other logit carries the -inf
// bias, so it can never be drawn); the fast candidates are all C codes.
// Greedy = argmax with the lowest id on ties.  Top-p: e_i = exp((z_i -
// zmax)/T), in the order (e desc, id asc) keep the shortest prefix whose
// mass reaches top_p * total, draw the first kept index whose cumulative
// mass exceeds u * kept mass (found by radix selection, see tp_select).
#include "common.h"
#include "internal.h"

#define SMP_THREADS 1024

// ---------------------------------------------------------------------------
// fusion / embedding
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(DUALAR_WG) embed_kernel(EmbedParams p) {
  // grid (rows, ceil(dim / 256)): one element of one row per thread.  Prefill
  // row r is position step + i - (t_max - plen[b]) of sequence b
  // (r = b*rows_per_seq + i); the last row of a sequence also sets its state
  // position.
  const int row = blockIdx.x;
  int b = row;
  const int tid = threadIdx.x;
  // The column (N + 1 <= 33 ids) is read with compile-time indexes only, so
  // it stays in registers (a runtime-indexed private array goes to scratch).
  int col[33];
  int act = 1;
  const int* src;
  size_t stride = 1;
  if (p.prefill) {
    b = row / p.rows_per_seq;
    const int i = row % p.rows_per_seq;
    const int t = p.step + i - (p.t_max - p.st.plen[b]);
    act = t >= 0;
    if (blockIdx.y == 0 && tid == 0) {
      if (p.pos_out) p.pos_out[row] = act ? t : -1;
      if (i == p.rows_per_seq - 1) p.st.pos[b] = act ? t : -1;
    }
    src = p.tokens + (size_t)b * (p.N + 1) * p.t_max + (act ? t : 0);
    stride = (size_t)p.t_max;
  } else {
    act = !p.st.done[b];
    src = p.st.cur + (size_t)b * (p.N + 1);
  }
  const int d = blockIdx.y * DUALAR_WG + tid;
  float* x = p.x + (size_t)row * p.dim;
  if (!act) {
    if (d < p.dim) x[d] = 0.f;
    return;
  }
#pragma unroll
  for (int r = 0; r < 33; ++r) col[r] = r <= p.N ? src[r * stride] : 0;
  int bad = 0;
  if (col[0] < 0 || col[0] >= p.V) { bad = 1; col[0] = 0; }
  const bool sem = col[0] >= p.sb && col[0] <= p.se;
  if (sem) {
#pragma unroll
    for (int k = 0; k < 32; ++k)
      if (k < p.N && (col[1 + k] < 0 || col[1 + k] >= p.C)) { bad = 1; col[1 + k] = 0; }
  }
  if (bad && blockIdx.y == 0 && tid == 0) atomicOr(p.st.status, ST_BAD_TOKEN);
  if (d >= p.dim) return;
  const float e0 = ElemT<T>::load(p.tok_emb, (size_t)col[0] * p.dim + d);
  if (!sem) { x[d] = e0; return; }
  float v[32];
#pragma unroll
  for (int k = 0; k < 32; ++k)
    if (k < p.N) v[k] = ElemT<T>::load(p.cb_emb, ((size_t)k * p.C + col[1 + k]) * p.dim + d);
  float s = e0;
#pragma unroll
  for (int k = 0; k < 32; ++k)
    if (k < p.N) s += v[k];
  if (p.scale) s = s / sqrtf((float)(p.N + 1));
  x[d] = s;
}

// ---------------------------------------------------------------------------
// sampler
// ---------------------------------------------------------------------------
struct Best { float v; int i; };
__device__ __forceinline__ Best better(Best a, Best b) {
  // larger value wins; equal values -> lower index (ids are ascending in index)
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}

#define DPP_I(v, ctrl) __builtin_amdgcn_update_dpp(0, (v), ctrl, 0xF, 0xF, true)
__device__ __forceinline__ Best best_dpp(Best x, int ctrl_sel) {
  Best y;
  switch (ctrl_sel) {
    case 0: y.v = xor1_of(x.v); y.i = DPP_I(x.i, 0xB1); break;
    case 1: y.v = xor2_of(x.v); y.i = DPP_I(x.i, 0x4E); break;
    case 2: y.v = mir8_of(x.v); y.i = DPP_I(x.i, 0x141); break;
    default: y.v = mir16_of(x.v); y.i = DPP_I(x.i, 0x140); break;
  }
  return better(x, y);
}
__device__ __forceinline__ Best best_swap(Best x, bool wide) {
  const auto rv = wide ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x.v), __float_as_uint(x.v), false, false)
                       : __builtin_amdgcn_permlane16_swap(__float_as_uint(x.v), __float_as_uint(x.v), false, false);
  const auto ri = wide ? __builtin_amdgcn_permlane32_swap((unsigned)x.i, (unsigned)x.i, false, false)
                       : __builtin_amdgcn_permlane16_swap((unsigned)x.i, (unsigned)x.i, false, false);
  return better(Best{__uint_as_float(rv[0]), (int)ri[0]}, Best{__uint_as_float(rv[1]), (int)ri[1]});
}

__device__ __forceinline__ Best block_best(Best x, Best* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int c = 0; c < 4; ++c) x = best_dpp(x, c);
  x = best_swap(x, false);
  x = best_swap(x, true);
  if (lane == 0) sh[wave] = x;
  __syncthreads();
  Best r = sh[0];
  for (int w = 1; w < SMP_THREADS / 64; ++w) r = better(r, sh[w]);
  __syncthreads();
  return r;
}


// Top-p without a sort.  The candidates' order (e desc, index asc) is that
// of the 45-bit keys e_bits << 13 | (8191 - i) (e >= 0, so its float bits
// order as its value), and masses are fixed point, m = e * 2^40 rounded
// (integer sums: the same in any order, so the draw is reproducible).  The
// nucleus is the shortest prefix of the order whose mass reaches top_p * T,
// i.e. it ends at the largest key K with mass(keys >= K) >= top_p * T; the
// draw is the first kept candidate whose cumulative mass exceeds u * kept,
// i.e. the largest key with mass(keys >= K) > u * kept.  Both keys are found
// by a radix descent: 8 key bits per pass, a histogram of (mass, count) over
// the candidates that share the bits found so far, suffix sums over the
// 256 digits from the top, and the digit where the condition still holds;
// a pass whose digit holds a single candidate ends the descent.  The
// descent starts below the bits that every candidate key shares (the common
// prefix of the smallest and the largest key): a digit there would hold the
// whole set, so its pass would choose it without narrowing anything.
#define TP_E 5                              // candidates per thread: nc <= 5120
#define TP_IDX_BITS 13
#define TP_KEY_BITS (32 + TP_IDX_BITS)
#define TP_NB 256
#define TP_WAVES (SMP_THREADS / 64)
static_assert(TP_E * SMP_THREADS >= 4097, "the slow candidates fit");

struct TopPShared {
  unsigned long long mass[TP_WAVES][TP_NB];   // per-wave histograms
  unsigned cnt[TP_WAVES][TP_NB];
  unsigned long long wtot[TP_WAVES];
  unsigned long long wmin[TP_WAVES], wmax[TP_WAVES];
  int cand_t[TP_NB / 64];                     // per digit wave: its chosen digit, or -1
  unsigned long long cand_above[TP_NB / 64];
  int cand_single[TP_NB / 64];
  unsigned long long found_key, found_mass;
};

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum of v over the workgroup (fixed order: lanes, then waves 0..15).
__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v, TopPShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_sum_u64(v);
  if (lane == 0) sh.wtot[wave] = v;
  __syncthreads();
  unsigned long long t = 0;
#pragma unroll
  for (int w = 0; w < TP_WAVES; ++w) t += sh.wtot[w];
  __syncthreads();
  return t;
}

// Smallest and largest candidate key over the workgroup (key 0 = none).
__device__ __forceinline__ void block_key_range(const unsigned long long (&key)[TP_E], TopPShared& sh,
                                                unsigned long long* kmin, unsigned long long* kmax) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long lo = ~0ull, hi = 0ull;
#pragma unroll
  for (int s = 0; s < TP_E; ++s)
    if (key[s] != 0ull) { lo = min(lo, key[s]); hi = max(hi, key[s]); }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    lo = min(lo, (unsigned long long)__shfl_xor(lo, o));
    hi = max(hi, (unsigned long long)__shfl_xor(hi, o));
  }
  if (lane == 0) { sh.wmin[wave] = lo; sh.wmax[wave] = hi; }
  __syncthreads();
  lo = sh.wmin[0];
  hi = sh.wmax[0];
#pragma unroll
  for (int w = 1; w < TP_WAVES; ++w) { lo = min(lo, sh.wmin[w]); hi = max(hi, sh.wmax[w]); }
  __syncthreads();
  *kmin = lo;
  *kmax = hi;
}

// The largest candidate key K with mass(keys >= K) >= thr (strict: > thr),
// and mass(keys >= K).  The caller guarantees that the whole set satisfies
// the condition.
__device__ __forceinline__ void tp_select(const unsigned long long (&key)[TP_E], const unsigned long long (&m)[TP_E],
                                          double thr, bool strict, TopPShared& sh, unsigned long long* k_out,
                                          unsigned long long* m_out, unsigned long long kmin,
                                          unsigned long long kmax) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // bits [lo, TP_KEY_BITS) are common to every key (all of them when the
  // set holds one candidate: keys are distinct); nothing lies above them
  int lo = kmin == kmax ? 0 : 64 - __clzll(kmin ^ kmax);
  unsigned long long P = kmin >> lo, above = 0;
  while (lo > 0) {
    const int hi = lo;                       // bits [lo, hi) are this pass's digit
    lo = hi > 8 ? hi - 8 : 0;
    const int w = hi - lo;
    for (int j = lane; j < TP_NB; j += 64) { sh.mass[wave][j] = 0ull; sh.cnt[wave][j] = 0u; }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int s = 0; s < TP_E; ++s)
      if (key[s] != 0ull && (key[s] >> hi) == P) {
        const int d = (int)((key[s] >> lo) & ((1ull << w) - 1));
        atomicAdd(&sh.mass[wave][d], m[s]);
        atomicAdd(&sh.cnt[wave][d], 1u);
      }
    __syncthreads();
    // digit t = tid (first four waves): its mass and count over the waves,
    // then suffix sums from the top digit down
    unsigned long long mt = 0, suf = 0;
    unsigned ct = 0;
    if (tid < TP_NB) {
#pragma unroll
      for (int ww = 0; ww < TP_WAVES; ++ww) { mt += sh.mass[ww][tid]; ct += sh.cnt[ww][tid]; }
      suf = mt;     // inclusive suffix sum within the wave (lanes above this one)
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long y = __shfl_down(suf, o);
        if (lane + o < 64) suf += y;
      }
      if (lane == 0) sh.wtot[wave] = suf;
    }
    __syncthreads();
    // the highest non-empty digit whose suffix mass meets the condition:
    // the wanted key is the largest one that does, so it lies in that digit
    if (tid < TP_NB) {
      for (int ww = wave + 1; ww < TP_NB / 64; ++ww) suf += sh.wtot[ww];
      const double s_t = (double)(above + suf);
      const bool c_t = tid < (1 << w) && ct > 0u && (strict ? s_t > thr : s_t >= thr);
      const unsigned long long bal = __ballot(c_t);
      if (bal == 0ull) {
        if (lane == 0) sh.cand_t[wave] = -1;
      } else if (lane == 63 - __clzll(bal)) {
        sh.cand_t[wave] = tid;
        sh.cand_above[wave] = above + (suf - mt);
        sh.cand_single[wave] = ct == 1u;
      }
    }
    __syncthreads();
    int bw = TP_NB / 64 - 1;
    while (bw > 0 && sh.cand_t[bw] < 0) --bw;
    // (a digit always qualifies: the set holds the wanted key)
    const int dt = sh.cand_t[bw] < 0 ? 0 : sh.cand_t[bw];
    P = (P << w) | (unsigned long long)dt;
    above = sh.cand_above[bw];
    const int single = sh.cand_single[bw];
    __syncthreads();
    if (single) break;
  }
  // the one candidate with these high bits
#pragma unroll
  for (int s = 0; s < TP_E; ++s)
    if (key[s] != 0ull && (key[s] >> lo) == P) { sh.found_key = key[s]; sh.found_mass = m[s]; }
  __syncthreads();
  *k_out = sh.found_key;
  *m_out = above + sh.found_mass;
  __syncthreads();
}

template <typename T>
__global__ void __launch_bounds__(SMP_THREADS) sample_kernel(SampleParams p) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ TopPShared tps;
  __shared__ Best shb[SMP_THREADS / 64];
  __shared__ int choice;
  __shared__ int ras_hit;

  const int f = *p.st.frame_idx;
  const int was_done = p.st.done[b];
  int* crow = p.codes ? p.codes + (size_t)b * p.c_row_stride + (size_t)f * p.c_frame_stride : nullptr;
  if (was_done) {
    if (p.slow && crow && tid <= p.N) crow[p.c_col + tid] = -1;
    return;
  }

  const int C = p.C;
  const int nc = p.slow ? C + 1 : C;
  const bool end_first = p.end_id < p.sb;
  const bool allow_end = p.slow && (p.st.frames[b] >= p.min_frames);
  const float* z = p.logits + (size_t)b * p.ld;
  // candidate index -> token id (ascending)
  auto cand_id = [&](int i) -> int {
    if (!p.slow) return i;
    if (end_first) return i == 0 ? p.end_id : p.sb + i - 1;
    return i == C ? p.end_id : p.sb + i;
  };
  auto cand_ok = [&](int i) -> bool { return !p.slow || cand_id(i) != p.end_id || allow_end; };

  // max (and argmax) over the candidates
  Best best{-INFINITY, 0x7fffffff};
  int bad = 0;
  for (int i = tid; i < nc; i += SMP_THREADS) {
    if (!cand_ok(i)) continue;
    const float v = z[p.restricted ? i : cand_id(i)];
    if (!(v == v) || v == INFINITY) bad = 1;
    best = better(best, Best{v, i});
  }
  if (bad) atomicOr(p.st.status, ST_NONFINITE);
  best = block_best(best, shb);

  // top-p draw with uniform u: every thread takes part; sets choice
  auto topp = [&](float temperature, float top_p, float u) __attribute__((always_inline)) {
    const float zmax = best.v;
    const float invT = 1.0f / temperature;
    unsigned long long key[TP_E], m[TP_E];
    unsigned long long tot = 0;
#pragma unroll
    for (int s = 0; s < TP_E; ++s) {
      const int i = tid + s * SMP_THREADS;
      float e = 0.f;
      if (i < nc && cand_ok(i)) e = expf((z[p.restricted ? i : cand_id(i)] - zmax) * invT);
      // key 0 marks "no candidate": a candidate's key is never 0 (its index
      // bits are 8191 - i > 0 for i < 8191)
      key[s] = i < nc ? ((unsigned long long)__float_as_uint(e) << TP_IDX_BITS) |
                            (unsigned long long)((1 << TP_IDX_BITS) - 1 - i)
                      : 0ull;
      m[s] = __float2ull_rn(e * 1099511627776.0f);   // e * 2^40
      tot += m[s];
    }
    tot = block_sum_u64(tot, tps);
    unsigned long long kmin, kmax;
    block_key_range(key, tps, &kmin, &kmax);
    unsigned long long kb, kept;
    tp_select(key, m, fmin((double)top_p * (double)tot, (double)tot), false, tps, &kb, &kept, kmin, kmax);
    const double target = (double)u * (double)kept;
    unsigned long long kd = kb, md;
    // the draw lies among the kept keys (>= kb)
    if (target < (double)kept) tp_select(key, m, target, true, tps, &kd, &md, kb, kmax);
    if (tid == 0) choice = (1 << TP_IDX_BITS) - 1 - (int)(kd & ((1ull << TP_IDX_BITS) - 1));
  };
  const float* ub = p.uniforms ? p.uniforms + (size_t)f * p.u_frame_stride + (size_t)b * p.u_row_stride : nullptr;
  if (p.greedy) {
    if (tid == 0) choice = best.i;
  } else {
    topp(p.temperature, p.top_p, ub[p.k]);
  }
  __syncthreads();

  // Loop breaker ([P2] "Two autoregressions ...", the paragraph after Eq. 1):
  // a slow draw that repeats a semantic id of the sequence's last ras_window
  // frames is replaced by a second top-p draw with its own uniform (slot N).
  // Every emitted slow id (but <|im_end|>) enters a ring of RAS_HIST_STRIDE
  // slots at slot frames % RAS_HIST_STRIDE, whether or not the breaker is on
  // for this call, so the window is always the last min(frames, ras_window)
  // frames of this generation, also when calls change the window or turn
  // the breaker on and off.
  if (p.slow) {
    const int fr = p.st.frames[b];
    int* hist = p.st.ras_hist + (size_t)b * RAS_HIST_STRIDE;
    if (p.ras_window > 0) {
      if (tid == 0) {
        const int id0 = cand_id((choice >= 0 && choice < nc) ? choice : 0);
        int hit = 0;
        if (id0 != p.end_id)
          for (int i = 0; i < min(fr, p.ras_window); ++i) hit |= hist[(fr - 1 - i) & (RAS_HIST_STRIDE - 1)] == id0;
        ras_hit = hit;
      }
      __syncthreads();
      if (ras_hit) {
        topp(p.ras_temperature, p.ras_top_p, ub[p.N]);
        __syncthreads();
      }
    }
    if (tid == 0) {
      const int id1 = cand_id((choice >= 0 && choice < nc) ? choice : 0);
      if (id1 != p.end_id) hist[fr & (RAS_HIST_STRIDE - 1)] = id1;
    }
  }

  const int ci = (choice >= 0 && choice < nc) ? choice : 0;   // NaN logits: stay in range
  const int id = cand_id(ci);
  if (p.slow) {
    if (id == p.end_id) {
      if (tid == 0) p.st.done[b] = 1;
      if (crow && tid <= p.N) crow[p.c_col + tid] = tid == 0 ? id : -1;
      if (p.x_next)
        for (int d = tid; d < p.fast_dim; d += SMP_THREADS) p.x_next[(size_t)b * p.fast_dim + d] = 0.f;
      return;
    }
    const int q0 = id - p.sb;
    if (tid == 0) {
      p.st.cur[b * (p.N + 1)] = id;
      p.st.cur[b * (p.N + 1) + 1] = q0;
      if (crow) { crow[p.c_col] = id; crow[p.c_col + 1] = q0; }
    }
    if (p.x_next)
      for (int d = tid; d < p.fast_dim; d += SMP_THREADS)
        p.x_next[(size_t)b * p.fast_dim + d] = ElemT<T>::load(p.fast_emb, (size_t)q0 * p.fast_dim + d);
  } else {
    if (tid == 0) {
      if (!p.fast_only) p.st.cur[b * (p.N + 1) + 1 + p.k] = id;
      if (crow) crow[p.c_col] = id;
    }
    if (p.x_next)
      for (int d = tid; d < p.fast_dim; d += SMP_THREADS)
        p.x_next[(size_t)b * p.fast_dim + d] = ElemT<T>::load(p.fast_emb, (size_t)id * p.fast_dim + d);
  }
}

// ---------------------------------------------------------------------------
// fast-AR-only frame start: x_slow <- given hidden, x_fast <- E_fast[q0]
// ---------------------------------------------------------------------------
template <typename T>
__global__ void __launch_bounds__(DUALAR_WG) fast_begin_kernel(FastBeginParams p) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int f = *p.st.frame_idx;
  int q = p.q0[(size_t)f * p.B + b];
  if (q < 0 || q >= p.C) {
    if (tid == 0) atomicOr(p.st.status, ST_BAD_TOKEN);
    q = 0;
  }
  if (tid == 0) {
    p.st.done[b] = 0;
    if (p.codes) p.codes[(size_t)b * p.c_row_stride + (size_t)f * p.c_frame_stride] = q;
  }
  const float* h = p.hidden + ((size_t)f * p.B + b) * p.dim;
  for (int d = tid; d < p.dim; d += DUALAR_WG) {
    p.x_slow[(size_t)b * p.dim + d] = h[d];
    p.x_fast[(size_t)b * p.dim + d] = ElemT<T>::load(p.fast_emb, (size_t)q * p.dim + d);
  }
}

// ---------------------------------------------------------------------------
// bookkeeping
// ---------------------------------------------------------------------------
__global__ void frame_end_kernel(SeqState st, int B, int advance_pos) {
  const int b = threadIdx.x;
  if (b < B && advance_pos) {
    st.pos[b] += 1;
    if (!st.done[b]) st.frames[b] += 1;
  }
  if (b == 0) *st.frame_idx += 1;
}

__global__ void frame_reset_kernel(SeqState st) { *st.frame_idx = 0; }

struct PlenArg { int v[256]; };
__global__ void prefill_begin_kernel(SeqState st, PlenArg plen, int B, int N) {
  const int b = threadIdx.x;
  if (b < B) {
    st.plen[b] = plen.v[b];
    st.done[b] = 0;
    st.frames[b] = 0;
    for (int r = 0; r <= N; ++r) st.cur[b * (N + 1) + r] = 0;
    for (int i = 0; i < RAS_HIST_STRIDE; ++i) st.ras_hist[b * RAS_HIST_STRIDE + i] = 0;
  }
  if (b == 0) *st.frame_idx = 0;
}

// Retire the sequences whose bit is set: finished (later frames emit -1 rows
// and no samples), no frames emitted, no pending frame, an empty loop-breaker
// window.  Their rows keep being computed on zero input with the batch, at
// positions that keep advancing, and are never read by another sequence.
struct SlotMask { uint64_t w[4]; };
__global__ void seq_reset_kernel(SeqState st, SlotMask m, int B, int N) {
  const int b = threadIdx.x;
  if (b >= B || !((m.w[b >> 6] >> (b & 63)) & 1)) return;
  st.done[b] = 1;
  st.frames[b] = 0;
  for (int r = 0; r <= N; ++r) st.cur[b * (N + 1) + r] = 0;
  for (int i = 0; i < RAS_HIST_STRIDE; ++i) st.ras_hist[b * RAS_HIST_STRIDE + i] = 0;
}

hipError_t launch_seq_reset(SeqState st, const int* ids, int n, int B, int N, hipStream_t s) {
  SlotMask m{};
  for (int i = 0; i < n; ++i) m.w[ids[i] >> 6] |= 1ull << (ids[i] & 63);
  hipLaunchKernelGGL(seq_reset_kernel, dim3(1), dim3(256), 0, s, st, m, B, N);
  return hipGetLastError();
}

template <typename T> hipError_t launch_embed(const EmbedParams& p, hipStream_t s) {
  const int rows = p.prefill ? p.B * p.rows_per_seq : p.B;
  hipLaunchKernelGGL(embed_kernel<T>, dim3(rows, (p.dim + DUALAR_WG - 1) / DUALAR_WG), dim3(DUALAR_WG), 0, s, p);
  return hipGetLastError();
}
template <typename T> hipError_t launch_sample(const SampleParams& p, hipStream_t s) {
  hipLaunchKernelGGL(sample_kernel<T>, dim3(p.B), dim3(SMP_THREADS), 0, s, p);
  return hipGetLastError();
}
template <typename T> hipError_t launch_fast_begin(const FastBeginParams& p, hipStream_t s) {
  hipLaunchKernelGGL(fast_begin_kernel<T>, dim3(p.B), dim3(DUALAR_WG), 0, s, p);
  return hipGetLastError();
}
hipError_t launch_frame_end(SeqState st, int B, int advance_pos, hipStream_t s) {
  hipLaunchKernelGGL(frame_end_kernel, dim3(1), dim3(256), 0, s, st, B, advance_pos);
  return hipGetLastError();
}
hipError_t launch_frame_reset(SeqState st, hipStream_t s) {
  hipLaunchKernelGGL(frame_reset_kernel, dim3(1), dim3(1), 0, s, st);
  return hipGetLastError();
}
hipError_t launch_prefill_begin(SeqState st, const int* plen, int B, int N, hipStream_t s) {
  PlenArg a;
  for (int b = 0; b < 256; ++b) a.v[b] = b < B ? plen[b] : 0;
  hipLaunchKernelGGL(prefill_begin_kernel, dim3(1), dim3(256), 0, s, st, a, B, N);
  return hipGetLastError();
}

template hipError_t launch_embed<float>(const EmbedParams&, hipStream_t);
template hipError_t launch_embed<bf16_t>(const EmbedParams&, hipStream_t);
template hipError_t launch_sample<float>(const SampleParams&, hipStream_t);
template hipError_t launch_sample<bf16_t>(const SampleParams&, hipStream_t);
template hipError_t launch_fast_begin<float>(const FastBeginParams&, hipStream_t);
template hipError_t launch_fast_begin<bf16_t>(const FastBeginParams&, hipStream_t);
