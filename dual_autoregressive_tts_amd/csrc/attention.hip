// GQA decode attention for one new position per sequence (slow AR over the
// time cache, fast AR over the N-slot depth cache).
//
// attn_partial_kernel, grid (split, kv_head, batch): a workgroup takes one
// chunk of CH = 4 waves x PPW x IT consecutive cache positions of one KV
// head and the rep = H/KV query heads sharing it (contiguous grouping: query
// head h uses KV head h / rep).  It
//   1. issues every K and V load of its chunk up front (they do not depend on
//      q), so one memory latency covers the chunk;
//   2. applies QK-norm (per-head RMSNorm with one [hd] gain) and RoPE to the
//      new q heads, folding in the 1/sqrt(hd) score scale;
//   3. if its chunk holds the new position, normalises/rotates the new k,
//      rounds k and v to the cache type and appends them (the new entry is
//      taken from LDS, never re-read from memory);
//   4. computes scores, a chunk-local softmax (max m, sum l) and the
//      unnormalised P.V, and writes (o, m, l) -- or, when the whole context
//      fits one chunk, the final o = P.V / l.
// attn_merge_kernel, grid (batch, H): o = sum_s e^(m_s-M) o_s / sum_s e^(m_s-M) l_s.
// There are no atomics or cross-workgroup fences: the merge is its own launch.
// K/V rows are read with 16-byte lane loads: LPP = hd*sizeof(KT)/16 lanes
// cover one position, so a wave reads PPW = 64/LPP positions per load.
#include "common.h"
#include "internal.h"

#define ATT_MAXHD 128
#define ATT_MAXCH 256
#define ATT_MAXSPLIT 4096   // max_seq_len <= 65536 and chunks of >= 16 positions

typedef __bf16 att_bf16x8 __attribute__((ext_vector_type(8)));
typedef float att_f32x4 __attribute__((ext_vector_type(4)));

// MQK (bf16 cache, head_dim 128, IT = 4 or 8): the scores come from
// v_mfma_f32_16x16x32_bf16 with 16 cache positions as the A operand (lane l:
// position l%16, dims 8*(l/16)..+8 of a 32-dim step, read straight from the
// cache) and the rep query heads as the B operand (three bf16 terms of the
// fp32 q, so the product is the fp32 one), instead of per-lane dot products
// and 16-lane reductions.  The V side is unchanged.
template <typename T, typename KT, int IT, int REP, bool MQK = false>
__global__ void __launch_bounds__(DUALAR_WG) attn_partial_kernel(AttnParams p) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int pos = row_position(p.pos, p.pos_const, b, p.max_pos, p.status);
  if (pos < 0) return;                      // inactive row (prefill padding)
  const int L = pos + 1;
  const int n_splits = (L + p.chunk - 1) / p.chunk;
  if (split >= n_splits) return;
  const int c0 = split * p.chunk, c1 = min(c0 + p.chunk, L);
  const int hd = p.hd;
  constexpr int rep = REP;   // query heads per KV head
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  constexpr int EPL = ElemT<KT>::EPV;
  const int LPP = hd / EPL;
  const int PPW = 64 / LPP;
  const int sub = lane % LPP, grp = lane / LPP;

  __shared__ float qs[REP][ATT_MAXHD];
  __shared__ float knew[ATT_MAXHD], vnew[ATT_MAXHD];
  __shared__ float sc[REP][ATT_MAXCH];
  __shared__ float accs[4][REP][ATT_MAXHD];
  __shared__ float ml[REP][2];
  constexpr int GW = MQK ? IT / 4 : 1;        // MQK: 16-position groups per wave
  __shared__ __attribute__((aligned(16))) uint16_t qp[MQK ? 3 : 1][REP][MQK ? ATT_MAXHD : 1];

  const size_t head_base = ((size_t)b * p.KV + g) * p.max_pos;
  const char* kbase = (const char*)p.kcache + head_base * hd * sizeof(KT);
  const char* vbase = (const char*)p.vcache + head_base * hd * sizeof(KT);

  // ---- 1. the chunk's K/V loads, first ----
  // Lanes whose position is outside the chunk, or is the entry being
  // appended, read entry 0 of this head instead and discard it.
  u32x4 kr[IT], vr[IT];
  int jj[IT];
  u32x4 kq[GW][4];
  int kpos[GW];
  if constexpr (MQK) {
#pragma unroll
    for (int mm = 0; mm < GW; ++mm) {
      const int j = c0 + 16 * (wave + 4 * mm) + (lane & 15);
      kpos[mm] = j;
      const bool ok = j < c1 && j != pos;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kq[mm][ks] = ld_vec(kbase + ((size_t)(ok ? j : 0) * hd + 32 * ks + 8 * (lane >> 4)) * sizeof(KT));
    }
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int j = c0 + (it * 4 + wave) * PPW + grp;
    jj[it] = j;
    const bool ok = j < c1 && j != pos;
    const size_t off = ((size_t)(ok ? j : 0) * hd + sub * EPL) * sizeof(KT);
    if constexpr (!MQK) kr[it] = ld_vec(kbase + off);
    vr[it] = ld_vec(vbase + off);
  }

  const float* row = p.qkv + (size_t)b * p.ld_qkv;
  const float2* rope = p.rope + (size_t)pos * (hd / 2);
  const bool pair_live = 2 * lane < hd;
  const int pl = pair_live ? 2 * lane : 0;
  const float qscale = 1.0f / sqrtf((float)hd);
  const bool has_new = c1 == L;

  // ---- 2. every other global load, before any of them is used ----
  // q pairs of this wave's heads (hl = wave, wave + 4), the gains, the RoPE
  // entry of the pair, and (workgroup holding pos) the new k pair / v values.
  float qa[2], qc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int hl = min(wave + 4 * i, rep - 1);
    const float* qp = row + (size_t)(g * rep + hl) * hd;
    qa[i] = qp[pl];
    qc[i] = qp[pl + 1];
  }
  const float2 cs = rope[pair_live ? lane : 0];
  float qga = 1.f, qgc = 1.f, kga = 1.f, kgc = 1.f;
  if (p.q_norm) { qga = ElemT<T>::load(p.q_norm, pl); qgc = ElemT<T>::load(p.q_norm, pl + 1); }
  float ka = 0.f, kc = 0.f, vv0 = 0.f, vv1 = 0.f;
  if (has_new && wave == 0) {
    const float* kp = row + (size_t)p.H * hd + (size_t)g * hd;
    ka = kp[pl];
    kc = kp[pl + 1];
    if (p.k_norm) { kga = ElemT<T>::load(p.k_norm, pl); kgc = ElemT<T>::load(p.k_norm, pl + 1); }
  }
  if (has_new && wave == 1) {
    const float* vp = row + (size_t)(p.H + p.KV) * hd + (size_t)g * hd;
    vv0 = vp[lane];
    vv1 = vp[min(lane + 64, hd - 1)];
  }

  // ---- 3. new q heads: QK-norm, RoPE, scale ----
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int hl = wave + 4 * i;
    if (hl >= rep) break;
    float a = pair_live ? qa[i] : 0.f, c = pair_live ? qc[i] : 0.f;
    if (p.q_norm) {
      const float inv = 1.0f / sqrtf(wave_sum(a * a + c * c) / (float)hd + p.eps);
      a = a * inv * qga;
      c = c * inv * qgc;
    }
    if (pair_live) {
      qs[hl][2 * lane] = (a * cs.x - c * cs.y) * qscale;
      qs[hl][2 * lane + 1] = (a * cs.y + c * cs.x) * qscale;
    }
  }
  // ---- new k / v appended by the workgroup holding position pos ----
  if (has_new && wave == 0) {
    float a = pair_live ? ka : 0.f, c = pair_live ? kc : 0.f;
    if (p.k_norm) {
      const float inv = 1.0f / sqrtf(wave_sum(a * a + c * c) / (float)hd + p.eps);
      a = a * inv * kga;
      c = c * inv * kgc;
    }
    if (pair_live) {
      const float ra = ElemT<KT>::round(a * cs.x - c * cs.y);
      const float rc = ElemT<KT>::round(a * cs.y + c * cs.x);
      knew[2 * lane] = ra;
      knew[2 * lane + 1] = rc;
      ElemT<KT>::store(p.kcache, (head_base + pos) * hd + 2 * lane, ra);
      ElemT<KT>::store(p.kcache, (head_base + pos) * hd + 2 * lane + 1, rc);
    }
  } else if (has_new && wave == 1) {
    const float r0 = ElemT<KT>::round(vv0);
    vnew[lane] = r0;
    ElemT<KT>::store(p.vcache, (head_base + pos) * hd + lane, r0);
    if (lane + 64 < hd) {
      const float r1 = ElemT<KT>::round(vv1);
      vnew[lane + 64] = r1;
      ElemT<KT>::store(p.vcache, (head_base + pos) * hd + lane + 64, r1);
    }
  }
  __syncthreads();

  // ---- 4a. scores ----
  if constexpr (MQK) {
    // q as three bf16 planes (rep rows), then 3 MFMAs per 32-dim step
    for (int i = tid; i < rep * ATT_MAXHD; i += DUALAR_WG) {
      const int hl = i / ATT_MAXHD, d = i % ATT_MAXHD;
      const float v = qs[hl][d];
      const uint16_t a0 = f32_to_bf16_rne(v);
      const float r1 = v - bf16_bits_to_f32(a0);
      const uint16_t a1 = f32_to_bf16_rne(r1);
      qp[0][hl][d] = a0;
      qp[1][hl][d] = a1;
      qp[2][hl][d] = f32_to_bf16_rne(r1 - bf16_bits_to_f32(a1));
    }
    __syncthreads();
    const int col = lane & 15;                  // query head (B column)
    const bool live_col = col < rep;
#pragma unroll
    for (int mm = 0; mm < GW; ++mm) {
      att_f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        att_bf16x8 a = __builtin_bit_cast(att_bf16x8, kq[mm][ks]);
        if (kpos[mm] == pos) {
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] = (__bf16)knew[32 * ks + 8 * (lane >> 4) + e];
        }
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          const u32x4 z = {0u, 0u, 0u, 0u};
          const u32x4 bq = live_col ? *(const u32x4*)&qp[q][live_col ? col : 0][32 * ks + 8 * (lane >> 4)] : z;
          acc4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(att_bf16x8, bq), acc4, 0, 0, 0);
        }
      }
      if (live_col) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = c0 + 16 * (wave + 4 * mm) + 4 * (lane >> 4) + r;
          if (j < c1) sc[col][j - c0] = acc4[r];
        }
      }
    }
  } else {
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int j = jj[it];
    float kv[EPL];
    ElemT<KT>::unpack(kr[it], kv);
    if (j == pos) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) kv[e] = knew[sub * EPL + e];
    }
#pragma unroll
    for (int hl = 0; hl < REP; ++hl) {
      if (hl >= rep) break;
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) d = fmaf(qs[hl][sub * EPL + e], kv[e], d);
      d = group_sum(d, LPP);
      if (sub == 0 && j < c1) sc[hl][j - c0] = d;
    }
  }
  }
  __syncthreads();

  // ---- 4b. chunk-local softmax ----
  const int n = c1 - c0;
  for (int hl = wave; hl < rep; hl += 4) {
    float m = -INFINITY;
    for (int i = lane; i < n; i += 64) m = fmaxf(m, sc[hl][i]);
    m = wave_max(m);
    float l = 0.f;
    for (int i = lane; i < n; i += 64) {
      const float e = expf(sc[hl][i] - m);
      sc[hl][i] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) { ml[hl][0] = m; ml[hl][1] = l; }
  }
  __syncthreads();

  // ---- 4c. unnormalised P.V ----
  float acc[REP][EPL];
#pragma unroll
  for (int hl = 0; hl < REP; ++hl)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hl][e] = 0.f;
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int j = jj[it];
    if (j >= c1) continue;
    float vv[EPL];
    ElemT<KT>::unpack(vr[it], vv);
    if (j == pos) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) vv[e] = vnew[sub * EPL + e];
    }
#pragma unroll
    for (int hl = 0; hl < REP; ++hl) {
      if (hl >= rep) break;
      const float pj = sc[hl][j - c0];
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[hl][e] = fmaf(pj, vv[e], acc[hl][e]);
    }
  }
#pragma unroll
  for (int hl = 0; hl < REP; ++hl) {
    if (hl >= rep) break;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      acc[hl][e] = across_groups_sum(acc[hl][e], LPP);
    }
  }
  if (grp == 0) {
    for (int hl = 0; hl < rep; ++hl)
#pragma unroll
      for (int e = 0; e < EPL; ++e) accs[wave][hl][sub * EPL + e] = acc[hl][e];
  }
  __syncthreads();
  for (int i = tid; i < rep * hd; i += DUALAR_WG) {
    const int hl = i / hd, e = i % hd;
    const float o = (accs[0][hl][e] + accs[1][hl][e]) + (accs[2][hl][e] + accs[3][hl][e]);
    if (n_splits == 1) {
      const size_t col = (size_t)(g * rep + hl) * hd + e;
      if (p.out_planes) store_planes(p.out_planes, (size_t)p.B * p.H * hd, (size_t)b * p.H * hd + col, o / ml[hl][1]);
      else p.out[(size_t)b * p.ld_out + col] = o / ml[hl][1];
    } else {
      float* pp = p.part + (((size_t)b * p.H + g * rep + hl) * p.max_splits + checked_index(split, p.max_splits, p.status)) * (hd + 2);
      pp[e] = o;
      if (e == 0) { pp[hd] = ml[hl][0]; pp[hd + 1] = ml[hl][1]; }
    }
  }
}

// Query preparation for the flash-decoding form, grid (B, H + KV), one
// wave: query head hh gets QK-norm, RoPE at the row's position and the
// 1/sqrt(hd) scale, and is stored as three bf16 terms (planes [3][B][H*hd]);
// KV head hh - H gets QK-norm and RoPE on k, and k, v rounded to the cache
// type are appended at the position.  Same arithmetic as the other attention
// kernels, so the cache entries do not depend on the form.
template <typename T, typename KT>
__global__ void __launch_bounds__(64) attn_prep_kernel(AttnParams p) {
  const int b = blockIdx.x, hh = blockIdx.y, lane = threadIdx.x;
  const int pos = row_position(p.pos, p.pos_const, b, p.max_pos, p.status);
  if (pos < 0) return;
  const int hd = p.hd;
  const bool live = 2 * lane < hd;
  const int pl = live ? 2 * lane : 0;
  const float* row = p.qkv + (size_t)b * p.ld_qkv;
  const float2 cs = p.rope[(size_t)pos * (hd / 2) + (live ? lane : 0)];
  if (hh < p.H) {
    const float* qp = row + (size_t)hh * hd;
    float a = live ? qp[pl] : 0.f, c = live ? qp[pl + 1] : 0.f;
    if (p.q_norm) {
      const float inv = 1.0f / sqrtf(wave_sum(a * a + c * c) / (float)hd + p.eps);
      a = a * inv * ElemT<T>::load(p.q_norm, pl);
      c = c * inv * ElemT<T>::load(p.q_norm, pl + 1);
    }
    const float qscale = 1.0f / sqrtf((float)hd);
    if (live) {
      const size_t plane = (size_t)p.B * p.H * hd, at = ((size_t)b * p.H + hh) * hd + pl;
      store_planes(p.q_planes, plane, at, (a * cs.x - c * cs.y) * qscale);
      store_planes(p.q_planes, plane, at + 1, (a * cs.y + c * cs.x) * qscale);
    }
    return;
  }
  const int g = hh - p.H;
  const size_t at = (((size_t)b * p.KV + g) * p.max_pos + pos) * hd;
  const float* kp = row + (size_t)p.H * hd + (size_t)g * hd;
  float a = live ? kp[pl] : 0.f, c = live ? kp[pl + 1] : 0.f;
  if (p.k_norm) {
    const float inv = 1.0f / sqrtf(wave_sum(a * a + c * c) / (float)hd + p.eps);
    a = a * inv * ElemT<T>::load(p.k_norm, pl);
    c = c * inv * ElemT<T>::load(p.k_norm, pl + 1);
  }
  if (live) {
    ElemT<KT>::store(p.kcache, at + pl, ElemT<KT>::round(a * cs.x - c * cs.y));
    ElemT<KT>::store(p.kcache, at + pl + 1, ElemT<KT>::round(a * cs.y + c * cs.x));
  }
  const float* vp = row + (size_t)(p.H + p.KV) * hd + (size_t)g * hd;
  for (int d = lane; d < hd; d += 64) ElemT<KT>::store(p.vcache, at + d, ElemT<KT>::round(vp[d]));
}

// Flash-decoding form for the batched bf16 cache with head_dim 128 (up to
// 64 sequences), after attn_prep_kernel.  The work is balanced across the
// grid like a stream-K product: the 128-position tiles of every (sequence,
// KV head), in (sequence, head, tile) order, are U work units, and
// workgroup g takes q or q + 1 consecutive ones (U = q*G + r, the first r
// workgroups taking one more).  Sequence lengths differ by up to 8x, so
// fixed splits leave most of the chip idle while the longest heads finish.
// A workgroup's units fall into segments of one head; for each it runs the
// tile loop below and writes the segment's (P.V, m, l) to slot
// (g - first workgroup of the head) of the head's partial area, or the
// final output when it holds the whole head.
//
// Tile loop: in each tile wave w owns positions 32w..32w+31 for both the
// scores and P.V, so the waves run their tiles independently (no barrier
// inside the loop).  Per tile a wave
//   - has the tile's K (A-operand layout of v_mfma_f32_16x16x32_bf16:
//     16 positions x 32 dims per step, two 16-position groups) and V (16
//     lanes x 8 dims per position, four positions per load) in one register
//     buffer each;
//   - gets the scores of its 32 positions for the rep query heads from the
//     matrix cores (q as three bf16 terms read straight from the prepared
//     planes: the fp32 product), then issues the next tile's K into the
//     buffer the scores no longer need;
//   - reduces each head's max and sum across the four lanes that hold it and
//     keeps a running max m and sum l per head;
//   - passes the probabilities through a wave-private LDS slot into the P.V
//     layout, rescales its accumulators by e^(m_old - m_new), adds P.V, and
//     issues the next tile's V.
// So each load is in flight behind half a tile of arithmetic.  Two whole
// tiles in flight per wave (two register buffers, 242 registers), and K two
// tiles ahead with V one (210), measured slower.  Positions
// past the segment (and the tile after the last) are loaded from entry 0
// (cached) and left out of the scores and the P.V, so every load of the
// loop is unconditional and the compiler's waits are by count only.
#define FL_TILE 128
#define FL_MAXB 64
#define FL_SLOTS 512   // workgroups of the balanced flash-decoding form (two per compute unit)

// Tiles of each sequence and their exclusive prefix over sequences (times
// KV), one sequence per lane (B <= 64): lanes >= B hold the total.
__device__ __forceinline__ void fl_prefix(const AttnParams& p, int lane, int* E, int* cnt) {
  int n = 0;
  if (lane < p.B) {
    const int pos = row_position(p.pos, p.pos_const, lane, p.max_pos, p.status);
    n = pos < 0 ? 0 : ((pos + 1 + FL_TILE - 1) / FL_TILE) * p.KV;
  }
  int x = n;       // inclusive scan
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  *E = x - n;
  *cnt = n;
}

__device__ __forceinline__ int fl_owner(int u, int q, int r) {
  const int big = r * (q + 1);
  return u < big ? u / (q + 1) : r + (u - big) / q;
}

template <int REP>
__global__ void __launch_bounds__(DUALAR_WG, 2) attn_flash_kernel(AttnParams p, int ng) {
  constexpr int HD = 128, GW = 2, IT = 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane & 15, grp = lane >> 4;     // P.V layout: dims 8*sub.., position 4*it + grp
  const int col = lane & 15;                      // query head (B column) of the score layout
  const bool live_col = col < REP;

  __shared__ __attribute__((aligned(16))) float pw[4][4][8][REP];   // [wave][grp][it][head]
  __shared__ float accs[4][REP][HD];
  __shared__ float mlw[4][REP][2];
  __shared__ __attribute__((aligned(16))) uint16_t qlds[3][REP][HD];  // the segment's q terms

  int E, cnt;
  fl_prefix(p, lane, &E, &cnt);
  const int U = __shfl(E + cnt, 63, 64);
  const int wg = blockIdx.x;
  const int q = U / ng, rr = U % ng;
  const int u0 = wg * q + min(wg, rr), u1 = u0 + q + (wg < rr ? 1 : 0);

  for (int u = u0; u < u1;) {
    // the segment's head
    const int b = __builtin_amdgcn_readfirstlane(__popcll(__ballot(E <= u)) - 1);
    const int Eb = __builtin_amdgcn_readfirstlane(__shfl(E, b, 64));
    const int ntb = __builtin_amdgcn_readfirstlane(__shfl(cnt, b, 64)) / p.KV;
    const int g = (u - Eb) / ntb, t0 = (u - Eb) % ntb;
    const int hfirst = Eb + g * ntb, hend = hfirst + ntb;
    const int useg = min(u1, hend);
    const int pos = row_position(p.pos, p.pos_const, b, p.max_pos, p.status);
    const int c0 = t0 * FL_TILE, c1 = min((useg - hfirst) * FL_TILE, pos + 1);
    const int ntile = useg - u;
    const int slot = wg - fl_owner(hfirst, q, rr);
    const bool whole = u == hfirst && useg == hend;
    u = useg;

    const size_t head_base = ((size_t)b * p.KV + g) * p.max_pos;
    const char* kbase = (const char*)p.kcache + head_base * HD * 2;
    const char* vbase = (const char*)p.vcache + head_base * HD * 2;

    u32x4 ka[GW][4], va[IT];
    auto load_k = [&](u32x4 (&kk)[GW][4], int t) __attribute__((always_inline)) {
      const int base = c0 + t * FL_TILE + 32 * wave;
#pragma unroll
      for (int mm = 0; mm < GW; ++mm) {
        const int j = base + 16 * mm + (lane & 15);
        const size_t e = (size_t)(j < c1 ? j : 0) * HD + 8 * (lane >> 4);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kk[mm][ks] = ld_vec(kbase + (e + 32 * ks) * 2);
      }
    };
    auto load_v = [&](u32x4 (&vv)[IT], int t) __attribute__((always_inline)) {
      const int base = c0 + t * FL_TILE + 32 * wave;
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        const int j = base + 4 * it + grp;
        vv[it] = ld_vec(vbase + ((size_t)(j < c1 ? j : 0) * HD + sub * 8) * 2);
      }
    };
    // the segment's q terms into LDS (3 x REP x 128 bf16, 16 bytes per thread)
    {
      const size_t plane = (size_t)p.B * p.H * HD;
      const uint16_t* qsrc = p.q_planes + ((size_t)b * p.H + g * REP) * HD;
      for (int i = tid; i < 3 * REP * HD / 8; i += DUALAR_WG) {
        const int qq = i / (REP * HD / 8), r = i % (REP * HD / 8);
        *(u32x4*)(&qlds[0][0][0] + (size_t)i * 8) = ld_vec(qsrc + qq * plane + (size_t)r * 8);
      }
    }
    load_k(ka, 0);
    load_v(va, 0);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    float m_run = -INFINITY, l_run = 0.f;     // for head `col` (lanes with col < REP)
    float acc[REP][8];
#pragma unroll
    for (int hl = 0; hl < REP; ++hl)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hl][e] = 0.f;

    auto tile = [&](u32x4 (&kk)[GW][4], u32x4 (&vv)[IT], int t) __attribute__((always_inline)) {
      const int base = c0 + t * FL_TILE + 32 * wave;
      float sv[GW][4];
#pragma unroll
      for (int mm = 0; mm < GW; ++mm) {
        att_f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const att_bf16x8 a = __builtin_bit_cast(att_bf16x8, kk[mm][ks]);
#pragma unroll
          for (int qq = 0; qq < 3; ++qq) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            const u32x4 bq = live_col ? *(const u32x4*)&qlds[qq][live_col ? col : 0][32 * ks + 8 * (lane >> 4)] : z;
            acc4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(att_bf16x8, bq), acc4, 0, 0, 0);
          }
        }
        // acc4[r]: position base + 16 mm + 4 (lane >> 4) + r, head col
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[mm][r] = base + 16 * mm + 4 * (lane >> 4) + r < c1 ? acc4[r] : -INFINITY;
      }
      load_k(kk, t + 1);                      // the scores are done with this buffer
      float mt = -INFINITY;
#pragma unroll
      for (int mm = 0; mm < GW; ++mm)
#pragma unroll
        for (int r = 0; r < 4; ++r) mt = fmaxf(mt, sv[mm][r]);
      mt = max_xor32(max_xor16(mt));          // over the wave's 32 positions of head col
      const float m_new = fmaxf(m_run, mt);
      // a wave whose positions so far are all past the segment keeps m = -inf, p = 0
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      float ls = 0.f;
#pragma unroll
      for (int mm = 0; mm < GW; ++mm)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pv = expf(sv[mm][r] - m_use);
          ls += pv;
          const int qp = 16 * mm + 4 * (lane >> 4) + r;        // position in the wave's 32
          if (live_col) pw[wave][qp & 3][qp >> 2][col] = pv;
        }
      ls = add_xor32(add_xor16(ls));
      const float cf = expf(m_run - m_use);   // 0 while m_run = -inf
      l_run = l_run * cf + ls;
      m_run = m_new;
#pragma unroll
      for (int hl = 0; hl < REP; ++hl) {       // lane hl holds head hl
        const float ch = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(cf), hl));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hl][e] *= ch;
      }
      __builtin_amdgcn_wave_barrier();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const float* pr = &pw[wave][grp][0][0];
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        // past the segment: p = 0, and the entry loaded in its place may be
        // one that was never written (a depth-cache slot on the first frame)
        if (base + 4 * it + grp >= c1) continue;
        float vf[8];
        ElemT<bf16_t>::unpack(vv[it], vf);
#pragma unroll
        for (int hl = 0; hl < REP; ++hl) {
          const float pj = pr[it * REP + hl];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[hl][e] = fmaf(pj, vf[e], acc[hl][e]);
        }
      }
      load_v(vv, t + 1);                        // and the P.V with this one
      __builtin_amdgcn_wave_barrier();
    };

    for (int t = 0; t < ntile; ++t) tile(ka, va, t);

    // ---- combine: the four position groups of each wave, then the waves ----
#pragma unroll
    for (int hl = 0; hl < REP; ++hl)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hl][e] = across_groups_sum(acc[hl][e], 16);
    if (grp == 0) {
#pragma unroll
      for (int hl = 0; hl < REP; ++hl)
#pragma unroll
        for (int e = 0; e < 8; ++e) accs[wave][hl][sub * 8 + e] = acc[hl][e];
    }
    if (lane < REP) { mlw[wave][lane][0] = m_run; mlw[wave][lane][1] = l_run; }
    __syncthreads();
    for (int i = tid; i < REP * HD; i += DUALAR_WG) {
      const int hl = i / HD, e = i % HD;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, mlw[w][hl][0]);
      float o = 0.f, l = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = mlw[w][hl][0] == -INFINITY ? 0.f : expf(mlw[w][hl][0] - M);
        o += f * accs[w][hl][e];
        l += f * mlw[w][hl][1];
      }
      if (whole) {
        const size_t colx = (size_t)(g * REP + hl) * HD + e;
        if (p.out_planes) store_planes(p.out_planes, (size_t)p.B * p.H * HD, (size_t)b * p.H * HD + colx, o / l);
        else p.out[(size_t)b * p.ld_out + colx] = o / l;
      } else {
        float* pp = p.part + (((size_t)b * p.H + g * REP + hl) * p.max_splits + checked_index(slot, p.max_splits, p.status)) * (HD + 2);
        pp[e] = o;
        if (e == 0) { pp[HD] = M; pp[HD + 1] = l; }
      }
    }
    __syncthreads();     // accs / mlw are reused by the next segment
  }
}

// Merge for the balanced form: grid (B, H), the slots of head (b, h / rep)
// are those of the workgroups its tiles went to (none to merge when one
// workgroup held the whole head).
__global__ void __launch_bounds__(128) attn_flash_merge_kernel(AttnParams p, int ng) {
  const int b = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int pos = row_position(p.pos, p.pos_const, b, p.max_pos, p.status);
  if (pos < 0) return;
  int E, cnt;
  fl_prefix(p, lane, &E, &cnt);
  const int U = __shfl(E + cnt, 63, 64);
  const int q = U / ng, rr = U % ng;
  const int Eb = __shfl(E, b, 64), ntb = __shfl(cnt, b, 64) / p.KV;
  const int g = h / (p.H / p.KV);
  const int hfirst = Eb + g * ntb;
  const int n_slots = fl_owner(hfirst + ntb - 1, q, rr) - fl_owner(hfirst, q, rr) + 1;
  if (n_slots == 1) return;                    // the flash kernel wrote o
  const int hd = p.hd;
  const float* pp = p.part + ((size_t)b * p.H + h) * p.max_splits * (hd + 2);
  // a head's tiles can go to as many workgroups as the grid has (one tile
  // each when a few long heads make up the whole walk)
  __shared__ float wsh[FL_SLOTS];
  __shared__ float red[2];
  __shared__ float lred[2];
  float mloc = -INFINITY;
  for (int s = t; s < n_slots; s += 128) mloc = fmaxf(mloc, pp[(size_t)s * (hd + 2) + hd]);
  mloc = wave_max(mloc);
  if (lane == 0) red[wv] = mloc;
  __syncthreads();
  const float M = fmaxf(red[0], red[1]);
  float lloc = 0.f;
  for (int s = t; s < n_slots; s += 128) {
    const float* qv = pp + (size_t)s * (hd + 2);
    const float w = expf(qv[hd] - M);
    wsh[checked_index(s, FL_SLOTS, p.status)] = w;
    lloc += qv[hd + 1] * w;
  }
  lloc = wave_sum(lloc);
  if (lane == 0) lred[wv] = lloc;
  __syncthreads();
  const float lsum = lred[0] + lred[1];
  if (t >= hd) return;
  float o = 0.f;
  for (int s0 = 0; s0 < n_slots; s0 += 8) {
    float ov[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) ov[i] = pp[(size_t)min(s0 + i, n_slots - 1) * (hd + 2) + t];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (s0 + i < n_slots) o = fmaf(ov[i], wsh[s0 + i], o);
  }
  if (p.out_planes) store_planes(p.out_planes, (size_t)p.B * p.H * hd, (size_t)b * p.H * hd + (size_t)h * hd + t, o / lsum);
  else p.out[(size_t)b * p.ld_out + (size_t)h * hd + t] = o / lsum;
}

// One workgroup per (sequence, query head) merges the split partials:
// M = max_s m_s and the weights w_s = e^(m_s - M) are computed for all splits
// at once (one split per thread), then o[e] = sum_s w_s o_s[e] / sum_s w_s l_s
// with the o_s loads issued 16 at a time.  Fixed summation order.
#define MERGE_T 128
__global__ void __launch_bounds__(MERGE_T) attn_merge_kernel(AttnParams p) {
  const int b = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int pos = row_position(p.pos, p.pos_const, b, p.max_pos, p.status);
  if (pos < 0) return;
  const int n_splits = (pos + 1 + p.chunk - 1) / p.chunk;
  if (n_splits == 1) return;                   // the partial kernel wrote o
  const int hd = p.hd;
  const float* pp = p.part + ((size_t)b * p.H + h) * p.max_splits * (hd + 2);
  __shared__ float wsh[ATT_MAXSPLIT];
  __shared__ float red[2];
  __shared__ float lred[2];
  // 1. weights of every split
  float mloc = -INFINITY;
  for (int s = t; s < n_splits; s += MERGE_T) mloc = fmaxf(mloc, pp[(size_t)s * (hd + 2) + hd]);
  mloc = wave_max(mloc);
  if (lane == 0) red[wv] = mloc;
  __syncthreads();
  const float M = fmaxf(red[0], red[1]);
  float lloc = 0.f;
  for (int s = t; s < n_splits; s += MERGE_T) {
    const float* q = pp + (size_t)s * (hd + 2);
    const float w = expf(q[hd] - M);
    wsh[s] = w;
    lloc += q[hd + 1] * w;
  }
  lloc = wave_sum(lloc);
  if (lane == 0) lred[wv] = lloc;
  __syncthreads();
  const float lsum = lred[0] + lred[1];
  // 2. weighted sum of the partial outputs
  if (t >= hd) return;
  float o = 0.f;
  for (int s0 = 0; s0 < n_splits; s0 += 16) {
    float ov[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) ov[i] = pp[(size_t)min(s0 + i, n_splits - 1) * (hd + 2) + t];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (s0 + i < n_splits) o = fmaf(ov[i], wsh[s0 + i], o);
  }
  if (p.out_planes) store_planes(p.out_planes, (size_t)p.B * p.H * hd, (size_t)b * p.H * hd + (size_t)h * hd + t, o / lsum);
  else p.out[(size_t)b * p.ld_out + (size_t)h * hd + t] = o / lsum;
}

// The plain merge alone, for a caller that ran its own split kernel with the
// same partial layout (one slot of hd + 2 floats per head and split).
hipError_t launch_attn_merge(const AttnParams& p, hipStream_t s) {
  if (p.max_splits <= 1) return hipSuccess;   // the split kernel wrote o
  hipLaunchKernelGGL(attn_merge_kernel, dim3(p.B, p.H), dim3(MERGE_T), 0, s, p);
  return hipGetLastError();
}

int attn_chunk(int kv_esz, int hd, int it) {
  const int lpp = hd * kv_esz / 16;
  return 4 * (64 / lpp) * it;
}


// Batched attention over a short cache (at most 16 positions: the fast AR's
// depth cache), bf16 cache, head_dim 128, 4 query heads per KV head, after
// the QKV finish (or attn_prep_kernel) has written q as three bf16 terms and
// appended k, v.  One wave per (row, KV head): K rows and the q terms go
// straight into the matrix-core operands (positions as A, query heads as B),
// softmax in registers across the four lane groups of a column, then P.V in
// the dim layout (lane l: dims 2l, 2l+1 of the 4 heads) with the output
// written as three bf16 planes (or fp32).  Same arithmetic steps as the
// other decode attention kernels.
__global__ void __launch_bounds__(64) attn_depth_kernel(AttnParams p) {
  constexpr int HD = 128, REP = 4, MAXL = 16;
  __shared__ __attribute__((aligned(16))) float pe[REP][MAXL];
  const int lane = threadIdx.x;
  const int b = blockIdx.x / p.KV, g = blockIdx.x % p.KV;
  const int pos = row_position(p.pos, p.pos_const, b, p.max_pos, p.status);
  if (pos < 0) return;                        // inactive row
  const int L = pos + 1;
  const int jm = lane & 15, kq = lane >> 4;
  const size_t head_base = ((size_t)b * p.KV + g) * p.max_pos;
  const char* kbase = (const char*)p.kcache + head_base * HD * sizeof(bf16_t);
  const uint32_t* vbase = (const uint32_t*)((const char*)p.vcache + head_base * HD * sizeof(bf16_t));
  // operands: K (A, positions past the context read position 0 and are
  // masked), the q terms (B, column n = query head n % 4), V (dim layout)
  u32x4 ka[4], qb[3][4];
  {
    const int jl = jm < L ? jm : 0;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) ka[ks] = ld_vec(kbase + ((size_t)jl * HD + 32 * ks + 8 * kq) * sizeof(bf16_t));
    const size_t plane = (size_t)p.B * p.H * HD;
    const uint16_t* qsrc = p.q_planes + ((size_t)b * p.H + g * REP + (jm & 3)) * HD + 8 * kq;
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qb[t][ks] = ld_vec(qsrc + t * plane + 32 * ks);
  }
  uint32_t vc[MAXL];
#pragma unroll
  for (int jj = 0; jj < MAXL; ++jj) {
    vc[jj] = 0u;
    if (jj < L) vc[jj] = vbase[(size_t)jj * (HD / 2) + lane];
  }
  att_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int t = 0; t < 3; ++t)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(att_bf16x8, ka[ks]),
                                                    __builtin_bit_cast(att_bf16x8, qb[t][ks]), acc, 0, 0, 0);
  // lane l holds S[position 4 (l / 16) + r][head (l % 16) % 4]
  float sv[4];
  float m = -INFINITY;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sv[r] = 4 * kq + r < L ? acc[r] : -INFINITY;
    m = fmaxf(m, sv[r]);
  }
  m = max_xor32(max_xor16(m));
  float l = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    sv[r] = 4 * kq + r < L ? expf(sv[r] - m) : 0.f;
    l += sv[r];
  }
  l = add_xor32(add_xor16(l));
  if (jm < REP) {
#pragma unroll
    for (int r = 0; r < 4; ++r) pe[jm][4 * kq + r] = sv[r] / l;
  }
  __builtin_amdgcn_wave_barrier();
  float o[REP][2];
#pragma unroll
  for (int h = 0; h < REP; ++h) o[h][0] = o[h][1] = 0.f;
#pragma unroll
  for (int q4 = 0; q4 < MAXL / 4; ++q4) {
    if (4 * q4 < L) {
      float4 pv[REP];
#pragma unroll
      for (int h = 0; h < REP; ++h) pv[h] = *(const float4*)&pe[h][4 * q4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jj = 4 * q4 + r;
        const float va = bf16_bits_to_f32(vc[jj] & 0xffffu), vb = bf16_bits_to_f32(vc[jj] >> 16);
#pragma unroll
        for (int h = 0; h < REP; ++h) {
          const float pj = r == 0 ? pv[h].x : r == 1 ? pv[h].y : r == 2 ? pv[h].z : pv[h].w;
          o[h][0] = fmaf(pj, va, o[h][0]);
          o[h][1] = fmaf(pj, vb, o[h][1]);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < REP; ++h) {
    const size_t col = (size_t)(g * REP + h) * HD + 2 * lane;
    if (p.out_planes) {
      const size_t plane = (size_t)p.B * p.H * HD, at = (size_t)b * p.H * HD + col;
      store_planes(p.out_planes, plane, at, o[h][0]);
      store_planes(p.out_planes, plane, at + 1, o[h][1]);
    } else {
      p.out[(size_t)b * p.ld_out + col] = o[h][0];
      p.out[(size_t)b * p.ld_out + col + 1] = o[h][1];
    }
  }
}

template <typename T, typename KT> hipError_t launch_attn(const AttnParams& p0, hipStream_t s) {
  AttnParams p = p0;
  const int rep = p.H / p.KV;
  if constexpr (sizeof(KT) == 2) {
    // the balanced flash-decoding form: bf16 cache, head_dim 128, batched
    // contexts of at most 16 positions (the depth cache): one wave per (row, KV head)
    if (!p.no_merge && p.hd == 128 && p.it >= 8 && p.q_planes && rep == 4 && p.lmax <= 16) {
      if (!p.prepped) hipLaunchKernelGGL((attn_prep_kernel<T, KT>), dim3(p.B, p.H + p.KV), dim3(64), 0, s, p);
      hipLaunchKernelGGL(attn_depth_kernel, dim3(p.B * p.KV), dim3(64), 0, s, p);
      return hipGetLastError();
    }
    if (!p.no_merge && p.hd == 128 && p.it >= 8 && p.q_planes && p.B <= FL_MAXB && (rep == 1 || rep == 2 || rep == 4)) {
      const int nt_max = (p.lmax + FL_TILE - 1) / FL_TILE;
      // upper bound of the units: every row at lmax
      const long long u_max = (long long)p.B * p.KV * nt_max;
      const int ng = (int)std::min<long long>(FL_SLOTS, std::max<long long>(1, u_max));
      // slots per head: at most the head's tiles + 1 (a workgroup holds >= 1 unit
      // whenever U >= ng; with U < ng some hold none and the rest one each)
      p.max_splits = nt_max + 1;
      if (!p.prepped) hipLaunchKernelGGL((attn_prep_kernel<T, KT>), dim3(p.B, p.H + p.KV), dim3(64), 0, s, p);
      switch (rep) {
        case 1: hipLaunchKernelGGL((attn_flash_kernel<1>), dim3(ng), dim3(DUALAR_WG), 0, s, p, ng); break;
        case 2: hipLaunchKernelGGL((attn_flash_kernel<2>), dim3(ng), dim3(DUALAR_WG), 0, s, p, ng); break;
        default: hipLaunchKernelGGL((attn_flash_kernel<4>), dim3(ng), dim3(DUALAR_WG), 0, s, p, ng); break;
      }
      // with every context inside one tile (the fast AR's depth cache) each
      // head is one unit in one workgroup, which writes o itself: no merge
      if (nt_max > 1) hipLaunchKernelGGL(attn_flash_merge_kernel, dim3(p.B, p.H), dim3(128), 0, s, p, ng);
      return hipGetLastError();
    }
  }
  p.chunk = attn_chunk((int)sizeof(KT), p.hd, p.it);
  p.max_splits = (p.lmax + p.chunk - 1) / p.chunk;
  dim3 grid(p.max_splits, p.KV, p.B);
  // the matrix-core score path: bf16 cache, head_dim 128, 4+ loads per lane
  const bool mqk = sizeof(KT) == 2 && p.hd == 128 && p.it >= 4;
#define ATT_GO(IT, REP)                                                                                      \
  do {                                                                                                       \
    if constexpr (sizeof(KT) == 2 && IT >= 4) {                                                              \
      if (mqk) { hipLaunchKernelGGL((attn_partial_kernel<T, KT, IT, REP, true>), grid, dim3(DUALAR_WG), 0, s, p); break; } \
    }                                                                                                        \
    hipLaunchKernelGGL((attn_partial_kernel<T, KT, IT, REP>), grid, dim3(DUALAR_WG), 0, s, p);               \
  } while (0)
#define ATT_REP(IT)                       \
  if (rep == 1) ATT_GO(IT, 1);            \
  else if (rep == 2) ATT_GO(IT, 2);       \
  else if (rep == 4) ATT_GO(IT, 4);       \
  else ATT_GO(IT, 8);
  if (p.it == 2) { ATT_REP(2) }
  else if (p.it == 4) { ATT_REP(4) }
  else if (p.it == 16) { ATT_REP(16) }
  else { ATT_REP(8) }
#undef ATT_REP
#undef ATT_GO
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.max_splits == 1 || p.no_merge) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(p.B, p.H), dim3(MERGE_T), 0, s, p);
  return hipGetLastError();
}

template hipError_t launch_attn<float, float>(const AttnParams&, hipStream_t);
template hipError_t launch_attn<float, bf16_t>(const AttnParams&, hipStream_t);
template hipError_t launch_attn<bf16_t, float>(const AttnParams&, hipStream_t);
template hipError_t launch_attn<bf16_t, bf16_t>(const AttnParams&, hipStream_t);
