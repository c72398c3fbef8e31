// GQA decode attention for one new position per sequence (slow AR over the
// time cache, fast AR over the N-slot depth cache).
//
// Grid (split, kv_head, batch).  A workgroup takes `chunk` consecutive cache
// positions of one KV head and the rep = H/KV query heads that share it
// (contiguous grouping: query head h uses KV head h / rep).  It
//   1. applies QK-norm (per-head RMSNorm, one [hd] gain) and RoPE to the new
//      q heads, folding in the 1/sqrt(hd) score scale;
//   2. if its chunk holds the new position, normalises/rotates the new k,
//      rounds k and v to the cache type and appends them;
//   3. computes scores, a chunk-local softmax (max m, sum l) and the
//      unnormalised P.V, and writes (o, m, l) partials;
//   4. the last workgroup of a (sequence, KV head) to finish (atomic
//      counter) merges the partials: o = sum_s e^(m_s-M) o_s / sum_s e^(m_s-M) l_s.
// K/V rows are read with 16-byte lane loads: LPP = hd*sizeof(KT)/16 lanes
// cover one position, so a wave reads 64/LPP positions per load.
#include "common.h"
#include "internal.h"

#define ATT_MAXREP 8
#define ATT_MAXHD 128
#define ATT_MAXCHUNK 256

template <typename T, typename KT>
__global__ void __launch_bounds__(DUALAR_WG) attn_kernel(AttnParams p) {
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int pos = p.pos ? p.pos[b] : p.pos_const;
  if (pos < 0) return;                      // inactive row (prefill padding)
  const int L = pos + 1;
  const int n_splits = (L + p.chunk - 1) / p.chunk;
  if (split >= n_splits) return;
  const int c0 = split * p.chunk, c1 = min(c0 + p.chunk, L);
  const int hd = p.hd, rep = p.H / p.KV;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  __shared__ float qs[ATT_MAXREP][ATT_MAXHD];
  __shared__ float knew[ATT_MAXHD], vnew[ATT_MAXHD];
  __shared__ float sc[ATT_MAXREP][ATT_MAXCHUNK];
  __shared__ float accs[4][ATT_MAXREP][ATT_MAXHD];
  __shared__ float ml[ATT_MAXREP][2];
  __shared__ int is_last;

  const float* row = p.qkv + (size_t)b * p.ld_qkv;
  const float2* rope = p.rope + (size_t)pos * (hd / 2);
  const bool pair_live = 2 * lane < hd;
  const float qscale = 1.0f / sqrtf((float)hd);

  // ---- 1. new q heads: QK-norm, RoPE, scale ----
  for (int hl = wave; hl < rep; hl += 4) {
    const float* qp = row + (size_t)(g * rep + hl) * hd;
    float a = pair_live ? qp[2 * lane] : 0.f, c = pair_live ? qp[2 * lane + 1] : 0.f;
    if (p.q_norm) {
      const float inv = 1.0f / sqrtf(wave_sum(a * a + c * c) / (float)hd + p.eps);
      if (pair_live) {
        a = a * inv * ElemT<T>::load(p.q_norm, 2 * lane);
        c = c * inv * ElemT<T>::load(p.q_norm, 2 * lane + 1);
      }
    }
    if (pair_live) {
      const float2 cs = rope[lane];
      qs[hl][2 * lane] = (a * cs.x - c * cs.y) * qscale;
      qs[hl][2 * lane + 1] = (a * cs.y + c * cs.x) * qscale;
    }
  }
  // ---- 2. new k / v (only the workgroup holding position pos) ----
  const size_t head_base = ((size_t)b * p.KV + g) * p.max_pos;
  if (c1 == L) {
    if (wave == 0) {
      const float* kp = row + (size_t)p.H * hd + (size_t)g * hd;
      float a = pair_live ? kp[2 * lane] : 0.f, c = pair_live ? kp[2 * lane + 1] : 0.f;
      if (p.k_norm) {
        const float inv = 1.0f / sqrtf(wave_sum(a * a + c * c) / (float)hd + p.eps);
        if (pair_live) {
          a = a * inv * ElemT<T>::load(p.k_norm, 2 * lane);
          c = c * inv * ElemT<T>::load(p.k_norm, 2 * lane + 1);
        }
      }
      if (pair_live) {
        const float2 cs = rope[lane];
        const float ra = ElemT<KT>::round(a * cs.x - c * cs.y);
        const float rc = ElemT<KT>::round(a * cs.y + c * cs.x);
        knew[2 * lane] = ra;
        knew[2 * lane + 1] = rc;
        ElemT<KT>::store(p.kcache, (head_base + pos) * hd + 2 * lane, ra);
        ElemT<KT>::store(p.kcache, (head_base + pos) * hd + 2 * lane + 1, rc);
      }
    } else if (wave == 1) {
      const float* vp = row + (size_t)(p.H + p.KV) * hd + (size_t)g * hd;
      for (int e = lane; e < hd; e += 64) {
        const float v = ElemT<KT>::round(vp[e]);
        vnew[e] = v;
        ElemT<KT>::store(p.vcache, (head_base + pos) * hd + e, v);
      }
    }
  }
  __syncthreads();

  // ---- 3a. scores ----
  constexpr int EPL = ElemT<KT>::EPV;
  const int LPP = hd / EPL;
  const int PPW = 64 / LPP;
  const int sub = lane % LPP, grp = lane / LPP;
  const char* kbase = (const char*)p.kcache + head_base * hd * sizeof(KT);
  const char* vbase = (const char*)p.vcache + head_base * hd * sizeof(KT);
  for (int j0 = c0 + wave * PPW; j0 < c1; j0 += 4 * PPW) {
    const int j = j0 + grp;
    float kv[EPL];
    if (j < c1 && j != pos) {
      ElemT<KT>::unpack(ld_vec(kbase + ((size_t)j * hd + sub * EPL) * sizeof(KT)), kv);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) kv[e] = (j == pos) ? knew[sub * EPL + e] : 0.f;
    }
#pragma unroll
    for (int hl = 0; hl < ATT_MAXREP; ++hl) {
      if (hl >= rep) break;
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) d = fmaf(qs[hl][sub * EPL + e], kv[e], d);
      d = group_sum(d, LPP);
      if (sub == 0 && j < c1) sc[hl][j - c0] = d;
    }
  }
  __syncthreads();

  // ---- 3b. chunk-local softmax ----
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

  // ---- 3c. unnormalised P.V ----
  float acc[ATT_MAXREP][EPL];
#pragma unroll
  for (int hl = 0; hl < ATT_MAXREP; ++hl)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[hl][e] = 0.f;
  for (int j0 = c0 + wave * PPW; j0 < c1; j0 += 4 * PPW) {
    const int j = j0 + grp;
    if (j < c1) {
      float vv[EPL];
      if (j != pos) {
        ElemT<KT>::unpack(ld_vec(vbase + ((size_t)j * hd + sub * EPL) * sizeof(KT)), vv);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vv[e] = vnew[sub * EPL + e];
      }
#pragma unroll
      for (int hl = 0; hl < ATT_MAXREP; ++hl) {
        if (hl >= rep) break;
        const float pj = sc[hl][j - c0];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hl][e] = fmaf(pj, vv[e], acc[hl][e]);
      }
    }
  }
#pragma unroll
  for (int hl = 0; hl < ATT_MAXREP; ++hl) {
    if (hl >= rep) break;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      float v = acc[hl][e];
      for (int o = LPP; o < 64; o <<= 1) v += __shfl_xor(v, o);
      acc[hl][e] = v;
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
    float* pp = p.part + (((size_t)b * p.H + g * rep + hl) * p.max_splits + split) * (hd + 2);
    pp[e] = o;
    if (e == 0) { pp[hd] = ml[hl][0]; pp[hd + 1] = ml[hl][1]; }
  }

  // ---- 4. last workgroup merges the splits ----
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned prev = atomicAdd(&p.counters[b * p.KV + g], 1u);
    is_last = (prev == (unsigned)(n_splits - 1));
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  for (int i = tid; i < rep * hd; i += DUALAR_WG) {
    const int hl = i / hd, e = i % hd;
    const int h = g * rep + hl;
    const float* pp = p.part + ((size_t)b * p.H + h) * p.max_splits * (hd + 2);
    float M = -INFINITY;
    for (int s = 0; s < n_splits; ++s) M = fmaxf(M, pp[(size_t)s * (hd + 2) + hd]);
    float lsum = 0.f, o = 0.f;
    for (int s = 0; s < n_splits; ++s) {
      const float* q = pp + (size_t)s * (hd + 2);
      const float w = expf(q[hd] - M);
      lsum = fmaf(q[hd + 1], w, lsum);
      o = fmaf(q[e], w, o);
    }
    p.out[(size_t)b * p.ld_out + (size_t)h * hd + e] = o / lsum;
  }
  if (tid == 0) atomicExch(&p.counters[b * p.KV + g], 0u);
}

template <typename T, typename KT> hipError_t launch_attn(const AttnParams& p, hipStream_t s) {
  dim3 grid(p.max_splits, p.KV, p.B);
  hipLaunchKernelGGL((attn_kernel<T, KT>), grid, dim3(DUALAR_WG), 0, s, p);
  return hipGetLastError();
}

template hipError_t launch_attn<float, float>(const AttnParams&, hipStream_t);
template hipError_t launch_attn<float, bf16_t>(const AttnParams&, hipStream_t);
template hipError_t launch_attn<bf16_t, float>(const AttnParams&, hipStream_t);
template hipError_t launch_attn<bf16_t, bf16_t>(const AttnParams&, hipStream_t);
