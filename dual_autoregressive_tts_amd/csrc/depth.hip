// Teacher-forced fast AR: the fast layers over every (slow hidden state,
// frame codes) pair at once, as in the training forward of [P1] "Fast
// Transformer: The Codebook Decoder" (Step 3: the hidden state followed by
// the codebook embeddings, through the fast layers, fast_norm and
// fast_output).  Rows r = i*N + k hold depth position k of pair i: the
// pair's slow hidden state at k = 0, E_F[q^(k-1)] at k = 1..N-1.  The
// products run over all n*N rows like a prefill step; attention is causal
// along depth inside each pair.
//
// depth_attn_kernel, grid (n, KV), 256 threads: the workgroup takes pair i
// and KV head g with its REP query heads.  Each of the pair's N rows gets
// the decode arithmetic: QK-norm (one [hd] gain) and RoPE at position k on
// q and k, the 1/sqrt(hd) scale on q, k and v rounded to the cache type (the
// values the incremental fast passes keep in their depth cache), all in
// LDS.  Then, per query head (one wave): lane t takes the (query, key) pairs
// t and t + 64 of the N x N score matrix (full 128-wide dots; keys after
// the query are masked), lane kq < N turns row kq into probabilities, and
// lane l sums P.V for dims 2l, 2l+1 of every row.  LDS rows are padded so
// that lanes reading different rows at one dim hit different banks.
#include "common.h"
#include "internal.h"

#define DEPTH_MAXN 11     // N*N score pairs fit two per lane
#define DEPTH_MAXREP 8
#define DEPTH_MAXHD 128

template <typename T>
__global__ void __launch_bounds__(DUALAR_WG) tf_embed_kernel(TfParams p) {
  const int r = blockIdx.x, i = r / p.N, k = r % p.N;
  float* x = p.x + (size_t)r * p.dim;
  if (k == 0) {
    const float* h = p.hidden + (size_t)i * p.dim;
    for (int d = threadIdx.x; d < p.dim; d += DUALAR_WG) x[d] = h[d];
    return;
  }
  int q = p.codes[(size_t)i * p.N + k - 1];
  if (q < 0 || q >= p.C) {          // out-of-range code: latched, row 0 of the table used
    if (threadIdx.x == 0) atomicOr(p.status, ST_BAD_TOKEN);
    q = 0;
  }
  for (int d = threadIdx.x; d < p.dim; d += DUALAR_WG) x[d] = ElemT<T>::load(p.fast_emb, (size_t)q * p.dim + d);
}

template <typename T, typename KT, int REP>
__global__ void __launch_bounds__(256) depth_attn_kernel(PrefillParams p) {
  constexpr int RS = DEPTH_MAXHD + 1;   // padded row stride
  const int i = blockIdx.x, g = blockIdx.y;
  const int N = p.C, hd = p.hd;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float ks[DEPTH_MAXN * RS];
  __shared__ float vs[DEPTH_MAXN * DEPTH_MAXHD];
  __shared__ float qs[REP][DEPTH_MAXN * RS];
  __shared__ float ps[4][DEPTH_MAXN][DEPTH_MAXN + 1];

  // ---- prep: N rows x (k, v, REP q heads) vectors, one wave per vector ----
  const bool live = 2 * lane < hd;
  const int pl = live ? 2 * lane : 0;
  const float qscale = 1.0f / sqrtf((float)hd);
  const int nvec = N * (2 + REP);
  for (int t = wave; t < nvec; t += 4) {
    const int k = t / (2 + REP), kind = t % (2 + REP);   // 0: k, 1: v, 2..: q head kind - 2
    const float* row = p.qkv + (size_t)(i * N + k) * p.ld_qkv;
    if (kind == 1) {
      const float* vp = row + (size_t)(p.H + p.KV) * hd + (size_t)g * hd;
      if (live) {
        vs[k * DEPTH_MAXHD + pl] = ElemT<KT>::round(vp[pl]);
        vs[k * DEPTH_MAXHD + pl + 1] = ElemT<KT>::round(vp[pl + 1]);
      }
      continue;
    }
    const int hl = kind - 2;
    const float* src = kind == 0 ? row + (size_t)p.H * hd + (size_t)g * hd : row + (size_t)(g * REP + hl) * hd;
    const void* gain = kind == 0 ? p.k_norm : p.q_norm;
    float a = live ? src[pl] : 0.f, c = live ? src[pl + 1] : 0.f;
    if (gain) {
      const float inv = 1.0f / sqrtf(wave_sum(a * a + c * c) / (float)hd + p.eps);
      a = a * inv * ElemT<T>::load(gain, pl);
      c = c * inv * ElemT<T>::load(gain, pl + 1);
    }
    const float2 cs = p.rope[(size_t)k * (hd / 2) + (live ? lane : 0)];
    const float ra = a * cs.x - c * cs.y, rc = a * cs.y + c * cs.x;
    if (!live) continue;
    if (kind == 0) {
      ks[k * RS + pl] = ElemT<KT>::round(ra);
      ks[k * RS + pl + 1] = ElemT<KT>::round(rc);
    } else {
      qs[hl][k * RS + pl] = ra * qscale;
      qs[hl][k * RS + pl + 1] = rc * qscale;
    }
  }
  __syncthreads();

  // ---- causal attention along depth, one wave per query head ----
  for (int hl = wave; hl < REP; hl += 4) {
    const float* q = qs[hl];
    // scores of pairs t = lane, lane + 64: query t / N, key t % N
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = lane + 64 * u;
      if (t >= N * N) continue;
      const int kq = t / N, j = t % N;
      float s = -INFINITY;
      if (j <= kq) {
        float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
        for (int e = 0; e < hd; e += 4) {
          d0 = fmaf(q[kq * RS + e], ks[j * RS + e], d0);
          d1 = fmaf(q[kq * RS + e + 1], ks[j * RS + e + 1], d1);
          d2 = fmaf(q[kq * RS + e + 2], ks[j * RS + e + 2], d2);
          d3 = fmaf(q[kq * RS + e + 3], ks[j * RS + e + 3], d3);
        }
        s = (d0 + d1) + (d2 + d3);
      }
      ps[wave][kq][j] = s;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    if (lane < N) {   // row lane: probabilities of keys 0..lane
      float m = -INFINITY;
      for (int j = 0; j <= lane; ++j) m = fmaxf(m, ps[wave][lane][j]);
      float l = 0.f;
      for (int j = 0; j <= lane; ++j) {
        const float e = expf(ps[wave][lane][j] - m);
        ps[wave][lane][j] = e;
        l += e;
      }
      const float inv = 1.0f / l;
      for (int j = 0; j <= lane; ++j) ps[wave][lane][j] *= inv;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    if (live) {
      const size_t col = (size_t)(g * REP + hl) * hd + pl;
      for (int kq = 0; kq < N; ++kq) {
        float o0 = 0.f, o1 = 0.f;
        for (int j = 0; j <= kq; ++j) {
          const float pj = ps[wave][kq][j];
          o0 = fmaf(pj, vs[j * DEPTH_MAXHD + pl], o0);
          o1 = fmaf(pj, vs[j * DEPTH_MAXHD + pl + 1], o1);
        }
        const size_t r = (size_t)i * N + kq;
        if (p.out_planes) {
          store_planes(p.out_planes, (size_t)p.R * p.H * hd, r * p.H * hd + col, o0);
          store_planes(p.out_planes, (size_t)p.R * p.H * hd, r * p.H * hd + col + 1, o1);
        } else {
          p.out[r * p.ld_out + col] = o0;
          p.out[r * p.ld_out + col + 1] = o1;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <typename T> hipError_t launch_tf_embed(const TfParams& p, hipStream_t s) {
  hipLaunchKernelGGL((tf_embed_kernel<T>), dim3(p.n * p.N), dim3(DUALAR_WG), 0, s, p);
  return hipGetLastError();
}

template <typename T, typename KT> hipError_t launch_depth_attn(const PrefillParams& p, hipStream_t s) {
  if (p.C < 1 || p.C > DEPTH_MAXN || p.hd > DEPTH_MAXHD || p.hd % 4 || p.H % p.KV || p.H / p.KV > DEPTH_MAXREP)
    return hipErrorInvalidValue;
  switch (p.H / p.KV) {
    case 1: hipLaunchKernelGGL((depth_attn_kernel<T, KT, 1>), dim3(p.B, p.KV), dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((depth_attn_kernel<T, KT, 2>), dim3(p.B, p.KV), dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((depth_attn_kernel<T, KT, 4>), dim3(p.B, p.KV), dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((depth_attn_kernel<T, KT, 8>), dim3(p.B, p.KV), dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_tf_embed<float>(const TfParams&, hipStream_t);
template hipError_t launch_tf_embed<bf16_t>(const TfParams&, hipStream_t);
template hipError_t launch_depth_attn<float, float>(const PrefillParams&, hipStream_t);
template hipError_t launch_depth_attn<bf16_t, bf16_t>(const PrefillParams&, hipStream_t);
template hipError_t launch_depth_attn<bf16_t, float>(const PrefillParams&, hipStream_t);
template hipError_t launch_depth_attn<float, bf16_t>(const PrefillParams&, hipStream_t);
