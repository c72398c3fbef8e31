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
// and KV head g with its rep query heads.  Each of the pair's N rows gets
// the decode arithmetic: QK-norm (one [hd] gain) and RoPE at position k on
// q and k, the 1/sqrt(hd) scale on q, k and v rounded to the cache type (the
// values the incremental fast passes keep in their depth cache), all in
// LDS.  Then row k of query head h attends to rows 0..k: lane j < N holds
// the score against row j, a 16-lane softmax, and lane l sums P.V for dims
// 2l, 2l+1.
#include "common.h"
#include "internal.h"

#define DEPTH_MAXN 16
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

template <typename T, typename KT>
__global__ void __launch_bounds__(256) depth_attn_kernel(PrefillParams p) {
  const int i = blockIdx.x, g = blockIdx.y;
  const int N = p.C, hd = p.hd, rep = p.H / p.KV;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float ks[DEPTH_MAXN][DEPTH_MAXHD + 1];
  __shared__ float vs[DEPTH_MAXN][DEPTH_MAXHD];
  __shared__ float qs[DEPTH_MAXREP][DEPTH_MAXN][DEPTH_MAXHD];
  __shared__ float ps[4][DEPTH_MAXN];

  // ---- prep: N rows x (k, v, rep q heads) vectors, one wave per vector ----
  const bool live = 2 * lane < hd;
  const int pl = live ? 2 * lane : 0;
  const float qscale = 1.0f / sqrtf((float)hd);
  const int nvec = N * (2 + rep);
  for (int t = wave; t < nvec; t += 4) {
    const int k = t / (2 + rep), kind = t % (2 + rep);   // 0: k, 1: v, 2..: q head kind - 2
    const float* row = p.qkv + (size_t)(i * N + k) * p.ld_qkv;
    if (kind == 1) {
      const float* vp = row + (size_t)(p.H + p.KV) * hd + (size_t)g * hd;
      if (live) {
        vs[k][pl] = ElemT<KT>::round(vp[pl]);
        vs[k][pl + 1] = ElemT<KT>::round(vp[pl + 1]);
      }
      continue;
    }
    const int hl = kind - 2;
    const float* src = kind == 0 ? row + (size_t)p.H * hd + (size_t)g * hd : row + (size_t)(g * rep + hl) * hd;
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
      ks[k][pl] = ElemT<KT>::round(ra);
      ks[k][pl + 1] = ElemT<KT>::round(rc);
    } else {
      qs[hl][k][pl] = ra * qscale;
      qs[hl][k][pl + 1] = rc * qscale;
    }
  }
  __syncthreads();

  // ---- causal attention along depth ----
  for (int hl = wave; hl < rep; hl += 4) {
    const size_t col = (size_t)(g * rep + hl) * hd;
    for (int kq = 0; kq < N; ++kq) {
      float s = -INFINITY;
      if (lane <= kq) {
        float d = 0.f;
        for (int e = 0; e < hd; ++e) d = fmaf(qs[hl][kq][e], ks[lane][e], d);
        s = d;
      }
      const float m = wave_max(s);
      const float e = lane <= kq ? expf(s - m) : 0.f;
      const float l = wave_sum(e);
      if (lane < DEPTH_MAXN) ps[wave][lane] = e;
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      float o0 = 0.f, o1 = 0.f;
      for (int j = 0; j <= kq; ++j) {
        const float pj = ps[wave][j];
        if (live) {
          o0 = fmaf(pj, vs[j][pl], o0);
          o1 = fmaf(pj, vs[j][pl + 1], o1);
        }
      }
      __builtin_amdgcn_wave_barrier();
      if (live) {
        const size_t r = (size_t)i * N + kq;
        const float inv = 1.0f / l;
        if (p.out_planes) {
          store_planes(p.out_planes, (size_t)p.R * p.H * hd, r * p.H * hd + col + pl, o0 * inv);
          store_planes(p.out_planes, (size_t)p.R * p.H * hd, r * p.H * hd + col + pl + 1, o1 * inv);
        } else {
          p.out[r * p.ld_out + col + pl] = o0 * inv;
          p.out[r * p.ld_out + col + pl + 1] = o1 * inv;
        }
      }
    }
  }
}

template <typename T> hipError_t launch_tf_embed(const TfParams& p, hipStream_t s) {
  hipLaunchKernelGGL((tf_embed_kernel<T>), dim3(p.n * p.N), dim3(DUALAR_WG), 0, s, p);
  return hipGetLastError();
}

template <typename T, typename KT> hipError_t launch_depth_attn(const PrefillParams& p, hipStream_t s) {
  if (p.C < 1 || p.C > DEPTH_MAXN || p.hd > DEPTH_MAXHD || p.hd % 2 || p.H % p.KV || p.H / p.KV > DEPTH_MAXREP)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL((depth_attn_kernel<T, KT>), dim3(p.B, p.KV), dim3(256), 0, s, p);
  return hipGetLastError();
}

template hipError_t launch_tf_embed<float>(const TfParams&, hipStream_t);
template hipError_t launch_tf_embed<bf16_t>(const TfParams&, hipStream_t);
template hipError_t launch_depth_attn<float, float>(const PrefillParams&, hipStream_t);
template hipError_t launch_depth_attn<bf16_t, bf16_t>(const PrefillParams&, hipStream_t);
template hipError_t launch_depth_attn<bf16_t, float>(const PrefillParams&, hipStream_t);
template hipError_t launch_depth_attn<float, bf16_t>(const PrefillParams&, hipStream_t);
