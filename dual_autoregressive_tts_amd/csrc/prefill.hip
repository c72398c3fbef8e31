// Prefill of a chunk of prompt positions for every sequence at once (the
// causal form of the slow-AR forward; decode is the one-position case).
//
// prefill_append_kernel, grid (R, H + KV) (or (R, KV) from head H for the k/v
// append alone), one wave: row r's q head (QK-norm
// with the per-head [hd] gain, RoPE at the row's position, times
// 1/sqrt(hd)) goes to qbuf; its k head (QK-norm, RoPE) and v head are
// rounded to the cache type and written at the row's position.  The
// arithmetic is the decode kernel's, so a position gets the same cache entry
// whether it was prefilled in a chunk or one step at a time.
//
// prefill_attn_kernel, grid (ceil(C / QB), KV, B), 256 threads: QB = 64/REP
// consecutive positions of sequence b times the REP query heads of KV head
// g make 64 query rows, four threads per row.  The workgroup streams the
// cache entries 0..(largest position of its rows) of (b, g) through LDS in
// tiles of 32 positions, once for all its rows, and keeps a running
// (max, sum, P.V) per row: masked scores (position > the row's) are -inf.
// fp32 throughout; K/V are read at the cache's precision.
#include "common.h"
#include "internal.h"

#define PF_TK 32          // cache positions per LDS tile
#define PF_MAXHD 128

template <typename T, typename KT>
__global__ void __launch_bounds__(64) prefill_append_kernel(PrefillParams p, int head0) {
  const int r = blockIdx.x, hh = head0 + blockIdx.y, lane = threadIdx.x;
  const int pos = p.pos ? p.pos[r] : p.pos_const;
  if (pos < 0) return;
  const int b = r / p.C, hd = p.hd;
  const bool live = 2 * lane < hd;
  const int pl = live ? 2 * lane : 0;
  const float* row = p.qkv + (size_t)r * p.ld_qkv;
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
      float* q = p.qbuf + (size_t)r * p.ld_q + (size_t)hh * hd;
      q[2 * lane] = (a * cs.x - c * cs.y) * qscale;
      q[2 * lane + 1] = (a * cs.y + c * cs.x) * qscale;
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
    ElemT<KT>::store(p.kcache, at + 2 * lane, ElemT<KT>::round(a * cs.x - c * cs.y));
    ElemT<KT>::store(p.kcache, at + 2 * lane + 1, ElemT<KT>::round(a * cs.y + c * cs.x));
  }
  const float* vp = row + (size_t)(p.H + p.KV) * hd + (size_t)g * hd;
  for (int d = lane; d < hd; d += 64) ElemT<KT>::store(p.vcache, at + d, ElemT<KT>::round(vp[d]));
}

// Dims owned by thread slice sl (0..3): d = 16*e + 4*sl + c, c < 4 -- the four
// slices of a row read 64 consecutive bytes of an LDS row per step.
template <typename KT, int REP>
__global__ void __launch_bounds__(256) prefill_attn_kernel(PrefillParams p) {
  constexpr int QB = 64 / REP;
  constexpr int E4 = PF_MAXHD / 16;           // float4 groups per slice (max)
  const int b = blockIdx.z, g = blockIdx.y, i0 = blockIdx.x * QB;
  const int t = threadIdx.x, qr = t >> 2, sl = t & 3;
  const int hd = p.hd, ne4 = hd / 16;
  const int i = i0 + qr / REP, h = g * REP + qr % REP;
  const int r = b * p.C + i;
  const int pos = i < p.C ? p.pos[r] : -1;
  // positions grow with i inside a chunk: the block's last real row has the largest
  const int last = min(i0 + QB, p.C) - 1;
  const int pmax = p.pos[b * p.C + last];
  if (pmax < 0) return;                         // whole block is padding (uniform)

  __shared__ __attribute__((aligned(16))) float Ks[PF_TK][PF_MAXHD];
  __shared__ __attribute__((aligned(16))) float Vs[PF_TK][PF_MAXHD];

  float4 q[E4], o[E4];
  const float* qsrc = p.qbuf + (size_t)r * p.ld_q + (size_t)h * hd;
#pragma unroll
  for (int e = 0; e < E4; ++e) {
    o[e] = make_float4(0.f, 0.f, 0.f, 0.f);
    q[e] = (e < ne4 && pos >= 0) ? *(const float4*)(qsrc + 16 * e + 4 * sl) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float m = -INFINITY, l = 0.f;

  const size_t head = ((size_t)b * p.KV + g) * p.max_pos;
  constexpr int EPV = ElemT<KT>::EPV;          // elements per 16-byte load
  const int vec_per_row = hd / EPV, vec_per_tile = PF_TK * vec_per_row;
  for (int j0 = 0; j0 <= pmax; j0 += PF_TK) {
    // tile load: cache rows j0..j0+31 (zeros past pmax)
    for (int v = t; v < vec_per_tile; v += 256) {
      const int jj = v / vec_per_row, c0 = (v % vec_per_row) * EPV;
      const int j = j0 + jj;
      float kf[EPV], vf[EPV];
      if (j <= pmax) {
        const size_t off = ((head + j) * hd + c0) * sizeof(KT);
        ElemT<KT>::unpack(ld_vec((const char*)p.kcache + off), kf);
        ElemT<KT>::unpack(ld_vec((const char*)p.vcache + off), vf);
      } else {
#pragma unroll
        for (int e = 0; e < EPV; ++e) kf[e] = vf[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        Ks[jj][c0 + e] = kf[e];
        Vs[jj][c0 + e] = vf[e];
      }
    }
    __syncthreads();
    float s[PF_TK];
    float tmax = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < PF_TK; ++jj) {
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < E4; ++e) {
        if (e < ne4) {
          const float4 k4 = *(const float4*)&Ks[jj][16 * e + 4 * sl];
          d = fmaf(q[e].x, k4.x, d);
          d = fmaf(q[e].y, k4.y, d);
          d = fmaf(q[e].z, k4.z, d);
          d = fmaf(q[e].w, k4.w, d);
        }
      }
      d += xor1_of(d);
      d += xor2_of(d);
      s[jj] = j0 + jj <= pos ? d : -INFINITY;
      tmax = fmaxf(tmax, s[jj]);
    }
    if (pos >= 0 && tmax > -INFINITY) {
      const float mn = fmaxf(m, tmax);
      const float corr = expf(m - mn);          // m = -inf on the first tile: 0
      l *= corr;
#pragma unroll
      for (int e = 0; e < E4; ++e) {
        o[e].x *= corr; o[e].y *= corr; o[e].z *= corr; o[e].w *= corr;
      }
#pragma unroll
      for (int jj = 0; jj < PF_TK; ++jj) {
        const float w = expf(s[jj] - mn);
        l += w;
#pragma unroll
        for (int e = 0; e < E4; ++e) {
          if (e < ne4) {
            const float4 v4 = *(const float4*)&Vs[jj][16 * e + 4 * sl];
            o[e].x = fmaf(w, v4.x, o[e].x);
            o[e].y = fmaf(w, v4.y, o[e].y);
            o[e].z = fmaf(w, v4.z, o[e].z);
            o[e].w = fmaf(w, v4.w, o[e].w);
          }
        }
      }
      m = mn;
    }
    __syncthreads();
  }
  if (pos < 0) return;
  const float inv = 1.0f / l;
  if (p.out_planes) {
    const size_t plane = (size_t)p.R * p.H * hd, at = (size_t)r * p.H * hd + (size_t)h * hd;
#pragma unroll
    for (int e = 0; e < E4; ++e)
      if (e < ne4) {
        store_planes(p.out_planes, plane, at + 16 * e + 4 * sl + 0, o[e].x * inv);
        store_planes(p.out_planes, plane, at + 16 * e + 4 * sl + 1, o[e].y * inv);
        store_planes(p.out_planes, plane, at + 16 * e + 4 * sl + 2, o[e].z * inv);
        store_planes(p.out_planes, plane, at + 16 * e + 4 * sl + 3, o[e].w * inv);
      }
    return;
  }
  float* dst = p.out + (size_t)r * p.ld_out + (size_t)h * hd;
#pragma unroll
  for (int e = 0; e < E4; ++e)
    if (e < ne4) *(float4*)(dst + 16 * e + 4 * sl) = make_float4(o[e].x * inv, o[e].y * inv, o[e].z * inv, o[e].w * inv);
}

template <typename T, typename KT>
hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t s) {
  if (p.hd % 16 != 0 || p.hd > PF_MAXHD || p.H % p.KV != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_append_kernel<T, KT>), dim3(p.R, p.H + p.KV), dim3(64), 0, s, p, 0);
  const int rep = p.H / p.KV;
  const int qb = 64 / rep;
  const dim3 grid((p.C + qb - 1) / qb, p.KV, p.B);
  switch (rep) {
    case 1: hipLaunchKernelGGL((prefill_attn_kernel<KT, 1>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((prefill_attn_kernel<KT, 2>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((prefill_attn_kernel<KT, 4>), grid, dim3(256), 0, s, p); break;
    case 8: hipLaunchKernelGGL((prefill_attn_kernel<KT, 8>), grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, typename KT>
hipError_t launch_kv_append(const PrefillParams& p, hipStream_t s) {
  if (p.hd > PF_MAXHD) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_append_kernel<T, KT>), dim3(p.R, p.KV), dim3(64), 0, s, p, p.H);
  return hipGetLastError();
}

template hipError_t launch_kv_append<float, float>(const PrefillParams&, hipStream_t);
template hipError_t launch_kv_append<bf16_t, bf16_t>(const PrefillParams&, hipStream_t);
template hipError_t launch_kv_append<bf16_t, float>(const PrefillParams&, hipStream_t);
template hipError_t launch_kv_append<float, bf16_t>(const PrefillParams&, hipStream_t);
template hipError_t launch_prefill_attn<float, float>(const PrefillParams&, hipStream_t);
template hipError_t launch_prefill_attn<bf16_t, bf16_t>(const PrefillParams&, hipStream_t);
template hipError_t launch_prefill_attn<bf16_t, float>(const PrefillParams&, hipStream_t);
template hipError_t launch_prefill_attn<float, bf16_t>(const PrefillParams&, hipStream_t);
