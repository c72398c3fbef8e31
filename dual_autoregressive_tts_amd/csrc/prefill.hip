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
#include "mfma.h"

#define PF_TK 32          // cache positions per LDS tile
#define PF_MAXHD 128

template <typename T, typename KT>
__global__ void __launch_bounds__(64) prefill_append_kernel(PrefillParams p, int head0) {
  const int r = blockIdx.x, hh = head0 + blockIdx.y, lane = threadIdx.x;
  const int pos = row_position(p.pos, p.pos_const, r, p.max_pos, p.status);
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
  const int pmax = row_position(p.pos, 0, b * p.C + last, p.max_pos, p.status);
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

// Matrix-core causal attention for a bf16 cache with head_dim 128 and four
// query heads per KV head (prefill_flash16_kernel below).  All products are
// exact fp32 products of the stored operands (q and the probabilities as
// three bf16 terms), accumulated in fp32.  Masked scores (key > query
// position, padding rows) are -inf.
#define PF_STG 3                  // K/V block stages: two blocks in flight while one is used
typedef __bf16 pf_bf16x8 __attribute__((ext_vector_type(8)));
typedef short pf_s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void pf_split3(const float (&x)[8], pf_bf16x8* t) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 a0 = (__bf16)x[e];
    const float r1 = x[e] - (float)a0;
    const __bf16 a1 = (__bf16)r1;
    t[0][e] = a0;
    t[1][e] = a1;
    t[2][e] = (__bf16)(r1 - (float)a1);
  }
}

// Grid: one workgroup of 256 threads per (16 consecutive positions of
// sequence b, KV head g); wave w takes query head 4g + w.  The 1-D grid maps
// id -> (query block qb, g, b) with the query blocks in descending order, so
// the blocks with the most keys start first.  Key blocks of 32 positions,
// from 0 to the block's last position, are copied into LDS by LDS DMA
// (global_load_lds_dwordx4), K and V alike as 256-byte key rows whose
// 16-byte pieces sit at slot piece ^ (key & 15), PF_STG stages deep (each
// wave copies a quarter of a block; its own vmcnt wait plus the barrier
// make the block visible).  Per key block, on v_mfma_f32_16x16x32_bf16:
//   S^T = K Q^T as two 16-key x 16-query products (K as the A operand: lane
//   l holds key l%16 of the half, dims 32s + 8(l/16) .. +8; q^T as the B
//   operand: query l%16, the same dims, three bf16 terms held in registers),
//   so lane l holds keys 16h + 4(l/16) + {0..3}, h = 0, 1, of query l%16;
//   O^T += V^T P^T with P^T as the B operand straight from those registers
//   (three bf16 terms; k index 8(l/16) + j is key 16(j/4) + 4(l/16) + j%4)
//   and V^T as the A operand, read from the row-major V block with the
//   gfx950 transposing LDS read ds_read_b64_tr_b16: within each 16-lane
//   group, lane j receives element j%4 of the 8-byte words read by lanes
//   4e + j/4 (e = 0..3), so lane (g, i) reading 4 consecutive dims
//   16 dt + 4(i%4) of key 4g + i/4 (+16) hands lane (g, d) the four keys
//   its operand needs for dim 16 dt + d.  Lane l holds O^T rows
//   16 dt + 4(l/16) + r of query l%16, so the running max, sum and rescale
//   of its query are lane-local after reductions over the four lanes of a
//   query.
// Sixteen queries per wave keep a wave at ~150 registers, so three waves
// share each SIMD and one wave's softmax and LDS waits hide under another's
// products (32 queries per wave with 32x32 products needed 318 registers:
// one wave per SIMD, 1.7 s against 1.05 s for the 16,384-position prefill).
#define PF16_QB 16
typedef float pf_f32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) prefill_flash16_kernel(PrefillParams p, int nqb) {
  constexpr int HD = 128;
  const int per_qb = p.KV * p.B;
  const int qb = nqb - 1 - (int)blockIdx.x / per_qb, rest = (int)blockIdx.x % per_qb;
  const int g = rest % p.KV, b = rest / p.KV;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, grp = lane >> 4, col = lane & 15;
  const int i0 = qb * PF16_QB;
  const int last = min(i0 + PF16_QB, p.C) - 1;
  const int pmax = row_position(p.pos, 0, b * p.C + last, p.max_pos, p.status);
  if (pmax < 0) return;                          // the whole block is padding (uniform)
  const int nkb = pmax / 32 + 1;

  // [stage][K, V][32 key rows of 256 bytes, pieces swizzled]
  __shared__ __attribute__((aligned(1024))) char kv[PF_STG][2][32 * 256];

  // this lane's query and its three q terms for the four 32-dim steps
  const int iq = i0 + col;
  const int posq = iq < p.C ? p.pos[b * p.C + iq] : -1;
  const int hq = g * 4 + wave;
  pf_bf16x8 qt[4][3];
  {
    const float* qrow = p.qbuf + (size_t)(b * p.C + (iq < p.C ? iq : last)) * p.ld_q + (size_t)hq * HD + 8 * grp;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8];
      const float4 a = *(const float4*)(qrow + 32 * s), c = *(const float4*)(qrow + 32 * s + 4);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
      pf_split3(x, qt[s]);
    }
  }
  const size_t head_base = ((size_t)b * p.KV + g) * p.max_pos;
  const char* kg = (const char*)p.kcache + head_base * HD * 2;
  const char* vg = (const char*)p.vcache + head_base * HD * 2;
  // block kb to stage st: 16 DMA instructions of 4 key rows (1 KB) each, four
  // per wave (waves 0-1: K, 2-3: V); lane l takes piece (l%16) ^ (key & 15)
  // of key 4i + l/16, which lands at slot l%16 of that row
  auto issue = [&](int kb, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * wave + j, isv = i >> 3, ii = i & 7;
      const int kl = 4 * ii + (lane >> 4), key = kb * 32 + kl;
      const int piece = (lane & 15) ^ (kl & 15);
      const char* src = (isv ? vg : kg) + ((size_t)(key <= pmax ? key : 0) * HD + piece * 8) * 2;
      dma16(src, &kv[st][isv][ii * 1024]);
    }
  };

  pf_f32x4 o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;          // of query col (the four lanes of a query agree)

  issue(0, 0);
  if (nkb > 1) issue(1, 1);
  int st = 0;
  for (int kb = 0; kb < nkb; ++kb) {
    // this wave's copies of block kb are done once at most the next block's
    // four are outstanding; after the barrier every wave's are, and every
    // wave is done with the stage block kb + 2 overwrites
    if (kb + 1 < nkb) wait_vm_barrier<4>();
    else wait_vm_barrier<0>();
    if (kb + 2 < nkb) issue(kb + 2, st == 0 ? 2 : st - 1);
    const char* ks = kv[st][0];
    const char* vs = kv[st][1];
    // ---- S^T = K q^T: two halves of 16 keys x 16 queries ----
    pf_f32x4 sacc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sacc[h][r] = 0.f;
      const int key = 16 * h + col;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int pc = 4 * s + grp;
        const pf_bf16x8 a = *(const pf_bf16x8*)(ks + key * 256 + ((pc ^ (key & 15)) << 4));
#pragma unroll
        for (int t = 0; t < 3; ++t) sacc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qt[s][t], sacc[h], 0, 0, 0);
      }
    }
    // register r of half h: key kb*32 + 16h + 4 grp + r of query col
    float mt = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb * 32 + 16 * h + 4 * grp + r;
        if (key > posq) sacc[h][r] = -INFINITY;
        mt = fmaxf(mt, sacc[h][r]);
      }
    mt = max_xor32(max_xor16(mt));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    float x[8], ls = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] = expf(sacc[j >> 2][j & 3] - m_use);
      ls += x[j];
    }
    ls = add_xor32(add_xor16(ls));
    const float cf = expf(m_run - m_use);       // 0 while m_run = -inf
    l_run = l_run * cf + ls;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) o[dt][r] *= cf;
    // ---- O^T += V^T P^T ----
    pf_bf16x8 pt[3];
    pf_split3(x, pt);
    // lane (grp, i) reads dims 16 dt + 4(i%4) .. +3 of key 4 grp + i/4 (+16)
    const int vkey = 4 * grp + (col >> 2), vd = 4 * (col & 3);
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = 16 * dt + vd, pd = d >> 3, w = (d & 7) * 2;
      typedef __attribute__((address_space(3))) pf_s16x4* lds_s16x4;
      const char* a0 = vs + vkey * 256 + ((pd ^ (vkey & 15)) << 4) + w;
      const char* a1 = vs + (vkey + 16) * 256 + ((pd ^ ((vkey + 16) & 15)) << 4) + w;
      const pf_s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(lds_void*)a0);
      const pf_s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(lds_void*)a1);
      const pf_s16x4 both[2] = {lo, hi};
      const pf_bf16x8 aa = __builtin_bit_cast(pf_bf16x8, both);
#pragma unroll
      for (int t = 0; t < 3; ++t) o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aa, pt[t], o[dt], 0, 0, 0);
    }
    st = st == 2 ? 0 : st + 1;
  }
  // ---- normalise and store: lane holds dims 16 dt + 4 grp + r of query col ----
  if (iq >= p.C || posq < 0) return;
  const int row = b * p.C + iq;
  const float inv = 1.0f / l_run;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    const size_t colx = (size_t)hq * HD + 16 * dt + 4 * grp;
    if (p.out_planes) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        store_planes(p.out_planes, (size_t)p.R * p.H * HD, (size_t)row * p.H * HD + colx + r, o[dt][r] * inv);
    } else {
      *(float4*)(p.out + (size_t)row * p.ld_out + colx) =
          make_float4(o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
    }
  }
}

template <typename T, typename KT>
hipError_t launch_prefill_attn(const PrefillParams& p, hipStream_t s) {
  if (p.hd % 16 != 0 || p.hd > PF_MAXHD || p.H % p.KV != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_append_kernel<T, KT>), dim3(p.R, p.H + p.KV), dim3(64), 0, s, p, 0);
  const int rep = p.H / p.KV;
  if (sizeof(KT) == 2 && p.hd == 128 && rep == 4) {
    const int nqb = (p.C + PF16_QB - 1) / PF16_QB;
    hipLaunchKernelGGL(prefill_flash16_kernel, dim3(nqb * p.KV * p.B), dim3(256), 0, s, p, nqb);
    return hipGetLastError();
  }
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
