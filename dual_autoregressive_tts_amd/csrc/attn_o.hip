// Batch-1 attention over a short cache fused with the O product and its
// residual: x += W_o . softmax(q K^T / sqrt(hd)) V.
//
// The fast AR attends along codebook depth, so its cache never holds more
// than num_codebooks (10) positions ([P2] "Two autoregressions…": the fast
// loop and its per-frame cache).  At batch 1 a separate attention launch
// costs a full dispatch for a few KB of work, while the O product that
// follows streams 21 MB of weights that do not depend on the attention.
// Here every workgroup issues its small attention loads, then its share of
// W_o, and computes the attention for all query heads while the weights are
// in flight; the attention output never leaves the workgroup.
//
// Shape (S2 fast AR): H = 32 query heads, KV = 8 KV heads, head_dim 128,
// bf16 weights and cache, at most 16 positions.  A workgroup is 8 waves;
// wave w owns KV head w and its query heads 4w..4w+3 (contiguous grouping),
// which are exactly columns [512 w, 512 w + 512) of W_o: the wave's
// attention output is the wave's eighth of the product input.  Two waves
// per SIMD hide each other's reduction and matrix-core latencies.
//
// Arithmetic follows the other decode attention kernels: per-head RMSNorm
// of q and k with one [hd] gain, RoPE on interleaved pairs from the bf16
// table, the 1/sqrt(hd) scale folded into q, the new k and v rounded to the
// cache type before use, scores on the matrix cores with q as three bf16
// terms (the fp32 product), fp32 softmax and accumulation.  Every workgroup
// computes the same values; workgroup 0 alone appends k and v.
#include "common.h"
#include "internal.h"

namespace {
constexpr int HD = 128;      // head_dim
constexpr int REP = 4;       // query heads per KV head (= per wave)
constexpr int NW = 8;        // waves per workgroup (= KV heads)
constexpr int MAXL = 16;     // positions
constexpr int WGT = NW * 64;
typedef __bf16 att_bf16x8 __attribute__((ext_vector_type(8)));
typedef float att_f32x4 __attribute__((ext_vector_type(4)));
}

template <int R>
__global__ void __launch_bounds__(WGT) attn_o_b1_kernel(AttnOParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t qp[NW][3][REP][HD];   // q as three bf16 terms
  __shared__ __attribute__((aligned(16))) float kn[NW][HD];
  __shared__ __attribute__((aligned(16))) float sc[NW][REP][MAXL];
  __shared__ __attribute__((aligned(16))) float os[NW][REP * HD];
  __shared__ float part[NW][R];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = wave;                       // KV head
  const int pos = checked_index(p.pos, p.max_pos, p.status), L = pos + 1;
  const int K = p.H * HD;
  const int row0 = blockIdx.x * R;

  // ---- 1. attention inputs, issued before the weights ----
  const float* qkv = p.qkv;
  float2 q2[REP];
#pragma unroll
  for (int h4 = 0; h4 < REP; ++h4) q2[h4] = *(const float2*)(qkv + (size_t)(g * REP + h4) * HD + 2 * lane);
  const float2 k2 = *(const float2*)(qkv + (size_t)p.H * HD + (size_t)g * HD + 2 * lane);
  const float2 v2 = *(const float2*)(qkv + (size_t)(p.H + p.KV) * HD + (size_t)g * HD + 2 * lane);
  uint32_t qg = 0x3f803f80u, kg = 0x3f803f80u;   // bf16 pair (1, 1)
  if (p.q_norm) qg = ((const uint32_t*)p.q_norm)[lane];
  if (p.k_norm) kg = ((const uint32_t*)p.k_norm)[lane];
  const float2 cs = p.rope[(size_t)pos * (HD / 2) + lane];
  const float xres = (threadIdx.x < R && row0 + (int)threadIdx.x < p.dim) ? p.x[row0 + threadIdx.x] : 0.f;
  // cached K as the A operand of the score product (16 positions x 32 dims
  // per step): lane l holds position l % 16, dims 32 ks + 8 (l / 16) .. +8;
  // lanes at or past pos read position 0 (always written) and never use it
  const int jm = lane & 15, kq = lane >> 4;
  const int jl = jm < pos ? jm : 0;
  u32x4 kc[4];
  {
    const char* src = (const char*)p.kcache + (((size_t)g * p.max_pos + jl) * HD + 8 * kq) * sizeof(bf16_t);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kc[ks] = ld_vec(src + 64 * ks);
  }
  // cached V in the dim layout: lane l holds dims 2l, 2l+1 of every position
  uint32_t vc[MAXL];
  {
    const uint32_t* src = (const uint32_t*)((const char*)p.vcache + ((size_t)g * p.max_pos * HD + 2 * lane) * sizeof(bf16_t));
#pragma unroll
    for (int jj = 0; jj < MAXL; ++jj) {
      vc[jj] = 0u;
      if (jj < pos) vc[jj] = src[(size_t)jj * (HD / 2)];
    }
  }

  // ---- 2. this workgroup's rows of W_o, the wave's 512 columns ----
  u32x4 w[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = min(row0 + r, p.dim - 1);
    w[r] = ld_stream((const char*)p.wo + ((size_t)row * K + (size_t)wave * 512 + lane * 8) * sizeof(bf16_t));
  }

  // ---- 3. q: QK-norm, RoPE, score scale; new k: QK-norm, RoPE, rounding ----
  const float qscale = 1.0f / sqrtf((float)HD);
  const float qga = bf16_bits_to_f32(qg & 0xffffu), qgc = bf16_bits_to_f32(qg >> 16);
  const float kga = bf16_bits_to_f32(kg & 0xffffu), kgc = bf16_bits_to_f32(kg >> 16);
#pragma unroll
  for (int h4 = 0; h4 < REP; ++h4) {
    float a = q2[h4].x, c = q2[h4].y;
    if (p.q_norm) {
      const float inv = 1.0f / sqrtf(wave_sum(a * a + c * c) / (float)HD + p.eps);
      a = a * inv * qga;
      c = c * inv * qgc;
    }
    const float ra = (a * cs.x - c * cs.y) * qscale, rc = (a * cs.y + c * cs.x) * qscale;
    // three bf16 terms t0 + t1 + t2 of each value, so that the bf16 product
    // with the (bf16) keys is the fp32 one
    const uint16_t a0 = f32_to_bf16_rne(ra), c0 = f32_to_bf16_rne(rc);
    const float a1f = ra - bf16_bits_to_f32(a0), c1f = rc - bf16_bits_to_f32(c0);
    const uint16_t a1 = f32_to_bf16_rne(a1f), c1 = f32_to_bf16_rne(c1f);
    const uint16_t a2 = f32_to_bf16_rne(a1f - bf16_bits_to_f32(a1));
    const uint16_t c2 = f32_to_bf16_rne(c1f - bf16_bits_to_f32(c1));
    *(uint32_t*)&qp[wave][0][h4][2 * lane] = (uint32_t)a0 | ((uint32_t)c0 << 16);
    *(uint32_t*)&qp[wave][1][h4][2 * lane] = (uint32_t)a1 | ((uint32_t)c1 << 16);
    *(uint32_t*)&qp[wave][2][h4][2 * lane] = (uint32_t)a2 | ((uint32_t)c2 << 16);
  }
  float vn0, vn1;
  {
    float a = k2.x, c = k2.y;
    if (p.k_norm) {
      const float inv = 1.0f / sqrtf(wave_sum(a * a + c * c) / (float)HD + p.eps);
      a = a * inv * kga;
      c = c * inv * kgc;
    }
    const uint16_t ka = f32_to_bf16_rne(a * cs.x - c * cs.y);
    const uint16_t kb = f32_to_bf16_rne(a * cs.y + c * cs.x);
    const uint16_t va = f32_to_bf16_rne(v2.x), vb = f32_to_bf16_rne(v2.y);
    kn[wave][2 * lane] = bf16_bits_to_f32(ka);
    kn[wave][2 * lane + 1] = bf16_bits_to_f32(kb);
    vn0 = bf16_bits_to_f32(va);
    vn1 = bf16_bits_to_f32(vb);
    if (blockIdx.x == 0) {
      const size_t at = ((size_t)g * p.max_pos + pos) * HD + 2 * lane;
      *(uint32_t*)((char*)p.kcache + at * sizeof(bf16_t)) = (uint32_t)ka | ((uint32_t)kb << 16);
      *(uint32_t*)((char*)p.vcache + at * sizeof(bf16_t)) = (uint32_t)va | ((uint32_t)vb << 16);
    }
  }
  __builtin_amdgcn_wave_barrier();   // qp[wave], kn[wave]: this wave's own

  // ---- 4. scores on the matrix cores: S^T = K . q^T, softmax in registers ----
  // A = 16 positions x 32 dims of K (bf16, exact), B = 32 dims x 16 columns
  // (column n: query head n % 4, one bf16 term of q per product, the three
  // accumulated); lane l gets S[4 (l / 16) + r][l % 16].  The four lanes of
  // a column (l / 16 = 0..3) hold its 16 positions: max and sum across them
  // by the row / half swaps.  All LDS data from here to the product input is
  // the wave's own: wave-level barriers only.
  {
    att_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      att_bf16x8 a = __builtin_bit_cast(att_bf16x8, kc[ks]);
      if (jm == pos) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = (__bf16)kn[wave][32 * ks + 8 * kq + e];
      }
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const u32x4 b = *(const u32x4*)&qp[wave][t][jm & 3][32 * ks + 8 * kq];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(att_bf16x8, b), acc, 0, 0, 0);
      }
    }
    float sv[4];
    float m = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = 4 * kq + r < L ? acc[r] : -INFINITY;
      m = fmaxf(m, sv[r]);
    }
    m = max_xor16(m);
    m = max_xor32(m);
    float l = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = 4 * kq + r < L ? expf(sv[r] - m) : 0.f;
      l += sv[r];
    }
    l = add_xor16(l);
    l = add_xor32(l);
    if (jm < REP) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sc[wave][jm][4 * kq + r] = sv[r] / l;
    }
  }
  __builtin_amdgcn_wave_barrier();

  // ---- 6. P.V in the dim layout, then the wave's eighth of the product input ----
  float pr[REP][MAXL];
#pragma unroll
  for (int h4 = 0; h4 < REP; ++h4)
#pragma unroll
    for (int qd = 0; qd < MAXL / 4; ++qd) {
      const float4 t = *(const float4*)&sc[wave][h4][4 * qd];
      pr[h4][4 * qd] = t.x; pr[h4][4 * qd + 1] = t.y; pr[h4][4 * qd + 2] = t.z; pr[h4][4 * qd + 3] = t.w;
    }
  float o[REP][2];
#pragma unroll
  for (int h4 = 0; h4 < REP; ++h4) o[h4][0] = o[h4][1] = 0.f;
#pragma unroll
  for (int jj = 0; jj < MAXL; ++jj) {
    if (jj < L) {
      float va, vb;
      if (jj == pos) { va = vn0; vb = vn1; }
      else { va = bf16_bits_to_f32(vc[jj] & 0xffffu); vb = bf16_bits_to_f32(vc[jj] >> 16); }
#pragma unroll
      for (int h4 = 0; h4 < REP; ++h4) {
        o[h4][0] = fmaf(pr[h4][jj], va, o[h4][0]);
        o[h4][1] = fmaf(pr[h4][jj], vb, o[h4][1]);
      }
    }
  }
#pragma unroll
  for (int h4 = 0; h4 < REP; ++h4) *(float2*)&os[wave][h4 * HD + 2 * lane] = make_float2(o[h4][0], o[h4][1]);
  __builtin_amdgcn_wave_barrier();   // os[wave]: this wave's own
  float ov[8];
  {
    const float4 t0 = *(const float4*)&os[wave][lane * 8];
    const float4 t1 = *(const float4*)&os[wave][lane * 8 + 4];
    ov[0] = t0.x; ov[1] = t0.y; ov[2] = t0.z; ov[3] = t0.w;
    ov[4] = t1.x; ov[5] = t1.y; ov[6] = t1.z; ov[7] = t1.w;
  }

  // ---- 7. dot products, the eight column blocks summed in order, residual ----
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float wf[8];
    ElemT<bf16_t>::unpack(w[r], wf);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(wf[e], ov[e], acc);
    acc = wave_sum(acc);
    if (lane == 0) part[wave][r] = acc;
  }
  __syncthreads();
  if (threadIdx.x < R && row0 + (int)threadIdx.x < p.dim) {
    const int r = threadIdx.x;
    float v = part[0][r];
#pragma unroll
    for (int q = 1; q < NW; ++q) v += part[q][r];
    p.x[row0 + r] = xres + v;
  }
}

// 10 rows of W_o per workgroup: 256 workgroups of 8 waves, about one per
// compute unit (5 and 20 rows were slower).
constexpr int ATTN_O_ROWS = 10;

bool attn_o_b1_fits(int H, int KV, int hd, int dim, int L) {
  return KV == NW && H == NW * REP && hd == HD && L >= 1 && L <= MAXL && dim > 0;
}

hipError_t launch_attn_o_b1(const AttnOParams& p, hipStream_t s) {
  if (!attn_o_b1_fits(p.H, p.KV, p.hd, p.dim, p.pos + 1) || p.pos >= p.max_pos) return hipErrorInvalidValue;
  const int nwg = (p.dim + ATTN_O_ROWS - 1) / ATTN_O_ROWS;
  launch_timed(attn_o_b1_kernel<ATTN_O_ROWS>, dim3(nwg), dim3(WGT), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Batch-1 merge of the split attention partials fused with the O product
// (slow AR, split form): x += W_o . o with o_h = sum_s e^(m_s - M) o_s /
// sum_s e^(m_s - M) l_s over the splits s of head h, M = max_s m_s.
// The wide O layout puts KV head w's query heads 4w..4w+3 on wave w and
// columns 8 (l % 16) .. +8 of head 4w + l / 16 on lane l, so every lane
// merges exactly the eight values it multiplies, from at most MAXS splits
// (loads issued before the weights).  With one split the split kernel has
// written o itself and the lane reads it.
template <int R, int MAXS>
__global__ void __launch_bounds__(WGT) merge_o_b1_kernel(MergeOParams p) {
  __shared__ float part[NW][R];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * R;
  const int K = p.H * HD;
  const int L = p.pos[0] + 1;
  const int ns = checked_index((L + p.chunk - 1) / p.chunk - 1, min(p.max_splits, MAXS), p.status) + 1;
  const int h = wave * REP + (lane >> 4), d0 = (lane & 15) * 8;

  // 1. partials (or o), residual, then the weights
  float2 po[MAXS][4];
  float pm[MAXS], pl[MAXS];
  float4 o0 = make_float4(0.f, 0.f, 0.f, 0.f), o1 = o0;
  if (ns == 1) {
    const float* src = p.att + (size_t)h * HD + d0;
    o0 = *(const float4*)src;
    o1 = *(const float4*)(src + 4);
  } else {
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
      if (s < ns) {
        const float* q = p.part + ((size_t)h * p.max_splits + s) * (HD + 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) po[s][i] = *(const float2*)(q + d0 + 2 * i);
        pm[s] = q[HD];
        pl[s] = q[HD + 1];
      }
    }
  }
  const float xres = (threadIdx.x < R && row0 + (int)threadIdx.x < p.dim) ? p.x[row0 + threadIdx.x] : 0.f;
  u32x4 w[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = min(row0 + r, p.dim - 1);
    w[r] = ld_stream((const char*)p.wo + ((size_t)row * K + (size_t)wave * 512 + lane * 8) * sizeof(bf16_t));
  }

  // 2. merge, splits in order
  float ov[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
  if (ns > 1) {
    float M = pm[0];
#pragma unroll
    for (int s = 1; s < MAXS; ++s)
      if (s < ns) M = fmaxf(M, pm[s]);
    float lsum = 0.f;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
      if (s < ns) {
        const float ws = expf(pm[s] - M);
        lsum = fmaf(pl[s], ws, lsum);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] = fmaf(po[s][i].x, ws, acc[2 * i]);
          acc[2 * i + 1] = fmaf(po[s][i].y, ws, acc[2 * i + 1]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[e] = acc[e] / lsum;
  }

  // 3. dot products, the eight column blocks summed in order, residual
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float wf[8];
    ElemT<bf16_t>::unpack(w[r], wf);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(wf[e], ov[e], acc);
    acc = wave_sum(acc);
    if (lane == 0) part[wave][r] = acc;
  }
  __syncthreads();
  if (threadIdx.x < R && row0 + (int)threadIdx.x < p.dim) {
    const int r = threadIdx.x;
    float v = part[0][r];
#pragma unroll
    for (int q = 1; q < NW; ++q) v += part[q][r];
    p.x[row0 + r] = xres + v;
  }
}

// At most 10 splits merged inside the O product (the split kernel's chunks
// grow from 128 to 256 positions past 1,280 positions to stay within it).
constexpr int MERGE_O_MAXS = 10;

int merge_o_b1_max_splits() { return MERGE_O_MAXS; }

hipError_t launch_merge_o_b1(const MergeOParams& p, hipStream_t s) {
  if (!attn_o_b1_fits(p.H, p.H / REP, p.hd, p.dim, 1) || p.max_splits > MERGE_O_MAXS || p.chunk <= 0)
    return hipErrorInvalidValue;
  const int nwg = (p.dim + ATTN_O_ROWS - 1) / ATTN_O_ROWS;
  launch_timed(merge_o_b1_kernel<ATTN_O_ROWS, MERGE_O_MAXS>, dim3(nwg), dim3(WGT), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Batch-1 split attention over the slow cache (bf16, S2 head shape), for the
// merge inside the O product: workgroup (split, g) takes 8 * NPW consecutive
// positions of KV head g and its 4 query heads, one wave per NPW positions.
// Waves 0-3 prepare one query head each (QK-norm, RoPE, score scale, three
// bf16 terms), the workgroup holding the new position appends k and v; then
// every wave scores its positions on the matrix cores, takes a wave-local
// softmax (max m_w, sum l_w) and its unnormalised P.V in registers, and the
// eight waves' (m_w, l_w, o_w) are combined once in LDS into the split's
// (o, m, l) -- or o / l when the context is one split.  Same partial layout
// and arithmetic steps as the other decode attention kernels.
template <int NPW>
__global__ void __launch_bounds__(WGT) attn_split_b1_kernel(AttnParams p) {
  constexpr int GW = NPW / 16;                 // 16-position score groups per wave
  constexpr int CH = NW * NPW;                 // positions per split
  __shared__ __attribute__((aligned(16))) uint16_t qp[3][REP][HD];
  __shared__ __attribute__((aligned(16))) float kn[HD];
  __shared__ float vn[HD];
  __shared__ __attribute__((aligned(16))) float pe[NW][REP][NPW];
  __shared__ float mw[NW][REP], lw[NW][REP];
  __shared__ __attribute__((aligned(16))) float ow[NW][REP][HD];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int split = blockIdx.x, g = blockIdx.y;
  const int pos = row_position(p.pos, p.pos_const, 0, p.max_pos, p.status);
  const int L = pos + 1;
  const int n_splits = (L + CH - 1) / CH;
  if (split >= n_splits) return;
  const int c0 = split * CH, c1 = min(c0 + CH, L);
  const int w0 = c0 + wave * NPW;              // the wave's first position
  const bool has_new = pos >= c0 && pos < c1;
  const size_t head_base = (size_t)g * p.max_pos;
  const char* kbase = (const char*)p.kcache + head_base * HD * sizeof(bf16_t);
  const uint32_t* vbase = (const uint32_t*)((const char*)p.vcache + head_base * HD * sizeof(bf16_t));

  // ---- 1. loads: K (score operand), V (dim layout), q / new k, v, gains, RoPE ----
  const int jm = lane & 15, kq = lane >> 4;
  u32x4 kc[GW][4];
#pragma unroll
  for (int mm = 0; mm < GW; ++mm) {
    const int j = w0 + 16 * mm + jm;
    const int jl = (j < c1 && j != pos) ? j : 0;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kc[mm][ks] = ld_vec(kbase + ((size_t)jl * HD + 32 * ks + 8 * kq) * sizeof(bf16_t));
  }
  uint32_t vc[NPW];
#pragma unroll
  for (int jj = 0; jj < NPW; ++jj) {
    const int j = w0 + jj;
    vc[jj] = 0u;
    if (j < c1 && j != pos) vc[jj] = vbase[(size_t)j * (HD / 2) + lane];
  }
  const float* row = p.qkv;
  float2 qv = make_float2(0.f, 0.f), kv2 = qv, vv2 = qv;
  if (wave < REP) qv = *(const float2*)(row + (size_t)(g * REP + wave) * HD + 2 * lane);
  if (has_new && wave == REP) {
    kv2 = *(const float2*)(row + (size_t)p.H * HD + (size_t)g * HD + 2 * lane);
    vv2 = *(const float2*)(row + (size_t)(p.H + p.KV) * HD + (size_t)g * HD + 2 * lane);
  }
  uint32_t qg = 0x3f803f80u, kg = 0x3f803f80u;   // bf16 pair (1, 1)
  if (p.q_norm) qg = ((const uint32_t*)p.q_norm)[lane];
  if (p.k_norm) kg = ((const uint32_t*)p.k_norm)[lane];
  const float2 cs = p.rope[(size_t)pos * (HD / 2) + lane];

  // ---- 2. q (waves 0-3) and the new k, v (wave 4 of the split holding pos) ----
  if (wave < REP) {
    float a = qv.x, c = qv.y;
    if (p.q_norm) {
      const float inv = 1.0f / sqrtf(wave_sum(a * a + c * c) / (float)HD + p.eps);
      a = a * inv * bf16_bits_to_f32(qg & 0xffffu);
      c = c * inv * bf16_bits_to_f32(qg >> 16);
    }
    const float qscale = 1.0f / sqrtf((float)HD);
    const float ra = (a * cs.x - c * cs.y) * qscale, rc = (a * cs.y + c * cs.x) * qscale;
    const uint16_t a0 = f32_to_bf16_rne(ra), c0b = f32_to_bf16_rne(rc);
    const float a1f = ra - bf16_bits_to_f32(a0), c1f = rc - bf16_bits_to_f32(c0b);
    const uint16_t a1 = f32_to_bf16_rne(a1f), c1b = f32_to_bf16_rne(c1f);
    const uint16_t a2 = f32_to_bf16_rne(a1f - bf16_bits_to_f32(a1));
    const uint16_t c2 = f32_to_bf16_rne(c1f - bf16_bits_to_f32(c1b));
    *(uint32_t*)&qp[0][wave][2 * lane] = (uint32_t)a0 | ((uint32_t)c0b << 16);
    *(uint32_t*)&qp[1][wave][2 * lane] = (uint32_t)a1 | ((uint32_t)c1b << 16);
    *(uint32_t*)&qp[2][wave][2 * lane] = (uint32_t)a2 | ((uint32_t)c2 << 16);
  } else if (has_new && wave == REP) {
    float a = kv2.x, c = kv2.y;
    if (p.k_norm) {
      const float inv = 1.0f / sqrtf(wave_sum(a * a + c * c) / (float)HD + p.eps);
      a = a * inv * bf16_bits_to_f32(kg & 0xffffu);
      c = c * inv * bf16_bits_to_f32(kg >> 16);
    }
    const uint16_t ka = f32_to_bf16_rne(a * cs.x - c * cs.y);
    const uint16_t kb = f32_to_bf16_rne(a * cs.y + c * cs.x);
    const uint16_t va = f32_to_bf16_rne(vv2.x), vb = f32_to_bf16_rne(vv2.y);
    kn[2 * lane] = bf16_bits_to_f32(ka);
    kn[2 * lane + 1] = bf16_bits_to_f32(kb);
    vn[2 * lane] = bf16_bits_to_f32(va);
    vn[2 * lane + 1] = bf16_bits_to_f32(vb);
    const size_t at = (head_base + pos) * HD + 2 * lane;
    *(uint32_t*)((char*)p.kcache + at * sizeof(bf16_t)) = (uint32_t)ka | ((uint32_t)kb << 16);
    *(uint32_t*)((char*)p.vcache + at * sizeof(bf16_t)) = (uint32_t)va | ((uint32_t)vb << 16);
  }
  __syncthreads();

  // ---- 3. scores on the matrix cores, column n = query head n % 4 ----
  // lane l gets S[position 4 (l / 16) + r of group mm][head (l % 16) % 4]
  float sv[GW][4];
#pragma unroll
  for (int mm = 0; mm < GW; ++mm) {
    att_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      att_bf16x8 a = __builtin_bit_cast(att_bf16x8, kc[mm][ks]);
      if (w0 + 16 * mm + jm == pos) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = (__bf16)kn[32 * ks + 8 * kq + e];
      }
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const u32x4 b = *(const u32x4*)&qp[t][jm & 3][32 * ks + 8 * kq];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(att_bf16x8, b), acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[mm][r] = (w0 + 16 * mm + 4 * kq + r < c1) ? acc[r] : -INFINITY;
  }

  // ---- 4. wave-local softmax over the wave's positions (per head column) ----
  float m = -INFINITY;
#pragma unroll
  for (int mm = 0; mm < GW; ++mm)
#pragma unroll
    for (int r = 0; r < 4; ++r) m = fmaxf(m, sv[mm][r]);
  m = max_xor16(m);
  m = max_xor32(m);
  float ls = 0.f;
#pragma unroll
  for (int mm = 0; mm < GW; ++mm)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = sv[mm][r] == -INFINITY ? 0.f : expf(sv[mm][r] - m);
      sv[mm][r] = e;
      ls += e;
    }
  ls = add_xor16(ls);
  ls = add_xor32(ls);
  if (jm < REP) {
#pragma unroll
    for (int mm = 0; mm < GW; ++mm)
#pragma unroll
      for (int r = 0; r < 4; ++r) pe[wave][jm][16 * mm + 4 * kq + r] = sv[mm][r];
    if (kq == 0) { mw[wave][jm] = m; lw[wave][jm] = ls; }
  }
  __syncthreads();

  // ---- 5. the wave's unnormalised P.V (lane: dims 2l, 2l+1 of the 4 heads) ----
  float o[REP][2];
#pragma unroll
  for (int h = 0; h < REP; ++h) o[h][0] = o[h][1] = 0.f;
#pragma unroll
  for (int q4 = 0; q4 < NPW / 4; ++q4) {
    float4 pv[REP];
#pragma unroll
    for (int h = 0; h < REP; ++h) pv[h] = *(const float4*)&pe[wave][h][4 * q4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int jj = 4 * q4 + r;
      float va = bf16_bits_to_f32(vc[jj] & 0xffffu), vb = bf16_bits_to_f32(vc[jj] >> 16);
      if (w0 + jj == pos) { va = vn[2 * lane]; vb = vn[2 * lane + 1]; }
#pragma unroll
      for (int h = 0; h < REP; ++h) {
        const float pj = r == 0 ? pv[h].x : r == 1 ? pv[h].y : r == 2 ? pv[h].z : pv[h].w;
        o[h][0] = fmaf(pj, va, o[h][0]);
        o[h][1] = fmaf(pj, vb, o[h][1]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < REP; ++h) *(float2*)&ow[wave][h][2 * lane] = make_float2(o[h][0], o[h][1]);
  __syncthreads();

  // ---- 6. combine the waves (thread t: head t / 128, dim t % 128), waves in order ----
  {
    const int h = threadIdx.x >> 7, d = threadIdx.x & 127;
    float M = mw[0][h];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, mw[w][h]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = mw[w][h] == -INFINITY ? 0.f : expf(mw[w][h] - M);
      acc = fmaf(f, ow[w][h][d], acc);
      lsum = fmaf(f, lw[w][h], lsum);
    }
    const int hh = g * REP + h;
    if (n_splits == 1) {
      p.out[(size_t)hh * HD + d] = acc / lsum;
    } else {
      float* pp = p.part + ((size_t)hh * p.max_splits + checked_index(split, p.max_splits, p.status)) * (HD + 2);
      pp[d] = acc;
      if (d == 0) { pp[HD] = M; pp[HD + 1] = lsum; }
    }
  }
}

// chunk = 8 waves x 16 or 32 positions; returns false for other chunks
bool launch_attn_split_b1(const AttnParams& p, hipStream_t s) {
  if (p.B != 1 || p.H != NW * REP || p.KV != NW || p.hd != HD || p.max_splits < 1) return false;
  if (p.chunk == NW * 16) hipLaunchKernelGGL(attn_split_b1_kernel<16>, dim3(p.max_splits, p.KV), dim3(WGT), 0, s, p);
  else if (p.chunk == NW * 32) hipLaunchKernelGGL(attn_split_b1_kernel<32>, dim3(p.max_splits, p.KV), dim3(WGT), 0, s, p);
  else return false;
  return true;
}
