// Batch-1 layer stack in one persistent launch (S2 shapes, bf16 weights and
// cache).
//
// At batch 1 every product of a layer streams 21-100 MB of weights that do
// not depend on the activations, yet with one launch per product the
// weight stream stops at every product boundary: the previous launch drains,
// the next one is dispatched, and its first loads take a full HBM round
// trip ([P2] "The slow AR is Qwen3-4B. The fast AR is not small": batch-1
// decode is bound by reading weights; the fast AR runs four layers ten times
// a frame).  Here one cooperative launch of 256 workgroups (one per compute
// unit, 8 waves each) runs a whole stack of layers.  Each workgroup owns a
// fixed slice of every product's rows.  Between two products it does not
// wait at a launch boundary: it first issues the loads of its slice of the
// next product's weights into registers, and only then waits for the
// product's input vector.
//
// Hand-off between workgroups: every value a product writes for the next one
// (the residual stream x, q|k|v, the SwiGLU output h) is stored as one
// 64-bit word, the fp32 bits in the low half and a tag in the high half,
// with a device-scope store; a consumer loads the words with device-scope
// loads until every tag is the one its producer phase writes.  Tags grow
// from launch to launch, so buffers need no clearing.  Waits are bounded:
// past the spin limit a status bit is latched (dualar_sync reports it) and
// the workgroup carries on, so every launch ends.
//
// Phases of a fast layer (the fast AR attends over at most num_codebooks
// positions, so every workgroup computes the whole attention itself):
//   Q   q|k|v = W_qkv RMSNorm(x)       24 rows per workgroup, 3 per wave
//   AO  x += W_o attention(q, k, v)    all heads per workgroup (wave w = KV
//                                      head w), 10 rows of W_o per workgroup
//   F1  h = silu(W1 n) * (W3 n), n = RMSNorm(x)   38 row pairs per workgroup
//   F2  x += W2 h                      10 rows per workgroup, the 19 units of
//                                      512 inputs split over the 8 waves
// The arithmetic is that of the per-product kernels: RMSNorm as a wave
// reduction, fp32 fused multiply-adds in a fixed order, wave sums, the
// attention of the batch-1 fused attention + O kernel.
#include "common.h"
#include "internal.h"

namespace {

constexpr int G = SB_GRID;           // workgroups
constexpr int NW = 8;                // waves per workgroup
constexpr int T = NW * 64;
constexpr int D = 2560, DU = D / 512;            // model width, 512-input units
constexpr int H = 32, KVH = 8, HD = 128, REP = 4;
constexpr int QROWS = (H + 2 * KVH) * HD;        // 6144
constexpr int ATT = H * HD, AU = ATT / 512;      // 4096, 8
constexpr int FF = 9728, FU = FF / 512;          // 9728, 19
constexpr int RQ = QROWS / G;                    // 24 rows of q|k|v per workgroup
constexpr int RO = D / G;                        // 10 rows of O and W2 per workgroup
constexpr int RP = FF / G;                       // 38 gate/up row pairs per workgroup
constexpr int MAXL = 16;                         // fast cache positions
constexpr int NPF = 20;                          // 16-byte weight loads held per lane
static_assert(RQ == 3 * NW && RO == 10 && RP == 38 && QROWS % G == 0 && D % G == 0 && FF % G == 0, "shapes");
typedef __bf16 sb_bf16x8 __attribute__((ext_vector_type(8)));
typedef float sb_f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64;

typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
typedef __attribute__((address_space(1))) u64 g_u64;

// 16 bytes at base + off: `base` is wave-uniform (a scalar register pair)
// and `off` the lane's 32-bit offset, so the load takes the scalar-base form.
__device__ __forceinline__ u32x4 ldw(const void* base, uint32_t off) {
  return __builtin_nontemporal_load((g_u32x4*)((const char*)base + off));
}

__device__ __forceinline__ void ll_put(u64* p, float v, unsigned tag) {
  __hip_atomic_store((g_u64*)p, ((u64)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool timed_out(const StackB1Params& p) {
  return __hip_atomic_load(p.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & ST_SYNC_TIMEOUT;
}

// Wait until words [0, n) of src all carry `tag` and copy their values to
// dst (LDS).  n <= 20 * T.  Ends with a workgroup barrier.  Each thread owns
// words tid + k T and polls them ten at a time.
__device__ __forceinline__ void ll_gather(const u64* src, int n, unsigned tag, float* dst, const StackB1Params& p) {
  const int tid = threadIdx.x;
  __syncthreads();   // every wave is done reading dst's previous contents
  // an opaque copy of the (loop-invariant) buffer address: its twenty lane
  // addresses are then formed here, not kept live across the whole kernel
  asm volatile("" : "+s"(src));
  constexpr int K = 10;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int b = tid + half * K * T;
    uint32_t pending = 0;
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (b + k * T < n) pending |= 1u << k;
    int spins = 0;
    while (pending) {
      u64 v[K];
#pragma unroll
      for (int k = 0; k < K; ++k)
        if (pending & (1u << k))
          v[k] = __hip_atomic_load((g_u64*)((const char*)(src + half * K * T + k * T) + (uint32_t)tid * 8),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int k = 0; k < K; ++k)
        if ((pending & (1u << k)) && (unsigned)(v[k] >> 32) == tag) {
          dst[b + k * T] = __uint_as_float((unsigned)v[k]);
          pending &= ~(1u << k);
        }
      if (pending) {
        ++spins;
        if (spins > p.spin_limit || ((spins & 255) == 0 && timed_out(p))) {
          atomicOr(p.status, ST_SYNC_TIMEOUT);
          break;
        }
      }
    }
  }
  __syncthreads();
}

// Plain copy of an fp32 vector written by an earlier launch.
__device__ __forceinline__ void plain_gather(const float* src, int n, float* dst) {
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += T) dst[i] = src[i];
  __syncthreads();
}

__device__ __forceinline__ const char* qkv_row(const B1Layer& L, int r) {
  if (r < H * HD) return (const char*)L.wq + (size_t)r * D * 2;
  r -= H * HD;
  if (r < KVH * HD) return (const char*)L.wk + (size_t)r * D * 2;
  return (const char*)L.wv + (size_t)(r - KVH * HD) * D * 2;
}

// The lane's 40 inputs of a 2560-wide row (units u = 0..4, elements
// 512 u + 8 lane .. +8), RMS-normalised with the gain.
__device__ __forceinline__ void norm_slice(const float* vin, const u32x4 (&gv)[DU], float eps, float (&xs)[DU][8]) {
  const int lane = threadIdx.x & 63;
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < DU; ++u) {
    const float4 a = *(const float4*)&vin[u * 512 + 8 * lane];
    const float4 b = *(const float4*)&vin[u * 512 + 8 * lane + 4];
    xs[u][0] = a.x; xs[u][1] = a.y; xs[u][2] = a.z; xs[u][3] = a.w;
    xs[u][4] = b.x; xs[u][5] = b.y; xs[u][6] = b.z; xs[u][7] = b.w;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += xs[u][e] * xs[u][e];
  }
  const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)D + eps);
#pragma unroll
  for (int u = 0; u < DU; ++u) {
    float g[8];
    ElemT<bf16_t>::unpack(gv[u], g);
#pragma unroll
    for (int e = 0; e < 8; ++e) xs[u][e] = xs[u][e] * inv * g[e];
  }
}

__device__ __forceinline__ float dot_row(const u32x4* w, const float (&xs)[DU][8]) {
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < DU; ++u) {
    float wf[8];
    ElemT<bf16_t>::unpack(w[u], wf);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(wf[e], xs[u][e], acc);
  }
  return wave_sum(acc);
}

__device__ __forceinline__ void load_gain(const void* g, u32x4 (&gv)[DU]) {
  const uint32_t loff = (threadIdx.x & 63) * 16;
#pragma unroll
  for (int u = 0; u < DU; ++u) gv[u] = *(g_u32x4*)((const char*)g + u * 1024 + loff);
}

struct Smem {
  float vin[FF];                                  // the phase's input vector
  float xres[RO];                                 // this workgroup's rows of x
  float part[NW][RO];
  uint16_t qp[NW][3][REP][HD];                    // q as three bf16 terms
  float kn[NW][HD];
  float sc[NW][REP][MAXL];
  float os[NW][REP * HD];
};

}  // namespace

__global__ void __launch_bounds__(T) stack_b1_kernel(StackB1Params p) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  // the wave index in a scalar register: row addresses are then scalar bases
  // plus a per-lane 32-bit offset
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.x;
  const int row0 = g * RO;
  u32x4 wpf[NPF];
  u32x4 gv[DU];

  if (threadIdx.x < RO) sm.xres[threadIdx.x] = p.x[row0 + threadIdx.x];
  const int nl = p.n_layer;
  auto tag_of = [&](int l, int ph) __attribute__((always_inline)) { return p.tag0 + (unsigned)(l * 4 + ph) + 1u; };

  // ---- issue helpers: the first weight loads of a phase into wpf ----
  const uint32_t loff = (uint32_t)lane * 16;   // the lane's 16 bytes of a 1 KB row unit
  auto issue_q = [&](const B1Layer& L, bool kv_only) __attribute__((always_inline)) {
    if (kv_only) {
      const char* base = qkv_row(L, H * HD + g * NW + wave);        // K|V rows: 8 per workgroup
#pragma unroll
      for (int u = 0; u < DU; ++u) wpf[u] = ldw(base + u * 1024, loff);
    } else {
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        const char* base = qkv_row(L, g * RQ + 3 * wave + r);
#pragma unroll
        for (int u = 0; u < DU; ++u) wpf[r * DU + u] = ldw(base + u * 1024, loff);
      }
    }
    load_gain(L.attn_norm, gv);
  };
  auto issue_o = [&](const B1Layer& L) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < RO; ++r) wpf[r] = ldw((const char*)L.wo + ((size_t)(row0 + r) * ATT + wave * 512) * 2, loff);
  };
  auto pair_load = [&](const B1Layer& L, int i, int slot) __attribute__((always_inline)) {
    const size_t pr = (size_t)(g * RP + wave + 8 * i) * D * 2;
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      wpf[slot * 10 + u] = ldw((const char*)L.w1 + pr + u * 1024, loff);
      wpf[slot * 10 + DU + u] = ldw((const char*)L.w3 + pr + u * 1024, loff);
    }
  };
  auto issue_f1 = [&](const B1Layer& L) __attribute__((always_inline)) {
    pair_load(L, 0, 0);
    pair_load(L, 1, 1);
    load_gain(L.ffn_norm, gv);
  };
  // W2: the wave's units wave, wave + 8 (and wave + 16 for waves 0..2) of
  // every row; units j = 0, 1 are prefetched, unit 2 loaded after the wait
  auto f2_unit_load = [&](const B1Layer& L, int j, int slot) __attribute__((always_inline)) {
    const int u = wave + 8 * j;
#pragma unroll
    for (int r = 0; r < RO; ++r) wpf[slot * RO + r] = ldw((const char*)L.w2 + ((size_t)(row0 + r) * FF + u * 512) * 2, loff);
  };
  auto issue_f2 = [&](const B1Layer& L) __attribute__((always_inline)) {
    f2_unit_load(L, 0, 0);
    f2_unit_load(L, 1, 1);
  };

  const bool kv_last = p.kv_only_last != 0;
  issue_q(p.layers[0], kv_last && nl == 1);

  for (int l = 0; l < nl; ++l) {
    const B1Layer& L = p.layers[l];
    const bool kv_only = kv_last && l == nl - 1;
    char* kc_l = (char*)p.kcache + (size_t)l * p.layer_stride * 2;
    char* vc_l = (char*)p.vcache + (size_t)l * p.layer_stride * 2;
    // opaque per-layer copies of loop-invariant parameters: the per-lane
    // addresses derived from them are formed where they are used instead of
    // being kept live across the whole launch
    int pos = p.pos, max_pos = p.max_pos;
    const float2* rope = p.rope;
    asm volatile("" : "+s"(pos), "+s"(max_pos), "+s"(rope));

    // ================= Q: q|k|v = W_qkv RMSNorm(x) =================
    if (l == 0) plain_gather(p.x, D, sm.vin);
    else ll_gather(p.ll_x, D, tag_of(l - 1, 3), sm.vin, p);
    {
      float xs[DU][8];
      norm_slice(sm.vin, gv, p.eps, xs);
      if (kv_only) {
        const float v = dot_row(&wpf[0], xs);
        if (lane == 0) ll_put(p.ll_qkv + H * HD + g * NW + wave, v, tag_of(l, 0));
      } else {
#pragma unroll
        for (int r = 0; r < 3; ++r) {
          const float v = dot_row(&wpf[r * DU], xs);
          if (lane == 0) ll_put(p.ll_qkv + g * RQ + 3 * wave + r, v, tag_of(l, 0));
        }
      }
    }
    if (kv_only) {
      // fast pass 0's last layer: only K and V at position pos reach the
      // cache (its attention output, O and FFN feed logits nobody reads)
      if (g == 0) {
        ll_gather(p.ll_qkv + H * HD, 2 * KVH * HD, tag_of(l, 0), sm.vin, p);
        const float2 cs = rope[(size_t)pos * (HD / 2) + lane];
        float a = sm.vin[wave * HD + 2 * lane], c = sm.vin[wave * HD + 2 * lane + 1];
        if (L.k_norm) {
          const uint32_t kg = ((const uint32_t*)L.k_norm)[lane];
          const float inv = 1.0f / sqrtf(wave_sum(a * a + c * c) / (float)HD + p.eps);
          a = a * inv * bf16_bits_to_f32(kg & 0xffffu);
          c = c * inv * bf16_bits_to_f32(kg >> 16);
        }
        const uint16_t ka = f32_to_bf16_rne(a * cs.x - c * cs.y), kb = f32_to_bf16_rne(a * cs.y + c * cs.x);
        const uint16_t va = f32_to_bf16_rne(sm.vin[KVH * HD + wave * HD + 2 * lane]);
        const uint16_t vb = f32_to_bf16_rne(sm.vin[KVH * HD + wave * HD + 2 * lane + 1]);
        const size_t at = ((size_t)wave * max_pos + pos) * HD + 2 * lane;
        *(uint32_t*)(kc_l + at * 2) = (uint32_t)ka | ((uint32_t)kb << 16);
        *(uint32_t*)(vc_l + at * 2) = (uint32_t)va | ((uint32_t)vb << 16);
      }
      break;
    }

    // ================= AO: x += W_o attention(q, k, v) =================
    issue_o(L);
    const int Lc = pos + 1;
    const int jm = lane & 15, kq = lane >> 4;
    u32x4 kcr[4];
    {
      const int jl = jm < pos ? jm : 0;   // positions past pos read position 0 and are not used
      const char* src = kc_l + (((size_t)wave * max_pos + jl) * HD + 8 * kq) * 2;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kcr[ks] = ld_vec(src + 64 * ks);
    }
    uint32_t vcr[MAXL];
    {
      const uint32_t* src = (const uint32_t*)(vc_l + ((size_t)wave * max_pos * HD + 2 * lane) * 2);
#pragma unroll
      for (int jj = 0; jj < MAXL; ++jj) vcr[jj] = jj < pos ? src[(size_t)jj * (HD / 2)] : 0u;
    }
    uint32_t qg = 0x3f803f80u, kg = 0x3f803f80u;
    if (L.q_norm) qg = ((const uint32_t*)L.q_norm)[lane];
    if (L.k_norm) kg = ((const uint32_t*)L.k_norm)[lane];
    const float2 cs = rope[(size_t)pos * (HD / 2) + lane];
    ll_gather(p.ll_qkv, QROWS, tag_of(l, 0), sm.vin, p);
    {
      const float qscale = 1.0f / sqrtf((float)HD);
#pragma unroll
      for (int h4 = 0; h4 < REP; ++h4) {
        float a = sm.vin[(wave * REP + h4) * HD + 2 * lane], c = sm.vin[(wave * REP + h4) * HD + 2 * lane + 1];
        if (L.q_norm) {
          const float inv = 1.0f / sqrtf(wave_sum(a * a + c * c) / (float)HD + p.eps);
          a = a * inv * bf16_bits_to_f32(qg & 0xffffu);
          c = c * inv * bf16_bits_to_f32(qg >> 16);
        }
        const float ra = (a * cs.x - c * cs.y) * qscale, rc = (a * cs.y + c * cs.x) * qscale;
        const uint16_t a0 = f32_to_bf16_rne(ra), c0 = f32_to_bf16_rne(rc);
        const float a1f = ra - bf16_bits_to_f32(a0), c1f = rc - bf16_bits_to_f32(c0);
        const uint16_t a1 = f32_to_bf16_rne(a1f), c1 = f32_to_bf16_rne(c1f);
        const uint16_t a2 = f32_to_bf16_rne(a1f - bf16_bits_to_f32(a1));
        const uint16_t c2 = f32_to_bf16_rne(c1f - bf16_bits_to_f32(c1));
        *(uint32_t*)&sm.qp[wave][0][h4][2 * lane] = (uint32_t)a0 | ((uint32_t)c0 << 16);
        *(uint32_t*)&sm.qp[wave][1][h4][2 * lane] = (uint32_t)a1 | ((uint32_t)c1 << 16);
        *(uint32_t*)&sm.qp[wave][2][h4][2 * lane] = (uint32_t)a2 | ((uint32_t)c2 << 16);
      }
    }
    float vn0, vn1;
    {
      float a = sm.vin[H * HD + wave * HD + 2 * lane], c = sm.vin[H * HD + wave * HD + 2 * lane + 1];
      if (L.k_norm) {
        const float inv = 1.0f / sqrtf(wave_sum(a * a + c * c) / (float)HD + p.eps);
        a = a * inv * bf16_bits_to_f32(kg & 0xffffu);
        c = c * inv * bf16_bits_to_f32(kg >> 16);
      }
      const uint16_t ka = f32_to_bf16_rne(a * cs.x - c * cs.y), kb = f32_to_bf16_rne(a * cs.y + c * cs.x);
      const uint16_t va = f32_to_bf16_rne(sm.vin[(H + KVH) * HD + wave * HD + 2 * lane]);
      const uint16_t vb = f32_to_bf16_rne(sm.vin[(H + KVH) * HD + wave * HD + 2 * lane + 1]);
      sm.kn[wave][2 * lane] = bf16_bits_to_f32(ka);
      sm.kn[wave][2 * lane + 1] = bf16_bits_to_f32(kb);
      vn0 = bf16_bits_to_f32(va);
      vn1 = bf16_bits_to_f32(vb);
      if (g == 0) {
        const size_t at = ((size_t)wave * max_pos + pos) * HD + 2 * lane;
        *(uint32_t*)(kc_l + at * 2) = (uint32_t)ka | ((uint32_t)kb << 16);
        *(uint32_t*)(vc_l + at * 2) = (uint32_t)va | ((uint32_t)vb << 16);
      }
    }
    __builtin_amdgcn_wave_barrier();   // qp[wave], kn[wave]: this wave's own
    {
      // S^T = K q^T on the matrix cores (positions as A, the 4 query heads'
      // three bf16 terms as B), softmax across the four lane groups
      sb_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        sb_bf16x8 a = __builtin_bit_cast(sb_bf16x8, kcr[ks]);
        if (jm == pos) {
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] = (__bf16)sm.kn[wave][32 * ks + 8 * kq + e];
        }
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          const u32x4 b = *(const u32x4*)&sm.qp[wave][t][jm & 3][32 * ks + 8 * kq];
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(sb_bf16x8, b), acc, 0, 0, 0);
        }
      }
      float sv[4];
      float m = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[r] = 4 * kq + r < Lc ? acc[r] : -INFINITY;
        m = fmaxf(m, sv[r]);
      }
      m = max_xor16(m);
      m = max_xor32(m);
      float lsum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[r] = 4 * kq + r < Lc ? expf(sv[r] - m) : 0.f;
        lsum += sv[r];
      }
      lsum = add_xor16(lsum);
      lsum = add_xor32(lsum);
      if (jm < REP) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.sc[wave][jm][4 * kq + r] = sv[r] / lsum;
      }
    }
    __builtin_amdgcn_wave_barrier();
    {
      float o[REP][2];
#pragma unroll
      for (int h4 = 0; h4 < REP; ++h4) o[h4][0] = o[h4][1] = 0.f;
#pragma unroll
      for (int jj = 0; jj < MAXL; ++jj) {
        if (jj < Lc) {
          float va, vb;
          if (jj == pos) { va = vn0; vb = vn1; }
          else { va = bf16_bits_to_f32(vcr[jj] & 0xffffu); vb = bf16_bits_to_f32(vcr[jj] >> 16); }
#pragma unroll
          for (int h4 = 0; h4 < REP; ++h4) {
            const float pr = sm.sc[wave][h4][jj];
            o[h4][0] = fmaf(pr, va, o[h4][0]);
            o[h4][1] = fmaf(pr, vb, o[h4][1]);
          }
        }
      }
#pragma unroll
      for (int h4 = 0; h4 < REP; ++h4) *(float2*)&sm.os[wave][h4 * HD + 2 * lane] = make_float2(o[h4][0], o[h4][1]);
    }
    __builtin_amdgcn_wave_barrier();   // os[wave]: this wave's own
    {
      float ov[8];
      const float4 t0 = *(const float4*)&sm.os[wave][lane * 8];
      const float4 t1 = *(const float4*)&sm.os[wave][lane * 8 + 4];
      ov[0] = t0.x; ov[1] = t0.y; ov[2] = t0.z; ov[3] = t0.w;
      ov[4] = t1.x; ov[5] = t1.y; ov[6] = t1.z; ov[7] = t1.w;
#pragma unroll
      for (int r = 0; r < RO; ++r) {
        float wf[8];
        ElemT<bf16_t>::unpack(wpf[r], wf);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(wf[e], ov[e], acc);
        acc = wave_sum(acc);
        if (lane == 0) sm.part[wave][r] = acc;
      }
    }
    __syncthreads();
    if (threadIdx.x < RO) {
      const int r = threadIdx.x;
      float v = sm.part[0][r];
#pragma unroll
      for (int q = 1; q < NW; ++q) v += sm.part[q][r];
      const float xn = sm.xres[r] + v;
      sm.xres[r] = xn;
      ll_put(p.ll_x + row0 + r, xn, tag_of(l, 1));
    }
    issue_f1(L);

    // ================= F1: h = silu(W1 n) * (W3 n) =================
    ll_gather(p.ll_x, D, tag_of(l, 1), sm.vin, p);
    {
      float xs[DU][8];
      norm_slice(sm.vin, gv, p.eps, xs);
      auto pair = [&](int i, int slot) __attribute__((always_inline)) {
        const float gt = dot_row(&wpf[slot * 10], xs);
        const float up = dot_row(&wpf[slot * 10 + DU], xs);
        if (lane == 0) ll_put(p.ll_h + g * RP + wave + 8 * i, silu_f(gt) * up, tag_of(l, 2));
      };
      // two pairs in flight: pair i + 2 is loaded into the slot pair i frees
      // (pairs wave + 8 i, i < 4 for every wave, i = 4 for waves 0..5)
      const bool five = wave + 32 < RP;
      pair(0, 0);
      pair_load(L, 2, 0);
      pair(1, 1);
      pair_load(L, 3, 1);
      pair(2, 0);
      if (five) pair_load(L, 4, 0);
      pair(3, 1);
      if (five) pair(4, 0);
    }
    issue_f2(L);

    // ================= F2: x += W2 h =================
    ll_gather(p.ll_h, FF, tag_of(l, 2), sm.vin, p);
    {
      float acc[RO];
#pragma unroll
      for (int r = 0; r < RO; ++r) acc[r] = 0.f;
      auto unit = [&](int j, int slot) __attribute__((always_inline)) {
        const int u = wave + 8 * j;
        const float4 a = *(const float4*)&sm.vin[u * 512 + 8 * lane];
        const float4 b = *(const float4*)&sm.vin[u * 512 + 8 * lane + 4];
#pragma unroll
        for (int r = 0; r < RO; ++r) {
          float wf[8];
          ElemT<bf16_t>::unpack(wpf[slot * RO + r], wf);
          acc[r] = fmaf(wf[0], a.x, acc[r]); acc[r] = fmaf(wf[1], a.y, acc[r]);
          acc[r] = fmaf(wf[2], a.z, acc[r]); acc[r] = fmaf(wf[3], a.w, acc[r]);
          acc[r] = fmaf(wf[4], b.x, acc[r]); acc[r] = fmaf(wf[5], b.y, acc[r]);
          acc[r] = fmaf(wf[6], b.z, acc[r]); acc[r] = fmaf(wf[7], b.w, acc[r]);
        }
      };
      const bool three = wave + 16 < FU;
      unit(0, 0);
      if (three) f2_unit_load(L, 2, 0);
      unit(1, 1);
      if (three) unit(2, 0);
#pragma unroll
      for (int r = 0; r < RO; ++r) {
        const float v = wave_sum(acc[r]);
        if (lane == 0) sm.part[wave][r] = v;
      }
    }
    __syncthreads();
    if (threadIdx.x < RO) {
      const int r = threadIdx.x;
      float v = sm.part[0][r];
#pragma unroll
      for (int q = 1; q < NW; ++q) v += sm.part[q][r];
      const float xn = sm.xres[r] + v;
      sm.xres[r] = xn;
      ll_put(p.ll_x + row0 + r, xn, tag_of(l, 3));
    }
    if (l + 1 < nl) issue_q(p.layers[l + 1], kv_last && l + 1 == nl - 1);
    // sm.part and sm.vin are rewritten only after the next gather's barrier
  }
  if (threadIdx.x < RO) p.x[row0 + threadIdx.x] = sm.xres[threadIdx.x];
}

bool stack_b1_fits(int dim, int H_, int KV_, int hd, int ffn, int n_pos) {
  return dim == D && H_ == H && KV_ == KVH && hd == HD && ffn == FF && n_pos >= 1 && n_pos <= MAXL;
}

hipError_t launch_stack_b1(const StackB1Params& p, hipStream_t s) {
  if (p.n_layer < 1 || p.pos < 0 || p.pos >= p.max_pos || p.pos >= MAXL) return hipErrorInvalidValue;
  void* args[] = {const_cast<StackB1Params*>(&p)};
  return hipLaunchCooperativeKernel((const void*)stack_b1_kernel, dim3(G), dim3(T), args, 0, s);
}

int stack_b1_max_blocks() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void*)stack_b1_kernel, T, 0) != hipSuccess) return 0;
  return n;
}
