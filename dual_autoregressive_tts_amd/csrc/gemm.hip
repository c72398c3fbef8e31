// Matrix products for 8..32+ activation rows (batched decode, batched
// prefill steps) on the gfx950 matrix cores: Y[b][n] = sum_k W[n][k] X[b][k].
//
// v_mfma_f32_32x32x16_bf16 with W as the A operand (32 output rows; lane l
// holds W[n0 + l%32][k + 8*(l/32) .. +8]) and the activations as the B
// operand (32 activation rows; lane l holds X[b0 + l%32][k + 8*(l/32) .. +8]).
// Activations are fp32: xsplit_kernel splits each into three bf16 terms,
// x = t0 + t1 + t2 + r with t0 = bf16(x), t1 = bf16(x - t0),
// t2 = bf16(x - t0 - t1) (every subtraction exact in fp32, |r| <= 2^-24 |x|),
// stored as three planes, and the three products are accumulated in fp32
// (one accumulator per term, added smallest first at the end).  The weights are bf16
// already, so the product is the fp32 product of the stored weights and the
// fp32 activations up to accumulation order.  (Two terms would leave ~2^-17
// relative error per activation, enough to move bf16-rounded K/V entries one
// ulp far more often than fp32 rounding order does.)
//
// Memory path.  Read straight in the operand layout, every load instruction
// touches 32 rows, i.e. 32 cache lines per KB, and the activation operand
// costs two such loads per step: the cache-line request rate, not HBM, then
// bounds the kernel.  Here both operands go through LDS instead.  A workgroup
// owns ROWS output rows (gate and up rows for SwiGLU) and one 32-row
// activation tile, and walks its K range in chunks of 64: each chunk of
// weights (ROWS*NR rows x 128 B) and activation planes (3 x 32 rows x 128 B)
// is copied by LDS DMA (global_load_lds_dwordx4: lane i's 16 bytes land at
// the wave's LDS base + 16 i), each instruction covering 8 whole 128-byte
// lines.
// Pieces are XOR-swizzled within their row so that the operand-layout LDS
// reads are bank-conflict free.  Three stages: while a chunk is multiplied
// the next two are in flight; one barrier per chunk.  Waves split rows, not
// K, so no cross-wave reduction is needed; the epilogue goes through LDS so
// that each store writes 128-byte runs.  With ksw > 1 the workgroups of a
// row block write partial sums that mfma_finish_kernel adds in a fixed order.
// RMSNorm, when the product has a gain, is applied by xsplit_kernel.
#include "mfma.h"

#define GM_KC 64                     // k per chunk
#define GM_STAGES 3
#define GM_TILE_ROWS GEMM_TILE_MIN_ROWS   // from this many activation rows: 2-D tiles (gemm_tile.hip)

// Workgroup shape: WAVES waves, each owning T 32-row output tiles (times NR
// segments); the workgroup covers ROWS = 32*WAVES*T output rows.
template <int NR, int WAVES, int T> struct Gm {
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int ROWS = 32 * WAVES * T;
  static constexpr int W_BYTES = ROWS * NR * GM_KC * 2;     // weight chunk
  static constexpr int X_BYTES = 3 * 32 * GM_KC * 2;        // activation planes chunk
  static constexpr int STAGE = W_BYTES + X_BYTES;
  static constexpr int W_INSTR = W_BYTES / 1024 / WAVES;     // DMA instructions per wave per chunk
  static constexpr int X_INSTR = X_BYTES / 1024 / WAVES;
  static constexpr int DMA = W_INSTR + X_INSTR;
  static_assert(W_BYTES % (1024 * WAVES) == 0 && X_BYTES % (1024 * WAVES) == 0, "DMA split");
  static_assert((WAVES > 3 ? 2 : 1) * NR * T * 32 * 33 * 4 <= STAGE, "epilogue transposes fit the stages");
};


// Per-lane DMA sources of this workgroup's chunk 0; chunk c adds c*64
// elements.
template <class G> struct GmSrc {
  const char* w[G::W_INSTR];
  const char* x[G::X_INSTR];
};

// Weight row r of a chunk (segment r / ROWS, output row n0 + r % ROWS)
// lands at r*128 + 16*(piece ^ ((r >> 1) & 7)); activation row rr at
// rr*256 + 16*(piece ^ (rr & 15)).
template <int NR, class G>
__device__ __forceinline__ void gm_sources(const GemvParams& p, GmSrc<G>& src, int n0, int b0, int kbeg, int wave,
                                           int lane) {
  const RowSpace rs(p);
#pragma unroll
  for (int j = 0; j < G::W_INSTR; ++j) {
    const int i = wave * G::W_INSTR + j;
    const int r = 8 * i + (lane >> 3);
    const int piece = (lane & 7) ^ ((r >> 1) & 7);
    const int n = min(n0 + r % G::ROWS, p.n_out - 1);
    src.w[j] = rs.row(n, r / G::ROWS) + (size_t)(kbeg + piece * 8) * 2;
  }
  // activation plane q, row rr (0..31) of a chunk lands at
  // q*4096 + rr*128 + 16*(piece ^ ((rr >> 1) & 7)), like the weights
  const uint16_t* xs = (const uint16_t*)p.xn;
  const size_t plane = (size_t)p.B * p.K;
#pragma unroll
  for (int j = 0; j < G::X_INSTR; ++j) {
    const int i = wave * G::X_INSTR + j;            // 0..11
    const int q = i >> 2, rr = 8 * (i & 3) + (lane >> 3);
    const int piece = (lane & 7) ^ ((rr >> 1) & 7);
    const int b = b0 + rr < p.B ? b0 + rr : 0;      // padding columns: never stored
    src.x[j] = (const char*)(xs + q * plane + (size_t)b * p.K + kbeg + piece * 8);
  }
}

template <class G>
__device__ __forceinline__ void gm_issue(const GmSrc<G>& src, char* stage, int c, int wave) {
#pragma unroll
  for (int j = 0; j < G::W_INSTR; ++j)
    dma16(src.w[j] + (size_t)c * GM_KC * 2, stage + (wave * G::W_INSTR + j) * 1024);
  char* xs = stage + G::W_BYTES;
#pragma unroll
  for (int j = 0; j < G::X_INSTR; ++j)
    dma16(src.x[j] + (size_t)c * GM_KC * 2, xs + (wave * G::X_INSTR + j) * 1024);
}

// The four 16-wide k-steps of one chunk.  The three activation terms are
// read once per step and used for the wave's T tiles and NR segments; each
// term has its own accumulator, so the three products of a step do not wait
// on each other.
template <int NR, int T, class G>
__device__ __forceinline__ void gm_compute_wx(const char* stage, const char* xs, int wave, int lane,
                                              f32x16 (*acc)[NR][3]) {
  const int h = lane >> 5, b = lane & 31;
  const int bsw = (b >> 1) & 7;
#pragma unroll
  for (int t = 0; t < GM_KC / 16; ++t) {
    const int pc = 2 * t + h;
    bf16x8 tx[3];
#pragma unroll
    for (int q = 0; q < 3; ++q) tx[q] = *(const bf16x8*)(xs + q * 4096 + b * 128 + ((pc ^ bsw) << 4));
#pragma unroll
    for (int tt = 0; tt < T; ++tt)
#pragma unroll
      for (int s = 0; s < NR; ++s) {
        const int r = s * G::ROWS + 32 * (wave * T + tt) + b;
        const bf16x8 av = *(const bf16x8*)(stage + r * 128 + ((pc ^ ((r >> 1) & 7)) << 4));
#pragma unroll
        for (int q = 0; q < 3; ++q)
          acc[tt][s][q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, tx[q], acc[tt][s][q], 0, 0, 0);
      }
  }
}
template <int NR, int T, class G>
__device__ __forceinline__ void gm_compute(const char* stage, int wave, int lane, f32x16 (*acc)[NR][3]) {
  gm_compute_wx<NR, T, G>(stage, stage + G::W_BYTES, wave, lane, acc);
}

// One pipeline step: chunk cc from stage S; chunk cc+2 goes to stage
// (S+2)%3.  This wave's copies of chunk cc are done once at most the next
// chunk's are outstanding; after the barrier every wave's are, and every
// wave has finished reading the stage that chunk cc+2 overwrites.
template <int NR, int T, class G, int S>
__device__ __forceinline__ void gm_step(const GmSrc<G>& src, char* st0, char* st1, char* st2, int cc, int nch,
                                        int wave, int lane, f32x16 (*acc)[NR][3]) {
  char* const cur = S == 0 ? st0 : (S == 1 ? st1 : st2);
  char* const nxt = S == 0 ? st2 : (S == 1 ? st0 : st1);     // stage (S+2)%3
  if (cc + 1 < nch) wait_vm_barrier<G::DMA>();
  else wait_vm_barrier<0>();
  if (cc + 2 < nch) gm_issue<G>(src, nxt, cc + 2, wave);
  gm_compute<NR, T, G>(cur, wave, lane, acc);
}

// Grid (ceil(n_out/ROWS), ksw, ceil(B/32)), THREADS threads.  The host
// guarantees K % (ksw*64) == 0.
template <int NR, int WAVES, int T>
__global__ void __launch_bounds__(64 * WAVES) mfma_gemm_kernel(GemvParams p) {
  using G = Gm<NR, WAVES, T>;
  __shared__ __attribute__((aligned(1024))) char st0[G::STAGE];
  __shared__ __attribute__((aligned(1024))) char st1[G::STAGE];
  __shared__ __attribute__((aligned(1024))) char st2[G::STAGE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int nt = blockIdx.x, kw = blockIdx.y, zt = blockIdx.z;
  if (p.zswz) {   // one-dimensional grid: id = 8 * (q * zswz + z) + xcd, row block 8 * q + xcd
    const int id = blockIdx.x, xcd = id & 7, t = id >> 3;
    nt = 8 * (t / p.zswz) + xcd;
    zt = t % p.zswz;
    kw = 0;
    if (nt * G::ROWS >= p.n_out) return;
  }
  const int n0 = nt * G::ROWS, b0 = zt * 32;
  const int Kw = p.K / p.ksw, kbeg = kw * Kw;
  const int nch = Kw / GM_KC;

  f32x16 acc[T][NR][3];
#pragma unroll
  for (int tt = 0; tt < T; ++tt)
#pragma unroll
    for (int s = 0; s < NR; ++s)
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tt][s][j][r] = 0.f;

  GmSrc<G> src;
  gm_sources<NR, G>(p, src, n0, b0, kbeg, wave, lane);
  gm_issue<G>(src, st0, 0, wave);
  if (nch > 1) gm_issue<G>(src, st1, 1, wave);
  for (int c = 0; c < nch; c += 3) {
    gm_step<NR, T, G, 0>(src, st0, st1, st2, c, nch, wave, lane, acc);
    if (c + 1 >= nch) break;
    gm_step<NR, T, G, 1>(src, st0, st1, st2, c + 1, nch, wave, lane, acc);
    if (c + 2 >= nch) break;
    gm_step<NR, T, G, 2>(src, st0, st1, st2, c + 2, nch, wave, lane, acc);
  }

  // Epilogue.  The three term sums are added smallest first; D[row][col] of
  // register r in lane l is at row (r/4)*8 + (l/32)*4 + r%4, col l%32.
  // Transpose through this wave's slice of stage 0..2 so that lanes 0..31
  // store 32 consecutive outputs of one b.
  __syncthreads();
  char* const mine = wave % 3 == 0 ? st0 : (wave % 3 == 1 ? st1 : st2);
  float* tr = (float*)mine + (wave / 3) * (T * NR * 32 * 33);
#pragma unroll
  for (int tt = 0; tt < T; ++tt)
#pragma unroll
    for (int s = 0; s < NR; ++s)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        tr[((tt * NR + s) * 32 + (lane & 31)) * 33 + row] = acc[tt][s][0][r] + (acc[tt][s][1][r] + acc[tt][s][2][r]);
      }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  const int nl = lane & 31;
#pragma unroll
  for (int tt = 0; tt < T; ++tt) {
    const int n = n0 + 32 * (wave * T + tt) + nl;
    if (n >= p.n_out) continue;
#pragma unroll 4
    for (int j = 0; j < 16; ++j) {
      const int bl = 2 * j + (lane >> 5), b = b0 + bl;
      if (b >= p.B) continue;
      float v[NR];
#pragma unroll
      for (int s = 0; s < NR; ++s) v[s] = tr[((tt * NR + s) * 32 + bl) * 33 + nl];
      if (p.ksw > 1) {
        float* dst = p.part + ((size_t)kw * p.B + b) * p.ldp;
#pragma unroll
        for (int s = 0; s < NR; ++s) dst[(size_t)s * p.n_out + n] = v[s];
      } else {
        float out;
        if (p.mode == GEMV_SWIGLU) out = silu_f(v[0]) * v[NR - 1];
        else if (p.mode == GEMV_ADD) out = p.res[(size_t)b * p.ldres + n] + v[0];
        else out = v[0];
        if (p.yplanes) store_planes((uint16_t*)p.yplanes, (size_t)p.B * p.n_out, (size_t)b * p.n_out + n, out);
        else p.y[(size_t)b * p.ldy + n] = out;
      }
    }
  }
}

#define FIN_MAXK 32   // largest K split
#define FIN_BATCH 8   // partials loaded together

// Sum the ksw partials (fixed order, kw = 0, 1, ...) and apply the epilogue.
__global__ void __launch_bounds__(DUALAR_WG) mfma_finish_kernel(GemvParams p) {
  const size_t i = (size_t)blockIdx.x * DUALAR_WG + threadIdx.x;
  if (i >= (size_t)p.B * p.n_out) return;
  const int b = (int)(i / p.n_out), n = (int)(i % p.n_out);
  const bool glu = p.mode == GEMV_SWIGLU;
  const float r = p.mode == GEMV_ADD ? p.res[(size_t)b * p.ldres + n] : 0.f;
  float v0 = 0.f, v1 = 0.f;
  for (int k0 = 0; k0 < p.ksw; k0 += FIN_BATCH) {
    float g[FIN_BATCH], u[FIN_BATCH];
#pragma unroll
    for (int j = 0; j < FIN_BATCH; ++j) {
      if (k0 + j < p.ksw) {
        const float* src = p.part + ((size_t)(k0 + j) * p.B + b) * p.ldp;
        g[j] = src[n];
        u[j] = glu ? src[(size_t)p.n_out + n] : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < FIN_BATCH; ++j) {
      if (k0 + j < p.ksw) {
        v0 += g[j];
        v1 += u[j];
      }
    }
  }
  float out;
  if (glu) out = silu_f(v0) * v1;
  else if (p.mode == GEMV_ADD) out = r + v0;
  else out = v0;
  if (p.yplanes) store_planes((uint16_t*)p.yplanes, (size_t)p.B * p.n_out, (size_t)b * p.n_out + n, out);
  else p.y[(size_t)b * p.ldy + n] = out;
}

#define NORM_MAXV 12   // float4s per thread: K <= 12288

// Split row b of the activations into three bf16 planes (x = t0 + t1 + t2
// + r, |r| <= 2^-24 |x|): plane q at xn + q*B*K.  With a gain the row is
// first RMS-normalised: x / sqrt(mean(x^2) + eps) * g.  One workgroup per
// row; the row is read once, with every load issued before the first use.
__global__ void __launch_bounds__(DUALAR_WG) xsplit_kernel(GemvParams p) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float red[4];
  const float4* x = (const float4*)(p.x + (size_t)b * p.ldx);
  const int nv = p.K / 4;
  float4 v[NORM_MAXV];
#pragma unroll
  for (int j = 0; j < NORM_MAXV; ++j)
    if (tid + j * DUALAR_WG < nv) v[j] = x[tid + j * DUALAR_WG];
  float inv = 1.f;
  if (p.gain) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NORM_MAXV; ++j)
      if (tid + j * DUALAR_WG < nv) ss += (v[j].x * v[j].x + v[j].y * v[j].y) + (v[j].z * v[j].z + v[j].w * v[j].w);
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    inv = 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)p.K + p.eps);
  }
  const uint2* g = (const uint2*)p.gain;
  uint2* xs = (uint2*)p.xn;
  const size_t plane = (size_t)p.B * p.K / 4;      // in 4-element units
#pragma unroll
  for (int j = 0; j < NORM_MAXV; ++j) {
    const int k = tid + j * DUALAR_WG;
    if (k < nv) {
      float o[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
      if (p.gain) {
        const uint2 gg = g[k];
        o[0] = o[0] * inv * bf16_bits_to_f32(gg.x & 0xffffu);
        o[1] = o[1] * inv * bf16_bits_to_f32(gg.x >> 16);
        o[2] = o[2] * inv * bf16_bits_to_f32(gg.y & 0xffffu);
        o[3] = o[3] * inv * bf16_bits_to_f32(gg.y >> 16);
      }
      uint32_t t[3][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t a0 = f32_to_bf16_rne(o[e]);
        const float r1 = o[e] - bf16_bits_to_f32(a0);
        const uint16_t a1 = f32_to_bf16_rne(r1);
        t[0][e] = a0;
        t[1][e] = a1;
        t[2][e] = f32_to_bf16_rne(r1 - bf16_bits_to_f32(a1));
      }
      const size_t at = (size_t)b * nv + k;
#pragma unroll
      for (int q = 0; q < 3; ++q) xs[q * plane + at] = make_uint2(t[q][0] | (t[q][1] << 16), t[q][2] | (t[q][3] << 16));
    }
  }
}

// Split-K finish of a residual product fused with the next product's input
// preparation, one workgroup per row b (n_out <= 4096): out = res +
// sum_kw part[kw] (the partials added in kw order, as in mfma_finish_kernel,
// loaded six splits at a time), written to y; then
// out / sqrt(mean(out^2) + eps) * next_gain split into three bf16 planes
// (plane stride B*n_out).
__global__ void __launch_bounds__(DUALAR_WG) finish_split_kernel(GemvParams p) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float red[4];
  const int nv = p.n_out / 4;
  constexpr int J = 4;              // float4s per thread: n_out <= 4096 on this path
  constexpr int KB = 6;             // partials loaded together
  float4 v[J];
#pragma unroll
  for (int j = 0; j < J; ++j) v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* pb = p.part + (size_t)b * p.ldp;
  const size_t kstride = (size_t)p.B * p.ldp;
  for (int k0 = 0; k0 < p.ksw; k0 += KB) {
    float4 q[KB][J];
#pragma unroll
    for (int u = 0; u < KB; ++u)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int k = tid + j * DUALAR_WG;
        q[u][j] = (k0 + u < p.ksw && k < nv) ? *(const float4*)(pb + (k0 + u) * kstride + 4 * k)
                                              : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
    for (int u = 0; u < KB; ++u)       // kw order, as in mfma_finish_kernel
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (k0 + u < p.ksw) { v[j].x += q[u][j].x; v[j].y += q[u][j].y; v[j].z += q[u][j].z; v[j].w += q[u][j].w; }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int k = tid + j * DUALAR_WG;
    if (k < nv) {
      const float4 r = *(const float4*)(p.res + (size_t)b * p.ldres + 4 * k);
      float4 a = v[j];
      a.x = r.x + a.x; a.y = r.y + a.y; a.z = r.z + a.z; a.w = r.w + a.w;
      *(float4*)(p.y + (size_t)b * p.ldy + 4 * k) = a;
      ss += (a.x * a.x + a.y * a.y) + (a.z * a.z + a.w * a.w);
      v[j] = a;
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)p.n_out + p.eps);
  const uint2* g = (const uint2*)p.next_gain;
  uint2* xs = (uint2*)p.next_planes;
  const size_t plane = (size_t)p.B * nv;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int k = tid + j * DUALAR_WG;
    if (k < nv) {
      const uint2 gg = g[k];
      float o[4] = {v[j].x * inv * bf16_bits_to_f32(gg.x & 0xffffu), v[j].y * inv * bf16_bits_to_f32(gg.x >> 16),
                    v[j].z * inv * bf16_bits_to_f32(gg.y & 0xffffu), v[j].w * inv * bf16_bits_to_f32(gg.y >> 16)};
      uint32_t t[3][4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t a0 = f32_to_bf16_rne(o[e]);
        const float r1 = o[e] - bf16_bits_to_f32(a0);
        const uint16_t a1 = f32_to_bf16_rne(r1);
        t[0][e] = a0;
        t[1][e] = a1;
        t[2][e] = f32_to_bf16_rne(r1 - bf16_bits_to_f32(a1));
      }
      const size_t at = (size_t)b * nv + k;
#pragma unroll
      for (int q = 0; q < 3; ++q) xs[q * plane + at] = make_uint2(t[q][0] | (t[q][1] << 16), t[q][2] | (t[q][3] << 16));
    }
  }
}

// ---------------------------------------------------------------------------
// Stream-K form for the decode shapes (one or two activation tiles, K of
// 2560..9728, a few dozen row tiles).  Split-K over a grid sized to the
// chip leaves whole rounds of workgroups waiting on a few (76 row blocks x 4
// splits = 304 workgroups for 256 compute units take two rounds), and short
// K ranges spend most of their time filling the pipeline.  Here the tiles'
// 64-wide chunks, in (tile, chunk) order, are dealt out as U work units:
// workgroup g of the grid (one per slot the chip holds) takes q or q + 1
// consecutive units, so every workgroup streams the same number of weight
// bytes, and its copy pipeline runs on across tile boundaries.  Where a
// workgroup's range leaves a tile it writes that tile's partial sums to slot
// (g - first owner of the tile) of the tile's partial area, laid out
// [slot][segment s][activation row 0..31][tile row] so that a finish kernel
// reads each activation row's sums as contiguous runs; it adds a tile's
// slots in slot order and applies the epilogue.
// ---------------------------------------------------------------------------

// Workgroup that owns unit u when U = q*G + r units go q + 1 to each of the
// first r workgroups and q to the rest.
__host__ __device__ __forceinline__ int sk_owner(int u, int q, int r) {
  const int big = r * (q + 1);
  return u < big ? u / (q + 1) : r + (u - big) / q;
}

template <int NR, int WAVES, int T>
struct Sk {
  static constexpr int BLOCKS = WAVES * T;                 // 32-row blocks per tile
  static constexpr int ROWS = 32 * BLOCKS;
  static constexpr int TE = NR * 32 * ROWS;                 // floats per partial tile
};

// Wave-specialised stream-K.  A form whose LDS stages each hold a weight
// chunk and the 12 KB of activation planes it is multiplied with keeps at
// most 48-64 KB of weights in flight per compute unit, because a wave's
// copies complete in issue order.  Here WAVES compute waves copy only
// the weight chunks (WS stages, WS - 1 chunks ahead) and multiply, and one
// more wave copies only the planes (XS slots, XS - 1 chunks ahead): each
// wave's vmcnt then counts one kind of copy, waiting for a chunk's planes
// never waits for newer weight copies, and the LDS the planes no longer
// share holds the weight pipeline.  The planes must be copied as far ahead
// as the weights: a compute unit's copies appear to be served in issue
// order across its waves, so planes issued one chunk ahead still wait
// behind every weight chunk in flight (batch 32: weights 2 chunks ahead and
// planes 1 ahead took 36.8 us for W1|W3, both 2 ahead 33.9 us; for the
// other products 4 and 4 matched 5 and 3, 6 and 4).  One barrier per chunk
// for all waves; the partial tiles are laid out as described above.
template <int NR, int WAVES, int T, int WS, int XS>
struct Skw {
  using G = Gm<NR, WAVES, T>;
  static constexpr int WI = G::W_BYTES / 1024 / WAVES;   // weight copies per compute wave per chunk
  static constexpr int XI = G::X_BYTES / 1024;           // plane copies per chunk (the plane wave)
  static constexpr int LDS = WS * G::W_BYTES + XS * G::X_BYTES;
  static_assert(LDS <= 160 * 1024, "LDS");
  static_assert(WS >= 2 && XS >= 2 && (WS - 2) * WI < 64 && (XS - 2) * XI < 64, "vmcnt range");
};

// s_waitcnt vmcnt(a * STEP) + barrier for a runtime a in 0..MAXA.
template <int STEP, int MAXA> __device__ __forceinline__ void wait_ahead_barrier(int a) {
  if constexpr (MAXA <= 0) {
    wait_vm_barrier<0>();
  } else {
    if (a >= MAXA) wait_vm_barrier<MAXA * STEP>();
    else wait_ahead_barrier<STEP, MAXA - 1>(a);
  }
}

template <int NR, int WAVES, int T, int WS, int XS>
__global__ void __launch_bounds__(64 * (WAVES + 1)) mfma_skw_kernel(GemvParams p) {
  using G = Gm<NR, WAVES, T>;
  using K = Skw<NR, WAVES, T, WS, XS>;
  __shared__ __attribute__((aligned(1024))) char lds[K::LDS];
  char* const wst = lds;                        // weight stage i at wst + i * W_BYTES
  char* const xsl = lds + WS * G::W_BYTES;      // plane slot i at xsl + i * X_BYTES
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = blockIdx.x, q = p.sk_q, rr = p.sk_r, nch = p.sk_nch;
  const int u0 = g * q + min(g, rr);
  const int nf = q + (g < rr ? 1 : 0);
  if (nf == 0) return;
  const int Z = (p.B + 31) / 32;

  if (wave == WAVES) {
    // ---- the plane wave: chunk f's planes to slot f % XS ----
    const uint16_t* xs = (const uint16_t*)p.xn;
    const size_t plane = (size_t)p.B * p.K;
    const char* src[K::XI];
    int xt = u0 / nch, xc = u0 % nch;
    auto sources = [&]() {
      const int b0 = (xt % Z) * 32;
#pragma unroll
      for (int j = 0; j < K::XI; ++j) {
        const int qq = j >> 2, r8 = 8 * (j & 3) + (lane >> 3);
        const int piece = (lane & 7) ^ ((r8 >> 1) & 7);
        const int b = b0 + r8 < p.B ? b0 + r8 : 0;   // padding columns: never stored
        src[j] = (const char*)(xs + qq * plane + (size_t)b * p.K + piece * 8);
      }
    };
    auto issue = [&](int f) {
      char* dst = xsl + (f % XS) * G::X_BYTES;
#pragma unroll
      for (int j = 0; j < K::XI; ++j) dma16(src[j] + (size_t)xc * GM_KC * 2, dst + j * 1024);
      if (++xc == nch) {
        xc = 0;
        ++xt;
        sources();
      }
    };
    sources();
    for (int f = 0; f < XS - 1 && f < nf; ++f) issue(f);
    for (int f = 0; f < nf; ++f) {
      wait_ahead_barrier<K::XI, XS - 2>(min(nf - 1 - f, XS - 2));
      if (f + XS - 1 < nf) issue(f + XS - 1);
    }
    return;
  }

  // ---- compute waves: weight chunk f to stage f % WS, multiply ----
  const RowSpace rs(p);
  const char* src[K::WI];
  int it = u0 / nch, ic = u0 % nch;
  auto sources = [&]() {
    const int n0 = (it / Z) * G::ROWS;
#pragma unroll
    for (int j = 0; j < K::WI; ++j) {
      const int i = wave * K::WI + j;
      const int r = 8 * i + (lane >> 3);
      const int piece = (lane & 7) ^ ((r >> 1) & 7);
      const int n = min(n0 + r % G::ROWS, p.n_out - 1);
      src[j] = rs.row(n, r / G::ROWS) + (size_t)piece * 16;
    }
  };
  auto issue = [&](int f) {
    char* dst = wst + (f % WS) * G::W_BYTES;
#pragma unroll
    for (int j = 0; j < K::WI; ++j) dma16(src[j] + (size_t)ic * GM_KC * 2, dst + (wave * K::WI + j) * 1024);
    if (++ic == nch) {
      ic = 0;
      ++it;
      sources();
    }
  };
  f32x16 acc[T][NR][3];
#pragma unroll
  for (int tt = 0; tt < T; ++tt)
#pragma unroll
    for (int s = 0; s < NR; ++s)
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[tt][s][j][r] = 0.f;

  sources();
  for (int f = 0; f < WS - 1 && f < nf; ++f) issue(f);
  int ct = u0 / nch, cc = u0 % nch;   // compute side: tile / chunk of the next chunk to multiply
  bool drain = false;   // partial-sum stores are in flight: wait for everything
  for (int f = 0; f < nf; ++f) {
    if (drain) wait_vm_barrier<0>();
    else wait_ahead_barrier<K::WI, WS - 2>(min(nf - 1 - f, WS - 2));
    drain = false;
    if (f + WS - 1 < nf) issue(f + WS - 1);
    gm_compute_wx<NR, T, G>(wst + (f % WS) * G::W_BYTES, xsl + (f % XS) * G::X_BYTES, wave, lane, acc);
    if (++cc == nch || f == nf - 1) {
      const int slot = g - sk_owner(ct * nch, q, rr);
      float* dst = p.part + ((size_t)ct * p.sk_smax + checked_index(slot, p.sk_smax, p.status)) * Sk<NR, WAVES, T>::TE;
#pragma unroll
      for (int tt = 0; tt < T; ++tt)
#pragma unroll
        for (int sN = 0; sN < NR; ++sN) {
          float* d = dst + (size_t)(sN * 32 + (lane & 31)) * G::ROWS + 32 * (wave * T + tt) + 4 * (lane >> 5);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float4 v;
            v.x = acc[tt][sN][0][4 * j + 0] + (acc[tt][sN][1][4 * j + 0] + acc[tt][sN][2][4 * j + 0]);
            v.y = acc[tt][sN][0][4 * j + 1] + (acc[tt][sN][1][4 * j + 1] + acc[tt][sN][2][4 * j + 1]);
            v.z = acc[tt][sN][0][4 * j + 2] + (acc[tt][sN][1][4 * j + 2] + acc[tt][sN][2][4 * j + 2]);
            v.w = acc[tt][sN][0][4 * j + 3] + (acc[tt][sN][1][4 * j + 3] + acc[tt][sN][2][4 * j + 3]);
            *(float4*)(d + 8 * j) = v;
          }
#pragma unroll
          for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[tt][sN][j][r] = 0.f;
        }
      drain = true;
      cc = 0;
      ++ct;
    }
  }
}

#define SK_KB 8   // partial slots loaded together

// Sum each tile's slots (slot order) and apply the epilogue.  Thread th of
// tile t takes four consecutive tile rows (th % (ROWS/4)) of activation row
// th / (ROWS/4), for each of the NR segments.
template <int NR, int WAVES, int T>
__global__ void __launch_bounds__(DUALAR_WG) sk_finish_kernel(GemvParams p) {
  using S = Sk<NR, WAVES, T>;
  constexpr int ROWS = S::ROWS, PER_TILE = 32 * ROWS / 4;
  const int Z = (p.B + 31) / 32;
  const int tiles = ((p.n_out + ROWS - 1) / ROWS) * Z;
  const size_t gid = (size_t)blockIdx.x * DUALAR_WG + threadIdx.x;
  const int t = (int)(gid / PER_TILE), th = (int)(gid % PER_TILE);
  if (t >= tiles) return;
  const int bl = th / (ROWS / 4), r4 = th % (ROWS / 4);
  const int b = (t % Z) * 32 + bl;
  const int n0 = (t / Z) * ROWS + 4 * r4;
  if (b >= p.B || n0 >= p.n_out) return;
  const int nch = p.sk_nch;
  const int nsl = sk_owner(t * nch + nch - 1, p.sk_q, p.sk_r) - sk_owner(t * nch, p.sk_q, p.sk_r) + 1;
  const float* base = p.part + (size_t)t * p.sk_smax * S::TE + (size_t)bl * ROWS + 4 * r4;
  // The attention preparation's position and QK-norm gain go out with the
  // slots, so only the RoPE table (indexed by the position) waits for them.
  // Both loads are unconditional (a load under a branch would be waited for
  // where the branch ends, before the slots are issued): where they do not
  // apply they read the thread's first slot instead, and the value is unused.
  const bool prep = NR == 1 && p.prep.q_planes;
  const int hh_p = t / Z;
  const uint16_t* qk_gain = (const uint16_t*)(hh_p < p.prep.H ? p.prep.q_norm : p.prep.k_norm);
  const bool has_gain = prep && hh_p < p.prep.H + p.prep.KV && qk_gain;
  const uint16_t* gsrc = has_gain ? qk_gain + 4 * r4 : (const uint16_t*)base;
  const int* psrc = prep && p.prep.pos ? p.prep.pos + b : (const int*)base;
  uint16_t graw[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) graw[e] = gsrc[e];
  const int praw = *psrc;
  float4 v[NR];
#pragma unroll
  for (int s = 0; s < NR; ++s) v[s] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k0 = 0; k0 < nsl; k0 += SK_KB) {
    float4 a[SK_KB][NR];
#pragma unroll
    for (int u = 0; u < SK_KB; ++u)
#pragma unroll
      for (int s = 0; s < NR; ++s)
        if (k0 + u < nsl) a[u][s] = *(const float4*)(base + (size_t)(k0 + u) * S::TE + (size_t)s * 32 * ROWS);
#pragma unroll
    for (int u = 0; u < SK_KB; ++u)
#pragma unroll
      for (int s = 0; s < NR; ++s)
        if (k0 + u < nsl) {
          v[s].x += a[u][s].x; v[s].y += a[u][s].y; v[s].z += a[u][s].z; v[s].w += a[u][s].w;
        }
  }
  const float g4[4] = {v[0].x, v[0].y, v[0].z, v[0].w};
  const float u4[4] = {v[NR - 1].x, v[NR - 1].y, v[NR - 1].z, v[NR - 1].w};
  if (NR == 1 && p.prep.q_planes) {
    // QKV output feeding the attention: tile t / Z is head hh, and the 32
    // threads of this activation row (one half-wave) hold its 128 dims, four
    // each: RMS over the half-wave, RoPE on the two local pairs.
    const QkPrep& q = p.prep;
    const int hh = t / Z, d0 = 4 * r4, hd = q.hd;
    const int pv = q.pos ? praw : q.pos_const;
    const int pos = pv < 0 ? pv : checked_index(pv, q.max_pos, q.status);
    float a[4] = {g4[0], g4[1], g4[2], g4[3]};
    *(float4*)(p.y + (size_t)b * p.ldy + n0) = make_float4(a[0], a[1], a[2], a[3]);
    const bool isq = hh < q.H, isk = !isq && hh < q.H + q.KV;
    if (isq || isk) {
      const void* gain = isq ? q.q_norm : q.k_norm;
      if (gain) {
        const float ss = group_sum((a[0] * a[0] + a[1] * a[1]) + (a[2] * a[2] + a[3] * a[3]), 32);
        const float inv = 1.0f / sqrtf(ss / (float)hd + p.eps);
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = a[e] * inv * bf16_bits_to_f32(graw[e]);
      }
      if (pos < 0) return;
      const float2* rp = q.rope + (size_t)pos * (hd / 2) + d0 / 2;
      float r[4];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float2 cs = rp[k];
        r[2 * k] = a[2 * k] * cs.x - a[2 * k + 1] * cs.y;
        r[2 * k + 1] = a[2 * k] * cs.y + a[2 * k + 1] * cs.x;
      }
      if (isq) {
        const float qscale = 1.0f / sqrtf((float)hd);
        const size_t plane = (size_t)p.B * q.H * hd, at = ((size_t)b * q.H + hh) * hd + d0;
#pragma unroll
        for (int e = 0; e < 4; ++e) store_planes(q.q_planes, plane, at + e, r[e] * qscale);
      } else {
        uint16_t* kc = (uint16_t*)q.kcache + (((size_t)b * q.KV + (hh - q.H)) * q.max_pos + pos) * hd + d0;
#pragma unroll
        for (int e = 0; e < 4; ++e) kc[e] = f32_to_bf16_rne(r[e]);
      }
    } else if (pos >= 0) {
      uint16_t* vc = (uint16_t*)q.vcache + (((size_t)b * q.KV + (hh - q.H - q.KV)) * q.max_pos + pos) * hd + d0;
#pragma unroll
      for (int e = 0; e < 4; ++e) vc[e] = f32_to_bf16_rne(a[e]);
    }
    return;
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int n = n0 + e;
    if (n >= p.n_out) break;
    float out;
    if (p.mode == GEMV_SWIGLU) out = silu_f(g4[e]) * u4[e];
    else if (p.mode == GEMV_ADD) out = p.res[(size_t)b * p.ldres + n] + g4[e];
    else out = g4[e];
    if (p.yplanes) store_planes((uint16_t*)p.yplanes, (size_t)p.B * p.n_out, (size_t)b * p.n_out + n, out);
    else p.y[(size_t)b * p.ldy + n] = out;
  }
}

// The stream-K finish of a residual product whose output feeds the next
// product, one 1,024-thread workgroup per activation row b (n_out <= 4,096,
// a multiple of 4): thread k sums the slots of output float4 k (contiguous
// runs of a tile's row-major partial area, all loads issued together), adds
// the residual, writes y, and the workgroup then RMS-normalises the row with
// next_gain and writes it as three bf16 planes for the next product.
#define SKR_T 1024
template <int WAVES, int T>
__global__ void __launch_bounds__(SKR_T) sk_finish_rows_kernel(GemvParams p) {
  using S = Sk<1, WAVES, T>;
  constexpr int ROWS = S::ROWS;
  constexpr int KB = 16;                      // slots loaded together
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float red[SKR_T / 64];
  const int nv = p.n_out / 4, Z = (p.B + 31) / 32, nch = p.sk_nch;
  const bool live = tid < nv;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  uint2 gg = make_uint2(0u, 0u);
  if (live) {
    const int n = 4 * tid, t = (n / ROWS) * Z + b / 32;
    // the residual and the next gain go out with the slots: one memory round trip
    const float4 r = *(const float4*)(p.res + (size_t)b * p.ldres + n);
    gg = ((const uint2*)p.next_gain)[tid];
    const float* src = p.part + (size_t)t * p.sk_smax * S::TE + (size_t)(b & 31) * ROWS + n % ROWS;
    const int nsl = sk_owner(t * nch + nch - 1, p.sk_q, p.sk_r) - sk_owner(t * nch, p.sk_q, p.sk_r) + 1;
    for (int k0 = 0; k0 < nsl; k0 += KB) {
      float4 a[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u)
        if (k0 + u < nsl) a[u] = *(const float4*)(src + (size_t)(k0 + u) * S::TE);
#pragma unroll
      for (int u = 0; u < KB; ++u)
        if (k0 + u < nsl) { v.x += a[u].x; v.y += a[u].y; v.z += a[u].z; v.w += a[u].w; }
    }
    v.x = r.x + v.x; v.y = r.y + v.y; v.z = r.z + v.z; v.w = r.w + v.w;
    *(float4*)(p.y + (size_t)b * p.ldy + n) = v;
  }
  float ss = (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < SKR_T / 64; ++w) tot += red[w];
  if (!live) return;
  const float inv = 1.0f / sqrtf(tot / (float)p.n_out + p.eps);
  const float o[4] = {v.x * inv * bf16_bits_to_f32(gg.x & 0xffffu), v.y * inv * bf16_bits_to_f32(gg.x >> 16),
                      v.z * inv * bf16_bits_to_f32(gg.y & 0xffffu), v.w * inv * bf16_bits_to_f32(gg.y >> 16)};
  uint32_t tt[3][4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint16_t a0 = f32_to_bf16_rne(o[e]);
    const float r1 = o[e] - bf16_bits_to_f32(a0);
    const uint16_t a1 = f32_to_bf16_rne(r1);
    tt[0][e] = a0;
    tt[1][e] = a1;
    tt[2][e] = f32_to_bf16_rne(r1 - bf16_bits_to_f32(a1));
  }
  uint2* xs = (uint2*)p.next_planes;
  const size_t plane = (size_t)p.B * nv, at = (size_t)b * nv + tid;
#pragma unroll
  for (int q = 0; q < 3; ++q) xs[q * plane + at] = make_uint2(tt[q][0] | (tt[q][1] << 16), tt[q][2] | (tt[q][3] << 16));
}

// Stream-K plan: U = tiles x chunks work units dealt to the grid (false
// when there is no partial buffer or the partial tiles do not fit it).
template <int NR, int WAVES, int T>
static bool sk_plan(GemvParams& p, int slots, int* ng_out) {
  using S = Sk<NR, WAVES, T>;
  constexpr int ROWS = 32 * WAVES * T;
  const int Z = (p.B + 31) / 32;
  const int tiles = ((p.n_out + ROWS - 1) / ROWS) * Z;
  const int nch = p.K / GM_KC;
  const long long U = (long long)tiles * nch;
  if (!p.part || U >= (1LL << 30)) return false;
  int ng = slots;
  if (U < 4LL * ng) ng = (int)std::max(1LL, U / 4);      // at least four chunks per workgroup
  const int q = (int)(U / ng), r = (int)(U % ng);
  int smax = 1;
  for (int t = 0; t < tiles; ++t) smax = std::max(smax, sk_owner(t * nch + nch - 1, q, r) - sk_owner(t * nch, q, r) + 1);
  if ((size_t)tiles * smax * S::TE > p.part_elems) return false;
  p.sk_q = q;
  p.sk_r = r;
  p.sk_smax = smax;
  p.sk_nch = nch;
  *ng_out = ng;
  return true;
}

template <int NR, int WAVES, int T>
static void sk_finish(GemvParams& p, hipStream_t s) {
  using S = Sk<NR, WAVES, T>;
  constexpr int ROWS = 32 * WAVES * T;
  const int tiles = ((p.n_out + ROWS - 1) / ROWS) * ((p.B + 31) / 32);
  // a residual product feeding the next one: finish and normalise per row
  const bool rows = NR == 1 && p.next_planes && p.mode == GEMV_ADD && !p.yplanes && p.n_out % 4 == 0 &&
                    p.n_out <= 4 * SKR_T;
  if (rows) {
    if (p.next_done) *p.next_done = 1;
    if (p.prep_done) *p.prep_done = 0;
    hipLaunchKernelGGL((sk_finish_rows_kernel<WAVES, T>), dim3(p.B), dim3(SKR_T), 0, s, p);
    return;
  }
  const size_t n = (size_t)tiles * 32 * S::ROWS / 4;
  // the attention preparation applies when one row tile is one head
  const bool prep = NR == 1 && p.prep.q_planes && p.mode == GEMV_STORE && !p.yplanes && S::ROWS == p.prep.hd &&
                    p.n_out == (p.prep.H + 2 * p.prep.KV) * p.prep.hd;
  if (!prep) p.prep.q_planes = nullptr;
  if (p.prep_done) *p.prep_done = prep ? 1 : 0;
  hipLaunchKernelGGL((sk_finish_kernel<NR, WAVES, T>), dim3((unsigned)((n + DUALAR_WG - 1) / DUALAR_WG)),
                     dim3(DUALAR_WG), 0, s, p);
  // A residual product whose output feeds the next product: RMS-normalise
  // each finished row with next_gain and split it into planes (the rows are
  // read once more; one workgroup per row, like the finish itself would need).
  const bool next = p.next_planes && p.mode == GEMV_ADD && p.n_out <= NORM_MAXV * 4 * DUALAR_WG &&
                    p.n_out % 4 == 0;
  if (p.next_done) *p.next_done = next ? 1 : 0;
  if (next) {
    GemvParams q = p;
    q.x = p.y;
    q.ldx = p.ldy;
    q.K = p.n_out;
    q.gain = p.next_gain;
    q.xn = p.next_planes;
    hipLaunchKernelGGL(xsplit_kernel, dim3(p.B), dim3(DUALAR_WG), 0, s, q);
  }
}

template <int NR, int WAVES, int T, int WS, int XS>
static bool launch_skw(GemvParams& p, hipStream_t s) {
  int ng = 0;
  if (!sk_plan<NR, WAVES, T>(p, 256, &ng)) return false;
  hipLaunchKernelGGL((mfma_skw_kernel<NR, WAVES, T, WS, XS>), dim3(ng), dim3(64 * (WAVES + 1)), 0, s, p);
  sk_finish<NR, WAVES, T>(p, s);
  return true;
}

template <int NR, int WAVES, int T>
static void launch_gm(GemvParams& p, int ksw_preset, int slots, hipStream_t s, bool* ok) {
  using G = Gm<NR, WAVES, T>;
  const int tiles = ((p.n_out + G::ROWS - 1) / G::ROWS) * ((p.B + 31) / 32);
  // Split K over ksw workgroups per row block (K % (ksw*64) == 0, partial
  // buffer holds ksw*B rows): the smallest split that fills the slots while
  // each workgroup keeps >= 4 chunks, else the largest that keeps 4 chunks.
  auto fits = [&](int c) {
    return p.K % (c * GM_KC) == 0 && (c == 1 || (p.part && (size_t)c * p.B * p.n_out * NR <= p.part_elems));
  };
  int ksw = ksw_preset;
  if (ksw > 0) {
    if (ksw > FIN_MAXK || !fits(ksw)) { *ok = false; return; }
  } else {
    ksw = 1;
    for (int c = 2; c <= FIN_MAXK && tiles * ksw < slots; ++c)
      if (fits(c) && p.K / (c * GM_KC) >= 4) ksw = c;
  }
  p.ksw = ksw;
  p.ldp = p.n_out * NR;
  const int n_tiles = (p.n_out + G::ROWS - 1) / G::ROWS, z_tiles = (p.B + 31) / 32;
  if (ksw == 1 && z_tiles > 1) {
    // several activation tiles: one-dimensional grid in which the z_tiles
    // workgroups of a row block are consecutive ids on one XCD (id % 8), so
    // they run together and share the block's weights through that L2
    p.zswz = z_tiles;
    hipLaunchKernelGGL((mfma_gemm_kernel<NR, WAVES, T>), dim3(8 * ((n_tiles + 7) / 8) * z_tiles), dim3(G::THREADS), 0,
                       s, p);
  } else {
    p.zswz = 0;
    hipLaunchKernelGGL((mfma_gemm_kernel<NR, WAVES, T>), dim3(n_tiles, ksw, z_tiles), dim3(G::THREADS), 0, s, p);
  }
  *ok = true;
}

// Matrix-core path for bf16 weights, B >= 2, K a multiple of 64 (returns
// false when it does not apply).  Shapes: SwiGLU 4 waves x 128 rows x (gate,
// up); tall products (>= 16384 rows, e.g. the tied head) 4 waves x 2 tiles =
// 256 rows; the rest 2 waves x 64 rows.  `slots` is how many such
// workgroups the chip holds at once (LDS bound).
bool launch_gemm_mfma(const GemvParams& p0, hipStream_t s, hipError_t* err) {
  if (p0.B < 2 || p0.K % GM_KC != 0 || !p0.xn || p0.K > NORM_MAXV * 4 * DUALAR_WG) return false;
  // 4-bit weights: 2 to GEMV_W4_MAX_ROWS rows or the 2-D tile form
  if (p0.q4[0] && p0.B > GEMV_W4_MAX_ROWS && p0.B < GM_TILE_ROWS) return false;
  GemvParams p = p0;
  if (p.q4[0] && p.B <= GEMV_W4_MAX_ROWS) {
    if (p.prep_done) *p.prep_done = 0;
    if (p.next_done) *p.next_done = 0;
    if (p.xplanes) p.xn = const_cast<void*>(p.xplanes);
    else if (!gemv_w4_rows_normalises(p)) hipLaunchKernelGGL(xsplit_kernel, dim3(p.B), dim3(DUALAR_WG), 0, s, p);
    if (!launch_gemv_w4_rows(p, s, err)) *err = hipErrorInvalidValue;
    return true;
  }
  if (p.xplanes) p.xn = const_cast<void*>(p.xplanes);   // input already split by its producer
  else hipLaunchKernelGGL(xsplit_kernel, dim3(p.B), dim3(DUALAR_WG), 0, s, p);
  bool ok = false;
  const bool glu = p.mode == GEMV_SWIGLU;
  const int z_tiles = (p.B + 31) / 32;
  if (p.B >= GM_TILE_ROWS) {   // 2-D output tiles (prefill steps)
    if (p.prep_done) *p.prep_done = 0;
    if (p.next_done) *p.next_done = 0;
    const bool ok = p.q4[0] ? launch_gemm_tile_w4(p, s) : launch_gemm_tile(p, gemm_tile_wide(p), s);
    *err = ok ? hipGetLastError() : hipErrorInvalidValue;
    return true;
  }
  // Stream-K (wave-specialised, one workgroup per compute unit) for the
  // decode shapes; the tall head (hundreds of row tiles) balances well as it
  // is and its partials would be as large as its output.
  if (z_tiles <= 2 && p.K / GM_KC >= 8 && p0.ksw == 0 && p.n_out < 16384) {
    if (glu ? launch_skw<2, 4, 1, 3, 3>(p, s) : launch_skw<1, 4, 1, 5, 5>(p, s)) {
      *err = hipGetLastError();
      return true;
    }
    // partial tiles do not fit the partial buffer: the split-K form below
  }
  // split-K form: (NR, WAVES, T), slots = workgroups the chip holds at once (LDS bound)
  const int cfg = glu ? 2 : (p.n_out >= 16384 ? 3 : 1);
  if (p.prep_done) *p.prep_done = 0;
  switch (cfg) {
    case 1: if (glu) launch_gm<2, 2, 1>(p, p0.ksw, 256, s, &ok); else launch_gm<1, 2, 1>(p, p0.ksw, 512, s, &ok); break;
    case 2: if (glu) launch_gm<2, 4, 1>(p, p0.ksw, 256, s, &ok); else launch_gm<1, 4, 1>(p, p0.ksw, 256, s, &ok); break;
    case 3: if (!glu) launch_gm<1, 4, 2>(p, p0.ksw, 256, s, &ok); break;
    default: break;
  }
  if (!ok) {
    *err = hipErrorInvalidValue;
    return true;
  }
  const bool fuse_next = p.next_planes && p.mode == GEMV_ADD && p.ksw > 1 && p.n_out % 4 == 0 &&
                        p.n_out <= 4 * 4 * DUALAR_WG;
  if (p.next_done) *p.next_done = fuse_next ? 1 : 0;
  if (fuse_next) {
    hipLaunchKernelGGL(finish_split_kernel, dim3(p.B), dim3(DUALAR_WG), 0, s, p);
  } else if (p.ksw > 1) {
    const size_t n = (size_t)p.B * p.n_out;
    hipLaunchKernelGGL(mfma_finish_kernel, dim3((unsigned)((n + DUALAR_WG - 1) / DUALAR_WG)), dim3(DUALAR_WG), 0, s, p);
  }
  *err = hipGetLastError();
  return true;
}
