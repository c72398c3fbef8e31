// Matrix products for 8..32+ activation rows (batched decode, batched
// prefill steps) on the gfx950 matrix cores: Y[b][n] = sum_k W[n][k] X[b][k].
//
// v_mfma_f32_32x32x16_bf16 with W as the A operand (32 output rows, lane l
// holds W[n0 + l%32][k + 8*(l/32) .. +8], 16 contiguous bytes) and the
// activations as the B operand (32 activation rows, lane l holds
// X[b0 + l%32][k + 8*(l/32) .. +8]).  Activations are fp32: each is split
// into three bf16 terms, x = t0 + t1 + t2 + r with t0 = bf16(x),
// t1 = bf16(x - t0), t2 = bf16(x - t0 - t1) (every subtraction exact in
// fp32, |r| <= 2^-24 |x|), and the three products are accumulated in fp32.
// The weights are bf16 already, so the product is the fp32 product of the
// stored weights and the fp32 activations up to accumulation order.  A
// two-term split would leave ~2^-17 relative error per activation, which is
// enough to move bf16-rounded K/V entries one ulp far more often than fp32
// rounding order does.  The third product is cheap: at B <= 32 one 1 KB
// weight tile feeds 3 x 32 MFMA cycles per SIMD, about 3x the HBM rate.
//
// A workgroup owns one 32-row tile (gate and up tiles for SwiGLU) and a
// 1/ksw slice of K, split again over its 4 waves; the 4 wave partials meet in
// LDS in a fixed order.  With ksw > 1 the workgroups write partial sums and
// mfma_finish_kernel adds them (fixed order) and applies the epilogue.
// RMSNorm, when the product has a gain, runs first in rownorm_kernel.
//
// Each wave streams its K range in batches of U k-steps; the next batch's
// loads are issued before the current batch's MFMAs so that a wave always
// has a batch in flight.  Weight rows are read 32 B per lane-pair per step
// (the operand layout), so the loads go through the cache: the four reads
// that make up one 128-byte line then cost one HBM fetch.  Activation
// columns past B are loaded from row 0 and never stored (MFMA output column
// b depends only on operand column b).
#include "common.h"
#include "internal.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ const char* mrow(const GemvParams& p, int row, int s) {
  if (p.mode == GEMV_SWIGLU) return (const char*)p.w[s] + (size_t)row * p.K * 2;
  if (row < p.rows[0]) return (const char*)p.w[0] + (size_t)row * p.K * 2;
  row -= p.rows[0];
  if (row < p.rows[1]) return (const char*)p.w[1] + (size_t)row * p.K * 2;
  row -= p.rows[1];
  return (const char*)p.w[2] + (size_t)row * p.K * 2;
}

// Output element of accumulator register r in lane `lane` of a 32x32 tile.
__device__ __forceinline__ int tile_row(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

template <int NR, int U>
struct Batch {
  u32x4 a[U][NR];
  float4 x[U][2];
};

template <int NR, int U>
__device__ __forceinline__ void load_batch(Batch<NR, U>& bt, const char* const* wa, const float* xb, int st) {
#pragma unroll
  for (int u = 0; u < U; ++u) {   // activations first (cache-resident), then weights
    bt.x[u][0] = *(const float4*)(xb + (st + u) * 16);
    bt.x[u][1] = *(const float4*)(xb + (st + u) * 16 + 4);
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int s = 0; s < NR; ++s) bt.a[u][s] = ld_vec(wa[s] + (size_t)(st + u) * 32);
}

// x = t0 + t1 + t2 (+ a residual below 2^-24 |x|), each term bf16.
template <int NR, int U>
__device__ __forceinline__ void mma_batch(const Batch<NR, U>& bt, f32x16* acc) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const f32x8 v = {bt.x[u][0].x, bt.x[u][0].y, bt.x[u][0].z, bt.x[u][0].w,
                     bt.x[u][1].x, bt.x[u][1].y, bt.x[u][1].z, bt.x[u][1].w};
    const bf16x8 t0 = __builtin_convertvector(v, bf16x8);
    const f32x8 r1 = v - __builtin_convertvector(t0, f32x8);
    const bf16x8 t1 = __builtin_convertvector(r1, bf16x8);
    const bf16x8 t2 = __builtin_convertvector(r1 - __builtin_convertvector(t1, f32x8), bf16x8);
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, bt.a[u][s]);
      acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, t0, acc[s], 0, 0, 0);
      acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, t1, acc[s], 0, 0, 0);
      acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, t2, acc[s], 0, 0, 0);
    }
  }
}

// Grid (ceil(n_out/32), ksw, ceil(B/32)).  The host guarantees K % (ksw*64) == 0
// and that each wave's step count (K/(ksw*64)) is a multiple of 2U.
template <int NR, int U>
__global__ void __launch_bounds__(DUALAR_WG) mfma_gemm_kernel(GemvParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 32, kw = blockIdx.y, b0 = blockIdx.z * 32;
  const int Kw = p.K / p.ksw, Kq = Kw / 4;
  const int kbeg = kw * Kw + wave * Kq;
  const int nsteps = Kq / 16;
  const int koff = kbeg + 8 * (lane >> 5);

  const char* wa[NR];
  const int arow = min(n0 + (lane & 31), p.n_out - 1);
#pragma unroll
  for (int s = 0; s < NR; ++s) wa[s] = mrow(p, arow, s) + (size_t)koff * 2;
  const int brow = b0 + (lane & 31);
  const float* xb = p.x + (size_t)(brow < p.B ? brow : 0) * p.ldx + koff;

  f32x16 acc[NR];
#pragma unroll
  for (int s = 0; s < NR; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[s][r] = 0.f;

  // Double-buffered, two batches per trip: the next batch's loads are
  // always issued (past the end they re-read the last batch, a cache hit),
  // and scheduling barriers keep each batch's loads together ahead of the
  // other batch's MFMAs, so every wait leaves one whole batch in flight.  (A
  // conditional prefetch, a loop with two exits, or letting the scheduler
  // sink each load next to its use all make the compiler wait for
  // everything.)
  Batch<NR, U> b0b, b1b;
  const int last = nsteps - U;
  load_batch<NR, U>(b0b, wa, xb, 0);
  int st = 0;
  do {
    load_batch<NR, U>(b1b, wa, xb, min(st + U, last));
    __builtin_amdgcn_sched_barrier(0);
    mma_batch<NR, U>(b0b, acc);
    __builtin_amdgcn_sched_barrier(0);
    load_batch<NR, U>(b0b, wa, xb, min(st + 2 * U, last));
    __builtin_amdgcn_sched_barrier(0);
    mma_batch<NR, U>(b1b, acc);
    __builtin_amdgcn_sched_barrier(0);
    st += 2 * U;
  } while (st < nsteps);

  // The 4 waves' partials, added in a fixed order.  The rows are padded to
  // 65 floats so that reading them in output order is conflict-free; thread
  // i then owns output row n0 + i%32 of activation row b0 + i/32 (+8j), so
  // each store instruction writes whole 128-byte runs of y or part.
  __shared__ float red[4][NR][16][65];
#pragma unroll
  for (int s = 0; s < NR; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][s][r][lane] = acc[s][r];
  __syncthreads();
  const int nl = threadIdx.x & 31;
  const int n = n0 + nl;
  const int r = ((nl >> 3) << 2) | (nl & 3);        // inverse of tile_row
  const int lhi = ((nl >> 2) & 1) << 5;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int bl = (threadIdx.x >> 5) + 8 * j;
    const int b = b0 + bl, l = lhi | bl;
    if (n >= p.n_out || b >= p.B) continue;
    float v[NR];
#pragma unroll
    for (int s = 0; s < NR; ++s) v[s] = (red[0][s][r][l] + red[1][s][r][l]) + (red[2][s][r][l] + red[3][s][r][l]);
    if (p.ksw > 1) {
      float* dst = p.part + ((size_t)kw * p.B + b) * p.ldp;
#pragma unroll
      for (int s = 0; s < NR; ++s) dst[(size_t)s * p.n_out + n] = v[s];
    } else {
      float out;
      if (p.mode == GEMV_SWIGLU) out = silu_f(v[0]) * v[NR - 1];
      else if (p.mode == GEMV_ADD) out = p.res[(size_t)b * p.ldres + n] + v[0];
      else out = v[0];
      p.y[(size_t)b * p.ldy + n] = out;
    }
  }
}

#define FIN_MAXK 8   // largest ksw the finish kernel reads with all loads issued up front

// Sum the ksw partials (fixed order) and apply the epilogue.
__global__ void __launch_bounds__(DUALAR_WG) mfma_finish_kernel(GemvParams p) {
  const size_t i = (size_t)blockIdx.x * DUALAR_WG + threadIdx.x;
  if (i >= (size_t)p.B * p.n_out) return;
  const int b = (int)(i / p.n_out), n = (int)(i % p.n_out);
  const bool glu = p.mode == GEMV_SWIGLU;
  float g[FIN_MAXK], u[FIN_MAXK];
#pragma unroll
  for (int kw = 0; kw < FIN_MAXK; ++kw) {
    if (kw < p.ksw) {
      const float* src = p.part + ((size_t)kw * p.B + b) * p.ldp;
      g[kw] = src[n];
      u[kw] = glu ? src[(size_t)p.n_out + n] : 0.f;
    }
  }
  const float r = p.mode == GEMV_ADD ? p.res[(size_t)b * p.ldres + n] : 0.f;
  float v0 = 0.f, v1 = 0.f;
#pragma unroll
  for (int kw = 0; kw < FIN_MAXK; ++kw) {
    if (kw < p.ksw) {
      v0 += g[kw];
      v1 += u[kw];
    }
  }
  float out;
  if (glu) out = silu_f(v0) * v1;
  else if (p.mode == GEMV_ADD) out = r + v0;
  else out = v0;
  p.y[(size_t)b * p.ldy + n] = out;
}

#define NORM_MAXV 12   // float4s per thread: K <= 12288

// xn[b] = x[b] / sqrt(mean(x[b]^2) + eps) * g, one workgroup per row; the
// row is read once, with every load issued before the first use.
__global__ void __launch_bounds__(DUALAR_WG) rownorm_kernel(GemvParams p) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float red[4];
  const float4* x = (const float4*)(p.x + (size_t)b * p.ldx);
  const int nv = p.K / 4;
  float4 v[NORM_MAXV];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NORM_MAXV; ++j)
    if (tid + j * DUALAR_WG < nv) v[j] = x[tid + j * DUALAR_WG];
#pragma unroll
  for (int j = 0; j < NORM_MAXV; ++j)
    if (tid + j * DUALAR_WG < nv) ss += (v[j].x * v[j].x + v[j].y * v[j].y) + (v[j].z * v[j].z + v[j].w * v[j].w);
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)p.K + p.eps);
  float4* xn = (float4*)(p.xn + (size_t)b * p.K);
  const uint2* g = (const uint2*)p.gain;
#pragma unroll
  for (int j = 0; j < NORM_MAXV; ++j) {
    const int k = tid + j * DUALAR_WG;
    if (k < nv) {
      const uint2 gg = g[k];
      float4 o;
      o.x = v[j].x * inv * bf16_bits_to_f32(gg.x & 0xffffu);
      o.y = v[j].y * inv * bf16_bits_to_f32(gg.x >> 16);
      o.z = v[j].z * inv * bf16_bits_to_f32(gg.y & 0xffffu);
      o.w = v[j].w * inv * bf16_bits_to_f32(gg.y >> 16);
      xn[k] = o;
    }
  }
}

template <int NR, int U>
static void launch_main(const GemvParams& p, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((mfma_gemm_kernel<NR, U>), grid, dim3(DUALAR_WG), 0, s, p);
}

// Matrix-core path for bf16 weights, B >= 8, K a multiple of 64 (returns
// false when it does not apply).
bool launch_gemm_mfma(const GemvParams& p0, hipStream_t s, hipError_t* err) {
  if (p0.B < 8 || p0.K % 64 != 0 || !p0.part || !p0.xn || p0.K > NORM_MAXV * 4 * DUALAR_WG) return false;
  GemvParams p = p0;
  const int NR = p.mode == GEMV_SWIGLU ? 2 : 1;
  const int tiles = ((p.n_out + 31) / 32) * ((p.B + 31) / 32);
  // Split K over ksw workgroups.  Each wave must get a whole number of
  // 16-wide k-steps (K % (ksw*64) == 0) and the partial buffer must hold
  // ksw * B rows.  Take the smallest split that gives >= 512 workgroups with
  // batches of >= 2 steps, else the one with the most workgroups among those
  // with batches of >= 2 steps.  A caller may preset p.ksw.
  // U = the largest of 4, 2, 1 with nsteps % (2U) == 0 (the main loop
  // consumes two batches per trip); odd step counts are not launched.
  auto u_of = [&](int c) { const int n = p.K / (c * 64); return n % 8 == 0 ? 4 : (n % 4 == 0 ? 2 : 1); };
  auto ok = [&](int c) {
    return p.K % (c * 64) == 0 && (p.K / (c * 64)) % 2 == 0 &&
           (c == 1 || (size_t)c * p.B * p.n_out * NR <= p.part_elems);
  };
  int ksw = 0;
  if (p0.ksw > 0) {
    if (p0.ksw > FIN_MAXK || !ok(p0.ksw)) return false;
    ksw = p0.ksw;
  } else {
    int best = 0;
    for (int c = 1; c <= FIN_MAXK; ++c) {
      if (!ok(c) || (c > 1 && u_of(c) < 2)) continue;
      if (tiles * c >= 512) { ksw = c; break; }
      best = c;
    }
    if (!ksw) ksw = best;
    if (!ksw) return false;
  }
  if (p.gain) {
    hipLaunchKernelGGL(rownorm_kernel, dim3(p.B), dim3(DUALAR_WG), 0, s, p);
    p.x = p.xn;
    p.ldx = p.K;
  }
  p.ksw = ksw;
  p.ldp = p.n_out * NR;
  const int U = u_of(ksw);
  dim3 grid((p.n_out + 31) / 32, ksw, (p.B + 31) / 32);
  if (NR == 2) {
    if (U == 4) launch_main<2, 4>(p, grid, s);
    else if (U == 2) launch_main<2, 2>(p, grid, s);
    else launch_main<2, 1>(p, grid, s);
  } else {
    if (U == 4) launch_main<1, 4>(p, grid, s);
    else if (U == 2) launch_main<1, 2>(p, grid, s);
    else launch_main<1, 1>(p, grid, s);
  }
  if (ksw > 1) {
    const size_t n = (size_t)p.B * p.n_out;
    hipLaunchKernelGGL(mfma_finish_kernel, dim3((unsigned)((n + DUALAR_WG - 1) / DUALAR_WG)), dim3(DUALAR_WG), 0, s, p);
  }
  *err = hipGetLastError();
  return true;
}
