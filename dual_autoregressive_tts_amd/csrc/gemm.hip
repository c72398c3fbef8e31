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
#include "common.h"
#include "internal.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define MF_U 4   // k-steps whose loads are issued together

__device__ __forceinline__ const char* mrow(const GemvParams& p, int row, int s) {
  if (p.mode == GEMV_SWIGLU) return (const char*)p.w[s] + (size_t)row * p.K * 2;
  if (row < p.rows[0]) return (const char*)p.w[0] + (size_t)row * p.K * 2;
  row -= p.rows[0];
  if (row < p.rows[1]) return (const char*)p.w[1] + (size_t)row * p.K * 2;
  row -= p.rows[1];
  return (const char*)p.w[2] + (size_t)row * p.K * 2;
}

__device__ __forceinline__ bf16x8 pack8(const uint32_t* b) {
  u32x4 h;
  h.x = b[0] | (b[1] << 16); h.y = b[2] | (b[3] << 16); h.z = b[4] | (b[5] << 16); h.w = b[6] | (b[7] << 16);
  return __builtin_bit_cast(bf16x8, h);
}

// x = t[0] + t[1] + t[2] (+ a residual below 2^-24 |x|), each term bf16.
__device__ __forceinline__ void split3(const float* v, bf16x8* t) {
  uint32_t b0[8], b1[8], b2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint16_t a = f32_to_bf16_rne(v[i]);
    const float r1 = v[i] - bf16_bits_to_f32(a);
    const uint16_t c = f32_to_bf16_rne(r1);
    b0[i] = a;
    b1[i] = c;
    b2[i] = f32_to_bf16_rne(r1 - bf16_bits_to_f32(c));
  }
  t[0] = pack8(b0);
  t[1] = pack8(b1);
  t[2] = pack8(b2);
}

// Output element of accumulator register r in lane `lane` of a 32x32 tile.
__device__ __forceinline__ int tile_row(int r, int lane) { return (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); }

template <int NR>
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
  const bool bok = brow < p.B;
  const float* xb = p.x + (size_t)(bok ? brow : 0) * p.ldx + koff;

  f32x16 acc[NR];
#pragma unroll
  for (int s = 0; s < NR; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[s][r] = 0.f;

  for (int st = 0; st < nsteps; st += MF_U) {
    u32x4 a[MF_U][NR];
    float4 xv[MF_U][2];
#pragma unroll
    for (int u = 0; u < MF_U; ++u) {
      const int ss = min(st + u, nsteps - 1);
#pragma unroll
      for (int s = 0; s < NR; ++s) a[u][s] = ld_stream(wa[s] + (size_t)ss * 32);
      xv[u][0] = *(const float4*)(xb + ss * 16);
      xv[u][1] = *(const float4*)(xb + ss * 16 + 4);
    }
#pragma unroll
    for (int u = 0; u < MF_U; ++u) {
      if (st + u >= nsteps) break;
      float v[8] = {xv[u][0].x, xv[u][0].y, xv[u][0].z, xv[u][0].w, xv[u][1].x, xv[u][1].y, xv[u][1].z, xv[u][1].w};
      if (!bok) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.f;
      }
      bf16x8 t[3];
      split3(v, t);
#pragma unroll
      for (int s = 0; s < NR; ++s) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, a[u][s]);
        acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, t[0], acc[s], 0, 0, 0);
        acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, t[1], acc[s], 0, 0, 0);
        acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, t[2], acc[s], 0, 0, 0);
      }
    }
  }

  // the 4 waves' partials, added in a fixed order
  __shared__ float red[4][NR][16][64];
#pragma unroll
  for (int s = 0; s < NR; ++s)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave][s][r][lane] = acc[s][r];
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * 64; i += DUALAR_WG) {
    const int r = i >> 6, l = i & 63;
    const int n = n0 + tile_row(r, l), b = b0 + (l & 31);
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

// Sum the ksw partials (fixed order) and apply the epilogue.
__global__ void __launch_bounds__(DUALAR_WG) mfma_finish_kernel(GemvParams p) {
  const size_t i = (size_t)blockIdx.x * DUALAR_WG + threadIdx.x;
  if (i >= (size_t)p.B * p.n_out) return;
  const int b = (int)(i / p.n_out), n = (int)(i % p.n_out);
  float v0 = 0.f, v1 = 0.f;
  for (int kw = 0; kw < p.ksw; ++kw) {
    const float* src = p.part + ((size_t)kw * p.B + b) * p.ldp;
    v0 += src[n];
    if (p.mode == GEMV_SWIGLU) v1 += src[(size_t)p.n_out + n];
  }
  float out;
  if (p.mode == GEMV_SWIGLU) out = silu_f(v0) * v1;
  else if (p.mode == GEMV_ADD) out = p.res[(size_t)b * p.ldres + n] + v0;
  else out = v0;
  p.y[(size_t)b * p.ldy + n] = out;
}

// xn[b] = x[b] / sqrt(mean(x[b]^2) + eps) * g, one workgroup per row.
__global__ void __launch_bounds__(DUALAR_WG) rownorm_kernel(GemvParams p) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float red[4];
  const float* x = p.x + (size_t)b * p.ldx;
  float ss = 0.f;
  for (int k = tid; k < p.K; k += DUALAR_WG) ss += x[k] * x[k];
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const float inv = 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)p.K + p.eps);
  float* xn = p.xn + (size_t)b * p.K;
  for (int k = tid; k < p.K; k += DUALAR_WG) xn[k] = x[k] * inv * ElemT<bf16_t>::load(p.gain, k);
}

// Matrix-core path for bf16 weights, B >= 8, K a multiple of 64 (returns
// false when it does not apply).
bool launch_gemm_mfma(const GemvParams& p0, hipStream_t s, hipError_t* err) {
  if (p0.B < 8 || p0.K % 64 != 0 || !p0.part || !p0.xn) return false;
  GemvParams p = p0;
  if (p.gain) {
    hipLaunchKernelGGL(rownorm_kernel, dim3(p.B), dim3(DUALAR_WG), 0, s, p);
    p.x = p.xn;
    p.ldx = p.K;
  }
  const int NR = p.mode == GEMV_SWIGLU ? 2 : 1;
  const int tiles = ((p.n_out + 31) / 32) * ((p.B + 31) / 32);
  // split K over workgroups until there are >= 512 of them (K/(ksw*4) a
  // multiple of 16, and the partial buffer must hold ksw * B rows)
  int ksw = 1;
  while (tiles * ksw < 512 && p.K % (ksw * 2 * 64) == 0 && (size_t)ksw * 2 * p.B * p.n_out * NR <= p.part_elems)
    ksw *= 2;
  p.ksw = ksw;
  p.ldp = p.n_out * NR;
  dim3 grid((p.n_out + 31) / 32, ksw, (p.B + 31) / 32);
  if (NR == 2) hipLaunchKernelGGL(mfma_gemm_kernel<2>, grid, dim3(DUALAR_WG), 0, s, p);
  else hipLaunchKernelGGL(mfma_gemm_kernel<1>, grid, dim3(DUALAR_WG), 0, s, p);
  if (ksw > 1) {
    const size_t n = (size_t)p.B * p.n_out;
    hipLaunchKernelGGL(mfma_finish_kernel, dim3((unsigned)((n + DUALAR_WG - 1) / DUALAR_WG)), dim3(DUALAR_WG), 0, s, p);
  }
  *err = hipGetLastError();
  return true;
}
