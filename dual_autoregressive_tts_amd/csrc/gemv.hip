// Bandwidth-bound matrix-vector products of the decode step (batch <= 4 per
// pass): y = W . f(x) with W streamed once from HBM in 16-byte lane loads.
//
// Layout: a workgroup is 4 waves; each wave owns RPW output rows (RPW pairs
// for the SwiGLU gate/up product).  Lane l reads elements
// [u*64*EPV + l*EPV, +EPV) of a row for unit u, so one wave load covers 1 KB
// of one row, contiguous.  The activation rows (BT of them, fp32) are staged
// in LDS once per workgroup; when a norm gain is given the RMSNorm of the
// activations is applied while staging (fused prologue).  Partial dot
// products are reduced across the wave with a fixed butterfly, so results
// are deterministic.
#include "common.h"
#include "internal.h"

template <typename T> __device__ __forceinline__ const char* seg_row(const GemvParams& p, int row, int s) {
  // SwiGLU: s selects gate (w[0]) or up (w[1]) at the same row.
  if (p.mode == GEMV_SWIGLU) return (const char*)p.w[s] + (size_t)row * p.K * sizeof(T);
  if (row < p.rows[0]) return (const char*)p.w[0] + (size_t)row * p.K * sizeof(T);
  row -= p.rows[0];
  if (row < p.rows[1]) return (const char*)p.w[1] + (size_t)row * p.K * sizeof(T);
  row -= p.rows[1];
  return (const char*)p.w[2] + (size_t)row * p.K * sizeof(T);
}

template <typename T, int BT, int RPW, int NR>
__global__ void __launch_bounds__(DUALAR_WG) gemv_kernel(GemvParams p) {
  extern __shared__ float xs[];  // [BT][K]
  __shared__ float red[BT][4];
  constexpr int EPV = ElemT<T>::EPV;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.K;
  const int b0 = blockIdx.y * BT;

  // ---- stage activations (+ fused RMSNorm) ----
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) {
    const int b = b0 + bb;
    float ss = 0.f;
    for (int k = tid; k < K; k += DUALAR_WG) {
      float v = (b < p.B) ? p.x[(size_t)b * p.ldx + k] : 0.f;
      xs[bb * K + k] = v;
      ss += v * v;
    }
    if (p.gain) {
      ss = wave_sum(ss);
      if (lane == 0) red[bb][wave] = ss;
    }
  }
  __syncthreads();
  if (p.gain) {
#pragma unroll
    for (int bb = 0; bb < BT; ++bb) {
      const float tot = (red[bb][0] + red[bb][1]) + (red[bb][2] + red[bb][3]);
      const float inv = 1.0f / sqrtf(tot / (float)K + p.eps);
      for (int k = tid; k < K; k += DUALAR_WG)
        xs[bb * K + k] = xs[bb * K + k] * inv * ElemT<T>::load(p.gain, k);
    }
    __syncthreads();
  }

  // ---- rows ----
  const int row0 = (blockIdx.x * 4 + wave) * RPW;
  if (row0 >= p.n_out) return;
  const int n_units = K / (64 * EPV);
  const char* wp[RPW][NR];
  bool live[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    live[r] = (row0 + r) < p.n_out;
    const int row = live[r] ? row0 + r : row0;
#pragma unroll
    for (int s = 0; s < NR; ++s) wp[r][s] = seg_row<T>(p, row, s) + (size_t)lane * EPV * sizeof(T);
  }
  float acc[RPW][NR][BT];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int s = 0; s < NR; ++s)
#pragma unroll
      for (int bb = 0; bb < BT; ++bb) acc[r][s][bb] = 0.f;

  u32x4 cur[RPW][NR];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int s = 0; s < NR; ++s) cur[r][s] = ld_stream(wp[r][s]);

  for (int u = 0; u < n_units; ++u) {
    u32x4 nxt[RPW][NR];
    const bool more = (u + 1) < n_units;
    const size_t off = (size_t)(u + 1) * 64 * EPV * sizeof(T);
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int s = 0; s < NR; ++s) nxt[r][s] = more ? ld_stream(wp[r][s] + off) : cur[r][s];

    const int kb = u * 64 * EPV + lane * EPV;
    float xv[BT][EPV];
#pragma unroll
    for (int bb = 0; bb < BT; ++bb)
#pragma unroll
      for (int e = 0; e < EPV; e += 4) {
        const float4 t = *(const float4*)&xs[bb * K + kb + e];
        xv[bb][e] = t.x; xv[bb][e + 1] = t.y; xv[bb][e + 2] = t.z; xv[bb][e + 3] = t.w;
      }
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int s = 0; s < NR; ++s) {
        float wf[EPV];
        ElemT<T>::unpack(cur[r][s], wf);
#pragma unroll
        for (int bb = 0; bb < BT; ++bb)
#pragma unroll
          for (int e = 0; e < EPV; ++e) acc[r][s][bb] = fmaf(wf[e], xv[bb][e], acc[r][s][bb]);
      }
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int s = 0; s < NR; ++s) cur[r][s] = nxt[r][s];
  }

#pragma unroll
  for (int r = 0; r < RPW; ++r) {
#pragma unroll
    for (int bb = 0; bb < BT; ++bb) {
      float v0 = wave_sum(acc[r][0][bb]);
      float v1 = (NR == 2) ? wave_sum(acc[r][NR - 1][bb]) : 0.f;
      const int b = b0 + bb;
      if (lane == 0 && live[r] && b < p.B) {
        const int row = row0 + r;
        float out;
        if (p.mode == GEMV_SWIGLU) out = silu_f(v0) * v1;
        else if (p.mode == GEMV_ADD) out = p.res[(size_t)b * p.ldres + row] + v0;
        else out = v0;
        p.y[(size_t)b * p.ldy + row] = out;
      }
    }
  }
}

template <typename T, int BT, int RPW, int NR>
static hipError_t go(const GemvParams& p, hipStream_t s) {
  dim3 grid((p.n_out + 4 * RPW - 1) / (4 * RPW), (p.B + BT - 1) / BT);
  size_t lds = (size_t)BT * p.K * sizeof(float);
  hipLaunchKernelGGL((gemv_kernel<T, BT, RPW, NR>), grid, dim3(DUALAR_WG), lds, s, p);
  return hipGetLastError();
}

template <typename T, int BT, int NR>
static hipError_t pick_rpw(const GemvParams& p, hipStream_t s) {
  // Enough workgroups to cover 256 CUs several times over.
  if (p.n_out >= 8192 * 4 / NR) return go<T, BT, 4, NR>(p, s);
  if (p.n_out >= 4096) return go<T, BT, 2, NR>(p, s);
  return go<T, BT, 1, NR>(p, s);
}

template <typename T, int NR>
static hipError_t pick_bt(const GemvParams& p, hipStream_t s) {
  const size_t lim = 48 * 1024;   // dynamic LDS for the staged activations
  if (p.B >= 3 && 4 * (size_t)p.K * 4 <= lim) return pick_rpw<T, 4, NR>(p, s);
  if (p.B >= 2 && 2 * (size_t)p.K * 4 <= lim) return pick_rpw<T, 2, NR>(p, s);
  return pick_rpw<T, 1, NR>(p, s);
}

template <typename T> hipError_t launch_gemv(const GemvParams& p, hipStream_t s) {
  if (p.mode == GEMV_SWIGLU) return pick_bt<T, 2>(p, s);
  return pick_bt<T, 1>(p, s);
}

template hipError_t launch_gemv<float>(const GemvParams&, hipStream_t);
template hipError_t launch_gemv<bf16_t>(const GemvParams&, hipStream_t);
