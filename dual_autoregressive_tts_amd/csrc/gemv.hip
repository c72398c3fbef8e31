// Bandwidth-bound matrix-vector products of the decode step (up to 4
// activation rows per pass): y = W . f(x), W streamed once from HBM in
// 16-byte lane loads.
//
// A workgroup is 4 waves; each wave owns RPW output rows (RPW gate/up row
// pairs for SwiGLU).  Lane l reads elements [u*64*EPV + l*EPV, +EPV) of a row
// for unit u, so one wave load covers 1 KB of one row, contiguous.
//
// gemv_unrolled_kernel (rows of exactly NU units, NU a compile-time
// constant): every weight load of the wave is issued first -- NU*RPW*NR
// 16-byte loads per lane in flight -- and only then are the activations
// staged into LDS (with the fused RMSNorm prologue when a gain is given), so
// staging hides under the weight latency.  gemv_loop_kernel serves any other
// row length with a two-deep software pipeline.
//
// Partial dot products are reduced across the wave with a fixed butterfly,
// so results are deterministic.  Epilogues: store, residual add, SwiGLU
// (silu(gate) * up).
#include "common.h"
#include "internal.h"

thread_local LaunchEvents g_launch_ev{nullptr, nullptr};

template <typename T> __device__ __forceinline__ const char* seg_row(const GemvParams& p, int row, int s) {
  // SwiGLU: s selects gate (w[0]) or up (w[1]) at the same row.
  if (p.mode == GEMV_SWIGLU) return (const char*)p.w[s] + (size_t)row * p.K * sizeof(T);
  if (row < p.rows[0]) return (const char*)p.w[0] + (size_t)row * p.K * sizeof(T);
  row -= p.rows[0];
  if (row < p.rows[1]) return (const char*)p.w[1] + (size_t)row * p.K * sizeof(T);
  row -= p.rows[1];
  return (const char*)p.w[2] + (size_t)row * p.K * sizeof(T);
}

// Activation rows for the LDS-staged kernels: a thread's share of BT rows
// (XR float4 per row) is loaded into registers first, before any weight load
// of the wave, then written to LDS once the weights are in flight.
template <int BT, int XR>
struct XRegs { float4 v[BT][XR]; };

template <int BT, int XR>
__device__ __forceinline__ void load_x(const GemvParams& p, XRegs<BT, XR>& xr, int b0) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) {
    const int b = b0 + bb;
    const float4* src = (const float4*)(p.x + (size_t)b * p.ldx);
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      const int k4 = tid + i * DUALAR_WG;
      xr.v[bb][i] = (b < p.B && k4 < p.K / 4) ? src[k4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// Write the staged rows to LDS, then apply RMSNorm * gain when a gain is set.
template <typename T, int BT, int XR>
__device__ __forceinline__ void store_x(const GemvParams& p, const XRegs<BT, XR>& xr, float* xs, float (*red)[4]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.K;
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) {
    float ss = 0.f;
    float4* dst = (float4*)(xs + bb * K);
#pragma unroll
    for (int i = 0; i < XR; ++i) {
      const int k4 = tid + i * DUALAR_WG;
      const float4 v = xr.v[bb][i];
      if (k4 < K / 4) dst[k4] = v;
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
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
      for (int k = tid; k < K; k += DUALAR_WG) xs[bb * K + k] = xs[bb * K + k] * inv * ElemT<T>::load(p.gain, k);
    }
    __syncthreads();
  }
}

// Generic staging for arbitrary K (loop kernel).
template <typename T, int BT>
__device__ __forceinline__ void stage_x(const GemvParams& p, float* xs, float (*red)[4], int b0) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = p.K;
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) {
    const int b = b0 + bb;
    float ss = 0.f;
    const float4* src = (const float4*)(p.x + (size_t)b * p.ldx);
    float4* dst = (float4*)(xs + bb * K);
    for (int k4 = tid; k4 < K / 4; k4 += DUALAR_WG) {
      const float4 v = (b < p.B) ? src[k4] : make_float4(0.f, 0.f, 0.f, 0.f);
      dst[k4] = v;
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
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
      for (int k = tid; k < K; k += DUALAR_WG) xs[bb * K + k] = xs[bb * K + k] * inv * ElemT<T>::load(p.gain, k);
    }
    __syncthreads();
  }
}

template <int RPW, int NR, int BT>
__device__ __forceinline__ void gemv_epilogue(const GemvParams& p, float (&acc)[RPW][NR][BT], int row0, int b0) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
#pragma unroll
    for (int bb = 0; bb < BT; ++bb) {
      const float v0 = wave_sum(acc[r][0][bb]);
      const float v1 = (NR == 2) ? wave_sum(acc[r][NR - 1][bb]) : 0.f;
      const int b = b0 + bb, row = row0 + r;
      if (lane == 0 && row < p.n_out && b < p.B) {
        float out;
        if (p.mode == GEMV_SWIGLU) out = silu_f(v0) * v1;
        else if (p.mode == GEMV_ADD) out = p.res[(size_t)b * p.ldres + row] + v0;
        else out = v0;
        p.y[(size_t)b * p.ldy + row] = out;
      }
    }
  }
}

template <typename T, int BT, int RPW, int NR, int NU>
__global__ void __launch_bounds__(DUALAR_WG) gemv_unrolled_kernel(GemvParams p) {
  extern __shared__ float xs[];  // [BT][K]
  __shared__ float red[BT][4];
  constexpr int EPV = ElemT<T>::EPV;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b0 = blockIdx.y * BT;
  const int row0 = (blockIdx.x * 4 + wave) * RPW;

  // 1. this thread's share of the activation rows, then all weight loads
  constexpr int XR = (NU * 64 * EPV / 4 + DUALAR_WG - 1) / DUALAR_WG;
  XRegs<BT, XR> xr;
  load_x<BT, XR>(p, xr, b0);
  u32x4 w[NU][RPW][NR];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = min(row0 + r, p.n_out - 1);
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      const char* base = seg_row<T>(p, row, s) + (size_t)lane * EPV * sizeof(T);
#pragma unroll
      for (int u = 0; u < NU; ++u) w[u][r][s] = ld_stream(base + (size_t)u * 64 * EPV * sizeof(T));
    }
  }
  // 2. activations to LDS (+ RMSNorm) while the weights are in flight
  store_x<T, BT, XR>(p, xr, xs, red);

  // 3. dot products
  float acc[RPW][NR][BT];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int s = 0; s < NR; ++s)
#pragma unroll
      for (int bb = 0; bb < BT; ++bb) acc[r][s][bb] = 0.f;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int kb = u * 64 * EPV + lane * EPV;
    float xv[BT][EPV];
#pragma unroll
    for (int bb = 0; bb < BT; ++bb)
#pragma unroll
      for (int e = 0; e < EPV; e += 4) {
        const float4 t = *(const float4*)&xs[bb * p.K + kb + e];
        xv[bb][e] = t.x; xv[bb][e + 1] = t.y; xv[bb][e + 2] = t.z; xv[bb][e + 3] = t.w;
      }
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int s = 0; s < NR; ++s) {
        float wf[EPV];
        ElemT<T>::unpack(w[u][r][s], wf);
#pragma unroll
        for (int bb = 0; bb < BT; ++bb)
#pragma unroll
          for (int e = 0; e < EPV; ++e) acc[r][s][bb] = fmaf(wf[e], xv[bb][e], acc[r][s][bb]);
      }
  }
  gemv_epilogue<RPW, NR, BT>(p, acc, row0, b0);
}

// One activation row, rows of NU units: every lane loads the activation
// slice it multiplies (NU * EPV floats, the same k indices for every row it
// owns) before issuing its weight loads, so waiting for the activations never
// waits behind the weights (loads complete in order).  The 64 lanes of a wave
// hold all of x between them, so the RMSNorm prologue is a wave reduction: no
// LDS, no barrier.
template <typename T, int RPW, int NR, int NU>
__global__ void __launch_bounds__(DUALAR_WG) gemv_rx_kernel(GemvParams p) {
  constexpr int EPV = ElemT<T>::EPV;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * 4 + wave) * RPW;

  // 1. activation slice (+ gain slice)
  float xv[NU][EPV];
  const float* xb = p.x + lane * EPV;
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int e = 0; e < EPV; e += 4) {
      const float4 t = *(const float4*)(xb + u * 64 * EPV + e);
      xv[u][e] = t.x; xv[u][e + 1] = t.y; xv[u][e + 2] = t.z; xv[u][e + 3] = t.w;
    }
  u32x4 gv[NU];
  if (p.gain) {
#pragma unroll
    for (int u = 0; u < NU; ++u) gv[u] = ld_vec((const char*)p.gain + (size_t)(u * 64 + lane) * EPV * sizeof(T));
  }
  // 2. weights
  u32x4 w[NU][RPW][NR];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = min(row0 + r, p.n_out - 1);
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      const char* base = seg_row<T>(p, row, s) + (size_t)lane * EPV * sizeof(T);
#pragma unroll
      for (int u = 0; u < NU; ++u) w[u][r][s] = ld_stream(base + (size_t)u * 64 * EPV * sizeof(T));
    }
  }
  // 3. RMSNorm * gain, in registers
  if (p.gain) {
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int e = 0; e < EPV; ++e) ss += xv[u][e] * xv[u][e];
    const float inv = 1.0f / sqrtf(wave_sum(ss) / (float)p.K + p.eps);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      float g[EPV];
      ElemT<T>::unpack(gv[u], g);
#pragma unroll
      for (int e = 0; e < EPV; ++e) xv[u][e] = xv[u][e] * inv * g[e];
    }
  }
  // 4. dot products
  float acc[RPW][NR][1];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int s = 0; s < NR; ++s) acc[r][s][0] = 0.f;
#pragma unroll
  for (int u = 0; u < NU; ++u)
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int s = 0; s < NR; ++s) {
        float wf[EPV];
        ElemT<T>::unpack(w[u][r][s], wf);
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[r][s][0] = fmaf(wf[e], xv[u][e], acc[r][s][0]);
      }
  gemv_epilogue<RPW, NR, 1>(p, acc, row0, 0);
}

// One activation row, rows of NU units split in KS parts: the 4 waves of a
// workgroup are 4/KS row groups x KS k-parts.  Each wave loads its
// activation (and gain) slice first (NUP units), then its weights; the KS
// partial sums of squares (RMSNorm) and the KS partial dot products of a row
// meet in LDS.
template <typename T, int RPW, int NR, int NU, int KS>
__global__ void __launch_bounds__(DUALAR_WG) gemv_ks_kernel(GemvParams p) {
  constexpr int EPV = ElemT<T>::EPV;
  constexpr int NUP = (NU + KS - 1) / KS;
  __shared__ float part[4][RPW][NR];
  __shared__ float ssq[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kp = wave % KS;
  const int row0 = (blockIdx.x * (4 / KS) + wave / KS) * RPW;
  const int u0 = kp * NUP;

  float xv[NUP][EPV];
  const float* xb = p.x + lane * EPV;
#pragma unroll
  for (int u = 0; u < NUP; ++u) {
    const int uu = min(u0 + u, NU - 1);
#pragma unroll
    for (int e = 0; e < EPV; e += 4) {
      const float4 t = *(const float4*)(xb + uu * 64 * EPV + e);
      const bool live = u0 + u < NU;
      xv[u][e] = live ? t.x : 0.f; xv[u][e + 1] = live ? t.y : 0.f;
      xv[u][e + 2] = live ? t.z : 0.f; xv[u][e + 3] = live ? t.w : 0.f;
    }
  }
  u32x4 gv[NUP];
  if (p.gain) {
#pragma unroll
    for (int u = 0; u < NUP; ++u) {
      const int uu = min(u0 + u, NU - 1);
      gv[u] = ld_vec((const char*)p.gain + (size_t)(uu * 64 + lane) * EPV * sizeof(T));
    }
  }
  u32x4 w[NUP][RPW][NR];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = min(row0 + r, p.n_out - 1);
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      const char* base = seg_row<T>(p, row, s) + (size_t)lane * EPV * sizeof(T);
#pragma unroll
      for (int u = 0; u < NUP; ++u) {
        const int uu = min(u0 + u, NU - 1);
        w[u][r][s] = ld_stream(base + (size_t)uu * 64 * EPV * sizeof(T));
      }
    }
  }
  if (p.gain) {
    // every row group holds the whole activation row across its KS waves
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < NUP; ++u)
#pragma unroll
      for (int e = 0; e < EPV; ++e) ss += xv[u][e] * xv[u][e];
    ss = wave_sum(ss);
    if (lane == 0) ssq[wave] = ss;
    __syncthreads();
    float tot = 0.f;
    const int g0 = wave - kp;
    for (int q = 0; q < KS; ++q) tot += ssq[g0 + q];
    const float inv = 1.0f / sqrtf(tot / (float)p.K + p.eps);
#pragma unroll
    for (int u = 0; u < NUP; ++u) {
      float g[EPV];
      ElemT<T>::unpack(gv[u], g);
#pragma unroll
      for (int e = 0; e < EPV; ++e) xv[u][e] = xv[u][e] * inv * g[e];
    }
  }
  float acc[RPW][NR];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int s = 0; s < NR; ++s) acc[r][s] = 0.f;
#pragma unroll
  for (int u = 0; u < NUP; ++u)
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int s = 0; s < NR; ++s) {
        float wf[EPV];
        ElemT<T>::unpack(w[u][r][s], wf);
#pragma unroll
        for (int e = 0; e < EPV; ++e) acc[r][s] = fmaf(wf[e], xv[u][e], acc[r][s]);
      }
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      const float v = wave_sum(acc[r][s]);
      if (lane == 0) part[wave][r][s] = v;
    }
  __syncthreads();
  if (kp != 0 || lane != 0) return;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = row0 + r;
    if (row >= p.n_out) continue;
    float v[NR];
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      v[s] = 0.f;
      for (int q = 0; q < KS; ++q) v[s] += part[wave + q][r][s];
    }
    float out;
    if (p.mode == GEMV_SWIGLU) out = silu_f(v[0]) * v[NR - 1];
    else if (p.mode == GEMV_ADD) out = p.res[row] + v[0];
    else out = v[0];
    p.y[row] = out;
  }
}

// One activation row, bf16 rows of U units (512 elements): one workgroup per
// R consecutive output rows, sized so that the product is about one
// workgroup per compute unit.  The NW waves split into NR segment groups
// (gate, up for SwiGLU) of NWS = NW / NR waves; wave w of a group owns units
// u = w, w + NWS, ... of every row of the workgroup, so each lane keeps
// R * ceil(U / NWS) 16-byte weight loads in flight behind its activation
// slice.  Fewer, larger workgroups than the 4-wave kernels: at batch 1 the
// per-workgroup dispatch and ramp are a visible share of a 20-100 MB
// product.  The RMSNorm prologue's sum of squares meets in LDS (each unit
// belongs to one wave of a group); per-wave partial dot products are summed
// over the group's waves in order.
template <int NW, int R, int NR, int U>
__global__ void __launch_bounds__(NW * 64) gemv_wide_kernel(GemvParams p) {
  constexpr int NWS = NW / NR;
  constexpr int UPW = (U + NWS - 1) / NWS;
  __shared__ float part[NR][R][NWS];
  __shared__ float ssq[NWS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int seg = wave / NWS, wv = wave % NWS;
  const int row0 = blockIdx.x * R;

  // 1. the activation slices of the wave's units (+ gain)
  float xv[UPW][8];
  u32x4 gv[UPW];
#pragma unroll
  for (int i = 0; i < UPW; ++i) {
    const int u = wv + NWS * i;
    const bool live = u < U;
    const float* xs = p.x + (size_t)(live ? u : 0) * 512 + lane * 8;
    const float4 a = *(const float4*)xs, b = *(const float4*)(xs + 4);
    xv[i][0] = live ? a.x : 0.f; xv[i][1] = live ? a.y : 0.f; xv[i][2] = live ? a.z : 0.f; xv[i][3] = live ? a.w : 0.f;
    xv[i][4] = live ? b.x : 0.f; xv[i][5] = live ? b.y : 0.f; xv[i][6] = live ? b.z : 0.f; xv[i][7] = live ? b.w : 0.f;
    if (p.gain) gv[i] = ld_vec((const char*)p.gain + ((size_t)(live ? u : 0) * 512 + lane * 8) * sizeof(bf16_t));
  }
  // 2. weights
  u32x4 w[R][UPW];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = min(row0 + r, p.n_out - 1);
    // SwiGLU: the wave's segment (gate or up) by a compare, not an index
    // into the argument array (which would go through scratch)
    const char* base = (NR == 2 ? (const char*)(seg == 0 ? p.w[0] : p.w[1]) + (size_t)row * p.K * sizeof(bf16_t)
                                : seg_row<bf16_t>(p, row, 0)) + (size_t)lane * 8 * sizeof(bf16_t);
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      const int u = min(wv + NWS * i, U - 1);
      w[r][i] = ld_stream(base + (size_t)u * 512 * sizeof(bf16_t));
    }
  }
  // 3. RMSNorm * gain: the group's waves hold every unit once
  if (p.gain) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < UPW; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += xv[i][e] * xv[i][e];
    ss = wave_sum(ss);
    if (lane == 0 && seg == 0) ssq[wv] = ss;
    __syncthreads();
    float tot = ssq[0];
#pragma unroll
    for (int q = 1; q < NWS; ++q) tot += ssq[q];
    const float inv = 1.0f / sqrtf(tot / (float)p.K + p.eps);
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      float g[8];
      ElemT<bf16_t>::unpack(gv[i], g);
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[i][e] = xv[i][e] * inv * g[e];
    }
  }
  // 4. dot products over the wave's units, reduced across the wave
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < UPW; ++i) {
      float wf[8];
      ElemT<bf16_t>::unpack(w[r][i], wf);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(wf[e], xv[i][e], acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) part[seg][r][wv] = acc;
  }
  __syncthreads();
  // 5. epilogue: one thread per row
  if ((int)threadIdx.x < R && row0 + (int)threadIdx.x < p.n_out) {
    const int r = threadIdx.x, row = row0 + r;
    float v[NR];
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      v[s] = part[s][r][0];
#pragma unroll
      for (int q = 1; q < NWS; ++q) v[s] += part[s][r][q];
    }
    float out;
    if (p.mode == GEMV_SWIGLU) out = silu_f(v[0]) * v[NR - 1];
    else if (p.mode == GEMV_ADD) out = p.res[row] + v[0];
    else out = v[0];
    p.y[row] = out;
  }
}

template <typename T, int BT, int RPW, int NR>
__global__ void __launch_bounds__(DUALAR_WG) gemv_loop_kernel(GemvParams p) {
  extern __shared__ float xs[];  // [BT][K]
  __shared__ float red[BT][4];
  constexpr int EPV = ElemT<T>::EPV;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int b0 = blockIdx.y * BT;
  const int row0 = (blockIdx.x * 4 + wave) * RPW;
  const int n_units = p.K / (64 * EPV);

  const char* wp[RPW][NR];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = min(row0 + r, p.n_out - 1);
#pragma unroll
    for (int s = 0; s < NR; ++s) wp[r][s] = seg_row<T>(p, row, s) + (size_t)lane * EPV * sizeof(T);
  }
  u32x4 cur[RPW][NR];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int s = 0; s < NR; ++s) cur[r][s] = ld_stream(wp[r][s]);
  stage_x<T, BT>(p, xs, red, b0);

  float acc[RPW][NR][BT];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int s = 0; s < NR; ++s)
#pragma unroll
      for (int bb = 0; bb < BT; ++bb) acc[r][s][bb] = 0.f;
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
        const float4 t = *(const float4*)&xs[bb * p.K + kb + e];
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
  gemv_epilogue<RPW, NR, BT>(p, acc, row0, b0);
}

// ---------------------------------------------------------------------------
// 4-bit weights (W4A16), one activation row
// ---------------------------------------------------------------------------
// Rows of K inputs as packed 4-bit two's-complement values (input 2j in the
// low nibble of byte j) with a bf16 scale per group of 128 inputs.  A row is
// read in units of 512 inputs: lane l takes dword l of each unit (inputs
// 8l .. 8l+7, all in group l/16 of the unit), so one wave load covers 256
// contiguous bytes of a row and every lane of a wave has work for any K that
// is a multiple of 512.  As in the bf16 register-staged kernels, each lane
// loads its activation (and gain) slice before its weights, and the RMSNorm
// sum of squares is a wave reduction (with KS > 1 the KS waves of a row
// group split the units and meet in LDS).  Per dword, t' = t ^ 8 turns each
// nibble into v + 8 in [0, 15]; the low nibbles convert from their bytes,
// the high ones from their bytes as 16 (v + 8) against activations
// pre-divided by 16 (exact), and the lane adds scale * (sum t' x - 8 sum x)
// to its row.
template <int NR>
__device__ __forceinline__ const char* w4_row(const GemvParams& p, int row, int s, const uint16_t** sc) {
  int seg = 0;
  if (p.mode == GEMV_SWIGLU) seg = s;
  else if (row >= p.rows[0]) {
    row -= p.rows[0];
    seg = 1;
    if (row >= p.rows[1]) { row -= p.rows[1]; seg = 2; }
  }
  const void* q = seg == 0 ? p.q4[0] : seg == 1 ? p.q4[1] : p.q4[2];
  const void* g = seg == 0 ? p.s4[0] : seg == 1 ? p.s4[1] : p.s4[2];
  *sc = (const uint16_t*)g + (size_t)row * (p.K / 128);
  return (const char*)q + (size_t)row * (p.K / 2);
}

template <int RPW, int NR, int NUP, int KS, bool RAG>
__global__ void __launch_bounds__(DUALAR_WG) gemv_w4_kernel(GemvParams p) {
  // RAG: the units do not divide evenly among the KS waves, so the last
  // wave's trailing units are dead (their loads are clamped, their x zeroed)
  __shared__ float part[4][RPW][NR];
  __shared__ float ssq[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kp = wave % KS;
  const int row0 = (blockIdx.x * (4 / KS) + wave / KS) * RPW;
  const int U = p.K >> 9;
  const int u0 = kp * NUP;
  auto unit = [&](int u) { return RAG ? min(u0 + u, U - 1) : u0 + u; };

  // 1. activation slice (+ gain slice): inputs 8 (64 u + lane) .. + 7
  float xv[NUP][8];
#pragma unroll
  for (int u = 0; u < NUP; ++u) {
    const float* xb = p.x + (size_t)(unit(u) * 64 + lane) * 8;
    const float4 a = *(const float4*)xb, b = *(const float4*)(xb + 4);
    const bool live = !RAG || u0 + u < U;
    xv[u][0] = live ? a.x : 0.f; xv[u][1] = live ? a.y : 0.f; xv[u][2] = live ? a.z : 0.f; xv[u][3] = live ? a.w : 0.f;
    xv[u][4] = live ? b.x : 0.f; xv[u][5] = live ? b.y : 0.f; xv[u][6] = live ? b.z : 0.f; xv[u][7] = live ? b.w : 0.f;
  }
  u32x4 gv[NUP];
  if (p.gain) {
#pragma unroll
    for (int u = 0; u < NUP; ++u) gv[u] = ld_vec((const char*)p.gain + (size_t)(unit(u) * 64 + lane) * 16);
  }
  // 2. packed weights and their scales
  uint32_t wq[NUP][RPW][NR], sc[NUP][RPW][NR];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int row = min(row0 + r, p.n_out - 1);
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      const uint16_t* sb;
      const uint32_t* qb = (const uint32_t*)w4_row<NR>(p, row, s, &sb);
      if constexpr (!RAG) {
        qb += u0 * 64 + lane;
        sb += u0 * 4 + (lane >> 4);
      }
#pragma unroll
      for (int u = 0; u < NUP; ++u) {
        if constexpr (RAG) {
          const int d = unit(u) * 64 + lane;
          wq[u][r][s] = __builtin_nontemporal_load(qb + d);
          sc[u][r][s] = sb[d >> 4];
        } else {
          wq[u][r][s] = __builtin_nontemporal_load(qb + 64 * u);
          sc[u][r][s] = sb[4 * u];
        }
      }
    }
  }
  // 3. RMSNorm: x * gain here, the 1 / rms factor on the finished sums
  float inv = 1.f;
  if (p.gain) {
    float ss = 0.f;
#pragma unroll
    for (int u = 0; u < NUP; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += xv[u][e] * xv[u][e];
    ss = wave_sum(ss);
    float tot = ss;
    if constexpr (KS > 1) {
      if (lane == 0) ssq[wave] = ss;
      __syncthreads();
      tot = 0.f;
      for (int q = 0; q < KS; ++q) tot += ssq[wave - kp + q];
    }
    inv = 1.0f / sqrtf(tot / (float)p.K + p.eps);
#pragma unroll
    for (int u = 0; u < NUP; ++u) {
      float g[8];
      ElemT<bf16_t>::unpack(gv[u], g);
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[u][e] *= g[e];
    }
  }
  // 4. -8 sum x per unit (shared by every row), odd inputs / 16
  float m8[NUP];
#pragma unroll
  for (int u = 0; u < NUP; ++u) {
    float t = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) t += xv[u][e];
    m8[u] = -8.f * t;
#pragma unroll
    for (int e = 1; e < 8; e += 2) xv[u][e] *= 0.0625f;
  }
  // 5. dot products
  float acc[RPW][NR][1];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int s = 0; s < NR; ++s) acc[r][s][0] = 0.f;
#pragma unroll
  for (int u = 0; u < NUP; ++u)
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int s = 0; s < NR; ++s) {
        const uint32_t t = wq[u][r][s] ^ 0x88888888u;
        uint32_t lo = t & 0x0F0F0F0Fu, hi = t & 0xF0F0F0F0u;
        // hide the known-zero bits, so that each byte converts in one
        // v_cvt_f32_ubyte{0..3} rather than a bit-field extract and a convert
        __asm__("" : "+v"(lo), "+v"(hi));
        float d = m8[u];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          d = fmaf((float)((lo >> (8 * b)) & 0xFFu), xv[u][2 * b], d);
          d = fmaf((float)((hi >> (8 * b)) & 0xFFu), xv[u][2 * b + 1], d);
        }
        acc[r][s][0] = fmaf(bf16_bits_to_f32(sc[u][r][s]), d, acc[r][s][0]);
      }
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int s = 0; s < NR; ++s) acc[r][s][0] *= inv;
  if constexpr (KS == 1) {
    gemv_epilogue<RPW, NR, 1>(p, acc, row0, 0);
  } else {
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int s = 0; s < NR; ++s) {
        const float v = wave_sum(acc[r][s][0]);
        if (lane == 0) part[wave][r][s] = v;
      }
    __syncthreads();
    if (kp != 0 || lane != 0) return;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int row = row0 + r;
      if (row >= p.n_out) continue;
      float v[NR];
#pragma unroll
      for (int s = 0; s < NR; ++s) {
        v[s] = 0.f;
        for (int q = 0; q < KS; ++q) v[s] += part[wave + q][r][s];
      }
      float out;
      if (p.mode == GEMV_SWIGLU) out = silu_f(v[0]) * v[NR - 1];
      else if (p.mode == GEMV_ADD) out = p.res[row] + v[0];
      else out = v[0];
      p.y[row] = out;
    }
  }
}

// 4-bit weights on the matrix cores (v_mfma_f32_16x16x32_bf16): a workgroup
// owns 16 output rows (x NR segments) and its NWV waves split the row's
// 128-input groups (chunks; one bf16 scale each) in ranges of NCH.  Per chunk
// and segment, lane (q = lane / 16, n = lane % 16) loads 16 bytes of row n:
// dwords 4q .. 4q+3, i.e. the 8-input octets 4q + i, i = 0..3.  Product step i
// takes octet 4q + i from every lane: B = the 16 rows' weights (one dword,
// eight nibbles, is one lane's fragment), A = the activation as three bf16
// terms in rows 0..2 (rows 3..15 feed only D rows that are never read).  A
// nibble t' = v + 8 becomes the exact bf16 128 + t' by a byte permute with
// the constant byte 0x43, so the products give sum (136 + v) x; the
// accumulator starts at -136 sum x for the chunk, and row n's chunk result
// d0 + d1 + d2 is scaled into its sum.  The wave builds its own range's
// activation terms in LDS (per product step: 4 octet slots x 3 terms x
// 16 bytes), in the octet order the permute produces: inputs 0 2 4 6 1 3 5 7.
// RMSNorm: the terms are of x * gain, and 1 / rms scales the finished sums.
typedef __bf16 w4m_bf16x8 __attribute__((ext_vector_type(8)));
typedef float w4m_f32x4 __attribute__((ext_vector_type(4)));

template <int NR, int NCH, int NWV>
__global__ void __launch_bounds__(NWV * 64) gemv_w4m_kernel(GemvParams p) {
  extern __shared__ u32x4 xa[];                 // [NWV][NCH * 4 steps][12 slots]
  __shared__ float part[NWV][NR][16];
  __shared__ float ssq[NWV];
  __shared__ float sxs[NWV][NCH];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, n = lane & 15;
  const int C = p.K >> 7;
  const int c0 = wave * NCH;
  const int cnt = min(NCH, C - c0);              // chunks of this wave (<= 0: none)
  const int r0 = blockIdx.x * 16;
  u32x4* xw = xa + (size_t)wave * NCH * 4 * 12;

  // 1. activation octets of the wave's range: octet o -> lane o % 64, pass o / 64
  constexpr int NO = (16 * NCH + 63) / 64;
  float xv[NO][8];
  u32x4 gv[NO];
#pragma unroll
  for (int it = 0; it < NO; ++it) {
    const int o = lane + 64 * it;
    const int og = min(max(16 * c0 + o, 0), 16 * C - 1);
    const float* xb = p.x + (size_t)og * 8;
    const float4 a = *(const float4*)xb, b = *(const float4*)(xb + 4);
    xv[it][0] = a.x; xv[it][1] = a.y; xv[it][2] = a.z; xv[it][3] = a.w;
    xv[it][4] = b.x; xv[it][5] = b.y; xv[it][6] = b.z; xv[it][7] = b.w;
    if (p.gain) gv[it] = ld_vec((const char*)p.gain + (size_t)og * 16);
  }
  // 2. weights and scales of the 16 rows
  u32x4 wq[NCH][NR];
  uint32_t sc[NCH][NR];
  {
    const int row = min(r0 + n, p.n_out - 1);
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      const uint16_t* sb;
      const char* qb = w4_row<NR>(p, row, s, &sb);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int cc = min(c0 + c, C - 1);
        wq[c][s] = ld_stream(qb + (size_t)cc * 64 + q * 16);
        sc[c][s] = sb[cc];
      }
    }
  }
  // 3. x * gain as three bf16 terms into LDS; chunk sums; sum of squares
  float ss = 0.f;
#pragma unroll
  for (int it = 0; it < NO; ++it) {
    const int o = lane + 64 * it;
    const bool live = o < 16 * cnt;
    float g[8];
    if (p.gain) ElemT<bf16_t>::unpack(gv[it], g);
    float sx = 0.f;
    uint32_t t0[4], t1[4], t2[4];
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      // fragment pair e2 holds inputs (2 e2, 2 e2 + 2) for e2 < 2, (2 e2 - 3, 2 e2 - 1) after
      const int ea = e2 < 2 ? 4 * e2 : 4 * (e2 - 2) + 1, eb = ea + 2;
      uint32_t h[2], m[2], l[2];
      const int es[2] = {ea, eb};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float x = live ? xv[it][es[k]] : 0.f;
        ss = fmaf(x, x, ss);
        const float xg = p.gain ? x * g[es[k]] : x;
        h[k] = f32_to_bf16_rne(xg);
        const float r1 = xg - bf16_bits_to_f32(h[k]);
        m[k] = f32_to_bf16_rne(r1);
        const float r2 = r1 - bf16_bits_to_f32(m[k]);
        l[k] = f32_to_bf16_rne(r2);
        sx += bf16_bits_to_f32(h[k]) + bf16_bits_to_f32(m[k]) + bf16_bits_to_f32(l[k]);
      }
      t0[e2] = h[0] | (h[1] << 16);
      t1[e2] = m[0] | (m[1] << 16);
      t2[e2] = l[0] | (l[1] << 16);
    }
    if (live) {
      const int j = o >> 4, oo = o & 15;         // local chunk, octet in the chunk
      u32x4* slot = xw + (size_t)(4 * j + (oo & 3)) * 12 + (oo >> 2) * 3;
      slot[0] = u32x4{t0[0], t0[1], t0[2], t0[3]};
      slot[1] = u32x4{t1[0], t1[1], t1[2], t1[3]};
      slot[2] = u32x4{t2[0], t2[1], t2[2], t2[3]};
    }
    sx = group_sum(sx, 16);                      // the 16 octets of chunk 4 it + q
    if (n == 0 && 4 * it + q < cnt) sxs[wave][4 * it + q] = sx;
  }
  ss = wave_sum(ss);
  if (lane == 0) ssq[wave] = ss;
  __builtin_amdgcn_wave_barrier();               // xw, sxs[wave]: this wave's own
  __builtin_amdgcn_s_waitcnt(0xc07f);            // lgkmcnt(0): the LDS writes are done

  // 4. the products
  float acc[NR];
#pragma unroll
  for (int s = 0; s < NR; ++s) acc[s] = 0.f;
  const int slot_a = q * 3 + min(n, 2);          // A row n (term n for n < 3), octet slot q
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c < cnt) {
    const float m136 = -136.f * sxs[wave][c];
    u32x4 av[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) av[i] = xw[(size_t)(4 * c + i) * 12 + slot_a];
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      w4m_f32x4 d = {m136, 0.f, 0.f, 0.f};
      const uint32_t wd[4] = {wq[c][s].x, wq[c][s].y, wq[c][s].z, wq[c][s].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t t = wd[i] ^ 0x88888888u;
        const uint32_t lo = t & 0x0F0F0F0Fu, hi = (t >> 4) & 0x0F0F0F0Fu;
        // bytes (v, 0x43, v', 0x43): two exact bf16 values 128 + t'
        const u32x4 b = {__builtin_amdgcn_perm(0x43434343u, lo, 0x04010400u),
                         __builtin_amdgcn_perm(0x43434343u, lo, 0x04030402u),
                         __builtin_amdgcn_perm(0x43434343u, hi, 0x04010400u),
                         __builtin_amdgcn_perm(0x43434343u, hi, 0x04030402u)};
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(w4m_bf16x8, av[i]),
                                                    __builtin_bit_cast(w4m_bf16x8, b), d, 0, 0, 0);
      }
      acc[s] = fmaf(bf16_bits_to_f32(sc[c][s]), (d[0] + d[1]) + d[2], acc[s]);
    }
    }
  }
  // 5. lanes 0..15 hold row n's partial sums; the waves meet in LDS
  if (q == 0) {
#pragma unroll
    for (int s = 0; s < NR; ++s) part[wave][s][n] = acc[s];
  }
  __syncthreads();
  if (threadIdx.x >= 16) return;
  const int row = r0 + threadIdx.x;
  if (row >= p.n_out) return;
  float inv = 1.f;
  if (p.gain) {
    float tot = 0.f;
    for (int w = 0; w < NWV; ++w) tot += ssq[w];
    inv = 1.0f / sqrtf(tot / (float)p.K + p.eps);
  }
  float v[NR];
#pragma unroll
  for (int s = 0; s < NR; ++s) {
    v[s] = 0.f;
    for (int w = 0; w < NWV; ++w) v[s] += part[w][s][threadIdx.x];
    v[s] *= inv;
  }
  float out;
  if (p.mode == GEMV_SWIGLU) out = silu_f(v[0]) * v[NR - 1];
  else if (p.mode == GEMV_ADD) out = p.res[row] + v[0];
  else out = v[0];
  p.y[row] = out;
}

template <int NR, int NCH, int NWV>
static hipError_t go_w4m(const GemvParams& p, hipStream_t s) {
  const size_t lds = (size_t)NWV * NCH * 4 * 12 * 16;
  launch_timed(gemv_w4m_kernel<NR, NCH, NWV>, dim3((p.n_out + 15) / 16), dim3(NWV * 64), (uint32_t)lds, s, p);
  return hipGetLastError();
}

// Chunks of 128 inputs per row: 20 (2,560), 32 (4,096), 76 (9,728).  The
// matrix-core form serves the single-segment products (QKV, O, W2: 6.00 /
// 5.70 / 8.56 us at the S2 shapes against 6.54 / 5.86 / 8.73 us for the
// VALU form, with 8 or 16 waves per workgroup; 4 waves were slower); the
// gate|up product stays on the VALU form (11.2 us against 12.0 / 12.5 us).
template <int NR>
static bool launch_w4m(const GemvParams& p, hipStream_t s, hipError_t* e) {
  if (NR != 1 || p.B != 1 || p.K % 128 || p.xplanes || p.yplanes) return false;
  if constexpr (NR == 1) {
    const int C = p.K / 128;
    if (C <= 24) { *e = go_w4m<1, 3, 8>(p, s); return true; }
    if (C <= 32) { *e = go_w4m<1, 2, 16>(p, s); return true; }
    if (C <= 48) { *e = go_w4m<1, 3, 16>(p, s); return true; }
    if (C <= 80) { *e = go_w4m<1, 5, 16>(p, s); return true; }
  }
  return false;
}

// ---------------------------------------------------------------------------
// 4-bit weights, 2 to 8 activation rows (batched W4A16 decode)
// ---------------------------------------------------------------------------
// The matrix-core form above with the activations taken from the three bf16
// planes [3][B][K] of the batched path (the input split, or a producer's
// output planes), which already hold the normalised input: A row 4b + t of
// v_mfma_f32_16x16x32_bf16 is term t of activation row b (t < 3, b < B; the
// other rows repeat a clamped row and their results are never read), so lane
// group q = b of the result holds row b's three term sums (with two groups
// of four rows, a second product per weight fragment covers rows 4..7).  The
// chunk loop has no branches (a wave's chunks past the row
// are clamped loads with a zero scale) and the segment pointers are chosen by
// selects among SGPR copies, so that every load is issued up front.  The
// weights are unpacked exactly (the nibble's v + 8 less 8 in
// the integer domain, then a convert: bf16 holds every value of [-8, 7]), so
// every product is exact, as in the bf16 path.  (The batch-1 form's byte
// permute to 136 + v with a -136 sum-of-x start measured a fast-logit
// distance of 2.0e-3 at batch 4 on a bf16 cache, against 8.9e-4 exact.)
// Per chunk of 128 inputs (one scale): 4 product steps; at step i lane
// (q, n) takes octet 4q + i of its row, of the weights and of the activation
// term alike.  A wave loads all of its chunks' weights first, then each
// chunk's activation fragments one chunk ahead.  The fragments of A rows
// that feed no result (t = 3, or b >= B) are loaded from a clamped row and
// left unmasked, so every load is unconditional.
__device__ __forceinline__ u32x4 w4b_unpack(uint32_t d) {
  const uint32_t u = d ^ 0x88888888u;
  uint32_t lo = u & 0x0F0F0F0Fu, hi = (u >> 4) & 0x0F0F0F0Fu;
  __asm__("" : "+v"(lo), "+v"(hi));     // known-zero bits: one byte convert each
  u32x4 o;
#pragma unroll
  for (int b = 0; b < 4; ++b)
    o[b] = (uint32_t)f32_to_bf16_rne((float)((lo >> (8 * b)) & 0xFFu) - 8.0f) |
           ((uint32_t)f32_to_bf16_rne((float)((hi >> (8 * b)) & 0xFFu) - 8.0f) << 16);
  return o;
}

typedef __attribute__((address_space(1))) const u32x4 w4b_gvec;
typedef __attribute__((address_space(1))) const uint16_t w4b_gu16;

// NORM: the input is x (fp32, RMSNorm with p.gain when set) rather than
// planes: the workgroup splits x * gain into the three terms in LDS itself
// (its input loads issued before the weights, so that waiting for them leaves
// the weights in flight), sums each row's squares, and scales the finished
// sums by 1 / rms -- no separate split launch.
#define W4B_XU 8   // NORM: float4 input units per thread at most

// G groups of 4 activation rows (B <= 4 G): each unpacked weight fragment
// feeds G products, one per group.
template <int NR, int NCH, int NWV, bool NORM, int G>
__global__ void __launch_bounds__(NWV * 64) gemv_w4b_kernel(GemvParams p) {
  static_assert(!NORM || G == 1, "the input terms of more than 4 rows do not fit the LDS budget");
  extern __shared__ __attribute__((aligned(16))) uint16_t xl[];   // NORM: the input terms [3][B][K]
  __shared__ float part[NWV][4 * G][NR][16];
  __shared__ float ssw[NWV][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, n = lane & 15;
  const int C = p.K >> 7;
  const int c0 = wave * NCH;
  const int cnt = min(NCH, C - c0);              // chunks of this wave (<= 0: none)
  const int r0 = blockIdx.x * 16;
  constexpr int NT = NWV * 64;
  const int nx4 = p.B * p.K / 4;                 // NORM: float4 units of the input
  float4 xv[NORM ? W4B_XU : 1];
  uint2 gv[NORM ? W4B_XU : 1];
  if constexpr (NORM) {
#pragma unroll
    for (int u = 0; u < W4B_XU; ++u) {
      const int e = 4 * min((int)threadIdx.x + u * NT, nx4 - 1);
      const int b = e / p.K, k = e - b * p.K;
      xv[u] = *(const float4*)(p.x + (size_t)b * p.ldx + k);
      gv[u] = p.gain ? *(const uint2*)((const uint16_t*)p.gain + k) : make_uint2(0x3F803F80u, 0x3F803F80u);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // weights and scales of the 16 rows
  u32x4 wq[NCH][NR];
  uint32_t sc[NCH][NR];
  {
    uint64_t q0 = (uint64_t)p.q4[0], q1 = (uint64_t)p.q4[1], q2 = (uint64_t)p.q4[2];
    uint64_t s0 = (uint64_t)p.s4[0], s1 = (uint64_t)p.s4[1], s2 = (uint64_t)p.s4[2];
    asm volatile("" : "+s"(q0), "+s"(q1), "+s"(q2), "+s"(s0), "+s"(s1), "+s"(s2));
    const int row0 = min(r0 + n, p.n_out - 1);
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      int row = row0, seg = s;
      if (NR == 1) {   // rows of up to three segments one after the other
        seg = row >= p.rows[0] ? (row >= p.rows[0] + p.rows[1] ? 2 : 1) : 0;
        row -= seg == 0 ? 0 : (seg == 1 ? p.rows[0] : p.rows[0] + p.rows[1]);
      }
      // (global address space: through a plain pointer rebuilt from an
      // integer these would be flat loads)
      const uint64_t qb = (seg == 0 ? q0 : (seg == 1 ? q1 : q2)) + (uint64_t)row * (p.K / 2) + q * 16;
      const uint64_t sb = (seg == 0 ? s0 : (seg == 1 ? s1 : s2)) + (uint64_t)row * C * 2;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int cc = min(c0 + c, C - 1);
        wq[c][s] = __builtin_nontemporal_load((w4b_gvec*)(qb + (uint64_t)cc * 64));
        sc[c][s] = ((w4b_gu16*)sb)[cc];
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  float ss[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (NORM) {
    // x * gain as three bf16 terms into LDS; each row's sum of squares of x
#pragma unroll
    for (int u = 0; u < W4B_XU; ++u) {
      const int e4 = (int)threadIdx.x + u * NT;
      if (e4 >= nx4) break;
      const int e = 4 * e4, b = e / p.K, k = e - b * p.K;
      const float xs[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
      const uint32_t gs[4] = {gv[u].x & 0xffffu, gv[u].x >> 16, gv[u].y & 0xffffu, gv[u].y >> 16};
      uint32_t t[3][2] = {{0u, 0u}, {0u, 0u}, {0u, 0u}};
      float sq = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sq = fmaf(xs[j], xs[j], sq);
        const float xg = xs[j] * bf16_bits_to_f32(gs[j]);
        const uint32_t a0 = f32_to_bf16_rne(xg);
        const float r1 = xg - bf16_bits_to_f32(a0);
        const uint32_t a1 = f32_to_bf16_rne(r1);
        const uint32_t a2 = f32_to_bf16_rne(r1 - bf16_bits_to_f32(a1));
        t[0][j >> 1] |= a0 << (16 * (j & 1));
        t[1][j >> 1] |= a1 << (16 * (j & 1));
        t[2][j >> 1] |= a2 << (16 * (j & 1));
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) ss[r] += b == r ? sq : 0.f;
#pragma unroll
      for (int tt = 0; tt < 3; ++tt)
        *(uint2*)&xl[((size_t)tt * p.B + b) * p.K + k] = make_uint2(t[tt][0], t[tt][1]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = wave_sum(ss[r]);
      if (lane == 0) ssw[wave][r] = v;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // the weights stay in flight
  }
  // activation fragments: A row n of group g = term (n & 3) of activation
  // row 4 g + (n >> 2); rows with n & 3 == 3 or past B read a clamped row:
  // their result rows are never read
  const int at = min(n & 3, 2);
  const uint16_t* xbase = (NORM ? (const uint16_t*)xl : (const uint16_t*)p.xn) + (size_t)at * p.B * p.K + 32 * q;
  auto load_x = [&](u32x4 (&xa)[G][4], int c) __attribute__((always_inline)) {
    const int cc = min(c0 + c, C - 1);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint16_t* xp = xbase + (size_t)min(4 * g + (n >> 2), p.B - 1) * p.K + (size_t)cc * 128;
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[g][i] = ld_vec(xp + 8 * i);
    }
  };
  float acc[G][NR];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int s = 0; s < NR; ++s) acc[g][s] = 0.f;
  u32x4 xc[G][4], xn[G][4];
  load_x(xc, 0);
  // keep every load above issued here: left alone, the scheduler sinks each
  // chunk's weight loads to just before their use
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (c + 1 < NCH) load_x(xn, c + 1);
    __builtin_amdgcn_sched_barrier(0);   // the next chunk's fragments in flight during this one
#pragma unroll
    for (int s = 0; s < NR; ++s) {
      w4m_f32x4 d[G];
#pragma unroll
      for (int g = 0; g < G; ++g) d[g] = w4m_f32x4{0.f, 0.f, 0.f, 0.f};
      const uint32_t wd[4] = {wq[c][s].x, wq[c][s].y, wq[c][s].z, wq[c][s].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 w = w4b_unpack(wd[i]);
#pragma unroll
        for (int g = 0; g < G; ++g)
          d[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(w4m_bf16x8, xc[g][i]),
                                                         __builtin_bit_cast(w4m_bf16x8, w), d[g], 0, 0, 0);
      }
      // chunks past the row (clamped loads) count with scale 0
      const float scale = c < cnt ? bf16_bits_to_f32(sc[c][s]) : 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g][s] = fmaf(scale, (d[g][0] + d[g][1]) + d[g][2], acc[g][s]);
    }
    if (c + 1 < NCH) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) xc[g][i] = xn[g][i];
    }
  }
  // lane group q of group g holds activation row 4 g + q's sums; the waves
  // meet in LDS
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int s = 0; s < NR; ++s) part[wave][4 * g + q][s][n] = acc[g][s];
  __syncthreads();
  if (threadIdx.x >= 64 * G) return;
  const int b = threadIdx.x >> 4, row = r0 + (threadIdx.x & 15);
  if (b >= p.B || row >= p.n_out) return;
  float inv = 1.f;
  if (NORM && p.gain) {
    float tot = 0.f;
    for (int w = 0; w < NWV; ++w) tot += ssw[w][b];
    inv = 1.0f / sqrtf(tot / (float)p.K + p.eps);
  }
  float v[NR];
#pragma unroll
  for (int s = 0; s < NR; ++s) {
    v[s] = 0.f;
    for (int w = 0; w < NWV; ++w) v[s] += part[w][b][s][threadIdx.x & 15];
    v[s] *= inv;
  }
  float out;
  if (p.mode == GEMV_SWIGLU) out = silu_f(v[0]) * v[NR - 1];
  else if (p.mode == GEMV_ADD) out = p.res[(size_t)b * p.ldres + row] + v[0];
  else out = v[0];
  if (p.yplanes) store_planes((uint16_t*)p.yplanes, (size_t)p.B * p.n_out, (size_t)b * p.n_out + row, out);
  else p.y[(size_t)b * p.ldy + row] = out;
}

template <int NR, int NCH, int NWV>
static hipError_t go_w4b(const GemvParams& p, bool norm, hipStream_t s) {
  const dim3 grid((p.n_out + 15) / 16), block(NWV * 64);
  if (norm)
    launch_timed(gemv_w4b_kernel<NR, NCH, NWV, true, 1>, grid, block, (uint32_t)(6 * p.B * p.K), s, p);
  else if (p.B <= 4)
    launch_timed(gemv_w4b_kernel<NR, NCH, NWV, false, 1>, grid, block, 0u, s, p);
  else
    launch_timed(gemv_w4b_kernel<NR, NCH, NWV, false, 2>, grid, block, 0u, s, p);
  return hipGetLastError();
}

// Threads per workgroup of the 4-bit batched form for a row of K inputs.
static int w4b_threads(int K) { return K / 128 <= 24 ? 512 : 1024; }

// Whether the 4-bit batched form splits (and normalises) its fp32 input
// itself: the terms of the B rows must fit in LDS (64 KB) and the input in
// W4B_XU float4 units per thread.
bool gemv_w4_rows_normalises(const GemvParams& p) {
  return !p.xplanes && p.B <= 4 && 6 * p.B * p.K <= 65536 && p.B * p.K <= 4 * W4B_XU * w4b_threads(p.K) &&
         p.K % 4 == 0;
}

// 2 to GEMV_W4_MAX_ROWS activation rows with 4-bit weights: the input planes at p.xn, or
// (gemv_w4_rows_normalises) the fp32 input at p.x (K a multiple of 128, at
// most 10,240).
bool launch_gemv_w4_rows(const GemvParams& p, hipStream_t s, hipError_t* e) {
  if (p.B < 2 || p.B > GEMV_W4_MAX_ROWS || p.K % 128 || p.K > 10240 || !p.q4[0]) return false;
  const bool norm = gemv_w4_rows_normalises(p);
  const int C = p.K / 128;
  if (p.mode == GEMV_SWIGLU) {
    if (C <= 24) *e = go_w4b<2, 3, 8>(p, norm, s);
    else if (C <= 48) *e = go_w4b<2, 3, 16>(p, norm, s);
    else *e = go_w4b<2, 5, 16>(p, norm, s);
  } else {
    if (C <= 24) *e = go_w4b<1, 3, 8>(p, norm, s);
    else if (C <= 32) *e = go_w4b<1, 2, 16>(p, norm, s);
    else if (C <= 48) *e = go_w4b<1, 3, 16>(p, norm, s);
    else *e = go_w4b<1, 5, 16>(p, norm, s);
  }
  return true;
}

// Two rows per wave for every 4-bit product (4 rows per wave measured slower
// for each of them: 3.24-3.44 ms per frame against 3.17).
template <int NR, int NUP, int KS>
static hipError_t go_w4(const GemvParams& p, hipStream_t s) {
  constexpr int RPW = 2;
  constexpr int rows = (4 / KS) * RPW;
  const dim3 grid((p.n_out + rows - 1) / rows);
  if (NUP * KS == p.K / 512)
    launch_timed(gemv_w4_kernel<RPW, NR, NUP, KS, false>, grid, dim3(DUALAR_WG), 0, s, p);
  else
    launch_timed(gemv_w4_kernel<RPW, NR, NUP, KS, true>, grid, dim3(DUALAR_WG), 0, s, p);
  return hipGetLastError();
}

// Units per wave at most 5: one wave per row group up to 2,560 inputs, two
// up to 5,120, four up to 10,240.
template <int NR>
static hipError_t launch_w4(const GemvParams& p, hipStream_t s) {
  if (p.B != 1 || p.K % 512 || p.K > 10240 || p.xplanes || p.yplanes) return hipErrorInvalidValue;
  const int U = p.K / 512;
  switch (U) {
    case 1: return go_w4<NR, 1, 1>(p, s);
    case 2: return go_w4<NR, 2, 1>(p, s);
    case 3: return go_w4<NR, 3, 1>(p, s);
    case 4: return go_w4<NR, 4, 1>(p, s);
    case 5: return go_w4<NR, 5, 1>(p, s);
    case 6: return go_w4<NR, 3, 2>(p, s);
    case 7: case 8: return go_w4<NR, 4, 2>(p, s);
    case 9: case 10: return go_w4<NR, 5, 2>(p, s);
    case 11: case 12: return go_w4<NR, 3, 4>(p, s);
    case 13: case 14: case 15: case 16: return go_w4<NR, 4, 4>(p, s);
    default: return go_w4<NR, 5, 4>(p, s);   // 17 .. 20 units
  }
}

// ---------------------------------------------------------------------------
// launch selection
// ---------------------------------------------------------------------------
// NU > 0 and BT == 1: register-staged kernel (one activation row, the
// caller guarantees B == 1); NU > 0 and BT > 1: LDS-staged unrolled kernel;
// NU == 0: loop kernel for any row length.
template <typename T, int BT, int RPW, int NR, int NU>
static hipError_t go(const GemvParams& p, hipStream_t s) {
  dim3 grid((p.n_out + 4 * RPW - 1) / (4 * RPW), (p.B + BT - 1) / BT);
  const size_t lds = (size_t)BT * p.K * sizeof(float);
  if constexpr (NU > 0 && BT == 1)
    launch_timed(gemv_rx_kernel<T, RPW, NR, NU>, grid, dim3(DUALAR_WG), 0, s, p);
  else if constexpr (NU > 0)
    launch_timed(gemv_unrolled_kernel<T, BT, RPW, NR, NU>, grid, dim3(DUALAR_WG), (uint32_t)lds, s, p);
  else
    launch_timed(gemv_loop_kernel<T, BT, RPW, NR>, grid, dim3(DUALAR_WG), (uint32_t)lds, s, p);
  return hipGetLastError();
}

template <typename T, int RPW, int NR, int NU, int KS>
static hipError_t go_ks(const GemvParams& p, hipStream_t s) {
  dim3 grid((p.n_out + (4 / KS) * RPW - 1) / ((4 / KS) * RPW));
  launch_timed(gemv_ks_kernel<T, RPW, NR, NU, KS>, grid, dim3(DUALAR_WG), 0, s, p);
  return hipGetLastError();
}

template <int NW, int R, int NR, int U>
static hipError_t go_wide(const GemvParams& p, hipStream_t s) {
  launch_timed(gemv_wide_kernel<NW, R, NR, U>, dim3((p.n_out + R - 1) / R), dim3(NW * 64), 0, s, p);
  return hipGetLastError();
}

// One activation row of bf16 rows of 2560 / 4096 / 9728: the variants that
// measured fastest for each S2 matrix (rows per wave, k-split; or the wide
// form with about one workgroup per compute unit for the S2 row counts).
template <typename T, int NR>
static bool pick_b1(const GemvParams& p, hipStream_t s, hipError_t* e) {
  if constexpr (sizeof(T) == 2) {
    // The wide form for the long rows of O and W2 (5.8 / 10.0 us against 6.6
    // / 10.9 us for the k-split kernel); 8 waves x 10 rows for O, 10 waves x
    // 10 rows for W2 (8 x 10, 8 x 8 and 12 x 12 were slower).  With 5 units
    // per row it has too few waves per SIMD and the 4-wave kernels stay
    // faster (QKV, W1|W3, fast head).
    if constexpr (NR == 1) {
      const int wunits = p.K / 512;
      if (wunits == 8 && p.n_out == 2560) { *e = go_wide<8, 10, 1, 8>(p, s); return true; }     // O
      if (wunits == 19 && p.n_out == 2560) { *e = go_wide<10, 10, 1, 19>(p, s); return true; }  // W2
    }
    const int units = p.K / (64 * ElemT<T>::EPV);
    if (units == 5) {
      // rows per wave: 3 for QKV (512 workgroups; 7.6 us against 7.8), 2 for
      // W1|W3 (1 / 3 / 4 rows took 18.7 / 19.9 / 19.7 us against 18.0)
      if (NR == 1 && p.n_out >= 65536) *e = go<T, 1, 4, NR, 5>(p, s);  // tied head
      else if (NR == 2) *e = go<T, 1, 2, NR, 5>(p, s);                 // W1|W3
      else if (p.n_out == 6144) *e = go<T, 1, 3, NR, 5>(p, s);         // QKV
      else *e = go<T, 1, 2, NR, 5>(p, s);                              // fast head, K|V rows
      return true;
    }
    if constexpr (NR == 1) {
      if (units == 8) { *e = go_ks<T, 2, 1, 8, 4>(p, s); return true; }   // O
      if (units == 19) { *e = go_ks<T, 2, 1, 19, 4>(p, s); return true; } // W2
    }
  }
  return false;
}

// Several activation rows (BT per workgroup, activations staged in LDS):
// unrolled rows for the S2 row lengths 2560 / 4096, a loop otherwise.
template <typename T, int BT, int NR>
static hipError_t pick_multi(const GemvParams& p, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    const int units = p.K / (64 * ElemT<T>::EPV);
    if (units == 5) return go<T, BT, 2, NR, 5>(p, s);
    if (units == 8 && NR == 1) return go<T, BT, 1, NR, 8>(p, s);
  }
  return go<T, BT, 1, NR, 0>(p, s);
}

template <typename T, int NR>
static hipError_t pick_bt(const GemvParams& p, hipStream_t s) {
  if (p.B == 1) {
    hipError_t e;
    if (pick_b1<T, NR>(p, s, &e)) return e;
    return go<T, 1, 1, NR, 0>(p, s);
  }
  const size_t lim = 48 * 1024;   // dynamic LDS for the staged activations
  if (p.B >= 3 && 4 * (size_t)p.K * 4 <= lim) return pick_multi<T, 4, NR>(p, s);
  if (2 * (size_t)p.K * 4 <= lim) return pick_multi<T, 2, NR>(p, s);
  return go<T, 1, 1, NR, 0>(p, s);
}

template <typename T> hipError_t launch_gemv(const GemvParams& p, hipStream_t s) {
  if (p.q4[0]) {
    if constexpr (sizeof(T) != 2) return hipErrorInvalidValue;
    if (p.B >= 2) {   // 2 to GEMV_W4_MAX_ROWS rows, or prefill steps of GEMM_TILE_MIN_ROWS+ rows (the 2-D tiles)
      hipError_t e;
      return launch_gemm_mfma(p, s, &e) ? e : hipErrorInvalidValue;
    }
    if (p.next_done) *p.next_done = 0;
    hipError_t e;
    if (p.mode != GEMV_SWIGLU && launch_w4m<1>(p, s, &e)) return e;
    return p.mode == GEMV_SWIGLU ? launch_w4<2>(p, s) : launch_w4<1>(p, s);
  }
  if constexpr (sizeof(T) == 2) {
    hipError_t e;
    if (launch_gemm_mfma(p, s, &e)) return e;   // 2+ activation rows on the matrix cores
  }
  if (p.xplanes || p.yplanes) return hipErrorInvalidValue;   // planes exist on the matrix-core path only
  if (p.next_done) *p.next_done = 0;
  if (p.mode == GEMV_SWIGLU) return pick_bt<T, 2>(p, s);
  return pick_bt<T, 1>(p, s);
}

template hipError_t launch_gemv<float>(const GemvParams&, hipStream_t);
template hipError_t launch_gemv<bf16_t>(const GemvParams&, hipStream_t);
