// Matrix products over many activation rows (the prefill steps: every
// sequence's chunk of prompt positions at once) on the gfx950 matrix cores:
// Y[b][n] = sum_k W[n][k] X[b][k], with the activations as three bf16 terms
// (planes, x = t0 + t1 + t2 up to 2^-24 |x|) and bf16 weights, accumulated in
// fp32 -- the same product as the decode-shaped kernels, which stream each
// weight row once per 32 activation rows.  At hundreds of rows that re-reads
// the weights many times over; here a workgroup owns a 2-D output tile of
// NROWS weight rows x BROWS activation rows, so each loaded operand byte
// feeds BROWS (weights) or NROWS (activations) multiply-adds per term.
//
// v_mfma_f32_32x32x16_bf16 with the activation term as the A operand (lane l
// holds X_t[b0 + l%32][k + 8*(l/32) .. +8]) and the weights as the B operand
// (lane l holds W[n0 + l%32][k + 8*(l/32) .. +8]): D[b][n] in register r of
// lane l is row b = (r/4)*8 + (l/32)*4 + r%4, column n = l%32, so the 32
// lanes of a half-wave store 32 consecutive outputs of one row.  The three
// terms go into one accumulator (terms of one k-step in order t0, t1, t2).
//
// GN x GW waves as GN (weight rows) x GW (activation rows); a wave owns 32*WN
// weight rows x 32*WB activation rows.  K is walked in chunks of 32 (64
// bytes per row); each chunk of weights (NROWS x 64 B) and activation planes
// (3 x BROWS x 64 B) is copied by LDS DMA, 16 rows per instruction, piece p
// of row r stored at slot p ^ ((r >> 2) & 3) so that the operand reads of 16
// consecutive rows hit distinct banks.  Three stages: two chunks in flight
// while one is multiplied; one barrier per chunk.
//
// SwiGLU tiles hold NROWS/2 output columns: wave row h (weight rows
// [h*32*WN, (h+1)*32*WN)) holds gate rows then up rows of 16*WN columns, so
// silu(gate) * up is formed in registers.
//
// Tiles are numbered in groups of TL_GB activation tiles (all weight tiles
// of a group, then the next group) and dealt to the 8 XCDs in contiguous
// ranges (workgroup id % 8 is its XCD): the ~32 workgroups an XCD runs at
// once then cover about 4 weight tiles x 8 activation tiles and share both
// operands through that XCD's L2.
#include "mfma.h"

#define TL_KC 32
#define TL_GB 8

template <int WN, int WB, int GN, int GW, int STG = 3> struct Tl {
  static constexpr int WAVES = GN * GW;   // GN wave rows (weights) x GW wave columns (activations)
  static constexpr int NROWS = 32 * WN * GN;   // weight rows per tile
  static constexpr int BROWS = 32 * WB * GW;   // activation rows per tile
  static constexpr int W_BYTES = NROWS * TL_KC * 2;
  static constexpr int X_BYTES = 3 * BROWS * TL_KC * 2;
  static constexpr int STAGE = W_BYTES + X_BYTES;
  static constexpr int W_INSTR = W_BYTES / 1024 / WAVES;   // DMA instructions per wave per chunk
  static constexpr int X_INSTR = X_BYTES / 1024 / WAVES;
  static constexpr int DMA = W_INSTR + X_INSTR;
  static_assert(W_BYTES % (1024 * WAVES) == 0 && X_BYTES % (1024 * WAVES) == 0, "DMA split");
  static_assert(WN % 2 == 0, "SwiGLU pairs gate and up blocks");
  static_assert(BROWS == GEMM_TILE_BROWS, "the prefill live-tile mask counts tiles of GEMM_TILE_BROWS rows");
};

template <int WN, int WB, int GN, int GW> struct TlSrc {
  const char* w[Tl<WN, WB, GN, GW>::W_INSTR];
  const char* x[Tl<WN, WB, GN, GW>::X_INSTR];
};

template <int WN, int WB, int GN, int GW>
__device__ __forceinline__ void tl_issue(const TlSrc<WN, WB, GN, GW>& src, char* stage, int c, int wave) {
  using L = Tl<WN, WB, GN, GW>;
#pragma unroll
  for (int j = 0; j < L::W_INSTR; ++j) dma16(src.w[j] + (size_t)c * TL_KC * 2, stage + (wave * L::W_INSTR + j) * 1024);
  char* xs = stage + L::W_BYTES;
#pragma unroll
  for (int j = 0; j < L::X_INSTR; ++j) dma16(src.x[j] + (size_t)c * TL_KC * 2, xs + (wave * L::X_INSTR + j) * 1024);
}

// The two 16-wide k-steps of one chunk: the wave's WB x 3 activation
// fragments and WN weight fragments, then 3*WN*WB products ordered so that
// consecutive ones use different accumulators.
template <int WN, int WB, int GN, int GW>
__device__ __forceinline__ void tl_compute(const char* stage, int wn, int wb, int lane, f32x16 (*acc)[WB]) {
  using L = Tl<WN, WB, GN, GW>;
  const char* xs = stage + L::W_BYTES;
  const int h = lane >> 5, l32 = lane & 31, sw = (l32 >> 2) & 3;
#pragma unroll
  for (int t = 0; t < TL_KC / 16; ++t) {
    const int slot = ((2 * t + h) ^ sw) << 4;
    bf16x8 xf[WB][3], wf[WN];
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int q = 0; q < 3; ++q)
        xf[j][q] = *(const bf16x8*)(xs + q * (L::BROWS * 64) + (32 * (wb * WB + j) + l32) * 64 + slot);
#pragma unroll
    for (int i = 0; i < WN; ++i) wf[i] = *(const bf16x8*)(stage + (32 * (wn * WN + i) + l32) * 64 + slot);
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int i = 0; i < WN; ++i)
#pragma unroll
        for (int j = 0; j < WB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[j][q], wf[i], acc[i][j], 0, 0, 0);
  }
}

// Index of the n-th set bit (from 0) of the two-word mask, n < its population.
__device__ __forceinline__ int nth_live_tile(const uint64_t (&m)[2], int n) {
  const int c0 = __popcll(m[0]);
  const int word = n < c0 ? 0 : 1;
  uint64_t w = word ? m[1] : m[0];
  if (word) n -= c0;
  for (int i = 0; i < n; ++i) w &= w - 1;   // clear the n lowest set bits
  return 64 * word + __ffsll((long long)w) - 1;
}

// Epilogue straight from the accumulators: lanes 0..31 hold 32 consecutive
// columns of row b, lanes 32..63 the same columns of row b + 4.
template <int WN, int WB>
__device__ __forceinline__ void tl_epilogue(const GemvParams& p, f32x16 (*acc)[WB], bool glu, int n0, int b0, int wn,
                                            int wb, int lane) {
  const int l32 = lane & 31, h = lane >> 5;
  const size_t plane_out = (size_t)p.B * p.n_out;
  auto put = [&](int b, int n, float out) {
    if (p.yplanes) store_planes((uint16_t*)p.yplanes, plane_out, (size_t)b * p.n_out + n, out);
    else p.y[(size_t)b * p.ldy + n] = out;
  };
  if (glu) {
#pragma unroll
    for (int i = 0; i < WN / 2; ++i) {
      const int n = n0 + wn * 16 * WN + 32 * i + l32;
      if (n >= p.n_out) continue;
#pragma unroll
      for (int j = 0; j < WB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int b = b0 + 32 * (wb * WB + j) + (r >> 2) * 8 + h * 4 + (r & 3);
          if (b < p.B) put(b, n, silu_f(acc[i][j][r]) * acc[i + WN / 2][j][r]);
        }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < WN; ++i) {
    const int n = n0 + 32 * (wn * WN + i) + l32;
    if (n >= p.n_out) continue;
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int b = b0 + 32 * (wb * WB + j) + (r >> 2) * 8 + h * 4 + (r & 3);
        if (b >= p.B) continue;
        const float v = acc[i][j][r];
        put(b, n, p.mode == GEMV_ADD ? p.res[(size_t)b * p.ldres + n] + v : v);
      }
  }
}

// Tile coordinates of workgroup blockIdx.x: tiles are numbered in groups of
// TL_GB activation tiles and dealt to the XCDs in contiguous ranges.
// Returns false for the workgroups past the last tile.
__device__ __forceinline__ bool tl_place(const GemvParams& p, int nrows, int brows, int& n0, int& b0) {
  const int cols = p.mode == GEMV_SWIGLU ? nrows / 2 : nrows;   // output columns per tile
  // activation tiles: all of them, or the live ones of a prefill step
  const int tb = p.bt_masked ? __popcll(p.live_bt[0]) + __popcll(p.live_bt[1]) : (p.B + brows - 1) / brows;
  const int tn = (p.n_out + cols - 1) / cols;
  const int tiles = tn * tb, per = (tiles + 7) / 8;
  const int li = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (li >= tiles) return false;
  const int grp = li / (TL_GB * tn), fb = grp * TL_GB, gs = min(TL_GB, tb - fb), rem = li - grp * TL_GB * tn;
  int bt = fb + rem % gs;
  if (p.bt_masked) bt = nth_live_tile(p.live_bt, bt);
  n0 = (rem / gs) * cols;
  b0 = bt * brows;
  return true;
}

// Weight row of tile row r (the LDS row): for SwiGLU, wave row h's block of
// 32*WN rows holds 16*WN gate rows, then the up rows of the same columns.
template <int WN>
__device__ __forceinline__ int tl_row(bool glu, int n0, int r, int& seg) {
  seg = 0;
  if (!glu) return n0 + r;
  const int within = r % (32 * WN);
  seg = within / (16 * WN);
  return n0 + (r / (32 * WN)) * 16 * WN + within % (16 * WN);
}

// One-dimensional grid of 8 * ceil(tiles / 8) workgroups of 256 threads.
// The host guarantees K % 32 == 0, B >= 1 and n_out >= 1.
template <int WN, int WB, int GN, int GW, int STG = 3>
__global__ void __launch_bounds__(64 * GN * GW, 1) mfma_tile_kernel(GemvParams p) {
  using L = Tl<WN, WB, GN, GW>;
  static_assert(STG == 2 || STG == 3, "stages");
  __shared__ __attribute__((aligned(1024))) char smem[STG * L::STAGE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave / GW, wb = wave % GW;
  const bool glu = p.mode == GEMV_SWIGLU;
  int n0, b0;
  if (!tl_place(p, L::NROWS, L::BROWS, n0, b0)) return;

  // DMA sources of chunk 0: instruction i covers LDS rows 16 i .. 16 i + 15,
  // lane -> row 16 i + lane/4, slot lane%4 (piece slot ^ ((row >> 2) & 3))
  TlSrc<WN, WB, GN, GW> src;
  {
    const RowSpace rs(p);
#pragma unroll
    for (int j = 0; j < L::W_INSTR; ++j) {
      const int r = 16 * (wave * L::W_INSTR + j) + (lane >> 2);
      const int piece = (lane & 3) ^ ((r >> 2) & 3);
      int seg;
      const int n = tl_row<WN>(glu, n0, r, seg);
      src.w[j] = rs.row(min(n, p.n_out - 1), seg) + piece * 16;
    }
    const uint16_t* xs = (const uint16_t*)p.xn;
    const size_t plane = (size_t)p.B * p.K;
#pragma unroll
    for (int j = 0; j < L::X_INSTR; ++j) {
      const int i = wave * L::X_INSTR + j;
      const int q = i / (L::BROWS / 16), rr = 16 * (i % (L::BROWS / 16)) + (lane >> 2);
      const int piece = (lane & 3) ^ ((rr >> 2) & 3);
      const int b = min(b0 + rr, p.B - 1);   // rows past B: loaded, never stored
      src.x[j] = (const char*)(xs + q * plane + (size_t)b * p.K) + piece * 16;
    }
  }

  f32x16 acc[WN][WB];
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Chunk c is multiplied from stage c % 3 while chunks c+1 and c+2 are in
  // flight.  Before chunk c+2 overwrites stage (c+2) % 3, every wave's copies
  // of chunk c have landed (at most the next chunk's DMA outstanding) and
  // every wave is done with chunk c-1 (barrier).  The steady loop has no
  // branches; the last two chunks follow it.
  const int nch = p.K / TL_KC;
  if constexpr (STG == 3) {
    tl_issue<WN, WB, GN, GW>(src, smem, 0, wave);
    if (nch > 1) tl_issue<WN, WB, GN, GW>(src, smem + L::STAGE, 1, wave);
    int cs = 0;   // stage of chunk c
    for (int c = 0; c + 2 < nch; ++c) {
      wait_vm_barrier<L::DMA>();
      const int ns = cs == 0 ? 2 : cs - 1;   // (c + 2) % 3
      tl_issue<WN, WB, GN, GW>(src, smem + ns * L::STAGE, c + 2, wave);
      tl_compute<WN, WB, GN, GW>(smem + cs * L::STAGE, wn, wb, lane, acc);
      cs = cs == 2 ? 0 : cs + 1;
    }
    if (nch > 1) {
      wait_vm_barrier<L::DMA>();
      tl_compute<WN, WB, GN, GW>(smem + cs * L::STAGE, wn, wb, lane, acc);
      cs = cs == 2 ? 0 : cs + 1;
    }
    wait_vm_barrier<0>();
    tl_compute<WN, WB, GN, GW>(smem + cs * L::STAGE, wn, wb, lane, acc);
  } else {
    // two stages: chunk c+1 is in flight while chunk c is multiplied
    tl_issue<WN, WB, GN, GW>(src, smem, 0, wave);
    int cs = 0;
    for (int c = 0; c + 1 < nch; ++c) {
      wait_vm_barrier<0>();
      tl_issue<WN, WB, GN, GW>(src, smem + (cs ^ 1) * L::STAGE, c + 1, wave);
      tl_compute<WN, WB, GN, GW>(smem + cs * L::STAGE, wn, wb, lane, acc);
      cs ^= 1;
    }
    wait_vm_barrier<0>();
    tl_compute<WN, WB, GN, GW>(smem + cs * L::STAGE, wn, wb, lane, acc);
  }

  tl_epilogue<WN, WB>(p, acc, glu, n0, b0, wn, wb, lane);
}

// ---------------------------------------------------------------------------
// 4-bit weights (W4A16) on the same 2-D tiles
// ---------------------------------------------------------------------------
// The 256 x 128 tile of eight 64 x 64 waves with the weights as packed 4-bit
// rows ([rows][K/2] bytes, input 2j in the low nibble of byte j, two's
// complement) and one bf16 scale per row and group of 128 inputs:
//   Y[b][n] = sum_g s[n][g] * sum_{k in g} q[n][k] X[b][k].
// q is an integer in [-8, 7], exact in bf16, so each group's inner sum runs
// on the matrix cores exactly as in the bf16 tile (three activation terms)
// into a group accumulator, which is then scaled into the output
// accumulator in fp32.
//
// K is walked in chunks of 64 inputs (32 bytes of a 4-bit row, 128 bytes of
// an activation term row), two stages, so a scale group is two chunks.  All
// of the tile's scales are copied into LDS before the loop ([group][tile
// row], K <= 10,240).  Within a chunk the matrix-core k-slots take the inputs
// in a permuted order that both operands share: lane half h, k-step t covers
// inputs 32 h + 8 t .. + 8, so a lane reads its 16 weight bytes of the chunk
// once (4 k-steps x 8 nibbles) and converts 8 nibbles per k-step.
// LDS layout per stage: weights [256 rows][32 B] with 16-byte piece p of row
// r at slot p ^ ((r >> 2) & 1); activation terms [3][128 rows][128 B] with
// piece p of row r at slot p ^ (r & 7): eight consecutive rows' reads of one
// piece then hit distinct bank groups.
#define T4_KC 64
#define T4_GMAX 80

struct T4 {
  static constexpr int WN = 2, WB = 2, GN = 4, GW = 2, WAVES = GN * GW;
  static constexpr int NROWS = 32 * WN * GN;           // 256 weight rows
  static constexpr int BROWS = 32 * WB * GW;           // 128 activation rows
  static constexpr int W_BYTES = NROWS * T4_KC / 2;    // 8 KB of nibbles
  static constexpr int X_BYTES = 3 * BROWS * T4_KC * 2;
  static constexpr int STAGE = W_BYTES + X_BYTES;
  static constexpr int W_INSTR = W_BYTES / 1024 / WAVES;
  static constexpr int X_INSTR = X_BYTES / 1024 / WAVES;
  static_assert(W_BYTES == 1024 * WAVES && X_BYTES % (1024 * WAVES) == 0, "DMA split");
  static_assert(BROWS == GEMM_TILE_BROWS, "the prefill live-tile mask counts tiles of GEMM_TILE_BROWS rows");
  static_assert(2 * STAGE + T4_GMAX * NROWS * 2 <= 160 * 1024, "LDS");
};

// Packed 4-bit row n of the product (segments as in RowSpace) and its
// scales.  The segment pointers are pinned in SGPRs and chosen by selects
// (a per-lane index into the kernel arguments becomes a memory load).
__device__ __forceinline__ const char* t4_row(const GemvParams& p, int n, int seg, const uint16_t** sc) {
  if (p.mode != GEMV_SWIGLU && n >= p.rows[0]) {
    n -= p.rows[0];
    seg = 1;
    if (n >= p.rows[1]) { n -= p.rows[1]; seg = 2; }
  }
  uint64_t q0 = (uint64_t)p.q4[0], q1 = (uint64_t)p.q4[1], q2 = (uint64_t)p.q4[2];
  uint64_t s0 = (uint64_t)p.s4[0], s1 = (uint64_t)p.s4[1], s2 = (uint64_t)p.s4[2];
  asm volatile("" : "+s"(q0), "+s"(q1), "+s"(q2), "+s"(s0), "+s"(s1), "+s"(s2));
  const uint64_t q = seg == 0 ? q0 : (seg == 1 ? q1 : q2);
  const uint64_t s = seg == 0 ? s0 : (seg == 1 ? s1 : s2);
  *sc = (const uint16_t*)s + (size_t)n * (p.K / 128);
  return (const char*)q + (size_t)n * (p.K / 2);
}

// Eight 4-bit values (dword d, value j in bits 4j..4j+3) as bf16, in order.
// v ^ 8 is v + 8 in [0, 15] for a two's-complement nibble v.
__device__ __forceinline__ bf16x8 t4_unpack(uint32_t d) {
  const uint32_t u = d ^ 0x88888888u;
  uint32_t lo = u & 0x0F0F0F0Fu, hi = (u >> 4) & 0x0F0F0F0Fu;
  // hide the known-zero bits: each byte then converts in one v_cvt_f32_ubyte
  __asm__("" : "+v"(lo), "+v"(hi));
  bf16x8 o;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    o[2 * b] = (__bf16)((float)((lo >> (8 * b)) & 0xFFu) - 8.0f);
    o[2 * b + 1] = (__bf16)((float)((hi >> (8 * b)) & 0xFFu) - 8.0f);
  }
  return o;
}

struct T4Src {
  const char* w;
  const char* x[T4::X_INSTR];
};

__device__ __forceinline__ void t4_issue(const T4Src& src, char* stage, int c, int wave) {
  dma16(src.w + (size_t)c * (T4_KC / 2), stage + wave * 1024);
  char* xs = stage + T4::W_BYTES;
#pragma unroll
  for (int j = 0; j < T4::X_INSTR; ++j) dma16(src.x[j] + (size_t)c * T4_KC * 2, xs + (wave * T4::X_INSTR + j) * 1024);
}

// The four k-steps of one chunk into the group accumulators.
__device__ __forceinline__ void t4_compute(const char* stage, int wn, int wb, int lane, f32x16 (*acc)[T4::WB]) {
  constexpr int WN = T4::WN, WB = T4::WB;
  const char* xs = stage + T4::W_BYTES;
  const int h = lane >> 5, l32 = lane & 31;
  u32x4 wr[WN];
#pragma unroll
  for (int i = 0; i < WN; ++i)
    wr[i] = *(const u32x4*)(stage + (32 * (wn * WN + i) + l32) * 32 + ((h ^ ((l32 >> 2) & 1)) << 4));
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int slot = ((4 * h + t) ^ (l32 & 7)) << 4;
    bf16x8 xf[WB][3], wf[WN];
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int q = 0; q < 3; ++q)
        xf[j][q] = *(const bf16x8*)(xs + (q * T4::BROWS + 32 * (wb * WB + j) + l32) * 128 + slot);
#pragma unroll
    for (int i = 0; i < WN; ++i) wf[i] = t4_unpack(wr[i][t]);
#pragma unroll
    for (int q = 0; q < 3; ++q)
#pragma unroll
      for (int i = 0; i < WN; ++i)
#pragma unroll
        for (int j = 0; j < WB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf[j][q], wf[i], acc[i][j], 0, 0, 0);
  }
}

// One-dimensional grid of 8 * ceil(tiles / 8) workgroups of 512 threads.
// The host guarantees K % 128 == 0, K <= 128 * T4_GMAX, B >= 1, n_out >= 1.
__global__ void __launch_bounds__(64 * T4::WAVES, 1) mfma_tile_w4_kernel(GemvParams p) {
  constexpr int WN = T4::WN, WB = T4::WB;
  __shared__ __attribute__((aligned(1024))) char smem[2 * T4::STAGE];
  __shared__ uint16_t ssc[T4_GMAX * T4::NROWS];   // [group][tile row]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wn = wave / T4::GW, wb = wave % T4::GW;
  const bool glu = p.mode == GEMV_SWIGLU;
  int n0, b0;
  if (!tl_place(p, T4::NROWS, T4::BROWS, n0, b0)) return;
  const int G = p.K / 128;

  // the tile's scales, before any copy is in flight
  for (int i = threadIdx.x; i < G * T4::NROWS; i += 64 * T4::WAVES) {
    const int r = i / G, g = i - r * G;
    int seg;
    const int n = tl_row<WN>(glu, n0, r, seg);
    const uint16_t* sc;
    (void)t4_row(p, min(n, p.n_out - 1), seg, &sc);
    ssc[g * T4::NROWS + r] = sc[g];
  }

  // DMA sources of chunk 0.  Weights: wave w's instruction covers tile rows
  // 32 w .. 32 w + 31, lane -> row 32 w + lane/2, slot lane%2.  Activations:
  // instruction i covers 8 rows of one term, lane -> row 8 (i % 16) + lane/8,
  // slot lane%8.
  T4Src src;
  {
    const int r = 32 * wave + (lane >> 1);
    const int piece = (lane & 1) ^ ((r >> 2) & 1);
    int seg;
    const int n = tl_row<WN>(glu, n0, r, seg);
    const uint16_t* sc;
    src.w = t4_row(p, min(n, p.n_out - 1), seg, &sc) + piece * 16;
    const uint16_t* xs = (const uint16_t*)p.xn;
    const size_t plane = (size_t)p.B * p.K;
#pragma unroll
    for (int j = 0; j < T4::X_INSTR; ++j) {
      const int i = wave * T4::X_INSTR + j;
      const int q = i / (T4::BROWS / 8), rr = 8 * (i % (T4::BROWS / 8)) + (lane >> 3);
      const int pc = (lane & 7) ^ (rr & 7);
      const int b = min(b0 + rr, p.B - 1);   // rows past B: loaded, never stored
      src.x[j] = (const char*)(xs + q * plane + (size_t)b * p.K) + pc * 16;
    }
  }
  __syncthreads();   // scales visible to every wave

  f32x16 acc[WN][WB], gacc[WN][WB];
#pragma unroll
  for (int i = 0; i < WN; ++i)
#pragma unroll
    for (int j = 0; j < WB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Group g = chunks 2g (stage 0) and 2g + 1 (stage 1).  Before a chunk is
  // copied into a stage, every wave's copies of the previous chunk have
  // landed and every wave is done with the chunk that stage held (barrier).
  t4_issue(src, smem, 0, wave);
  const int l32 = lane & 31;
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int i = 0; i < WN; ++i)
#pragma unroll
      for (int j = 0; j < WB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) gacc[i][j][r] = 0.f;
    wait_vm_barrier<0>();
    t4_issue(src, smem + T4::STAGE, 2 * g + 1, wave);
    t4_compute(smem, wn, wb, lane, gacc);
    wait_vm_barrier<0>();
    if (g + 1 < G) t4_issue(src, smem, 2 * g + 2, wave);
    t4_compute(smem + T4::STAGE, wn, wb, lane, gacc);
#pragma unroll
    for (int i = 0; i < WN; ++i) {
      const float s = bf16_bits_to_f32(ssc[g * T4::NROWS + 32 * (wn * WN + i) + l32]);
#pragma unroll
      for (int j = 0; j < WB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(s, gacc[i][j][r], acc[i][j][r]);
    }
  }
  tl_epilogue<WN, WB>(p, acc, glu, n0, b0, wn, wb, lane);
}

bool launch_gemm_tile_w4(const GemvParams& p, hipStream_t s) {
  if (p.K % 128 != 0 || p.K > 128 * T4_GMAX || p.B < 1 || p.n_out < 1 || !p.q4[0]) return false;
  const int tb = p.bt_masked ? __builtin_popcountll(p.live_bt[0]) + __builtin_popcountll(p.live_bt[1])
                            : (p.B + GEMM_TILE_BROWS - 1) / GEMM_TILE_BROWS;
  if (tb == 0) return true;
  const int cols = p.mode == GEMV_SWIGLU ? T4::NROWS / 2 : T4::NROWS;
  const int tiles = ((p.n_out + cols - 1) / cols) * tb;
  hipLaunchKernelGGL(mfma_tile_w4_kernel, dim3(8 * ((tiles + 7) / 8)), dim3(64 * T4::WAVES), 0, s, p);
  return true;
}

// Launch the tiled product: the 8-wave 256 x 128 tile (waves of 64 x 64),
// or with `wide` the 8-wave 512 x 128 tile (waves of 128 x 64, two
// stages).  The input planes are at p.xn.  Returns false when the shape does
// not apply.
bool launch_gemm_tile(const GemvParams& p, bool wide, hipStream_t s) {
  if (p.K % TL_KC != 0 || p.B < 1 || p.n_out < 1) return false;
  const int tb = p.bt_masked ? __builtin_popcountll(p.live_bt[0]) + __builtin_popcountll(p.live_bt[1])
                            : (p.B + GEMM_TILE_BROWS - 1) / GEMM_TILE_BROWS;
  if (tb == 0) return true;   // a prefill step without prompt rows: nothing to compute
  auto grid = [&](int nrows) {
    const int cols = p.mode == GEMV_SWIGLU ? nrows / 2 : nrows;
    const int tiles = ((p.n_out + cols - 1) / cols) * tb;
    return dim3(8 * ((tiles + 7) / 8));
  };
  if (wide) hipLaunchKernelGGL((mfma_tile_kernel<4, 2, 4, 2, 2>), grid(512), dim3(512), 0, s, p);
  else hipLaunchKernelGGL((mfma_tile_kernel<2, 2, 4, 2>), grid(256), dim3(512), 0, s, p);
  return true;
}

// Tile shape for a product.  The 8-wave 256 x 128 tile (two waves per SIMD,
// so one wave's LDS waits and barrier hide under the other's products) ran
// the S2 prefill products at 37-48 % of the matrix-core peak over the three
// terms, against 30-41 % for 4-wave tiles (256 or 128 weight rows) at any
// shape.  Wide products take the 8-wave 512 x 128 tile (waves of 128 x 64
// read 0.42 KB of operand fragments per product instead of 0.67 KB; two
// stages to fit LDS): 2-3 % faster there; on 2,560 output rows it would leave
// a quarter round.
bool gemm_tile_wide(const GemvParams& p) { return p.n_out >= 4096; }
