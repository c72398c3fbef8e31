// Matrix-core building blocks shared by the product kernels (gfx950):
// operand vector types, LDS DMA, the vmcnt wait + barrier and the
// weight row space of a product.
#pragma once
#include "common.h"
#include "internal.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

// The product's weight row space held in scalar registers: for SwiGLU,
// segment s is W1 (s = 0) or W3; otherwise the rows of w[0], w[1], w[2]
// follow each other.  (The empty asm pins each pointer in an SGPR: left
// alone, the compiler turns the select below into a per-lane indexed load
// of the kernel arguments.)
struct RowSpace {
  uint64_t w0, w1, w2;
  int r0, r1, swiglu;
  size_t ld;    // row bytes
  __device__ __forceinline__ explicit RowSpace(const GemvParams& p) {
    w0 = (uint64_t)p.w[0];
    w1 = (uint64_t)p.w[1];
    w2 = (uint64_t)p.w[2];
    asm volatile("" : "+s"(w0), "+s"(w1), "+s"(w2));
    r0 = p.rows[0];
    r1 = p.rows[1];
    swiglu = p.mode == GEMV_SWIGLU;
    ld = (size_t)p.K * 2;
  }
  // (Written as two 64-bit selects by offset: a three-way pointer select
  // is otherwise lowered to a per-lane indexed load from a stack array.)
  __device__ __forceinline__ const char* row(int r, int s) const {
    uint64_t base = w0;
    if (swiglu) {
      base += s == 0 ? 0 : w1 - w0;
    } else {
      const bool in1 = r >= r0, in2 = r >= r0 + r1;
      base += in2 ? w2 - w0 : (in1 ? w1 - w0 : 0);
      r -= in2 ? r0 + r1 : (in1 ? r0 : 0);
    }
    return (const char*)base + (size_t)r * ld;
  }
};

// LDS DMA of 16 bytes per lane: lane i's bytes land at lds + 16 i (lds is
// wave-uniform).  Written as inline asm so that the compiler does not track
// these copies: its conservative tracking of LDS DMA across the main loop's
// back edge would wait for every copy in flight before each LDS read.  The
// kernel waits for them itself (wait_vm_barrier) and issues no other vector
// memory loads while any is in flight.
__device__ __forceinline__ void dma16(const void* g, char* lds) {
  const unsigned la = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_void*)lds);
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(la) : "memory", "m0");
}

// Wait until at most N of this wave's vector memory operations are
// outstanding, then workgroup barrier.  One asm statement with a memory
// clobber, so that no LDS access moves across it.
template <int N> __device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}
