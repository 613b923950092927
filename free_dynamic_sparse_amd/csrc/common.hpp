// Device-side helpers shared by the Sol-Attn kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace solattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
// MI355X has 8 XCDs; consecutive workgroup ids are dealt round-robin to them.
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;

// Map a workgroup id to a work item so that every XCD receives one
// contiguous range of items (neighbouring query blocks of one head share
// key/value blocks, and each XCD has its own L2).  Bijective on [0, total).
__device__ __forceinline__ uint32_t xcd_contiguous_item(uint32_t bid, uint32_t total) {
  const uint32_t q = total / kXcds, r = total % kXcds;
  const uint32_t x = bid % kXcds, s = bid / kXcds;
  return x * q + (x < r ? x : r) + s;
}

// Head-striped schedule for the attention kernels: every XCD works through
// the (b, h) in the same order, XCD x taking for (b, h) = bh the contiguous
// query-block slab s = (x + bh) mod 8, items [s*per, (s+1)*per) with
// per = ceil(N / 8).  One head's K and V then stay resident in the shared
// last-level cache while each XCD's L2 sees neighbouring query blocks, whose
// selected key blocks overlap.  Rotating the slab with bh gives every XCD
// each slab equally often: where the work per query block depends on its
// position (sparsity varies along the sequence), a fixed slab per XCD would
// leave the XCDs with unequal totals and the whole launch waiting for the
// busiest one.  The grid has 8 * per * BH workgroups; a workgroup whose slab
// slot lies past N has no item (returns false).
__device__ __forceinline__ bool head_striped_item(uint32_t bid, uint32_t N, uint32_t per,
                                                  uint32_t* bh, uint32_t* i) {
  const uint32_t x = bid % kXcds, slot = bid / kXcds;
  *bh = slot / per;
  *i = ((x + *bh) % kXcds) * per + (slot - *bh * per);
  return *i < N;
}

// p as a global-memory pointer, so that accesses through it are global (not
// flat) instructions: a pointer read from memory, such as the kernel arguments
// the persistent kernel reloads per item, no longer carries that fact.  Flat
// loads would also count against the LDS wait counter, so a wait for LDS
// reads would wait for them too.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gbl(const T* p) {
  return (const __attribute__((address_space(1))) T*)p;
}
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gbl(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// 8 consecutive floats -> 8 bf16 (round to nearest even).
__device__ __forceinline__ bf16x8 pack_bf16x8(const float* f) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)f[e];
  return r;
}

__device__ __forceinline__ bf16x8 pack_bf16x8(f32x4 a, f32x4 b) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (bf16)a[e];
    r[4 + e] = (bf16)b[e];
  }
  return r;
}

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16), one wave.
// Operand lane layout: lane l holds row (A) / column (B) l % 32 and eight
// consecutive k values of half l / 32; result lane l holds column l % 32 and
// rows 8*(r/4) + 4*(l/32) + r%4 for register r.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row (A) / column (B) index inside a 32x32 MFMA result for register r of a
// lane in half h.
__device__ __forceinline__ constexpr int mfma_row(int r, int h) {
  return 8 * (r / 4) + 4 * h + (r % 4);
}

// Wait until at most N of this wave's vector-memory loads are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt vmcnt(0) issued through the builtin, so that the compiler's own
// waitcnt bookkeeping sees it: loads issued before it (the Q operand and
// other set-up loads) count as complete inside a block loop, which then
// needs no vector-memory wait of the compiler's own.  Encoding (gfx9):
// vmcnt 0, expcnt 7, lgkmcnt 15.
__device__ __forceinline__ void settle_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier that does not wait for outstanding direct-to-LDS loads.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS byte address of a __shared__ object (wave-uniform).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p);
}

// Direct-to-LDS load (global_load_lds_dwordx4): each lane fetches 16 bytes
// at sbase + voffset and the wave writes them to 1 KB of LDS at
// lds + 16 * lane.  sbase and lds must be wave-uniform.  Issued from inline
// assembly, so the compiler does not count it: the caller waits for it
// (wait_vm) before a barrier that publishes the data.  The s_nop covers the
// M0-write to LDS-DMA hazard.
__device__ __forceinline__ void lds_dma_16b(uint32_t voffset, const uint16_t* sbase,
                                            uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voffset), "s"(sbase),
               "{m0}"(lds)
               : "memory");
}

__device__ __forceinline__ float wave_max_pair(float x) {
  // lanes l and l^32 hold the two halves of one 32x32 result column
  return fmaxf(x, __shfl_xor(x, 32));
}

}  // namespace solattn
