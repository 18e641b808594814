// Device primitives shared by the bf16 kernels (gfx950): vector types, LDS
// addressing, raw buffer resources, the LDS-direct copy and its waits.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace magi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) const f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr unsigned kNoTile = 0x80000000u;    // scalar offset past any tile image buffer (< 2 GiB): reads give zeros
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return unsigned(reinterpret_cast<uintptr_t>(LDS_PTR(const char, p)));
}

// Raw buffer resource: base, stride 0, num_records = bytes (reads at or past
// `bytes` return zero), dword3 = 32-bit data format as used for raw buffers.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, unsigned bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  i32x4 r;
  r[0] = int(unsigned(a));
  r[1] = int(unsigned(a >> 32) & 0xffffu);
  r[2] = int(bytes);
  r[3] = 0x00020000;
  return r;
}

// Global -> LDS copy of 16 bytes per active lane: lane i (of the wave) reads
// buffer offset voff + soff (zeros past num_records) and writes LDS byte
// lds + 16 i, so a wave passes its own 1 KiB part of a ring stage as `lds`.
// Issued through asm so that the compiler does not order later LDS reads of
// other ring stages behind it; completion is awaited explicitly (vmcnt)
// before the barrier that publishes the stage. m0 is saved and restored
// inside the asm.
__device__ __forceinline__ void dma16(i32x4 rsrc, unsigned voff, unsigned soff, unsigned lds) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// All LDS traffic of this wave finished, then the workgroup barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory"); }

// Sum over the four 16-lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float sum_groups(float x) {
  x += __shfl_xor(x, 16, 64);
  x += __shfl_xor(x, 32, 64);
  return x;
}

}  // namespace
}  // namespace magi
