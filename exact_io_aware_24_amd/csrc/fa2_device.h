// Device helpers shared by the bf16 forward and backward kernels (gfx950).
// Internal: not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2 {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLog2e = 1.442695040888963407360f;
// Buffer descriptor word 3: 32-bit data format, raw (untyped) addressing.
constexpr int kBufWord3 = 0x00020000;

// (x of lanes 0-31, x of lanes 32-63) as seen from every lane.
__device__ __forceinline__ void halves(float x, float &lo, float &hi) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// Scheduling fence for LDS reads and MFMAs only: VALU, SALU, transcendental
// and VMEM instructions may still be moved across it.  It pins operand
// reads a whole MFMA group ahead of their consumers (the scheduler would
// otherwise sink them to just before use, exposing LDS latency).
__device__ __forceinline__ void pin_lds_mfma() {
  __builtin_amdgcn_sched_barrier(0x0002 | 0x0004 | 0x0010 | 0x0020 | 0x0040 |
                                 0x0200 | 0x0400);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

template <typename T>
__device__ __forceinline__ T lds_load(const char *base, int byte_off) {
  return *reinterpret_cast<const T *>(base + byte_off);
}

// Transposing LDS read: within each group of 16 lanes, lane L receives
// element L % 4 of the 8-byte chunks addressed by lanes 4e + L / 4, e = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr(const char *base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4 *)(base + byte_off));
}

// 16 bytes per lane from a raw buffer straight into LDS at lds_addr + 16 *
// lane (buffer_load_dwordx4 ... lds; M0 holds the wave-uniform LDS address).
// Issued through asm so that the compiler does not track it: it would
// otherwise wait for every such load before the next LDS read of ANY buffer,
// serialising the prefetch.  The kernels wait (vmcnt) before the barrier
// that publishes a filled buffer, which is the only ordering needed.  The
// kernels pass soff = 0 (see tile_desc).
__device__ __forceinline__ void dma16(u32x4 rsrc, int voff, int soff,
                                      uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_addr)
      : "memory", "m0");
}

// Raw buffer descriptor (words 0-3) for `bytes` bytes at `base`, made
// wave-uniform so that it lives in scalar registers.  Reads at offsets of
// `bytes` or more return zero.
__device__ __forceinline__ u32x4 make_desc(const void *base, int bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(bytes));
  r[3] = static_cast<uint32_t>(kBufWord3);
  return r;
}

// Descriptor of bytes [tile_byte, total_bytes) of the array at `base`.
// Loads through it address the tile from its first byte, and everything at
// or past the end of the array reads as zero: the whole offset is in the
// range-checked part of the address (descriptor base + per-lane offset),
// never in the scalar offset operand.
__device__ __forceinline__ u32x4 tile_desc(const void *base, int total_bytes,
                                           int tile_byte) {
  return make_desc(static_cast<const char *>(base) + tile_byte,
                   total_bytes - tile_byte);
}

__device__ __forceinline__ uint32_t lds_addr(const char *p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const char *)(p)));
}

// Workgroup id -> logical block id.  Hardware deals workgroups round-robin
// over the 8 XCDs; this mapping gives each XCD a contiguous range of logical
// blocks (so the blocks of one head share one L2), in dispatch order.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int per_xcd = total >> 3;
  return (w < (per_xcd << 3)) ? (w & 7) * per_xcd + (w >> 3) : w;
}

}  // namespace dev
}  // namespace fa2
