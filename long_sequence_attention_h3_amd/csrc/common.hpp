// common.hpp — types and small device helpers shared by the libh3attn kernels
// (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kHeadDim = 128;          // the only supported head size
constexpr int kChunks = kHeadDim / 8;  // 16-byte chunks (8 bf16) per head row
constexpr int kTileKeys = 64;          // keys per packed K/V tile

// Packed K/V tile image, the exact byte layout the attention kernel keeps in LDS:
//   K part: 64 key rows x (256 B of channels + 16 B pad)            = 17,408 B
//   V part: 128 channel rows x (128 B of keys + 16 B pad)            = 18,432 B
// The pads make every MFMA operand read of the attention kernel bank-conflict free
// with a plain base + immediate-offset address.
constexpr int kKRowPitch = kHeadDim * 2 + 16;             // 272
constexpr int kVRowPitch = kTileKeys * 2 + 16;            // 144
constexpr int kKImageBytes = kTileKeys * kKRowPitch;      // 17,408
constexpr int kVImageBytes = kHeadDim * kVRowPitch;       // 18,432
constexpr int kTileImageBytes = kKImageBytes + kVImageBytes;  // 35,840 = 35 KiB
// The pad of K row 0 carries the tile's largest K row norm (fp32, the norm of the bf16
// values stored) and then the fp32 factor the stored K rows were multiplied by before
// rounding (1: stored as given); the rest of every pad is zero.
constexpr int kKNormOffset = kHeadDim * 2;      // byte 256 of the image
constexpr int kKMulOffset = kKNormOffset + 4;   // byte 260

// Rotary descriptor as the kernels see it.
struct RopeArgs {
  double theta;
  int64_t n_1d;       // tokens [0, n_1d) are 1-D
  int32_t sec[3];     // 3-axis channel sections (multiples of 16)
  int32_t gt, gh, gw;
};

// bf16 <-> fp32.  Widening is exact; narrowing rounds to nearest even.
__device__ __forceinline__ float bf2f(__bf16 x) { return (float)x; }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ void unpack8(u32x4 raw, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w = raw[i];
    f[2 * i] = __uint_as_float(w << 16);
    f[2 * i + 1] = __uint_as_float(w & 0xffff0000u);
  }
}

__device__ __forceinline__ u32x4 pack8(const float* f) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return r;
}

// Value of x held by lane (l ^ 32), via v_permlane32_swap.
__device__ __forceinline__ float other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                            false);
  // lanes 0-31 receive the upper half in r[1]; lanes 32-63 the lower half in r[0]
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// max / sum of x over the lane pair (l, l ^ 32); identical bits in both lanes.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                            false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                            false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Copy 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4):
// lane i's 16 bytes at sbase + voff (voff its own) land at LDS byte lds_base + 16 i.
// The scalar-base form of the instruction takes the wave-uniform sbase in SGPRs and a
// 32-bit per-lane offset, so a copy costs no per-lane address arithmetic (with a 64-bit
// per-lane address the copies cost 64-bit vector adds in the attention loops, measured
// at 2 % of the bf16 kernel's time).
// Issued as inline assembly on purpose: the compiler cannot tell which LDS bytes the
// copy writes, and for the intrinsic it conservatively waits for every outstanding copy
// before the next LDS read; the callers instead wait for their own copies explicitly
// (s_waitcnt vmcnt) and publish them with a barrier before any lane reads the bytes.
// The LDS address goes in through the "{m0}" operand constraint: the compiler itself
// writes M0 before the copy and knows that the copy reads it, so no M0 value the
// compiler keeps live elsewhere can be disturbed.
__device__ __forceinline__ void dma_to_lds16(const void* sbase, uint32_t voff,
                                             uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "{m0}"(lds_base)
               : "memory");
}

// Workgroup -> logical tile.  Consecutive workgroup ids are dispatched round-robin over
// the 8 XCDs; this bijection hands each XCD one contiguous range of logical tiles, so
// the workgroups resident on one XCD (sharing its L2) work on the same head.
__device__ __forceinline__ int xcd_remap(int pid, int total) {
  constexpr int kXcd = 8;
  const int per = total / kXcd, rem = total % kXcd;
  const int xcd = pid % kXcd, idx = pid / kXcd;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

}  // namespace h3
