// Device-side helpers shared by the libsa kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, workgroups dealt round-robin

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Two floats -> packed bf16 pair with the hardware conversion (v_cvt_pk_bf16_f32,
// round to nearest even).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Global 16-byte load / store (the pointer must be 16-byte aligned).
__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void stg16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Workgroup index -> work item, so that each XCD receives one contiguous
// range of work items (neighbouring items share K/V and stay in that XCD's L2).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n / kXcds, r = n % kXcds;
  const int x = bid % kXcds, slot = bid / kXcds;
  return x * q + (x < r ? x : r) + slot;
}

// Order-preserving key of a float: larger float -> larger key; -0 and +0 map
// to the same key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// NaN or +-inf.
__device__ __forceinline__ bool nonfinite(float f) { return (__float_as_uint(f) & 0x7f800000u) == 0x7f800000u; }

// Bit 0 of the optional device flag: some score the call wrote is not finite.
__device__ __forceinline__ void flag_nonfinite(int32_t* err, bool bad) {
  if (bad && err != nullptr) atomicOr(reinterpret_cast<unsigned int*>(err), 1u);
}

// a + b and max(a, b) of a value with the one in lane l ^ 32, through
// v_permlane32_swap (a register exchange between the two wave halves, no LDS
// round trip).  Both operations are symmetric, so every lane gets exactly what
// op(v, __shfl_xor(v, 32)) gives.
__device__ __forceinline__ float xor32_add(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ bool is_nan(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu);
}

// Wait until at most N vector-memory operations of this wave are in flight.
// Inline assembly, because the compiler's wait-count pass does not see the
// inline-assembly copies below and would drop a builtin wait as redundant.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }
// Drain every vector-memory load the compiler issued (visible to its
// wait-count pass, so it also stops guarding those loads later on).
__device__ __forceinline__ void drain_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// One 16-byte direct global->LDS copy per lane: lane L of the wave writes LDS
// bytes [lds_off + 16L, +16).  Written as inline assembly so that the compiler
// does not guard every later LDS read with a wait for all copies in flight.
// A kernel that uses it waits on the vector-memory counter itself
// (wait_vmcnt) and issues no other vector-memory loads while copies are in
// flight, so its counts are exact.
__device__ __forceinline__ void dma16(uint32_t lds_off, const void* gptr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 1\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_off), "v"(gptr)
               : "memory", "m0");
}

// Same copy with a wave-uniform 64-bit base (SGPR pair) and a 32-bit per-lane
// byte offset, which saves the 64-bit address arithmetic per lane.
__device__ __forceinline__ void dma16_sb(uint32_t lds_off, const void* base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 1\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_off), "v"(voff), "s"(base)
               : "memory", "m0");
}

// The same two copies at device scope (sc1): the request skips the CU's
// vector cache and is served by L2.  For read-only tiles that the CU uses once
// this avoids filling the vector cache with lines nobody reads again; the
// bytes delivered are identical.
__device__ __forceinline__ void dma16_dev(uint32_t lds_off, const void* gptr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 1\n\tglobal_load_lds_dwordx4 %1, off sc1"
               :
               : "s"(lds_off), "v"(gptr)
               : "memory", "m0");
}
__device__ __forceinline__ void dma16_sb_dev(uint32_t lds_off, const void* base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 1\n\tglobal_load_lds_dwordx4 %1, %2 sc1"
               :
               : "s"(lds_off), "v"(voff), "s"(base)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// XOR key of row r for tiles of 256-byte rows (16 chunks of 16 bytes): chunk c
// of row r is stored at position c ^ key(r).  Sixteen consecutive rows get
// distinct keys, and 4 consecutive rows (a multiple of 4 apart from 0) x 4
// consecutive chunks (starting at a multiple of 4) map to 16 distinct positions.
__device__ __forceinline__ int swz_key128(int row) { return 4 * (row & 3) + ((row >> 2) & 3); }

// Transposing LDS read (ds_read_b64_tr_b16): in each 16-lane group, lane j
// points at 4 consecutive 16-bit values; lane j receives element j%4 of the
// values pointed at by lanes 4e + j/4 of its group, e = 0..3.
__device__ __forceinline__ v4i16 lds_read_tr16(const uint16_t* lds_elem) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const __attribute__((address_space(3))) uint16_t*)lds_elem);
}

}  // namespace sa
