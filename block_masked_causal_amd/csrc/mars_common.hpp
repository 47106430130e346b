// Shared device/host helpers for the MARS HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mars.h"

namespace mars {

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 32x32x16 bf16 MFMA, fp32 accumulate. Operand lane layout (wave64, lane l,
// i = l % 32, h = l / 32): A holds A[i][8h .. 8h+7], B holds B[8h .. 8h+7][i];
// the 16 accumulators of lane l hold C[8*(r/4) + 4h + (r%4)][i], r = 0..15.
// The K index only has to agree between A and B, so kernels are free to
// permute which physical element sits in which K slot.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Packs two floats into one dword of two bf16 (lo in the low half), RNE.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// Buffer resource over [base, base + bytes): raw buffer loads at byte offsets
// past `bytes` return zeros (hardware range check), which handles every tail
// without branches. Word 3 is the gfx9-family default descriptor format.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Direct global -> LDS load of 16 bytes per lane: lane l's bytes land at
// lds_block + 16 l (lds_block must be the same for the whole wave); reads
// outside the buffer view land as zeros.
__device__ __forceinline__ void lds_load16(rsrc_t r, void* lds_block, uint32_t byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_block,
                                           16, byte_off, 0, 0, 0);
}

// Buffer descriptor as four words (for inline assembly): base address, no
// stride, `bytes` records; reads outside [0, bytes) return zeros.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// As lds_load16, but issued as inline assembly so that the compiler inserts
// no waits of its own for it: the caller waits with wait_vm_upto before the
// barrier that publishes the data.
// The asm writes M0. The compiler treats M0 as a reserved register: it keeps
// no value of its own there across statements (it sets M0 right before each
// instruction that reads it) and refuses M0 in a clobber list. The one case in
// which it may reuse an M0 value it set is a run of its own direct-load
// builtins, so a kernel uses either this or lds_load16, never both.
__device__ __forceinline__ void lds_dma16(const u32x4& rsrc, void* lds_block, uint32_t byte_off) {
  const uint32_t la = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds_block;
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(la), "v"(byte_off), "s"(rsrc)
               : "memory");
}

// Wait until at most N vector-memory loads of this wave are in flight (loads
// complete in order, so everything older than the newest N has landed).
template <int N>
__device__ __forceinline__ void wait_vm_upto() {
  static_assert(N >= 0 && N < 16, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);  // vmcnt = N, expcnt and lgkmcnt unconstrained
}

__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

__device__ __forceinline__ void status_or(int32_t* status, int32_t bits) {
  if (status) atomicOr(status, bits);
}

}  // namespace mars

// ---- host-side argument checks ---------------------------------------------

#define MARS_REQUIRE(cond, code) \
  do {                           \
    if (!(cond)) return (code);  \
  } while (0)

static inline bool mars_aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

static inline int mars_launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MARS_OK : MARS_ERR_LAUNCH;
}

// Compute units of the current device (0 when the query fails).
static inline int mars_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return n;
}
