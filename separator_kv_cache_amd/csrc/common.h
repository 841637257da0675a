// Shared device/host helpers of the sepattn library (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sepattn.h"

// ---------------------------------------------------------------- host side

// Records an error text for sepattn_last_error() and returns `code`.
int sepattn_fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Checks a HIP call made while enqueueing work.
int sepattn_hip_check(hipError_t e, const char* what);
// Returns SEPATTN_OK if the current device is gfx950, else an error.
int sepattn_check_device();

// The backward's workspace: D, fp32 [B, Hq, L], rounded up to 256 bytes, then
// the dK/dV kernel's tile counters.
constexpr size_t SEPATTN_BWD_QUEUE_BYTES = 1024;
inline size_t sepattn_bwd_d_bytes(const sepattn_shape* s) {
  return ((size_t)s->B * s->Hq * s->L * 4 + 255) / 256 * 256;
}

#define SEPATTN_TRY(x)          \
  do {                          \
    int _rc = (x);              \
    if (_rc != SEPATTN_OK) return _rc; \
  } while (0)

// ---------------------------------------------------------------- device side

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// D(32x32) += A(32x16) B(16x32), bf16 inputs, fp32 accumulate.
// Lane l supplies A[l%32][8*(l/32) + 0..7] and B[8*(l/32) + 0..7][l%32];
// result register r of lane l is D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// D(32x32) += A(32x2) B(2x32), fp32.  Lane l supplies A[l%32][l/32] and
// B[l/32][l%32]; same result layout as above.
__device__ __forceinline__ f32x16 mfma32x2f(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// LDS transposing read of 16-bit elements.  Within each group of 16 lanes,
// lane i receives, for s = 0..3, element (i % 4) of the 4-element chunk
// addressed by lane 4*s + i/4 of the same group.
__device__ __forceinline__ bf16x4 lds_read_tr16(const void* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) char*)p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }

// Rows of one (stream, KV head) slice of a SepCache's K: its slots rounded
// up to whole 16-row tiles (the tiled K layout of the cache kernels).
__host__ __device__ inline int sepcache_k_rows_of(int slots) { return (slots + 15) & ~15; }

// 16-byte global loads and stores.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *(const u32x4*)p; }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *(u32x4*)p = v; }

// Raw buffer loads.  A resource covers `bytes` bytes from `base`; a load at an
// offset past the end returns zeros without touching memory, so absent rows
// need no branch.  Offsets are 32-bit, which bounds one resource to 2 GiB.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t BUF_OOB = 0x80000000u;  // an offset past the end of every resource
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // dword 3 = 0x00020000: 32-bit data format, the value raw buffer loads need on gfx9-family parts
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bld16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
// The same with the non-temporal hint (nt): for rows a launch reads once
// and that other launches' data will displace before they are read again.
__device__ __forceinline__ u32x4 bld16_nt(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
}
__device__ __forceinline__ int bld4(rsrc_t r, uint32_t off) {
  return (int)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

// Sum of the 16 elements of v as a balanced tree (short dependency chains).
// Plain adds on purpose: v_dot2 against a ones vector would take half the
// instructions, but on gfx950 it issues through the matrix pipe and then
// waits behind the MFMAs of the other wave on the SIMD.
__device__ __forceinline__ float tree_sum16(const f32x16& v) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = v[2 * i] + v[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = a[2 * i] + a[2 * i + 1];
  return (a[0] + a[1]) + (a[2] + a[3]);
}

// Swap values between lane l and lane l ^ 32.
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// max(x[l], x[l ^ 32]) without an LDS round trip.  v_permlane32_swap swaps the
// upper 32 lanes of its first register with the lower 32 lanes of its second,
// so on two copies of x every lane ends up holding x[l] in one and x[l ^ 32] in
// the other.  The s_nops give the VALU-write -> permlane and permlane -> VALU
// wait states.
__device__ __forceinline__ float max_xor32(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Data-parallel-primitive moves within a row of 16 lanes (no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7-i within 8
constexpr int DPP_MIRROR = 0x140;      // lane i <-> 15-i within 16

// Maximum over aligned groups of N lanes (N = 4, 8 or 16); every lane gets it.
template <int N>
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, dpp_mov<DPP_XOR1>(x));
  x = fmaxf(x, dpp_mov<DPP_XOR2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp_mov<DPP_HALF_MIRROR>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp_mov<DPP_MIRROR>(x));
  return x;
}

// Sum over aligned groups of N lanes (N = 4, 8 or 16); every lane gets it.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_mov<DPP_XOR1>(x);
  x += dpp_mov<DPP_XOR2>(x);
  if constexpr (N >= 8) x += dpp_mov<DPP_HALF_MIRROR>(x);
  if constexpr (N >= 16) x += dpp_mov<DPP_MIRROR>(x);
  return x;
}
