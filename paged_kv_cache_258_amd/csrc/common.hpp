// Shared device helpers for the nkv kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nkv {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

// log2(e): softmax is evaluated as exp2(x * scale * log2(e) - m).
constexpr float kLog2e = 1.4426950408889634f;

// Storage tags.  A bf16 element is kept as its raw 16 bits.
struct F32 {
  using elem = float;
  static constexpr int bytes = 4;
};
struct BF16 {
  using elem = uint16_t;
  static constexpr int bytes = 2;
};

// ---- bf16 <-> f32 --------------------------------------------------------------------
// A bf16 is the top half of a binary32, so widening is a 16-bit shift of the pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---- cross-lane --------------------------------------------------------------------
// DPP controls (gfx9 encoding).
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141; // lane i <- lane 7-i inside each 8-lane half row
constexpr int kDppRowRor8 = 0x128;       // lane i <- lane (i+8)%16 inside each 16-lane row

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}

// Sum over the 8 lanes of an aligned 8-lane group; every lane gets the total.
__device__ __forceinline__ float group8_sum(float x) {
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  return x;
}

// Sum / max with the lane 16 (resp. 32) positions away, every lane getting the result:
// v_permlane16_swap / v_permlane32_swap (gfx950) swap rows (halves) between two VGPRs,
// so swapping a value with itself yields both partners' values in the two outputs.
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Wait until at most N vector-memory operations of this wave are outstanding.  Used
// for loads that write LDS directly (global_load_lds), which the compiler does not
// track; the "memory" clobber keeps LDS reads from moving above the wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait for every outstanding vector memory operation, through the builtin so that the
// compiler's own wait-count tracking learns that register loads issued before it have
// landed (after an asm wait it would still guard their registers with another full wait).
// Encoding (gfx9): vmcnt[3:0]=0, expcnt[6:4]=7, lgkmcnt[11:8]=15, vmcnt[15:14]=0.
__device__ __forceinline__ void wait_vmem_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  asm volatile("" ::: "memory");
}

// Global -> LDS copies (global_load_lds, 16 or 4 bytes per lane; lane i writes
// lds_base + i*size, lds_base the same for the whole wave).  They are issued through
// inline asm so that the compiler neither tracks them nor guards every later LDS read
// with a "wait for all vector loads": each caller orders them itself with wait_vmcnt.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p)));
}
__device__ __forceinline__ void load_lds16(const void* gptr, void* lds_base) {
  uint32_t saved;  // m0 is reserved by the compiler: restore it before leaving the asm
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(gptr), "s"(lds_addr(lds_base)) : "memory");
}
// Same copy with the address split into a wave-uniform 64-bit base (SGPRs) and a 32-bit
// per-lane byte offset: no 64-bit address arithmetic per lane.
__device__ __forceinline__ void load_lds16_s(const void* sbase, uint32_t voff, void* lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(voff), "s"(sbase), "s"(lds_addr(lds_base)) : "memory");
}
// The same two copies with the LDS destination given as an LDS byte address (uniform).
// No immediate offset is used: the instruction's offset field moves the LDS destination
// as well as the global address.
__device__ __forceinline__ void load_lds16_s_at(const void* sbase, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(voff), "s"(sbase), "s"(lds) : "memory");
}
__device__ __forceinline__ void load_lds16_at(const void* gptr, uint32_t lds) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(gptr), "s"(lds) : "memory");
}
// The same with the nontemporal hint, for data read once and not again soon (a decode
// step's K/V stream): it leaves less of the caches to lines that will not be reused.
__device__ __forceinline__ void load_lds16_s_nt(const void* sbase, uint32_t voff, void* lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2 nt\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(voff), "s"(sbase), "s"(lds_addr(lds_base)) : "memory");
}
__device__ __forceinline__ void load_lds4(const void* gptr, void* lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved) : "v"(gptr), "s"(lds_addr(lds_base)) : "memory");
}

__device__ __forceinline__ float shfl_xor(float x, int mask) {
  int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}

// exp2 that returns exactly 0 for -inf (hardware v_exp_f32 does).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int64_t row_of(const int32_t* __restrict__ table_row, int pos,
                                          int log2_bs, int bs_mask) {
  const int64_t phys = table_row[pos >> log2_bs];
  return (phys << log2_bs) + (pos & bs_mask);
}

}  // namespace nkv
