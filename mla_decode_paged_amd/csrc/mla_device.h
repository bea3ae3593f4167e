// Device-side building blocks shared by the libmla kernels (gfx950 only).
//
// MFMA operand layouts used throughout (checked on the hardware by the GPU
// tests through the kernels that rely on them):
//  v_mfma_f32_32x32x16_bf16  A: lane l holds row l%32, 8 consecutive k of
//      group l/32; B: lane l holds column l%32, the same k group; C: lane l,
//      element v is row 8*(v/4) + 4*(l/32) + v%4, column l%32.
//  v_mfma_f32_16x16x32_bf16  A: lane l holds row l%16, 8 consecutive k of
//      group l/16; B: lane l holds column l%16, the same k group; C: lane l,
//      element i is row 4*(l/16) + i, column l%16.
//  ds_read_b64_tr_b16  within each 16-lane block, lane j supplies the address
//      of 4 consecutive 16-bit values in row r0 + j/4 at column c0 + 4*(j%4);
//      lane i receives column c0 + i of rows r0 .. r0+3. This yields a B (or
//      A) operand whose k runs along rows of a row-major tile in LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define MLA_LDS __attribute__((address_space(3)))

constexpr int kPage = MLA_PAGE_TOKENS;   // 64 tokens
constexpr int kDLat = MLA_D_LATENT;      // 512
constexpr int kDRope = MLA_D_ROPE;       // 64
constexpr int kDRow = MLA_D_ROW;         // 576
constexpr int kDNope = MLA_D_NOPE;       // 128
constexpr int kRowBytes = kDRow * 2;     // 1152

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Accumulate into an accumulator pinned to AGPRs. The compiler does not see
// inside the asm, so the hazards it would pad for a builtin MFMA are padded
// here: 2 wait states between a VALU write and an MFMA read of its operands,
// and callers run mfma_drain() before any VALU or memory read of `acc`.
__device__ __forceinline__ void mfma32_agpr(f32x16& acc, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// acc = 0 through the matrix core, so the accumulator never leaves AGPRs.
__device__ __forceinline__ void mfma32_agpr_zero(f32x16& acc, bf16x8 zero) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(zero));
}
// Wait states after an MFMA before its result may be read outside the matrix core.
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 15\n\ts_nop 15" ::: "memory"); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte LDS read at a byte offset from an LDS base.
__device__ __forceinline__ bf16x8 lds_read16(const MLA_LDS char* base, int byte_off) {
  return *reinterpret_cast<const MLA_LDS bf16x8*>(base + byte_off);
}

// Transposed 4 x bf16 LDS read (see the layout note above).
__device__ __forceinline__ bf16x4 lds_read_tr4(const MLA_LDS char* base, int byte_off) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<MLA_LDS i16x4*>(const_cast<MLA_LDS char*>(base) + byte_off));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat4(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Direct global -> LDS copy of 16 bytes per lane. `lds_wave_base` must be the
// same for every lane of the wave; lane l's bytes land at lds_wave_base + 16*l.
__device__ __forceinline__ void g2lds16(const void* gsrc, MLA_LDS char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(
      (const __attribute__((address_space(1))) void*)(gsrc),
      (MLA_LDS void*)(lds_wave_base), 16, 0, 0);
}

// The same copy written as inline assembly: `base` (wave-uniform, in SGPRs)
// plus a per-lane 32-bit offset, landing at LDS byte address lds_addr +
// 16 * lane. The compiler does not see this load, so it neither counts it in
// its own wait insertion (where a pending direct-to-LDS load makes it drain
// every LDS read, lgkmcnt(0), instead of keeping a read-ahead ring) nor waits
// for it before later LDS accesses: the caller waits (vmcnt) and synchronises.
__device__ __forceinline__ void g2lds16_untracked(const char* base, unsigned voff, unsigned lds_addr) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_addr) : "memory");
}

// The same for 4 bytes per lane (lane l's bytes land at lds_addr + 4 * lane).
__device__ __forceinline__ void g2lds4_untracked(const char* base, unsigned voff, unsigned lds_addr) {
  asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_addr) : "memory");
}

__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Eight fp8 e4m3 codes (bytes 0..7 of v) -> eight bf16 values in the same
// order, exactly (every e4m3 value is a bf16 value). Written as the
// instruction itself: lane layouts of the conversion builtins' second result
// were not what the hardware returns, while this form was checked on all 256
// codes. The two trailing wait states cover a matrix instruction that reads
// the result next (the compiler does not see the writes inside the asm).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(u32x2 v) {
  unsigned a, b, c, d;
  asm("v_cvt_scalef32_pk_bf16_fp8 %0, %4, 1.0\n\t"
      "v_cvt_scalef32_pk_bf16_fp8 %1, %4, 1.0 op_sel:[1,0,0]\n\t"
      "v_cvt_scalef32_pk_bf16_fp8 %2, %5, 1.0\n\t"
      "v_cvt_scalef32_pk_bf16_fp8 %3, %5, 1.0 op_sel:[1,0,0]\n\t"
      "s_nop 1"
      : "=&v"(a), "=&v"(b), "=&v"(c), "=&v"(d)
      : "v"(v[0]), "v"(v[1]));
  return as_bf16x8(u32x4{a, b, c, d});
}

// 8-byte LDS read.
__device__ __forceinline__ u32x2 lds_read8(const MLA_LDS char* base, int byte_off) {
  return *reinterpret_cast<const MLA_LDS u32x2*>(base + byte_off);
}

// Transposed 8-bit LDS read (ds_read_b64_tr_b8): within each 16-lane block,
// lane j supplies the address of 8 consecutive bytes of row r0 + j / 2 at
// byte column c0 + 8 (j % 2); lane i receives byte column c0 + i of rows
// r0 .. r0 + 7 (checked on the hardware for all 64 lanes).
__device__ __forceinline__ u32x2 lds_read_tr8(const MLA_LDS char* base, int byte_off) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      reinterpret_cast<MLA_LDS i32x2*>(const_cast<MLA_LDS char*>(base) + byte_off));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ int wave_id_uniform() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ unsigned short bf16_bits(float x) {
  return __builtin_bit_cast(unsigned short, (__bf16)x);
}

// Pack 8 floats into 8 bf16 (nearest even).
__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5,
                                        float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

}  // namespace mla
