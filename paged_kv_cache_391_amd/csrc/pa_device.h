// Device-side helpers shared by every kernel of the library: element types,
// exact widening, round-to-nearest-even narrowing, the paged address
// translation and 16-lane row reductions.
//
// Target: gfx950 (CDNA4), wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_bounds.h"

namespace pa {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum class Dt : int { F32 = 0, F16 = 1, BF16 = 2 };

template <Dt DT> struct ElemT;
template <> struct ElemT<Dt::F32> { using storage = uint32_t; static constexpr int bytes = 4; };
template <> struct ElemT<Dt::F16> { using storage = uint16_t; static constexpr int bytes = 2; };
template <> struct ElemT<Dt::BF16> { using storage = uint16_t; static constexpr int bytes = 2; };

// ---- widening (exact) -----------------------------------------------------

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// element `i` (0/1) of a packed 32-bit word holding two 16-bit values, or
// the word itself for fp32
template <Dt DT> __device__ __forceinline__ float widen_lo(uint32_t w) {
  if constexpr (DT == Dt::F32) return __uint_as_float(w);
  else if constexpr (DT == Dt::F16) return f16_bits_to_f32(w & 0xffffu);
  else return __uint_as_float(w << 16);
}
template <Dt DT> __device__ __forceinline__ float widen_hi(uint32_t w) {
  if constexpr (DT == Dt::F16) return f16_bits_to_f32(w >> 16);
  else return __uint_as_float(w & 0xffff0000u);
}

// ---- narrowing (round to nearest even) -------------------------------------

__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
  // v_cvt_f16_f32 rounds with the default round-to-nearest-even mode
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // keep NaN quiet
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// ---- matrix cores ------------------------------------------------------------

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// D = A B + C on v_mfma_f32_16x16x32_{f16,bf16}: A 16x32 (lane l holds row
// l%16, k = 8*(l/16)..+7), B 32x16 (lane l holds column l%16, the same 8 k),
// C/D 16x16 fp32 (lane l holds rows 4*(l/16)..+3 of column l%16).
template <Dt DT> __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == Dt::F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// 16-bit bits of x in the input type (round to nearest even), and back
template <Dt DT> __device__ __forceinline__ uint32_t to_bits(float x) {
  if constexpr (DT == Dt::F16) return f32_to_f16_bits(x);
  else return f32_to_bf16_bits(x);
}
template <Dt DT> __device__ __forceinline__ float from_bits(uint32_t b) {
  if constexpr (DT == Dt::F16) return f16_bits_to_f32(b);
  else return bf16_bits_to_f32(b);
}

// Two floats narrowed into one word of two 16-bit values (lo in bits 0..15),
// round to nearest even, on the packed v_cvt_pk_{f16,bf16}_f32 converts.
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <Dt DT> __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (DT == Dt::F16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, half2_t));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf162_t));
}
// 1.0 in both halves of a word, in the input type
template <Dt DT> constexpr uint32_t ones2() { return DT == Dt::F16 ? 0x3C003C00u : 0x3F803F80u; }

// ---- paged address translation ---------------------------------------------
// Caches are [num_blocks][H][BS][D]. Logical token t of a sequence lives in
// physical block table[t / BS] at offset t % BS; one (block, head) tile of
// BS*D elements is contiguous.

__device__ __forceinline__ int64_t kv_tile_offset(int32_t phys_block, int head, int H, int BS, int D) {
  return ((int64_t)phys_block * H + head) * (int64_t)BS * D;
}
__device__ __forceinline__ int64_t kv_row_offset(int32_t phys_block, int head, int off, int H, int BS, int D) {
  return kv_tile_offset(phys_block, head, H, BS, D) + (int64_t)off * D;
}

// ---- reductions over the 16 lanes of a DPP row ------------------------------
// quad_perm [1,0,3,2] and [2,3,0,1] exchange within quads, row_half_mirror
// pairs the two quads of each half-row and row_mirror the two half-rows, so
// after four steps every lane of the row holds the row total.

template <int CTRL> __device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm(1,0,3,2)
  x += dpp_f<0x4E>(x);   // quad_perm(2,3,0,1)
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  return x;
}

// Max / sum over the four 16-lane rows of the wave (lanes i, i^16, i^32,
// i^48), on the gfx950 row-swap instructions: with both operands holding x,
// v_permlane16_swap leaves x and its xor-16 partner in the two results (in
// one order or the other, which max and + do not mind), v_permlane32_swap
// does the same for the xor-32 partner. VALU only, no LDS round trip; the
// sum adds in the order (x0 + x16) + (x32 + x48). Every lane must be active.
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
  x = fmaxf(__builtin_bit_cast(float, (int)a[0]), __builtin_bit_cast(float, (int)a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (int)b[0]), __builtin_bit_cast(float, (int)b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
  x = __builtin_bit_cast(float, (int)a[0]) + __builtin_bit_cast(float, (int)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
  return __builtin_bit_cast(float, (int)b[0]) + __builtin_bit_cast(float, (int)b[1]);
}

// Max and sum of a float over the whole wave, every lane receiving the same
// bits: the DPP steps within each 16-lane row, then the row-swap steps.
__device__ __forceinline__ float wave_max_f(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  x = fmaxf(x, dpp_f<0x140>(x));
  return rows4_max(x);
}
__device__ __forceinline__ float wave_sum_f(float x) { return rows4_sum(row16_sum(x)); }

// Min of an int over the whole wave, every lane receiving it: DPP steps
// within each 16-lane row (as row16_sum), then the row-swap instructions
// across rows. VALU only. Every lane must be active.
__device__ __forceinline__ int wave_min_i(int x) {
  x = min(x, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xf, 0xf, false));   // quad_perm(1,0,3,2)
  x = min(x, __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xf, 0xf, false));   // quad_perm(2,3,0,1)
  x = min(x, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xf, 0xf, false));  // row_half_mirror
  x = min(x, __builtin_amdgcn_update_dpp(0, x, 0x140, 0xf, 0xf, false));  // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = min((int)a[0], (int)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return min((int)b[0], (int)b[1]);
}

// LDS byte offset of a __shared__ object
template <typename T> __device__ __forceinline__ uint32_t lds_offset(T* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from global memory straight into LDS: lane L's bytes
// land at LDS byte offset lds_off + 16 L (lds_off wave-uniform, via M0);
// the source is a wave-uniform 64-bit base in SGPRs plus a 32-bit per-lane
// byte offset, so the address adds happen in the load, not in VALU.
// Written as inline assembly so that the compiler, which waits for every
// such load before any later LDS read, leaves the waits to the kernel; the
// loads count in vmcnt like any vector load. M0 is written in the same
// assembly block as the load that reads it (one wait state between them),
// and the kernels that use it use M0 nowhere else, so clobbering a register
// the compiler does not preserve around inline assembly loses nothing.
__device__ __forceinline__ void lds_dma16s(const char* sbase, uint32_t voff, uint32_t lds_off) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(lds_off)
               : "memory", "m0");
}
// wait until none of this wave's vector loads is outstanding
__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace pa
