// Device helpers shared by the kernels of the Token Radius Attention library
// (tra_kernels.hip, tra_dense.hip): vector types, LDS access forms, wave
// reductions and the range-checked global -> LDS DMA.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

#define TRA_NEG_INF (-__builtin_inff())

__device__ __forceinline__ float bf16_to_float(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Integer square root floor(sqrt(x)) for 0 <= x < 2^31.  The hardware square
// root (v_sqrt_f32, about 1 ulp) of float(x) (exact below 2^24, within 2^-24
// relative above) lands within 0.02 of sqrt(x), so its truncation is off by at
// most one either way, and one exact integer correction in each direction
// gives the floor.
__device__ __forceinline__ int isqrt_i(int x) {
  // r <= 46341 here, so r*r and (r+1)*(r+1) stay below 2^31 + 2^17 and are
  // compared as unsigned 32-bit values.
  unsigned r = static_cast<unsigned>(__builtin_amdgcn_sqrtf(static_cast<float>(x)));
  const unsigned ux = static_cast<unsigned>(x);
  r -= (r * r > ux);
  r += ((r + 1) * (r + 1) <= ux);
  return static_cast<int>(r);
}

// XOR swizzle of 16-byte chunks in an LDS tile whose rows are NCH chunks wide.
// Rows 0..15 map chunk c to distinct banks for both the 16-byte MFMA operand
// reads (16 rows, same chunk) and the transposing 8-byte reads (4 consecutive
// rows, 2 adjacent chunks).
template <int NCH>
__device__ __forceinline__ int swz(int r) {
  if constexpr (NCH == 16) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    return ((r & 3) << 1) | ((r >> 2) & 1);
  }
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane 4r + j supplies the address of 4 consecutive bf16 (row r, columns
// 4j..4j+3 of a 4 x 16 block); lane i of the group receives column i of rows
// 0..3.  elem_off is in elements.  Results stay packed: element-wise access
// to bf16 vectors is avoided throughout (whole-vector bit casts only).
__device__ __forceinline__ uint2 lds_read_tr(const uint16_t* base, int elem_off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)((__attribute__((address_space(3))) char*)(base) + elem_off * 2)));
}

// Transposing LDS read at a byte address.
__device__ __forceinline__ uint2 lds_read_tr_b(const char* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)((__attribute__((address_space(3))) char*)(p))));
}

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Wave-wide min / max with a wave-uniform result: DPP inside rows of 16, then
// the four row results combined through readlane.
__device__ __forceinline__ int wave_min_u(int v) {
  v = min(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false));
  v = min(v, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ int wave_max_u(int v) {
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false));
  v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));
  return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
// Wave-wide OR with a wave-uniform result (same DPP pattern).
__device__ __forceinline__ uint32_t wave_or_u(uint32_t v) {
  v |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false));
  v |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false));
  v |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x124, 0xF, 0xF, false));
  v |= static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xF, 0xF, false));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 0) |
                               __builtin_amdgcn_readlane(static_cast<int>(v), 16) |
                               __builtin_amdgcn_readlane(static_cast<int>(v), 32) |
                               __builtin_amdgcn_readlane(static_cast<int>(v), 48));
}
__device__ __forceinline__ uint64_t wave_or_u64(uint64_t v) {
  return (static_cast<uint64_t>(wave_or_u(static_cast<uint32_t>(v >> 32))) << 32) |
         wave_or_u(static_cast<uint32_t>(v));
}
// Wave-wide sum with a wave-uniform result (same DPP pattern: pairs, quads,
// then rotations by 4 and 8 inside each row of 16).
__device__ __forceinline__ int wave_sum_u(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);
  return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) + __builtin_amdgcn_readlane(v, 32) +
         __builtin_amdgcn_readlane(v, 48);
}
// Exclusive prefix sum over the wave's lanes; *total receives the wave sum.
__device__ __forceinline__ int wave_excl_scan(int v, int lane, int* total) {
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  *total = __builtin_amdgcn_readlane(x, 63);
  return x - v;
}

// Workgroup barrier for LDS hand-offs: this wave's LDS reads are complete
// (lgkmcnt(0)) before it arrives.  Unlike __syncthreads() it carries no
// release fence, so it does not wait for this wave's outstanding DMA loads into
// the other buffer; those are ordered by wait_vmcnt before the next barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16-byte global -> LDS DMA (buffer_load_dwordx4 ... lds): lane l's 16 bytes
// land at LDS byte address lds_base + 16*l (lds_base wave-uniform, through
// M0).  Issued from inline assembly so that the compiler's wait-count
// insertion does not treat every later LDS read as dependent on it; the kernel
// orders the hand-off itself with wait_vmcnt + lds_barrier.  The instruction
// has no register results; one wait state separates the M0 write from its use.
typedef int i32x4 __attribute__((ext_vector_type(4)));
// Raw buffer resource over [base, base + bytes): reads at offsets >= bytes
// return zero.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a)));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
  r[3] = 0x00020000;
  return r;
}
// Lane l's 16 bytes at byte offset `off` of the resource (range-checked per
// lane) go to LDS lds_base + 16*l.
__device__ __forceinline__ void lds_dma16_buf(i32x4 rsrc, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(rsrc), "s"(lds_base)
               : "memory", "m0");
}

// The same with 4 bytes per lane (lane l's dword goes to lds_base + 4*l).
__device__ __forceinline__ void lds_dma4_buf(i32x4 rsrc, uint32_t off, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(rsrc), "s"(lds_base)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left unconstrained)
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

}  // namespace tra
