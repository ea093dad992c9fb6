// tile16.h -- device helpers shared by the 16-bit attention kernels (forward and backward):
// vector types, the 32x32x16 matrix instruction, 16-bit packing, lane-half reductions, the LDS
// tile layout of a K/V (or Q/dO) tile and the buffer-to-LDS copies that produce it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

template <bool BF16>
__device__ __forceinline__ f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Two fp32 values to a packed pair of 16-bit values (round to nearest even).
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  f32x2 v = {lo, hi};
  if constexpr (BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  }
}

// Reductions across the two 32-lane halves of a wave64 (lane l pairs with l ^ 32): after
// v_permlane32_swap on two copies of x, element 0 holds the low half's value and element 1
// the high half's value of every lane pair.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- LDS tile layout -------------------------------------------------------------------------
// A K or V tile of BC rows x D columns (16-bit) is stored as blocks of 16 rows; inside a block
// the 16-byte chunks are chunk-major (chunk c of the 16 rows is contiguous) and the row order
// inside a chunk column is XOR-ed with 4*(c mod 4).  With 64 LDS banks this makes both operand
// reads conflict free: a b128 read of one chunk by 16 lanes (16 rows of K) and a b64
// transpose read of 4 rows x 16 columns by 16 or 32 lanes (V).  The buffer-to-LDS copies write
// 64 consecutive 16-byte positions per instruction, so the layout is produced by choosing, per
// lane, which (row, chunk) of global memory it fetches.
template <int D>
__device__ __forceinline__ int tile_pos(int row, int chunk) {
  constexpr int NCH = D / 8;
  return (row >> 4) * 16 * NCH + chunk * 16 + ((row & 15) ^ (4 * (chunk & 3)));
}
template <int D>
__device__ __forceinline__ void tile_row_chunk(int p, int& row, int& chunk) {
  constexpr int NCH = D / 8;
  const int blk = p / (16 * NCH), o = p % (16 * NCH);
  chunk = o >> 4;
  row = 16 * blk + ((o & 15) ^ (4 * (chunk & 3)));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// ---- buffer-to-LDS copies ------------------------------------------------------------------
// One copy moves 16 bytes per lane from byte offset voff of the buffer [base, base + nbytes)
// to lds + 16*lane; offsets at or past nbytes read as zero.  In the tile layout, the NI copies
// a wave issues for one tile fetch, per lane, row(0) + 16*(i / IPB) and chunk(0) + 4*(i % IPB)
// (IPB copies fill one 16-row block), so copy i's lane offset is
// voff + (i / IPB) * blk_bytes + 64 * (i % IPB).  The extra offset goes into the lane offset,
// not the instruction's immediate offset, which would also move the LDS destination.  (The
// buffer resource type exists only in the device pass; the host pass sees empty bodies.)
template <int I, int NI, int IPB>
struct CopyRows {
  template <typename R>
  static __device__ __forceinline__ void run(R r, char* lds_dst, int voff, int blk_bytes) {
    if constexpr (I < NI) {
#if defined(__HIP_DEVICE_COMPILE__)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(void, lds_dst + 1024 * I), 16,
                                               voff + (I / IPB) * blk_bytes + 64 * (I % IPB), 0, 0, 0);
#endif
      CopyRows<I + 1, NI, IPB>::run(r, lds_dst, voff, blk_bytes);
    }
  }
};

template <int NI, int IPB>
__device__ __forceinline__ void copy_rows_to_lds(const char* base, int nbytes, char* lds_dst, int voff,
                                                 int blk_bytes) {
#if defined(__HIP_DEVICE_COMPILE__)
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, nbytes, 0x00020000);
  CopyRows<0, NI, IPB>::run(r, lds_dst, voff, blk_bytes);
#endif
}

}  // namespace
}  // namespace attn
