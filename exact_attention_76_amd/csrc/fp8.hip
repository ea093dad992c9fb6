// fp8.hip -- the FP8 e4m3 path for gfx950: the pre-pass (incoherent processing + power-of-two
// block quantisation) and the attention forward pass on e4m3 inputs.
//
// Sources: FlashAttention-3 pages, zenmind digest section 3.5 ("FP8 adaptation": block
// quantisation with one scale per block of Q, K, V; incoherent processing with a random +-1
// diagonal times a Hadamard matrix applied to Q and K; the in-kernel layout work for the second
// product), and the blog article's FP8 section (power-of-two scales, uniform inside a block;
// softmax and accumulation in fp32).
//
// gfx950 design (ours):
//   * Pre-pass: one workgroup per (tensor, batch, head, 64-token block); four lanes per token
//     row hold 32 elements each; the Walsh-Hadamard butterflies run in fp64 (five stages in
//     registers, two across the lane quad), so the rotated values are exact; the block's
//     largest magnitude picks the exponent and every element is rounded to e4m3 from its exact
//     fp64 value (fp64 -> fp32 rounded to odd, then the hardware's nearest-even conversion).
//     With rotary tables, Q and K are first embedded (fp32, rounded to bf16) in registers, so
//     the fused pre-pass reads and writes what the plain one does plus the tables.
//     Per-tensor scaling (the usual practice that block quantisation replaces) takes three
//     launches: the same kernel writes each block's exponent into its scale slot, one
//     workgroup per tensor reduces the slots to the tensor's exponent and writes its scale
//     everywhere, and the kernel runs again with that exponent.  Every scale is kept at
//     2^-126 or more, a normal fp32 whose exponent is the E8M0 operand the attention uses.
//   * Attention (dense or packed sequences, causal or not, grouped-query heads): the plain loop
//     of the 16-bit kernel (scores formed transposed, online softmax in fp32, K/V tiles copied
//     buffer-to-LDS, two LDS stages, one barrier per tile) with four waves (128 queries) per
//     workgroup and three workgroups per CU -- the softmax is the larger share here, and three
//     free-running waves per SIMD hide its latencies better than a two-stage loop or a ping-pong
//     of two waves (both measured slower on MI355X) -- and both products on
//     v_mfma_scale_f32_32x32x64_f8f6f4.  A tile's K/V scales are loaded with its
//     copy, one tile ahead, so no wait on a scale waits for a copy.  The per-block power-of-two
//     scales of Q, K and V go into the instruction's E8M0 scale operands, so they cost nothing.
//     P is quantised as e4m3 of 2^6 * P (the 2^6 rides in the exp2 argument and cancels against
//     the row sum, which is summed from the unquantised values).  V is read transposed from LDS
//     with ds_read_b64_tr_b8, the key order matching the byte order of the P operand.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include "decompose.h"
#include "internal.h"

namespace attn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ============================================================================================
// Pre-pass
// ============================================================================================

struct PrepTensor {
  const uint16_t* x;  // bf16 [B, N, H, 128]
  uint8_t* x8;        // e4m3 codes, same layout
  float* scale;       // [B, H, nblk]
  int H;
  int rotate;         // multiply by diag(signs) * Hadamard first
  int scale_shift;    // log2 of the extra divisor folded into the scale (7 for rotated K)
  int embed;          // Q or K: takes the rotary embedding when there is one
};

// fp64 -> fp32 rounded to odd: the value truncated toward zero, its last bit set when the
// conversion is inexact.  Rounding to odd at fp32's 24 bits and then to nearest even at e4m3's
// 4 bits gives the nearest-even e4m3 value of the fp64 input itself (the intermediate keeps
// more than one extra bit), so the hardware fp32 -> e4m3 conversion can finish the job.
__device__ __forceinline__ float f32_round_odd(double z) {
  const float f = (float)z;
  const double back = (double)f;
  uint32_t fb = __float_as_uint(f);
  if (back != z) fb = (fb - (fabs(back) > fabs(z) ? 1u : 0u)) | 1u;
  return __uint_as_float(fb);
}

__device__ __forceinline__ double shfl_xor_d(double x, int mask) {
  const long long v = __double_as_longlong(x);
  const int lo = __shfl_xor((int)(v & 0xffffffff), mask);
  const int hi = __shfl_xor((int)(v >> 32), mask);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// The value of lane (lane ^ M) of the same quad, M = 1 or 2: two DPP quad permutations (a
// vector-ALU move with no LDS round trip).  Every lane of the wave must be active.
template <int M>
__device__ __forceinline__ double quad_xor_d(double x) {
  static_assert(M == 1 || M == 2, "quad partner");
  constexpr int kQuadPerm = M == 1 ? 0xB1 : 0x4E;  // source lanes [1,0,3,2] / [2,3,0,1]
  const long long v = __double_as_longlong(x);
  const int lo = __builtin_amdgcn_mov_dpp((int)(v & 0xffffffff), kQuadPerm, 0xF, 0xF, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(v >> 32), kQuadPerm, 0xF, 0xF, true);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Smallest exponent of a normal fp32 scale.
constexpr int kScaleExpMin = -126;
// The smallest e with amax <= 448 * 2^e (0 for amax = 0): amax = f * 2^ex with f in [0.5, 1),
// and 448 = 0.875 * 2^9.  amax is a normal fp64 (a magnitude of a bf16 value or of a sum of
// them), so its exponent field gives ex.
__device__ __forceinline__ int block_exponent(double amax) {
  if (!(amax > 0.0)) return 0;
  const long long bits = __double_as_longlong(amax);
  const int ex = (int)((bits >> 52) & 0x7FF) - 1022;
  const long long frac = bits & 0xFFFFFFFFFFFFFLL;  // f = (1 + frac / 2^52) / 2
  return (frac <= (3LL << 50)) ? ex - 9 : ex - 8;
}

// What one launch of the pre-pass kernel does.
enum PrepPass : int {
  kPrepBlock = 0,        // per-block scaling: codes and block scales
  kPrepTensorScan = 1,   // per-tensor, first pass: each block's own exponent, as an int, into its
                         // scale slot (INT_MIN for an all-zero block); no codes
  kPrepTensorCodes = 2,  // per-tensor, last pass: codes with the exponent the slot now holds
};

// Rotary embedding of one lane's 32 features (16 interleaved pairs, pairs 16p .. 16p+15) at
// position pos: fp32 products and sums rounded one by one (no fused multiply-add), then bf16
// (nearest even) -- the tensor an unfused fp32 rotary kernel would write.
__device__ __forceinline__ void rope32(double* y, const float* __restrict__ cos_row,
                                       const float* __restrict__ sin_row) {
#pragma clang fp contract(off)
  float c[16], s[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 a = reinterpret_cast<const u32x4*>(cos_row)[i];
    const u32x4 b = reinterpret_cast<const u32x4*>(sin_row)[i];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c[4 * i + e] = __uint_as_float(a[e]);
      s[4 * i + e] = __uint_as_float(b[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float x0 = (float)y[2 * e], x1 = (float)y[2 * e + 1];  // exact: bf16 values
    const float r0 = x0 * c[e] - x1 * s[e];  // contraction is off in this function
    const float r1 = x0 * s[e] + x1 * c[e];
    const f32x2 r = {r0, r1};
    const uint32_t packed = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
    y[2 * e] = (double)__uint_as_float(packed << 16);
    y[2 * e + 1] = (double)__uint_as_float(packed & 0xFFFF0000u);
  }
}

// Dense: B sequences of N tokens.  Packed (cu != nullptr): sequence b holds tokens cu[b] ..
// cu[b+1]-1 (at most N of them), and its blocks count from its first token.  ROPE: Q and K are
// first embedded at each token's position in its sequence with the fp32 tables rope_cos,
// rope_sin [positions, 64].
template <int PASS, bool ROPE>
__global__ __launch_bounds__(256, 4) void fp8_prepare_kernel(PrepTensor t0, PrepTensor t1, PrepTensor t2, int B, int N,
                                                          int nblk, const int* __restrict__ cu,
                                                          const signed char* __restrict__ signs,
                                                          const float* __restrict__ rope_cos,
                                                          const float* __restrict__ rope_sin) {
  const PrepTensor t = blockIdx.y == 0 ? t0 : (blockIdx.y == 1 ? t1 : t2);
  const int H = t.H;
  if ((int)blockIdx.x >= B * H * nblk) return;  // this tensor has fewer heads than the grid
  const int blk = blockIdx.x % nblk;
  const int bh = blockIdx.x / nblk;
  const int h = bh % H, b = bh / H;
  const int tid = threadIdx.x;
  float* const slot = t.scale + ((int64_t)b * H + h) * nblk + blk;
  int seq_start = b * N, n = N;
  if (cu != nullptr) {
    seq_start = cu[b];
    n = min(cu[b + 1] - seq_start, N);
    if (blk * 64 >= n) {  // past the end of this sequence: no codes; the scan leaves no exponent
      if (PASS == kPrepTensorScan && tid == 0) *slot = __int_as_float(INT_MIN);
      return;
    }
  }
  const int r = tid >> 2, p = tid & 3;  // token row of the block, quarter of the 128 features
  const int token = blk * 64 + r;
  const bool valid = token < n;
  const int64_t rowoff = ((int64_t)seq_start + (valid ? token : 0)) * H + h;

  u32x4 raw[4];  // this lane's 32 bf16 values, as loaded
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(t.x + rowoff * 128 + 32 * p);
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[c] = valid ? src[c] : u32x4{0, 0, 0, 0};
  }
  // value i (exact in fp32) of the lane's 32
  auto bf16_at = [&](int i) {
    const uint32_t w = raw[i >> 3][(i >> 1) & 3];
    return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
  };
  // Without rotation or rotary embedding (V always; Q and K when no signs are given) the values
  // stay the bf16 inputs: exact in fp32, and so is their scaling by 2^-e except where the
  // product falls below fp32's normal range, far under half of e4m3's smallest step (2^-10), so
  // the nearest-even e4m3 conversion of the fp32 product gives the code of the exact value.
  // Uniform per workgroup.
  auto narrow_path = [&]() {
    int e;
    if constexpr (PASS == kPrepTensorCodes) {
      e = (int)((__float_as_uint(*slot) >> 23) & 0xFF) - 127 + t.scale_shift;
    } else {
      float amax = 0.f;
      if (valid) {
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(bf16_at(i)));
      }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m));
      __shared__ float wmaxf[4];
      if ((tid & 63) == 0) wmaxf[tid >> 6] = amax;
      __syncthreads();
      amax = fmaxf(fmaxf(wmaxf[0], wmaxf[1]), fmaxf(wmaxf[2], wmaxf[3]));
      e = block_exponent((double)amax);
      if constexpr (PASS == kPrepTensorScan) {
        if (tid == 0) *slot = __int_as_float(amax > 0.f ? e : INT_MIN);
        return;
      }
      e = max(e, t.scale_shift + kScaleExpMin);
    }
    // 2^-e as fp32: e lies in [kScaleExpMin + shift, 128] here, so 2^-e is a normal fp32
    const float inv = __uint_as_float((uint32_t)(127 - e) << 23);
    if (valid) {
      uint32_t w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // fma(x, 2^-e, +0): the exact product, an exact -0 turned into +0 (a zero encodes as +0)
        const float f0 = __builtin_fmaf(bf16_at(4 * j), inv, 0.0f);
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f0, __builtin_fmaf(bf16_at(4 * j + 1), inv, 0.0f), __float_as_int(f0), false);
        w[j] = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_fmaf(bf16_at(4 * j + 2), inv, 0.0f),
                                               __builtin_fmaf(bf16_at(4 * j + 3), inv, 0.0f), lo, true);
      }
      u32x4* dst = reinterpret_cast<u32x4*>(t.x8 + rowoff * 128 + 32 * p);
      dst[0] = u32x4{w[0], w[1], w[2], w[3]};
      dst[1] = u32x4{w[4], w[5], w[6], w[7]};
    }
    if constexpr (PASS == kPrepBlock) {
      if (tid == 0) *slot = __uint_as_float((uint32_t)(e - t.scale_shift + 127) << 23);
    }
  };
  // (the test reads an opaque copy of the rotate flag: knowing the flag set on the path below,
  // the compiler merged that path into one scheduling region that held twice the registers)
  int rotate = t.rotate;
  asm volatile("" : "+s"(rotate));
  if (!rotate && !(ROPE && t.embed)) {
    narrow_path();
    return;
  }
  double y[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) y[i] = (double)bf16_at(i);
  if constexpr (ROPE) {
    if (t.embed) {
      const int64_t row = (int64_t)(valid ? token : 0) * 64 + 16 * p;
      rope32(y, rope_cos + row, rope_sin + row);
    }
  }
  if (t.rotate) {
    {
      // this lane's 32 sign bytes as two 16-byte words (each +1 or -1: bit 7 is the sign),
      // applied to the doubles' sign bits
      const u32x4* sp = reinterpret_cast<const u32x4*>(signs + 32 * p);
      const u32x4 s0 = sp[0], s1 = sp[1];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const uint32_t word = (i < 16 ? s0 : s1)[(i & 15) >> 2];
        const uint32_t neg = (word >> (8 * (i & 3) + 7)) & 1u;
        y[i] = __longlong_as_double(__double_as_longlong(y[i]) ^ ((long long)neg << 63));
      }
    }
    // Walsh-Hadamard butterflies (a, b) -> (a + b, a - b) at strides 1 .. 64 over the 128
    // features give y H with H[i][j] = (-1)^popcount(i & j); strides below 32 stay in a lane.
#pragma unroll
    for (int hs = 1; hs < 32; hs <<= 1)
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if ((i & hs) == 0) {
          const double a = y[i], c = y[i + hs];
          y[i] = a + c;
          y[i + hs] = a - c;
        }
    // strides 32 and 64: partner lane p ^ 1, then p ^ 2, in the same quad.  The lower lane
    // keeps a + b and the upper lane a - b, each as fma(+-1, own, partner): one rounding, the
    // same as the add or subtract.
    auto cross = [&](auto xchg, int m) {
      const double sg = (p & m) ? -1.0 : 1.0;
      // eight values at a time, so that the partner values of all 32 are not held at once
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int i = 8 * c; i < 8 * c + 8; ++i) y[i] = __builtin_fma(sg, y[i], xchg(y[i]));
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    cross([](double x) { return quad_xor_d<1>(x); }, 1);
    cross([](double x) { return quad_xor_d<2>(x); }, 2);
  }
  int e;
  if constexpr (PASS == kPrepTensorCodes) {
    e = (int)((__float_as_uint(*slot) >> 23) & 0xFF) - 127 + t.scale_shift;  // slot holds 2^(e - shift)
  } else {
    // block amax (exact, fp64)
    double amax = 0.0;
    if (valid) {
#pragma unroll
      for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(y[i]));
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) amax = fmax(amax, shfl_xor_d(amax, m));
    __shared__ double wmax[4];
    if ((tid & 63) == 0) wmax[tid >> 6] = amax;
    __syncthreads();
    amax = fmax(fmax(wmax[0], wmax[1]), fmax(wmax[2], wmax[3]));
    e = block_exponent(amax);
    if constexpr (PASS == kPrepTensorScan) {
      if (tid == 0) *slot = __int_as_float(amax > 0.0 ? e : INT_MIN);
      return;
    }
    e = max(e, t.scale_shift + kScaleExpMin);  // the scale 2^(e - shift) stays a normal fp32
  }
  const double inv = __longlong_as_double((long long)(1023 - e) << 52);  // 2^-e, exact
  if (valid) {
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // |y| * 2^-e <= 448 by the choice of e, so the conversions never saturate.  The + 0.0f
      // turns an exact -0 into +0 (an exact zero encodes as +0) and leaves every nonzero value,
      // fp32 subnormals included (denormals are kept), as it is.
      const float f0 = f32_round_odd(y[4 * j] * inv) + 0.0f;
      const int lo =
          __builtin_amdgcn_cvt_pk_fp8_f32(f0, f32_round_odd(y[4 * j + 1] * inv) + 0.0f, __float_as_int(f0), false);
      w[j] = __builtin_amdgcn_cvt_pk_fp8_f32(f32_round_odd(y[4 * j + 2] * inv) + 0.0f,
                                             f32_round_odd(y[4 * j + 3] * inv) + 0.0f, lo, true);
    }
    u32x4* dst = reinterpret_cast<u32x4*>(t.x8 + rowoff * 128 + 32 * p);
    dst[0] = u32x4{w[0], w[1], w[2], w[3]};
    dst[1] = u32x4{w[4], w[5], w[6], w[7]};
  }
  if constexpr (PASS == kPrepBlock) {
    if (tid == 0) *slot = __uint_as_float((uint32_t)(e - t.scale_shift + 127) << 23);
  }
}

// Per-tensor scaling, middle pass: one workgroup per tensor takes the largest block exponent
// left in its scale slots by the scan pass (an all-zero tensor gets 0), raises it to the
// floor, and writes the tensor's scale into every slot.  Every slot is read before the
// barrier inside the reduction and written after it.
__global__ __launch_bounds__(1024) void fp8_tensor_scale_kernel(PrepTensor t0, PrepTensor t1, PrepTensor t2, int B,
                                                                int nblk) {
  const PrepTensor t = blockIdx.x == 0 ? t0 : (blockIdx.x == 1 ? t1 : t2);
  const int64_t n = (int64_t)B * t.H * nblk;
  int m = INT_MIN;
  for (int64_t i = threadIdx.x; i < n; i += 1024) m = max(m, __float_as_int(t.scale[i]));
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) m = max(m, __shfl_xor(m, s));
  __shared__ int wmax[16];
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  m = wmax[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) m = max(m, wmax[w]);
  const int e = max(m == INT_MIN ? 0 : m, t.scale_shift + kScaleExpMin);
  const float scale = __uint_as_float((uint32_t)(e - t.scale_shift + 127) << 23);
  for (int64_t i = threadIdx.x; i < n; i += 1024) t.scale[i] = scale;
}

// ============================================================================================
// Attention on e4m3 inputs
// ============================================================================================

constexpr int kD = 128;  // head dim (bytes per row of an e4m3 tile)

// LDS tile layout: blocks of 16 rows, chunk-major inside a block (16-byte chunks), rows inside
// a chunk column XOR-ed with 4*(chunk & 1).  Conflict free for 16-lane b128 reads of one chunk
// (K) and for 32-lane ds_read_b64_tr_b8 reads of 8 rows x 32 bytes (V).
__device__ __forceinline__ void f8_tile_row_chunk(int p, int& row, int& chunk) {
  const int blk = p >> 7, o = p & 127;
  chunk = o >> 4;
  row = 16 * blk + ((o & 15) ^ (4 * (chunk & 1)));
}

template <int NI>
__device__ __forceinline__ void copy_rows_to_lds8(const char* base, int nbytes, char* lds_dst, const int* voff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, nbytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < NI; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(void, lds_dst + 1024 * i), 16, voff[i], 0, 0, 0);
#endif
}

__device__ __forceinline__ f32x16 mma_f8(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  // format 0 = e4m3 for both operands; sa / sb are E8M0 power-of-two scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ int e8m0_of(float pow2) { return (int)((__float_as_uint(pow2) >> 23) & 0xFF); }

__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// P is quantised as e4m3(2^kPExp * P); with a row maximum at most kRescaleSlack (exp2 domain)
// above the stabiliser, 2^kPExp * P <= 2^(kPExp + kRescaleSlack) <= 448.
constexpr int kPExp = 6;
constexpr float kRescaleSlack = 2.75f;
static_assert(kPExp + kRescaleSlack <= 8.807f, "2^(kPExp + kRescaleSlack) must not exceed 448 = 2^8.807");

// WAVES waves of 32 queries per workgroup; BC keys per tile (64 or 128, a multiple of the
// 64-token scale block).  CAUSAL: key j visible to query i iff j <= i.  VARLEN: packed sequences
// [T, H, d] delimited by cu_seqlens, scale blocks counted from each sequence's first token.
// WINDOW (implies CAUSAL): query i sees keys i-window+1 .. i only.
// One stage per tile: two K/V buffers, one barrier per tile; with four waves per workgroup three
// workgroups share a CU (three waves per SIMD), and co-resident waves interleave freely.
template <int WAVES, int BC, bool CAUSAL, bool VARLEN, bool WINDOW>
__global__ __launch_bounds__(64 * WAVES, (WAVES == 4 ? 3 : 1)) void fwd_fp8_kernel(
    const uint8_t* __restrict__ q, const uint8_t* __restrict__ k, const uint8_t* __restrict__ v,
    const float* __restrict__ qs, const float* __restrict__ ks_, const float* __restrict__ vs_,
    uint16_t* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, int N, const int* __restrict__ cu_seqlens,
    int nseq, float alpha, int num_qblocks, int window) {
  constexpr int BR = 32 * WAVES;        // queries per workgroup
  constexpr int TILE = BC * kD;         // bytes of one K or V tile
  constexpr int NI = TILE / 1024 / WAVES;  // 1 KB copies per wave per tensor
  constexpr int NB_C = BC / 32;         // 32-key score blocks per tile
  constexpr int KS = BC / 64;           // 64-key k-steps of the second product
  static_assert(BC % 64 == 0 && NI >= 1 && NI * WAVES * 1024 == TILE, "tile shape");
  __shared__ __attribute__((aligned(1024))) char st0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) char st1[2 * TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int nblk = (N + 63) / 64;

  int qb, h, b;
  decompose<CAUSAL>(blockIdx.x, num_qblocks, Hq, Hkv, nseq, qb, h, b);
  int seq_start, n;
  if constexpr (VARLEN) {
    seq_start = cu_seqlens[b];
    n = cu_seqlens[b + 1] - seq_start;
    if (n > N) n = N;
  } else {
    seq_start = b * N;
    n = N;
  }
  const int q0 = qb * BR;
  const int g = h / (Hq / Hkv);
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;
  if (q0 >= n) return;

  // Q fragment: query qi, bytes 64*st + 32*hi .. +31
  i32x8 qf[2];
  {
    const int row = qi < n ? qi : n - 1;
    const u32x4* qp = reinterpret_cast<const u32x4*>(q + ((int64_t)(seq_start + row) * Hq + h) * kD + 32 * hi);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x4 a = qp[4 * s], c = qp[4 * s + 1];
      qf[s] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)c[0], (int)c[1], (int)c[2], (int)c[3]};
    }
  }
  const int qblock = (qw < n ? qw : n - 1) / 64;
  const int sq = e8m0_of(qs[((int64_t)b * Hq + h) * nblk + qblock]);
  const float* ksc = ks_ + ((int64_t)b * Hkv + g) * nblk;
  const float* vsc = vs_ + ((int64_t)b * Hkv + g) * nblk;

  const int rowbytes = Hkv * kD;
  int voff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    int row, chunk;
    f8_tile_row_chunk((wave * NI + i) * 64 + lane, row, chunk);
    voff[i] = row * rowbytes + chunk * 16;
  }
  const char* kbase = reinterpret_cast<const char*>(k) + ((int64_t)seq_start * Hkv + g) * kD;
  const char* vbase = reinterpret_cast<const char*>(v) + ((int64_t)seq_start * Hkv + g) * kD;
  const int nbytes = (n - 1) * rowbytes + kD;
  // Raw K and V scales of one tile (one per 64-key block).  A tile's scales are loaded just
  // before its copies are issued and read only after the wait that ends the previous tile, so
  // no wait on a scale load also waits for a tile copy still in flight.
  struct TileScales {
    float k[KS], v[KS];
  };
  auto issue_tile = [&](char* stage, int tile, TileScales& sc) {
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      const int blk = min(tile * (BC / 64) + i, nblk - 1);
      sc.k[i] = ksc[blk];
      sc.v[i] = vsc[blk];
    }
    const int off = tile * BC * rowbytes;
    copy_rows_to_lds8<NI>(kbase + off, nbytes - off, stage + wave * NI * 1024, voff);
    copy_rows_to_lds8<NI>(vbase + off, nbytes - off, stage + TILE + wave * NI * 1024, voff);
  };

  // K operand: row 32*cb + l32, chunks 4*st + 2*hi + e (e = 0, 1)
  int koff[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) koff[e] = 16 * ((l32 >> 4) * 128 + (2 * hi + e) * 16 + ((lane & 15) ^ (4 * e)));
  // V operand by transpose reads: lane 16G + 2r + c reads 8 bytes (half c) of row
  // 64*ks + 16u + 4*(G/2) + 8*(r/4) + r%4, chunk 2*db + (G%2)
  int vtoff;
  {
    const int G = lane >> 4, r = (lane >> 1) & 7, c = lane & 1;
    const int rowm = 4 * (G >> 1) + 8 * (r >> 2) + (r & 3);
    vtoff = 16 * ((G & 1) * 16 + (rowm ^ (4 * (G & 1)))) + 8 * c;
  }

  f32x16 oacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) oacc[i] = f32x16{};
  float m = -INFINITY;
  float l = 0.f;
  const float c = alpha * kLog2e;
  // derived from m, updated only when m changes: the rescale threshold in units of the scores
  // (m + kRescaleSlack / c; -inf while m is) and the exp2 offset m c - kPExp (m = -inf counts as
  // 0, so fully masked rows give exp2(-inf) = 0 rather than NaN)
  float thr = -INFINITY;
  float mc = -(float)kPExp;
  const float slack_s = kRescaleSlack / c;
  const int kv_end = CAUSAL ? min(n, q0 + BR) : n;  // keys any query of the workgroup sees
  static_assert(!WINDOW || CAUSAL, "a sliding window is causal");
  // the loop counts tiles from t0, the first one any query of the workgroup sees
  const int t0 = WINDOW ? max(0, q0 - window + 1) / BC : 0;
  const int ntiles = (kv_end + BC - 1) / BC - t0;
  auto wave_needs = [&](int j) {  // this wave sees a key of loop tile j
    const int k0 = (t0 + j) * BC;
    return !CAUSAL || (k0 <= qw + 31 && (!WINDOW || k0 + BC - 1 > qw - window));
  };

  // first product of loop tile j: S^T = K Q^T from the K half of its buffer; the two 32-key
  // blocks alternate, so consecutive matrix instructions do not depend on each other
  auto gemm1 = [&](const char* stage, const TileScales& sc, f32x16* s) {
    const char* kt = stage;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int cb = 0; cb < NB_C; ++cb) {
        const int sk = e8m0_of(sc.k[cb >> 1]);
        if (st == 0) s[cb] = f32x16{};
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(kt + koff[0] + cb * 4096 + st * 1024);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(kt + koff[1] + cb * 4096 + st * 1024);
        const i32x8 a = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        s[cb] = mma_f8(a, qf[st], s[cb], sk, sq);
      }
  };
  // mask and online softmax of loop tile j (scores s), packed into the e4m3 B operands pf of the
  // second product
  auto softmax = [&](int j, f32x16* s, i32x8* pf) {
    const int k0 = (t0 + j) * BC;
    if (k0 + BC > n || (CAUSAL && (k0 + BC - 1 > qw || (WINDOW && k0 <= qw + 31 - window)))) {
#pragma unroll
      for (int cb = 0; cb < NB_C; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + cb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if constexpr (WINDOW) {  // visible iff 0 <= qi - key < window (one unsigned compare)
            if (key >= n || (unsigned)(qi - key) >= (unsigned)window) s[cb][r] = -INFINITY;
          } else {
            if (key >= n || (CAUSAL && key > qi)) s[cb][r] = -INFINITY;
          }
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int cb = 0; cb < NB_C; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[cb][r]);
    // P' = 2^kPExp * exp2((s - m) c) must stay at or below 448 (largest e4m3): rescale once some
    // row's maximum exceeds the stabiliser by more than kRescaleSlack in the exp2 domain
    // (2^(6 + 2.75) = 430.5; the 0.057 left to 448 = 2^8.807 covers the rounding of thr).  A
    // smaller kPExp leaves more slack, so rescales are rarer.  The test needs no row maximum:
    // some lane's maximum over its half of the keys exceeds the threshold exactly when some
    // row's does.  The branch is uniform, so the lane swap is safe.
    if (__builtin_amdgcn_ballot_w64(mt > thr)) {
      mt = halves_max(mt);
      const float mnew = fmaxf(m, mt);
      const float corr = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - mnew) * c);
      m = mnew;
      l *= corr;
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] *= corr;
      thr = m + slack_s;
      mc = ((m == -INFINITY) ? 0.f : m * c) - (float)kPExp;
    }
    float rs0 = -0.f, rs1 = -0.f;  // -0 + p = p exactly, so the first adds fold away
#pragma unroll
    for (int cb = 0; cb < NB_C; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[cb][r], c, -mc));
        s[cb][r] = p;
        if (r & 1) rs1 += p; else rs0 += p;
      }
    l += rs0 + rs1;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      // P'^T as the B operand of k-step kk: byte 16*cb' + r holds register r of block 2*kk + cb'
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int cb = 2 * kk + (w >> 2), r0 = 4 * (w & 3);
        // the first conversion writes the low half of the word and keeps the rest of its old
        // input, which the second conversion overwrites: any old value will do, and the first
        // source (dead after this instruction) costs no register initialisation
        const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(s[cb][r0], s[cb][r0 + 1], __float_as_int(s[cb][r0]), false);
        pf[kk][w] = __builtin_amdgcn_cvt_pk_fp8_f32(s[cb][r0 + 2], s[cb][r0 + 3], lo, true);
      }
    }
  };
  // V^T operand of the second product for k-step kk and 32-row d block db, by transpose reads
  auto v_operand = [&](const char* vt, int kk, int db) {
    i32x8 a;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const i32x2 t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_PTR(i32x2, vt + vtoff + kk * 8192 + u * 2048 + db * 512));
      a[2 * u] = t[0];
      a[2 * u + 1] = t[1];
    }
    return a;
  };
  // second product of a tile: O^T += V^T P'^T from the V tile at vt
  auto gemm2 = [&](const char* vt, const TileScales& sc, const i32x8* pf) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int sv = e8m0_of(sc.v[kk]);
#pragma unroll
      for (int db = 0; db < 4; ++db) oacc[db] = mma_f8(v_operand(vt, kk, db), pf[kk], oacc[db], sv, 127);
    }
  };
  auto softmax_gemm2 = [&](const char* stage, int j, const TileScales& sc, f32x16* s) {
    i32x8 pf[KS];
    softmax(j, s, pf);
    gemm2(stage + TILE, sc, pf);
  };

  // The Q fragment must have arrived before the loop: loads still in flight at its entry would
  // make every iteration wait for all vector memory operations, the tile copies included.
  asm volatile("" ::"v"(qf[0]), "v"(qf[1]));
  // causal: a wave skips the tiles that lie wholly above its diagonal or before its window; it
  // still copies and waits.  A lane whose keys in a tile are all masked keeps m = -inf and adds
  // nothing (P = exp2(-inf) = 0).
  TileScales sc0, sc1;  // scales of the tiles in st0 and st1
  issue_tile(st0, t0, sc0);
  sc1 = sc0;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 s[NB_C];
  for (int j = 0; j < ntiles; j += 2) {
    if (j + 1 < ntiles) issue_tile(st1, t0 + j + 1, sc1);
    if (wave_needs(j)) {
      gemm1(st0, sc0, s);
      softmax_gemm2(st0, j, sc0, s);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 >= ntiles) break;
    if (j + 2 < ntiles) issue_tile(st0, t0 + j + 2, sc0);
    if (wave_needs(j + 1)) {
      gemm1(st1, sc1, s);
      softmax_gemm2(st1, j + 1, sc1, s);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  const float lt = halves_sum(l);
  if (qi < n) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* op = o + ((int64_t)(seq_start + qi) * Hq + h) * kD + 4 * hi;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        u32x2 pr = {pack_bf16x2(oacc[db][4 * gq + 0] * inv, oacc[db][4 * gq + 1] * inv),
                    pack_bf16x2(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + db * 32 + gq * 8) = pr;
      }
    if (hi == 0) {
      // l carries the factor 2^kPExp of P'
      const int64_t idx = VARLEN ? (int64_t)h * cu_seqlens[nseq] + seq_start + qi : ((int64_t)b * Hq + h) * N + qi;
      lse[idx] = lt > 0.f ? m * alpha + __logf(lt) - (float)kPExp * kLn2 : -INFINITY;
    }
  }
}

#ifndef ATTN_FP8_SHAPE
#define ATTN_FP8_SHAPE 4, 64
#endif

}  // namespace

template <bool ROPE>
hipError_t launch_prepare_passes(const PrepareArgs& a, hipStream_t stream) {
  const int nblk = (a.N + 63) / 64;
  // Q and K take the rotary embedding (if any) and the Hadamard rotation (if signs are given)
  const bool rot = a.signs != nullptr;
  PrepTensor tq{static_cast<const uint16_t*>(a.q), static_cast<uint8_t*>(a.q8), a.q_scale, a.Hq, rot, 0, 1};
  PrepTensor tk{static_cast<const uint16_t*>(a.k), static_cast<uint8_t*>(a.k8), a.k_scale, a.Hkv, rot, rot ? 7 : 0, 1};
  PrepTensor tv{static_cast<const uint16_t*>(a.v), static_cast<uint8_t*>(a.v8), a.v_scale, a.Hkv, 0, 0, 0};
  const long long grid = (long long)a.B * a.Hq * nblk;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid, 3);
  if (!a.per_tensor) {
    hipLaunchKernelGGL((fp8_prepare_kernel<kPrepBlock, ROPE>), g, dim3(256), 0, stream, tq, tk, tv, a.B, a.N, nblk,
                       a.cu_seqlens, a.signs, a.rope_cos, a.rope_sin);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((fp8_prepare_kernel<kPrepTensorScan, ROPE>), g, dim3(256), 0, stream, tq, tk, tv, a.B, a.N, nblk,
                     a.cu_seqlens, a.signs, a.rope_cos, a.rope_sin);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(fp8_tensor_scale_kernel, dim3(3), dim3(1024), 0, stream, tq, tk, tv, a.B, nblk);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((fp8_prepare_kernel<kPrepTensorCodes, ROPE>), g, dim3(256), 0, stream, tq, tk, tv, a.B, a.N,
                     nblk, a.cu_seqlens, a.signs, a.rope_cos, a.rope_sin);
  return hipGetLastError();
}

hipError_t launch_fp8_prepare(const PrepareArgs& a, hipStream_t stream) {
  return a.rope_cos != nullptr ? launch_prepare_passes<true>(a, stream) : launch_prepare_passes<false>(a, stream);
}

template <bool CAUSAL, bool VARLEN, bool WINDOW = false>
hipError_t launch_fp8_mode(const FwdArgs& a, hipStream_t stream) {
  constexpr int kWaves = [] { int w[] = {ATTN_FP8_SHAPE}; return w[0]; }();
  const int br = 32 * kWaves;
  const int nqb = (a.N + br - 1) / br;
  const long long grid = (long long)nqb * a.Hq * a.B;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_fp8_kernel<ATTN_FP8_SHAPE, CAUSAL, VARLEN, WINDOW>), dim3((unsigned)grid), dim3(64 * kWaves), 0,
                     stream, static_cast<const uint8_t*>(a.q), static_cast<const uint8_t*>(a.k),
                     static_cast<const uint8_t*>(a.v), a.q_scale, a.k_scale, a.v_scale,
                     static_cast<uint16_t*>(a.o), a.lse, a.Hq, a.Hkv, a.N, a.cu_seqlens, a.B, a.alpha, nqb, a.window);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t stream) {
  const bool varlen = a.cu_seqlens != nullptr;
  if (a.window > 0)
    return varlen ? launch_fp8_mode<true, true, true>(a, stream) : launch_fp8_mode<true, false, true>(a, stream);
  if (a.causal) return varlen ? launch_fp8_mode<true, true>(a, stream) : launch_fp8_mode<true, false>(a, stream);
  return varlen ? launch_fp8_mode<false, true>(a, stream) : launch_fp8_mode<false, false>(a, stream);
}

}  // namespace attn
