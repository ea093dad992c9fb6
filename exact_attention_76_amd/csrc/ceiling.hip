// ceiling.hip -- measurement only, built into its own library (libceiling.so), not part of
// the attention path: the sustained rate of the bf16 matrix instruction the attention
// kernels use (v_mfma_f32_32x32x16_bf16) on random operands, with no LDS traffic and no
// vector-ALU work around it.  Under a power limit this rate, not the nominal peak, is the
// ceiling the attention kernels run against: data-dependent switching power decides the
// clock once every CU issues matrix instructions.
//
// Each wave holds 8 random A and 8 random B operands (read once from a buffer of 65536
// operands) and rotates them through four independent accumulators, so consecutive
// instructions never repeat their inputs and never wait on each other's results.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kOperands = 65536;  // bf16x8 operands in the source buffer

__global__ __launch_bounds__(256) void mfma_ceiling_kernel(const bf16x8* __restrict__ src, float* __restrict__ sink,
                                                           int iters) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = src[(t * 16 + i) & (kOperands - 1)];
    b[i] = src[(t * 16 + 8 + i) & (kOperands - 1)];
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; i += 4) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[(i + 3) & 7], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i + 1], b[(i + 5) & 7], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i + 2], b[(i + 1) & 7], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i + 3], b[(i + 6) & 7], c3, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[t] = s;  // keeps the products live
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// The same for the e4m3 instruction the FP8 attention kernel uses
// (v_mfma_scale_f32_32x32x64_f8f6f4, unit E8M0 scales): 8 random A and 8 random B operands of
// 32 e4m3 codes per lane, rotated through four accumulators.
__global__ __launch_bounds__(256) void mfma_ceiling_fp8_kernel(const i32x8* __restrict__ src, float* __restrict__ sink,
                                                               int iters) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  i32x8 a[8], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = src[(t * 16 + i) & (kOperands / 2 - 1)];
    b[i] = src[(t * 16 + 8 + i) & (kOperands / 2 - 1)];
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; i += 4) {
      c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[(i + 3) & 7], c0, 0, 0, 0, 127, 0, 127);
      c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i + 1], b[(i + 5) & 7], c1, 0, 0, 0, 127, 0, 127);
      c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i + 2], b[(i + 1) & 7], c2, 0, 0, 0, 127, 0, 127);
      c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i + 3], b[(i + 6) & 7], c3, 0, 0, 0, 127, 0, 127);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[t] = s;
}

}  // namespace

// src: device buffer of 32768 operands of 32 e4m3 codes (1 MiB, no NaN codes); sink: device
// float[grid * 256].  Each wave issues 8 * iters instructions of 32*32*64*2 FLOP.
extern "C" int ceiling_mfma_fp8(const void* src, float* sink, int iters, int grid, hipStream_t stream) {
  if (src == nullptr || sink == nullptr || iters <= 0 || grid <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_ceiling_fp8_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const i32x8*>(src), sink,
                     iters);
  return (int)hipGetLastError();
}

// src: device buffer of 65536 bf16x8 operands (1 MiB); sink: device float[grid * 256].
// Launches grid workgroups of 4 waves, each wave issuing 8 * iters matrix instructions of
// 32*32*16*2 FLOP.  Returns a hipError_t value (0 on success).
extern "C" int ceiling_mfma_bf16(const void* src, float* sink, int iters, int grid, hipStream_t stream) {
  if (src == nullptr || sink == nullptr || iters <= 0 || grid <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const bf16x8*>(src), sink,
                     iters);
  return (int)hipGetLastError();
}
