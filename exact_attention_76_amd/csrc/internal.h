// internal.h -- launcher interface between the C-ABI layer (api.hip) and the kernel files.
// Arguments reaching these launchers have already been validated by api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, N;          // N: sequence length (dense) or longest sequence (varlen)
  const int* cu_seqlens;      // device int32 [B+1] or nullptr
  int d;
  int causal;
  int window;                 // causal sliding window of this many keys, or 0 for none
  float alpha;
  const float* q_scale;       // fp8 only
  const float* k_scale;
  const float* v_scale;
};

// 16-bit inputs (bf16 when is_bf16, else fp16); d in {64, 128, 256}.
hipError_t launch_fwd_16bit(const FwdArgs& a, bool is_bf16, hipStream_t stream);

// e4m3 inputs with per-block scales; d == 128; dense or packed, causal or not.
hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t stream);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* workspace;           // fp32, B * Hq * N entries (D = rowsum(dO * O), LSE layout)
  int B, Hq, Hkv, N;          // N: sequence length (dense) or longest sequence (packed)
  const int* cu_seqlens;      // device int32 [B+1] or nullptr
  int d;
  int causal;
  int window;                 // causal sliding window of this many keys, or 0 for none
  float alpha;
};

// 16-bit backward pass (bf16 when is_bf16, else fp16); d in {64, 128}.
hipError_t launch_bwd_16bit(const BwdArgs& a, bool is_bf16, hipStream_t stream);

struct PrepareArgs {
  const void* q;
  const void* k;
  const void* v;
  void* q8;
  void* k8;
  void* v8;
  float* q_scale;
  float* k_scale;
  float* v_scale;
  int B, Hq, Hkv, N, d;       // N: sequence length (dense) or longest sequence (packed)
  const int* cu_seqlens;      // device int32 [B+1] or nullptr
  const signed char* signs;
  int per_tensor;             // one scale per tensor instead of one per 64-token block
  const float* rope_cos;      // rotary tables [positions, d/2] fp32, or nullptr
  const float* rope_sin;
};

hipError_t launch_fp8_prepare(const PrepareArgs& a, hipStream_t stream);

}  // namespace attn
