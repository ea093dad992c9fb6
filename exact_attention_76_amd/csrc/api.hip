// api.hip -- the C ABI of libattn (declared in include/attn.h): argument validation and
// dispatch to the kernel launchers.  Host code only.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn.h"
#include "internal.h"

#include <mutex>

// Workspace of attn_bwd_noalloc: D = rowsum(dO * O) for up to ATTN_BWD_NOALLOC_MAX_ROWS rows.
// Each GPU the library runs on holds its own copy of this array, at its own address, until the
// process ends.  In host code its name is only a stand-in: the device address of each copy is
// looked up once per device (scratch_on) and only that address is passed to kernels.
static __device__ __align__(256) float scratch[ATTN_BWD_NOALLOC_MAX_ROWS];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
float* scratch_ptr[kMaxDevices] = {};

// Device address of `dev`'s copy of scratch, looked up on the first use with that device
// current (the caller's current device is restored).
int scratch_on(int dev, float** out) {
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return ATTN_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return ATTN_ERR_HIP;
    void* p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (err != hipSuccess || p == nullptr) return ATTN_ERR_HIP;
    scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = scratch_ptr[dev];
  return ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest element count any one tensor may have, so 64-bit offsets never overflow and the
// per-row arithmetic in the kernels stays in int range.
constexpr long long kMaxTokens = 1LL << 31;

int validate_common(const void* q, const void* k, const void* v, const void* o, const void* out2,
                    int B, int Hq, int Hkv, int N) {
  if (!q || !k || !v || !o || !out2) return ATTN_ERR_INVALID;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || N <= 0) return ATTN_ERR_INVALID;
  if (Hq % Hkv != 0) return ATTN_ERR_INVALID;
  if ((long long)B * N >= kMaxTokens) return ATTN_ERR_INVALID;
  return ATTN_OK;
}

// Clears an error that earlier, unrelated HIP work left pending, so that the launches of this
// call are judged by their own hipGetLastError().  Called once, after validation and before the
// first launch.
void clear_pending_error() { (void)hipGetLastError(); }

int status_of(hipError_t err) {
  if (err == hipSuccess) return ATTN_OK;
  if (err == hipErrorNotSupported) return ATTN_ERR_UNSUPPORTED;
  return ATTN_ERR_HIP;
}

// attn_fwd and attn_fwd_window: window = 0 is no window.
int fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int N,
        const int* cu_seqlens, int d, int causal, int window, float alpha, attn_dtype_t dtype, const float* q_scale,
        const float* k_scale, const float* v_scale, hipStream_t stream) {
  int rc = validate_common(q, k, v, o, lse, B, Hq, Hkv, N);
  if (rc != ATTN_OK) return rc;
  if (!(isfinite(alpha) && alpha > 0.f)) return ATTN_ERR_INVALID;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_ALIGN;

  attn::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, cu_seqlens, d, causal, window, alpha, q_scale, k_scale, v_scale};
  hipError_t err;
  switch (dtype) {
    case ATTN_BF16:
    case ATTN_FP16:
      if (d != 64 && d != 128 && d != 256) return ATTN_ERR_UNSUPPORTED;
      // the kernels address one head's K/V rows with 32-bit byte offsets
      if ((long long)N * Hkv * d * 2 > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
      clear_pending_error();
      err = attn::launch_fwd_16bit(a, dtype == ATTN_BF16, stream);
      break;
    case ATTN_FP8_E4M3:
      if (!q_scale || !k_scale || !v_scale) return ATTN_ERR_INVALID;
      if (d != 128) return ATTN_ERR_UNSUPPORTED;
      if ((long long)N * Hkv * d > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
      clear_pending_error();
      err = attn::launch_fwd_fp8(a, stream);
      break;
    default:
      return ATTN_ERR_UNSUPPORTED;
  }
  return status_of(err);
}

// Argument checks of the backward entry points (everything but the window).
int bwd_validate(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                 void* dq, void* dk, void* dv, const float* workspace, int B, int Hq, int Hkv, int N, int d,
                 int causal, float alpha, attn_dtype_t dtype) {
  int rc = validate_common(q, k, v, o, lse, B, Hq, Hkv, N);
  if (rc != ATTN_OK) return rc;
  if (!dout || !dq || !dk || !dv || !workspace) return ATTN_ERR_INVALID;
  if (!(isfinite(alpha) && alpha > 0.f)) return ATTN_ERR_INVALID;
  if (causal != 0 && causal != 1) return ATTN_ERR_INVALID;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  // the kernels address one head's Q (and dO) rows with 32-bit byte offsets
  if ((long long)N * Hq * d * 2 > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
    return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

// attn_bwd and attn_bwd_window: window = 0 is no window.
int bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
        void* dk, void* dv, float* workspace, int B, int Hq, int Hkv, int N, const int* cu_seqlens, int d, int causal,
        int window, float alpha, attn_dtype_t dtype, hipStream_t stream) {
  const int rc = bwd_validate(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, d, causal, alpha, dtype);
  if (rc != ATTN_OK) return rc;
  attn::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, cu_seqlens, d, causal, window, alpha};
  clear_pending_error();
  return status_of(attn::launch_bwd_16bit(a, dtype == ATTN_BF16, stream));
}

}  // namespace

extern "C" {

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_INVALID: return "invalid argument (null pointer, non-positive size, Hq % Hkv != 0, "
                                  "alpha not finite and > 0, or FP8 without scales)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported combination of head dim, dtype and mode";
    case ATTN_ERR_ALIGN: return "tensor pointer not 16-byte aligned";
    case ATTN_ERR_HIP: return "HIP runtime refused the launch";
    case ATTN_ERR_TOO_LARGE: return "B * Hq * N exceeds the static workspace of attn_bwd_noalloc "
                                    "(ATTN_BWD_NOALLOC_MAX_ROWS)";
    default: return "unknown status";
  }
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
             int N, const int* cu_seqlens, int d, int causal, float alpha, attn_dtype_t dtype,
             const float* q_scale, const float* k_scale, const float* v_scale, hipStream_t stream) {
  return fwd(q, k, v, o, lse, B, Hq, Hkv, N, cu_seqlens, d, causal, 0, alpha, dtype, q_scale, k_scale, v_scale,
             stream);
}

int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                    int N, const int* cu_seqlens, int d, int window, float alpha, attn_dtype_t dtype,
                    const float* q_scale, const float* k_scale, const float* v_scale, hipStream_t stream) {
  if (window < 1) return ATTN_ERR_INVALID;
  // a window of N or more keys is plain causal attention
  return fwd(q, k, v, o, lse, B, Hq, Hkv, N, cu_seqlens, d, 1, window < N ? window : 0, alpha, dtype, q_scale,
             k_scale, v_scale, stream);
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int N) {
  if (B <= 0 || Hq <= 0 || N <= 0) return 0;
  return (size_t)B * (size_t)Hq * (size_t)N * sizeof(float);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, float* workspace, int B, int Hq, int Hkv, int N, const int* cu_seqlens,
             int d, int causal, float alpha, attn_dtype_t dtype, hipStream_t stream) {
  return bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, cu_seqlens, d, causal, 0, alpha, dtype,
             stream);
}

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, const int* cu_seqlens, int d,
                     int causal, float alpha, attn_dtype_t dtype, hipStream_t stream) {
  if (B > 0 && Hq > 0 && N > 0 && (long long)B * Hq * N > ATTN_BWD_NOALLOC_MAX_ROWS) return ATTN_ERR_TOO_LARGE;
  // every other argument is checked exactly as attn_bwd checks it before the workspace is
  // looked up; a non-null stand-in passes the workspace check
  float* const probe = reinterpret_cast<float*>(256);
  int rc = bwd_validate(q, k, v, o, lse, dout, dq, dk, dv, probe, B, Hq, Hkv, N, d, causal, alpha, dtype);
  if (rc != ATTN_OK) return rc;
  int dev = -1;
  if (stream != nullptr ? hipStreamGetDevice(stream, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
    return ATTN_ERR_HIP;
  float* ws = nullptr;
  rc = scratch_on(dev, &ws);
  if (rc != ATTN_OK) return rc;
  return bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, N, cu_seqlens, d, causal, 0, alpha, dtype, stream);
}

int attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                    void* dq, void* dk, void* dv, float* workspace, int B, int Hq, int Hkv, int N,
                    const int* cu_seqlens, int d, int window, float alpha, attn_dtype_t dtype, hipStream_t stream) {
  if (window < 1) return ATTN_ERR_INVALID;
  return bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, Hq, Hkv, N, cu_seqlens, d, 1, window < N ? window : 0,
             alpha, dtype, stream);
}

int attn_fp8_prepare(const void* q, const void* k, const void* v, void* q8, void* k8, void* v8,
                     float* q_scale, float* k_scale, float* v_scale, int B, int Hq, int Hkv, int N, int d,
                     const signed char* hadamard_signs, hipStream_t stream) {
  return attn_fp8_prepare_ex(q, k, v, q8, k8, v8, q_scale, k_scale, v_scale, B, Hq, Hkv, N, nullptr, d, nullptr,
                             nullptr, hadamard_signs, ATTN_FP8_SCALE_BLOCK, stream);
}

int attn_fp8_prepare_ex(const void* q, const void* k, const void* v, void* q8, void* k8, void* v8, float* q_scale,
                        float* k_scale, float* v_scale, int B, int Hq, int Hkv, int N, const int* cu_seqlens, int d,
                        const float* rope_cos, const float* rope_sin, const signed char* hadamard_signs,
                        attn_fp8_scaling_t scaling, hipStream_t stream) {
  if (scaling != ATTN_FP8_SCALE_BLOCK && scaling != ATTN_FP8_SCALE_TENSOR) return ATTN_ERR_INVALID;
  if ((rope_cos == nullptr) != (rope_sin == nullptr)) return ATTN_ERR_INVALID;
  int rc = validate_common(q, k, v, q8, k8, B, Hq, Hkv, N);
  if (rc != ATTN_OK) return rc;
  if (!v8 || !q_scale || !k_scale || !v_scale) return ATTN_ERR_INVALID;
  if (d != 128) return ATTN_ERR_UNSUPPORTED;
  if ((long long)B * Hq * ((N + 63) / 64) > 0x7fffffffLL) return ATTN_ERR_UNSUPPORTED;  // grid size
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q8) || !aligned16(k8) || !aligned16(v8) ||
      !aligned16(rope_cos) || !aligned16(rope_sin) || !aligned16(hadamard_signs))
    return ATTN_ERR_ALIGN;
  attn::PrepareArgs a{q, k, v, q8, k8, v8, q_scale, k_scale, v_scale, B, Hq, Hkv, N, d, cu_seqlens, hadamard_signs,
                      scaling == ATTN_FP8_SCALE_TENSOR, rope_cos, rope_sin};
  clear_pending_error();
  return status_of(attn::launch_fp8_prepare(a, stream));
}

}  // extern "C"
