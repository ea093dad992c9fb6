/*
 * attn.h -- C ABI of libattn, the fused exact-attention forward pass for AMD gfx950 (MI355X).
 *
 * What is computed (FlashAttention-3 pages; the zenmind digest "FlashAttention-3: pushing
 * attention to Hopper's peak with asynchrony and low precision", section 3.1 for the
 * definition and section 3.2 / Algorithm 1 for the tiled forward pass and its outputs):
 *
 *   for every sequence b, query head h and query i of that sequence
 *     S_ij = alpha * <q_i, k_j>            over the visible keys j
 *     P_ij = softmax_j(S_ij)               (row maximum subtracted before exp)
 *     O_i  = sum_j P_ij v_j
 *     L_i  = m_i + ln(l_i)                 (m_i = max_j S_ij, l_i = sum_j exp(S_ij - m_i))
 *
 * S and P never reach device memory: the kernels tile the keys and use an online softmax.
 * Visible keys: all keys of the same sequence (non-causal) or keys j <= i (causal).
 * Grouped-query attention: query head h reads key/value head h / (Hq / Hkv); K and V are
 * never replicated (digest section 3.2, "MQA/GQA").
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library allocates
 *     nothing and keeps no state between calls, so calls are thread-safe; the one exception
 *     is attn_bwd_noalloc, whose per-GPU static workspace makes overlapping calls on one GPU
 *     race (see there).
 *   - Work is enqueued on `stream` (NULL = the default stream) and the call returns without
 *     synchronising.  Faults of the enqueued kernels surface at the caller's next sync.
 *   - Every argument is validated before anything is enqueued: ATTN_ERR_INVALID,
 *     ATTN_ERR_UNSUPPORTED and ATTN_ERR_ALIGN mean nothing was launched.  ATTN_ERR_HIP means
 *     the HIP runtime refused a launch; an entry point that enqueues several kernels (the
 *     backward pass, per-tensor FP8 scaling) may already have enqueued the ones before it.
 *     An error left pending by earlier, unrelated HIP work is cleared before the first
 *     launch, so it is not reported here.  attn_strerror() names a status.
 *   - Tensors are contiguous with the head dimension innermost (d contiguous), and every
 *     q/k/v/o pointer must be 16-byte aligned (misaligned or strided views are the silent-
 *     wrong-result pitfall named in the blog article's deployment section, so they are
 *     rejected instead).
 */
#ifndef LIBATTN_ATTN_H
#define LIBATTN_ATTN_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q/k/v.  The output o is bf16 for ATTN_BF16 and ATTN_FP8_E4M3 inputs and
 * fp16 for ATTN_FP16 inputs; lse is always fp32. */
typedef enum {
  ATTN_BF16 = 0,
  ATTN_FP16 = 1,
  ATTN_FP8_E4M3 = 2 /* OCP E4M3 ("fn": max 448, no infinities) with per-block scales */
} attn_dtype_t;

enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = -1,     /* null pointer, non-positive size, Hq % Hkv != 0, bad alpha,
                                FP8 without scales */
  ATTN_ERR_UNSUPPORTED = -2, /* head dim / dtype / mode combination without a kernel */
  ATTN_ERR_ALIGN = -3,       /* a tensor pointer is not 16-byte aligned */
  ATTN_ERR_HIP = -4,         /* the HIP runtime refused the launch */
  ATTN_ERR_TOO_LARGE = -5    /* attn_bwd_noalloc: the problem needs more than the library's
                                static workspace holds */
};

/*
 * attn_fwd -- O and L of exact attention, one call per batch.
 *
 * Dense layout (cu_seqlens == NULL):
 *   q, o  [B, N, Hq, d]     k, v [B, N, Hkv, d]     lse [B, Hq, N]
 * Variable-length layout (cu_seqlens != NULL; sequences packed along one token axis, the
 * varlen interface of the guijiagi overview's "variable-length sequences" paragraph):
 *   cu_seqlens: int32 [B + 1] on the device, cu_seqlens[0] = 0, non-decreasing; sequence b
 *   holds tokens cu_seqlens[b] .. cu_seqlens[b+1]-1 and T = cu_seqlens[B].  The offsets are
 *   read on the device only, so the library cannot validate them: offsets that decrease or
 *   pass the T tokens the tensors hold make the kernels access memory outside the tensors.
 *   q, o  [T, Hq, d]        k, v [T, Hkv, d]        lse [Hq, T]
 *   N must be >= the longest sequence (it sizes the grid, so no device-to-host copy is
 *   needed; the library cannot check it without one).  A longer sequence is treated as its
 *   first N tokens: its results are wrong and its rows past N are left unwritten.
 *
 * d:       64, 128 or 256 for ATTN_BF16 / ATTN_FP16; 128 for ATTN_FP8_E4M3.
 * causal:  0 = every key of the sequence is visible; 1 = key j visible to query i iff j <= i.
 * alpha:   score scale, finite and > 0 (usually 1/sqrt(d), digest section 3.1).
 * dtype:   element type of q, k, v.
 * q_scale, k_scale, v_scale (ATTN_FP8_E4M3 only, else ignored): fp32 device arrays of
 *   powers of two, [B, Hq, ceil(N/64)] for q and [B, Hkv, ceil(N/64)] for k and v; block c
 *   covers tokens 64c .. 64c+63 of a (batch, head).  The attention inputs are
 *   e4m3(x) * scale (digest section 3.5, block quantisation).  In the packed layout, b is
 *   the sequence and block c covers tokens 64c .. 64c+63 counted from the sequence's first
 *   token.  Each scale must be a normal fp32 power of two, 2^-126 .. 2^127: the kernel
 *   passes its exponent to the matrix instruction as an E8M0 scale.
 * lse:     fp32, natural log, in units of the scaled scores S.  A row without visible keys
 *          gets O = 0 and L = -inf.
 *
 * Limits: one head's K (or V) rows must span less than 2 GiB, i.e. N * Hkv * d * sizeof(element)
 * < 2^31 (ATTN_ERR_UNSUPPORTED otherwise); B * N < 2^31 tokens.
 *
 * Returns ATTN_OK or a negative status; on a validation error nothing is enqueued.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int N, const int* cu_seqlens,
             int d, int causal, float alpha, attn_dtype_t dtype,
             const float* q_scale, const float* k_scale, const float* v_scale,
             hipStream_t stream);

/*
 * attn_fwd_window -- causal attention inside a sliding window (the guijiagi overview's
 * "sliding window attention" paragraph: attention taken only inside a local window, read as
 * the causal window of the W most recent positions).
 *
 * Query i of a sequence sees keys j with i - window < j <= i: the window keys ending at
 * itself.  window must be >= 1 (ATTN_ERR_INVALID otherwise); window >= N is plain causal
 * attention.  Every other argument, layout, limit and status is that of attn_fwd with
 * causal = 1; bf16, fp16 and e4m3 inputs are accepted alike.
 */
int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int N, const int* cu_seqlens,
                    int d, int window, float alpha, attn_dtype_t dtype,
                    const float* q_scale, const float* k_scale, const float* v_scale,
                    hipStream_t stream);

/*
 * attn_bwd -- gradients of attn_fwd's output with respect to q, k and v (16-bit inputs).
 *
 * The backward pass of the FlashAttention-3 pages (zenmind digest, section 4, data path step
 * 5): a pre-processing step forms D = rowsum(dout * o) per (query, head), and P is recomputed
 * from the stored lse instead of being kept.  With S = alpha q k^T and P = exp(S - lse) over
 * the visible keys:
 *   dv = P^T dout,  dS = P * (dout v^T - D),  dq = alpha dS k,  dk = alpha dS^T q,
 * dk and dv summed over the query heads that share a key/value head.
 *
 * q, k, v, o, lse: the inputs and outputs of the attn_fwd call being differentiated (same
 *   layouts, dtype, B, Hq, Hkv, N, cu_seqlens, d, causal and alpha).
 * dout: gradient of the loss with respect to o, o's layout and dtype.
 * dq, dk, dv: outputs in q's, k's and v's layouts and dtype; every element is written.
 * workspace: fp32 device memory of at least attn_bwd_workspace_bytes(B, Hq, N) bytes, owned by
 *   the caller; on return it holds D in lse's layout.  Nothing is allocated.
 * d: 64 or 128; dtype: ATTN_BF16 or ATTN_FP16 (ATTN_ERR_UNSUPPORTED otherwise).
 * Limits: N * Hq * d * 2 < 2^31 (one head's q rows addressed with 32-bit offsets).
 * Three kernels run in order on `stream`.  Returns ATTN_OK or a negative status (see the
 * conventions at the top for what each means about enqueued work).
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, float* workspace,
             int B, int Hq, int Hkv, int N, const int* cu_seqlens,
             int d, int causal, float alpha, attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_bwd_window -- attn_bwd for attn_fwd_window's output: causal attention inside a
 * sliding window of `window` keys (query i sees keys i-window+1 .. i; window >= 1, else
 * ATTN_ERR_INVALID; window >= N is plain causal).  Arguments otherwise as attn_bwd with
 * causal = 1.
 */
int attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, float* workspace,
                    int B, int Hq, int Hkv, int N, const int* cu_seqlens,
                    int d, int window, float alpha, attn_dtype_t dtype, hipStream_t stream);

/* Bytes of workspace attn_bwd needs (B * Hq * N floats); 0 for non-positive sizes. */
size_t attn_bwd_workspace_bytes(int B, int Hq, int N);

/* Rows (B * Hq * N) the static workspace of attn_bwd_noalloc holds: 2^22 fp32 values, 16 MiB. */
#define ATTN_BWD_NOALLOC_MAX_ROWS (1 << 22)

/*
 * attn_bwd_noalloc -- attn_bwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, same
 * kernels and bit-identical results as attn_bwd, without the workspace argument: D lives in a
 * device array of ATTN_BWD_NOALLOC_MAX_ROWS floats that the library holds, one per GPU it runs
 * on, for the life of the process.
 *   - B * Hq * N must not exceed ATTN_BWD_NOALLOC_MAX_ROWS (ATTN_ERR_TOO_LARGE otherwise;
 *     checked before anything else is looked up or enqueued).
 *   - The device is that of `stream` (the current device for the NULL stream).  The first call
 *     on a device looks up that device's copy of the array (hipGetSymbolAddress); no call
 *     allocates device memory.
 *   - Every call on one GPU shares that GPU's array: calls that overlap on one GPU (different
 *     streams or threads) race on it and give wrong gradients; serialise them.  Each call
 *     writes every entry it reads first, so nothing needs clearing between calls.
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv,
                     int B, int Hq, int Hkv, int N, const int* cu_seqlens,
                     int d, int causal, float alpha, attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_fp8_prepare -- the FP8 pre-pass (digest section 3.5: block quantisation and
 * incoherent processing; power-of-two block scales as the blog article's FP8 section
 * requires).
 *
 * Inputs q [B, N, Hq, d], k and v [B, N, Hkv, d], bf16, dense layout, d = 128.
 * If hadamard_signs (device int8 [d], each +1 or -1, 16-byte aligned) is non-NULL, q and k are first
 * multiplied along d by D H, where D = diag(signs) and H is the unnormalised Sylvester
 * Hadamard matrix (entries +-1); v is never rotated.  NULL skips the rotation.
 * Then, per (batch, head, block of 64 tokens), with amax the largest magnitude in the
 * block, e is the smallest integer with amax <= 448 * 2^e (e = 0 for an all-zero block),
 * every element is divided by 2^e and rounded to the nearest e4m3 value (ties to even,
 * sign kept), and the block scale 2^e is written -- times 1/d for k when rotated, so that
 * (q8 * q_scale) . (k8 * k_scale) approximates q . k.
 * If that scale would be below 2^-126 (amax under 448 * 2^-127, about 2.6e-36, or under
 * 448 * 2^-120 for rotated k), e is raised until the scale is 2^-126, so every scale is a
 * normal fp32 as attn_fwd requires.
 * Outputs q8/k8/v8: uint8 e4m3 codes in the input layouts; scales fp32 [B, H, ceil(N/64)].
 * The rotated sums are formed in fp64, so each code is the rounding of the exact value.
 * Inputs must be finite.
 */
int attn_fp8_prepare(const void* q, const void* k, const void* v,
                     void* q8, void* k8, void* v8,
                     float* q_scale, float* k_scale, float* v_scale,
                     int B, int Hq, int Hkv, int N, int d,
                     const signed char* hadamard_signs,
                     hipStream_t stream);

/* Granularity of the FP8 pre-pass's power-of-two scales. */
typedef enum {
  ATTN_FP8_SCALE_BLOCK = 0,  /* one scale per (batch, head, block of 64 tokens) */
  ATTN_FP8_SCALE_TENSOR = 1  /* one scale per tensor */
} attn_fp8_scaling_t;

/*
 * attn_fp8_prepare_ex -- attn_fp8_prepare with every option: the packed variable-length
 * layout, a choice of scale granularity and a fused rotary embedding.
 *
 * cu_seqlens: NULL for the dense layout, or the packed layout of attn_fwd: int32 [B + 1] on the
 *   device, q [T, Hq, d], k and v [T, Hkv, d], N >= the longest sequence.  Blocks then count
 *   from each sequence's first token, so every sequence is quantised as it would be alone;
 *   the scales are [B, H, ceil(N/64)], and entries past a sequence's last block are not
 *   defined (attn_fwd never reads them).
 * scaling: ATTN_FP8_SCALE_BLOCK is attn_fp8_prepare's rule.  ATTN_FP8_SCALE_TENSOR is
 *   per-tensor scaling, the usual practice that the digest's section 3.5 contrasts with block
 *   quantisation and the baseline of the FlashAttention-3 paper's FP8 error ablation (section
 *   4.3, Table 3): e is chosen by the same rule from the largest magnitude of the whole
 *   (rotated) tensor, all batches, sequences and heads, and that one scale is written into
 *   every [b, h, block] entry, so the outputs feed attn_fwd unchanged.  The per-tensor pre-pass
 *   takes three kernel launches on `stream` and uses the scale arrays as working storage
 *   between them: their contents are defined only once all three have run.  Any other value
 *   returns ATTN_ERR_INVALID.
 * rope_cos, rope_sin: NULL (both), or fp32 device tables [P, d/2] with P >= N, 16-byte
 *   aligned: the pre-pass is then fused with a rotary position embedding (the digest's section
 *   3.5 fuses quantisation and the Hadamard rotation into the rotary embedding; the guijiagi
 *   overview's RoPE-fusion paragraph).  Before anything else, features (2i, 2i+1) of every
 *   q and k token at position m of its sequence (m counted from the sequence's first token)
 *   become x0*c - x1*s and x0*s + x1*c with c = rope_cos[m][i], s = rope_sin[m][i], each
 *   product and sum rounded to fp32 and the results rounded to bf16 (nearest even): the bf16
 *   tensors an unfused fp32 rotary kernel would write, which never reach memory here.  v is
 *   not embedded.  Only one of the two NULL returns ATTN_ERR_INVALID; misaligned tables
 *   ATTN_ERR_ALIGN.
 * Everything else is as for attn_fp8_prepare.
 */
int attn_fp8_prepare_ex(const void* q, const void* k, const void* v,
                        void* q8, void* k8, void* v8,
                        float* q_scale, float* k_scale, float* v_scale,
                        int B, int Hq, int Hkv, int N, const int* cu_seqlens, int d,
                        const float* rope_cos, const float* rope_sin,
                        const signed char* hadamard_signs, attn_fp8_scaling_t scaling,
                        hipStream_t stream);

/* Static description of a status code. */
const char* attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* LIBATTN_ATTN_H */
