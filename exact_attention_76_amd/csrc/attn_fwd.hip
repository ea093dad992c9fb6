// attn_fwd.hip -- fused exact-attention forward pass for gfx950, 16-bit inputs (bf16 / fp16).
//
// Method: the tiled forward pass with online softmax of the FlashAttention-3 pages (zenmind
// digest, section 3.2 / Algorithm 1): per block of queries, keep a running row maximum m, a
// running row sum l and an O accumulator; for every key/value tile compute S = Q K^T, update
// m, take P = exp(S - m), rescale l and O by exp(m_old - m_new), add P V; finally O / l and
// L = m + ln l.  S and P live only in registers.
//
// gfx950 mapping (our own design; the Hopper producer/consumer structure of the pages is not
// reproduced):
//   * A workgroup of 4 waves owns 128 queries of one (sequence, head); each wave owns 32.
//   * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_{bf16,f16}: the
//     32x32 accumulator of a wave then holds one query per lane column, so the row max and
//     row sum are in-lane plus a single exchange between the two lane halves.
//   * The P^T accumulator is fed straight back as the B operand of O^T = V^T P^T.  The keys
//     a lane holds in its accumulator are not contiguous; V^T is written to LDS with its key
//     columns permuted the same way, so one 16-byte LDS read gives a lane its A operand.
//     (This is the freedom the digest's section 3.5 describes for the FP8 accumulator-to-
//     operand layout: permuting P's columns together with V's rows leaves P V unchanged.)
//   * K and V tiles are double-buffered in LDS: the global loads of tile j+1 are in flight
//     while tile j is multiplied; one barrier per tile.
//   * exp2 with the scale alpha*log2(e) folded into one FMA per score.
//   * Workgroup ids are remapped so that the workgroups resident on one XCD (dispatch is
//     round-robin over the 8 XCDs) work on the same head and share its K/V in that XCD's L2;
//     causal grids run their longest query blocks first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

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
constexpr int kThreads = 256;
constexpr int kBr = 128;  // queries per workgroup (32 per wave)

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

// Bijection from hardware workgroup id to a logical id such that each XCD (hardware id mod 8)
// receives one contiguous range of logical ids.
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  constexpr int kXcd = 8;
  const int q = total / kXcd, r = total % kXcd;
  const int x = wg % kXcd, i = wg / kXcd;
  return x * q + (x < r ? x : r) + i;
}

// Position of key k (0..15 inside a 16-key group) in the permuted V^T tile: the order in
// which the P^T accumulator registers are handed to the second MFMA (see file comment).
__host__ __device__ constexpr int vpos16(int k) {
  return 8 * ((k >> 2) & 1) + (k & 3) + 4 * (k >> 3);
}

template <int D, int BC, bool BF16, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads, (D <= 128 ? 2 : 1)) void fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, int N,
    const int* __restrict__ cu_seqlens, int nseq, float alpha, int num_qblocks) {
  constexpr int KROW = D + 8;   // K tile row stride (elements); +16 B against bank conflicts
  constexpr int VROW = BC + 8;  // V^T tile row stride (elements)
  constexpr int STAGE = BC * KROW + D * VROW;
  constexpr int KS_D = D / 16;   // k-steps of the first product (over d)
  constexpr int KS_C = BC / 16;  // k-steps of the second product (over keys)
  constexpr int NB_C = BC / 32;  // 32-key accumulator blocks per tile
  constexpr int NB_D = D / 32;   // 32-wide d blocks of the O accumulator
  constexpr int K_ITEMS = BC * D / 8;            // 16-byte chunks of a K tile
  constexpr int K_PER = (K_ITEMS + kThreads - 1) / kThreads;
  constexpr int V_ITEMS = (BC / 4) * (D / 8);    // (4 keys x 8 d) pieces of a V tile
  constexpr int V_PER = (V_ITEMS + kThreads - 1) / kThreads;
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;

  // ---- which (sequence, head, query block) ----
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  int qb = logical % num_qblocks;
  const int bh = logical / num_qblocks;
  const int h = bh % Hq, b = bh / Hq;
  if (CAUSAL) qb = num_qblocks - 1 - qb;  // longest query blocks first
  int seq_start, n;
  if constexpr (VARLEN) {
    seq_start = cu_seqlens[b];
    n = cu_seqlens[b + 1] - seq_start;
    if (n > N) n = N;
  } else {
    seq_start = b * N;
    n = N;
  }
  const int q0 = qb * kBr;
  if (q0 >= n) return;  // whole workgroup: block lies past the end of this sequence
  const int g = h / (Hq / Hkv);
  const int64_t qstride = (int64_t)Hq * D, kvstride = (int64_t)Hkv * D;

  // ---- Q fragment of this lane: query qi, d = 16*ks + 8*hi .. +7 ----
  const int qw = q0 + wave * 32;     // first query of this wave
  const int qi = qw + l32;           // this lane's query (within the sequence)
  u32x4 qf[KS_D];
  {
    const int row = qi < n ? qi : n - 1;
    const uint16_t* qp = q + (int64_t)(seq_start + row) * qstride + (int64_t)h * D + 8 * hi;
#pragma unroll
    for (int s = 0; s < KS_D; ++s) qf[s] = *reinterpret_cast<const u32x4*>(qp + 16 * s);
  }

  const uint16_t* kb = k + (int64_t)seq_start * kvstride + (int64_t)g * D;
  const uint16_t* vb = v + (int64_t)seq_start * kvstride + (int64_t)g * D;
  const int kv_end = CAUSAL ? min(n, q0 + kBr) : n;
  const int ntiles = (kv_end + BC - 1) / BC;

  u32x4 kreg[K_PER];
  u32x4 vreg[V_PER][4];

  auto load_tile = [&](int tile) {
    const int k0 = tile * BC;
#pragma unroll
    for (int i = 0; i < K_PER; ++i) {
      const int c = tid + kThreads * i;
      if (K_ITEMS % kThreads == 0 || c < K_ITEMS) {
        const int row = c / (D / 8), col = c % (D / 8);
        const int r = min(k0 + row, n - 1);
        kreg[i] = *reinterpret_cast<const u32x4*>(kb + (int64_t)r * kvstride + col * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
      const int c = tid + kThreads * i;
      if (V_ITEMS % kThreads == 0 || c < V_ITEMS) {
        const int run = c / (D / 8), dch = c % (D / 8);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int r = min(k0 + run * 4 + rr, n - 1);
          vreg[i][rr] = *reinterpret_cast<const u32x4*>(vb + (int64_t)r * kvstride + dch * 8);
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* ks = smem + buf * STAGE;
    uint16_t* vs = ks + BC * KROW;
#pragma unroll
    for (int i = 0; i < K_PER; ++i) {
      const int c = tid + kThreads * i;
      if (K_ITEMS % kThreads == 0 || c < K_ITEMS) {
        const int row = c / (D / 8), col = c % (D / 8);
        *reinterpret_cast<u32x4*>(ks + row * KROW + col * 8) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < V_PER; ++i) {
      const int c = tid + kThreads * i;
      if (V_ITEMS % kThreads == 0 || c < V_ITEMS) {
        const int run = c / (D / 8), dch = c % (D / 8);
        // keys 4*run .. 4*run+3 land on 4 consecutive permuted positions
        const int pos = (run >> 2) * 16 + vpos16((run & 3) * 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          uint32_t p01, p23;
          if (e & 1) {
            p01 = (vreg[i][0][w] >> 16) | (vreg[i][1][w] & 0xFFFF0000u);
            p23 = (vreg[i][2][w] >> 16) | (vreg[i][3][w] & 0xFFFF0000u);
          } else {
            p01 = (vreg[i][0][w] & 0xFFFFu) | (vreg[i][1][w] << 16);
            p23 = (vreg[i][2][w] & 0xFFFFu) | (vreg[i][3][w] << 16);
          }
          u32x2 pr = {p01, p23};
          *reinterpret_cast<u32x2*>(vs + (dch * 8 + e) * VROW + pos) = pr;
        }
      }
    }
  };

  f32x16 oacc[NB_D];
#pragma unroll
  for (int i = 0; i < NB_D; ++i) oacc[i] = f32x16{};
  float m = -INFINITY;  // running max of raw scores q.k
  float l = 0.f;        // running sum over this lane's keys (the two halves are added at the end)
  const float c = alpha * kLog2e;

  load_tile(0);
  store_tile(0);
  for (int j = 0; j < ntiles; ++j) {
    if (j + 1 < ntiles) load_tile(j + 1);
    __syncthreads();
    const uint16_t* ks = smem + (j & 1) * STAGE;
    const uint16_t* vs = ks + BC * KROW;
    const int k0 = j * BC;
    const bool active = !CAUSAL || k0 <= qw + 31;
    if (active) {
      // S^T = K Q^T for this tile: lane holds query qi, keys k0 + 32*cb + 8*(r/4) + 4*hi + r%4
      f32x16 s[NB_C];
#pragma unroll
      for (int cb = 0; cb < NB_C; ++cb) {
        s[cb] = f32x16{};
        const uint16_t* arow = ks + (cb * 32 + l32) * KROW + 8 * hi;
#pragma unroll
        for (int st = 0; st < KS_D; ++st)
          s[cb] = mma32<BF16>(*reinterpret_cast<const u32x4*>(arow + 16 * st), qf[st], s[cb]);
      }
      const bool need_mask = (k0 + BC > n) || (CAUSAL && k0 + BC - 1 > qw);
      if (need_mask) {
#pragma unroll
        for (int cb = 0; cb < NB_C; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + cb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key >= n || (CAUSAL && key > qi)) s[cb][r] = -INFINITY;
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int cb = 0; cb < NB_C; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[cb][r]);
      mt = halves_max(mt);
      const float mnew = fmaxf(m, mt);
      const float mc = (mnew == -INFINITY) ? 0.f : mnew * c;
      const float corr = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m * c - mc);
      m = mnew;
      float rs = 0.f;
#pragma unroll
      for (int cb = 0; cb < NB_C; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[cb][r], c, -mc));
          s[cb][r] = p;
          rs += p;
        }
      l = l * corr + rs;
#pragma unroll
      for (int db = 0; db < NB_D; ++db) oacc[db] *= corr;
      // P^T as the B operand: k-step st takes accumulator registers 8*(st%2) .. +7 of block st/2
      u32x4 pf[KS_C];
#pragma unroll
      for (int st = 0; st < KS_C; ++st) {
        const int cb = st >> 1, base = (st & 1) * 8;
        pf[st] = u32x4{pack2<BF16>(s[cb][base + 0], s[cb][base + 1]),
                       pack2<BF16>(s[cb][base + 2], s[cb][base + 3]),
                       pack2<BF16>(s[cb][base + 4], s[cb][base + 5]),
                       pack2<BF16>(s[cb][base + 6], s[cb][base + 7])};
      }
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < NB_D; ++db) {
        const uint16_t* arow = vs + (db * 32 + l32) * VROW + 8 * hi;
#pragma unroll
        for (int st = 0; st < KS_C; ++st)
          oacc[db] = mma32<BF16>(*reinterpret_cast<const u32x4*>(arow + 16 * st), pf[st], oacc[db]);
      }
    }
    if (j + 1 < ntiles) store_tile((j + 1) & 1);
  }

  // ---- epilogue: O / l, L = alpha*m + ln l ----
  const float lt = halves_sum(l);
  if (qi < n) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    uint16_t* op = o + (int64_t)(seq_start + qi) * qstride + (int64_t)h * D + 4 * hi;
#pragma unroll
    for (int db = 0; db < NB_D; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        u32x2 pr = {pack2<BF16>(oacc[db][4 * gq + 0] * inv, oacc[db][4 * gq + 1] * inv),
                    pack2<BF16>(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + db * 32 + gq * 8) = pr;
      }
    if (hi == 0) {
      const float L = lt > 0.f ? m * alpha + __logf(lt) : -INFINITY;
      int64_t idx;
      if constexpr (VARLEN) idx = (int64_t)h * cu_seqlens[nseq] + seq_start + qi;
      else idx = ((int64_t)b * Hq + h) * N + qi;
      lse[idx] = L;
    }
  }
}

template <int D, int BC, bool BF16, bool CAUSAL, bool VARLEN>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int nqb = (a.N + kBr - 1) / kBr;
  const long long grid = (long long)nqb * a.Hq * a.B;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_kernel<D, BC, BF16, CAUSAL, VARLEN>), dim3((unsigned)grid), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.Hq, a.Hkv,
                     a.N, a.cu_seqlens, a.B, a.alpha, nqb);
  return hipGetLastError();
}

template <int D, int BC, bool BF16>
hipError_t launch_modes(const FwdArgs& a, hipStream_t stream) {
  const bool varlen = a.cu_seqlens != nullptr;
  if (a.causal) return varlen ? launch<D, BC, BF16, true, true>(a, stream) : launch<D, BC, BF16, true, false>(a, stream);
  return varlen ? launch<D, BC, BF16, false, true>(a, stream) : launch<D, BC, BF16, false, false>(a, stream);
}

template <bool BF16>
hipError_t launch_dims(const FwdArgs& a, hipStream_t stream) {
  switch (a.d) {
    case 64: return launch_modes<64, 64, BF16>(a, stream);
    case 128: return launch_modes<128, 64, BF16>(a, stream);
    case 256: return launch_modes<256, 32, BF16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fwd_16bit(const FwdArgs& a, bool is_bf16, hipStream_t stream) {
  return is_bf16 ? launch_dims<true>(a, stream) : launch_dims<false>(a, stream);
}

}  // namespace attn
