// attn_bwd.hip -- backward pass of exact attention for gfx950, 16-bit inputs (bf16 / fp16).
//
// Method (FlashAttention-3 pages, zenmind digest section 4, data path step 5: a pre-processing
// step forms D = rowsum(dO * O), and the backward pass recomputes P from the stored L instead of
// keeping it): with S = alpha Q K^T and P = exp(S - L),
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = alpha dS K,  dK = alpha dS^T Q,
// dK and dV summed over the query heads of a key/value group.  Five products, as the digest's
// section 7.1 counts (2.5 x the forward FLOPs).
//
// gfx950 mapping (ours):
//   * bwd_delta_kernel: D per (query, head), one 16-byte slice of dO and O per lane.
//   * bwd_dkdv_kernel: a workgroup of kKvWaves waves (eight: two per SIMD) owns 32 keys per
//     wave (256) of one (sequence, key/value head); its K and V rows stay in registers as matrix-instruction B operands (one key
//     per lane column).  It walks the query tiles of every query head of the group: Q and dO
//     tiles (and their L and D values) are copied buffer-to-LDS, two stages deep, and each
//     tile takes S = Q K^T and dP = dO V^T (A operands read from the tile rows), P and dS in
//     registers (the query of each accumulator row picks its L and D from LDS), then
//     dV^T += dO^T P and dK^T += Q^T dS (A operands read transposed from the same tiles, the
//     accumulators of P and dS fed back as B operands, as the forward pass feeds P^T).
//   * bwd_dq_kernel: the forward pass's shape -- four waves own 128 queries, one per lane
//     column; per key tile S^T = K Q^T and dP^T = V dO^T, dS^T in registers, dQ^T += K^T dS^T
//     with K read transposed.  Every gradient is written once; no atomics, so the result is
//     deterministic.
//   * In both kernels a tile's products run as two streams (the first products, then the
//     products with P and dS) whose LDS operands are read two to four products ahead in an order
//     pinned for the scheduler; the first operands of the second stream are read before the
//     softmax.  The masks of edge tiles stay behind a branch.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "decompose.h"
#include "internal.h"
#include "tile16.h"

namespace attn {
namespace {

constexpr int kWaves = 4;  // waves per workgroup of the dQ kernel
constexpr int kBlk = 32 * kWaves;  // queries per dQ workgroup
#ifndef ATTN_BWD_KV_WAVES
#define ATTN_BWD_KV_WAVES 8
#endif
constexpr int kKvWaves = ATTN_BWD_KV_WAVES;  // waves per dK/dV workgroup (32 keys each)
constexpr int kKvBlk = 32 * kKvWaves;         // keys per dK/dV workgroup
constexpr int kTile = 64;  // streamed rows per tile (dQ: keys; dK/dV: queries at d = 64)
// dK/dV at d = 128 streams 32-query tiles: its resident K, V and both accumulators leave no
// room for the scores of 64 queries without spilling
template <int D>
constexpr int dkdv_tile() { return D == 128 ? 32 : 64; }

// 16-bit values -> float
template <bool BF16>
__device__ __forceinline__ float lo16(uint32_t w) {
  if constexpr (BF16) return __uint_as_float(w << 16);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFF));
}
template <bool BF16>
__device__ __forceinline__ float hi16(uint32_t w) {
  if constexpr (BF16) return __uint_as_float(w & 0xFFFF0000u);
  else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// D[row] = sum over d of dO * O for every (token, query head) row; delta has the LSE layout.
// The grid covers B * N tokens; packed input has T = cu_seqlens[nseq] <= B * N of them.
template <int D, bool BF16>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                                        float* __restrict__ delta, int Hq, int N, int B,
                                                        const int* __restrict__ cu_seqlens) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  const int64_t T = cu_seqlens ? (int64_t)cu_seqlens[B] : (int64_t)B * N;
  const int64_t rows = T * Hq;
  const int packed = cu_seqlens != nullptr;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + row * D + 8 * part);
    const u32x4 g = *reinterpret_cast<const u32x4*>(dout + row * D + 8 * part);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += lo16<BF16>(a[e]) * lo16<BF16>(g[e]) + hi16<BF16>(a[e]) * hi16<BF16>(g[e]);
  }
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) acc += __shfl_xor(acc, m);
  if (row < rows && part == 0) {
    const int64_t t = row / Hq;
    const int h = (int)(row % Hq);
    const int64_t idx = packed ? (int64_t)h * T + t : ((t / N) * Hq + h) * N + t % N;
    delta[idx] = acc;
  }
}

// Operand read offsets inside a 16-bit tile (tile16.h layout), lane part.
//   rows: A operand from tile rows 32*cb + l32, k-step st over d (chunk 2*st + hi)
//   tr:   A operand of a transposed tile (d rows, tile rows as k) by ds_read_b64_tr_b16
template <int D>
__device__ __forceinline__ void operand_offsets(int lane, int* koff, int* vtoff) {
  constexpr int NCH = D / 8;
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int e = 0; e < 2; ++e)
    koff[e] = 16 * ((l32 >> 4) * 16 * NCH + (2 * e + hi) * 16 + ((lane & 15) ^ (4 * (2 * e + hi))));
  const int G = lane >> 4, r = (lane >> 2) & 3, c = lane & 3;
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int chunk = 2 * (G & 1) + (c >> 1);
    const int rowm = 4 * (G >> 1) + 8 * rd + r;
    vtoff[rd] = 16 * (chunk * 16 + (rowm ^ (4 * chunk))) + 8 * (c & 1);
  }
}

// k-step st of a 32-row accumulator block pair, packed as the B operand (registers 8*(st%2) ..
// of block st/2).
template <bool BF16>
__device__ __forceinline__ u32x4 pack_step(const f32x16* x, int st) {
  const int cb = st >> 1, base = (st & 1) * 8;
  return u32x4{pack2<BF16>(x[cb][base + 0], x[cb][base + 1]), pack2<BF16>(x[cb][base + 2], x[cb][base + 3]),
               pack2<BF16>(x[cb][base + 4], x[cb][base + 5]), pack2<BF16>(x[cb][base + 6], x[cb][base + 7])};
}

// A stream of N products whose operands come from LDS, each read PD products ahead of its
// matrix instruction: read(i) returns operand i, product(i, a) issues product i, and pin(i)
// names the LDS reads of operand i for the scheduler.  Without the pinned order the compiler
// reads each operand right before its product, and every matrix instruction waits the full
// LDS latency.  With PRIMED the first PD operands are already in `win` (read by prime()).
template <int N, int PD, bool PRIMED, class T, class Read, class Product, class Pin>
__device__ __forceinline__ void product_stream(Read read, Product product, Pin pin, T* win) {
  if constexpr (!PRIMED) {
#pragma unroll
    for (int i = 0; i < PD; ++i) win[i] = read(i);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const T a = win[i % PD];
    if (i + PD < N) win[i % PD] = read(i + PD);
    product(i, a);
  }
  if constexpr (!PRIMED) {
#pragma unroll
    for (int i = 0; i < PD; ++i) pin(i);
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i + PD < N) pin(i + PD);
  }
}
template <int PD, class T, class Read>
__device__ __forceinline__ void prime(Read read, T* win) {
#pragma unroll
  for (int i = 0; i < PD; ++i) win[i] = read(i);
}
// scheduler pins for operands of one and of two LDS reads
struct Pin1 {
  __device__ void operator()(int) const { __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); }
};
struct Pin2 {
  __device__ void operator()(int) const { __builtin_amdgcn_sched_group_barrier(0x100, 2, 0); }
};

// Transposed operand (D rows of 16 tile rows, k-step st, d block db) by two ds_read_b64_tr_b16.
template <int D>
__device__ __forceinline__ u32x4 tr_operand(const char* tile, const int* vtoff, int st, int db) {
  constexpr int NCH = D / 8;
  const int imm = st * 256 * NCH + db * 1024;
  const s16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, tile + vtoff[0] + imm));
  const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, tile + vtoff[1] + imm));
  const u32x2 a0 = __builtin_bit_cast(u32x2, t0), a1 = __builtin_bit_cast(u32x2, t1);
  return u32x4{a0[0], a0[1], a1[0], a1[1]};
}

// Accumulator row held by register r of a 32x32 block: 8*(r/4) + 4*hi + r%4.
__device__ __forceinline__ int acc_row(int r, int hi) { return 8 * (r >> 2) + 4 * hi + (r & 3); }

// Store a D x 32 transposed accumulator (lane = token column) as 16-bit rows, times scale.
template <int D, bool BF16>
__device__ __forceinline__ void store_rows(uint16_t* dst, const f32x16* acc, float scale, int hi) {
  constexpr int NB_D = D / 32;
  uint16_t* p = dst + 4 * hi;
#pragma unroll
  for (int db = 0; db < NB_D; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      u32x2 pr = {pack2<BF16>(acc[db][4 * gq + 0] * scale, acc[db][4 * gq + 1] * scale),
                  pack2<BF16>(acc[db][4 * gq + 2] * scale, acc[db][4 * gq + 3] * scale)};
      *reinterpret_cast<u32x2*>(p + db * 32 + gq * 8) = pr;
    }
}

template <int D, int ROWS, int WAVES>
__device__ __forceinline__ int copy_offset(int wave, int lane, int rowbytes) {
  constexpr int NI = ROWS * D * 2 / 1024 / WAVES;
  int row, chunk;
  tile_row_chunk<D>(wave * NI * 64 + lane, row, chunk);
  return row * rowbytes + chunk * 16;
}

// ---- dK, dV -------------------------------------------------------------------------------------
// WINDOW (implies CAUSAL): causal sliding window of `window` keys (query i sees keys
// i-window+1 .. i); otherwise `window` is unused.
template <int D, bool BF16, bool CAUSAL, bool VARLEN, bool WINDOW>
__global__ __launch_bounds__(64 * kKvWaves, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int Hq, int Hkv, int N, const int* __restrict__ cu_seqlens,
    int nseq, float alpha, int num_kblocks, int window) {
  constexpr int NCH = D / 8, KS_D = D / 16, NB_D = D / 32;
  constexpr int TQ = dkdv_tile<D>();  // queries per tile
  constexpr int TILE = TQ * D * 2;
  constexpr int NI = TILE / 1024 / kKvWaves, IPB = NCH / 4;
  constexpr int NB = TQ / 32, KS = TQ / 16;  // query blocks and k-steps of one tile
  // d = 128: V stays in LDS (the workgroup's rows, read per k-step as the B operand of dP)
  // instead of registers, so two waves fit on a SIMD without spilling
  constexpr bool V_LDS = D == 128;
  static_assert(!V_LDS || NB == 1, "dP from LDS is written for one 32-query block per tile");
  static_assert(NI * kKvWaves * 1024 == TILE && (NI % IPB == 0 || NI < IPB), "tile shape");
  __shared__ __attribute__((aligned(1024))) char qt0[TILE];
  __shared__ __attribute__((aligned(1024))) char qt1[TILE];
  __shared__ __attribute__((aligned(1024))) char gt0[TILE];
  __shared__ __attribute__((aligned(1024))) char gt1[TILE];
  __shared__ __attribute__((aligned(1024))) float ld0[2][256];  // L and D of a tile (64 used each)
  __shared__ __attribute__((aligned(1024))) float ld1[2][256];
  __shared__ __attribute__((aligned(1024))) char vres[V_LDS ? kKvBlk * D * 2 : 16];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;

  // ---- which (sequence, key/value head, key block): heads of the same sequence on one XCD;
  // causal: a key block sees every query from its own on, so the lowest blocks are the longest
  // and run first (the decomposition orders blocks longest first for query blocks, i.e. highest
  // index first; the key block index is its mirror image) ----
  int kbd, g, b;
  decompose<CAUSAL>(blockIdx.x, num_kblocks, Hkv, Hkv, nseq, kbd, g, b);
  const int kb = CAUSAL ? num_kblocks - 1 - kbd : kbd;
  int seq_start, n;
  if constexpr (VARLEN) {
    seq_start = cu_seqlens[b];
    n = cu_seqlens[b + 1] - seq_start;
    if (n > N) n = N;
  } else {
    seq_start = b * N;
    n = N;
  }
  const int k0 = kb * kKvBlk;
  if (k0 >= n) return;
  const int G = Hq / Hkv;
  const int kw = k0 + wave * 32;  // first key of this wave
  const int kj = kw + l32;        // this lane's key

  // K and V of this lane's key as B operands: d = 16*st + 8*hi .. +7
  u32x4 kf[KS_D], vf[V_LDS ? 1 : KS_D];
  {
    const int row = kj < n ? kj : n - 1;
    const int64_t off = ((int64_t)(seq_start + row) * Hkv + g) * D + 8 * hi;
#pragma unroll
    for (int s = 0; s < KS_D; ++s) {
      kf[s] = *reinterpret_cast<const u32x4*>(k + off + 16 * s);
      if constexpr (!V_LDS) vf[s] = *reinterpret_cast<const u32x4*>(v + off + 16 * s);
    }
  }
  if constexpr (V_LDS) {  // the workgroup's V rows (rows past n read as zero)
    constexpr int NIV = kKvBlk * D * 2 / 1024 / kKvWaves;
    const int kvrow = Hkv * D * 2;
    int row, chunk;
    tile_row_chunk<D>(wave * NIV * 64 + lane, row, chunk);
    const char* vb = reinterpret_cast<const char*>(v) + ((int64_t)(seq_start + k0) * Hkv + g) * D * 2;
    copy_rows_to_lds<NIV, NCH / 4>(vb, (n - 1 - k0) * kvrow + D * 2, vres + wave * NIV * 1024, row * kvrow + chunk * 16,
                                   16 * kvrow);
  }
  int koff[2], vtoff[2];
  operand_offsets<D>(lane, koff, vtoff);

  const int rowbytes = Hq * D * 2;  // Q and dO rows of one head
  const int voff = copy_offset<D, TQ, kKvWaves>(wave, lane, rowbytes);
  const int blk_bytes = 16 * rowbytes;
  const int nbytes = (n - 1) * rowbytes + D * 2;
  // causal: the first query tile that holds a query >= the block's first key; window: the last
  // one holds the last query that sees the block's last key
  const int t_first = CAUSAL ? k0 / TQ : 0;
  const int q_end = WINDOW ? min(n, k0 + kKvBlk - 1 + window) : n;
  const int ntiles = (q_end + TQ - 1) / TQ - t_first;
  const int total = G * ntiles;  // (head, tile) steps
  const int64_t lstride = VARLEN ? (int64_t)cu_seqlens[nseq] : (int64_t)N;

  // step s: head g*G + s / ntiles, query tile t_first + s % ntiles
  auto issue = [&](char* qdst, char* gdst, float (*lddst)[256], int s) {
    const int h = g * G + s / ntiles;
    const int q0 = (t_first + s % ntiles) * TQ;
    const int64_t base = ((int64_t)(seq_start + q0) * Hq + h) * D * 2;
    const int rem = nbytes - q0 * rowbytes;
    copy_rows_to_lds<NI, IPB>(reinterpret_cast<const char*>(q) + base, rem, qdst + wave * NI * 1024, voff,
                              blk_bytes);
    copy_rows_to_lds<NI, IPB>(reinterpret_cast<const char*>(dout) + base, rem, gdst + wave * NI * 1024, voff,
                              blk_bytes);
    if (wave == 0) {  // L and D of the tile's queries (TQ floats each; queries past n read as 0)
      const int64_t lrow = VARLEN ? (int64_t)h * lstride + seq_start + q0 : ((int64_t)b * Hq + h) * N + q0;
      const int bytes = (n - q0) * 4;
#if defined(__HIP_DEVICE_COMPILE__)
      __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc((void*)(lse + lrow), 0, bytes, 0x00020000);
      __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc((void*)(delta + lrow), 0, bytes, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, LDS_PTR(void, lddst[0]), 16, 16 * lane, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, LDS_PTR(void, lddst[1]), 16, 16 * lane, 0, 0, 0);
#endif
    }
  };

  f32x16 dka[NB_D], dva[NB_D];
#pragma unroll
  for (int i = 0; i < NB_D; ++i) dka[i] = dva[i] = f32x16{};
  // read-ahead of the two product streams (operands of two dP products fill as many registers
  // as four of the others)
  constexpr int PD1 = 2, PD2 = 4;
  const float c = alpha * kLog2e;

  auto compute = [&](const char* qt, const char* gt, float (*ldt)[256], int s) {
    const int q0 = (t_first + s % ntiles) * TQ;
    if (CAUSAL && q0 + TQ - 1 < kw) return;  // every query of the tile is before this wave's keys
    if (WINDOW && q0 > kw + 31 + window - 1) return;  // every query is past this wave's windows
    f32x16 sc[NB], dp[NB];
    // first stage, products 0 .. NP-1: S = Q K^T (rows: queries; column: this lane's key), NP ..
    // 2NP-1: dP = dO V^T (V from the workgroup's LDS rows at d = 128, else from registers);
    // each 32-query block's k-steps in order
    constexpr int NP = NB * KS_D;
    struct Op2 {
      u32x4 a, b;
    };
    auto read1 = [&](int i) -> Op2 {
      const int ii = i % NP, cb = ii % NB, st = ii / NB;
      const char* t = i < NP ? qt : gt;
      const u32x4 a = *reinterpret_cast<const u32x4*>(t + koff[st & 1] + cb * 512 * NCH + 512 * (st & ~1));
      if (V_LDS && i >= NP)
        return Op2{a, *reinterpret_cast<const u32x4*>(vres + koff[st & 1] + wave * 512 * NCH + 512 * (st & ~1))};
      return Op2{a, u32x4{}};
    };
    auto product1 = [&](int i, Op2 o) {
      const int ii = i % NP, cb = ii % NB, st = ii / NB;
      if (i < NP) {
        sc[cb] = mma32<BF16>(o.a, kf[st], st == 0 ? f32x16{} : sc[cb]);
      } else {
        if constexpr (V_LDS) dp[cb] = mma32<BF16>(o.a, o.b, st == 0 ? f32x16{} : dp[cb]);
        else dp[cb] = mma32<BF16>(o.a, vf[st], st == 0 ? f32x16{} : dp[cb]);
      }
    };
    auto pin1 = [](int i) {
      if (V_LDS && i >= NP) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    };
    Op2 win1[PD1];
    product_stream<2 * NP, PD1, false>(read1, product1, pin1, win1);
    __builtin_amdgcn_sched_barrier(0);
    // second stage: per k-step st, dV^T += dO^T P over the d blocks, then dK^T += Q^T dS; the
    // first PD2 operands are read before the softmax
    auto read2 = [&](int i) {
      const int st = i / (2 * NB_D), w = i % (2 * NB_D);
      return tr_operand<D>(w < NB_D ? gt : qt, vtoff, st, w % NB_D);
    };
    u32x4 win2[PD2];
    prime<PD2>(read2, win2);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PD2, 0);
    // P = exp(S - L) (the query of each accumulator row picks its L and D from LDS)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 L = *reinterpret_cast<const float4*>(&ldt[0][32 * cb + 8 * r4 + 4 * hi]);
        const float Lr[4] = {L.x, L.y, L.z, L.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sc[cb][4 * r4 + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[cb][4 * r4 + e], c, -Lr[e] * kLog2e));
      }
    const bool mask = (q0 + TQ > n) || (CAUSAL && q0 < kw + 31) || (WINDOW && q0 + TQ - 1 > kw + window - 1);
    if (mask) {
      asm volatile("");  // keeps the edge tiles' masking a branch (not selects on every tile)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = q0 + 32 * cb + acc_row(r, hi);
          if constexpr (WINDOW) {  // visible iff 0 <= qi - kj < window
            if (qi >= n || (unsigned)(qi - kj) >= (unsigned)window) sc[cb][r] = 0.f;
          } else {
            if (qi >= n || (CAUSAL && qi < kj)) sc[cb][r] = 0.f;
          }
        }
    }
    // dS = P (dP - D)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 Dv = *reinterpret_cast<const float4*>(&ldt[1][32 * cb + 8 * r4 + 4 * hi]);
        const float Dr[4] = {Dv.x, Dv.y, Dv.z, Dv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[cb][4 * r4 + e] = sc[cb][4 * r4 + e] * (dp[cb][4 * r4 + e] - Dr[e]);
      }
    u32x4 pv[KS], pk[KS];
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      pv[st] = pack_step<BF16>(sc, st);
      pk[st] = pack_step<BF16>(dp, st);
    }
    __builtin_amdgcn_sched_barrier(0);
    auto product2 = [&](int i, u32x4 a) {
      const int st = i / (2 * NB_D), w = i % (2 * NB_D);
      if (w < NB_D) dva[w] = mma32<BF16>(a, pv[st], dva[w]);
      else dka[w - NB_D] = mma32<BF16>(a, pk[st], dka[w - NB_D]);
    };
    product_stream<KS * 2 * NB_D, PD2, true>(read2, product2, Pin2{}, win2);
  };

  issue(qt0, gt0, ld0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // Unrolled by two, every LDS read names its buffer, and the compiler can tell it from the one
  // the next step's copies are filling.  With one body for both stages (buffers chosen at run
  // time) it waits for those copies before the step's first read of L.  The second inlined
  // copy of compute fits the registers of two waves per SIMD at d = 64 and for causal d = 128
  // (one spilled register, outside the loop); non-causal d = 128 would spill in the loop, so it
  // keeps the single body.
  constexpr bool UNROLL = D == 64 || CAUSAL;
  if constexpr (UNROLL) {
    for (int s = 0; s < total; s += 2) {
      if (s + 1 < total) issue(qt1, gt1, ld1, s + 1);
      compute(qt0, gt0, ld0, s);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (s + 1 >= total) break;
      if (s + 2 < total) issue(qt0, gt0, ld0, s + 2);
      compute(qt1, gt1, ld1, s + 1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  } else {
    for (int s = 0; s < total; ++s) {
      const bool odd = s & 1;
      if (s + 1 < total) issue(odd ? qt0 : qt1, odd ? gt0 : gt1, odd ? ld0 : ld1, s + 1);
      compute(odd ? qt1 : qt0, odd ? gt1 : gt0, odd ? ld1 : ld0, s);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  if (kj < n) {
    const int64_t off = ((int64_t)(seq_start + kj) * Hkv + g) * D;
    store_rows<D, BF16>(dk + off, dka, alpha, hi);
    store_rows<D, BF16>(dv + off, dva, 1.f, hi);
  }
}

// ---- dQ -----------------------------------------------------------------------------------------
template <int D, bool BF16, bool CAUSAL, bool VARLEN, bool WINDOW>
__global__ __launch_bounds__(64 * kWaves, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dq, int Hq, int Hkv, int N, const int* __restrict__ cu_seqlens, int nseq, float alpha,
    int num_qblocks, int window) {
  constexpr int NCH = D / 8, KS_D = D / 16, NB_D = D / 32;
  constexpr int TILE = kTile * D * 2;
  constexpr int NI = TILE / 1024 / kWaves, IPB = NCH / 4;
  constexpr int NB = kTile / 32, KS = kTile / 16;
  static_assert(NI * kWaves * 1024 == TILE && (NI % IPB == 0 || NI < IPB), "tile shape");
  __shared__ __attribute__((aligned(1024))) char kt0[TILE];
  __shared__ __attribute__((aligned(1024))) char kt1[TILE];
  __shared__ __attribute__((aligned(1024))) char vt0[TILE];
  __shared__ __attribute__((aligned(1024))) char vt1[TILE];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;

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
  const int q0 = qb * kBlk;
  if (q0 >= n) return;
  const int g = h / (Hq / Hkv);
  const int qw = q0 + wave * 32;
  const int qi = qw + l32;

  // Q and dO of this lane's query (B operands), its L and D
  u32x4 qf[KS_D], gf[KS_D];
  float Lc = 0.f, Dq = 0.f;
  {
    const int row = qi < n ? qi : n - 1;
    const int64_t off = ((int64_t)(seq_start + row) * Hq + h) * D + 8 * hi;
#pragma unroll
    for (int s = 0; s < KS_D; ++s) {
      qf[s] = *reinterpret_cast<const u32x4*>(q + off + 16 * s);
      gf[s] = *reinterpret_cast<const u32x4*>(dout + off + 16 * s);
    }
    const int64_t idx = VARLEN ? (int64_t)h * cu_seqlens[nseq] + seq_start + row : ((int64_t)b * Hq + h) * N + row;
    Lc = lse[idx] * kLog2e;
    Dq = delta[idx];
  }
  int koff[2], vtoff[2];
  operand_offsets<D>(lane, koff, vtoff);

  const int rowbytes = Hkv * D * 2;
  const int voff = copy_offset<D, kTile, kWaves>(wave, lane, rowbytes);
  const int blk_bytes = 16 * rowbytes;
  const char* kbase = reinterpret_cast<const char*>(k) + ((int64_t)seq_start * Hkv + g) * D * 2;
  const char* vbase = reinterpret_cast<const char*>(v) + ((int64_t)seq_start * Hkv + g) * D * 2;
  const int nbytes = (n - 1) * rowbytes + D * 2;
  const int kv_end = CAUSAL ? min(n, q0 + kBlk) : n;
  // window: the loop counts key tiles from t0, the first one the block's first query sees
  const int t0 = WINDOW ? max(0, q0 - window + 1) / kTile : 0;
  const int ntiles = (kv_end + kTile - 1) / kTile - t0;
  auto issue = [&](char* kdst, char* vdst, int j) {
    const int off = (t0 + j) * kTile * rowbytes;
    copy_rows_to_lds<NI, IPB>(kbase + off, nbytes - off, kdst + wave * NI * 1024, voff, blk_bytes);
    copy_rows_to_lds<NI, IPB>(vbase + off, nbytes - off, vdst + wave * NI * 1024, voff, blk_bytes);
  };

  f32x16 dqa[NB_D];
#pragma unroll
  for (int i = 0; i < NB_D; ++i) dqa[i] = f32x16{};
  const float c = alpha * kLog2e;

  auto compute = [&](const char* kt, const char* vt, int j) {
    const int j0 = (t0 + j) * kTile;
    if (CAUSAL && j0 > qw + 31) return;  // the tile lies wholly after this wave's queries
    if (WINDOW && j0 + kTile - 1 <= qw - window) return;  // wholly before this wave's windows
    f32x16 sc[NB], dp[NB];
    // products 0 .. NP-1: S^T = K Q^T (rows: keys; column: this lane's query), NP .. 2NP-1:
    // dP^T = V dO^T; the 32-key blocks alternate, each block's k-steps in order
    constexpr int NP = NB * KS_D, PD1 = 4, PD2 = 4;
    auto read1 = [&](int i) {
      const char* t = i < NP ? kt : vt;
      const int ii = i % NP, cb = ii % NB, st = ii / NB;
      return *reinterpret_cast<const u32x4*>(t + koff[st & 1] + cb * 512 * NCH + 512 * (st & ~1));
    };
    auto product1 = [&](int i, u32x4 a) {
      const int ii = i % NP, cb = ii % NB, st = ii / NB;
      if (i < NP) sc[cb] = mma32<BF16>(a, qf[st], st == 0 ? f32x16{} : sc[cb]);
      else dp[cb] = mma32<BF16>(a, gf[st], st == 0 ? f32x16{} : dp[cb]);
    };
    u32x4 win[PD1 > PD2 ? PD1 : PD2];
    product_stream<2 * NP, PD1, false>(read1, product1, Pin1{}, win);
    __builtin_amdgcn_sched_barrier(0);
    // dQ^T += K^T dS^T: product i is k-step i / NB_D of d block i % NB_D, its operand K read
    // transposed (two reads); the first PD2 are read before the softmax below
    auto read2 = [&](int i) { return tr_operand<D>(kt, vtoff, i / NB_D, i % NB_D); };
    prime<PD2>(read2, win);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PD2, 0);
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[cb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[cb][r], c, -Lc));
    const bool mask = (j0 + kTile > n) || (CAUSAL && j0 + kTile - 1 > qw) || (WINDOW && j0 <= qw + 31 - window);
    if (mask) {
      asm volatile("");  // keeps the edge tiles' masking a branch (not selects on every tile)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 32 * cb + acc_row(r, hi);
          if constexpr (WINDOW) {  // visible iff 0 <= qi - key < window
            if (key >= n || (unsigned)(qi - key) >= (unsigned)window) sc[cb][r] = 0.f;
          } else {
            if (key >= n || (CAUSAL && key > qi)) sc[cb][r] = 0.f;
          }
        }
    }
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[cb][r] = sc[cb][r] * (dp[cb][r] - Dq);
    u32x4 ds[KS];
#pragma unroll
    for (int st = 0; st < KS; ++st) ds[st] = pack_step<BF16>(dp, st);
    __builtin_amdgcn_sched_barrier(0);
    auto product2 = [&](int i, u32x4 a) {
      const int st = i / NB_D, db = i % NB_D;
      dqa[db] = mma32<BF16>(a, ds[st], dqa[db]);
    };
    product_stream<KS * NB_D, PD2, true>(read2, product2, Pin2{}, win);
  };

  issue(kt0, vt0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int j = 0; j < ntiles; j += 2) {
    if (j + 1 < ntiles) issue(kt1, vt1, j + 1);
    compute(kt0, vt0, j);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (j + 1 >= ntiles) break;
    if (j + 2 < ntiles) issue(kt0, vt0, j + 2);
    compute(kt1, vt1, j + 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (qi < n) store_rows<D, BF16>(dq + ((int64_t)(seq_start + qi) * Hq + h) * D, dqa, alpha, hi);
}

template <int D, bool BF16, bool CAUSAL, bool VARLEN, bool WINDOW = false>
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
  const int nblk = (a.N + kBlk - 1) / kBlk, nkv = (a.N + kKvBlk - 1) / kKvBlk;
  const long long grid_kv = (long long)nkv * a.Hkv * a.B, grid_q = (long long)nblk * a.Hq * a.B;
  if (grid_q > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  // delta: one row per (token, query head); the grid covers the B * N tokens packed input can hold
  const int64_t blocks = ((int64_t)a.B * a.N * a.Hq * (D / 8) + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((bwd_delta_kernel<D, BF16>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a.o), static_cast<const uint16_t*>(a.dout), a.workspace, a.Hq, a.N,
                     a.B, a.cu_seqlens);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, BF16, CAUSAL, VARLEN, WINDOW>), dim3((unsigned)grid_kv), dim3(64 * kKvWaves), 0,
                     stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.dout), a.lse, a.workspace,
                     static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv), a.Hq, a.Hkv, a.N, a.cu_seqlens, a.B,
                     a.alpha, nkv, a.window);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((bwd_dq_kernel<D, BF16, CAUSAL, VARLEN, WINDOW>), dim3((unsigned)grid_q), dim3(64 * kWaves), 0, stream,
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.dout), a.lse, a.workspace,
                     static_cast<uint16_t*>(a.dq), a.Hq, a.Hkv, a.N, a.cu_seqlens, a.B, a.alpha, nblk, a.window);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_bwd_modes(const BwdArgs& a, hipStream_t stream) {
  const bool varlen = a.cu_seqlens != nullptr;
  if (a.window > 0)
    return varlen ? launch_bwd<D, BF16, true, true, true>(a, stream) : launch_bwd<D, BF16, true, false, true>(a, stream);
  if (a.causal) return varlen ? launch_bwd<D, BF16, true, true>(a, stream) : launch_bwd<D, BF16, true, false>(a, stream);
  return varlen ? launch_bwd<D, BF16, false, true>(a, stream) : launch_bwd<D, BF16, false, false>(a, stream);
}

}  // namespace

hipError_t launch_bwd_16bit(const BwdArgs& a, bool is_bf16, hipStream_t stream) {
  switch (a.d) {
    case 64: return is_bf16 ? launch_bwd_modes<64, true>(a, stream) : launch_bwd_modes<64, false>(a, stream);
    case 128: return is_bf16 ? launch_bwd_modes<128, true>(a, stream) : launch_bwd_modes<128, false>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
