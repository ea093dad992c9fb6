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
//   * A workgroup of eight waves owns 256 queries of one (sequence, head); each wave owns 32.
//   * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_{bf16,f16}: the
//     32x32 accumulator of a wave then holds one query per lane column, so the row max and
//     row sum are in-lane plus a single exchange between the two lane halves.
//   * The P^T accumulator is fed straight back as the B operand of O^T = V^T P^T.  The keys a
//     lane holds in its accumulator are not contiguous; the V transpose reads
//     (ds_read_b64_tr_b16) pick, per operand slot, the key that accumulator register holds.
//     (This is the freedom the digest's section 3.5 describes for the FP8 accumulator-to-
//     operand layout: permuting P's columns together with V's rows leaves P V unchanged.)
//   * K and V tiles are copied buffer-to-LDS (no registers, no VALU) while earlier tiles are
//     multiplied.  Two loops: the plain one (two K and two V buffers, one barrier per tile,
//     the two waves of a SIMD overlapping freely) and, for d = 256 and d = 128 (short non-causal
//     sequences aside), a ping-pong loop
//     (the digest's section 3.3 idea, enforced with workgroup barriers): the two halves of the
//     workgroup run one phase apart, so that on every SIMD one wave multiplies while the other
//     takes its softmax; operand reads run a few products ahead of the matrix instructions,
//     and K/V rotate through three buffers.  Short dense non-causal d = 128 inputs run the plain
//     loop in persistent workgroups (one per CU, each taking a fixed share of the query blocks
//     in turn and fetching the next block's first tile and Q during the current block), the
//     persistent scheduling the digest's section 9 names for short sequences.
//   * exp2 with the scale alpha*log2(e) folded into one FMA per score.
//   * Work decomposition: each XCD (dispatch is round-robin over the 8 XCDs) owns the same
//     heads of every sequence, whole KV groups where possible, so that packed sequences of
//     unequal length load the XCDs alike and a group's query heads share its K/V in the XCD's
//     L2; causal grids run their longest query blocks first.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "decompose.h"
#include "internal.h"
#include "tile16.h"

namespace attn {
namespace {

// Tile-loop shape of one (d, BC) instance:
//   WAVES     waves per workgroup, 32 queries each (the workgroup owns 32 * WAVES queries);
//   PP        ping-pong: the waves of the two halves of the workgroup (one of each per SIMD)
//             run one phase apart, so that one half's products and the other half's softmax
//             occupy a SIMD at the same time (see the main loop).  Otherwise the plain loop,
//             which takes a tile's exponentials one k-step at a time next to that k-step's
//             products.
//   PD        (ping-pong only) how many products ahead the LDS operand reads are issued.
//   PERSIST   (plain loop, non-causal dense inputs) a workgroup takes the query blocks
//             blockIdx.x, blockIdx.x + G, ... (G workgroups, one per CU) in turn, as one stream
//             of key tiles: the next block's first K/V tile is copied while the current block's
//             last tile is multiplied, and its Q fragment loaded during the current block's first
//             tile, so no block pays its start-up alone.  Every block must have an even number of
//             key tiles (the two buffers then alternate the same way in every block).
template <int WAVES_, bool PP_ = false, int PD_ = 4, bool PERSIST_ = false>
struct LoopShape {
  static constexpr int WAVES = WAVES_;
  static constexpr bool PP = PP_;
  static constexpr int PD = PD_;
  static constexpr bool PERSIST = PERSIST_;
};

// Workgroup barrier between ping-pong phases.  The asm statement is a compiler memory barrier
// (no LDS access moves across it); LDS reads of this wave are complete before it arrives.
__device__ __forceinline__ void phase_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// WINDOW (implies CAUSAL): causal sliding window of `window` keys; otherwise `window` is unused.
// `blocks`: the number of (sequence, head, query block) work items (used by PERSIST only).
template <int D, int BC, typename SH, bool BF16, bool CAUSAL, bool VARLEN, bool WINDOW>
__global__ __launch_bounds__(64 * SH::WAVES) void fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, float* __restrict__ lse, int Hq, int Hkv, int N,
    const int* __restrict__ cu_seqlens, int nseq, float alpha, int num_qblocks, int window, int blocks) {
  constexpr int WAVES = SH::WAVES;
  constexpr int BR = 32 * WAVES;                   // queries per workgroup
  constexpr int NCH = D / 8;                       // 16-byte chunks per row
  constexpr int TILE_BYTES = BC * D * 2;
  constexpr int NI = TILE_BYTES / 1024 / WAVES;    // 1 KB copies per wave per tensor
  constexpr int IPB = NCH / 4;                     // copies per 16-row block
  constexpr int KS_D = D / 16;                     // k-steps of the first product (over d)
  constexpr int KS_C = BC / 16;                    // k-steps of the second product (over keys)
  constexpr int NB_C = BC / 32;                    // 32-key accumulator blocks per tile
  constexpr int NB_D = D / 32;                     // 32-wide d blocks of the O accumulator
  static_assert(BC % 32 == 0 && D % 32 == 0 && NI * WAVES * 1024 == TILE_BYTES && (NI % IPB == 0 || NI < IPB),
                "tile shape");

  // two (ping-pong: three) K and V tile buffers; separate objects so the compiler can tell
  // them apart
  constexpr int NBUF = SH::PP ? 3 : 2;
  __shared__ __attribute__((aligned(1024))) char kb0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char kb1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char kb2[NBUF > 2 ? TILE_BYTES : 1];
  __shared__ __attribute__((aligned(1024))) char vb0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vb2[NBUF > 2 ? TILE_BYTES : 1];
  // persistent shape: each wave's 32 rows of O, staged between blocks
  // (placed after the K/V buffers, whose operand reads then keep addresses below 64 KB that
  // fit the LDS instructions' immediate offsets)
  __shared__ __attribute__((aligned(16))) char ob[SH::PERSIST ? WAVES * 32 * D * 2 : 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;

  // ---- which (sequence, head, query block) ----
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
  int q0 = qb * BR;
  if (q0 >= n) return;  // whole workgroup: block lies past the end of this sequence
  int g = h / (Hq / Hkv);
  const int64_t qstride = (int64_t)Hq * D;
  const int rowbytes = Hkv * D * 2;  // distance between consecutive tokens of one K/V head

  // ---- Q fragment of this lane: query qi, d = 16*st + 8*hi .. +7 ----
  int qw = q0 + wave * 32;  // first query of this wave
  int qi = qw + l32;        // this lane's query (within the sequence)
  // Q fragment of the block (seq_start_, h_, q0_) into dst
  auto load_q = [&](int seq_start_, int h_, int q0_, u32x4* dst) {
    const int qi_ = q0_ + wave * 32 + l32;
    const int row = qi_ < n ? qi_ : n - 1;
    const uint16_t* qp = q + (int64_t)(seq_start_ + row) * qstride + (int64_t)h_ * D + 8 * hi;
#pragma unroll
    for (int s = 0; s < KS_D; ++s) dst[s] = *reinterpret_cast<const u32x4*>(qp + 16 * s);
  };
  u32x4 qf[KS_D];
  load_q(seq_start, h, q0, qf);

  // ---- K/V copies ----
  int voff;
  {
    int row, chunk;
    tile_row_chunk<D>(wave * NI * 64 + lane, row, chunk);
    voff = row * rowbytes + chunk * 16;
  }
  const int blk_bytes = 16 * rowbytes;
  // byte offset of the K (and V) rows of KV head g_ of the sequence starting at token seq_start_
  auto kv_head = [&](int seq_start_, int g_) { return ((int64_t)seq_start_ * Hkv + g_) * D * 2; };
  const char* kbase = reinterpret_cast<const char*>(k) + kv_head(seq_start, g);
  const char* vbase = reinterpret_cast<const char*>(v) + kv_head(seq_start, g);
  const int nbytes = (n - 1) * rowbytes + D * 2;  // bytes of this head's K (or V) rows
  // rows at or past n fall outside the buffer and read as zero
  auto issue_tile_from = [&](const char* kb, const char* vb, char* kdst, char* vdst, int tile) {
    const int off = tile * BC * rowbytes;
    copy_rows_to_lds<NI, IPB>(kb + off, nbytes - off, kdst + wave * NI * 1024, voff, blk_bytes);
    copy_rows_to_lds<NI, IPB>(vb + off, nbytes - off, vdst + wave * NI * 1024, voff, blk_bytes);
  };
  auto issue_tile = [&](char* kdst, char* vdst, int tile) { issue_tile_from(kbase, vbase, kdst, vdst, tile); };

  // ---- operand read offsets (bytes inside a tile), lane part ----
  // K (A operand of S^T = K Q^T): row 32*cb + l32, chunk 2*st + hi; the XOR term depends on st&1
  int koff[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
    koff[e] = 16 * ((l32 >> 4) * 16 * NCH + (2 * e + hi) * 16 + ((lane & 15) ^ (4 * (2 * e + hi))));
  // V (A operand of O^T = V^T P^T) by transpose reads: lane 16G + 4r + c reads 8 bytes of row
  // 16*st + 4*(G/2) + 8*rd + r, chunk 4*db + 2*(G%2) + c/2, half c%2
  int vtoff[2];
  {
    const int G = lane >> 4, r = (lane >> 2) & 3, c = lane & 3;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int chunk = 2 * (G & 1) + (c >> 1);
      const int rowm = 4 * (G >> 1) + 8 * rd + r;
      vtoff[rd] = 16 * (chunk * 16 + (rowm ^ (4 * chunk))) + 8 * (c & 1);
    }
  }

  f32x16 oacc[NB_D];
#pragma unroll
  for (int i = 0; i < NB_D; ++i) oacc[i] = f32x16{};
  float m = -INFINITY;  // running max of raw scores q.k (the stabiliser; may trail the true max)
  float l = 0.f;        // running sum over this lane's keys (lane halves are added at the end)
  const float c = alpha * kLog2e;
  // derived from m, updated only when m changes: the rescale threshold in units of the scores
  // (m + 8 / c; -inf while m is) and the stabiliser m c (0 while m = -inf)
  float thr = -INFINITY;
  float mc_cur = 0.f;
  const float slack_s = 8.f / c;

  static_assert(!WINDOW || CAUSAL, "a sliding window is causal");
  const int kv_end = CAUSAL ? min(n, q0 + BR) : n;
  // Sliding window: query i sees keys i-window+1 .. i.  Tiles before t0 hold no key any query
  // of the workgroup sees; the loops count tiles from t0.
  const int t0 = WINDOW ? max(0, q0 - window + 1) / BC : 0;
  const int ntiles = (kv_end + BC - 1) / BC - t0;
  // whether this wave sees any key of loop tile j (it still copies and passes the barriers)
  auto wave_needs = [&](int j) {
    const int k0 = (t0 + j) * BC;
    return !CAUSAL || (k0 <= qw + 31 && (!WINDOW || k0 + BC - 1 > qw - window));
  };

  // S^T = K Q^T: lane holds query qi, keys k0 + 32*cb + 8*(r/4) + 4*hi + r%4
  auto gemm1 = [&](const char* ks, f32x16* s) {
#pragma unroll
    for (int cb = 0; cb < NB_C; ++cb) {
      s[cb] = f32x16{};
#pragma unroll
      for (int st = 0; st < KS_D; ++st) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(ks + koff[st & 1] + cb * 512 * NCH + 512 * (st & ~1));
        s[cb] = mma32<BF16>(a, qf[st], s[cb]);
      }
    }
  };
  // Mask, running maximum and lazy rescale of loop tile j; returns the stabiliser m*c.  A lane
  // whose keys in the tile are all masked keeps m = -inf and adds nothing.
  auto update_max = [&](f32x16* s, int j) -> float {
    const int k0 = (t0 + j) * BC;
    const bool need_mask = (k0 + BC > n) || (CAUSAL && (k0 + BC - 1 > qw || (WINDOW && k0 <= qw + 31 - window)));
    if (need_mask) {
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
    // Rescale only when some row's maximum grew by more than 2^8 in the exp2 domain; otherwise
    // keep the old stabiliser (P then stays below about 2^8).  O / l and L are exact either way.
    // The test needs no row maximum: some lane's maximum over its half of the keys exceeds the
    // threshold exactly when some row's does.  The branch is uniform, so the lane swap is safe.
    if (__builtin_amdgcn_ballot_w64(mt > thr)) {
      mt = halves_max(mt);
      const float mnew = fmaxf(m, mt);
      const float corr = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - mnew) * c);
      m = mnew;
      l *= corr;
#pragma unroll
      for (int db = 0; db < NB_D; ++db) oacc[db] *= corr;
      thr = m + slack_s;
      mc_cur = (m == -INFINITY) ? 0.f : m * c;
    }
    return mc_cur;
  };
  // O^T += V^T P^T for one k-step (16 keys): accumulator registers 8*(st%2) .. +7 of block st/2
  auto gemm2_step = [&](const char* vs, int st, u32x4 pf) {
#pragma unroll
    for (int db = 0; db < NB_D; ++db) {
      const int imm = st * 256 * NCH + db * 1024;
      const s16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vs + vtoff[0] + imm));
      const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vs + vtoff[1] + imm));
      const u32x2 a0 = __builtin_bit_cast(u32x2, t0), a1 = __builtin_bit_cast(u32x2, t1);
      oacc[db] = mma32<BF16>(u32x4{a0[0], a0[1], a1[0], a1[1]}, pf, oacc[db]);
    }
  };

  auto compute_tile = [&](const char* ks, const char* vs, int j) {
    f32x16 s[NB_C];
    gemm1(ks, s);
    const float mc = update_max(s, j);
    float rs0 = -0.f, rs1 = -0.f;  // -0 + p = p exactly, so the first adds fold away
#pragma unroll
    for (int st = 0; st < KS_C; ++st) {
      const int cb = st >> 1, base = (st & 1) * 8;
      float p[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        p[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[cb][base + t], c, -mc));
        if (t & 1) rs1 += p[t]; else rs0 += p[t];
      }
      gemm2_step(vs, st, u32x4{pack2<BF16>(p[0], p[1]), pack2<BF16>(p[2], p[3]), pack2<BF16>(p[4], p[5]),
                               pack2<BF16>(p[6], p[7])});
    }
    l += rs0 + rs1;
  };

  // ---- epilogue of the current block: O / l, L = alpha*m + ln l ----
  auto finish = [&]() {
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
  };

  if constexpr (SH::PERSIST) {
    // ---- persistent stream of blocks: this workgroup's blocks blockIdx.x + i * G ----
    // G is a multiple of 8 whenever a workgroup takes more than one block, so all of them belong
    // to its XCD's share of the decomposition.  Each block has ntiles (even) tiles: tile j of a
    // block sits in buffer j % 2, and the next block's tile 0 is copied into buffer 0 while the
    // current block's last tile (buffer 1) is multiplied.
    static_assert(!SH::PP && !CAUSAL && !VARLEN && !WINDOW, "persistent blocks: plain loop, non-causal, dense");
    // A finished block's O goes out through LDS: each wave writes its 32 rows of D 16-bit values
    // row-major into its own LDS area (the 16-byte chunks of row r at chunk ^ (r mod 16), so that
    // both the writes and the reads back are free of bank conflicts), then stores four whole rows
    // (1 KB of 128-byte lines) per instruction.  Straight from the accumulators, every store
    // would touch 32 rows at 16 bytes each; those stores take longer to drain, and the next
    // block's first copy wait waits for them.
    constexpr int ROWB = D * 2;
    static_assert(ROWB == 256, "the write-out assumes 16 chunks of 16 bytes per row");
    auto finish_staged = [&]() {
      char* const ow = ob + wave * 32 * ROWB;
      const float lt = halves_sum(l);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int db = 0; db < NB_D; ++db)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const u32x2 pr = {pack2<BF16>(oacc[db][4 * gq + 0] * inv, oacc[db][4 * gq + 1] * inv),
                            pack2<BF16>(oacc[db][4 * gq + 2] * inv, oacc[db][4 * gq + 3] * inv)};
          *LDS_PTR(u32x2, ow + l32 * ROWB + (((4 * db + gq) ^ (l32 & 15)) * 16) + 8 * hi) = pr;
        }
      if (hi == 0 && qi < n) lse[((int64_t)b * Hq + h) * N + qi] = lt > 0.f ? m * alpha + __logf(lt) : -INFINITY;
      // step t: lane (lr = lane / 16, cc = lane % 16) stores chunk cc of row r = 4t + lr, held at
      // chunk cc ^ (r mod 16) = (cc ^ lr) ^ 4 (t mod 4) of its LDS row
      const int lr = lane >> 4, cc = lane & 15;
      const int src = lr * ROWB + ((cc ^ lr) * 16);
      char* const dst = reinterpret_cast<char*>(o + (int64_t)(seq_start + qw + lr) * qstride + (int64_t)h * D) + cc * 16;
      const int rows = min(32, n - qw);
#pragma unroll
      for (int t = 0; t < 32 / 4; ++t) {
        const u32x4 x = *LDS_PTR(u32x4, ow + t * 4 * ROWB + (src ^ (64 * (t & 3))));
        if (4 * t + lr < rows) *reinterpret_cast<u32x4*>(dst + (int64_t)t * 4 * qstride * 2) = x;
      }
    };
    const int G = gridDim.x;
    const int mine = (blocks - (int)blockIdx.x + G - 1) / G;
    u32x4 qn[KS_D];
    issue_tile(kb0, vb0, 0);
    __builtin_amdgcn_s_waitcnt(0);  // Q fragments and the first tile have arrived
    __syncthreads();
    for (int i = 0;; ++i) {
      const bool more = i + 1 < mine;
      int nqb = 0, nh = 0, nb = 0;
      if (more) decompose<false>((int)blockIdx.x + (i + 1) * G, num_qblocks, Hq, Hkv, nseq, nqb, nh, nb);
      const int ng = nh / (Hq / Hkv);
      const char* nkbase = reinterpret_cast<const char*>(k) + kv_head(nb * N, ng);
      const char* nvbase = reinterpret_cast<const char*>(v) + kv_head(nb * N, ng);
      for (int j = 0; j < ntiles; j += 2) {
        issue_tile(kb1, vb1, j + 1);
        if (j == 0 && more) load_q(nb * N, nh, nqb * BR, qn);  // held through this block
        compute_tile(kb0, vb0, j);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (j + 2 < ntiles) issue_tile(kb0, vb0, j + 2);
        else if (more) issue_tile_from(nkbase, nvbase, kb0, vb0, 0);
        compute_tile(kb1, vb1, j + 1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
      finish_staged();
      if (!more) return;
      // the next block becomes the current one, with a fresh online softmax
#pragma unroll
      for (int db = 0; db < NB_D; ++db) oacc[db] = f32x16{};
      m = -INFINITY;
      l = 0.f;
      thr = -INFINITY;
      mc_cur = 0.f;
#pragma unroll
      for (int s = 0; s < KS_D; ++s) qf[s] = qn[s];
      h = nh;
      b = nb;
      seq_start = nb * N;
      q0 = nqb * BR;
      qw = q0 + wave * 32;
      qi = qw + l32;
      kbase = nkbase;
      vbase = nvbase;
    }
  } else if constexpr (!SH::PP) {
    // ---- main loop: two buffer pairs, unrolled by two so each half names its buffers ----
    issue_tile(kb0, vb0, t0);
    __builtin_amdgcn_s_waitcnt(0);  // Q fragments and the first tile have arrived
    __syncthreads();
    for (int j = 0; j < ntiles; j += 2) {
      if (j + 1 < ntiles) issue_tile(kb1, vb1, t0 + j + 1);
      if (wave_needs(j)) compute_tile(kb0, vb0, j);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (j + 1 >= ntiles) break;
      if (j + 2 < ntiles) issue_tile(kb0, vb0, t0 + j + 2);
      if (wave_needs(j + 1)) compute_tile(kb1, vb1, j + 1);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  } else {
    // ---- ping-pong main loop ----
    // Every wave runs the phases M_0 V_0 M_1 V_1 ... M_J (J tiles): M_j multiplies P_{j-1} by
    // V_{j-1} (second product of the previous tile) and forms S_j = K_j Q^T; V_j takes the
    // softmax of S_j into the packed P_j.  A barrier ends every phase.  The second half of the
    // workgroup (waves HW..) passes one extra barrier at the start, so it runs one phase behind
    // the first half: while one wave of a SIMD multiplies, the other takes exponentials.
    // Barrier step t holds phase t of the first half and phase t-1 of the second half.
    // Tiles rotate through three K and three V buffers (tile j in kb[j%3], vb[j%3]).  In its
    // phase V_j the first half copies K_{j+2} (step 2j+1) and the second half copies V_{j+1}
    // (step 2j+2); both buffers were last read in the phases M_{j-1} (steps 2j-2, 2j-1).  Each
    // half waits for its copies at the end of its next M phase (steps 2j+2 and 2j+3); both
    // tiles are first read in the first half's M_{j+2}, at step 2j+4.
    constexpr int HW = WAVES / 2;
    constexpr int NIB = TILE_BYTES / 1024 / HW;  // copies per wave per tile
    static_assert(NIB * HW * 1024 == TILE_BYTES && (NIB % IPB == 0 || NIB < IPB), "copy split");
    const bool second = wave >= HW;
    const int wb = wave % HW;
    int voffb;
    {
      int row, chunk;
      tile_row_chunk<D>(wb * NIB * 64 + lane, row, chunk);
      voffb = row * rowbytes + chunk * 16;
    }
    // copies of this wave's part of loop tile j; a tile past the end reads as zero
    auto copy = [&](const char* base, char* dst, int j) {
      const int64_t off = (int64_t)(t0 + j) * BC * rowbytes;
      const int rem = off < nbytes ? (int)(nbytes - off) : 0;
      copy_rows_to_lds<NIB, IPB>(base + (rem ? off : 0), rem, dst + wb * NIB * 1024, voffb, blk_bytes);
    };
    // loop tiles jlo .. jw-1 hold keys this wave sees (causal: up to its diagonal, and from its
    // first query's window on)
    const int jw = CAUSAL ? min(ntiles, (qw + 31) / BC + 1 - t0) : ntiles;
    const int jlo = WINDOW ? max(0, qw - window + 1) / BC - t0 : 0;
    f32x16 s[NB_C];
    u32x4 pf[KS_C];
    // An M phase is one stream of products (the second product of the previous tile, then the
    // first product of this tile) whose LDS operands are read PD products ahead.  In the first
    // product the 32-key blocks alternate, so consecutive matrix instructions do not accumulate
    // into the same registers.
    constexpr int N2 = KS_C * NB_D, N1 = NB_C * KS_D, PD = SH::PD;
    auto operand = [&](const char* ks, const char* vs, int i) -> u32x4 {
      if (i < N2) {
        const int st = i / NB_D, db = i % NB_D;
        const int imm = st * 256 * NCH + db * 1024;
        const s16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vs + vtoff[0] + imm));
        const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(s16x4, vs + vtoff[1] + imm));
        const u32x2 a0 = __builtin_bit_cast(u32x2, t0), a1 = __builtin_bit_cast(u32x2, t1);
        return u32x4{a0[0], a0[1], a1[0], a1[1]};
      }
      const int cb = (i - N2) % NB_C, st = (i - N2) / NB_C;
      return *reinterpret_cast<const u32x4*>(ks + koff[st & 1] + cb * 512 * NCH + 512 * (st & ~1));
    };
    auto product = [&](int i, u32x4 a) {
      if (i < N2) {
        const int st = i / NB_D, db = i % NB_D;
        oacc[db] = mma32<BF16>(a, pf[st], oacc[db]);
      } else {
        const int cb = (i - N2) % NB_C, st = (i - N2) / NB_C;
        if (st == 0) s[cb] = f32x16{};
        s[cb] = mma32<BF16>(a, qf[st], s[cb]);
      }
    };
    // Every M phase from this wave's first tile to its last runs the whole stream: in M_jlo P is
    // still zero and the V buffer holds finite values (in M_0 a copy of V_0), so the second
    // product adds exact zeros; in M_jw the first product is formed and not used.
    auto mphase = [&](const char* ks, const char* vs, int j) {
      if (j >= jlo && j <= jw) {
        u32x4 win[PD];
#pragma unroll
        for (int i = 0; i < PD; ++i) win[i] = operand(ks, vs, i);
#pragma unroll
        for (int i = 0; i < N2 + N1; ++i) {
          const u32x4 a = win[i % PD];
          if (i + PD < N2 + N1) win[i % PD] = operand(ks, vs, i + PD);
          product(i, a);
        }
        // keep that order through instruction scheduling: the reads of the first PD operands,
        // then per product: the product, the reads of the operand PD places ahead (a V^T
        // operand is two LDS reads, a K operand one)
        auto reads = [](int i) {
          if (i < N2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        };
#pragma unroll
        for (int i = 0; i < PD; ++i) reads(i);
#pragma unroll
        for (int i = 0; i < N2 + N1; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i + PD < N2 + N1) reads(i + PD);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);  // this wave's copies (issued in the last V phase) have landed
    };
    // V phase: softmax of S_j into P_j; the copies of this phase are spread over it
    auto vphase = [&](char* kdst, char* vdst, int j) {
      if (!second) copy(kbase, kdst, j + 2);
      else copy(vbase, vdst, j + 1);
      if (j >= jlo && j < jw) {
        const float mc = update_max(s, j);
        float rs0 = -0.f, rs1 = -0.f;  // -0 + p = p exactly, so the first adds fold away
#pragma unroll
        for (int st = 0; st < KS_C; ++st) {
          const int cb = st >> 1, base = (st & 1) * 8;
          float p[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            p[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[cb][base + t], c, -mc));
            if (t & 1) rs1 += p[t]; else rs0 += p[t];
          }
          pf[st] = u32x4{pack2<BF16>(p[0], p[1]), pack2<BF16>(p[2], p[3]), pack2<BF16>(p[4], p[5]),
                         pack2<BF16>(p[6], p[7])};
        }
        l += rs0 + rs1;
      }
    };
    if (!second) {
      copy(kbase, kb0, 0);
      copy(kbase, kb1, 1);
    } else {
      copy(vbase, vb0, 0);
      copy(vbase, vb2, 0);  // read (times P = 0) by M_0
    }
#pragma unroll
    for (int st = 0; st < KS_C; ++st) pf[st] = u32x4{0, 0, 0, 0};
    __builtin_amdgcn_s_waitcnt(0);  // Q fragments and tiles K_0, K_1, V_0 have arrived
    __syncthreads();
    if (second) phase_barrier();
    for (int j = 0;; j += 3) {
      mphase(kb0, vb2, j);
      phase_barrier();
      if (j == ntiles) break;
      vphase(kb2, vb1, j);
      phase_barrier();
      mphase(kb1, vb0, j + 1);
      phase_barrier();
      if (j + 1 == ntiles) break;
      vphase(kb0, vb2, j + 1);
      phase_barrier();
      mphase(kb2, vb1, j + 2);
      phase_barrier();
      if (j + 2 == ntiles) break;
      vphase(kb1, vb0, j + 2);
      phase_barrier();
    }
    // the first half passes one barrier fewer in the loop; it joins the second half's last
    // barrier after its epilogue (below)
  }

  finish();
  if constexpr (SH::PP) {
    if (wave < WAVES / 2) phase_barrier();
  }
}

template <int D, int BC, typename SH, bool BF16, bool CAUSAL, bool VARLEN, bool WINDOW = false>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  constexpr int BR = 32 * SH::WAVES;
  const int nqb = (a.N + BR - 1) / BR;
  const long long grid = (long long)nqb * a.Hq * a.B;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_kernel<D, BC, SH, BF16, CAUSAL, VARLEN, WINDOW>), dim3((unsigned)grid), dim3(64 * SH::WAVES), 0,
                     stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.Hq, a.Hkv,
                     a.N, a.cu_seqlens, a.B, a.alpha, nqb, a.window, (int)grid);
  return hipGetLastError();
}

// Persistent blocks (LoopShape PERSIST, non-causal dense inputs): one workgroup per CU, at most
// as many as there are blocks; when there are more blocks than CUs, the grid is the CU count
// rounded down to a multiple of the 8 XCDs.
template <int D, int BC, typename SH, bool BF16>
hipError_t launch_persistent(const FwdArgs& a, hipStream_t stream) {
  static_assert(SH::PERSIST, "persistent loop shape");
  constexpr int BR = 32 * SH::WAVES;
  const int nqb = (a.N + BR - 1) / BR;
  const long long blocks = (long long)nqb * a.Hq * a.B;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  int dev = 0, cus = 0;
  hipError_t err = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  const long long slots = cus >= 8 ? cus / 8 * 8 : 1;
  const long long grid = blocks < slots ? blocks : slots;
  hipLaunchKernelGGL((fwd_kernel<D, BC, SH, BF16, false, false, false>), dim3((unsigned)grid), dim3(64 * SH::WAVES), 0,
                     stream, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse, a.Hq, a.Hkv,
                     a.N, nullptr, a.B, a.alpha, nqb, 0, (int)blocks);
  return hipGetLastError();
}

template <int D, int BC, typename SH, bool BF16>
hipError_t launch_modes(const FwdArgs& a, hipStream_t stream) {
  const bool varlen = a.cu_seqlens != nullptr;
  if (a.causal)
    return varlen ? launch<D, BC, SH, BF16, true, true>(a, stream) : launch<D, BC, SH, BF16, true, false>(a, stream);
  return varlen ? launch<D, BC, SH, BF16, false, true>(a, stream) : launch<D, BC, SH, BF16, false, false>(a, stream);
}

template <int D, int BC, typename SH, bool BF16>
hipError_t launch_noncausal(const FwdArgs& a, hipStream_t stream) {
  return a.cu_seqlens != nullptr ? launch<D, BC, SH, BF16, false, true>(a, stream)
                                 : launch<D, BC, SH, BF16, false, false>(a, stream);
}

template <int D, int BC, typename SH, bool BF16>
hipError_t launch_window(const FwdArgs& a, hipStream_t stream) {
  return a.cu_seqlens != nullptr ? launch<D, BC, SH, BF16, true, true, true>(a, stream)
                                 : launch<D, BC, SH, BF16, true, false, true>(a, stream);
}

// Per head dim: keys per tile and loop shape.  Eight waves (256 queries) per workgroup, one
// workgroup per CU: the K/V tile copies are shared by all eight waves.  d = 128 and d = 256 run
// the ping-pong loop (measured on MI355X: +4-7% over the plain loop); at d = 64 the softmax
// outweighs the products and the plain loop, which lets the two waves of a SIMD share the
// VALU freely, is as fast.  With a sliding window, d = 256 runs the plain loop: the window's
// bookkeeping does not fit the ping-pong loop's 256 registers without spilling.  Non-causal
// d = 128 with at most kShortKeys keys per sequence (eight tiles) runs the plain loop too: a
// workgroup then lives for only a few tiles, and the ping-pong loop's extra phase at either
// end (the second half starts one phase late and finishes one phase after the first) costs
// more than its overlap gains (measured: +5-8% at N = 512, even at N = 1024, and the ping-pong
// loop ahead from N = 2048 on).  Dense non-causal d = 128 with at most kPersistKeys keys and an
// even number of key tiles runs the plain loop over persistent blocks, which also hides each
// block's start-up behind its predecessor (measured: +5% at N = 512 and +4% at N = 1024 over
// the next best loop; 1% and 4% behind the ping-pong loop at N = 2048 and 4096).
constexpr int kShortKeys = 512;
constexpr int kPersistKeys = 1024;
#ifndef ATTN_D128_SHORT_SHAPE
#define ATTN_D128_SHORT_SHAPE 64, LoopShape<8>
#endif
#ifndef ATTN_D128_PERSIST_SHAPE
#define ATTN_D128_PERSIST_SHAPE 64, LoopShape<8, false, 4, true>
#endif
#ifndef ATTN_D64_SHAPE
#define ATTN_D64_SHAPE 64, LoopShape<8>
#endif
#ifndef ATTN_D128_SHAPE
#define ATTN_D128_SHAPE 64, LoopShape<8, true, 3>
#endif
#ifndef ATTN_D256_SHAPE
#define ATTN_D256_SHAPE 32, LoopShape<8, true, 4>
#endif
#ifndef ATTN_D256_WINDOW_SHAPE
#define ATTN_D256_WINDOW_SHAPE 32, LoopShape<8>
#endif

template <bool BF16>
hipError_t launch_dims(const FwdArgs& a, hipStream_t stream) {
  if (a.window > 0) {
    switch (a.d) {
      case 64: return launch_window<64, ATTN_D64_SHAPE, BF16>(a, stream);
      case 128: return launch_window<128, ATTN_D128_SHAPE, BF16>(a, stream);
      case 256: return launch_window<256, ATTN_D256_WINDOW_SHAPE, BF16>(a, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.d) {
    case 64: return launch_modes<64, ATTN_D64_SHAPE, BF16>(a, stream);
    case 128:
      if (!a.causal && a.cu_seqlens == nullptr && a.N <= kPersistKeys && ((a.N + 63) / 64) % 2 == 0)
        return launch_persistent<128, ATTN_D128_PERSIST_SHAPE, BF16>(a, stream);
      if (!a.causal && a.N <= kShortKeys) return launch_noncausal<128, ATTN_D128_SHORT_SHAPE, BF16>(a, stream);
      return launch_modes<128, ATTN_D128_SHAPE, BF16>(a, stream);
    case 256: return launch_modes<256, ATTN_D256_SHAPE, BF16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_fwd_16bit(const FwdArgs& a, bool is_bf16, hipStream_t stream) {
  return is_bf16 ? launch_dims<true>(a, stream) : launch_dims<false>(a, stream);
}

}  // namespace attn
