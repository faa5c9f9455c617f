// Small-n integer GEMM of the rank-augmented W4A4 layer (gfx950): the
// weight-streaming kernel for a few tokens (n <= 32).
//
// acc[i][j] = sum_k cx[i][k] * cw[j][k] with exact int32 accumulation on the
// int8 MFMA (TwinQuant notes, "TwinQuant: Learnable Subspace Decomposition
// for W4A4 LLM Quantization", section 02 note on INT32 accumulation and
// section 04.C, Figure 4), followed by one shared epilogue that dequantises
// with s_x[i] s_w[j] and adds the second low-rank stage T L2 before a single
// store of Y (section 04.C; the SVDQuant form of section 02.A).
//
// Operand pairing: an MFMA computes sum over (lane group, byte) of
// A[lane i][byte] * B[lane j][byte]; A and B fragments are always built the
// same way from the same code bytes, so each product pairs equal k.  Integer
// sums are exact in any order, which leaves the k order inside a fragment
// free.

#include "tq_prologue.h"

namespace tq {

// ---------------------------------------------------------------------------
// Small-n kernel (M <= 32): memory-bound on the weight codes.
//   Block: 16 output channels; WAVES waves split K into contiguous ranges of
//   64-byte steps (lane group g of 16 lanes loads bytes 16 g .. 16 g + 15 of
//   each step for channel lane % 16).  Every load of a batch of U steps --
//   weights, the matching activation codes, and the low-rank operands -- is
//   issued before the first wait, so a block pays one memory round trip per
//   batch.  XL: when the activation codes of all M rows fit in a few KB of
//   LDS, the block copies them there first and the product reads them from
//   LDS, so the vector memory stream carries only the weights.  MFMA 16x16x64 int8 (TWO: a second 16-token tile shares each
//   weight fragment); the waves' int32 partials are summed exactly through
//   LDS in wave order.
//   Epilogue: T is the sum over the k-chunks of the fp32 partials of X L1
//   written by the prologue (P; chunk order, then rounded to bf16; block 0
//   also writes it to Tout); T L2 for the block's 16 channels
//   is one 16x16 bf16 MFMA chain whose result layout matches the integer
//   accumulator's (lane l, element i -> token 4 (l / 16) + i, channel l % 16).
//
// FU, the one-launch form (up to 16 tokens): the prologue's work runs in the
// same grid (TwinQuant notes, section 04.C: the activations are quantised
// while the residual GEMM runs, and both components meet in one epilogue).
// Blocks [0, nqb) quantise one token row each (codes, s_x, and z_x for
// asymmetric activations), blocks [nqb, nprod) compute one fp32 partial of T
// each (rows 16 rt.., k-chunk c, 32 columns), and the GEMM blocks follow,
// each with GB groups of 16 output channels.  A GEMM block issues its first batch of weight
// loads, which depend on nothing, and only then waits for the producers:
//  * a producer stores its results at agent scope (written through to the
//    device's point of coherence, past the XCDs' separate L2s), waits until
//    every one of them has completed, and after a block barrier adds one to
//    each copy of the done counter;
//  * wave 0 of a GEMM block polls one copy (agent-scope loads, which those
//    L2s cannot serve stale) until it reaches nprod, and releases the
//    other waves with a barrier that does not wait for their weight loads in
//    flight.  Codes, scales and partials are then loaded with plain loads.
//    No L2 can hold a stale copy of them: the dispatch of the kernel
//    invalidated the caches, no block reads them before the count is
//    complete, and a line first brought in after that point holds the
//    stored values.  An acquire at agent scope would invalidate the XCD's
//    whole L2 in every GEMM block, which costs more than the call itself.
// The GEMM blocks count themselves out in two levels: each adds one to its
// group's counter (groups of at least 32 consecutive blocks, at most
// kFGroups groups), the last of a group resets it and adds one to kFFin, and
// the last group's last block subtracts nprod from every copy of the done
// counter and the number of groups from kFFin, so every counter is zero
// again when the kernel ends, whatever the order in which the blocks ran.
// One counter for all the blocks would serialise hundreds of returning
// atomics on one address at the end of the kernel.  The wait is bounded: a
// block whose wait gives up sets the sticky flag word kWFlag and writes NaN
// to its outputs, and GEMM blocks that find the flag set when they start
// write NaN too, until the workspace is zero-filled again.
// ---------------------------------------------------------------------------
// Most bytes of activation codes the small-n GEMM stages in LDS: what
// leaves the blocks per CU of its launch bounds (2 of 8 waves, 4 of 4 waves)
// within the 160 KB of LDS next to the static arrays.
__host__ __device__ constexpr int gemv_xl_bytes(int waves) { return waves == 8 ? 24576 : 12288; }

// DBG: the test-hook instance, which also stores the exact int32 sums of the
// residual product (g.acc) and, for the quantised low-rank branch, of its
// second stage (g.acc2); its code is this template's, with those stores added.
// hand-off words (uint32 indices into the sync region): the sticky
// wait-limit flag (shared with the decode kernel), kFCopies copies of the
// producers-done counter (kFDone + kFStride i: 256 bytes apart, so that the
// GEMM blocks' polls spread over several memory channels), the counter of
// finished groups of GEMM blocks, and from kFGroup on one counter per group
// (4 words apart, at most kFGroups groups)
constexpr int kWFlag = 32, kFDone = 48, kFStride = 64, kFCopies = 8, kFFin = 80, kFGroup = 512, kFGroups = 128;

__device__ __forceinline__ uint32_t ld_agent(const unsigned* p) {
  return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A producer block of the one-launch form (X of type XT): one row's codes and s_x,
// or one fp32 partial of T (QS = 2: 32 columns), then the signal once its
// stores have completed.  smem: the block's LDS.
template <int WAVES, typename XT>
__device__ __forceinline__ void small_producer(const SmallFuse& f, uint8_t* smem) {
  const PrologueArgs& a = f.pa;
  const int b = blockIdx.x;
  if (b < a.nqb) {
    constexpr int CHB = WAVES == 4 ? 2 : 4;  // 8-value chunks per thread: rows up to 4096 (4 waves), 16384 (8 waves)
    const XT* row = (const XT*)a.X + (size_t)b * a.d;
    uint8_t* codes = a.xc + (size_t)b * (a.d >> 1);
    if (f.zx)
      quant_row_block_asym<XT, CHB>(row, a.d, codes, a.sx + b, f.zx + b, reinterpret_cast<float*>(smem));
    else
      quant_row_block_reg<XT, CHB, true>(row, a.d, codes, a.sx + b, reinterpret_cast<float*>(smem));
  } else {
    auto sP = reinterpret_cast<float (*)[16][33]>(smem);
    const TBlock t = t_block_products<XT, 2, WAVES, 8>(a, b - a.nqb, sP);
    __syncthreads();
    const int rows = min(16, a.n - 16 * t.rt), col0 = 32 * t.qg;
    for (int e = threadIdx.x; e < rows * 32; e += WAVES * 64) {
      const int rr = e >> 5, cc = e & 31;
      float v = 0.0f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) v += sP[w][rr][cc];  // wave order
      __hip_atomic_store(&a.P[((size_t)t.c * a.n + 16 * t.rt + rr) * a.r_pad + col0 + cc], v, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // every store of this thread has completed
  __syncthreads();
  if (threadIdx.x < kFCopies && !f.silent)
    __hip_atomic_fetch_add(f.sync + kFDone + kFStride * threadIdx.x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// FU: 0, or the one-launch form with bf16 (1) or fp32 (2) X.  GB: groups of
// 16 output channels per block (GB > 1: one 16-token tile, the rank-augmented
// epilogue); every wave streams its k-range of all GB groups' weights and
// uses each activation fragment GB times, and wave w finishes group w, so a
// block fetches the codes and the partials of T once for 16 GB channels.
template <int BITS, int EPI, int WAVES, bool TWO, bool XL, bool DBG = false, int FU = 0, int GB = 1>
__global__ __launch_bounds__(WAVES * 64, (WAVES == 4) ? 4 : 2) void k_gemv(GemmArgs g, SmallFuse f) {
  static_assert(GB == 1 || (EPI == EPI_LINEAR && !TWO && GB <= WAVES), "channel groups: one token tile");
  constexpr int U = (WAVES == 4 && TWO && !XL) ? 4 : ((WAVES == 4 || TWO) ? 8 : 16);  // 64-byte steps per wave per batch
  constexpr int NT = WAVES * 64;
  constexpr int MT = TWO ? 32 : 16;  // token rows held for the low-rank stage
  constexpr bool LR = EPI == EPI_LINEAR;
  constexpr bool QL = EPI == EPI_QLR;  // quantised low-rank branch: second stage on the int8 MFMA
  // LDS: red [WAVES][RT][4][64] int | sT [MT x 256] bf16 | sL [16 GB x 256]
  // bf16 | sPart [NT][2] float4; a producer block (FU) reuses it whole
  constexpr int RT = TWO ? 2 : GB;  // finished tiles: token tiles, or channel groups
  constexpr int B_RED = WAVES * RT * 4 * 64 * 4;
  constexpr int B_ST = LR ? MT * 256 * 2 : 16, B_SL = LR ? 16 * GB * 256 * 2 : 16, B_SP = LR ? NT * 32 : 16;
  constexpr int B_GEMV = B_RED + B_ST + B_SL + B_SP, B_PRO = FU != 0 ? WAVES * 16 * 33 * 4 : 0;
  __shared__ __attribute__((aligned(16))) uint8_t smem[B_GEMV > B_PRO ? B_GEMV : B_PRO];
  __shared__ int s_ok;
  auto red = reinterpret_cast<int (*)[RT][4][64]>(smem);
  bf16_t* sT = reinterpret_cast<bf16_t*>(smem + B_RED);
  bf16_t* sL = reinterpret_cast<bf16_t*>(smem + B_RED + B_ST);
  auto sPart = reinterpret_cast<float4 (*)[2]>(smem + B_RED + B_ST + B_SL);
  if constexpr (FU != 0) {
    if ((int)blockIdx.x < f.nprod) {
      small_producer<WAVES, std::conditional_t<FU == 1, bf16_t, float>>(f, smem);
      return;
    }
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int n0 = (FU != 0 ? (int)blockIdx.x - f.nprod : (int)blockIdx.x) * 16 * GB;
  const int wg = GB > 1 ? min(wave, GB - 1) : 0;  // the group this wave finishes (GB > 1)
  const uint8_t* bp[GB];
#pragma unroll
  for (int gb = 0; gb < GB; ++gb) bp[gb] = g.B + (size_t)min(n0 + 16 * gb + l16, g.N - 1) * g.ldb + 16 * lg;
  const uint8_t* ap0 = g.A + (size_t)min(l16, g.M - 1) * g.lda + 16 * lg;
  const uint8_t* ap1 = g.A + (size_t)min(16 + l16, g.M - 1) * g.lda + 16 * lg;
  const int KS = (g.Kb + 63) / 64;
  const int per = (KS + WAVES - 1) / WAVES;
  const int sbeg = wave * per, send = min(KS, sbeg + per);
  const int rp = LR ? g.r_pad : 0;
  const int rq = rp / 8;  // 16-byte pieces (8 values) per low-rank row
  const int grp0 = LR ? group_of(g.groups, n0) : 0;
  const int toff = grp0 * rp;                          // this block's layer in T and the partials
  const bool tfirst = LR && n0 == g.groups.start[grp0];  // first block of its layer writes T
  // T pieces: NP = M rows x rq; G thread groups (no more than there are
  // chunks) split the k-chunks of each piece, at most two chunks per group
  const int NP = g.M * rq;
  const int G = max(1, min(NT / max(NP, 1), LR ? g.nchunk : 1));

  // XL: the M rows of activation codes, row stride Kb + 16 bytes (rows of a
  // 16-row operand read then fall on distinct banks); XLN 16-byte pieces per
  // thread cover the largest staging the launcher allows
  extern __shared__ __attribute__((aligned(16))) uint8_t xl_lds[];
  constexpr int XLN = XL ? gemv_xl_bytes(WAVES) / 16 / NT : 1;
  const int XS = g.Kb + 16, kp = g.Kb >> 4;
  uint4 xst[XLN];
  auto load_xl = [&]() {
#pragma unroll
    for (int i = 0; i < XLN; ++i) {
      const int idx = min(tid + NT * i, g.M * kp - 1);
      xst[i] = *reinterpret_cast<const uint4*>(g.A + (size_t)(idx / kp) * g.lda + 16 * (idx % kp));
    }
  };
  if (XL && FU == 0) load_xl();

  // Loads are unconditional, from clamped (always valid) addresses, and
  // masked where used: conditional loads become branches whose register
  // merges force early waits on every load in flight.
  const int kb_last = max(0, min((max(send, sbeg + 1) - 1) * 64, g.Kb - 16 - 16 * lg));
  uint4 bv[GB][U], av0[U], av1[U];
  auto load_w = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int gb = 0; gb < GB; ++gb)
        bv[gb][u] = *reinterpret_cast<const uint4*>(bp[gb] + min((s0 + u) * 64, kb_last));
  };
  auto load_x = [&](int s0) {
    if (XL) return;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = min((s0 + u) * 64, kb_last);
      av0[u] = *reinterpret_cast<const uint4*>(ap0 + kb);
      if (TWO) av1[u] = *reinterpret_cast<const uint4*>(ap1 + kb);
    }
  };
  auto load_batch = [&](int s0) {
    load_w(s0);
    load_x(s0);
  };
  const uint8_t* xl0 = xl_lds + min(l16, g.M - 1) * XS + 16 * lg;
  const uint8_t* xl1 = xl_lds + min(16 + l16, g.M - 1) * XS + 16 * lg;
  i32x4 acc0[GB], acc1 = {0, 0, 0, 0};
#pragma unroll
  for (int gb = 0; gb < GB; ++gb) acc0[gb] = i32x4{0, 0, 0, 0};
  auto mma_batch = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u >= send) continue;
      if (XL) {
        const int kb = min((s0 + u) * 64, kb_last);
        av0[u] = *reinterpret_cast<const uint4*>(xl0 + kb);
        if (TWO) av1[u] = *reinterpret_cast<const uint4*>(xl1 + kb);
      }
      if ((s0 + u) * 64 + 16 * lg >= g.Kb) {  // this lane group's 16 bytes lie past the row: zero codes
#pragma unroll
        for (int gb = 0; gb < GB; ++gb) bv[gb][u] = uint4{0, 0, 0, 0};
        av0[u] = uint4{0, 0, 0, 0};
        av1[u] = uint4{0, 0, 0, 0};
      }
      if (BITS == 4) {
        const i32x4 a0 = unpack16(av0[u].x, av0[u].y), a1 = unpack16(av0[u].z, av0[u].w);
#pragma unroll
        for (int gb = 0; gb < GB; ++gb) {
          const i32x4 b0 = unpack16(bv[gb][u].x, bv[gb][u].y), b1 = unpack16(bv[gb][u].z, bv[gb][u].w);
          acc0[gb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, acc0[gb], 0, 0, 0);
          acc0[gb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, acc0[gb], 0, 0, 0);
          if (TWO) {
            acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16(av1[u].x, av1[u].y), b0, acc1, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16(av1[u].z, av1[u].w), b1, acc1, 0, 0, 0);
          }
        }
      } else {
        const i32x4 b0 = __builtin_bit_cast(i32x4, bv[0][u]);
        acc0[0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, av0[u]), b0, acc0[0], 0, 0, 0);
        if (TWO) acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, av1[u]), b0, acc1, 0, 0, 0);
      }
    }
  };

  // ---- issue every load of the first batch before any wait ----
  float sxv[4], swv = 0.0f;  // epilogue scales
  // asymmetric activations (codes u - 8): per row z + 8 s_x, per channel
  // s_w colsum(C_w) (CoQuant Eq. 1 with a zero-point)
  float zzv[4] = {0.f, 0.f, 0.f, 0.f}, wzv = 0.0f;
  const int trow = TWO ? 16 * (wave & 1) : 0;  // first token row of the tile this wave may finish
  auto load_sx = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) sxv[i] = g.sx[min(trow + 4 * lg + i, g.M - 1)];
  };
  auto load_zz = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = min(trow + 4 * lg + i, g.M - 1);
      zzv[i] = g.zx[rr] + 8.0f * g.sx[rr];
    }
  };
  if (LR || QL) {
    swv = g.sw[min(n0 + 16 * wg + l16, g.N - 1)];
    if (FU == 0) load_sx();
    if (LR && g.zx) {
      wzv = swv * (float)g.csw[min(n0 + 16 * wg + l16, g.N - 1)];
      if (FU == 0) load_zz();
    }
  }
  // QL: the first 64 ranks of the second stage's operands and its scales
  // (lane: token or channel l % 16, the 16 ranks 16 (l / 16) ..; ranks past
  // r_pad are zero), loaded with the first batch
  i32x4 qa = {0, 0, 0, 0};
  uint2 qb = {0u, 0u};
  float qs[4], qsv = 0.0f;
  const uint8_t* qtp = nullptr;
  const uint8_t* qvp = nullptr;
  if constexpr (QL) {
    qtp = g.Tq + (size_t)min(16 * (wave & 1) + l16, g.M - 1) * g.r_pad + 16 * lg;
    qvp = g.Vq + (size_t)min(n0 + l16, g.N - 1) * (g.r_pad / 2) + 8 * lg;
    if (16 * lg < g.r_pad) {
      qa = *reinterpret_cast<const i32x4*>(qtp);
      qb = *reinterpret_cast<const uint2*>(qvp);
    }
    qsv = g.sv[min(n0 + l16, g.N - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i) qs[i] = g.st[min(16 * (wave & 1) + 4 * lg + i, g.M - 1)] * (1.0f / 16);
  }
  uint4 lv;
  bool ok = true;  // FU: the producers' results arrived (else the block writes NaN)
  if constexpr (FU != 0) {
    // the weights of the first batch and the rows of L2^T depend on nothing
    load_w(sbeg);
    if (LR && rp > 0) {
      const int el = min(tid, 16 * GB * rq - 1);
      lv = *reinterpret_cast<const uint4*>(g.L2t + (size_t)min(n0 + el / rq, g.N - 1) * rp + 8 * (el % rq));
    }
    if (wave == 0) {
      const unsigned* sy = f.sync;
      const bool clean = ld_agent(sy + kWFlag) == 0;
      bool done = false;
      for (unsigned it = 0;; ++it) {
        if ((int)ld_agent(sy + kFDone + kFStride * (blockIdx.x % kFCopies)) >= f.nprod) {
          done = true;
          break;
        }
        if (it >= f.spin) break;
        __builtin_amdgcn_s_sleep(2);
      }
      if (!done && lane == 0)
        __hip_atomic_store(const_cast<unsigned*>(sy + kWFlag), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0) s_ok = (done && clean) ? 1 : 0;
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): s_ok written
    }
    // a barrier that does not wait for the weight loads in flight
    asm volatile("s_barrier" ::: "memory");
    ok = s_ok != 0;
    if (LR || QL) load_sx();
    if (LR && g.zx) load_zz();
    if (XL)
      load_xl();
    else
      load_x(sbeg);
  } else {
    load_batch(sbeg);
  }
  // Low-rank operands, with clamped (always valid) indices, masked where used,
  // so that none of them needs a wait before the integer product: piece
  // tid of L2^T (16 x rp), and for thread (piece p, group q), q < G, of T
  // the chunks q and q + G of the prologue's fp32 partials.
  float4 pv[2][2];
  if (LR && rp > 0) {
    if (FU == 0) {
      const int el = min(tid, 16 * GB * rq - 1);
      lv = *reinterpret_cast<const uint4*>(g.L2t + (size_t)min(n0 + el / rq, g.N - 1) * rp + 8 * (el % rq));
    }
    if (tid < NP * G) {
      const int pc = tid % NP, grp = tid / NP;
      const int rowt = pc / rq, qt = pc % rq;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = min(grp + G * j, g.nchunk - 1);
        const float4* pp = reinterpret_cast<const float4*>(g.P + ((size_t)c * g.M + rowt) * g.ldt + toff + 8 * qt);
        pv[j][0] = pp[0];
        pv[j][1] = pp[1];
      }
    }
  }

  if (XL) {
#pragma unroll
    for (int i = 0; i < XLN; ++i) {
      const int idx = tid + NT * i;
      if (idx < g.M * kp) *reinterpret_cast<uint4*>(xl_lds + (idx / kp) * XS + 16 * (idx % kp)) = xst[i];
    }
    __syncthreads();
  }

  // ---- integer product ----
  mma_batch(sbeg);
  for (int s0 = sbeg + U; s0 < send; s0 += U) {
    load_batch(s0);
    mma_batch(s0);
  }

  // ---- low-rank operands into LDS (T rows >= M are zero) ----
  if (LR && rp > 0) {
    if (tid < 16 * GB * rq) *reinterpret_cast<uint4*>(sL + tid * 8) = (n0 + tid / rq < g.N) ? lv : uint4{0, 0, 0, 0};
    for (int e = tid + NT; e < 16 * GB * rq; e += NT) {
      const int c = e / rq, q = e % rq;
      uint4 v = uint4{0, 0, 0, 0};
      if (n0 + c < g.N) v = *reinterpret_cast<const uint4*>(g.L2t + (size_t)(n0 + c) * rp + 8 * q);
      *reinterpret_cast<uint4*>(sL + e * 8) = v;
    }
    if (tid < NP * G) {
      const int grp = tid / NP;
      float4 t0 = float4{0.f, 0.f, 0.f, 0.f}, t1 = float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (grp + G * j < g.nchunk) {
          t0.x += pv[j][0].x; t0.y += pv[j][0].y; t0.z += pv[j][0].z; t0.w += pv[j][0].w;
          t1.x += pv[j][1].x; t1.y += pv[j][1].y; t1.z += pv[j][1].z; t1.w += pv[j][1].w;
        }
      }
      sPart[tid][0] = t0;
      sPart[tid][1] = t1;
    }
    __syncthreads();
    // piece p: groups in order -> bf16; rows M .. MT - 1 zero
    for (int pc = tid; pc < MT * rq; pc += NT) {
      const int row = pc / rq, q = pc % rq;
      uint4 v = uint4{0, 0, 0, 0};
      if (row < g.M) {
        float t[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (pc < NT) {
          for (int gi = 0; gi < G; ++gi) {
            const float4 x0 = sPart[gi * NP + pc][0], x1 = sPart[gi * NP + pc][1];
            t[0] += x0.x; t[1] += x0.y; t[2] += x0.z; t[3] += x0.w;
            t[4] += x1.x; t[5] += x1.y; t[6] += x1.z; t[7] += x1.w;
          }
        } else {  // pieces beyond the block's threads (G == 1): all chunks here
          for (int k = 0; k < g.nchunk; ++k) {
            const float4* pp = reinterpret_cast<const float4*>(g.P + ((size_t)k * g.M + row) * g.ldt + toff + 8 * q);
            const float4 x0 = pp[0], x1 = pp[1];
            t[0] += x0.x; t[1] += x0.y; t[2] += x0.z; t[3] += x0.w;
            t[4] += x1.x; t[5] += x1.y; t[6] += x1.z; t[7] += x1.w;
          }
        }
        v = uint4{pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3]), pack_bf16x2(t[4], t[5]), pack_bf16x2(t[6], t[7])};
        if (tfirst && g.Tout) *reinterpret_cast<uint4*>(g.Tout + (size_t)row * g.ldt + toff + 8 * q) = v;
      }
      *reinterpret_cast<uint4*>(sT + pc * 8) = v;
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int gb = 0; gb < GB; ++gb) red[wave][gb][i][lane] = acc0[gb][i];
    if (TWO) red[wave][TWO ? 1 : 0][i][lane] = acc1[i];
  }
  __syncthreads();
  // wave t (t < number of 16-token tiles, or of channel groups) finishes
  // tile t, or group t
  if (wave >= RT) return;
  const int tile = TWO ? wave : 0;
  int sacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int v = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[w][wave][i][lane];
    sacc[i] = (BITS == 4) ? (v >> 8) : v;
  }
  const int col = n0 + 16 * wg + l16;
  if constexpr (DBG && EPI != EPI_ACC) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * tile + 4 * lg + i;
      if (row < g.M && col < g.N) g.acc[(size_t)row * g.N + col] = sacc[i];
    }
  }
  if constexpr (EPI == EPI_ACC) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * tile + 4 * lg + i;
      if (row < g.M && col < g.N) g.acc[(size_t)row * g.N + col] = sacc[i];
    }
  } else {
    f32x4 lr = {0.f, 0.f, 0.f, 0.f};
    if constexpr (QL) {
      // (s_x s_t) s_v (Q(T) Q(V)) for the tile's 16 tokens and the block's 16
      // channels: exact int32 over the ranks (V expanded by unpack16: a factor
      // 16, taken out with s_t), 64 ranks per v_mfma_i32_16x16x64_i8
      i32x4 q2 = {0, 0, 0, 0};
      q2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa, unpack16(qb.x, qb.y), q2, 0, 0, 0);
      for (int q0 = 64; q0 < g.r_pad; q0 += 64) {
        const bool ok = q0 + 16 * lg < g.r_pad;
        const i32x4 a = ok ? *reinterpret_cast<const i32x4*>(qtp + q0) : i32x4{0, 0, 0, 0};
        const uint2 b = ok ? *reinterpret_cast<const uint2*>(qvp + q0 / 2) : uint2{0u, 0u};
        q2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, unpack16(b.x, b.y), q2, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) lr[i] = (float)q2[i] * (sxv[i] * qs[i] * qsv);
      if constexpr (DBG) {  // C_t C_v^T exactly (the expanded V carries 16 x code)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * tile + 4 * lg + i;
          if (row < g.M && col < g.N) g.acc2[(size_t)row * g.N + col] = q2[i] >> 4;
        }
      }
    }
    for (int t0 = 0; t0 < rp; t0 += 32) {
      // A: T rows (tokens), B: L2^T rows (channels); 8 consecutive t per lane
      const uint4 a8 = *reinterpret_cast<const uint4*>(sT + (16 * tile + l16) * rp + t0 + 8 * lg);
      const uint4 b8 = *reinterpret_cast<const uint4*>(sL + (16 * wg + l16) * rp + t0 + 8 * lg);
      lr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a8), as_bf16x8(b8), lr, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * tile + 4 * lg + i;
      if (row >= g.M || col >= g.N) continue;
      const float y = ok ? (float)sacc[i] * (sxv[i] * swv) + lr[i] + zzv[i] * wzv : __builtin_nanf("");
      if (g.y_bf16)
        reinterpret_cast<bf16_t*>(g.Y)[(size_t)row * g.ldy + col] = (bf16_t)f32_to_bf16_bits(y);
      else
        reinterpret_cast<float*>(g.Y)[(size_t)row * g.ldy + col] = y;
    }
  }
  if constexpr (FU != 0) {
    if (wave == 0 && lane == 0) {
      // the last block overall brings the counters back to zero (every GEMM
      // block has passed its wait, so no poll of kFDone is still to come)
      const unsigned ncons = gridDim.x - (unsigned)f.nprod, cb = blockIdx.x - (unsigned)f.nprod;
      const unsigned gs = max(32u, (ncons + kFGroups - 1) / kFGroups), gi = cb / gs;
      const unsigned ngr = (ncons + gs - 1) / gs, gsize = min(gs, ncons - gi * gs);
      unsigned* gc = f.sync + kFGroup + 4 * gi;
      if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gsize - 1) {
        __hip_atomic_fetch_sub(gc, gsize, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__hip_atomic_fetch_add(f.sync + kFFin, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == ngr - 1) {
          if (!f.silent)
            for (int i = 0; i < kFCopies; ++i)
              __hip_atomic_fetch_sub(f.sync + kFDone + kFStride * i, (unsigned)f.nprod, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_fetch_sub(f.sync + kFFin, ngr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  }
}

int gemv_max_chunks(int M, int Kb, int r_pad) {
  const int nt = (Kb > 2048 ? 8 : 4) * 64;
  const int np = M * (r_pad / 8);
  return 2 * std::max(1, nt / std::max(np, 1));
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int BITS, int EPI, bool TWO, bool DBG>
static hipError_t gemv_cols_t(const GemmArgs& g, hipStream_t st) {
  const unsigned blocks = (unsigned)((g.N + 15) / 16);
  const size_t xl = (size_t)g.M * (size_t)(g.Kb + 16);  // activation codes in LDS
  const bool use_xl = xl <= (size_t)gemv_xl_bytes(g.Kb > 2048 ? 8 : 4) && g.Kb % 16 == 0;
  if (g.Kb > 2048) {
    if (use_xl)
      hipLaunchKernelGGL((k_gemv<BITS, EPI, 8, TWO, true, DBG>), dim3(blocks), dim3(512), xl, st, g, SmallFuse{});
    else
      hipLaunchKernelGGL((k_gemv<BITS, EPI, 8, TWO, false, DBG>), dim3(blocks), dim3(512), 0, st, g, SmallFuse{});
  } else {
    if (use_xl)
      hipLaunchKernelGGL((k_gemv<BITS, EPI, 4, TWO, true, DBG>), dim3(blocks), dim3(256), xl, st, g, SmallFuse{});
    else
      hipLaunchKernelGGL((k_gemv<BITS, EPI, 4, TWO, false, DBG>), dim3(blocks), dim3(256), 0, st, g, SmallFuse{});
  }
  return hipGetLastError();
}

// Groups of 16 channels per block of the one-launch form: 4 when rows are
// short (4-wave blocks) and more than two 16-channel blocks per compute unit
// would exist (gate/up of Llama-3-8B: 224 blocks of 64 channels instead of 896
// of 16, so the codes and the partials of T are fetched a quarter as often),
// else 1.
static int fused_gb(int N, int Kb) { return (Kb <= 2048 && (N + 15) / 16 > 512) ? 4 : 1; }

// One-launch form (up to 16 tokens): the producers first in the grid, then
// the GEMM blocks.
template <bool DBG, int FU>
static hipError_t gemv_fused_t(const GemmArgs& g, const SmallFuse& f, hipStream_t st) {
  const int gb = fused_gb(g.N, g.Kb);
  const dim3 grid((unsigned)(f.nprod + (g.N + 16 * gb - 1) / (16 * gb)));
  const size_t xl = (size_t)g.M * (size_t)(g.Kb + 16);
  const bool use_xl = xl <= (size_t)gemv_xl_bytes(g.Kb > 2048 ? 8 : 4) && g.Kb % 16 == 0;
  constexpr int E = EPI_LINEAR;
  if (g.Kb > 2048) {
    if (use_xl)
      launch_kernel(k_gemv<4, E, 8, false, true, DBG, FU>, grid, dim3(512), (unsigned)xl, st, g, f);
    else
      launch_kernel(k_gemv<4, E, 8, false, false, DBG, FU>, grid, dim3(512), 0u, st, g, f);
  } else if (gb == 4) {
    if (use_xl)
      launch_kernel(k_gemv<4, E, 4, false, true, DBG, FU, 4>, grid, dim3(256), (unsigned)xl, st, g, f);
    else
      launch_kernel(k_gemv<4, E, 4, false, false, DBG, FU, 4>, grid, dim3(256), 0u, st, g, f);
  } else {
    if (use_xl)
      launch_kernel(k_gemv<4, E, 4, false, true, DBG, FU>, grid, dim3(256), (unsigned)xl, st, g, f);
    else
      launch_kernel(k_gemv<4, E, 4, false, false, DBG, FU>, grid, dim3(256), 0u, st, g, f);
  }
  return hipGetLastError();
}

// Whether the one-launch grid is (nearly) resident at once on the current
// device: at most a quarter more blocks than fit.  The producers come first
// in the grid, so they never wait for a slot; but GEMM blocks beyond the
// resident ones start only as others finish, which cuts the weight stream in
// two.  Measured with blocks of 16 channels: 296 blocks on 256 slots (down
// projection, 8 tokens) still faster than two launches, 1816 on 1024 (gate
// and up grouped, 16 tokens) slower.
template <bool DBG, int FU>
static bool gemv_fused_fits_t(int M, int Kb, int N, int nprod) {
  int dev = 0, cus = 0, occ = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return false;
  const size_t xl = (size_t)M * (size_t)(Kb + 16);
  const bool use_xl = xl <= (size_t)gemv_xl_bytes(Kb > 2048 ? 8 : 4) && Kb % 16 == 0;
  const int gb = fused_gb(N, Kb);
  constexpr int E = EPI_LINEAR;
  hipError_t e;
  if (Kb > 2048)
    e = use_xl ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_gemv<4, E, 8, false, true, DBG, FU>, 512, xl)
               : hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_gemv<4, E, 8, false, false, DBG, FU>, 512, 0);
  else if (gb == 4)
    e = use_xl ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_gemv<4, E, 4, false, true, DBG, FU, 4>, 256, xl)
               : hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_gemv<4, E, 4, false, false, DBG, FU, 4>, 256, 0);
  else
    e = use_xl ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_gemv<4, E, 4, false, true, DBG, FU>, 256, xl)
               : hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_gemv<4, E, 4, false, false, DBG, FU>, 256, 0);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return 4 * ((int64_t)nprod + (N + 16 * gb - 1) / (16 * gb)) <= 5 * (int64_t)cus * occ;
}

bool gemv_fused_fits(int M, int Kb, int N, int nprod, bool x_bf16, bool dbg) {
  if (x_bf16) return dbg ? gemv_fused_fits_t<true, 1>(M, Kb, N, nprod) : gemv_fused_fits_t<false, 1>(M, Kb, N, nprod);
  return dbg ? gemv_fused_fits_t<true, 2>(M, Kb, N, nprod) : gemv_fused_fits_t<false, 2>(M, Kb, N, nprod);
}

hipError_t launch_gemv_fused(const GemmArgs& g, const SmallFuse& f, bool x_bf16, hipStream_t st) {
  const PrologueArgs& a = f.pa;
  // the producers' shapes: rows of at most 4096 (4 waves) or 16384 (8 waves)
  // values in registers, T partials of 32 columns each, all summed by the
  // GEMM blocks in one pass
  if (g.M < 1 || g.M > 16 || a.n != g.M || 2 * g.Kb != a.d || a.d % 32 || a.d > (g.Kb > 2048 ? 16384 : 4096) ||
      a.nqb != g.M || !f.sync || g.r_pad > 256 || (g.r_pad > 0 && (a.nqg < 1 || a.r_pad % 32 || !g.P)) ||
      f.nprod != a.nqb + (g.r_pad ? ((a.n + 15) / 16) * a.nchunk * a.nqg : 0) || g.nchunk != a.nchunk ||
      g.nchunk > gemv_max_chunks(g.M, g.Kb, g.ldt))
    return hipErrorInvalidValue;
  if (x_bf16) return g.acc ? gemv_fused_t<true, 1>(g, f, st) : gemv_fused_t<false, 1>(g, f, st);
  return g.acc ? gemv_fused_t<true, 2>(g, f, st) : gemv_fused_t<false, 2>(g, f, st);
}

template <int BITS, int EPI>
static hipError_t gemv_cols(const GemmArgs& g, hipStream_t st) {
  if (EPI == EPI_LINEAR && (g.r_pad > 256 || (g.r_pad > 0 && (!g.P || g.nchunk < 1)))) return hipErrorInvalidValue;
  // the accumulator-export instance (test hook) when an export buffer is set
  if (EPI != EPI_ACC && g.acc)
    return g.M > 16 ? gemv_cols_t<BITS, EPI, true, true>(g, st) : gemv_cols_t<BITS, EPI, false, true>(g, st);
  return g.M > 16 ? gemv_cols_t<BITS, EPI, true, false>(g, st) : gemv_cols_t<BITS, EPI, false, false>(g, st);
}

hipError_t launch_gemv(const GemmArgs& g, int bits, Epilogue epi, hipStream_t st) {
  if (bits == 4) {
    if (epi == EPI_ACC) return gemv_cols<4, EPI_ACC>(g, st);
    if (epi == EPI_LINEAR) return gemv_cols<4, EPI_LINEAR>(g, st);
    if (epi == EPI_QLR) return gemv_cols<4, EPI_QLR>(g, st);
  } else if (bits == 8 && epi == EPI_ACC) {
    return gemv_cols<8, EPI_ACC>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
