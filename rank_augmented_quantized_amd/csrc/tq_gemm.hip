// Integer GEMM kernels of the rank-augmented W4A4 layer (gfx950).
//
// acc[i][j] = sum_k cx[i][k] * cw[j][k] with exact int32 accumulation on the
// int8 MFMA (TwinQuant notes, "TwinQuant: Learnable Subspace Decomposition
// for W4A4 LLM Quantization", section 02 note on INT32 accumulation and
// section 04.C, Figure 4), followed by one shared epilogue that dequantises
// with s_x[i] s_w[j] and adds the second low-rank stage T L2 on the bf16
// MFMA before a single store of Y (section 04.C; the SVDQuant form of section
// 02.A).  The two-subspace epilogue adds the 8-bit high-precision product
// with its own scales (CoQuant, "CoQuant: Joint Weight-Activation Subspace
// Projection for Mixed-Precision LLMs", Eq. 9).
//
// Operand pairing: an MFMA computes sum over (lane group, byte) of
// A[lane i][byte] * B[lane j][byte]; A and B fragments are always built the
// same way from the same code bytes, so each product pairs equal k.  Integer
// sums are exact in any order, which leaves the k order inside a fragment
// free.

#include <stdlib.h>

#include <type_traits>

#include "tq_kernels.h"

namespace tq {

// ---------------------------------------------------------------------------
// Tile kernel (any M; chosen for M > 32).
//   The MFMA tile's rows are output channels (weight codes) and its columns
//   are tokens (activation codes), so each lane of a 32x32 result block holds
//   four consecutive channels of one token and the epilogue writes Y with
//   8-byte (bf16) or 16-byte (fp32) stores.
//   One k-stage = 128 k.  Codes are loaded from global one stage ahead into
//   registers and, when staged into LDS, 4-bit codes are unpacked once to
//   int8 (16 * code, see nib_lo / nib_hi): a 16-byte chunk of 32 packed codes
//   becomes two 16-byte LDS chunks (even k, odd k), so the MFMA fragments are
//   read from LDS ready to use.  LDS rows are 128 bytes = 8 chunks; chunk c of
//   row r sits at position c ^ (r & 7) ^ ((r >> 3) & 1), which keeps the
//   fragment reads of 8 or 16 consecutive rows on distinct banks.
//   Waves: WGM x WGN, wave tile (BM / WGM) x (BN / WGN) of 32x32 blocks.
// ---------------------------------------------------------------------------
template <int BITS, int EPI, int BM, int BN, int WGM, int WGN, bool PK>
__global__ __launch_bounds__(WGM * WGN * 64) void k_gemm(GemmArgs g) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WM = BM / WGM, WN = BN / WGN, FM = WM / 32, FN = WN / 32;
  // PK: 4-bit codes stay packed in LDS (256-k stages) and are unpacked when a
  // fragment is read; otherwise they are unpacked once when staged (128-k).
  constexpr bool PACKED = PK && BITS == 4;
  constexpr int CPR = (BITS == 4 && !PACKED) ? 4 : 8;  // 16-byte code chunks per row per stage
  constexpr int RPS = NT / CPR;             // rows per load pass
  constexpr int LA = BM / RPS, LB = BN / RPS;
  constexpr int STAGE = (BM + BN) * 128;
  static_assert(FM >= 1 && FN >= 1 && LA >= 1 && LB >= 1, "tile shape");
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int l32 = lane & 31, lgrp = lane >> 5;

  // rows of the tile: channels (g.B, g.N of them); columns: tokens (g.A, g.M)
  int tm, tn;
  tile_of_block(blockIdx.x, (g.N + BM - 1) / BM, (g.M + BN - 1) / BN, tm, tn);
  const int ch0 = tm * BM, tk0 = tn * BN;

  const int lc = tid % CPR, lr = tid / CPR;
  const uint8_t* pw[LA];
  const uint8_t* px[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) pw[i] = g.B + (size_t)min(ch0 + lr + RPS * i, g.N - 1) * g.ldb + 16 * lc;
#pragma unroll
  for (int i = 0; i < LB; ++i) px[i] = g.A + (size_t)min(tk0 + lr + RPS * i, g.M - 1) * g.lda + 16 * lc;

  uint4 rw[LA], rx[LB];
  auto gload = [&](const uint8_t* const (&qw)[LA], const uint8_t* const (&qx)[LB], int kt, int Kb) {
    const int kb = kt * CPR * 16;
    const bool ok = kb + 16 * lc < Kb;
#pragma unroll
    for (int i = 0; i < LA; ++i) rw[i] = ok ? *reinterpret_cast<const uint4*>(qw[i] + kb) : uint4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < LB; ++i) rx[i] = ok ? *reinterpret_cast<const uint4*>(qx[i] + kb) : uint4{0, 0, 0, 0};
  };
  auto put = [&](uint8_t* base, int r, const uint4& v, auto bits) {
    if constexpr (decltype(bits)::value == 4 && !PACKED) {
      const uint4 lo = {nib_lo(v.x), nib_lo(v.y), nib_lo(v.z), nib_lo(v.w)};
      const uint4 hi = {nib_hi(v.x), nib_hi(v.y), nib_hi(v.z), nib_hi(v.w)};
      *reinterpret_cast<uint4*>(base + r * 128 + 16 * swz(2 * lc, r)) = lo;
      *reinterpret_cast<uint4*>(base + r * 128 + 16 * swz(2 * lc + 1, r)) = hi;
    } else {
      *reinterpret_cast<uint4*>(base + r * 128 + 16 * swz(lc, r)) = v;
    }
  };
  auto sstore = [&](int buf, auto bits) {
    uint8_t* sW = smem + buf * STAGE;
    uint8_t* sX = sW + BM * 128;
#pragma unroll
    for (int i = 0; i < LA; ++i) put(sW, lr + RPS * i, rw[i], bits);
#pragma unroll
    for (int i = 0; i < LB; ++i) put(sX, lr + RPS * i, rx[i], bits);
  };

  i32x16 acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0;

  // One stage: 4 k-steps of 32; lane group g reads LDS chunk 2j + g (16 int8).
  auto mma_block = [&](int buf, int a, int b, i32x16& c) {
    const uint8_t* sW = smem + buf * STAGE;
    const uint8_t* sX = sW + BM * 128;
    const int rW = wm * WM + 32 * a + l32, rX = wn * WN + 32 * b + l32;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cc = 2 * j + lgrp;
      const uint4 fa = *reinterpret_cast<const uint4*>(sW + rW * 128 + 16 * swz(cc, rW));
      const uint4 fb = *reinterpret_cast<const uint4*>(sX + rX * 128 + 16 * swz(cc, rX));
      c = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, fa), __builtin_bit_cast(i32x4, fb), c, 0, 0,
                                                0);
    }
  };
  // Fragments of one 32-k step (lane group g reads LDS chunk 2j + g); packed
  // 16-byte chunks hold 32 codes = two MFMA k-steps, int8 chunks one.
  auto read_frags = [&](int buf, int j, uint4 (&fa)[FM], uint4 (&fb)[FN]) {
    const uint8_t* sW = smem + buf * STAGE;
    const uint8_t* sX = sW + BM * 128;
    const int cc = 2 * j + lgrp;
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      const int r = wm * WM + 32 * f + l32;
      fa[f] = *reinterpret_cast<const uint4*>(sW + r * 128 + 16 * swz(cc, r));
    }
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int r = wn * WN + 32 * f + l32;
      fb[f] = *reinterpret_cast<const uint4*>(sX + r * 128 + 16 * swz(cc, r));
    }
  };
  auto mma_step = [&](const uint4 (&fa)[FM], const uint4 (&fb)[FN]) {
    if constexpr (PACKED) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        i32x4 oa[FM], ob[FN];
#pragma unroll
        for (int f = 0; f < FM; ++f) oa[f] = h ? unpack16(fa[f].z, fa[f].w) : unpack16(fa[f].x, fa[f].y);
#pragma unroll
        for (int f = 0; f < FN; ++f) ob[f] = h ? unpack16(fb[f].z, fb[f].w) : unpack16(fb[f].x, fb[f].y);
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
          for (int b = 0; b < FN; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(oa[a], ob[b], acc[a][b], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, fa[a]),
                                                            __builtin_bit_cast(i32x4, fb[b]), acc[a][b], 0, 0, 0);
    }
  };
  // One stage, software-pipelined: the fragments of step j + 1 are read from
  // LDS while the MFMAs of step j run; step 0's fragments come in loaded.
  uint4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  auto compute = [&](int buf) {
    read_frags(buf, 1, fa1, fb1);
    mma_step(fa0, fb0);
    read_frags(buf, 2, fa0, fb0);
    mma_step(fa1, fb1);
    read_frags(buf, 3, fa1, fb1);
    mma_step(fa0, fb0);
    mma_step(fa1, fb1);
  };

  // ---- main loop ----
  const int KT = (g.Kb + CPR * 16 - 1) / (CPR * 16);
  using bits_t = std::integral_constant<int, BITS>;
  if (KT > 0) {
    gload(pw, px, 0, g.Kb);
    sstore(0, bits_t{});
  }
  __syncthreads();
  if (KT > 0) read_frags(0, 0, fa0, fb0);
  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    if (more) gload(pw, px, kt + 1, g.Kb);
    compute(kt & 1);
    if (more) sstore((kt + 1) & 1, bits_t{});
    __syncthreads();
    if (more) read_frags((kt + 1) & 1, 0, fa0, fb0);
  }

  // ---- epilogue ----
  // 32x32 result layout: lane l, element e -> row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32;
  // here row = channel, column = token.  ch(a, e4): first of the 4 channels of group e4.
  auto chan = [&](int a, int e4) { return ch0 + wm * WM + 32 * a + 8 * e4 + 4 * lgrp; };
  auto tok = [&](int b) { return tk0 + wn * WN + 32 * b + l32; };
  auto load4 = [&](const float* p, int c) -> float4 {  // p[c..c+3], clamped at the channel tail
    if (c + 3 < g.N) return *reinterpret_cast<const float4*>(p + c);
    return float4{p[min(c, g.N - 1)], p[min(c + 1, g.N - 1)], p[min(c + 2, g.N - 1)], p[min(c + 3, g.N - 1)]};
  };
  auto store4 = [&](int t, int c, float y0, float y1, float y2, float y3) {
    if (t >= g.M) return;
    if (g.y_bf16) {
      bf16_t* yp = reinterpret_cast<bf16_t*>(g.Y) + (size_t)t * g.ldy + c;
      if (c + 3 < g.N && ((g.ldy & 3) == 0)) {
        *reinterpret_cast<uint2*>(yp) = uint2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
      } else {
        const float v[4] = {y0, y1, y2, y3};
        for (int q = 0; q < 4; ++q)
          if (c + q < g.N) yp[q] = (bf16_t)f32_to_bf16_bits(v[q]);
      }
    } else {
      float* yp = reinterpret_cast<float*>(g.Y) + (size_t)t * g.ldy + c;
      if (c + 3 < g.N && ((g.ldy & 3) == 0)) {
        *reinterpret_cast<float4*>(yp) = float4{y0, y1, y2, y3};
      } else {
        const float v[4] = {y0, y1, y2, y3};
        for (int q = 0; q < 4; ++q)
          if (c + q < g.N) yp[q] = v[q];
      }
    }
  };
  constexpr int SH = (BITS == 4) ? 8 : 0;  // int8 lanes carry 16 * code: acc = 256 * sum

  // bf16 output of the rank-augmented epilogue is staged per wave in LDS (the
  // main loop's buffers are free by then): WN token rows of WM channels.
  // Row r, 16-byte chunk j (8 channels) sits at chunk j ^ sw(r) (sw = r % 16
  // for 256-byte rows, (r / 2) % 8 for 128-byte rows, whose odd rows already
  // sit on the other 32 banks), and rows with bit 4 set swap the two 8-byte
  // halves of each chunk, so the 8-byte writes of 32 consecutive rows and
  // the 16-byte reads of whole rows both touch every bank once per pass.
  constexpr bool STAGE_Y = EPI == EPI_LINEAR;
  constexpr int YCH = WM / 8;  // 16-byte chunks per staged row
  static_assert(!STAGE_Y || (WGM * WGN * WN * WM * 2 <= 2 * STAGE), "staged Y tile exceeds LDS");
  static_assert(!STAGE_Y || (YCH == 8 || YCH == 16), "staged row width");
  uint8_t* sYw = smem + wave * (WN * WM * 2);
  auto ychunk = [&](int row, int j) -> int {
    const int sw = (YCH == 16) ? (row & 15) : ((row >> 1) & 7);
    return row * (WM * 2) + 16 * (j ^ sw);
  };
  auto yslot = [&](int row, int j, int half) -> int { return ychunk(row, j) + 8 * (half ^ ((row >> 4) & 1)); };

  if constexpr (EPI == EPI_ACC) {
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b) {
        const int t = tok(b);
        if (t >= g.M) continue;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int c = chan(a, e4);
          int32_t* op = g.acc + (size_t)t * g.N + c;
          const int v0 = acc[a][b][4 * e4] >> SH, v1 = acc[a][b][4 * e4 + 1] >> SH;
          const int v2 = acc[a][b][4 * e4 + 2] >> SH, v3 = acc[a][b][4 * e4 + 3] >> SH;
          if (c + 3 < g.N && (g.N & 3) == 0) {
            *reinterpret_cast<int4*>(op) = int4{v0, v1, v2, v3};
          } else {
            const int v[4] = {v0, v1, v2, v3};
            for (int q = 0; q < 4; ++q)
              if (c + q < g.N) op[q] = v[q];
          }
        }
      }
    return;
  } else {
    // One 32x32 block at a time: dequantise (y = acc * s_w[channel] * s_x[token]),
    // add the second low-rank stage (rank-augmented layer) or the high-subspace
    // product (two-subspace layer), store.  Only one block's outputs are live.
    const int KT2 = (EPI == EPI_MP) ? (g.Kb2 + 127) / 128 : 0;
    if constexpr (EPI == EPI_MP) {
      if (KT2 > 0) {
        // stage the first 256 k of the high subspace (8-bit codes) into the two buffers
        constexpr int RPS8 = NT / 8, LA8 = BM / RPS8, LB8 = BN / RPS8;
        const int lc8 = tid & 7, lr8 = tid >> 3;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int kb = h * 128;
          const bool ok = (h < KT2) && (kb + 16 * lc8 < g.Kb2);
          uint8_t* sW = smem + h * STAGE;
          uint8_t* sX = sW + BM * 128;
#pragma unroll
          for (int i = 0; i < LA8; ++i) {
            const int r = lr8 + RPS8 * i;
            const uint8_t* p = g.B2 + (size_t)min(ch0 + r, g.N - 1) * g.ldb2 + 16 * lc8 + kb;
            *reinterpret_cast<uint4*>(sW + r * 128 + 16 * swz(lc8, r)) =
                ok ? *reinterpret_cast<const uint4*>(p) : uint4{0, 0, 0, 0};
          }
#pragma unroll
          for (int i = 0; i < LB8; ++i) {
            const int r = lr8 + RPS8 * i;
            const uint8_t* p = g.A2 + (size_t)min(tk0 + r, g.M - 1) * g.lda2 + 16 * lc8 + kb;
            *reinterpret_cast<uint4*>(sX + r * 128 + 16 * swz(lc8, r)) =
                ok ? *reinterpret_cast<const uint4*>(p) : uint4{0, 0, 0, 0};
          }
        }
        __syncthreads();
      }
    }
#pragma unroll
    for (int a = 0; a < FM; ++a) {
#pragma unroll
      for (int b = 0; b < FN; ++b) {
        const int tt = min(tok(b), g.M - 1);
        const float sx = g.sx[tt];
        f32x16 y;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const float4 w = load4(g.sw, chan(a, e4));
          y[4 * e4 + 0] = (float)(acc[a][b][4 * e4 + 0] >> SH) * (w.x * sx);
          y[4 * e4 + 1] = (float)(acc[a][b][4 * e4 + 1] >> SH) * (w.y * sx);
          y[4 * e4 + 2] = (float)(acc[a][b][4 * e4 + 2] >> SH) * (w.z * sx);
          y[4 * e4 + 3] = (float)(acc[a][b][4 * e4 + 3] >> SH) * (w.w * sx);
        }
        if constexpr (EPI == EPI_LINEAR) {
          // D[channel][token] += sum_t L2^T[channel][t] T[token][t] on the bf16 MFMA
          if (g.r_pad > 0) {
            const int c = min(ch0 + wm * WM + 32 * a + l32, g.N - 1);
            const bf16_t* lp = g.L2t + (size_t)c * g.r_pad + 8 * lgrp;
            const bf16_t* tp = g.T + (size_t)tt * g.r_pad + 8 * lgrp;
            for (int t0 = 0; t0 < g.r_pad; t0 += 16) {
              const uint4 av = *reinterpret_cast<const uint4*>(lp + t0);
              const uint4 bv = *reinterpret_cast<const uint4*>(tp + t0);
              y = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(bv), y, 0, 0, 0);
            }
          }
        } else {
          if (KT2 > 0) {
            i32x16 t;
#pragma unroll
            for (int i = 0; i < 16; ++i) t[i] = 0;
            mma_block(0, a, b, t);
            if (KT2 > 1) mma_block(1, a, b, t);
            // k beyond the 256 staged in LDS: fragments straight from global (L2)
            for (int kk = 2; kk < KT2; ++kk) {
              const int cw = min(ch0 + wm * WM + 32 * a + l32, g.N - 1);
              const uint8_t* pw2 = g.B2 + (size_t)cw * g.ldb2 + kk * 128 + 16 * lgrp;
              const uint8_t* px2 = g.A2 + (size_t)tt * g.lda2 + kk * 128 + 16 * lgrp;
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const bool ok = kk * 128 + 32 * j + 16 * lgrp < g.Kb2;
                const uint4 fa = ok ? *reinterpret_cast<const uint4*>(pw2 + 32 * j) : uint4{0, 0, 0, 0};
                const uint4 fb = ok ? *reinterpret_cast<const uint4*>(px2 + 32 * j) : uint4{0, 0, 0, 0};
                t = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, fa), __builtin_bit_cast(i32x4, fb),
                                                          t, 0, 0, 0);
              }
            }
            const float sxh = g.sx2[tt];
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
              const float4 w = load4(g.sw2, chan(a, e4));
              y[4 * e4 + 0] += (float)t[4 * e4 + 0] * (w.x * sxh);
              y[4 * e4 + 1] += (float)t[4 * e4 + 1] * (w.y * sxh);
              y[4 * e4 + 2] += (float)t[4 * e4 + 2] * (w.z * sxh);
              y[4 * e4 + 3] += (float)t[4 * e4 + 3] * (w.w * sxh);
            }
          }
        }
        if (STAGE_Y && g.y_bf16) {
          // bf16 result into the wave's LDS tile (see the write-out below)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int row = 32 * b + l32;
            *reinterpret_cast<uint2*>(sYw + yslot(row, 4 * a + e4, lgrp)) =
                uint2{pack_bf16x2(y[4 * e4], y[4 * e4 + 1]), pack_bf16x2(y[4 * e4 + 2], y[4 * e4 + 3])};
          }
        } else {
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4)
            store4(tok(b), chan(a, e4), y[4 * e4], y[4 * e4 + 1], y[4 * e4 + 2], y[4 * e4 + 3]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (STAGE_Y && g.y_bf16) {
      // Write-out of the wave's WN tokens x WM channels: 16 bytes per lane,
      // WM / 8 lanes per token row, so each token's WM * 2 contiguous bytes of
      // Y go out as whole cache lines.
      __syncthreads();
      constexpr int RPI = 64 / YCH;  // token rows per instruction
      const int jc = lane % YCH, rsub = lane / YCH;
      const int c = ch0 + wm * WM + 8 * jc;
#pragma unroll 4
      for (int r0 = 0; r0 < WN; r0 += RPI) {
        const int row = r0 + rsub;
        const int t = tk0 + wn * WN + row;
        uint4 v = *reinterpret_cast<const uint4*>(sYw + ychunk(row, jc));
        if ((row >> 4) & 1) v = uint4{v.z, v.w, v.x, v.y};
        if (t < g.M) {
          bf16_t* yp = reinterpret_cast<bf16_t*>(g.Y) + (size_t)t * g.ldy + c;
          if (c + 7 < g.N && (g.ldy & 7) == 0) {
            *reinterpret_cast<uint4*>(yp) = v;
          } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            for (int q = 0; q < 8; ++q)
              if (c + q < g.N) yp[q] = (bf16_t)((q & 1) ? (w[q >> 1] >> 16) : (w[q >> 1] & 0xFFFFu));
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Small-n kernel (M <= 32): memory-bound on the weight codes.
//   Block: 16 output channels; WAVES waves split K into contiguous ranges of
//   64-byte steps (lane group g of 16 lanes loads bytes 16 g .. 16 g + 15 of
//   each step for channel lane % 16).  Every load of a batch of U steps --
//   weights, the matching activation codes, and the low-rank operands -- is
//   issued before the first wait, so a block pays one memory round trip per
//   batch.  MFMA 16x16x64 int8 (TWO: a second 16-token tile shares each
//   weight fragment); the waves' int32 partials are summed exactly through
//   LDS in wave order.
//   Epilogue: T is the sum over the k-chunks of the fp32 partials of X L1
//   written by the prologue (P; chunk order, then rounded to bf16; block 0
//   also writes it to Tout); T L2 for the block's 16 channels
//   is one 16x16 bf16 MFMA chain whose result layout matches the integer
//   accumulator's (lane l, element i -> token 4 (l / 16) + i, channel l % 16).
// ---------------------------------------------------------------------------
template <int BITS, int EPI, int WAVES, bool TWO>
__global__ __launch_bounds__(WAVES * 64, (WAVES == 4) ? 4 : 2) void k_gemv(GemmArgs g) {
  constexpr int U = (WAVES == 4 || TWO) ? 8 : 16;  // 64-byte steps per wave per batch
  constexpr int NT = WAVES * 64;
  constexpr int MT = TWO ? 32 : 16;  // token rows held for the low-rank stage
  constexpr bool LR = EPI == EPI_LINEAR;
  __shared__ int red[WAVES][TWO ? 2 : 1][4][64];
  __shared__ __attribute__((aligned(16))) bf16_t sT[LR ? MT * 256 : 1];
  __shared__ __attribute__((aligned(16))) bf16_t sL[LR ? 16 * 256 : 1];
  __shared__ __attribute__((aligned(16))) float4 sPart[LR ? NT : 1][2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const uint8_t* bp = g.B + (size_t)min(n0 + l16, g.N - 1) * g.ldb + 16 * lg;
  const uint8_t* ap0 = g.A + (size_t)min(l16, g.M - 1) * g.lda + 16 * lg;
  const uint8_t* ap1 = g.A + (size_t)min(16 + l16, g.M - 1) * g.lda + 16 * lg;
  const int KS = (g.Kb + 63) / 64;
  const int per = (KS + WAVES - 1) / WAVES;
  const int sbeg = wave * per, send = min(KS, sbeg + per);
  const int rp = LR ? g.r_pad : 0;
  const int rq = rp / 8;  // 16-byte pieces (8 values) per low-rank row
  // T pieces: NP = M rows x rq; G thread groups (no more than there are
  // chunks) split the k-chunks of each piece, at most two chunks per group
  const int NP = g.M * rq;
  const int G = max(1, min(NT / max(NP, 1), LR ? g.nchunk : 1));

  // Loads are unconditional, from clamped (always valid) addresses, and
  // masked where used: conditional loads become branches whose register
  // merges force early waits on every load in flight.
  const int kb_last = max(0, min((max(send, sbeg + 1) - 1) * 64, g.Kb - 16 - 16 * lg));
  uint4 bv[U], av0[U], av1[U];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) bv[u] = *reinterpret_cast<const uint4*>(bp + min((s0 + u) * 64, kb_last));
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = min((s0 + u) * 64, kb_last);
      av0[u] = *reinterpret_cast<const uint4*>(ap0 + kb);
      if (TWO) av1[u] = *reinterpret_cast<const uint4*>(ap1 + kb);
    }
  };
  i32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  auto mma_batch = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u >= send) continue;
      if ((s0 + u) * 64 + 16 * lg >= g.Kb) {  // this lane group's 16 bytes lie past the row: zero codes
        bv[u] = uint4{0, 0, 0, 0};
        av0[u] = uint4{0, 0, 0, 0};
        av1[u] = uint4{0, 0, 0, 0};
      }
      if (BITS == 4) {
        const i32x4 b0 = unpack16(bv[u].x, bv[u].y), b1 = unpack16(bv[u].z, bv[u].w);
        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16(av0[u].x, av0[u].y), b0, acc0, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16(av0[u].z, av0[u].w), b1, acc0, 0, 0, 0);
        if (TWO) {
          acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16(av1[u].x, av1[u].y), b0, acc1, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16(av1[u].z, av1[u].w), b1, acc1, 0, 0, 0);
        }
      } else {
        const i32x4 b0 = __builtin_bit_cast(i32x4, bv[u]);
        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, av0[u]), b0, acc0, 0, 0, 0);
        if (TWO) acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, av1[u]), b0, acc1, 0, 0, 0);
      }
    }
  };

  // ---- issue every load of the first batch before any wait ----
  float sxv[4], swv = 0.0f;  // epilogue scales
  if (LR) {
    swv = g.sw[min(n0 + l16, g.N - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i) sxv[i] = g.sx[min(16 * (wave & 1) + 4 * lg + i, g.M - 1)];
  }
  load_batch(sbeg);
  // Low-rank operands, with clamped (always valid) indices, masked where used,
  // so that none of them needs a wait before the integer product: piece
  // tid of L2^T (16 x rp), and for thread (piece p, group q), q < G, of T
  // the chunks q and q + G of the prologue's fp32 partials.
  uint4 lv;
  float4 pv[2][2];
  if (LR && rp > 0) {
    const int el = min(tid, 16 * rq - 1);
    lv = *reinterpret_cast<const uint4*>(g.L2t + (size_t)min(n0 + el / rq, g.N - 1) * rp + 8 * (el % rq));
    if (tid < NP * G) {
      const int pc = tid % NP, grp = tid / NP;
      const int rowt = pc / rq, qt = pc % rq;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int c = min(grp + G * j, g.nchunk - 1);
        const float4* pp = reinterpret_cast<const float4*>(g.P + ((size_t)c * g.M + rowt) * rp + 8 * qt);
        pv[j][0] = pp[0];
        pv[j][1] = pp[1];
      }
    }
  }

  // ---- integer product ----
  mma_batch(sbeg);
  for (int s0 = sbeg + U; s0 < send; s0 += U) {
    load_batch(s0);
    mma_batch(s0);
  }

  // ---- low-rank operands into LDS (T rows >= M are zero) ----
  if (LR && rp > 0) {
    if (tid < 16 * rq) *reinterpret_cast<uint4*>(sL + tid * 8) = (n0 + tid / rq < g.N) ? lv : uint4{0, 0, 0, 0};
    for (int e = tid + NT; e < 16 * rq; e += NT) {
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
            const float4* pp = reinterpret_cast<const float4*>(g.P + ((size_t)k * g.M + row) * rp + 8 * q);
            const float4 x0 = pp[0], x1 = pp[1];
            t[0] += x0.x; t[1] += x0.y; t[2] += x0.z; t[3] += x0.w;
            t[4] += x1.x; t[5] += x1.y; t[6] += x1.z; t[7] += x1.w;
          }
        }
        v = uint4{pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3]), pack_bf16x2(t[4], t[5]), pack_bf16x2(t[6], t[7])};
        if (blockIdx.x == 0 && g.Tout) *reinterpret_cast<uint4*>(g.Tout + (size_t)row * rp + 8 * q) = v;
      }
      *reinterpret_cast<uint4*>(sT + pc * 8) = v;
    }
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    red[wave][0][i][lane] = acc0[i];
    if (TWO) red[wave][TWO ? 1 : 0][i][lane] = acc1[i];
  }
  __syncthreads();
  // wave t (t < number of 16-token tiles) finishes tile t
  constexpr int TILES = TWO ? 2 : 1;
  if (wave >= TILES) return;
  const int tile = wave;
  int sacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int v = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) v += red[w][tile][i][lane];
    sacc[i] = (BITS == 4) ? (v >> 8) : v;
  }
  const int col = n0 + l16;
  if constexpr (EPI == EPI_ACC) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * tile + 4 * lg + i;
      if (row < g.M && col < g.N) g.acc[(size_t)row * g.N + col] = sacc[i];
    }
  } else {
    f32x4 lr = {0.f, 0.f, 0.f, 0.f};
    for (int t0 = 0; t0 < rp; t0 += 32) {
      // A: T rows (tokens), B: L2^T rows (channels); 8 consecutive t per lane
      const uint4 a8 = *reinterpret_cast<const uint4*>(sT + (16 * tile + l16) * rp + t0 + 8 * lg);
      const uint4 b8 = *reinterpret_cast<const uint4*>(sL + l16 * rp + t0 + 8 * lg);
      lr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a8), as_bf16x8(b8), lr, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * tile + 4 * lg + i;
      if (row >= g.M || col >= g.N) continue;
      const float y = (float)sacc[i] * (sxv[i] * swv) + lr[i];
      if (g.y_bf16)
        reinterpret_cast<bf16_t*>(g.Y)[(size_t)row * g.ldy + col] = (bf16_t)f32_to_bf16_bits(y);
      else
        reinterpret_cast<float*>(g.Y)[(size_t)row * g.ldy + col] = y;
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
// Tile-kernel variants; the default is the fastest measured on MI355X, the
// TQ_GEMM_VARIANT environment variable (read once) overrides it for tuning:
//   0: 256x256 tile, 8 waves of 128x64, int8 LDS (128-k stages)
//   1: 256x256 tile, 8 waves of 128x64, packed LDS (256-k stages)
//   2: 256x256 tile, 4 waves of 128x128, packed LDS
//   3: 256x256 tile, 4 waves of 128x128, int8 LDS
static int gemm_variant() {
  static const int v = [] {
    const char* e = getenv("TQ_GEMM_VARIANT");
    return e ? atoi(e) : 1;
  }();
  return v;
}

template <int BITS, int EPI>
static hipError_t gemm_tiles(const GemmArgs& g, hipStream_t st) {
  const long big = (long)((g.M + 255) / 256) * ((g.N + 255) / 256);
  const dim3 grid((unsigned)big);
  if (big >= 224) {
    switch (gemm_variant()) {
      case 0: hipLaunchKernelGGL((k_gemm<BITS, EPI, 256, 256, 2, 4, false>), grid, dim3(512), 0, st, g); break;
      case 2: hipLaunchKernelGGL((k_gemm<BITS, EPI, 256, 256, 2, 2, true>), grid, dim3(256), 0, st, g); break;
      case 3: hipLaunchKernelGGL((k_gemm<BITS, EPI, 256, 256, 2, 2, false>), grid, dim3(256), 0, st, g); break;
      default: hipLaunchKernelGGL((k_gemm<BITS, EPI, 256, 256, 2, 4, true>), grid, dim3(512), 0, st, g); break;
    }
  } else {
    const unsigned blocks = (unsigned)(((g.M + 127) / 128) * ((g.N + 127) / 128));
    hipLaunchKernelGGL((k_gemm<BITS, EPI, 128, 128, 2, 2, true>), dim3(blocks), dim3(256), 0, st, g);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, int bits, Epilogue epi, hipStream_t st) {
  if (bits == 4) {
    switch (epi) {
      case EPI_ACC: return gemm_tiles<4, EPI_ACC>(g, st);
      case EPI_LINEAR: return gemm_tiles<4, EPI_LINEAR>(g, st);
      case EPI_MP: return gemm_tiles<4, EPI_MP>(g, st);
    }
  } else if (bits == 8 && epi == EPI_ACC) {
    return gemm_tiles<8, EPI_ACC>(g, st);
  }
  return hipErrorInvalidValue;
}

template <int BITS, int EPI, bool TWO>
static hipError_t gemv_cols_t(const GemmArgs& g, hipStream_t st) {
  const unsigned blocks = (unsigned)((g.N + 15) / 16);
  if (g.Kb > 2048)
    hipLaunchKernelGGL((k_gemv<BITS, EPI, 8, TWO>), dim3(blocks), dim3(512), 0, st, g);
  else
    hipLaunchKernelGGL((k_gemv<BITS, EPI, 4, TWO>), dim3(blocks), dim3(256), 0, st, g);
  return hipGetLastError();
}

template <int BITS, int EPI>
static hipError_t gemv_cols(const GemmArgs& g, hipStream_t st) {
  if (EPI == EPI_LINEAR && (g.r_pad > 256 || (g.r_pad > 0 && (!g.P || g.nchunk < 1)))) return hipErrorInvalidValue;
  return g.M > 16 ? gemv_cols_t<BITS, EPI, true>(g, st) : gemv_cols_t<BITS, EPI, false>(g, st);
}

hipError_t launch_gemv(const GemmArgs& g, int bits, Epilogue epi, hipStream_t st) {
  if (bits == 4) {
    if (epi == EPI_ACC) return gemv_cols<4, EPI_ACC>(g, st);
    if (epi == EPI_LINEAR) return gemv_cols<4, EPI_LINEAR>(g, st);
  } else if (bits == 8 && epi == EPI_ACC) {
    return gemv_cols<8, EPI_ACC>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
