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

#include "tq_kernels.h"

namespace tq {

// ---------------------------------------------------------------------------
// Tile kernel (any M; chosen for M > 32).
//   256 threads = 4 waves in a 2 x 2 grid; wave tile (BM/2) x (BN/2) made of
//   32 x 32 MFMA blocks.  One k-stage = 128 code bytes per row (256 k at 4
//   bits, 128 k at 8 bits), double-buffered in LDS; the next stage is loaded
//   from global into registers while the current one is multiplied.
//   LDS rows are 128 bytes = 8 chunks of 16 bytes; chunk c of row r is stored
//   at position c ^ (r & 7) ^ ((r >> 3) & 1) so that the 16-byte fragment
//   reads of 8 or 16 consecutive rows hit distinct banks.
//   4-bit codes stay packed in LDS and are unpacked in registers
//   (nib_lo / nib_hi: each int8 lane = 16 * code, so acc = 256 * true sum).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz(int c, int r) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

template <int BITS, int EPI, int BM, int BN>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g) {
  constexpr int WM = BM / 2, WN = BN / 2, FM = WM / 32, FN = WN / 32;
  constexpr int LA = BM / 32, LB = BN / 32;  // 16-byte global loads per thread per stage
  constexpr int STAGE = (BM + BN) * 128;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lgrp = lane >> 5;

  const int tiles_n = (g.N + BN - 1) / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;

  const int lc = tid & 7, lr = tid >> 3;
  const uint8_t* pa[LA];
  const uint8_t* pb[LB];
#pragma unroll
  for (int i = 0; i < LA; ++i) pa[i] = g.A + (size_t)min(m0 + lr + 32 * i, g.M - 1) * g.lda + 16 * lc;
#pragma unroll
  for (int i = 0; i < LB; ++i) pb[i] = g.B + (size_t)min(n0 + lr + 32 * i, g.N - 1) * g.ldb + 16 * lc;

  uint4 ra[LA], rb[LB];
  auto gload = [&](int kt, int Kb) {
    const int kb = kt * 128;
    const bool ok = kb + 16 * lc < Kb;
#pragma unroll
    for (int i = 0; i < LA; ++i) ra[i] = ok ? *reinterpret_cast<const uint4*>(pa[i] + kb) : uint4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < LB; ++i) rb[i] = ok ? *reinterpret_cast<const uint4*>(pb[i] + kb) : uint4{0, 0, 0, 0};
  };
  auto sstore = [&](int buf) {
    uint8_t* sA = smem + buf * STAGE;
    uint8_t* sB = sA + BM * 128;
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int r = lr + 32 * i;
      *reinterpret_cast<uint4*>(sA + r * 128 + 16 * swz(lc, r)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int r = lr + 32 * i;
      *reinterpret_cast<uint4*>(sB + r * 128 + 16 * swz(lc, r)) = rb[i];
    }
  };

  i32x16 acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0;

  auto compute = [&](int buf, int bits) {
    const uint8_t* sA = smem + buf * STAGE;
    const uint8_t* sB = sA + BM * 128;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 2 * j + lgrp;
      uint4 fa[FM], fb[FN];
#pragma unroll
      for (int f = 0; f < FM; ++f) {
        const int r = wm * WM + 32 * f + l32;
        fa[f] = *reinterpret_cast<const uint4*>(sA + r * 128 + 16 * swz(c, r));
      }
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        const int r = wn * WN + 32 * f + l32;
        fb[f] = *reinterpret_cast<const uint4*>(sB + r * 128 + 16 * swz(c, r));
      }
      if (bits == 4) {
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
    }
  };

  // ---- main loop over the first segment ----
  const int KT = (g.Kb + 127) / 128;
  if (KT > 0) {
    gload(0, g.Kb);
    sstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    if (more) gload(kt + 1, g.Kb);
    compute(kt & 1, BITS);
    if (more) sstore((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue ----
  // 32x32 MFMA result layout: lane l, element i -> row 8*(i/4) + 4*(l/32) + i%4, column l%32.
  if constexpr (EPI == EPI_ACC) {
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b) {
        const int col = n0 + wn * WN + 32 * b + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = m0 + wm * WM + 32 * a + 8 * (i >> 2) + 4 * lgrp + (i & 3);
          if (row < g.M && col < g.N) g.acc[(size_t)row * g.N + col] = (BITS == 4) ? (acc[a][b][i] >> 8) : acc[a][b][i];
        }
      }
    return;
  } else {
    f32x16 y[FM][FN];
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b) {
        const int col = min(n0 + wn * WN + 32 * b + l32, g.N - 1);
        const float swc = g.sw[col];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = min(m0 + wm * WM + 32 * a + 8 * (i >> 2) + 4 * lgrp + (i & 3), g.M - 1);
          const int v = (BITS == 4) ? (acc[a][b][i] >> 8) : acc[a][b][i];
          y[a][b][i] = (float)v * (g.sx[row] * swc);
        }
      }

    if constexpr (EPI == EPI_LINEAR) {
      if (g.r_pad > 0) {
        // second low-rank stage on the bf16 MFMA, accumulated onto the dequantised tile
#pragma unroll
        for (int a = 0; a < FM; ++a) {
          const int arow = min(m0 + wm * WM + 32 * a + l32, g.M - 1);
          const bf16_t* tp = g.T + (size_t)arow * g.r_pad + 8 * lgrp;
#pragma unroll
          for (int b = 0; b < FN; ++b) {
            const int col = min(n0 + wn * WN + 32 * b + l32, g.N - 1);
            const bf16_t* lp = g.L2t + (size_t)col * g.r_pad + 8 * lgrp;
            for (int t0 = 0; t0 < g.r_pad; t0 += 16) {
              const uint4 av = *reinterpret_cast<const uint4*>(tp + t0);
              const uint4 bv = *reinterpret_cast<const uint4*>(lp + t0);
              y[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(bv), y[a][b], 0, 0, 0);
            }
          }
        }
      }
    } else if constexpr (EPI == EPI_MP) {
      // high-precision (8-bit) segment: its own integer product per 32x32 block
      const int KT2 = (g.Kb2 + 127) / 128;
      const uint8_t* pa2[LA];
      const uint8_t* pb2[LB];
#pragma unroll
      for (int i = 0; i < LA; ++i) pa2[i] = g.A2 + (size_t)min(m0 + lr + 32 * i, g.M - 1) * g.lda2 + 16 * lc;
#pragma unroll
      for (int i = 0; i < LB; ++i) pb2[i] = g.B2 + (size_t)min(n0 + lr + 32 * i, g.N - 1) * g.ldb2 + 16 * lc;
      for (int kt = 0; kt < KT2; ++kt) {
        const int kb = kt * 128;
        const bool ok = kb + 16 * lc < g.Kb2;
#pragma unroll
        for (int i = 0; i < LA; ++i) ra[i] = ok ? *reinterpret_cast<const uint4*>(pa2[i] + kb) : uint4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < LB; ++i) rb[i] = ok ? *reinterpret_cast<const uint4*>(pb2[i] + kb) : uint4{0, 0, 0, 0};
        sstore(0);
        __syncthreads();
        const uint8_t* sA = smem;
        const uint8_t* sB = smem + BM * 128;
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
          for (int b = 0; b < FN; ++b) {
            i32x16 t;
#pragma unroll
            for (int i = 0; i < 16; ++i) t[i] = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int c = 2 * j + lgrp;
              const int rA = wm * WM + 32 * a + l32;
              const int rB = wn * WN + 32 * b + l32;
              const uint4 fa = *reinterpret_cast<const uint4*>(sA + rA * 128 + 16 * swz(c, rA));
              const uint4 fb = *reinterpret_cast<const uint4*>(sB + rB * 128 + 16 * swz(c, rB));
              t = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, fa), __builtin_bit_cast(i32x4, fb),
                                                        t, 0, 0, 0);
            }
            const int col = min(n0 + wn * WN + 32 * b + l32, g.N - 1);
            const float swc = g.sw2[col];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int row = min(m0 + wm * WM + 32 * a + 8 * (i >> 2) + 4 * lgrp + (i & 3), g.M - 1);
              y[a][b][i] += (float)t[i] * (g.sx2[row] * swc);
            }
          }
        __syncthreads();
      }
    }

    // ---- single store of Y ----
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b) {
        const int col = n0 + wn * WN + 32 * b + l32;
        if (col >= g.N) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = m0 + wm * WM + 32 * a + 8 * (i >> 2) + 4 * lgrp + (i & 3);
          if (row >= g.M) continue;
          if (g.y_bf16)
            reinterpret_cast<bf16_t*>(g.Y)[(size_t)row * g.ldy + col] = (bf16_t)f32_to_bf16_bits(y[a][b][i]);
          else
            reinterpret_cast<float*>(g.Y)[(size_t)row * g.ldy + col] = y[a][b][i];
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Small-n kernel (M <= 32): memory-bound on the weight codes.
//   Block: 16 output columns, WAVES waves splitting K in 64-byte steps (each
//   lane group of 16 lanes loads 16 bytes per column per step).  MFMA
//   16x16x64 int8 with up to two 16-row tiles sharing each weight fragment.
//   The waves' int32 partials are summed exactly through LDS; the epilogue
//   (dequantisation + T L2 on the VALU) produces one Y value per thread.
// ---------------------------------------------------------------------------
template <int BITS, int EPI, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_gemv(GemmArgs g) {
  constexpr int U = 4;  // steps in flight per wave
  __shared__ int red[WAVES][2][4][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const bool two = g.M > 16;
  const uint8_t* bp = g.B + (size_t)min(n0 + l16, g.N - 1) * g.ldb + 16 * lg;
  const uint8_t* ap0 = g.A + (size_t)min(l16, g.M - 1) * g.lda + 16 * lg;
  const uint8_t* ap1 = g.A + (size_t)min(16 + l16, g.M - 1) * g.lda + 16 * lg;
  const int KS = (g.Kb + 63) / 64;
  i32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
  for (int s0 = wave * U; s0 < KS; s0 += WAVES * U) {
    uint4 bv[U], av0[U], av1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = (s0 + u) * 64;
      const bool ok = (s0 + u < KS) && (kb + 16 * lg < g.Kb);
      bv[u] = ok ? *reinterpret_cast<const uint4*>(bp + kb) : uint4{0, 0, 0, 0};
      av0[u] = ok ? *reinterpret_cast<const uint4*>(ap0 + kb) : uint4{0, 0, 0, 0};
      av1[u] = (ok && two) ? *reinterpret_cast<const uint4*>(ap1 + kb) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (BITS == 4) {
        const i32x4 b0 = unpack16(bv[u].x, bv[u].y), b1 = unpack16(bv[u].z, bv[u].w);
        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16(av0[u].x, av0[u].y), b0, acc0, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16(av0[u].z, av0[u].w), b1, acc0, 0, 0, 0);
        if (two) {
          acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16(av1[u].x, av1[u].y), b0, acc1, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16(av1[u].z, av1[u].w), b1, acc1, 0, 0, 0);
        }
      } else {
        const i32x4 b0 = __builtin_bit_cast(i32x4, bv[u]);
        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, av0[u]), b0, acc0, 0, 0, 0);
        if (two) acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, av1[u]), b0, acc1, 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    red[wave][0][i][lane] = acc0[i];
    red[wave][1][i][lane] = acc1[i];
  }
  __syncthreads();
  // 16x16 MFMA result layout: lane l, element i -> row 4*(l/16) + i, column l%16.
  for (int o = tid; o < 512; o += WAVES * 64) {
    const int tile = o >> 8, ln = (o >> 2) & 63, i = o & 3;
    const int row = 16 * tile + 4 * (ln >> 4) + i, col = n0 + (ln & 15);
    if (row >= g.M || col >= g.N) continue;
    int s = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s += red[w][tile][i][ln];
    if (BITS == 4) s >>= 8;
    if constexpr (EPI == EPI_ACC) {
      g.acc[(size_t)row * g.N + col] = s;
    } else {
      float y = (float)s * (g.sx[row] * g.sw[col]);
      if (g.r_pad > 0) {
        const bf16_t* tp = g.T + (size_t)row * g.r_pad;
        const bf16_t* lp = g.L2t + (size_t)col * g.r_pad;
        for (int t = 0; t < g.r_pad; t += 8) {
          const uint4 a = *reinterpret_cast<const uint4*>(tp + t);
          const uint4 b = *reinterpret_cast<const uint4*>(lp + t);
          y = fmaf(bf16_lo(a.x), bf16_lo(b.x), y);
          y = fmaf(bf16_hi(a.x), bf16_hi(b.x), y);
          y = fmaf(bf16_lo(a.y), bf16_lo(b.y), y);
          y = fmaf(bf16_hi(a.y), bf16_hi(b.y), y);
          y = fmaf(bf16_lo(a.z), bf16_lo(b.z), y);
          y = fmaf(bf16_hi(a.z), bf16_hi(b.z), y);
          y = fmaf(bf16_lo(a.w), bf16_lo(b.w), y);
          y = fmaf(bf16_hi(a.w), bf16_hi(b.w), y);
        }
      }
      if (g.y_bf16)
        reinterpret_cast<bf16_t*>(g.Y)[(size_t)row * g.ldy + col] = (bf16_t)f32_to_bf16_bits(y);
      else
        reinterpret_cast<float*>(g.Y)[(size_t)row * g.ldy + col] = y;
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int BITS, int EPI>
static hipError_t gemm_tiles(const GemmArgs& g, hipStream_t st) {
  constexpr int BM = 128, BN = 128;
  const unsigned blocks = (unsigned)(((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN));
  hipLaunchKernelGGL((k_gemm<BITS, EPI, BM, BN>), dim3(blocks), dim3(256), 0, st, g);
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

template <int BITS, int EPI>
static hipError_t gemv_cols(const GemmArgs& g, hipStream_t st) {
  const unsigned blocks = (unsigned)((g.N + 15) / 16);
  if (g.Kb >= 4096)
    hipLaunchKernelGGL((k_gemv<BITS, EPI, 8>), dim3(blocks), dim3(512), 0, st, g);
  else
    hipLaunchKernelGGL((k_gemv<BITS, EPI, 4>), dim3(blocks), dim3(256), 0, st, g);
  return hipGetLastError();
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
