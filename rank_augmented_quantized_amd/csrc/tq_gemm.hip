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

#include "tq_kernels.h"

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
// ---------------------------------------------------------------------------
// Most bytes of activation codes the small-n GEMM stages in LDS: what
// leaves the blocks per CU of its launch bounds (2 of 8 waves, 4 of 4 waves)
// within the 160 KB of LDS next to the static arrays.
__host__ __device__ constexpr int gemv_xl_bytes(int waves) { return waves == 8 ? 24576 : 12288; }

template <int BITS, int EPI, int WAVES, bool TWO, bool XL>
__global__ __launch_bounds__(WAVES * 64, (WAVES == 4) ? 4 : 2) void k_gemv(GemmArgs g) {
  constexpr int U = (WAVES == 4 && TWO && !XL) ? 4 : ((WAVES == 4 || TWO) ? 8 : 16);  // 64-byte steps per wave per batch
  constexpr int NT = WAVES * 64;
  constexpr int MT = TWO ? 32 : 16;  // token rows held for the low-rank stage
  constexpr bool LR = EPI == EPI_LINEAR;
  constexpr bool QL = EPI == EPI_QLR;  // quantised low-rank branch: second stage on the int8 MFMA
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
  if (XL) {
#pragma unroll
    for (int i = 0; i < XLN; ++i) {
      const int idx = min(tid + NT * i, g.M * kp - 1);
      xst[i] = *reinterpret_cast<const uint4*>(g.A + (size_t)(idx / kp) * g.lda + 16 * (idx % kp));
    }
  }

  // Loads are unconditional, from clamped (always valid) addresses, and
  // masked where used: conditional loads become branches whose register
  // merges force early waits on every load in flight.
  const int kb_last = max(0, min((max(send, sbeg + 1) - 1) * 64, g.Kb - 16 - 16 * lg));
  uint4 bv[U], av0[U], av1[U];
  auto load_batch = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) bv[u] = *reinterpret_cast<const uint4*>(bp + min((s0 + u) * 64, kb_last));
    if (XL) return;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = min((s0 + u) * 64, kb_last);
      av0[u] = *reinterpret_cast<const uint4*>(ap0 + kb);
      if (TWO) av1[u] = *reinterpret_cast<const uint4*>(ap1 + kb);
    }
  };
  const uint8_t* xl0 = xl_lds + min(l16, g.M - 1) * XS + 16 * lg;
  const uint8_t* xl1 = xl_lds + min(16 + l16, g.M - 1) * XS + 16 * lg;
  i32x4 acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
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
  // asymmetric activations (codes u - 8): per row z + 8 s_x, per channel
  // s_w colsum(C_w) (CoQuant Eq. 1 with a zero-point)
  float zzv[4] = {0.f, 0.f, 0.f, 0.f}, wzv = 0.0f;
  if (LR || QL) {
    swv = g.sw[min(n0 + l16, g.N - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i) sxv[i] = g.sx[min(16 * (wave & 1) + 4 * lg + i, g.M - 1)];
    if (LR && g.zx) {
      wzv = swv * (float)g.csw[min(n0 + l16, g.N - 1)];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = min(16 * (wave & 1) + 4 * lg + i, g.M - 1);
        zzv[i] = g.zx[rr] + 8.0f * g.sx[rr];
      }
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
    }
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
      const float y = (float)sacc[i] * (sxv[i] * swv) + lr[i] + zzv[i] * wzv;
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
template <int BITS, int EPI, bool TWO>
static hipError_t gemv_cols_t(const GemmArgs& g, hipStream_t st) {
  const unsigned blocks = (unsigned)((g.N + 15) / 16);
  const size_t xl = (size_t)g.M * (size_t)(g.Kb + 16);  // activation codes in LDS
  const bool use_xl = xl <= (size_t)gemv_xl_bytes(g.Kb > 2048 ? 8 : 4) && g.Kb % 16 == 0;
  if (g.Kb > 2048) {
    if (use_xl)
      hipLaunchKernelGGL((k_gemv<BITS, EPI, 8, TWO, true>), dim3(blocks), dim3(512), xl, st, g);
    else
      hipLaunchKernelGGL((k_gemv<BITS, EPI, 8, TWO, false>), dim3(blocks), dim3(512), 0, st, g);
  } else {
    if (use_xl)
      hipLaunchKernelGGL((k_gemv<BITS, EPI, 4, TWO, true>), dim3(blocks), dim3(256), xl, st, g);
    else
      hipLaunchKernelGGL((k_gemv<BITS, EPI, 4, TWO, false>), dim3(blocks), dim3(256), 0, st, g);
  }
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
    if (epi == EPI_QLR) return gemv_cols<4, EPI_QLR>(g, st);
  } else if (bits == 8 && epi == EPI_ACC) {
    return gemv_cols<8, EPI_ACC>(g, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace tq
