// Tile GEMM of the rank-augmented W4A4 layer (gfx950): operands staged from
// HBM straight into LDS, weights kept nibble-packed in LDS and expanded to
// int8 at fragment read, activation codes consumed as int8.
//
// acc[i][j] = sum_k cx[i][k] cw[j][k], exact in int32 on v_mfma_i32_32x32x32_i8
// (TwinQuant notes, "TwinQuant: Learnable Subspace Decomposition for W4A4 LLM
// Quantization", section 02 note on INT32 accumulation, section 04.C and
// Figure 4), then one epilogue: s_x s_w dequantisation plus the second
// low-rank stage T L2 on the bf16 MFMA, and a single store of Y.
//
// Why this shape on gfx950:
//  * staging uses buffer_load ... lds (16 bytes per lane, written to LDS at
//    M0 + 16 x lane): no VGPRs, no VALU and no LDS stores are spent on it, so
//    three 128-k stages can be in flight: the loads of stage k + 2 are issued
//    while stage k is multiplied;
//  * a wave64 VALU instruction occupies its SIMD for 4 cycles and overlaps an
//    int8 MFMA (32 cycles) only partly, so the inner loop keeps VALU work low:
//    activation codes arrive as int8 (written that way by the quantiser)
//    and each wave expands only the packed weight fragments it
//    reads, 6 VALU per 32 x 32 x 32 fragment that feeds FN MFMAs;
//  * the direct loads cannot permute bytes within a lane's 16, so the LDS
//    XOR swizzles (chosen so that fragment reads of 8 or 16 consecutive rows
//    hit distinct banks) are applied to the global addresses instead;
//  * rows past the matrix end and chunks past the row end are fetched with
//    offsets beyond the buffer resource's size, which the hardware turns into
//    zeros: no clamping or masking in the loop.
//
// int8 code order: within every 8 consecutive k, the 4 codes of even k and
// then the 4 codes of odd k, one int8 byte per code.  Two packed weight
// dwords (16 codes, even k in the low nibbles) expand to exactly this order
// (unpack16, 16 x code per byte), so a lane's 16 activation bytes and its
// expanded weight bytes pair equal k in every MFMA slot; the int32 sum is
// 16 x the code product (256 x when the activations come packed and are
// expanded the same way) and is shifted back exactly.
//
// Tile: BM = 256 channels x BN tokens (BN = 256 or 128) per block of 8 waves,
// as a 4 x 2 grid of 64 x BN/2 wave tiles; for grids that would not fill the
// chip, BM = BN = 128 as a 2 x 4 grid of 64 x 32 wave tiles.  Stage: 128 k;
// LDS per stage: packed weights BM rows x 64 bytes, activations BN rows x 128
// bytes (int8) or x 64 bytes (packed, the integer check entry point).

#include "tq_kernels.h"

namespace tq {
namespace {

// Workgroup barrier without the memory-model fences of __syncthreads (which
// would wait for all outstanding vector memory operations); the memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Packed LDS rows (64 bytes = 4 chunks per stage): chunk c of row r sits at
// slot c ^ psw(r); any 8 or 16 consecutive rows read one chunk each on
// distinct banks.
__device__ __forceinline__ int psw(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

// KF: every row's code bytes are a whole number of stages, so no direct load
// needs the per-lane end-of-row test (which costs VALU slots next to the MFMAs)
// DBG: the test-hook instance, which also stores the exact int32 sums of the
// residual product (g.acc) and of the second integer product (g.acc2); its
// code is this template's, with those stores added.
// BM: channels per tile, 256 or 128 (then with BN = 128, the rank-augmented
// and integer-check epilogues only).
template <int EPI, bool XP, int BN, bool W8 = false, bool KF = false, bool DBG = false, int BM = 256>
__global__ __launch_bounds__(512) void k_gemm8(GemmArgs g) {
  static_assert(!W8 || (EPI == EPI_ACC && !XP), "8-bit weights: the integer check only");
  static_assert(BM == 256 || (BM == 128 && BN == 128 && (EPI == EPI_LINEAR || EPI == EPI_ACC)), "tile shapes");
  constexpr int WGM = BM / 64, WGN = 8 / WGM;    // wave grid: 4 x 2 or 2 x 4 (channels x tokens)
  constexpr int WM = BM / WGM, WN = BN / WGN;    // wave tile 64 x BN/2, or 64 x 32
  constexpr int FM = WM / 32, FN = WN / 32;      // 32 x 32 blocks per wave tile
  constexpr int XROW = XP ? 64 : 128;            // LDS bytes per activation row per stage
  constexpr int WROW = W8 ? 128 : 64;            // LDS bytes per weight row per stage
  constexpr int WPL = BM * WROW, XPL = BN * XROW;  // stage planes
  constexpr int SPL = WPL + XPL;
  // stage buffers, NST - 1 stages in flight (packed activations: four, whose
  // 128 KB also hold the bf16 Y staging)
  constexpr int NST = W8 ? 2 : (XP ? 4 : 3);
  constexpr int AHEAD = NST - 1;
  constexpr int WI = WPL / 1024 / 8, XI = XPL / 1024 / 8;  // direct loads per wave per stage
  static_assert(WI >= 1 && XI >= 1, "each wave fills whole 1 KB pieces");
  static_assert(EPI == EPI_ACC || 8 * WN * WM * 2 <= NST * SPL, "Y staging fits in the stage buffers");
  static_assert(EPI != EPI_MP || (BM + BN) * 128 <= NST * SPL, "a 128-k chunk of the 8-bit subspace fits");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NST * SPL];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WGM, wn = wave / WGM;
  const int l32 = lane & 31, lg = lane >> 5;
  int tm, tn;
  const int cend = g.c1 > 0 ? g.c1 : g.N;
  tile_of_block(blockIdx.x, (cend - g.c0 + BM - 1) / BM, (g.M + BN - 1) / BN, tm, tn);
  const int ch0 = g.c0 + tm * BM, tk0 = tn * BN;
  const int Kb = g.Kb;                       // weight code bytes per row (K / 2, or K for 8-bit)
  const int Kx = (XP || W8) ? Kb : 2 * Kb;   // activation bytes per row

  const i32x4 rw = buffer_rsrc(g.B + (size_t)ch0 * g.ldb, (uint32_t)(min(BM, g.N - ch0) * g.ldb));
  const i32x4 rx = buffer_rsrc(g.A + (size_t)tk0 * g.lda, (uint32_t)(min(BN, g.M - tk0) * g.lda));

  // ---- direct loads: load i of wave w fills 1 KB of a plane; lane L writes
  // its 16 bytes at 16 L, so it fetches the chunk whose swizzled slot that is.
  // Packed planes: 16 rows of 64 bytes per load, rows 16 (w + 8 i) + L / 4.
  const int cpk = (lane & 3) ^ (((lane >> 3) ^ (2 * (wave & 1) + (lane >> 5))) & 3);
  // int8 planes: 8 rows of 128 bytes per load, rows 8 (w + 8 i) + L / 8
  const int c8 = (lane & 7) ^ (lane >> 3) ^ (wave & 1);
  const int cw = W8 ? c8 : cpk;
  int vw[WI], vx[XI];
#pragma unroll
  for (int i = 0; i < WI; ++i)
    vw[i] = W8 ? (int)((8 * (wave + 8 * i) + (lane >> 3)) * g.ldb) + 16 * c8
               : (int)((16 * (wave + 8 * i) + (lane >> 2)) * g.ldb) + 16 * cpk;
  const int cx = XP ? cpk : c8;
#pragma unroll
  for (int i = 0; i < XI; ++i)
    vx[i] = XP ? (int)((16 * (wave + 8 * i) + (lane >> 2)) * g.lda) + 16 * cpk
               : (int)((8 * (wave + 8 * i) + (lane >> 3)) * g.lda) + 16 * c8;

  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  // load i (0 .. WI + XI - 1) of stage kt into buffer buf: weights first
  auto issue_one = [&](int i, int kt, int buf) {
    const uint32_t base = lds0 + buf * SPL;
    if (i < WI) {
      const int sw = WROW * kt;
      load_lds16(rw, base + 1024 * (wave + 8 * i), (KF || sw + 16 * cw < Kb) ? vw[i] : kOutOfRange, sw);
    } else {
      const int sx = (XP ? 64 : 128) * kt;
      load_lds16(rx, base + WPL + 1024 * (wave + 8 * (i - WI)), (KF || sx + 16 * cx < Kx) ? vx[i - WI] : kOutOfRange,
                 sx);
    }
  };
  constexpr int NL = WI + XI;

  // ---- fragments.  Step s (0..3) of a stage covers, for lane group lg,
  // the codes of packed chunk 2 (s / 2) + lg, half s % 2 (16 codes), which
  // is int8 chunk 4 (s / 2) + 2 lg + s % 2.  Weight lanes read the whole
  // packed chunk (both halves) once per pair of steps.  The 32-row blocks of
  // a wave are 2048 (packed) or 4096 (int8) bytes apart with equal swizzle.
  int fa[W8 ? 4 : 2], fb[XP ? 2 : 4];
  {
    const int ra = wm * WM + l32, rb = wn * WN + l32;
    if constexpr (W8) {
#pragma unroll
      for (int s = 0; s < 4; ++s) fa[s] = ra * 128 + 16 * swz(4 * (s >> 1) + 2 * lg + (s & 1), ra);
    } else {
#pragma unroll
      for (int p = 0; p < 2; ++p) fa[p] = ra * 64 + 16 * ((2 * p + lg) ^ psw(ra));
    }
    if constexpr (XP) {
#pragma unroll
      for (int p = 0; p < 2; ++p) fb[p] = WPL + rb * 64 + 16 * ((2 * p + lg) ^ psw(rb));
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) fb[s] = WPL + rb * 128 + 16 * swz(4 * (s >> 1) + 2 * lg + (s & 1), rb);
    }
  }
  constexpr int XF = XP ? 2048 : 4096;
  constexpr int WF = W8 ? 4096 : 2048;  // bytes between a wave's 32-row weight blocks

  i32x16 acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int b = 0; b < FN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0;

  // Multiply the stage in buffer buf.  The direct loads of stage kn (if
  // kn >= 0) into buffer nb are spread over the four k-steps, issued between
  // MFMAs: a wave that issues a whole stage's loads at once stalls on the
  // memory pipeline while its SIMD's MFMA unit idles.
  auto compute = [&](int buf, int kn, int nb) {
    const uint8_t* s0 = smem + buf * SPL;
    uint4 pa[2][FM];
    uint4 pb[2][FN];  // packed activation chunks (XP)
    i32x4 xb[2][FN];  // int8 activation fragments of steps s and s + 1
    i32x4 wb[2][FM];  // int8 weight fragments of steps s and s + 1 (W8)
#pragma unroll
    for (int f = 0; f < FM; ++f) {
      if constexpr (W8)
        wb[0][f] = *reinterpret_cast<const i32x4*>(s0 + fa[0] + WF * f);
      else
        pa[0][f] = *reinterpret_cast<const uint4*>(s0 + fa[0] + WF * f);
    }
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      if constexpr (XP)
        pb[0][f] = *reinterpret_cast<const uint4*>(s0 + fb[0] + XF * f);
      else
        xb[0][f] = *reinterpret_cast<const i32x4*>(s0 + fb[0] + XF * f);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int p = s >> 1, h = s & 1;
      if (s == 0 && !W8) {
#pragma unroll
        for (int f = 0; f < FM; ++f) pa[1][f] = *reinterpret_cast<const uint4*>(s0 + fa[1] + WF * f);
        if constexpr (XP) {
#pragma unroll
          for (int f = 0; f < FN; ++f) pb[1][f] = *reinterpret_cast<const uint4*>(s0 + fb[1] + XF * f);
        }
      }
      if constexpr (!XP) {
        if (s + 1 < 4) {
#pragma unroll
          for (int f = 0; f < FN; ++f)
            xb[(s + 1) & 1][f] = *reinterpret_cast<const i32x4*>(s0 + fb[s + 1] + XF * f);
        }
      }
      if constexpr (W8) {
        if (s + 1 < 4) {
#pragma unroll
          for (int f = 0; f < FM; ++f)
            wb[(s + 1) & 1][f] = *reinterpret_cast<const i32x4*>(s0 + fa[s + 1] + WF * f);
        }
      }
      i32x4 av[FM], bv[FN];
#pragma unroll
      for (int f = 0; f < FM; ++f) {
        if constexpr (W8)
          av[f] = wb[s & 1][f];
        else
          av[f] = h ? unpack16(pa[p][f].z, pa[p][f].w) : unpack16(pa[p][f].x, pa[p][f].y);
      }
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        if constexpr (XP)
          bv[f] = h ? unpack16(pb[p][f].z, pb[p][f].w) : unpack16(pb[p][f].x, pb[p][f].y);
        else
          bv[f] = xb[s & 1][f];
      }
#pragma unroll
      for (int a = 0; a < FM; ++a) {
#pragma unroll
        for (int b = 0; b < FN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[a], bv[b], acc[a][b], 0, 0, 0);
        if (a == 0 && kn >= 0) {
#pragma unroll
          for (int i = NL * s / 4; i < NL * (s + 1) / 4; ++i) issue_one(i, kn, nb);
        }
      }
    }
  };

  // ---- main loop: stage kt (128 k) sits in buffer kt % NST.  Each wave
  // waits for its own loads of stage kt (those of the later stages may stay
  // in flight); the barrier then publishes stage kt to all waves and frees the
  // buffer of stage kt - 1, which receives stage kt + AHEAD.
  const int KT = (Kb + WROW - 1) / WROW;
#pragma unroll
  for (int j = 0; j < AHEAD; ++j) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      if (j < KT) issue_one(i, j, j);
    }
  }
  int buf = 0;
  for (int kt = 0; kt < KT; ++kt) {
    if (AHEAD >= 2 && kt + AHEAD - 1 < KT)
      wait_vmcnt<(AHEAD - 1) * NL>();
    else
      wait_vmcnt<0>();
    stage_barrier();
    compute(buf, kt + AHEAD < KT ? kt + AHEAD : -1, buf == 0 ? NST - 1 : buf - 1);
    buf = buf == NST - 1 ? 0 : buf + 1;
  }

  // ---- epilogue ----
  // 32x32 result layout: lane l, element e -> row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32;
  // here row = channel, column = token.  chan(a, e4): first of the 4 channels of group e4.
  // the weights carry 16 x code, and so do packed activations once expanded:
  // acc = 16 (int8 activations) or 256 (packed) x the code product
  constexpr int SH = W8 ? 0 : (XP ? 8 : 4);
  auto chan = [&](int a, int e4) { return ch0 + wm * WM + 32 * a + 8 * e4 + 4 * lg; };
  auto tok = [&](int b) { return tk0 + wn * WN + 32 * b + l32; };
  // the 4 int32 sums v of block (a, b), group e4, to dst (M x N), shifted
  // right by sh (exact: the sums are multiples of 2^sh); add: on top of what
  // the same lane stored there before (8-bit chunks)
  auto store_i32 = [&](int32_t* dst, int a, int b, int e4, i32x4 v, int sh, bool add) {
    const int t = tok(b), c = chan(a, e4);
    if (t >= g.M) return;
    int32_t* op = dst + (size_t)t * g.N + c;
    v = v >> sh;
    if (c + 3 < g.N && (g.N & 3) == 0) {
      if (add) v += *reinterpret_cast<const i32x4*>(op);
      *reinterpret_cast<i32x4*>(op) = v;
    } else {
      for (int q = 0; q < 4; ++q)
        if (c + q < g.N) op[q] = add ? op[q] + v[q] : v[q];
    }
  };
  auto quad = [](const i32x16& x, int e4) { return i32x4{x[4 * e4], x[4 * e4 + 1], x[4 * e4 + 2], x[4 * e4 + 3]}; };
  // the main loop's exact sums (EPI_ACC, or the test hook of the other epilogues)
  auto export_acc = [&]() {
#pragma unroll
    for (int a = 0; a < FM; ++a)
#pragma unroll
      for (int b = 0; b < FN; ++b)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) store_i32(g.acc, a, b, e4, quad(acc[a][b], e4), SH, false);
  };
  if constexpr (EPI == EPI_ACC) {
    export_acc();
  } else {
    if constexpr (DBG) export_acc();
    auto load4 = [&](const float* p, int c) -> float4 {  // p[c..c+3], clamped at the channel tail
      if (c + 3 < g.N) return *reinterpret_cast<const float4*>(p + c);
      return float4{p[min(c, g.N - 1)], p[min(c + 1, g.N - 1)], p[min(c + 2, g.N - 1)], p[min(c + 3, g.N - 1)]};
    };
    f32x16 y[FM][FN];
    // bf16 Y is staged per wave in LDS (WN token rows of WM channels, 128-byte
    // rows: chunk j of row r at slot j ^ ((r >> 1) & 7), and rows with bit 4
    // set swap the 8-byte halves of each chunk, so the 32 rows a store
    // instruction touches land on distinct banks) and written as whole
    // 128-byte row pieces; fp32 Y is stored directly.
    // Dequantisation: the int32 sums carry the factor 2^SH, folded exactly
    // into s_x; acc is converted in place to the fp32 tile y (declared above).
    // The low-rank operands of the first TQ 16-t steps are loaded with the
    // scales, before the dequantisation, so the epilogue pays one L2 round
    // trip for both instead of one per step.
    constexpr int TQ = 2;
    const bf16_t* lp[FM];
    const bf16_t* tp[FN];
    uint4 lav[TQ][FM], lbv[TQ][FN];
    const bool lr_on = EPI == EPI_LINEAR && g.r_pad > 0;
    if (lr_on) {
#pragma unroll
      for (int a = 0; a < FM; ++a)
        lp[a] = g.L2t + (size_t)min(ch0 + wm * WM + 32 * a + l32, g.N - 1) * g.r_pad + 8 * lg;
      const int toff = group_of(g.groups, ch0) * g.r_pad;  // this tile's layer
#pragma unroll
      for (int b = 0; b < FN; ++b) tp[b] = g.T + (size_t)min(tok(b), g.M - 1) * g.ldt + toff + 8 * lg;
#pragma unroll
      for (int q = 0; q < TQ; ++q) {
        const int t0 = min(16 * q, g.r_pad - 16);  // r_pad >= 32: in range
#pragma unroll
        for (int a = 0; a < FM; ++a) lav[q][a] = *reinterpret_cast<const uint4*>(lp[a] + t0);
#pragma unroll
        for (int b = 0; b < FN; ++b) lbv[q][b] = *reinterpret_cast<const uint4*>(tp[b] + t0);
      }
    }
    {
      float4 swv[FM][4];
      float sxv[FN];
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) swv[a][e4] = load4(g.sw, chan(a, e4));
#pragma unroll
      for (int b = 0; b < FN; ++b) sxv[b] = g.sx[min(tok(b), g.M - 1)] * (1.0f / (1 << SH));
      // asymmetric two-subspace layer: per token z + 2^(N-1) s_x of each
      // subspace, per channel its s_w and weight code sum (an empty subspace
      // contributes zeros)
      const bool zp_on = EPI == EPI_MP && (g.zx != nullptr || g.zx2 != nullptr);
      float zzl[FN], zzh[FN];
      float4 swh[FM][4];
      int4 csl[FM][4], csh[FM][4];
      if constexpr (EPI == EPI_MP) {
        if (zp_on) {
          auto ld4i = [&](const int32_t* p, int c) -> int4 {
            if (c + 3 < g.N) return *reinterpret_cast<const int4*>(p + c);
            return int4{p[min(c, g.N - 1)], p[min(c + 1, g.N - 1)], p[min(c + 2, g.N - 1)], p[min(c + 3, g.N - 1)]};
          };
          const bool lo = g.zx && g.Kb > 0, hi = g.zx2 && g.Kb2 > 0;
#pragma unroll
          for (int b = 0; b < FN; ++b) {
            const int t = min(tok(b), g.M - 1);
            zzl[b] = lo ? g.zx[t] + 8.0f * g.sx[t] : 0.0f;
            zzh[b] = hi ? g.zx2[t] + 128.0f * g.sx2[t] : 0.0f;
          }
#pragma unroll
          for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
              const int c = chan(a, e4);
              csl[a][e4] = lo ? ld4i(g.csw, c) : int4{0, 0, 0, 0};
              csh[a][e4] = hi ? ld4i(g.csw2, c) : int4{0, 0, 0, 0};
              swh[a][e4] = hi ? load4(g.sw2, c) : float4{0.f, 0.f, 0.f, 0.f};
            }
        }
      }
      if (EPI == EPI_MP && g.Kb == 0) {  // no 4-bit subspace (its scales are never written)
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) swv[a][e4] = float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < FN; ++b) sxv[b] = 0.0f;
      }
#pragma unroll
      for (int a = 0; a < FM; ++a)
#pragma unroll
        for (int b = 0; b < FN; ++b)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            y[a][b][4 * e4 + 0] = (float)acc[a][b][4 * e4 + 0] * (swv[a][e4].x * sxv[b]);
            y[a][b][4 * e4 + 1] = (float)acc[a][b][4 * e4 + 1] * (swv[a][e4].y * sxv[b]);
            y[a][b][4 * e4 + 2] = (float)acc[a][b][4 * e4 + 2] * (swv[a][e4].z * sxv[b]);
            y[a][b][4 * e4 + 3] = (float)acc[a][b][4 * e4 + 3] * (swv[a][e4].w * sxv[b]);
          }
      if constexpr (EPI == EPI_MP) {
        // asymmetric activations: the codes are u - 8 (4-bit subspace) and
        // u - 128 (8-bit subspace), so each subspace adds its zero-point
        // term (z + 2^(N-1) s_x) s_w colsum(C_w) (CoQuant Eq. 1 with a
        // zero-point).  Both are added here, before the 8-bit product's
        // registers are live; their operands were loaded with the scales.
        if (zp_on) {
#pragma unroll
          for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
              const float w0 = swv[a][e4].x * (float)csl[a][e4].x, w1 = swv[a][e4].y * (float)csl[a][e4].y;
              const float w2 = swv[a][e4].z * (float)csl[a][e4].z, w3 = swv[a][e4].w * (float)csl[a][e4].w;
              const float h0 = swh[a][e4].x * (float)csh[a][e4].x, h1 = swh[a][e4].y * (float)csh[a][e4].y;
              const float h2 = swh[a][e4].z * (float)csh[a][e4].z, h3 = swh[a][e4].w * (float)csh[a][e4].w;
#pragma unroll
              for (int b = 0; b < FN; ++b) {
                y[a][b][4 * e4 + 0] += zzl[b] * w0 + zzh[b] * h0;
                y[a][b][4 * e4 + 1] += zzl[b] * w1 + zzh[b] * h1;
                y[a][b][4 * e4 + 2] += zzl[b] * w2 + zzh[b] * h2;
                y[a][b][4 * e4 + 3] += zzl[b] * w3 + zzh[b] * h3;
              }
            }
        }
      }
    }
    if (lr_on) {
      // D[channel][token] += sum_t L2^T[channel][t] T[token][t] on the bf16
      // MFMA, 16 t per step (r_pad is a multiple of 32); the L2 fragment of
      // each channel block and the T fragment of each token block are loaded
      // once per step, TQ steps at a time
      for (int t00 = 0; t00 < g.r_pad; t00 += 16 * TQ) {
        if (t00 > 0) {
#pragma unroll
          for (int q = 0; q < TQ; ++q) {
#pragma unroll
            for (int a = 0; a < FM; ++a) lav[q][a] = *reinterpret_cast<const uint4*>(lp[a] + t00 + 16 * q);
#pragma unroll
            for (int b = 0; b < FN; ++b) lbv[q][b] = *reinterpret_cast<const uint4*>(tp[b] + t00 + 16 * q);
          }
        }
#pragma unroll
        for (int q = 0; q < TQ; ++q)
#pragma unroll
          for (int a = 0; a < FM; ++a)
#pragma unroll
            for (int b = 0; b < FN; ++b)
              y[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(lav[q][a]), as_bf16x8(lbv[q][b]), y[a][b],
                                                                0, 0, 0);
      }
    }
    // Second stage of the quantised low-rank branch, (s_x s_t) s_v (Q(T) Q(V))
    // (TwinQuant notes, section 04.C: both stages on integer codes, merged in
    // the residual GEMM's epilogue), added block by block in the store loop
    // below: each 32 x 32 block takes its exact int32 product over the r_pad
    // ranks on v_mfma_i32_32x32x32_i8 and adds it to y in fp32 just before
    // the block is stored, so the fp32 tile shrinks as the int32 blocks come.
    // V rows are the channels' nibble-packed codes (r_pad / 2 bytes; step q,
    // lane group lg: bytes 16 q + 8 lg, 16 codes expanded by unpack16, so the
    // sum carries a factor 16, taken out exactly with the scale), T rows the
    // tokens' int8 codes (r_pad bytes; bytes 32 q + 16 lg: the same 16 ranks
    // in the same order).
    const uint8_t* vq[FM];
    const uint8_t* tq8[FN];
    float stv[FN];
    if constexpr (EPI == EPI_QLR) {
#pragma unroll
      for (int a = 0; a < FM; ++a)
        vq[a] = g.Vq + (size_t)min(ch0 + wm * WM + 32 * a + l32, g.N - 1) * (g.r_pad / 2) + 8 * lg;
#pragma unroll
      for (int b = 0; b < FN; ++b) {
        const int t = min(tok(b), g.M - 1);
        tq8[b] = g.Tq + (size_t)t * g.r_pad + 16 * lg;
        stv[b] = g.sx[t] * g.st[t] * (1.0f / 16);
      }
    }
    auto qlr_add = [&](int a, int b, const uint2& v0, const float4 (&svv)[4]) {
      i32x16 acc2;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc2[i] = 0;
      acc2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(unpack16(v0.x, v0.y), *reinterpret_cast<const i32x4*>(tq8[b]),
                                                   acc2, 0, 0, 0);
      for (int q = 1; q < (g.r_pad >> 5); ++q) {
        const uint2 va = *reinterpret_cast<const uint2*>(vq[a] + 16 * q);
        const i32x4 tb = *reinterpret_cast<const i32x4*>(tq8[b] + 32 * q);
        acc2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(unpack16(va.x, va.y), tb, acc2, 0, 0, 0);
      }
      if (DBG) {  // test hook: C_t C_v^T exactly (the expanded V carries 16 x code)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) store_i32(g.acc2, a, b, e4, quad(acc2, e4), 4, false);
      }
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        y[a][b][4 * e4 + 0] += (float)acc2[4 * e4 + 0] * (svv[e4].x * stv[b]);
        y[a][b][4 * e4 + 1] += (float)acc2[4 * e4 + 1] * (svv[e4].y * stv[b]);
        y[a][b][4 * e4 + 2] += (float)acc2[4 * e4 + 2] * (svv[e4].z * stv[b]);
        y[a][b][4 * e4 + 3] += (float)acc2[4 * e4 + 3] * (svv[e4].w * stv[b]);
      }
    };
    if constexpr (EPI == EPI_MP) {
      // Two-subspace layer: add the 8-bit subspace, s_x2 s_w2 (Q8(X_h) Q8(W_h))
      // (CoQuant notes, "CoQuant: Joint Weight-Activation Subspace Projection
      // for Mixed-Precision LLMs", Eq. 9, the high-precision term).  Its
      // int8 code rows (Kb2 bytes) are staged like the activation plane, one
      // 128-k chunk of both operands per pass into the now idle stage
      // buffers, and each 32 x 32 block takes its exact int32 product over
      // the chunk (no factor: both operands are plain codes); chunks beyond
      // the first (Kb2 > 128) add in fp32.
      const int K2 = g.Kb2;
      if (K2 > 0) {
        constexpr int PW = BM / 64, PX = BN / 64;  // 1 KB pieces per wave per plane
        const i32x4 rwh = buffer_rsrc(g.B2 + (size_t)ch0 * g.ldb2, (uint32_t)(min(BM, g.N - ch0) * g.ldb2));
        const i32x4 rxh = buffer_rsrc(g.A2 + (size_t)tk0 * g.lda2, (uint32_t)(min(BN, g.M - tk0) * g.lda2));
        const int rw8 = 8 * wave + (lane >> 3);  // row of piece wave (+ 64 i) for this lane
        float sx2[FN];
#pragma unroll
        for (int b = 0; b < FN; ++b) sx2[b] = g.sx2[min(tok(b), g.M - 1)];
        float4 sw2[FM][4];
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int c = chan(a, e4);
            sw2[a][e4] = c + 3 < g.N ? *reinterpret_cast<const float4*>(g.sw2 + c)
                                     : float4{g.sw2[min(c, g.N - 1)], g.sw2[min(c + 1, g.N - 1)],
                                              g.sw2[min(c + 2, g.N - 1)], g.sw2[min(c + 3, g.N - 1)]};
          }
        for (int k0 = 0; k0 < K2; k0 += 128) {
          stage_barrier();  // every wave is done with the LDS of the main loop or the last chunk
          {
            const bool ok = k0 + 16 * c8 < K2;
#pragma unroll
            for (int i = 0; i < PW; ++i)
              load_lds16(rwh, lds0 + 1024 * (wave + 8 * i),
                         ok ? (int)((rw8 + 64 * i) * g.ldb2) + 16 * c8 : kOutOfRange, k0);
#pragma unroll
            for (int i = 0; i < PX; ++i)
              load_lds16(rxh, lds0 + BM * 128 + 1024 * (wave + 8 * i),
                         ok ? (int)((rw8 + 64 * i) * g.lda2) + 16 * c8 : kOutOfRange, k0);
          }
          wait_vmcnt<0>();
          stage_barrier();
#pragma unroll
          for (int a = 0; a < FM; ++a) {
#pragma unroll
            for (int b = 0; b < FN; ++b) {
              // fragments as in the main loop: step s of lane group lg takes
              // chunk 4 (s / 2) + 2 lg + s % 2 of the rows (plain int8 codes)
              i32x16 acc2;
#pragma unroll
              for (int i = 0; i < 16; ++i) acc2[i] = 0;
              // empty asm fences on acc2 keep the blocks' MFMA chains in
              // sequence (interleaved, their accumulators would not fit)
              asm volatile("" : "+v"(acc2));
#pragma unroll
              for (int st = 0; st < 4; ++st) {
                // steps 2 p and 2 p + 1 together cover the 64 k from k0 + 64 p
                // (interleaved chunks); chunks past K2 were fetched as zeros
                if (k0 + 64 * (st >> 1) < K2) {
                  // weight rows wm WM + 32 a + l32 have the swizzle of token rows wn WN + l32
                  const i32x4 av = *reinterpret_cast<const i32x4*>(smem + (fb[st] - WPL) +
                                                                   (wm * WM - wn * WN + 32 * a) * 128);
                  const i32x4 bv = *reinterpret_cast<const i32x4*>(smem + BM * 128 + (fb[st] - WPL) + 4096 * b);
                  acc2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, acc2, 0, 0, 0);
                }
              }
              if (DBG) {  // test hook: the 8-bit segment's exact sums, chunks added in int32
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) store_i32(g.acc2, a, b, e4, quad(acc2, e4), 0, k0 > 0);
              }
#pragma unroll
              for (int e4 = 0; e4 < 4; ++e4) {
                y[a][b][4 * e4 + 0] += (float)acc2[4 * e4 + 0] * (sw2[a][e4].x * sx2[b]);
                y[a][b][4 * e4 + 1] += (float)acc2[4 * e4 + 1] * (sw2[a][e4].y * sx2[b]);
                y[a][b][4 * e4 + 2] += (float)acc2[4 * e4 + 2] * (sw2[a][e4].z * sx2[b]);
                y[a][b][4 * e4 + 3] += (float)acc2[4 * e4 + 3] * (sw2[a][e4].w * sx2[b]);
              }
              asm volatile("" : "+v"(acc2));
            }
          }
        }
      }
    }
    if (g.y_bf16) __syncthreads();  // every wave is done with the stage buffers
    uint8_t* sYw = smem + wave * (WN * WM * 2);
    auto ychunk = [&](int row, int j) -> int { return row * (WM * 2) + 16 * (j ^ ((row >> 1) & 7)); };
    auto yslot = [&](int row, int j, int half) -> int { return ychunk(row, j) + 8 * (half ^ ((row >> 4) & 1)); };
    // asymmetric activations of the rank-augmented layer (codes u - 8): the
    // zero-point term (z + 8 s_x) s_w colsum(C_w) (CoQuant Eq. 1 with a
    // zero-point), added block by block like the quantised branch
    const bool zp_lin = EPI == EPI_LINEAR && g.zx != nullptr;
    float zzv[FN];
    if (EPI == EPI_LINEAR && zp_lin) {
#pragma unroll
      for (int b = 0; b < FN; ++b) {
        const int t = min(tok(b), g.M - 1);
        zzv[b] = g.zx[t] + 8.0f * g.sx[t];
      }
    }
#pragma unroll
    for (int a = 0; a < FM; ++a) {
      uint2 v0;
      float4 svv[4];
      if constexpr (EPI == EPI_QLR) {
        v0 = *reinterpret_cast<const uint2*>(vq[a]);
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) svv[e4] = load4(g.sv, chan(a, e4));
      }
      if (EPI == EPI_LINEAR && zp_lin) {  // svv: s_w colsum of the block's channels
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int c = chan(a, e4);
          const float4 s4 = load4(g.sw, c);
          const int4 c4 = c + 3 < g.N ? *reinterpret_cast<const int4*>(g.csw + c)
                                      : int4{g.csw[min(c, g.N - 1)], g.csw[min(c + 1, g.N - 1)],
                                             g.csw[min(c + 2, g.N - 1)], g.csw[min(c + 3, g.N - 1)]};
          svv[e4] = float4{s4.x * (float)c4.x, s4.y * (float)c4.y, s4.z * (float)c4.z, s4.w * (float)c4.w};
        }
      }
#pragma unroll
      for (int b = 0; b < FN; ++b) {
        if constexpr (EPI == EPI_QLR) qlr_add(a, b, v0, svv);
        if (EPI == EPI_LINEAR && zp_lin) {
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            y[a][b][4 * e4 + 0] += zzv[b] * svv[e4].x;
            y[a][b][4 * e4 + 1] += zzv[b] * svv[e4].y;
            y[a][b][4 * e4 + 2] += zzv[b] * svv[e4].z;
            y[a][b][4 * e4 + 3] += zzv[b] * svv[e4].w;
          }
        }
        if (g.y_bf16) {
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int row = 32 * b + l32;
            *reinterpret_cast<uint2*>(sYw + yslot(row, 4 * a + e4, lg)) =
                uint2{pack_bf16x2(y[a][b][4 * e4], y[a][b][4 * e4 + 1]),
                      pack_bf16x2(y[a][b][4 * e4 + 2], y[a][b][4 * e4 + 3])};
          }
        } else {
          const int t = tok(b);
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int c = chan(a, e4);
            if (t >= g.M) continue;
            float* yp = reinterpret_cast<float*>(g.Y) + (size_t)t * g.ldy + c;
            if (c + 3 < g.N && (g.ldy & 3) == 0) {
              *reinterpret_cast<float4*>(yp) =
                  float4{y[a][b][4 * e4], y[a][b][4 * e4 + 1], y[a][b][4 * e4 + 2], y[a][b][4 * e4 + 3]};
            } else {
              for (int q = 0; q < 4; ++q)
                if (c + q < g.N) yp[q] = y[a][b][4 * e4 + q];
            }
          }
        }
      }
    }
    if (g.y_bf16) {
      // 16 bytes per lane, 8 lanes per token row of WM channels; a wave reads
      // only its own staging area, so a wave-level LDS wait suffices
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
      const int jc = lane & 7, rsub = lane >> 3;
      const int c = ch0 + wm * WM + 8 * jc;
#pragma unroll 4
      for (int r0 = 0; r0 < WN; r0 += 8) {
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

// Compute units of the chip: one 256 x 256 tile each per wave.
constexpr long kTileCUs = 256;

template <int EPI, bool XP, bool W8, bool KF, bool DBG>
hipError_t launch_kf(const GemmArgs& g, hipStream_t st) {
  const long tt = (g.M + 255) / 256, big = tt * ((g.N + 255) / 256);
  // the two-subspace epilogue keeps a 64 x 64 fp32 tile per wave (256 x 128
  // tiles): with 64 x 128 it would not fit the registers beside the 8-bit product
  if constexpr (EPI != EPI_MP) {
    if (big >= 224) {
      // A last wave of 256 x 256 tiles that would fill at most half of the
      // compute units (rem tiles, whole channel panels): those channels run
      // as 256 x 128 tiles in a second launch, twice the blocks at half the
      // work each, instead of a half-empty wave of full tiles.
      const long rem = big % kTileCUs;
      if (big > kTileCUs && rem > 0 && 2 * rem <= kTileCUs && rem % tt == 0) {
        GemmArgs g1 = g, g2 = g;
        g1.c1 = (int)((g.N + 255) / 256 - rem / tt) * 256;  // whole panels before the last rem / tt
        g2.c0 = g1.c1;
        launch_kernel(k_gemm8<EPI, XP, 256, W8, KF, DBG>, dim3((unsigned)(big - rem)), dim3(512), 0, st, g1);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
        launch_kernel(k_gemm8<EPI, XP, 128, W8, KF, DBG>, dim3((unsigned)(2 * rem)), dim3(512), 0, st, g2);
        return hipGetLastError();
      }
      launch_kernel(k_gemm8<EPI, XP, 256, W8, KF, DBG>, dim3((unsigned)big), dim3(512), 0, st, g);
      return hipGetLastError();
    }
  }
  const long mid = (long)((g.M + 127) / 128) * ((g.N + 255) / 256);
  if constexpr ((EPI == EPI_LINEAR || EPI == EPI_ACC) && !W8) {
    // fewer 256 x 128 tiles than compute units (up to some hundreds of
    // tokens): 128 x 128 tiles, twice the blocks
    if (mid < 224) {
      const unsigned blocks = (unsigned)(((g.M + 127) / 128) * ((g.N + 127) / 128));
      launch_kernel(k_gemm8<EPI, XP, 128, W8, KF, DBG, 128>, dim3(blocks), dim3(512), 0, st, g);
      return hipGetLastError();
    }
  }
  launch_kernel(k_gemm8<EPI, XP, 128, W8, KF, DBG>, dim3((unsigned)mid), dim3(512), 0, st, g);
  return hipGetLastError();
}

template <int EPI, bool XP, bool W8 = false>
hipError_t launch_t(const GemmArgs& g, hipStream_t st) {
  // whole stages: WROW weight bytes per row per stage, and then also whole
  // activation stages (XROW = 2 WROW for int8 activations, WROW otherwise)
  const bool kf = g.Kb % (W8 ? 128 : 64) == 0;
  // the accumulator-export instance (test hook) when an export buffer is set
  if (EPI != EPI_ACC && g.acc)
    return kf ? launch_kf<EPI, XP, W8, true, true>(g, st) : launch_kf<EPI, XP, W8, false, true>(g, st);
  return kf ? launch_kf<EPI, XP, W8, true, false>(g, st) : launch_kf<EPI, XP, W8, false, false>(g, st);
}

}  // namespace

// Channels x tokens tiles of 256 x 256 (256 x 128 for small grids and the
// two-subspace layer); x_int8: activation codes as int8 in the order above
// (lda bytes per row), else nibble-packed like the weights; w_bits 8: int8
// weight codes and activation codes in natural k order (the integer check
// only).  Buffer offsets are 32-bit: a tile's rows of codes must span less
// than 2 GiB.
hipError_t launch_gemm8(const GemmArgs& g, Epilogue epi, bool x_int8, int w_bits, hipStream_t st) {
  if ((int64_t)256 * g.ldb >= (1ll << 31) || (int64_t)256 * g.lda >= (1ll << 31)) return hipErrorInvalidValue;
  if (w_bits == 8) return (epi == EPI_ACC && x_int8) ? launch_t<EPI_ACC, false, true>(g, st) : hipErrorInvalidValue;
  if (w_bits != 4) return hipErrorInvalidValue;
  if (epi == EPI_LINEAR && x_int8) return launch_t<EPI_LINEAR, false>(g, st);
  if (epi == EPI_LINEAR && !x_int8) return launch_t<EPI_LINEAR, true>(g, st);
  if (epi == EPI_ACC && !x_int8) return launch_t<EPI_ACC, true>(g, st);
  if (epi == EPI_ACC && x_int8) return launch_t<EPI_ACC, false>(g, st);
  if (epi == EPI_MP && x_int8) return launch_t<EPI_MP, false>(g, st);
  if (epi == EPI_QLR && x_int8) return launch_t<EPI_QLR, false>(g, st);
  return hipErrorInvalidValue;
}

// The int8 MFMA ceiling that bounds the tile GEMM: every wave of `blocks`
// blocks of 512 threads chains `iters` rounds of 8 independent
// v_mfma_i32_32x32x32_i8 on register operands (no memory traffic, no LDS, no
// barrier), then stores the sum of its accumulator lanes, one int per thread,
// so the products stay live.
__global__ __launch_bounds__(512) void k_mfma_ceiling(int iters, int32_t* out) {
  const int lane = threadIdx.x & 63;
  const i32x4 a = {lane, lane + 1, lane + 2, lane + 3}, b = {3 * lane, lane, 7, lane ^ 5};
  i32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[j][i] = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[j], 0, 0, 0);
  }
  int sum = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += acc[j][i];
  out[(size_t)blockIdx.x * 512 + threadIdx.x] = sum;
}

hipError_t launch_mfma_ceiling(int iters, int blocks, int32_t* out, hipStream_t st) {
  launch_kernel(k_mfma_ceiling, dim3((unsigned)blocks), dim3(512), 0, st, iters, out);
  return hipGetLastError();
}

}  // namespace tq
