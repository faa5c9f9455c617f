// Internal launcher interface between the C ABI (tq_api.hip) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "tq_device.h"

namespace tq {

enum Epilogue { EPI_ACC = 0, EPI_LINEAR = 1, EPI_MP = 2, EPI_QLR = 3 };

// Timing events for the next launch, set by the library's profiler.  A
// launcher that supports them (hipExtLaunchKernelGGL: timestamps taken by
// the dispatch itself, without the gap of stream-recorded events) takes them
// and marks them used; otherwise the profiler's stream events stand.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;
};
LaunchEvents& launch_events();

// Several launches under one name: the start event is taken by the first,
// the stop event by each in turn, so the record spans first start to last end.
template <typename K, typename... Args>
void launch_kernel(K kernel, dim3 grid, dim3 block, unsigned lds, hipStream_t st, Args... args) {
  LaunchEvents& ev = launch_events();
  if (ev.start && ev.stop) {
    hipExtLaunchKernelGGL(kernel, grid, block, lds, st, ev.used ? nullptr : ev.start, ev.stop, 0, args...);
    ev.used = true;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
  }
}

// LDS rows of the tile kernels are 128 bytes = 8 chunks of 16 bytes; chunk c
// of row r sits at position c ^ (r & 7) ^ ((r >> 3) & 1), which keeps the
// fragment reads of 8 or 16 consecutive rows on distinct banks.
__device__ __forceinline__ int swz(int c, int r) { return c ^ (r & 7) ^ ((r >> 3) & 1); }

// Tile order: consecutive blocks are dispatched round-robin over the 8 XCDs,
// each with its own L2, so the block index is first regrouped per XCD
// (when the tile count is a multiple of 8) and the tiles of one XCD are then
// walked in groups of GM tile-rows, keeping the tiles a group shares in that
// XCD's L2.
__device__ __forceinline__ void tile_of_block(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GM = 4;
  const int T = tiles_m * tiles_n;
  int b = bid;
  if ((T & 7) == 0) b = (bid & 7) * (T >> 3) + (bid >> 3);
  const int gsz = GM * tiles_n;
  const int first = (b / gsz) * GM;
  const int gm = min(tiles_m - first, GM);
  const int r = b % gsz;
  tm = first + r % gm;
  tn = r / gm;
}

// Layers that share one input (several weights stacked along the output
// channels, one activation quantisation and one T for all of them): group g
// holds channels [gstart[g], gstart[g + 1]), and its T columns start at
// g * r_pad in rows of ldt.  Every group but the last spans whole 256-channel
// tiles, so a tile or block never straddles two groups.
constexpr int kMaxGroups = 8;
struct Groups {
  int n;                      // number of groups (1: a single layer)
  int start[kMaxGroups + 1];  // first channel of each group; start[n] = all channels
};
__device__ __forceinline__ int group_of(const Groups& gr, int c) {
  int g = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroups; ++i) g += (i < gr.n && c >= gr.start[i]) ? 1 : 0;
  return g;
}

// Arguments of the integer GEMM kernels: C = A B^T over K-contiguous codes.
struct GemmArgs {
  const uint8_t* A;  // x codes, M rows
  const uint8_t* B;  // w codes, N rows
  int64_t lda, ldb;  // bytes per row
  int M, N, Kb;      // Kb: code bytes per row of the main segment
  // tile GEMM: the launch covers output channels [c0, c1) (c1 = 0: [c0, N));
  // indexing, bounds and strides stay those of the whole N channels
  int c0, c1;
  // second (8-bit) segment of the two-subspace layer
  const uint8_t* A2;
  const uint8_t* B2;
  int64_t lda2, ldb2;
  int Kb2;
  const float* sx;   // M scales
  const float* sw;   // N scales
  const float* sx2;  // second-segment scales
  const float* sw2;
  const bf16_t* T;    // M rows of ldt (bf16); a layer's r_pad columns from its group's offset
  const bf16_t* L2t;  // N x r_pad (bf16) or null
  int r_pad;          // per layer
  int ldt;            // T row length (r_pad for one layer)
  Groups groups;
  // small-n path: T comes as nchunk fp32 partials P[c][M][ldt], summed in
  // chunk order by the kernel, which also writes the bf16 sum to Tout (the
  // first block of each group, its columns)
  const float* P;
  int nchunk;
  bf16_t* Tout;
  void* Y;
  int64_t ldy;  // elements
  int y_bf16;
  // EPI_ACC output, M x N.  With the other epilogues, when not null, the
  // kernel also stores there the exact int32 sums of its main loop (the
  // residual product C_x C_w^T) before dequantising them: a test hook that
  // exports the accumulators of the very kernel that produces Y.
  int32_t* acc;
  // Test hook of the second integer product, M x N, when not null: the 8-bit
  // segment's sums (EPI_MP) or the quantised low-rank branch's second stage
  // C_t C_v^T (EPI_QLR).
  int32_t* acc2;
  // EPI_QLR, the quantised low-rank branch: second-stage weight codes
  // (N rows of r_pad / 2 nibble-packed bytes) and scales, first-stage codes
  // (M rows of r_pad int8 bytes in the int8 code order) and scales
  const uint8_t* Vq;
  const float* sv;
  const uint8_t* Tq;
  const float* st;
  // EPI_MP with asymmetric activations: per-token zero-points of the two
  // segments and the weight code sums per channel (null: symmetric)
  const float* zx;
  const float* zx2;
  const int32_t* csw;
  const int32_t* csw2;
};

hipError_t launch_pack_weight(const void* W, bool bf16, int d, int m, int bits, void* codes, float* sw,
                              hipStream_t st);
// The same for a dv x mv matrix (row stride ldw elements) zero-padded to d x m.
hipError_t launch_pack_weight_padded(const void* W, bool bf16, int d, int m, int ldw, int dv, int mv, int bits,
                                     void* codes, float* sw, hipStream_t st);
// L1^T (rows1 rows of d, rows r.. zero) to out1 and L2^T (m x r_pad) to out2, bf16.
hipError_t launch_pack_lowrank(const void* L1, const void* L2, bool bf16, int d, int m, int r, int r_pad, int rows1,
                               void* out1, void* out2, hipStream_t st);
hipError_t launch_quant_rows(const void* X, bool bf16, int n, int d, int dl, int bits_a, int bits_b, void* ca,
                             float* sa, void* cb, float* sb, hipStream_t st);
// Work split of the tq_linear prologue (quantisation + T = X L1).
struct ProloguePlan {
  int kc, nchunk, qs, nqg, ntb, nqb, counters, waves;
  bool quant_in_prologue;
  bool partial;     // T left as fp32 partials per k-chunk (small-n path)
  bool sum_to_p0;   // small-n path with more chunks than the GEMM sums: the fp32 sum left in chunk 0
  bool row_blocks;  // quantise one row per block (few tokens)
  bool fused;       // many tokens: one pass over X makes codes, s_x and T (16-row blocks)
};
// small: few tokens (T as k-chunk partials for the small-n GEMM, which can sum
// at most max_chunks of them in one pass).
ProloguePlan plan_prologue(int n, int d, int r_pad, bool small, int max_chunks);
// The producers of the one-launch few-token layer (tq_prologue.h, SmallFuse):
// d % 32 == 0, d <= 16384, r_pad a multiple of 32 (or 0).
ProloguePlan plan_prologue_fused(int n, int d, int r_pad, int max_chunks);
// Most k-chunk partials of T the small-n GEMM sums in one pass for M tokens.
int gemv_max_chunks(int M, int Kb, int r_pad);
hipError_t launch_prologue(const void* X, bool bf16, int n, int d, const void* L1t, int r_pad, const ProloguePlan& p,
                           void* xc, float* sx, float* P, void* Tout, unsigned* counters, hipStream_t st);
// The prologue of the asymmetric layer: per-token asymmetric codes (u - 8;
// int8 for the tile GEMM, nibble-packed for the small-n GEMM when p is a
// small plan), scales and zero-points (zx), and T (or its k-chunk partials)
// as above.
hipError_t launch_prologue_asym(const void* X, bool bf16, int n, int d, const void* L1t, int r_pad,
                                const ProloguePlan& p, void* xc, float* sx, float* zx, float* P, void* Tout,
                                unsigned* counters, hipStream_t st);
// The same with the 4-bit codes of columns [0, dl) as int8 in the order of the
// int8 tile GEMM (dl bytes per row); columns [dl, d) take bits_b bits.
hipError_t launch_quant_rows_i8(const void* X, bool bf16, int n, int d, int dl, int bits_b, void* ca, float* sa,
                                void* cb, float* sb, hipStream_t st);
// The same for the two-subspace layer at bits_a / bits_b = 4 / 8 or 3 / 6
// (3-bit codes stored like 4-bit ones, 6-bit like 8-bit).
hipError_t launch_quant_rows_i8_bits(const void* X, bool bf16, int n, int d, int dl, int bits_a, int bits_b, void* ca,
                                     float* sa, void* cb, float* sb, hipStream_t st);
// Per-token quantiser with one wave per row (falls back to a block per row for very long rows).
hipError_t launch_quant_rows_fast(const void* X, bool bf16, int n, int d, int dl, int bits_a, int bits_b, void* ca,
                                  float* sa, void* cb, float* sb, hipStream_t st);
// Tile GEMM with operands staged HBM -> LDS by direct loads (tq_gemm8.hip):
// x_int8: activation codes as int8 (lda bytes per row), else nibble-packed;
// w_bits: 4 (nibble-packed weights) or 8 (int8 weights, EPI_ACC only).
hipError_t launch_gemm8(const GemmArgs& g, Epilogue epi, bool x_int8, int w_bits, hipStream_t st);
// Small-n integer GEMM (M <= 32).
hipError_t launch_gemv(const GemmArgs& g, int bits, Epilogue epi, hipStream_t st);

// Workspace bytes of the hand-off words of the one-launch few-token path.
constexpr int kSyncBytes = 4096;

// Online block-Hadamard rotation of the two-subspace quantiser: the packed
// rotation holds the signs as bits (d / 8 bytes, padded to 16) and then, for
// each rotated coordinate, its output position (uint16).  d % 128 == 0,
// d <= kRhtMaxD.
constexpr int kRhtMaxD = 8192;
__host__ __device__ constexpr size_t rht_signs_bytes(int d) { return ((size_t)d / 8 + 15) & ~(size_t)15; }
__host__ __device__ constexpr size_t rht_bytes(int d) { return rht_signs_bytes(d) + (((size_t)d * 2 + 15) & ~(size_t)15); }
hipError_t launch_pack_rht(const float* signs, const int32_t* perm, int d, void* rot, hipStream_t st);
// X (n x d) rotated online and quantised: columns [0, dl) of X' at 4 bits as
// int8 in the tile GEMM's order (dl bytes per row), [dl, d) at 8 bits.
hipError_t launch_quant_rows_rht(const void* X, bool bf16, int n, int d, int dl, const void* rot, void* xl,
                                 float* sxl, void* xh, float* sxh, hipStream_t st);
// First stage of the quantised low-rank branch (tq_qlr.hip): the exact
// integer product of the activation codes (n x d: int8 in the tile GEMM's
// order, or nibble-packed when `packed`) with the packed codes of U^T (r_pad
// rows of d / 2 bytes), scaled per rank by s_u in fp32 and re-quantised per
// token at 4 bits: codes to ct (n rows of r_pad int8 bytes, int8 code order),
// scales to st.  d % 32 == 0, r_pad in {32, 64, 128, 256}.
hipError_t launch_qlr_stage1(const uint8_t* xc, int n, int d, const uint8_t* uc, const float* su, int r_pad,
                             uint8_t* ct, float* st, bool packed, hipStream_t stream);
// The quantiser and the first stage in one launch (d <= 4096, r_pad <= 128):
// X (n x d) -> s_x, activation codes (int8 order, or nibble-packed when
// `packed`), first-stage codes and s_t as above.
bool qlr_fused_ok(int d, int r_pad);
hipError_t launch_qlr_prologue(const void* X, bool bf16, int n, int d, const uint8_t* uc, const float* su, int r_pad,
                               uint8_t* xc, float* sx, uint8_t* ct, float* st, bool packed, hipStream_t stream);
// Per-token asymmetric quantiser of the two-subspace layer (tq_asym.hip):
// columns [0, dl) at 4 bits (u - 8 as int8 in the tile GEMM's order, dl bytes
// per row), [dl, d) at 8 bits (u - 128, natural order); per row and segment
// the scale and the zero-point.  d <= kAsymMaxD.
constexpr int kAsymMaxD = 16384;
hipError_t launch_quant_rows_asym(const void* X, bool bf16, int n, int d, int dl, void* xl, float* sl, float* zl,
                                  void* xh, float* sh, float* zh, hipStream_t st, bool packed = false);
// colsum[j] = sum over k of code row j (m rows of k codes, 4 or 8 bits).
hipError_t launch_weight_colsum(const void* codes, int bits, int m, int k, int32_t* colsum, hipStream_t st);


// Few-token layer (one or two tokens) in one launch (tq_decode.hip): the
// first nt blocks compute one fp32 partial of T = X L1 each (16 columns, one
// k-chunk); every other block owns gpb groups of 16 output channels; the
// partials cross blocks as tagged words.
constexpr int kDecodeMaxN = 2;
constexpr int kDecodeMaxD = 16384;
constexpr int kDecodeSteps = 2;  // 32-k steps per wave in a partial of T (a chunk: 512 k values)
struct DecodePlan {
  int gpb;         // 16-channel groups per channel block (1 .. 4)
  int nqg;         // 16-column groups of T
  int kcs;         // 32-k steps per chunk of T
  int nchunk;      // chunks of T
  int nt;          // blocks that compute a partial (nchunk x nqg)
  int ncons;       // channel blocks
  int blocks;      // grid: nt + ncons
  unsigned lds;    // dynamic LDS bytes
  unsigned lds_a;  // bytes of the LDS region reused across phases
};
struct DecodeArgs {
  const void* X;
  int n, d, m;
  const uint8_t* wc;
  const float* sw;
  const bf16_t* L1t;  // ldt rows of d (every layer's L1^T)
  const bf16_t* L2t;  // m x r_pad
  int r_pad;          // per layer (a power of two, or 0)
  int lrp;            // log2(r_pad)
  int ldt;            // columns of T over all layers
  Groups groups;
  int nt, nqg, kcs, nchunk;
  uint8_t* xc;     // n x d / 2 activation codes (written by the first channel block)
  float* sx;       // n scales (idem)
  void* P;         // nchunk x n x ldt tagged 64-bit words {partial of T, epoch}, layer-major
  bf16_t* Tout;    // n x ldt: T as bf16 (written by the first block of each layer)
  unsigned* sync;  // hand-off words (kSyncBytes)
  void* Y;
  int y_bf16;
  int32_t* acc;    // test hook: the exact int32 sums of the residual product (n x m)
  unsigned spin;   // polls before a wait gives up
  int silent;      // test hook: partials carry the previous call's tag, so every wait gives up
  int gpb, ncons, lds_a;  // set by launch_decode from the plan
};
bool decode_ok(int n, int d, int ldt);
DecodePlan plan_decode(int n, int d, int m, int r_pad, int ldt, bool x_bf16);
size_t decode_partials_bytes(const DecodePlan& p, int n, int ldt);
hipError_t launch_decode(const DecodeArgs& a, const DecodePlan& p, bool x_bf16, hipStream_t st);
// reads `bytes` (a multiple of 16) once with `blocks` blocks; out: one word per block
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, int blocks, hipStream_t st);
hipError_t launch_mfma_ceiling(int iters, int blocks, int32_t* out, hipStream_t st);

}  // namespace tq
