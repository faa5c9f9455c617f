// Device code shared by the prologue of tq_linear (tq_quant.hip) and the
// one-launch few-token layer (tq_gemm.hip): the block-wide per-token
// quantiser of one row and the products of one block of the first low-rank
// stage T = X L1 (TwinQuant notes, "TwinQuant: Learnable Subspace
// Decomposition for W4A4 LLM Quantization", section 02 quantization formula
// and section 04.C, the two-stage low-rank product).
#pragma once

#include "tq_kernels.h"

namespace tq {

// ---------------------------------------------------------------------------
// One row quantised at 4 bits by a whole block, each thread holding CHB
// chunks of 8 values (chunk tid + blockDim.x i) in registers, so X is read
// once and the row's arithmetic is spread over all the block's waves (the
// few-token case, where one wave per row would leave the GPU idle).  Every
// thread of the block must call it (it contains a barrier).
// ---------------------------------------------------------------------------
// CO: codes and scale stored at agent scope (written through to the device's
// point of coherence, past the XCDs' separate L2s), for readers in other
// blocks of the same launch.
template <typename T, int CHB, bool CO = false>
__device__ __forceinline__ void quant_row_block_reg(const T* __restrict__ x, int d, uint8_t* __restrict__ c,
                                                    float* __restrict__ s, float* red) {
  auto put = [](uint8_t* p, uint32_t v) {
    if (CO)
      __hip_atomic_store(reinterpret_cast<uint32_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *reinterpret_cast<uint32_t*>(p) = v;
  };
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, w = tid >> 6, nw = nthr >> 6;
  const int nch = d >> 3;
  Row8<T> r[CHB];
#pragma unroll
  for (int i = 0; i < CHB; ++i) {
    const int ch = tid + nthr * i;
    if (ch < nch) r[i].load(x + 8 * ch);
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < CHB; ++i) {
    if (tid + nthr * i < nch) {
      float v[8];
      r[i].get(v);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
    }
  }
  m = wave_max(m);
  if (lane == 0) red[w] = m;
  __syncthreads();
  m = 0.0f;
  for (int i = 0; i < nw; ++i) m = fmaxf(m, red[i]);
  const RowScale rs = row_scale<4>(m);
  if (tid == 0) {
    if (CO)
      __hip_atomic_store(s, rs.s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *s = rs.s;
  }
  if (__builtin_amdgcn_readfirstlane(rs.fast ? 1 : 0)) {
#pragma unroll
    for (int i = 0; i < CHB; ++i) {
      const int ch = tid + nthr * i;
      if (ch < nch) {
        float v[8];
        int q[8];
        r[i].get(v);
        quant8_fast<4>(v, rs, q);
        put(c + (size_t)ch * 4, pack_nibbles(q));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < CHB; ++i) {
      const int ch = tid + nthr * i;
      if (ch < nch) {
        float v[8];
        int q[8];
        r[i].get(v);
        quant8_exact<4>(v, rs.s, q);
        put(c + (size_t)ch * 4, pack_nibbles(q));
      }
    }
  }
}

// The same row quantised at 4 bits with a per-token zero-point (CoQuant
// notes, "CoQuant: Joint Weight-Activation Subspace Projection for
// Mixed-Precision LLMs", Eq. 1 with a zero-point): z = min, s = fl32(fl32(max
// - min) / 15), codes u - 8 nibble-packed (even k in the low nibble), with
// the block-wide min and max (exact in any order).  Codes, s and z stored at
// agent scope, for readers in other blocks of the same launch.
template <typename T, int CHB>
__device__ __forceinline__ void quant_row_block_asym(const T* __restrict__ x, int d, uint8_t* __restrict__ c,
                                                     float* __restrict__ s, float* __restrict__ z, float* red) {
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, w = tid >> 6, nw = nthr >> 6;
  const int nch = d >> 3;
  Row8<T> r[CHB];
#pragma unroll
  for (int i = 0; i < CHB; ++i) {
    const int ch = tid + nthr * i;
    if (ch < nch) r[i].load(x + 8 * ch);
  }
  float mx = -INFINITY, nm = -INFINITY;  // max and -min (threads without values keep -inf)
#pragma unroll
  for (int i = 0; i < CHB; ++i) {
    if (tid + nthr * i < nch) {
      float v[8];
      r[i].get(v);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        mx = fmaxf(mx, v[e]);
        nm = fmaxf(nm, -v[e]);
      }
    }
  }
  mx = wave_fmax(mx);
  nm = wave_fmax(nm);
  if (lane == 0) {
    red[w] = mx;
    red[nw + w] = nm;
  }
  __syncthreads();
  mx = -INFINITY;
  nm = -INFINITY;
  for (int i = 0; i < nw; ++i) {
    mx = fmaxf(mx, red[i]);
    nm = fmaxf(nm, red[nw + i]);
  }
  const AsymScale a = asym_scale<4>(-nm, mx);
  if (tid == 0) {
    __hip_atomic_store(s, a.s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(z, a.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int i = 0; i < CHB; ++i) {
    const int ch = tid + nthr * i;
    if (ch < nch) {
      float v[8];
      int q[8];
      r[i].get(v);
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = code_asym<4>(v[e] - a.z, a);
      __hip_atomic_store(reinterpret_cast<uint32_t*>(c + (size_t)ch * 4), pack_nibbles(q), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// Prologue of tq_linear: one launch, two kinds of blocks.
//  * blocks [0, nqb): 4-bit codes and s_x of WAVES rows, one per wave, or,
//    for few tokens (row_blocks), of one row per block (skipped, nqb = 0,
//    when the row does not fit in registers); X8: codes as int8 in the order
//    of the int8 tile GEMM (d bytes per row), else nibble-packed;
//  * blocks [nqb, nqb + ntb): the first low-rank stage T = X L1 on
//    v_mfma_f32_16x16x32_bf16.  Block (rt, c, qg) takes rows 16 rt..16 rt+15,
//    the k-range [c kc, (c+1) kc) and the QS 16-column slices of group qg;
//    its waves take the 32-k steps round-robin, U steps per wave in flight,
//    and their partials are summed through LDS in wave order.
//    - partial mode (few tokens): the block writes its fp32 partial to
//      P[c]; the small-n GEMM sums the chunks;
//    - one k-chunk: the block writes T directly;
//    - otherwise the block writes its fp32 partial to P and the last block of
//      the (rt, qg) group to finish (agent-scope counter) sums the partials
//      in chunk order into T and resets the counter.
// MFMA operand layout: lane l supplies row (or T column) l % 16 and the 8
// consecutive k at 32 step + 8 (l / 16), for X and L1^T alike.
// ---------------------------------------------------------------------------
struct PrologueArgs {
  const void* X;
  int n, d;
  const bf16_t* L1t;
  int r_pad, kc, nchunk, qs, nqg, nqb, partial, row_blocks;
  int sum_to_p0;  // the last block also leaves the fp32 sum of the chunks in chunk 0 of P
  uint8_t* xc;
  float* sx;
  float* P;
  bf16_t* T;
  unsigned* counters;
};


// The one-launch few-token layer (tq_gemm.hip): the producers' work (pa in
// partial mode; zx: per-token zero-points of asymmetric activations, or null: pa.nqb = n row blocks, then the T blocks with QS = 2,
// pa.nqg = r_pad / 32), nprod = their number, the hand-off words, the polls
// before a wait gives up, and a test hook (silent: the producers never
// signal, so every wait gives up).
struct SmallFuse {
  PrologueArgs pa;
  float* zx;
  int nprod;
  unsigned* sync;
  unsigned spin;
  int silent;
};
hipError_t launch_gemv_fused(const GemmArgs& g, const SmallFuse& f, bool x_bf16, hipStream_t st);
// Whether that launch's grid (nprod producers, N / 16 GEMM blocks) is at most
// a quarter larger than what is resident at once on the current device, for
// X of that type; dbg: the accumulator-export instance.
bool gemv_fused_fits(int M, int Kb, int N, int nprod, bool x_bf16, bool dbg);

// The products of T block tb = (rt, c, qg) -- rows 16 rt .. 16 rt + 15, the
// k-chunk c, the QS 16-column slices of group qg -- left per wave in
// sP[wave][row][column] (WAVES x 16 x (16 QS + 1) fp32 of LDS); the caller
// synchronises the block before reading them.
struct TBlock {
  int rt, c, qg;
};
template <typename T, int QS, int WAVES, int U>
__device__ __forceinline__ TBlock t_block_products(const PrologueArgs& a, int tb, float (*sP)[16][16 * QS + 1]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int per_rt = a.nchunk * a.nqg;
  const int rt = tb / per_rt, c = (tb % per_rt) / a.nqg, qg = tb % a.nqg;
  const int d = a.d, n = a.n;
  // k-chunk c covers the 32-k steps [c * kc / 32, (c + 1) * kc / 32); wave w takes every WAVES-th
  const int s0 = c * (a.kc >> 5), s1 = min(d >> 5, s0 + (a.kc >> 5));
  const T* xr = (const T*)a.X + (size_t)min(16 * rt + lr, n - 1) * d;
  const bf16_t* lp = a.L1t + (size_t)(16 * qg * QS + lr) * d;

  f32x4 acc[QS];
#pragma unroll
  for (int q = 0; q < QS; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int sb = s0 + w; sb < s1; sb += WAVES * U) {  // batches of U steps, all loads in flight
    uint4 xa[U];
    uint4 lb[U][QS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = sb + WAVES * u;
      const int k = 32 * s + 8 * lg;
      if (s < s1) {
        float v[8];
        Load8<T>::load(xr + k, v, xa[u]);
#pragma unroll
        for (int q = 0; q < QS; ++q) lb[u][q] = *reinterpret_cast<const uint4*>(lp + (size_t)16 * q * d + k);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (sb + WAVES * u < s1) {
#pragma unroll
        for (int q = 0; q < QS; ++q)
          acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[u]), as_bf16x8(lb[u][q]), acc[q], 0, 0, 0);
      }
    }
  }
  // 16x16 result layout: lane l, element i -> row 4 (l / 16) + i, column l % 16.
#pragma unroll
  for (int q = 0; q < QS; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) sP[w][4 * lg + i][16 * q + lr] = acc[q][i];
  return TBlock{rt, c, qg};
}

}  // namespace tq
