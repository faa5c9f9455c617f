// Quantisation-side kernels of the rank-augmented W4A4 layer (gfx950):
// weight packing, low-rank factor layout, per-token activation quantisation
// and the two prologues of tq_linear that quantise X and compute the first
// low-rank stage T = X L1 on bf16 MFMA in the same pass over X.
//
// Quantiser: TwinQuant notes ("TwinQuant: Learnable Subspace Decomposition
// for W4A4 LLM Quantization") section 02 quantization formula, CoQuant
// ("CoQuant: Joint Weight-Activation Subspace Projection for Mixed-Precision
// LLMs") Eq. 1 with zero-point 0; per-token activations and per-channel
// weights (CoQuant experimental protocol).  Low-rank stage: TwinQuant notes
// section 02.A (X U V) and section 04.C (two-stage low-rank product).

#include "tq_kernels.h"

namespace tq {

// ---------------------------------------------------------------------------
// Per-output-channel weight packing.  Block: 64 output channels, 256 threads.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float ld_f32(const T* p);
template <>
__device__ __forceinline__ float ld_f32<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ld_f32<bf16_t>(const bf16_t* p) { return bf16_to_f32(*p); }

template <typename T, int BITS>
__global__ __launch_bounds__(256) void k_pack_weight(const T* __restrict__ W, int d, int m,
                                                     uint8_t* __restrict__ codes, float* __restrict__ sw) {
  __shared__ float red[4][64];
  __shared__ float tile[64][65];
  __shared__ float s_s[64], s_r[64];
  __shared__ int s_f[64];
  const int tid = threadIdx.x, tx = tid & 63, ty = tid >> 6;
  const int j0 = blockIdx.x * 64;
  const int j = min(j0 + tx, m - 1);
  float am = 0.0f;
  for (int k = ty; k < d; k += 4) am = fmaxf(am, fabsf(ld_f32<T>(W + (size_t)k * m + j)));
  red[ty][tx] = am;
  __syncthreads();
  if (ty == 0) {
    am = fmaxf(fmaxf(red[0][tx], red[1][tx]), fmaxf(red[2][tx], red[3][tx]));
    const RowScale rs = row_scale<BITS>(am);
    s_s[tx] = rs.s;
    s_r[tx] = rs.rcp;
    s_f[tx] = rs.fast ? 1 : 0;
    if (j0 + tx < m) sw[j0 + tx] = rs.s;
  }
  __syncthreads();
  const size_t row_bytes = (size_t)d * BITS / 8;
  const int c = tid >> 2, kg = tid & 3;
  const RowScale rs = {s_s[c], s_r[c], s_f[c] != 0};
  for (int k0 = 0; k0 < d; k0 += 64) {
    for (int kk = ty; kk < 64; kk += 4)
      tile[kk][tx] = (k0 + kk < d) ? ld_f32<T>(W + (size_t)(k0 + kk) * m + j) : 0.0f;
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kb = 16 * kg + 8 * h;
      if (j0 + c < m && k0 + kb < d) {
        float v[8];
        int q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = tile[kb + i][c];
        quant8<BITS>(v, rs, q);
        uint8_t* dst = codes + (size_t)(j0 + c) * row_bytes + (size_t)(k0 + kb) * BITS / 8;
        if (BITS == 4)
          *reinterpret_cast<uint32_t*>(dst) = pack_nibbles(q);
        else
          *reinterpret_cast<uint2*>(dst) = pack_bytes(q);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Low-rank factors -> bf16 L1^T (r_pad x d) followed by L2^T (m x r_pad).
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ bf16_t to_bf16(T v);
template <>
__device__ __forceinline__ bf16_t to_bf16<float>(float v) { return (bf16_t)f32_to_bf16_bits(v); }
template <>
__device__ __forceinline__ bf16_t to_bf16<bf16_t>(bf16_t v) { return v; }

template <typename T>
__global__ __launch_bounds__(256) void k_pack_lowrank(const T* __restrict__ L1, const T* __restrict__ L2, int d,
                                                      int m, int r, int r_pad, bf16_t* __restrict__ out) {
  const size_t n1 = (size_t)r_pad * d, n2 = (size_t)m * r_pad;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n1 + n2; e += (size_t)gridDim.x * blockDim.x) {
    bf16_t v = 0;
    if (e < n1) {
      const int t = (int)(e / d), k = (int)(e % d);
      if (t < r) v = to_bf16<T>(L1[(size_t)k * r + t]);
    } else {
      const size_t e2 = e - n1;
      const int jj = (int)(e2 / r_pad), t = (int)(e2 % r_pad);
      if (t < r) v = to_bf16<T>(L2[(size_t)t * m + jj]);
    }
    out[e] = v;
  }
}

// ---------------------------------------------------------------------------
// One row quantised by a whole 256-thread block.  Columns [0, dl) use BA
// bits, columns [dl, d) use BB bits with their own scale (the two-subspace
// split); dl == d for a single segment.  Two passes over the row: the second
// is served by L2 (the block read the same bytes a moment earlier).
// ---------------------------------------------------------------------------
template <typename T, int BA, int BB>
__device__ __forceinline__ void quant_row_block(const T* __restrict__ x, int d, int dl, uint8_t* __restrict__ ca,
                                                float* __restrict__ sa, uint8_t* __restrict__ cb,
                                                float* __restrict__ sb, float* red) {
  const int tid = threadIdx.x, nthr = blockDim.x, lane = tid & 63, w = tid >> 6, nw = nthr >> 6;
  const int nch = d >> 3, nchl = dl >> 3;
  float ma = 0.0f, mb = 0.0f;
  for (int ch = tid; ch < nch; ch += nthr) {
    float v[8];
    uint4 raw;
    Load8<T>::load(x + 8 * ch, v, raw);
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(v[i]));
    if (ch < nchl)
      ma = fmaxf(ma, mx);
    else
      mb = fmaxf(mb, mx);
  }
  ma = wave_max(ma);
  mb = wave_max(mb);
  if (lane == 0) {
    red[w] = ma;
    red[8 + w] = mb;
  }
  __syncthreads();
  ma = 0.0f;
  mb = 0.0f;
  for (int i = 0; i < nw; ++i) {
    ma = fmaxf(ma, red[i]);
    mb = fmaxf(mb, red[8 + i]);
  }
  const RowScale ra = row_scale<BA>(ma);
  const RowScale rb = row_scale<BB>(mb);
  if (tid == 0) {
    *sa = ra.s;
    if (dl < d) *sb = rb.s;
  }
  for (int ch = tid; ch < nch; ch += nthr) {
    float v[8];
    uint4 raw;
    int q[8];
    Load8<T>::load(x + 8 * ch, v, raw);
    if (ch < nchl) {
      quant8<BA>(v, ra, q);
      if (BA == 4)
        *reinterpret_cast<uint32_t*>(ca + (size_t)ch * 4) = pack_nibbles(q);
      else
        *reinterpret_cast<uint2*>(ca + (size_t)ch * 8) = pack_bytes(q);
    } else {
      quant8<BB>(v, rb, q);
      if (BB == 4)
        *reinterpret_cast<uint32_t*>(cb + (size_t)(ch - nchl) * 4) = pack_nibbles(q);
      else
        *reinterpret_cast<uint2*>(cb + (size_t)(ch - nchl) * 8) = pack_bytes(q);
    }
  }
}

template <typename T, int BA, int BB>
__global__ __launch_bounds__(256) void k_quant_rows(const T* __restrict__ X, int n, int d, int dl,
                                                    uint8_t* __restrict__ ca, float* __restrict__ sa,
                                                    uint8_t* __restrict__ cb, float* __restrict__ sb) {
  __shared__ float red[16];
  const int row = blockIdx.x;
  const size_t lda = (size_t)dl * BA / 8, ldb = (size_t)(d - dl) * BB / 8;
  quant_row_block<T, BA, BB>(X + (size_t)row * d, d, dl, ca + row * lda, sa + row, cb ? cb + row * ldb : nullptr,
                             sb ? sb + row : nullptr, red);
}

// ---------------------------------------------------------------------------
// Prefill prologue: 16 rows per block.  Pass A streams the rows once in the
// bf16 MFMA A-operand layout (lane: row lane%16, 8 consecutive k at
// 32*step + 8*(lane/16)), keeping each row's max|x| and accumulating
// T = X L1 with v_mfma_f32_16x16x32_bf16 against L1^T (same k layout for the
// B operand, so the pairing of k between A and B is the identity).  Waves
// take the 32-k steps round-robin.  Pass B re-reads the rows (L2 hits) and
// writes the 4-bit codes.  NQ = r_pad / 16 output slices of T.
// ---------------------------------------------------------------------------
template <typename T, int NQ>
__global__ __launch_bounds__(256) void k_prologue_prefill(const T* __restrict__ X, int n, int d,
                                                          const bf16_t* __restrict__ L1t, int r_pad,
                                                          uint8_t* __restrict__ xc, float* __restrict__ sx,
                                                          bf16_t* __restrict__ Tout) {
  constexpr int RP = NQ * 16 > 0 ? NQ * 16 : 1;
  __shared__ float smax[4][16];
  __shared__ float sT[16][RP];
  __shared__ float s_s[16], s_r[16];
  __shared__ int s_f[16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int row0 = blockIdx.x * 16;
  const int row = min(row0 + lr, n - 1);
  const T* xr = X + (size_t)row * d;
  const int nsteps = d >> 5;

  f32x4 acc[NQ > 0 ? NQ : 1];
#pragma unroll
  for (int q = 0; q < (NQ > 0 ? NQ : 1); ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  float amax = 0.0f;
  for (int s = w; s < nsteps; s += 4) {
    const int k = 32 * s + 8 * lg;
    float v[8];
    uint4 raw;
    Load8<T>::load(xr + k, v, raw);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    if constexpr (NQ > 0) {
      const bf16x8 a = as_bf16x8(raw);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const uint4 b = *reinterpret_cast<const uint4*>(L1t + (size_t)(16 * q + lr) * d + k);
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, as_bf16x8(b), acc[q], 0, 0, 0);
      }
    }
  }
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  if (lg == 0) smax[w][lr] = amax;
  // T partials of the four waves summed in a fixed order (deterministic).
  if constexpr (NQ > 0) {
    for (int ww = 0; ww < 4; ++ww) {
      if (w == ww) {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float& dst = sT[4 * lg + i][16 * q + lr];
            dst = (ww == 0) ? acc[q][i] : dst + acc[q][i];
          }
      }
      __syncthreads();
    }
  } else {
    __syncthreads();
  }
  if (tid < 16) {
    const float m = fmaxf(fmaxf(smax[0][tid], smax[1][tid]), fmaxf(smax[2][tid], smax[3][tid]));
    const RowScale rs = row_scale<4>(m);
    s_s[tid] = rs.s;
    s_r[tid] = rs.rcp;
    s_f[tid] = rs.fast ? 1 : 0;
    if (row0 + tid < n) sx[row0 + tid] = rs.s;
  }
  if constexpr (NQ > 0) {
    for (int e = tid; e < 16 * RP; e += 256) {
      const int rr = e / RP, cc = e % RP;
      if (row0 + rr < n) Tout[(size_t)(row0 + rr) * r_pad + cc] = (bf16_t)f32_to_bf16_bits(sT[rr][cc]);
    }
  }
  __syncthreads();
  const int nch = d >> 3;
  const int rows_here = min(16, n - row0);
  for (int rr = 0; rr < rows_here; ++rr) {
    const RowScale rs = {s_s[rr], s_r[rr], s_f[rr] != 0};
    const T* xp = X + (size_t)(row0 + rr) * d;
    uint8_t* cp = xc + (size_t)(row0 + rr) * (d >> 1);
    for (int ch = tid; ch < nch; ch += 256) {
      float v[8];
      uint4 raw;
      int q[8];
      Load8<T>::load(xp + 8 * ch, v, raw);
      quant8<4>(v, rs, q);
      *reinterpret_cast<uint32_t*>(cp + 4 * ch) = pack_nibbles(q);
    }
  }
}

// ---------------------------------------------------------------------------
// Small-n prologue (n <= 32).  Blocks [0, n) quantise one row each.  Blocks
// [n, n + nchunk * nq) compute a K-chunk partial of one 16-column slice of
// T for all rows (two 16-row MFMA tiles), write it to P, and the last block
// to finish a slice (agent-scope counter) sums the nchunk partials in chunk
// order into T and resets the counter.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_prologue_decode(const T* __restrict__ X, int n, int d,
                                                         const bf16_t* __restrict__ L1t, int r_pad, int kc,
                                                         int nchunk, uint8_t* __restrict__ xc,
                                                         float* __restrict__ sx, float* __restrict__ P,
                                                         bf16_t* __restrict__ Tout, unsigned* __restrict__ counters) {
  __shared__ float red[16];
  __shared__ float sP[32][17];
  __shared__ int s_last;
  const int b = blockIdx.x;
  if (b < n) {
    quant_row_block<T, 4, 4>(X + (size_t)b * d, d, d, xc + (size_t)b * (d >> 1), sx + b, nullptr, nullptr, red);
    return;
  }
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int nq = r_pad >> 4;
  const int bb = b - n, c = bb / nq, q = bb % nq;
  const int s0 = (c * kc) >> 5, s1 = min(d, (c + 1) * kc) >> 5;
  const bool two = n > 16;
  const T* x0 = X + (size_t)min(lr, n - 1) * d;
  const T* x1 = X + (size_t)min(16 + lr, n - 1) * d;
  const bf16_t* lp = L1t + (size_t)(16 * q + lr) * d;
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int s = s0 + w; s < s1; s += 4) {
    const int k = 32 * s + 8 * lg;
    const bf16x8 bv = as_bf16x8(*reinterpret_cast<const uint4*>(lp + k));
    float v[8];
    uint4 raw;
    Load8<T>::load(x0 + k, v, raw);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(raw), bv, acc0, 0, 0, 0);
    if (two) {
      Load8<T>::load(x1 + k, v, raw);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(raw), bv, acc1, 0, 0, 0);
    }
  }
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float& d0 = sP[4 * lg + i][lr];
        float& d1 = sP[16 + 4 * lg + i][lr];
        d0 = (ww == 0) ? acc0[i] : d0 + acc0[i];
        d1 = (ww == 0) ? acc1[i] : d1 + acc1[i];
      }
    }
    __syncthreads();
  }
  // partial of chunk c: P[c][row][16q + col]
  for (int e = tid; e < n * 16; e += 256) {
    const int rr = e >> 4, cc = e & 15;
    P[((size_t)c * n + rr) * r_pad + 16 * q + cc] = sP[rr][cc];
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned old = __hip_atomic_fetch_add(&counters[q], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == (unsigned)(nchunk - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int e = tid; e < n * 16; e += 256) {
    const int rr = e >> 4, cc = e & 15;
    float sum = 0.0f;
    for (int cc2 = 0; cc2 < nchunk; ++cc2)
      sum += __hip_atomic_load(&P[((size_t)cc2 * n + rr) * r_pad + 16 * q + cc], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    Tout[(size_t)rr * r_pad + 16 * q + cc] = (bf16_t)f32_to_bf16_bits(sum);
  }
  if (tid == 0) __hip_atomic_store(&counters[q], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename T>
static hipError_t launch_pack_weight_t(const void* W, int d, int m, int bits, void* codes, float* sw,
                                       hipStream_t st) {
  dim3 grid((m + 63) / 64), block(256);
  if (bits == 4)
    hipLaunchKernelGGL((k_pack_weight<T, 4>), grid, block, 0, st, (const T*)W, d, m, (uint8_t*)codes, sw);
  else
    hipLaunchKernelGGL((k_pack_weight<T, 8>), grid, block, 0, st, (const T*)W, d, m, (uint8_t*)codes, sw);
  return hipGetLastError();
}

hipError_t launch_pack_weight(const void* W, bool bf16, int d, int m, int bits, void* codes, float* sw,
                              hipStream_t st) {
  return bf16 ? launch_pack_weight_t<bf16_t>(W, d, m, bits, codes, sw, st)
              : launch_pack_weight_t<float>(W, d, m, bits, codes, sw, st);
}

hipError_t launch_pack_lowrank(const void* L1, const void* L2, bool bf16, int d, int m, int r, int r_pad, void* out,
                               hipStream_t st) {
  const size_t total = (size_t)r_pad * d + (size_t)m * r_pad;
  const unsigned blocks = (unsigned)std::min<size_t>((total + 255) / 256, 65536);
  if (bf16)
    hipLaunchKernelGGL((k_pack_lowrank<bf16_t>), dim3(blocks), dim3(256), 0, st, (const bf16_t*)L1,
                       (const bf16_t*)L2, d, m, r, r_pad, (bf16_t*)out);
  else
    hipLaunchKernelGGL((k_pack_lowrank<float>), dim3(blocks), dim3(256), 0, st, (const float*)L1,
                       (const float*)L2, d, m, r, r_pad, (bf16_t*)out);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_quant_rows_t(const void* X, int n, int d, int dl, int ba, int bb, void* ca, float* sa,
                                      void* cb, float* sb, hipStream_t st) {
  dim3 grid(n), block(256);
  const T* x = (const T*)X;
  uint8_t* a = (uint8_t*)ca;
  uint8_t* b = (uint8_t*)cb;
  if (ba == 4 && bb == 8)
    hipLaunchKernelGGL((k_quant_rows<T, 4, 8>), grid, block, 0, st, x, n, d, dl, a, sa, b, sb);
  else if (ba == 4)
    hipLaunchKernelGGL((k_quant_rows<T, 4, 4>), grid, block, 0, st, x, n, d, dl, a, sa, b, sb);
  else
    hipLaunchKernelGGL((k_quant_rows<T, 8, 8>), grid, block, 0, st, x, n, d, dl, a, sa, b, sb);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const void* X, bool bf16, int n, int d, int dl, int bits_a, int bits_b, void* ca,
                             float* sa, void* cb, float* sb, hipStream_t st) {
  return bf16 ? launch_quant_rows_t<bf16_t>(X, n, d, dl, bits_a, bits_b, ca, sa, cb, sb, st)
              : launch_quant_rows_t<float>(X, n, d, dl, bits_a, bits_b, ca, sa, cb, sb, st);
}

template <typename T>
static hipError_t launch_prologue_prefill_t(const void* X, int n, int d, const void* L1t, int r_pad, void* xc,
                                            float* sx, void* Tout, hipStream_t st) {
  dim3 grid((n + 15) / 16), block(256);
  const T* x = (const T*)X;
  const bf16_t* l = (const bf16_t*)L1t;
  uint8_t* c = (uint8_t*)xc;
  bf16_t* t = (bf16_t*)Tout;
  switch (r_pad) {
    case 0: hipLaunchKernelGGL((k_prologue_prefill<T, 0>), grid, block, 0, st, x, n, d, l, r_pad, c, sx, t); break;
    case 32: hipLaunchKernelGGL((k_prologue_prefill<T, 2>), grid, block, 0, st, x, n, d, l, r_pad, c, sx, t); break;
    case 64: hipLaunchKernelGGL((k_prologue_prefill<T, 4>), grid, block, 0, st, x, n, d, l, r_pad, c, sx, t); break;
    case 128: hipLaunchKernelGGL((k_prologue_prefill<T, 8>), grid, block, 0, st, x, n, d, l, r_pad, c, sx, t); break;
    case 256: hipLaunchKernelGGL((k_prologue_prefill<T, 16>), grid, block, 0, st, x, n, d, l, r_pad, c, sx, t); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prologue_prefill(const void* X, bool bf16, int n, int d, const void* L1t, int r_pad, void* xc,
                                   float* sx, void* Tout, hipStream_t st) {
  return bf16 ? launch_prologue_prefill_t<bf16_t>(X, n, d, L1t, r_pad, xc, sx, Tout, st)
              : launch_prologue_prefill_t<float>(X, n, d, L1t, r_pad, xc, sx, Tout, st);
}

hipError_t launch_prologue_decode(const void* X, bool bf16, int n, int d, const void* L1t, int r_pad, int kc,
                                  int nchunk, void* xc, float* sx, float* P, void* Tout, unsigned* counters,
                                  hipStream_t st) {
  const int nq = r_pad / 16;
  dim3 grid(n + (r_pad > 0 ? nchunk * nq : 0)), block(256);
  if (bf16)
    hipLaunchKernelGGL((k_prologue_decode<bf16_t>), grid, block, 0, st, (const bf16_t*)X, n, d,
                       (const bf16_t*)L1t, r_pad, kc, nchunk, (uint8_t*)xc, sx, P, (bf16_t*)Tout, counters);
  else
    hipLaunchKernelGGL((k_prologue_decode<float>), grid, block, 0, st, (const float*)X, n, d, (const bf16_t*)L1t,
                       r_pad, kc, nchunk, (uint8_t*)xc, sx, P, (bf16_t*)Tout, counters);
  return hipGetLastError();
}

}  // namespace tq
