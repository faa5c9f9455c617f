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

#include "tq_prologue.h"

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

// W is dv x mv (row stride ldw), taken as zero-padded to d x m: padded
// channels get scale 0 and codes 0, padded rows codes 0.
template <typename T, int BITS>
__global__ __launch_bounds__(256) void k_pack_weight(const T* __restrict__ W, int d, int m, int ldw, int dv, int mv,
                                                     uint8_t* __restrict__ codes, float* __restrict__ sw) {
  __shared__ float red[4][64];
  __shared__ float tile[64][65];
  __shared__ float s_s[64], s_r[64];
  __shared__ int s_f[64];
  const int tid = threadIdx.x, tx = tid & 63, ty = tid >> 6;
  const int j0 = blockIdx.x * 64;
  const int j = min(j0 + tx, mv - 1);
  const bool jv = j0 + tx < mv;
  float am = 0.0f;
  if (jv)
    for (int k = ty; k < dv; k += 4) am = fmaxf(am, fabsf(ld_f32<T>(W + (size_t)k * ldw + j)));
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
  const size_t row_bytes = (size_t)d * (BITS <= 4 ? 4 : 8) / 8;  // 3 / 6 bits stored like 4 / 8
  const int c = tid >> 2, kg = tid & 3;
  const RowScale rs = {s_s[c], s_r[c], s_f[c] != 0};
  for (int k0 = 0; k0 < d; k0 += 64) {
    for (int kk = ty; kk < 64; kk += 4)
      tile[kk][tx] = (jv && k0 + kk < dv) ? ld_f32<T>(W + (size_t)(k0 + kk) * ldw + j) : 0.0f;
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
        uint8_t* dst = codes + (size_t)(j0 + c) * row_bytes + (size_t)(k0 + kb) * (BITS <= 4 ? 4 : 8) / 8;
        if (BITS <= 4)
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

// L1^T into rows1 rows of d (rows r.. zero) at out1, L2^T into m rows of
// r_pad (columns r.. zero) at out2.
template <typename T>
__global__ __launch_bounds__(256) void k_pack_lowrank(const T* __restrict__ L1, const T* __restrict__ L2, int d,
                                                      int m, int r, int r_pad, int rows1, bf16_t* __restrict__ out1,
                                                      bf16_t* __restrict__ out2) {
  const size_t n1 = (size_t)rows1 * d, n2 = (size_t)m * r_pad;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n1 + n2; e += (size_t)gridDim.x * blockDim.x) {
    bf16_t v = 0;
    if (e < n1) {
      const int t = (int)(e / d), k = (int)(e % d);
      if (t < r) v = to_bf16<T>(L1[(size_t)k * r + t]);
      out1[e] = v;
    } else {
      const size_t e2 = e - n1;
      const int jj = (int)(e2 / r_pad), t = (int)(e2 % r_pad);
      if (t < r) v = to_bf16<T>(L2[(size_t)t * m + jj]);
      out2[e2] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// One row quantised by a whole 256-thread block.  Columns [0, dl) use BA
// bits, columns [dl, d) use BB bits with their own scale (the two-subspace
// split); dl == d for a single segment.  Two passes over the row: the second
// is served by L2 (the block read the same bytes a moment earlier).
// ---------------------------------------------------------------------------
template <typename T, int BA, int BB, bool X8 = false>
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
      if (BA <= 4 && X8)
        store_codes_int8(ca, ch, q);
      else if (BA <= 4)
        *reinterpret_cast<uint32_t*>(ca + (size_t)ch * 4) = pack_nibbles(q);
      else
        *reinterpret_cast<uint2*>(ca + (size_t)ch * 8) = pack_bytes(q);
    } else {
      quant8<BB>(v, rb, q);
      if (BB <= 4)
        *reinterpret_cast<uint32_t*>(cb + (size_t)(ch - nchl) * 4) = pack_nibbles(q);
      else
        *reinterpret_cast<uint2*>(cb + (size_t)(ch - nchl) * 8) = pack_bytes(q);
    }
  }
}

template <typename T, int BA, int BB, bool X8 = false>
__global__ __launch_bounds__(256) void k_quant_rows(const T* __restrict__ X, int n, int d, int dl,
                                                    uint8_t* __restrict__ ca, float* __restrict__ sa,
                                                    uint8_t* __restrict__ cb, float* __restrict__ sb) {
  __shared__ float red[16];
  const int row = blockIdx.x;
  const size_t lda = X8 ? (size_t)dl : (size_t)dl * (BA <= 4 ? 4 : 8) / 8,
               ldb = (size_t)(d - dl) * (BB <= 4 ? 4 : 8) / 8;
  quant_row_block<T, BA, BB, X8>(X + (size_t)row * d, d, dl, ca + row * lda, sa + row, cb ? cb + row * ldb : nullptr,
                                 sb ? sb + row : nullptr, red);
}

// ---------------------------------------------------------------------------
// One row quantised by one wave, the whole row held in registers (CH chunks
// of 8 values per lane, chunk index lane + 64 i), so X is read exactly once.
// Columns [0, dl) use BA bits, [dl, d) BB bits with their own scale.
// ---------------------------------------------------------------------------
template <typename T, int BA, int BB, int CH, bool X8 = false>
__device__ __forceinline__ void quant_row_wave(const T* __restrict__ x, int d, int dl, uint8_t* __restrict__ ca,
                                               float* __restrict__ sa, uint8_t* __restrict__ cb,
                                               float* __restrict__ sb) {
  const int lane = threadIdx.x & 63;
  const int nch = d >> 3, nchl = dl >> 3;
  Row8<T> c[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int ch = lane + 64 * i;
    if (ch < nch) c[i].load(x + 8 * ch);
  }
  float ma = 0.0f, mb = 0.0f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int ch = lane + 64 * i;
    if (ch < nch) {
      float v[8];
      c[i].get(v);
      float mx = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[e]));
      if (ch < nchl)
        ma = fmaxf(ma, mx);
      else
        mb = fmaxf(mb, mx);
    }
  }
  ma = wave_max(ma);
  if (dl < d) mb = wave_max(mb);
  const RowScale ra = row_scale<BA>(ma);
  const RowScale rb = row_scale<BB>(mb);
  if (lane == 0) {
    *sa = ra.s;
    if (dl < d) *sb = rb.s;
  }
  // The scales are the same in every lane: one scalar branch per row picks
  // the reciprocal fast path (with its rare per-chunk exact fallback) or the
  // division path, so neither is evaluated speculatively for the other.
  auto store = [&](int ch, const int (&q)[8]) {
    if (ch < nchl) {
      if (BA <= 4 && X8)
        store_codes_int8(ca, ch, q);
      else if (BA <= 4)
        *reinterpret_cast<uint32_t*>(ca + (size_t)ch * 4) = pack_nibbles(q);
      else
        *reinterpret_cast<uint2*>(ca + (size_t)ch * 8) = pack_bytes(q);
    } else {
      if (BB <= 4)
        *reinterpret_cast<uint32_t*>(cb + (size_t)(ch - nchl) * 4) = pack_nibbles(q);
      else
        *reinterpret_cast<uint2*>(cb + (size_t)(ch - nchl) * 8) = pack_bytes(q);
    }
  };
  const bool fast = ra.fast && (dl == d || rb.fast);
  if (__builtin_amdgcn_readfirstlane(fast ? 1 : 0)) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int ch = lane + 64 * i;
      if (ch < nch) {
        float v[8];
        int q[8];
        c[i].get(v);
        if (BA <= 4 && X8 && ch < nchl) {
          *reinterpret_cast<uint2*>(ca + 8 * ch) = quant8_int8<BA <= 4 ? BA : 4>(v, ra);
          continue;
        }
        if (ch < nchl)
          quant8_fast<BA>(v, ra, q);
        else
          quant8_fast<BB>(v, rb, q);
        store(ch, q);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int ch = lane + 64 * i;
      if (ch < nch) {
        float v[8];
        int q[8];
        c[i].get(v);
        if (ch < nchl)
          quant8_exact<BA>(v, ra.s, q);
        else
          quant8_exact<BB>(v, rb.s, q);
        store(ch, q);
      }
    }
  }
}

// 4 rows per 256-thread block, one per wave.
template <typename T, int BA, int BB, int CH, bool X8 = false>
__global__ __launch_bounds__(256) void k_quant_rows_wave(const T* __restrict__ X, int n, int d, int dl,
                                                         uint8_t* __restrict__ ca, float* __restrict__ sa,
                                                         uint8_t* __restrict__ cb, float* __restrict__ sb) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const size_t lda = X8 ? (size_t)dl : (size_t)dl * (BA <= 4 ? 4 : 8) / 8,
               ldb = (size_t)(d - dl) * (BB <= 4 ? 4 : 8) / 8;
  quant_row_wave<T, BA, BB, CH, X8>(X + (size_t)row * d, d, dl, ca + row * lda, sa + row,
                                    cb ? cb + row * ldb : nullptr, sb ? sb + row : nullptr);
}

template <typename T, int CH, int QS, int WAVES, int U, bool X8>
__global__ __launch_bounds__(WAVES * 64) void k_prologue(PrologueArgs a) {
  constexpr int COLS = 16 * QS;
  __shared__ float sP[WAVES][16][COLS + 1];
  __shared__ int s_last;
  const int b = blockIdx.x;
  const T* X = (const T*)a.X;
  if (b < a.nqb) {
    if (a.row_blocks) {
      // CH chunks per lane for one wave -> CH / WAVES per thread for the block
      constexpr int CHB = (CH >= WAVES) ? CH / WAVES : 1;
      __shared__ float red[WAVES];
      quant_row_block_reg<T, CHB>(X + (size_t)b * a.d, a.d, a.xc + (size_t)b * (a.d >> 1), a.sx + b, red);
      return;
    }
    const int row = b * WAVES + (threadIdx.x >> 6);
    if (row < a.n)
      quant_row_wave<T, 4, 4, CH, X8>(X + (size_t)row * a.d, a.d, a.d,
                                      a.xc + (size_t)row * (X8 ? a.d : (a.d >> 1)), a.sx + row, nullptr, nullptr);
    return;
  }
  const int tid = threadIdx.x;
  const TBlock tbk = t_block_products<T, QS, WAVES, U>(a, b - a.nqb, sP);
  const int rt = tbk.rt, c = tbk.c, qg = tbk.qg;
  const int n = a.n;
  __syncthreads();
  const int rows = min(16, n - 16 * rt);
  const int col0 = 16 * qg * QS;
  auto wave_sum = [&](int rr, int cc) {
    float v = 0.0f;
#pragma unroll
    for (int ww = 0; ww < WAVES; ++ww) v += sP[ww][rr][cc];
    return v;
  };
  if (a.partial) {
    for (int e = tid; e < rows * COLS; e += WAVES * 64) {
      const int rr = e / COLS, cc = e % COLS;
      a.P[((size_t)c * n + 16 * rt + rr) * a.r_pad + col0 + cc] = wave_sum(rr, cc);
    }
    return;
  }
  if (a.nchunk == 1) {
    for (int e = tid; e < rows * COLS; e += WAVES * 64) {
      const int rr = e / COLS, cc = e % COLS;
      a.T[(size_t)(16 * rt + rr) * a.r_pad + col0 + cc] = (bf16_t)f32_to_bf16_bits(wave_sum(rr, cc));
    }
    return;
  }
  // Cross-block sum without device-wide cache maintenance: partials are
  // written and read with agent-scope atomic stores / loads, which go to the
  // device's point of coherence, and the barrier below waits until every
  // wave's stores have completed before the counter is bumped.
  for (int e = tid; e < rows * COLS; e += WAVES * 64) {
    const int rr = e / COLS, cc = e % COLS;
    __hip_atomic_store(&a.P[((size_t)c * n + 16 * rt + rr) * a.r_pad + col0 + cc], wave_sum(rr, cc), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  unsigned* ctr = a.counters + rt * a.nqg + qg;
  if (tid == 0) {
    const unsigned old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (old == (unsigned)(a.nchunk - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  for (int e = tid; e < rows * COLS; e += WAVES * 64) {
    const int rr = e / COLS, cc = e % COLS;
    const float* pp = a.P + (size_t)(16 * rt + rr) * a.r_pad + col0 + cc;
    const size_t stride = (size_t)n * a.r_pad;
    const int nc = a.nchunk;
    float sum = 0.0f;
    for (int k0 = 0; k0 < nc; k0 += 8) {  // chunk order, 8 loads in flight
      float part[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k0 + k < nc) part[k] = __hip_atomic_load(pp + (k0 + k) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k0 + k < nc) sum += part[k];
    }
    a.T[(size_t)(16 * rt + rr) * a.r_pad + col0 + cc] = (bf16_t)f32_to_bf16_bits(sum);
    // chunk 0 of this element was read above by this thread only
    if (a.sum_to_p0) __hip_atomic_store(const_cast<float*>(pp), sum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <typename T>
static hipError_t launch_pack_weight_t(const void* W, int d, int m, int ldw, int dv, int mv, int bits, void* codes,
                                       float* sw, hipStream_t st) {
  dim3 grid((m + 63) / 64), block(256);
  const T* w = (const T*)W;
  uint8_t* c = (uint8_t*)codes;
  switch (bits) {
    case 3: hipLaunchKernelGGL((k_pack_weight<T, 3>), grid, block, 0, st, w, d, m, ldw, dv, mv, c, sw); break;
    case 4: hipLaunchKernelGGL((k_pack_weight<T, 4>), grid, block, 0, st, w, d, m, ldw, dv, mv, c, sw); break;
    case 6: hipLaunchKernelGGL((k_pack_weight<T, 6>), grid, block, 0, st, w, d, m, ldw, dv, mv, c, sw); break;
    case 8: hipLaunchKernelGGL((k_pack_weight<T, 8>), grid, block, 0, st, w, d, m, ldw, dv, mv, c, sw); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_pack_weight(const void* W, bool bf16, int d, int m, int bits, void* codes, float* sw,
                              hipStream_t st) {
  return launch_pack_weight_padded(W, bf16, d, m, m, d, m, bits, codes, sw, st);
}

hipError_t launch_pack_weight_padded(const void* W, bool bf16, int d, int m, int ldw, int dv, int mv, int bits,
                                     void* codes, float* sw, hipStream_t st) {
  return bf16 ? launch_pack_weight_t<bf16_t>(W, d, m, ldw, dv, mv, bits, codes, sw, st)
              : launch_pack_weight_t<float>(W, d, m, ldw, dv, mv, bits, codes, sw, st);
}

hipError_t launch_pack_lowrank(const void* L1, const void* L2, bool bf16, int d, int m, int r, int r_pad, int rows1,
                               void* out1, void* out2, hipStream_t st) {
  const size_t total = (size_t)rows1 * d + (size_t)m * r_pad;
  const unsigned blocks = (unsigned)std::min<size_t>((total + 255) / 256, 65536);
  if (bf16)
    hipLaunchKernelGGL((k_pack_lowrank<bf16_t>), dim3(blocks), dim3(256), 0, st, (const bf16_t*)L1,
                       (const bf16_t*)L2, d, m, r, r_pad, rows1, (bf16_t*)out1, (bf16_t*)out2);
  else
    hipLaunchKernelGGL((k_pack_lowrank<float>), dim3(blocks), dim3(256), 0, st, (const float*)L1,
                       (const float*)L2, d, m, r, r_pad, rows1, (bf16_t*)out1, (bf16_t*)out2);
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

static int chunks_for(int d) {
  int ch = 1;
  while (ch * 512 < d) ch <<= 1;
  return ch;  // 1, 2, 4, ...: row of d values in ch chunks of 8 per lane
}

template <typename T, int BA, int BB, bool X8 = false>
static hipError_t launch_quant_rows_wave_t(const void* X, int n, int d, int dl, void* ca, float* sa, void* cb,
                                           float* sb, hipStream_t st) {
  dim3 grid((n + 3) / 4), block(256);
  const T* x = (const T*)X;
  uint8_t* a = (uint8_t*)ca;
  uint8_t* b = (uint8_t*)cb;
  switch (chunks_for(d)) {
    case 1: hipLaunchKernelGGL((k_quant_rows_wave<T, BA, BB, 1, X8>), grid, block, 0, st, x, n, d, dl, a, sa, b, sb); break;
    case 2: hipLaunchKernelGGL((k_quant_rows_wave<T, BA, BB, 2, X8>), grid, block, 0, st, x, n, d, dl, a, sa, b, sb); break;
    case 4: hipLaunchKernelGGL((k_quant_rows_wave<T, BA, BB, 4, X8>), grid, block, 0, st, x, n, d, dl, a, sa, b, sb); break;
    case 8: hipLaunchKernelGGL((k_quant_rows_wave<T, BA, BB, 8, X8>), grid, block, 0, st, x, n, d, dl, a, sa, b, sb); break;
    case 16: hipLaunchKernelGGL((k_quant_rows_wave<T, BA, BB, 16, X8>), grid, block, 0, st, x, n, d, dl, a, sa, b, sb); break;
    case 32: hipLaunchKernelGGL((k_quant_rows_wave<T, BA, BB, 32, X8>), grid, block, 0, st, x, n, d, dl, a, sa, b, sb); break;
    default:  // rows beyond 16384 values: a block per row
      if constexpr (X8)
        hipLaunchKernelGGL((k_quant_rows<T, BA, BB, true>), dim3(n), dim3(256), 0, st, x, n, d, dl, a, sa, b, sb);
      else if constexpr ((BA == 4 || BA == 8) && (BB == 4 || BB == 8))
        return launch_quant_rows_t<T>(X, n, d, dl, BA, BB, ca, sa, cb, sb, st);
      else
        hipLaunchKernelGGL((k_quant_rows<T, BA, BB>), dim3(n), dim3(256), 0, st, x, n, d, dl, a, sa, b, sb);
  }
  return hipGetLastError();
}

hipError_t launch_quant_rows_i8(const void* X, bool bf16, int n, int d, int dl, int bits_b, void* ca, float* sa,
                                void* cb, float* sb, hipStream_t st) {
  if (bf16)
    return bits_b == 8 ? launch_quant_rows_wave_t<bf16_t, 4, 8, true>(X, n, d, dl, ca, sa, cb, sb, st)
                       : launch_quant_rows_wave_t<bf16_t, 4, 4, true>(X, n, d, dl, ca, sa, cb, sb, st);
  return bits_b == 8 ? launch_quant_rows_wave_t<float, 4, 8, true>(X, n, d, dl, ca, sa, cb, sb, st)
                     : launch_quant_rows_wave_t<float, 4, 4, true>(X, n, d, dl, ca, sa, cb, sb, st);
}

hipError_t launch_quant_rows_i8_bits(const void* X, bool bf16, int n, int d, int dl, int bits_a, int bits_b, void* ca,
                                     float* sa, void* cb, float* sb, hipStream_t st) {
#define TQ_QB(T)                                                                                                   \
  if (bits_a == 4) return bits_b == 8 ? launch_quant_rows_wave_t<T, 4, 8, true>(X, n, d, dl, ca, sa, cb, sb, st)    \
                                      : launch_quant_rows_wave_t<T, 4, 4, true>(X, n, d, dl, ca, sa, cb, sb, st);   \
  if (bits_a == 3) return bits_b == 6 ? launch_quant_rows_wave_t<T, 3, 6, true>(X, n, d, dl, ca, sa, cb, sb, st)    \
                                      : launch_quant_rows_wave_t<T, 3, 3, true>(X, n, d, dl, ca, sa, cb, sb, st);   \
  return hipErrorInvalidValue;
  if (bf16) {
    TQ_QB(bf16_t)
  } else {
    TQ_QB(float)
  }
#undef TQ_QB
}

hipError_t launch_quant_rows_fast(const void* X, bool bf16, int n, int d, int dl, int bits_a, int bits_b, void* ca,
                                  float* sa, void* cb, float* sb, hipStream_t st) {
#define TQ_QR(T)                                                                                          \
  if (bits_a == 4 && bits_b == 8) return launch_quant_rows_wave_t<T, 4, 8>(X, n, d, dl, ca, sa, cb, sb, st); \
  if (bits_a == 4) return launch_quant_rows_wave_t<T, 4, 4>(X, n, d, dl, ca, sa, cb, sb, st);               \
  if (bits_a == 6) return launch_quant_rows_wave_t<T, 6, 6>(X, n, d, dl, ca, sa, cb, sb, st);               \
  return launch_quant_rows_wave_t<T, 8, 8>(X, n, d, dl, ca, sa, cb, sb, st);
  if (bf16) {
    TQ_QR(bf16_t)
  } else {
    TQ_QR(float)
  }
#undef TQ_QR
}

// ---------------------------------------------------------------------------
// Prologue of tq_linear for many tokens, reading X once.  A block of 16
// waves takes 16 rows, one per wave:
//  * each wave, on its own (no block barrier, so a wave quantises while
//    others still wait for their rows): loads its row, takes the absmax
//    (wave reduction) and s_x, writes the int8 codes of the tile GEMM (same
//    quantiser as quant_row_wave) and leaves the row as bf16 in LDS (rows
//    padded by 16 bytes, so the 16 rows of an MFMA operand read hit distinct
//    banks);
//  * after one barrier, the first low-rank stage T = X L1 on
//    v_mfma_f32_16x16x32_bf16 (lane l: row or T column l % 16, the 8 k at
//    32 s + 8 (l / 16)), wave w taking the 32-k steps s = w mod 16, with
//    its first L1 operands fetched before the barrier; the 16 wave partials
//    are summed through LDS in wave order and rounded once to bf16.
// TwinQuant notes, "TwinQuant: Learnable Subspace Decomposition for W4A4
// LLM Quantization", section 04.C (per-token scales, T = X L1 feeding the
// shared epilogue).
// ---------------------------------------------------------------------------
struct FusedArgs {
  const void* X;
  int n, d;
  const bf16_t* L1t;
  int r_pad;
  uint8_t* xc;
  float* sx;
  bf16_t* T;
  float* zx;  // ASYM: per-token zero-points
};
constexpr int kFusedWaves = 16;
constexpr int kFusedMaxD = 4096;  // the 16 bf16 rows fill at most 128 KiB of LDS

__host__ __device__ constexpr int fused_row_bytes(int d) { return 2 * d + 16; }
__host__ __device__ constexpr int fused_lds_bytes(int d, int qs) {
  const int x = kFusedWaves * fused_row_bytes(d), p = kFusedWaves * 16 * (16 * qs + 1) * 4;
  return x > p ? x : p;
}

// ASYM: per-token asymmetric codes (u - 8, z = min, s = range / 15) and the
// zero-points, for the asymmetric layer.
template <typename T, int CH, int QS, bool ASYM = false>
__global__ __launch_bounds__(1024) void k_prologue_rows(FusedArgs a) {
  constexpr int WAVES = kFusedWaves, COLS = 16 * QS;
  constexpr int U = QS <= 2 ? 8 : (QS <= 4 ? 4 : 1);  // L1 steps fetched ahead
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int d = a.d, nch = d >> 3, XS = fused_row_bytes(d);
  const int row0 = 16 * blockIdx.x;

  // ---- per wave: one row -> s_x, codes, bf16 copy in LDS ----
  {
    const int row = row0 + w;
    uint8_t* sx_row = lds + w * XS;
    if (row < a.n) {
      const T* x = (const T*)a.X + (size_t)row * d;
      Row8<T> r[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int ch = lane + 64 * i;
        if (ch < nch) r[i].load(x + 8 * ch);
      }
      uint8_t* cr = a.xc + (size_t)row * d;
      if constexpr (ASYM) {
        float hi = -INFINITY, nlo = -INFINITY;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          if (lane + 64 * i < nch) {
            float v[8];
            r[i].get(v);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              hi = fmaxf(hi, v[e]);
              nlo = fmaxf(nlo, -v[e]);
            }
          }
        }
        const AsymScale as = asym_scale<4>(-wave_fmax(nlo), wave_fmax(hi));
        if (lane == 0) {
          a.sx[row] = as.s;
          a.zx[row] = as.z;
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          const int ch = lane + 64 * i;
          if (ch < nch) {
            float v[8];
            int q[8];
            r[i].get(v);
#pragma unroll
            for (int e = 0; e < 8; ++e) q[e] = code_asym<4>(v[e] - as.z, as);
            store_codes_int8(cr, ch, q);
            if constexpr (QS > 0) *reinterpret_cast<uint4*>(sx_row + 16 * ch) = r[i].bf16();
          }
        }
      } else {
        float mx = 0.0f;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          if (lane + 64 * i < nch) {
            float v[8];
            r[i].get(v);
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[e]));
          }
        }
        const RowScale rs = row_scale<4>(wave_max(mx));
        if (lane == 0) a.sx[row] = rs.s;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
          const int ch = lane + 64 * i;
          if (ch < nch) {
            float v[8];
            r[i].get(v);
            *reinterpret_cast<uint2*>(cr + 8 * ch) = quant8_int8(v, rs);
            if constexpr (QS > 0) *reinterpret_cast<uint4*>(sx_row + 16 * ch) = r[i].bf16();
          }
        }
      }
    } else if constexpr (QS > 0) {
      for (int ch = lane; ch < nch; ch += 64) *reinterpret_cast<uint4*>(sx_row + 16 * ch) = uint4{0, 0, 0, 0};
    }
  }
  if constexpr (QS == 0) return;

  // ---- T = X L1 over the 16 rows in LDS ----
  const int lr = lane & 15, lg = lane >> 4;
  const int nsteps = d >> 5;
  const bf16_t* lp = a.L1t + (size_t)lr * d + 8 * lg;
  uint4 lb[U][QS > 0 ? QS : 1];
  auto load_l1 = [&](int j) {
    const int s = w + WAVES * j;
#pragma unroll
    for (int q = 0; q < QS; ++q)
      lb[j % U][q] = *reinterpret_cast<const uint4*>(lp + (size_t)16 * q * d + 32 * s);
  };
  constexpr int SJ = (kFusedMaxD / 32 + WAVES - 1) / WAVES;  // steps per wave at most
#pragma unroll
  for (int j = 0; j < U; ++j)
    if (w + WAVES * j < nsteps) load_l1(j);
  __syncthreads();
  f32x4 acc[QS > 0 ? QS : 1];
#pragma unroll
  for (int q = 0; q < QS; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint8_t* ap = lds + lr * XS + 16 * lg;
#pragma unroll
  for (int j = 0; j < SJ; ++j) {
    const int s = w + WAVES * j;
    if (s < nsteps) {
      const uint4 xa = *reinterpret_cast<const uint4*>(ap + 64 * s);
      uint4 b[QS > 0 ? QS : 1];
#pragma unroll
      for (int q = 0; q < QS; ++q) b[q] = lb[j % U][q];
      if (j + U < SJ && s + WAVES * U < nsteps) load_l1(j + U);
#pragma unroll
      for (int q = 0; q < QS; ++q)
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), as_bf16x8(b[q]), acc[q], 0, 0, 0);
    }
  }
  __syncthreads();  // the LDS rows are free: partials go there
  float* sP = reinterpret_cast<float*>(lds);  // [WAVES][16][COLS + 1]
  // 16x16 result layout: lane l, element i -> row 4 (l / 16) + i, column l % 16
#pragma unroll
  for (int q = 0; q < QS; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) sP[(w * 16 + 4 * lg + i) * (COLS + 1) + 16 * q + lr] = acc[q][i];
  __syncthreads();
  const int rows = min(16, a.n - row0);
  for (int e = tid; e < rows * COLS; e += WAVES * 64) {
    const int rr = e / COLS, cc = e % COLS;
    float v = sP[rr * (COLS + 1) + cc];
#pragma unroll
    for (int ww = 1; ww < WAVES; ++ww) v += sP[(ww * 16 + rr) * (COLS + 1) + cc];
    a.T[(size_t)(row0 + rr) * a.r_pad + cc] = (bf16_t)f32_to_bf16_bits(v);
  }
}

static bool fused_fits(int d, int qs) {
  return d <= kFusedMaxD && (qs == 0 || qs == 2 || qs == 4 || qs == 8) && fused_lds_bytes(d, qs) <= 160 * 1024;
}

template <typename T, int CH, bool ASYM>
static hipError_t launch_rows_ch(const FusedArgs& a, int qs, hipStream_t st) {
  const dim3 grid((unsigned)((a.n + 15) / 16)), block(64 * kFusedWaves);
  const unsigned lds = (unsigned)fused_lds_bytes(a.d, qs);
  switch (qs) {
    case 0: launch_kernel(k_prologue_rows<T, CH, 0, ASYM>, grid, block, lds, st, a); break;
    case 2: launch_kernel(k_prologue_rows<T, CH, 2, ASYM>, grid, block, lds, st, a); break;
    case 4: launch_kernel(k_prologue_rows<T, CH, 4, ASYM>, grid, block, lds, st, a); break;
    case 8: launch_kernel(k_prologue_rows<T, CH, 8, ASYM>, grid, block, lds, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, bool ASYM>
static hipError_t launch_rows_t(const FusedArgs& a, int qs, hipStream_t st) {
  switch (chunks_for(a.d)) {
    case 1: return launch_rows_ch<T, 1, ASYM>(a, qs, st);
    case 2: return launch_rows_ch<T, 2, ASYM>(a, qs, st);
    case 4: return launch_rows_ch<T, 4, ASYM>(a, qs, st);
    case 8: return launch_rows_ch<T, 8, ASYM>(a, qs, st);
    default: return hipErrorInvalidValue;
  }
}

static hipError_t launch_prologue_fused(const void* X, bool bf16, int n, int d, const void* L1t, int r_pad,
                                        void* xc, float* sx, void* Tout, hipStream_t st, float* zx = nullptr) {
  const FusedArgs a{X, n, d, (const bf16_t*)L1t, r_pad, (uint8_t*)xc, sx, (bf16_t*)Tout, zx};
  const int qs = r_pad / 16;
  if (!fused_fits(d, qs)) return hipErrorInvalidValue;
  if (zx) return bf16 ? launch_rows_t<bf16_t, true>(a, qs, st) : launch_rows_t<float, true>(a, qs, st);
  return bf16 ? launch_rows_t<bf16_t, false>(a, qs, st) : launch_rows_t<float, false>(a, qs, st);
}

// Fewest tokens for the fused prologue.
constexpr int kFusedMinRows = 1024;
// Most k-chunks of T the few-token prologue sums itself.
constexpr int kMaxPrologueChunks = 64;

// The producers of the one-launch few-token layer: a block per token row,
// then T blocks of 32 columns each (QS = 2) over k-chunks of at least 16
// steps, at most max_chunks of them (the GEMM blocks sum them in one pass).
ProloguePlan plan_prologue_fused(int n, int d, int r_pad, int max_chunks) {
  ProloguePlan p{};
  const int steps = d / 32;
  p.waves = d > 4096 ? 8 : 4;
  p.qs = 2;
  p.quant_in_prologue = true;
  p.row_blocks = true;
  p.partial = true;
  p.nqb = n;
  if (r_pad == 0) {
    p.nqg = 0;
    p.nchunk = 1;
    p.kc = d;
    p.ntb = 0;
    return p;
  }
  p.nqg = r_pad / 32;
  const int nch = std::max(1, std::min((steps + 15) / 16, max_chunks));
  const int chunk_steps = (steps + nch - 1) / nch;
  p.kc = 32 * chunk_steps;
  p.nchunk = (steps + chunk_steps - 1) / chunk_steps;
  p.ntb = ((n + 15) / 16) * p.nchunk * p.nqg;
  return p;
}

ProloguePlan plan_prologue(int n, int d, int r_pad, bool small, int max_chunks) {
  ProloguePlan p{};
  const int nq = r_pad / 16;
  const int nrt = (n + 15) / 16;
  const int steps = (d + 31) / 32;  // 32-k MFMA steps along d
  p.waves = small ? 8 : 4;
  if (nq == 0) {
    p.qs = 1;
    p.nqg = 0;
    p.nchunk = 1;
    p.kc = d;
    p.ntb = 0;
  } else if (small) {
    // few tokens: all (up to 64) columns per block, 8 waves with up to 8
    // steps each in flight; k split into chunks of at least 16 steps, as
    // many as the small-n GEMM can sum in one pass (max_chunks), so that L1
    // is read by many CUs at once; fp32 partials per k-chunk, summed there
    p.qs = std::min(nq, 4);
    p.nqg = nq / p.qs;
    const int want = std::max(1, (steps + 15) / 16);
    // long rows with several row tiles want more chunks than the small-n
    // GEMM sums in one pass: then the last block of each (row tile, slice
    // group) sums them here and leaves the fp32 sum in chunk 0
    const int nch = want <= max_chunks ? want : std::min(want, kMaxPrologueChunks);
    const int chunk_steps = (steps + nch - 1) / nch;
    p.kc = 32 * chunk_steps;
    p.nchunk = (steps + chunk_steps - 1) / chunk_steps;
    p.partial = p.nchunk <= max_chunks;
    p.sum_to_p0 = !p.partial;
    p.ntb = nrt * p.nchunk * p.nqg;
  } else {
    // QS 16-column slices of T per block (all of them in one block when rows
    // are many, one per block otherwise); each of the 4 waves issues 8 / QS
    // steps at once.
    p.qs = (nrt >= 64) ? std::min(nq, 4) : 1;
    p.nqg = nq / p.qs;
    if (nrt * p.nqg >= 128) {
      // many row tiles: one block per (row tile, slice group) over all of k,
      // no partial sums to combine across blocks
      p.kc = 32 * steps;
      p.nchunk = 1;
    } else {
      // few row tiles: split k so that each wave issues all of its 8 / QS
      // steps at once, and combine the partials across blocks
      const int chunk_steps = 4 * (8 / p.qs);
      p.kc = 32 * chunk_steps;
      p.nchunk = (steps + chunk_steps - 1) / chunk_steps;
    }
    p.ntb = nrt * p.nchunk * p.nqg;
  }
  p.quant_in_prologue = chunks_for(d) <= 32;
  p.row_blocks = small;  // few tokens: a block per row
  if (!small && n >= kFusedMinRows && fused_fits(d, nq)) {
    ProloguePlan f{};
    f.fused = true;
    f.qs = nq;
    f.waves = kFusedWaves;
    return f;
  }
  p.nqb = p.quant_in_prologue ? (small ? n : (n + p.waves - 1) / p.waves) : 0;
  p.counters = (p.ntb > 0 && !p.partial && p.nchunk > 1) ? nrt * std::max(p.nqg, 1) : 0;
  return p;
}

template <typename T, int QS, int WAVES, int U, bool X8>
static hipError_t launch_prologue_q(const PrologueArgs& a, int ch, hipStream_t st) {
  const dim3 grid(a.nqb + (unsigned)(a.nqg ? ((a.n + 15) / 16) * a.nchunk * a.nqg : 0)), block(WAVES * 64);
  switch (ch) {
    case 1: hipLaunchKernelGGL((k_prologue<T, 1, QS, WAVES, U, X8>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_prologue<T, 2, QS, WAVES, U, X8>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_prologue<T, 4, QS, WAVES, U, X8>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_prologue<T, 8, QS, WAVES, U, X8>), grid, block, 0, st, a); break;
    case 16: hipLaunchKernelGGL((k_prologue<T, 16, QS, WAVES, U, X8>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((k_prologue<T, 32, QS, WAVES, U, X8>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

// few tokens (8 waves): nibble-packed codes for the small-n GEMM; otherwise
// int8 codes for the int8 tile GEMM
template <typename T>
static hipError_t launch_prologue_t(const PrologueArgs& a, int waves, int ch, hipStream_t st) {
  if (waves == 8)
    return a.qs == 4 ? launch_prologue_q<T, 4, 8, 8, false>(a, ch, st) : launch_prologue_q<T, 2, 8, 8, false>(a, ch, st);
  switch (a.qs) {
    case 1: return launch_prologue_q<T, 1, 4, 8, true>(a, ch, st);
    case 2: return launch_prologue_q<T, 2, 4, 4, true>(a, ch, st);
    default: return launch_prologue_q<T, 4, 4, 2, true>(a, ch, st);
  }
}

hipError_t launch_prologue_asym(const void* X, bool bf16, int n, int d, const void* L1t, int r_pad,
                                const ProloguePlan& p, void* xc, float* sx, float* zx, float* P, void* Tout,
                                unsigned* counters, hipStream_t st) {
  if (p.fused) return launch_prologue_fused(X, bf16, n, d, L1t, r_pad, xc, sx, Tout, st, zx);
  // the asymmetric quantiser (int8 codes for the tile GEMM), then the T blocks alone
  hipError_t e = launch_quant_rows_asym(X, bf16, n, d, d, xc, sx, zx, nullptr, nullptr, nullptr, st, p.row_blocks);
  if (e != hipSuccess || p.ntb == 0) return e;
  PrologueArgs a{X, n, d, (const bf16_t*)L1t, r_pad, p.kc, p.nchunk, p.qs, p.nqg, 0, p.partial ? 1 : 0,
                 p.row_blocks ? 1 : 0, p.sum_to_p0 ? 1 : 0, (uint8_t*)xc, sx, P, (bf16_t*)Tout, counters};
  const int ch = std::min(chunks_for(d), 32);
  return bf16 ? launch_prologue_t<bf16_t>(a, p.waves, ch, st) : launch_prologue_t<float>(a, p.waves, ch, st);
}

hipError_t launch_prologue(const void* X, bool bf16, int n, int d, const void* L1t, int r_pad, const ProloguePlan& p,
                           void* xc, float* sx, float* P, void* Tout, unsigned* counters, hipStream_t st) {
  if (p.fused) return launch_prologue_fused(X, bf16, n, d, L1t, r_pad, xc, sx, Tout, st);
  if (!p.quant_in_prologue) {
    hipError_t e;
    if (p.waves == 8) {
      e = launch_quant_rows(X, bf16, n, d, d, 4, 4, xc, sx, nullptr, nullptr, st);
    } else {  // int8 codes for the tile GEMM
      if (bf16)
        hipLaunchKernelGGL((k_quant_rows<bf16_t, 4, 4, true>), dim3(n), dim3(256), 0, st, (const bf16_t*)X, n, d, d,
                           (uint8_t*)xc, sx, nullptr, nullptr);
      else
        hipLaunchKernelGGL((k_quant_rows<float, 4, 4, true>), dim3(n), dim3(256), 0, st, (const float*)X, n, d, d,
                           (uint8_t*)xc, sx, nullptr, nullptr);
      e = hipGetLastError();
    }
    if (e != hipSuccess) return e;
    if (p.ntb == 0) return hipSuccess;
  }
  PrologueArgs a{X, n, d, (const bf16_t*)L1t, r_pad, p.kc, p.nchunk, p.qs, p.nqg, p.nqb, p.partial ? 1 : 0,
                 p.row_blocks ? 1 : 0, p.sum_to_p0 ? 1 : 0, (uint8_t*)xc, sx, P, (bf16_t*)Tout, counters};
  const int ch = std::min(chunks_for(d), 32);
  return bf16 ? launch_prologue_t<bf16_t>(a, p.waves, ch, st) : launch_prologue_t<float>(a, p.waves, ch, st);
}

}  // namespace tq
