// Per-token asymmetric activations for the two-subspace layer (CoQuant notes,
// "CoQuant: Joint Weight-Activation Subspace Projection for Mixed-Precision
// LLMs", Eq. 1 with a zero-point, and the experimental protocol: per-token
// asymmetric activations, per-channel symmetric weights).
//
// Each token row has two segments, [0, dl) at 4 bits and [dl, d) at 8 bits,
// each with its own zero-point z = min and scale s = fl32(fl32(max - min) /
// (2^N - 1)); the code of x is u = rne(fl32(fl32(x - z) / s)) in
// [0, 2^N - 1].  The GEMM consumes signed codes, so u - 2^(N-1) is stored
// (int8 bytes: the 4-bit segment in the tile GEMM's order, the 8-bit segment
// in natural order), and the epilogue adds the zero-point term
// (z + 2^(N-1) s) s_w colsum(C_w), colsum from tq_weight_colsum:
//   sum_k (u_k s + z) c_k s_w = s s_w sum_k (u_k - 2^(N-1)) c_k
//                               + (z + 2^(N-1) s) s_w sum_k c_k.
//
// One wave per row, the row in registers (CH chunks of 8 values per lane),
// so X is read once: min and max of both segments by wave reductions, then
// the codes with the reciprocal fast path and its exact fallback near ties.

#include "tq_kernels.h"

namespace tq {
namespace {

// PK: the 4-bit segment nibble-packed (dl / 2 bytes per row, even k in the
// low nibble) for the small-n GEMM, else int8 in the tile GEMM's order.
template <typename T, int CH, bool PK = false>
__global__ __launch_bounds__(256) void k_quant_rows_asym(const T* __restrict__ X, int n, int d, int dl,
                                                         uint8_t* __restrict__ xl, float* __restrict__ sl,
                                                         float* __restrict__ zl, uint8_t* __restrict__ xh,
                                                         float* __restrict__ sh, float* __restrict__ zh) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const int lane = threadIdx.x & 63;
  const int nch = d >> 3, nchl = dl >> 3, dh = d - dl;
  const T* x = X + (size_t)row * d;
  // rows up to 8192 values stay in registers; longer rows are read twice
  // (the second pass from L2)
  constexpr bool KEEP = CH <= 16;
  Row8<T> c[KEEP ? CH : 1];
  auto get = [&](int i, float (&v)[8]) {
    if constexpr (KEEP) {
      c[i].get(v);
    } else {
      Row8<T> t;
      t.load(x + 8 * (lane + 64 * i));
      t.get(v);
    }
  };
  if constexpr (KEEP) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int ch = lane + 64 * i;
      if (ch < nch) c[i].load(x + 8 * ch);
    }
  }
  // max and -min of each segment (lanes without values keep -inf)
  float mxl = -INFINITY, nml = -INFINITY, mxh = -INFINITY, nmh = -INFINITY;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int ch = lane + 64 * i;
    if (ch < nch) {
      float v[8];
      get(i, v);
      float hi = v[0], lo = v[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) {
        hi = fmaxf(hi, v[e]);
        lo = fminf(lo, v[e]);
      }
      if (ch < nchl) {
        mxl = fmaxf(mxl, hi);
        nml = fmaxf(nml, -lo);
      } else {
        mxh = fmaxf(mxh, hi);
        nmh = fmaxf(nmh, -lo);
      }
    }
  }
  AsymScale al{}, ah{};
  if (dl > 0) al = asym_scale<4>(-wave_fmax(nml), wave_fmax(mxl));
  if (dh > 0) ah = asym_scale<8>(-wave_fmax(nmh), wave_fmax(mxh));
  if (lane == 0) {
    if (dl > 0) {
      sl[row] = al.s;
      zl[row] = al.z;
    }
    if (dh > 0) {
      sh[row] = ah.s;
      zh[row] = ah.z;
    }
  }
  uint8_t* rl = xl + (size_t)row * (PK ? dl / 2 : dl);
  uint8_t* rh = xh + (size_t)row * dh;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int ch = lane + 64 * i;
    if (ch < nch) {
      float v[8];
      int q[8];
      get(i, v);
      if (ch < nchl) {
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = code_asym<4>(v[e] - al.z, al);
        if constexpr (PK)
          *reinterpret_cast<uint32_t*>(rl + 4 * ch) = pack_nibbles(q);
        else
          store_codes_int8(rl, ch, q);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = code_asym<8>(v[e] - ah.z, ah);
        *reinterpret_cast<uint2*>(rh + 8 * (ch - nchl)) = pack_bytes(q);
      }
    }
  }
}

// colsum[j] = sum_k codes[j][k] for m code rows of k codes (4-bit nibbles or
// int8 bytes), one wave per row.
template <int BITS>
__global__ __launch_bounds__(256) void k_weight_colsum(const uint8_t* __restrict__ codes, int m, int k,
                                                       int32_t* __restrict__ colsum) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= m) return;
  const int lane = threadIdx.x & 63;
  const size_t rb = (size_t)k * BITS / 8;
  const uint8_t* p = codes + (size_t)row * rb;
  int acc = 0;
  for (size_t o = 4 * (size_t)lane; o < rb; o += 256) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p + o);
    if (BITS == 4) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += ((int)(w << (28 - 4 * e))) >> 28;  // sign-extended nibble e
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc += ((int)(w << (24 - 8 * e))) >> 24;  // sign-extended byte e
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) colsum[row] = acc;
}

template <typename T, bool PK>
hipError_t launch_asym_t(const void* X, int n, int d, int dl, void* xl, float* sl, float* zl, void* xh, float* sh,
                         float* zh, hipStream_t st) {
  const dim3 grid((unsigned)((n + 3) / 4)), block(256);
  const T* x = (const T*)X;
  int ch = 1;
  while (ch * 512 < d) ch <<= 1;
#define TQ_ASYM(C)                                                                                            \
  case C:                                                                                                     \
    launch_kernel(k_quant_rows_asym<T, C, PK>, grid, block, 0, st, x, n, d, dl, (uint8_t*)xl, sl, zl, (uint8_t*)xh, \
                  sh, zh);                                                                                    \
    break;
  switch (ch) {
    TQ_ASYM(1)
    TQ_ASYM(2)
    TQ_ASYM(4)
    TQ_ASYM(8)
    TQ_ASYM(16)
    TQ_ASYM(32)
    default:
      return hipErrorInvalidValue;
  }
#undef TQ_ASYM
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_rows_asym(const void* X, bool bf16, int n, int d, int dl, void* xl, float* sl, float* zl,
                                  void* xh, float* sh, float* zh, hipStream_t st, bool packed) {
  if (n <= 0 || d <= 0 || d > kAsymMaxD || dl < 0 || dl > d || dl % 32 || (d - dl) % 16) return hipErrorInvalidValue;
  if (packed)
    return bf16 ? launch_asym_t<bf16_t, true>(X, n, d, dl, xl, sl, zl, xh, sh, zh, st)
                : launch_asym_t<float, true>(X, n, d, dl, xl, sl, zl, xh, sh, zh, st);
  return bf16 ? launch_asym_t<bf16_t, false>(X, n, d, dl, xl, sl, zl, xh, sh, zh, st)
              : launch_asym_t<float, false>(X, n, d, dl, xl, sl, zl, xh, sh, zh, st);
}

hipError_t launch_weight_colsum(const void* codes, int bits, int m, int k, int32_t* colsum, hipStream_t st) {
  const dim3 grid((unsigned)((m + 3) / 4)), block(256);
  if (bits == 4)
    hipLaunchKernelGGL(k_weight_colsum<4>, grid, block, 0, st, (const uint8_t*)codes, m, k, colsum);
  else
    hipLaunchKernelGGL(k_weight_colsum<8>, grid, block, 0, st, (const uint8_t*)codes, m, k, colsum);
  return hipGetLastError();
}

}  // namespace tq
