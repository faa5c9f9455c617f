// First stage of the fully quantised low-rank branch (TwinQuant notes,
// "TwinQuant: Learnable Subspace Decomposition for W4A4 LLM Quantization",
// section 04.A error expression Q(X)[Q(U)Q(V) + Q(R)] and section 04.C,
// Figure 4: the integer result of Q(X) Q(U) is re-quantised on-chip before it
// meets Q(V)).
//
// Block: 32 tokens, 8 waves.  Wave w takes the 128-k steps w, w + 8, ... of
// the rows: lane (l % 32, l / 32) holds the 64 code bytes [64 (l / 32), +64)
// of the step for token l % 32 (int8 codes in the tile GEMM's order), and
// the 32 packed bytes of the same 64 k for rank l % 32 of each 32-rank block,
// expanded by unpack16 to the same order (16 x code per byte).
// v_mfma_i32_32x32x32_i8 produces (rank rows, token columns) blocks; the
// waves' int32 partials are summed in LDS with integer atomics (exact and
// independent of their order).  Then per token: t = fl32(acc) * s_u in fp32,
// the absmax over the ranks, s_t = fl32(max / 7) and the 4-bit codes, stored
// in the int8 code order (8 bytes per 8 ranks) for the second stage in the
// tile GEMM's epilogue.  The int32 sums and t stay in LDS; only the codes
// (r_pad bytes per token) and s_t are written.

#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int kQlrTok = 32;   // tokens per block
constexpr int kQlrWaves = 8;  // waves per block, splitting the k steps

template <int NB, bool XPK>  // NB 32-rank blocks; XPK: nibble-packed activation codes (d / 2 bytes per row)
__global__ __launch_bounds__(kQlrWaves * 64) void k_qlr_stage1(const uint8_t* __restrict__ xc, int n, int d,
                                                                 const uint8_t* __restrict__ uc,
                                                                 const float* __restrict__ su,
                                                                 uint8_t* __restrict__ ct, float* __restrict__ st) {
  constexpr int R = 32 * NB;
  __shared__ int red[R][kQlrTok];  // integer sums (rank-major), then the fp32 t
  __shared__ float gmax[R / 8][kQlrTok];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lg = lane >> 5;
  const int tok0 = blockIdx.x * kQlrTok;
  for (int i = tid; i < R * kQlrTok; i += kQlrWaves * 64) (&red[0][0])[i] = 0;
  __syncthreads();

  const int steps = (d + 127) / 128;
  if (wave < steps) {
    const uint8_t* xr = xc + (size_t)min(tok0 + l32, n - 1) * (XPK ? d / 2 : d);  // rows past n: results unused
    const size_t ub = (size_t)d / 2;                               // packed bytes per rank row
    const uint8_t* ur = uc + (size_t)l32 * ub + 32 * lg;
    i32x16 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][i] = 0;
    for (int s = wave; s < steps; s += kQlrWaves) {
      const int o = 128 * s + 64 * lg;  // this lane's first k of the step (d % 32 == 0: chunks are whole)
      i32x4 xv[4];
      if constexpr (XPK) {  // 32 packed bytes, expanded like U's (16 x code)
        const uint4 p0 = o < d ? *reinterpret_cast<const uint4*>(xr + o / 2) : uint4{0u, 0u, 0u, 0u};
        const uint4 p1 = o + 32 < d ? *reinterpret_cast<const uint4*>(xr + o / 2 + 16) : uint4{0u, 0u, 0u, 0u};
        xv[0] = unpack16(p0.x, p0.y);
        xv[1] = unpack16(p0.z, p0.w);
        xv[2] = unpack16(p1.x, p1.y);
        xv[3] = unpack16(p1.z, p1.w);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          xv[q] = __builtin_bit_cast(i32x4, o + 16 * q < d ? *reinterpret_cast<const uint4*>(xr + o + 16 * q)
                                                           : uint4{0u, 0u, 0u, 0u});
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint8_t* up = ur + (size_t)32 * b * ub + 64 * s;
        const uint4 u0 = o < d ? *reinterpret_cast<const uint4*>(up) : uint4{0u, 0u, 0u, 0u};
        const uint4 u1 = o + 32 < d ? *reinterpret_cast<const uint4*>(up + 16) : uint4{0u, 0u, 0u, 0u};
        acc[b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(unpack16(u0.x, u0.y), xv[0], acc[b],
                                                       0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(unpack16(u0.z, u0.w), xv[1], acc[b],
                                                       0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(unpack16(u1.x, u1.y), xv[2], acc[b],
                                                       0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(unpack16(u1.z, u1.w), xv[3], acc[b],
                                                       0, 0, 0);
      }
    }
    // result layout: lane l, element e -> rank 8 (e / 4) + 4 (l / 32) + e % 4
    // of the block, token l % 32; the sums carry the factor 16 of unpack16
    // (256 with packed activations, expanded the same way)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        atomicAdd(&red[32 * b + 8 * (e >> 2) + 4 * lg + (e & 3)][l32], acc[b][e] >> (XPK ? 8 : 4));
  }
  __syncthreads();

  // t = fl32(acc) * s_u (|acc| < 2^24: exact in fp32), per 8 ranks of a token
  constexpr int G = R / 8;
  for (int i = tid; i < G * kQlrTok; i += kQlrWaves * 64) {
    const int tk = i % kQlrTok, gr = i / kQlrTok;
    float mx = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = (float)red[8 * gr + e][tk] * su[8 * gr + e];
      red[8 * gr + e][tk] = __float_as_int(v);
      mx = fmaxf(mx, fabsf(v));
    }
    gmax[gr][tk] = mx;
  }
  __syncthreads();
  for (int i = tid; i < G * kQlrTok; i += kQlrWaves * 64) {
    const int tk = i % kQlrTok, gr = i / kQlrTok;
    float amax = 0.0f;
    for (int j = 0; j < G; ++j) amax = fmaxf(amax, gmax[j][tk]);
    const RowScale rs = row_scale<4>(amax);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __int_as_float(red[8 * gr + e][tk]);
    const uint2 c = quant8_int8(v, rs);
    const int t = tok0 + tk;
    if (t < n) {
      *reinterpret_cast<uint2*>(ct + (size_t)t * R + 8 * gr) = c;
      if (gr == 0) st[t] = rs.s;
    }
  }
}

// ---------------------------------------------------------------------------
// The same first stage fused with the quantisation of X (rows of d <= 4096,
// r_pad <= 128, where the row and the accumulators fit the registers):
// a block of 16 waves takes 16 tokens.  Each wave quantises one row on its
// own (the row in registers, quant_row_i8_wave) and leaves its int8 codes in
// LDS as well (rows of d + 16 bytes, so the 16 rows of an MFMA operand read
// hit distinct banks); after one barrier, wave w takes the 64-k steps
// w, w + 16, ... on v_mfma_i32_16x16x64_i8 (lane l: token or rank l % 16, the
// 16 codes at 64 s + 16 (l / 16); U's first steps fetched before the
// barrier), the partials are summed with LDS atomics and the 16 rows are
// re-quantised as above.  X is read once and its codes never come back from
// memory.
// ---------------------------------------------------------------------------
constexpr int kQlrFusedMaxD = 4096;
constexpr int kQlrFusedWaves = 16;

__host__ __device__ constexpr int qlr_fused_lds(int d, int r_pad) {
  return 16 * (d + 16) + 16 * r_pad * 4 + (r_pad / 8) * 16 * 4;
}

template <typename T, int CH, int NQ, bool PK>  // NQ 16-rank groups; PK: activation codes to memory nibble-packed
__global__ __launch_bounds__(kQlrFusedWaves * 64) void k_qlr_prologue(const T* __restrict__ X, int n, int d,
                                                                     const uint8_t* __restrict__ uc,
                                                                     const float* __restrict__ su,
                                                                     uint8_t* __restrict__ xc, float* __restrict__ sx,
                                                                     uint8_t* __restrict__ ct,
                                                                     float* __restrict__ st) {
  constexpr int R = 16 * NQ, WAVES = kQlrFusedWaves, NT = WAVES * 64;
  constexpr int UA = NQ <= 2 ? 8 : (NQ <= 4 ? 4 : (NQ <= 8 ? 2 : 1));  // U steps fetched ahead
  constexpr int SJ = (kQlrFusedMaxD / 64 + WAVES - 1) / WAVES;          // steps per wave at most
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nch = d >> 3, XS = d + 16;
  const int row0 = 16 * blockIdx.x;
  int* red = reinterpret_cast<int*>(lds + 16 * XS);  // [16 tokens][R] integer sums, then fp32 t
  float* gmax = reinterpret_cast<float*>(red + 16 * R);
  for (int i = tid; i < 16 * R; i += NT) red[i] = 0;

  // ---- per wave: one row -> s_x, codes (memory and LDS) ----
  {
    const int row = row0 + w;
    uint8_t* lrow = lds + w * XS;
    if (row < n) {
      const float s =
          quant_row_i8_wave<T, CH, PK>(X + (size_t)row * d, nch, lane, xc + (size_t)row * (PK ? d / 2 : d), lrow);
      if (lane == 0) sx[row] = s;
    } else {
      for (int ch = lane; ch < nch; ch += 64) *reinterpret_cast<uint2*>(lrow + 8 * ch) = uint2{0u, 0u};
    }
  }

  // ---- acc1 = C_x C_u^T over the 16 rows in LDS ----
  const int lr = lane & 15, lg = lane >> 4;
  const int nsteps = (d + 63) / 64;
  const size_t ub = (size_t)d / 2;
  const uint8_t* up = uc + (size_t)lr * ub + 8 * lg;  // rank 16 q + lr at + 16 q ub
  uint2 ubuf[UA][NQ];
  auto load_u = [&](int j) {
    const int s = w + WAVES * j;
    const bool ok = 64 * s + 16 * lg < d;  // d % 32 == 0: a lane's 16 codes are all in or all out
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      ubuf[j % UA][q] = ok ? *reinterpret_cast<const uint2*>(up + (size_t)16 * q * ub + 32 * s) : uint2{0u, 0u};
  };
#pragma unroll
  for (int j = 0; j < UA; ++j)
    if (w + WAVES * j < nsteps) load_u(j);
  __syncthreads();
  i32x4 acc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) acc[q] = i32x4{0, 0, 0, 0};
  const uint8_t* ap = lds + lr * XS + 16 * lg;
#pragma unroll
  for (int j = 0; j < SJ; ++j) {
    const int s = w + WAVES * j;
    if (s < nsteps) {
      const i32x4 xa = 64 * s + 16 * lg < d ? *reinterpret_cast<const i32x4*>(ap + 64 * s) : i32x4{0, 0, 0, 0};
      uint2 b[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) b[q] = ubuf[j % UA][q];
      if (j + UA < SJ && s + WAVES * UA < nsteps) load_u(j + UA);
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        acc[q] = __builtin_amdgcn_mfma_i32_16x16x64_i8(xa, unpack16(b[q].x, b[q].y), acc[q], 0, 0, 0);
    }
  }
  // 16x16 result layout: lane l, element i -> token 4 (l / 16) + i, rank l % 16
  // of the group; the sums carry the factor 16 of unpack16
#pragma unroll
  for (int q = 0; q < NQ; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) atomicAdd(&red[(4 * lg + i) * R + 16 * q + lr], acc[q][i] >> 4);
  __syncthreads();

  // ---- per token: t = fl32(acc1) * s_u, absmax, s_t and the 4-bit codes ----
  constexpr int G = R / 8;
  for (int i = tid; i < 16 * G; i += NT) {
    const int tk = i / G, gr = i % G;
    int* rp = red + tk * R + 8 * gr;
    float mx = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = (float)rp[e] * su[8 * gr + e];
      rp[e] = __float_as_int(v);
      mx = fmaxf(mx, fabsf(v));
    }
    gmax[tk * G + gr] = mx;
  }
  __syncthreads();
  for (int i = tid; i < 16 * G; i += NT) {
    const int tk = i / G, gr = i % G;
    float amax = 0.0f;
    for (int j = 0; j < G; ++j) amax = fmaxf(amax, gmax[tk * G + j]);
    const RowScale rs = row_scale<4>(amax);
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __int_as_float(red[tk * R + 8 * gr + e]);
    const uint2 c = quant8_int8(v, rs);
    const int t = row0 + tk;
    if (t < n) {
      *reinterpret_cast<uint2*>(ct + (size_t)t * R + 8 * gr) = c;
      if (gr == 0) st[t] = rs.s;
    }
  }
}

template <typename T, int CH, bool PK>
hipError_t launch_fused_pk(const void* X, int n, int d, const uint8_t* uc, const float* su, int r_pad, uint8_t* xc,
                           float* sx, uint8_t* ct, float* st, hipStream_t stream) {
  const dim3 grid((unsigned)((n + 15) / 16)), block(kQlrFusedWaves * 64);
  const unsigned lds = (unsigned)qlr_fused_lds(d, r_pad);
  const T* x = (const T*)X;
  switch (r_pad) {
    case 32: launch_kernel(k_qlr_prologue<T, CH, 2, PK>, grid, block, lds, stream, x, n, d, uc, su, xc, sx, ct, st); break;
    case 64: launch_kernel(k_qlr_prologue<T, CH, 4, PK>, grid, block, lds, stream, x, n, d, uc, su, xc, sx, ct, st); break;
    case 128: launch_kernel(k_qlr_prologue<T, CH, 8, PK>, grid, block, lds, stream, x, n, d, uc, su, xc, sx, ct, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// few tokens (the small-n GEMM takes packed codes): packed; else int8
template <typename T, int CH>
hipError_t launch_fused_ch(const void* X, int n, int d, const uint8_t* uc, const float* su, int r_pad, uint8_t* xc,
                           float* sx, uint8_t* ct, float* st, bool packed, hipStream_t stream) {
  return packed ? launch_fused_pk<T, CH, true>(X, n, d, uc, su, r_pad, xc, sx, ct, st, stream)
                : launch_fused_pk<T, CH, false>(X, n, d, uc, su, r_pad, xc, sx, ct, st, stream);
}

template <typename T>
hipError_t launch_fused_t(const void* X, int n, int d, const uint8_t* uc, const float* su, int r_pad, uint8_t* xc,
                          float* sx, uint8_t* ct, float* st, bool packed, hipStream_t stream) {
  int ch = 1;
  while (ch * 512 < d) ch <<= 1;  // chunks of 8 values per lane for the whole row
  switch (ch) {
    case 1: return launch_fused_ch<T, 1>(X, n, d, uc, su, r_pad, xc, sx, ct, st, packed, stream);
    case 2: return launch_fused_ch<T, 2>(X, n, d, uc, su, r_pad, xc, sx, ct, st, packed, stream);
    case 4: return launch_fused_ch<T, 4>(X, n, d, uc, su, r_pad, xc, sx, ct, st, packed, stream);
    case 8: return launch_fused_ch<T, 8>(X, n, d, uc, su, r_pad, xc, sx, ct, st, packed, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int NB>
hipError_t launch_nb(const uint8_t* xc, int n, int d, const uint8_t* uc, const float* su, uint8_t* ct, float* st,
                     bool packed, hipStream_t stream) {
  const dim3 grid((unsigned)((n + kQlrTok - 1) / kQlrTok)), block(kQlrWaves * 64);
  if (packed)
    launch_kernel(k_qlr_stage1<NB, true>, grid, block, 0, stream, xc, n, d, uc, su, ct, st);
  else
    launch_kernel(k_qlr_stage1<NB, false>, grid, block, 0, stream, xc, n, d, uc, su, ct, st);
  return hipGetLastError();
}

}  // namespace

bool qlr_fused_ok(int d, int r_pad) {
  return d > 0 && d <= kQlrFusedMaxD && d % 32 == 0 && (r_pad == 32 || r_pad == 64 || r_pad == 128);
}

hipError_t launch_qlr_prologue(const void* X, bool bf16, int n, int d, const uint8_t* uc, const float* su, int r_pad,
                               uint8_t* xc, float* sx, uint8_t* ct, float* st, bool packed, hipStream_t stream) {
  if (n <= 0 || !qlr_fused_ok(d, r_pad)) return hipErrorInvalidValue;
  return bf16 ? launch_fused_t<bf16_t>(X, n, d, uc, su, r_pad, xc, sx, ct, st, packed, stream)
              : launch_fused_t<float>(X, n, d, uc, su, r_pad, xc, sx, ct, st, packed, stream);
}

hipError_t launch_qlr_stage1(const uint8_t* xc, int n, int d, const uint8_t* uc, const float* su, int r_pad,
                             uint8_t* ct, float* st, bool packed, hipStream_t stream) {
  if (n <= 0 || d <= 0 || d % 32) return hipErrorInvalidValue;
  switch (r_pad) {
    case 32:
      return launch_nb<1>(xc, n, d, uc, su, ct, st, packed, stream);
    case 64:
      return launch_nb<2>(xc, n, d, uc, su, ct, st, packed, stream);
    case 128:
      return launch_nb<4>(xc, n, d, uc, su, ct, st, packed, stream);
    case 256:
      return launch_nb<8>(xc, n, d, uc, su, ct, st, packed, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace tq
