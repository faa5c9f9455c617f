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

template <int NB>  // NB 32-rank blocks
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
    const uint8_t* xr = xc + (size_t)min(tok0 + l32, n - 1) * d;  // rows past n: any valid row, results unused
    const size_t ub = (size_t)d / 2;                               // packed bytes per rank row
    const uint8_t* ur = uc + (size_t)l32 * ub + 32 * lg;
    i32x16 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][i] = 0;
    for (int s = wave; s < steps; s += kQlrWaves) {
      const int o = 128 * s + 64 * lg;  // this lane's first k of the step (d % 32 == 0: chunks are whole)
      uint4 xv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xv[q] = o + 16 * q < d ? *reinterpret_cast<const uint4*>(xr + o + 16 * q) : uint4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const uint8_t* up = ur + (size_t)32 * b * ub + 64 * s;
        const uint4 u0 = o < d ? *reinterpret_cast<const uint4*>(up) : uint4{0u, 0u, 0u, 0u};
        const uint4 u1 = o + 32 < d ? *reinterpret_cast<const uint4*>(up + 16) : uint4{0u, 0u, 0u, 0u};
        acc[b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(unpack16(u0.x, u0.y), __builtin_bit_cast(i32x4, xv[0]), acc[b],
                                                       0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(unpack16(u0.z, u0.w), __builtin_bit_cast(i32x4, xv[1]), acc[b],
                                                       0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(unpack16(u1.x, u1.y), __builtin_bit_cast(i32x4, xv[2]), acc[b],
                                                       0, 0, 0);
        acc[b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(unpack16(u1.z, u1.w), __builtin_bit_cast(i32x4, xv[3]), acc[b],
                                                       0, 0, 0);
      }
    }
    // result layout: lane l, element e -> rank 8 (e / 4) + 4 (l / 32) + e % 4
    // of the block, token l % 32; the sums carry the factor 16 of unpack16
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) atomicAdd(&red[32 * b + 8 * (e >> 2) + 4 * lg + (e & 3)][l32], acc[b][e] >> 4);
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

template <int NB>
hipError_t launch_nb(const uint8_t* xc, int n, int d, const uint8_t* uc, const float* su, uint8_t* ct, float* st,
                     hipStream_t stream) {
  launch_kernel(k_qlr_stage1<NB>, dim3((unsigned)((n + kQlrTok - 1) / kQlrTok)), dim3(kQlrWaves * 64), 0, stream, xc,
                n, d, uc, su, ct, st);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qlr_stage1(const uint8_t* xc, int n, int d, const uint8_t* uc, const float* su, int r_pad,
                             uint8_t* ct, float* st, hipStream_t stream) {
  if (n <= 0 || d <= 0 || d % 32) return hipErrorInvalidValue;
  switch (r_pad) {
    case 32:
      return launch_nb<1>(xc, n, d, uc, su, ct, st, stream);
    case 64:
      return launch_nb<2>(xc, n, d, uc, su, ct, st, stream);
    case 128:
      return launch_nb<4>(xc, n, d, uc, su, ct, st, stream);
    case 256:
      return launch_nb<8>(xc, n, d, uc, su, ct, st, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace tq
