// Online randomised block-Hadamard rotation fused into the two-subspace
// quantiser: the layer takes unrotated X and quantises X' = X U with
// U = diag(signs) . blockdiag(H_128) / sqrt(128) . P (CoQuant notes, "CoQuant:
// Joint Weight-Activation Subspace Projection for Mixed-Precision LLMs", the
// rotation after Eq. 3 and the subspace split of Eq. 4-9; the randomised
// Hadamard transform of "Quantizing With Randomized Hadamard Transforms:
// Efficient Heuristic Now Proven").
//
// One wave per token row.  Lane L holds the 8-value chunks L + 64 i of the
// row, so the 16 chunks of a 128-column block sit in 16 consecutive lanes:
// the three butterfly stages of span 1, 2, 4 run inside a lane, those of span
// 8 .. 64 between lanes L and L ^ 1 .. L ^ 8.  Each stage is the fp32 pair
// (a + b, a - b), a the lower index, spans increasing, then one multiply by
// fl32(1 / sqrt(128)) -- the order the fp32 oracle fixes, so X' is reproduced
// bit for bit.  The absmax of each subspace (position j = pinv[k] of rotated
// coordinate k below d - d_hi, or not) comes from wave reductions; the codes
// are written byte by byte to a per-wave LDS row at their positions (4-bit
// subspace in the int8 order of the tile GEMM, 8-bit subspace in natural
// order) and copied out with 16-byte stores.

#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int kRhtBlock = 128;
constexpr int kRhtWaves = 4;

// One code with the fast reciprocal path of quant8_fast and its exact
// fallback (the same decision per element).
template <int BITS>
__device__ __forceinline__ int code_one(float x, const RowScale& rs) {
  if (rs.fast) {
    constexpr float MAGIC = 12582912.0f;  // 1.5 * 2^23
    const float t = __builtin_fmaf(x, rs.rcp, MAGIC);
    const float d = __builtin_fmaf(x, rs.rcp, -(t - MAGIC));
    if (!(fabsf(fabsf(d) - 0.5f) < QTraits<BITS>::NEAR)) return (int)(__float_as_uint(t) - 0x4B400000u);
  }
  return code_exact<BITS>(x, rs.s);
}

template <typename T, int CH>
__global__ __launch_bounds__(kRhtWaves * 64) void k_quant_rows_rht(const T* __restrict__ X, int n, int d, int dl,
                                                                  const int8_t* __restrict__ signs,
                                                                  const uint16_t* __restrict__ pinv,
                                                                  uint8_t* __restrict__ xl, float* __restrict__ sxl,
                                                                  uint8_t* __restrict__ xh, float* __restrict__ sxh) {
  __shared__ __attribute__((aligned(16))) uint8_t rowb[kRhtWaves][kRhtMaxD];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = blockIdx.x * kRhtWaves + w;
  if (row >= n) return;
  const int nch = d >> 3, dh = d - dl;
  const T* x = X + (size_t)row * d;

  float v[CH][8];
  uint4 pv[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int ch = min(lane + 64 * i, nch - 1);
    Row8<T> r;
    r.load(x + 8 * ch);
    const uint2 sg = *reinterpret_cast<const uint2*>(signs + 8 * ch);
    pv[i] = *reinterpret_cast<const uint4*>(pinv + 8 * ch);
    r.get(v[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sb = ((e < 4 ? sg.x : sg.y) >> (8 * (e & 3))) & 0x80u;  // sign bit of the int8 +-1
      v[i][e] = __uint_as_float(__float_as_uint(v[i][e]) ^ (sb << 24));   // x * +-1, exactly
    }
  }
  // butterflies of span 1, 2, 4 (inside the chunk), then 8 .. 64 (between lanes)
#pragma unroll
  for (int i = 0; i < CH; ++i) {
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!(e & h)) {
          const float a = v[i][e], b = v[i][e + h];
          v[i][e] = a + b;
          v[i][e + h] = a - b;
        }
  }
#pragma unroll
  for (int lm = 1; lm < 16; lm <<= 1) {
    const bool upper = lane & lm;
#pragma unroll
    for (int i = 0; i < CH; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __shfl_xor(v[i][e], lm, 64);
        v[i][e] = upper ? p - v[i][e] : v[i][e] + p;
      }
  }
  const float c = (float)(1.0 / 11.313708498984760390);  // fl32(1 / sqrt(128))
  float ml = 0.0f, mh = 0.0f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const bool live = lane + 64 * i < nch;
    const uint32_t pw[4] = {pv[i].x, pv[i].y, pv[i].z, pv[i].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[i][e] = v[i][e] * c;
      const int j = min((int)((pw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu), d - 1);
      const float a = live ? fabsf(v[i][e]) : 0.0f;
      if (j < dl)
        ml = fmaxf(ml, a);
      else
        mh = fmaxf(mh, a);
    }
  }
  ml = wave_max(ml);
  mh = wave_max(mh);
  const RowScale rl = row_scale<4>(ml), rh = row_scale<8>(mh);
  if (lane == 0) {
    if (dl > 0) sxl[row] = rl.s;
    if (dh > 0) sxh[row] = rh.s;
  }
  uint8_t* rb = rowb[w];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    if (lane + 64 * i >= nch) continue;
    const uint32_t pw[4] = {pv[i].x, pv[i].y, pv[i].z, pv[i].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = min((int)((pw[e >> 1] >> (16 * (e & 1))) & 0xFFFFu), d - 1);
      if (j < dl)  // 4-bit subspace: per 8 positions, the 4 even then the 4 odd
        rb[(j & ~7) + 4 * (j & 1) + ((j & 7) >> 1)] = (uint8_t)code_one<4>(v[i][e], rl);
      else
        rb[j] = (uint8_t)code_one<8>(v[i][e], rh);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS bytes are written
  __builtin_amdgcn_wave_barrier();
  for (int o = 16 * lane; o < dl; o += 1024)
    *reinterpret_cast<uint4*>(xl + (size_t)row * dl + o) = *reinterpret_cast<const uint4*>(rb + o);
  for (int o = 16 * lane; o < dh; o += 1024)
    *reinterpret_cast<uint4*>(xh + (size_t)row * dh + o) = *reinterpret_cast<const uint4*>(rb + dl + o);
}

// signs (fp32 +-1) -> int8 +-1; perm (position j -> rotated coordinate) ->
// its inverse (coordinate -> position), uint16
__global__ __launch_bounds__(256) void k_pack_rht(const float* __restrict__ signs, const int32_t* __restrict__ perm,
                                                  int d, int8_t* __restrict__ s8, uint16_t* __restrict__ pinv) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= d) return;
  s8[j] = signs[j] < 0.0f ? (int8_t)-1 : (int8_t)1;
  const int k = perm[j];
  if (k >= 0 && k < d) pinv[k] = (uint16_t)j;
}

template <typename T>
hipError_t launch_rht_t(const void* X, int n, int d, int dl, const void* rot, void* xl, float* sxl, void* xh,
                        float* sxh, hipStream_t st) {
  const int8_t* s8 = (const int8_t*)rot;
  const uint16_t* pinv = (const uint16_t*)((const uint8_t*)rot + rht_signs_bytes(d));
  const dim3 grid((unsigned)((n + kRhtWaves - 1) / kRhtWaves)), block(kRhtWaves * 64);
  const int nch = d / 8;
  const T* x = (const T*)X;
#define TQ_RHT(C)                                                                                                \
  hipLaunchKernelGGL((k_quant_rows_rht<T, C>), grid, block, 0, st, x, n, d, dl, s8, pinv, (uint8_t*)xl, sxl, \
                     (uint8_t*)xh, sxh)
  if (nch <= 64)
    TQ_RHT(1);
  else if (nch <= 128)
    TQ_RHT(2);
  else if (nch <= 256)
    TQ_RHT(4);
  else if (nch <= 512)
    TQ_RHT(8);
  else
    TQ_RHT(16);
#undef TQ_RHT
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_rht(const float* signs, const int32_t* perm, int d, void* rot, hipStream_t st) {
  hipLaunchKernelGGL(k_pack_rht, dim3((unsigned)((d + 255) / 256)), dim3(256), 0, st, signs, perm, d, (int8_t*)rot,
                     (uint16_t*)((uint8_t*)rot + rht_signs_bytes(d)));
  return hipGetLastError();
}

hipError_t launch_quant_rows_rht(const void* X, bool bf16, int n, int d, int dl, const void* rot, void* xl,
                                 float* sxl, void* xh, float* sxh, hipStream_t st) {
  if (d % kRhtBlock || d > kRhtMaxD || dl % 32 || (d - dl) % 16) return hipErrorInvalidValue;
  return bf16 ? launch_rht_t<bf16_t>(X, n, d, dl, rot, xl, sxl, xh, sxh, st)
              : launch_rht_t<float>(X, n, d, dl, rot, xl, sxl, xh, sxh, st);
}

}  // namespace tq
