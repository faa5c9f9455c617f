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
// 8 .. 64 between lanes L and L ^ 1 .. L ^ 8 (DPP moves).  Each stage is the
// fp32 pair (a + b, a - b), a the lower index, spans increasing, then one
// multiply by fl32(1 / sqrt(128)) -- the order the fp32 oracle fixes, so X'
// is reproduced bit for bit.  The row is rotated twice (for the absmax, then
// for the codes), one chunk slot at a time in a loop with the next slot
// fetched ahead, which keeps the kernel body and its registers small.  The absmax of each subspace (position j = pinv[k] of rotated
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

// v from lane L ^ m (m = 1, 2, 4, 8) through DPP moves, no LDS: quad
// permutations, and for 4 and 8 the half-row / row mirror followed by one
__device__ __forceinline__ float xor_lane(float v, int m) {
  int x = __float_as_int(v);
  if (m == 1) {
    x = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, true);  // quad_perm [1, 0, 3, 2]
  } else if (m == 2) {
    x = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, true);  // quad_perm [2, 3, 0, 1]
  } else if (m == 4) {
    x = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, true);  // row_half_mirror: 7 - i
    x = __builtin_amdgcn_update_dpp(0, x, 0x1B, 0xF, 0xF, true);   // quad_perm [3, 2, 1, 0]
  } else {
    x = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, true);  // row_mirror: 15 - i
    x = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, true);  // row_half_mirror
  }
  return __int_as_float(x);
}

template <typename T>
__global__ __launch_bounds__(kRhtWaves * 64) void k_quant_rows_rht(const T* __restrict__ X, int n, int d, int dl,
                                                                  const uint8_t* __restrict__ sbits,
                                                                  const uint16_t* __restrict__ pinv,
                                                                  uint8_t* __restrict__ xl, float* __restrict__ sxl,
                                                                  uint8_t* __restrict__ xh, float* __restrict__ sxh) {
  __shared__ __attribute__((aligned(16))) uint8_t rowb[kRhtWaves][kRhtMaxD];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = blockIdx.x * kRhtWaves + w;
  if (row >= n) return;
  const int nch = d >> 3, dh = d - dl;
  const int slots = (nch + 63) >> 6;  // chunks per lane (the last slot may be partly past the row)
  const T* x = X + (size_t)row * d;

  // chunk slot i of this lane: raw values, sign bits, positions; fetched one
  // slot ahead of its use (clamped in-row addresses, so no branch)
  struct Chunk {
    Row8<T> raw;
    uint32_t sg;
    uint4 pv;
  };
  auto fetch = [&](int i, Chunk& c) {
    const int ch = min(lane + 64 * min(i, slots - 1), nch - 1);
    c.raw.load(x + 8 * ch);
    c.sg = sbits[ch];
    c.pv = *reinterpret_cast<const uint4*>(pinv + 8 * ch);
  };
  const float sc = (float)(1.0 / 11.313708498984760390);  // fl32(1 / sqrt(128))
  auto rotate = [&](const Chunk& c, float (&v)[8]) {
    c.raw.get(v);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(__float_as_uint(v[e]) ^ (((c.sg >> e) & 1u) << 31));
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)  // spans 1, 2, 4: inside the chunk
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (!(e & h)) {
          const float a = v[e], b = v[e + h];
          v[e] = a + b;
          v[e + h] = a - b;
        }
#pragma unroll
    for (int lm = 1; lm < 16; lm <<= 1) {  // spans 8 .. 64: between lanes L and L ^ lm
      // lower lane: v + p; upper lane: p - v = p + (-v) (the same IEEE
      // operation on the same operands): one add, its operand through DPP
      const uint32_t flip = (lane & lm) ? 0x80000000u : 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = xor_lane(v[e], lm) + __uint_as_float(__float_as_uint(v[e]) ^ flip);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] * sc;
  };
  auto position = [&](const uint4& pv, int e) {
    const uint32_t wv = e < 2 ? pv.x : (e < 4 ? pv.y : (e < 6 ? pv.z : pv.w));
    return min((int)((wv >> (16 * (e & 1))) & 0xFFFFu), d - 1);
  };

  // pass 1: the absmax of each subspace
  float ml = 0.0f, mh = 0.0f;
  Chunk cur, nxt;
  fetch(0, cur);
  for (int i = 0; i < slots; ++i) {
    fetch(i + 1, nxt);
    float v[8];
    rotate(cur, v);
    if (lane + 64 * i < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (position(cur.pv, e) < dl)
          ml = fmaxf(ml, fabsf(v[e]));
        else
          mh = fmaxf(mh, fabsf(v[e]));
      }
    }
    cur = nxt;
  }
  ml = wave_max(ml);
  mh = wave_max(mh);
  const RowScale rl = row_scale<4>(ml), rh = row_scale<8>(mh);
  if (lane == 0) {
    if (dl > 0) sxl[row] = rl.s;
    if (dh > 0) sxh[row] = rh.s;
  }
  // pass 2: the same rotation again (the row now comes from L2), codes to
  // their positions in LDS
  uint8_t* rb = rowb[w];
  fetch(0, cur);
  for (int i = 0; i < slots; ++i) {
    fetch(i + 1, nxt);
    float v[8];
    rotate(cur, v);
    if (lane + 64 * i < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = position(cur.pv, e);
        if (j < dl)  // 4-bit subspace: per 8 positions, the 4 even then the 4 odd
          rb[(j & ~7) + 4 * (j & 1) + ((j & 7) >> 1)] = (uint8_t)code_one<4>(v[e], rl);
        else
          rb[j] = (uint8_t)code_one<8>(v[e], rh);
      }
    }
    cur = nxt;
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS bytes are written
  __builtin_amdgcn_wave_barrier();
  for (int o = 16 * lane; o < dl; o += 1024)
    *reinterpret_cast<uint4*>(xl + (size_t)row * dl + o) = *reinterpret_cast<const uint4*>(rb + o);
  for (int o = 16 * lane; o < dh; o += 1024)
    *reinterpret_cast<uint4*>(xh + (size_t)row * dh + o) = *reinterpret_cast<const uint4*>(rb + dl + o);
}

// signs (fp32 +-1) -> one bit per coordinate (set: -1; bit e of byte ch is
// coordinate 8 ch + e); perm (position j -> rotated coordinate) -> its
// inverse (coordinate -> position), uint16
__global__ __launch_bounds__(256) void k_pack_rht(const float* __restrict__ signs, const int32_t* __restrict__ perm,
                                                  int d, uint8_t* __restrict__ sbits, uint16_t* __restrict__ pinv) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < d) {
    const int k = perm[j];
    if (k >= 0 && k < d) pinv[k] = (uint16_t)j;
  }
  if (j < d / 8) {
    uint32_t b = 0;
    for (int e = 0; e < 8; ++e) b |= (signs[8 * j + e] < 0.0f ? 1u : 0u) << e;
    sbits[j] = (uint8_t)b;
  }
}

template <typename T>
hipError_t launch_rht_t(const void* X, int n, int d, int dl, const void* rot, void* xl, float* sxl, void* xh,
                        float* sxh, hipStream_t st) {
  const uint8_t* sb = (const uint8_t*)rot;
  const uint16_t* pinv = (const uint16_t*)((const uint8_t*)rot + rht_signs_bytes(d));
  const dim3 grid((unsigned)((n + kRhtWaves - 1) / kRhtWaves)), block(kRhtWaves * 64);
  const T* x = (const T*)X;
  hipLaunchKernelGGL((k_quant_rows_rht<T>), grid, block, 0, st, x, n, d, dl, sb, pinv, (uint8_t*)xl, sxl, (uint8_t*)xh,
                     sxh);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_rht(const float* signs, const int32_t* perm, int d, void* rot, hipStream_t st) {
  hipLaunchKernelGGL(k_pack_rht, dim3((unsigned)((d + 255) / 256)), dim3(256), 0, st, signs, perm, d, (uint8_t*)rot,
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
