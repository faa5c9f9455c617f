// Device-side helpers shared by the kernels of the rank-augmented W4A4 layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t bf16_t;  // raw bf16 bits

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
// Two floats to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// 8 consecutive activations loaded from memory as fp32 values.
template <typename T>
struct Load8;

template <>
struct Load8<bf16_t> {
  // 16 bytes
  static __device__ __forceinline__ void load(const bf16_t* p, float (&v)[8], uint4& raw) {
    raw = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16_lo(raw.x); v[1] = bf16_hi(raw.x);
    v[2] = bf16_lo(raw.y); v[3] = bf16_hi(raw.y);
    v[4] = bf16_lo(raw.z); v[5] = bf16_hi(raw.z);
    v[6] = bf16_lo(raw.w); v[7] = bf16_hi(raw.w);
  }
};

template <>
struct Load8<float> {
  // 32 bytes; raw receives the values rounded to bf16 (ties to even)
  static __device__ __forceinline__ void load(const float* p, float (&v)[8], uint4& raw) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    raw.x = pack_bf16x2(v[0], v[1]);
    raw.y = pack_bf16x2(v[2], v[3]);
    raw.z = pack_bf16x2(v[4], v[5]);
    raw.w = pack_bf16x2(v[6], v[7]);
  }
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8 consecutive values of a row kept in registers in their input format.
template <typename T>
struct Row8;
template <>
struct Row8<bf16_t> {
  uint4 r;
  __device__ __forceinline__ void load(const bf16_t* p) { r = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void get(float (&v)[8]) const {
    v[0] = bf16_lo(r.x); v[1] = bf16_hi(r.x); v[2] = bf16_lo(r.y); v[3] = bf16_hi(r.y);
    v[4] = bf16_lo(r.z); v[5] = bf16_hi(r.z); v[6] = bf16_lo(r.w); v[7] = bf16_hi(r.w);
  }
  __device__ __forceinline__ uint4 bf16() const { return r; }  // the 8 values as bf16 (exact)
};
template <>
struct Row8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void get(float (&v)[8]) const {
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  __device__ __forceinline__ uint4 bf16() const {  // rounded to bf16, ties to even
    return uint4{pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w), pack_bf16x2(b.x, b.y), pack_bf16x2(b.z, b.w)};
  }
};

// ---------------------------------------------------------------------------
// Symmetric quantiser: s = fl32(amax / qmax), code = clamp(rne(fl32(x / s))).
//
// Fast path (s in [2^-125, 2^125]): with y = RN(1/s) and the exact product
// p = x * y (formed inside an FMA, never rounded on its own), and t = x / s
// real, |t| <= 7.0000005 (4 bits) or 127.00001 (8 bits) and
// |p - t| = |t| |y s - 1| <= |t| 2^-24, i.e. < 2^-21 (4 bits) or < 2^-17
// (8 bits), while |fl32(t) - t| <= ulp(t) / 2 <= 2^-22 (resp. 2^-18).
//   c = fma(x, y, 1.5 * 2^23) = RN(p + 1.5 * 2^23): its unit-spaced binade
//       rounds p to the nearest integer, ties to even; the low bits of c are
//       that integer in two's complement;
//   d = fma(x, y, -(c - 1.5 * 2^23)) = RN(p - rne(p)), |d| <= 1/2;
//   e = | |d| - 1/2 | estimates the distance of p to the nearest
//       half-integer within 2^-25.
// If e >= NEAR (2^-18, resp. 2^-14) then t and fl32(t) lie strictly inside
// the same interval between consecutive half-integers as p, so
// rne(p) == rne(fl32(x / s)); otherwise the codes are recomputed with the
// IEEE division.  In the fast path |rne(p)| <= qmax, so no clamp is needed;
// the exact path clamps (it matters only for subnormal scales).
// ---------------------------------------------------------------------------
template <int BITS>
struct QTraits;
template <>
struct QTraits<4> {
  static constexpr int QMAX = 7;
  static constexpr float NEAR = 0x1p-18f;
};
template <>
struct QTraits<8> {
  static constexpr int QMAX = 127;
  static constexpr float NEAR = 0x1p-14f;
};
// 3 and 6 bits (the 6/3-bit two-subspace layer), stored like 4 and 8 bits
template <>
struct QTraits<3> {
  static constexpr int QMAX = 3;
  static constexpr float NEAR = 0x1p-18f;
};
template <>
struct QTraits<6> {
  static constexpr int QMAX = 31;
  static constexpr float NEAR = 0x1p-14f;
};

struct RowScale {
  float s;
  float rcp;
  bool fast;
};

template <int BITS>
__device__ __forceinline__ RowScale row_scale(float amax) {
  RowScale r;
  r.s = amax / (float)QTraits<BITS>::QMAX;  // correctly rounded fp32 division
  r.fast = (r.s >= 0x1p-125f) && (r.s <= 0x1p+125f);
  r.rcp = r.fast ? 1.0f / r.s : 0.0f;
  return r;
}

template <int BITS>
__device__ __forceinline__ int code_exact(float x, float s) {
  if (!(s > 0.0f)) return 0;
  const float q = x / s;  // correctly rounded fp32 division
  const int c = (int)rintf(q);
  return min(max(c, -QTraits<BITS>::QMAX - 1), QTraits<BITS>::QMAX);
}

template <int BITS>
__device__ __forceinline__ void quant8_exact(const float (&x)[8], float s, int (&c)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = code_exact<BITS>(x[i], s);
}

template <int BITS>
__device__ __forceinline__ void quant8_fast(const float (&x)[8], const RowScale& rs, int (&c)[8]) {
  constexpr float MAGIC = 12582912.0f;  // 1.5 * 2^23
  bool near = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = __builtin_fmaf(x[i], rs.rcp, MAGIC);
    const float d = __builtin_fmaf(x[i], rs.rcp, -(t - MAGIC));
    const float e = fabsf(fabsf(d) - 0.5f);
    near |= (e < QTraits<BITS>::NEAR);
    c[i] = (int)(__float_as_uint(t) - 0x4B400000u);
  }
  if (__builtin_expect(near, 0)) quant8_exact<BITS>(x, rs.s, c);
}

// Codes of 8 values of one row; each int holds the code (two's complement).
template <int BITS>
__device__ __forceinline__ void quant8(const float (&x)[8], const RowScale& rs, int (&c)[8]) {
  if (rs.fast)
    quant8_fast<BITS>(x, rs, c);
  else
    quant8_exact<BITS>(x, rs.s, c);
}

// 8 codes -> 8 nibbles (even index low) in one dword.
__device__ __forceinline__ uint32_t pack_nibbles(const int (&c)[8]) {
  uint32_t p = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) p |= ((uint32_t)c[i] & 0xFu) << (4 * i);
  return p;
}
// 8 codes of k = 8 ch .. 8 ch + 7 of a 4-bit row, stored for the int8 tile
// GEMM: one int8 byte per code, the 4 even-k codes first, then the 4 odd-k
// codes (the order in which two packed weight dwords expand, unpack16); row
// is the start of the row (d bytes).
__device__ __forceinline__ uint2 codes_int8(const int (&c)[8]) {
  uint32_t e = 0, o = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e |= ((uint32_t)c[2 * i] & 0xFFu) << (8 * i);
    o |= ((uint32_t)c[2 * i + 1] & 0xFFu) << (8 * i);
  }
  return uint2{e, o};
}
__device__ __forceinline__ void store_codes_int8(uint8_t* row, int ch, const int (&c)[8]) {
  *reinterpret_cast<uint2*>(row + 8 * ch) = codes_int8(c);
}

// The 4-bit codes of 8 values of one row (the same codes as quant8<4>),
// returned as the 8 int8 bytes of store_codes_int8.  Fast path: the
// near-half-integer test of quant8_fast is folded into one running minimum,
// and each code's byte is the low byte of t = fma(x, y, 1.5 * 2^23), whose
// bits are bits(1.5 * 2^23) + code with zero low mantissa bits in the
// constant; v_perm_b32 gathers the 4 bytes of a dword.
template <int BITS = 4>
__device__ __forceinline__ uint2 quant8_int8(const float (&x)[8], const RowScale& rs) {
  static_assert(BITS <= 4, "codes of at most 4 bits");
  if (rs.fast) {
    constexpr float MAGIC = 12582912.0f;  // 1.5 * 2^23
    uint32_t t[8];
    float em = 1.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float tf = __builtin_fmaf(x[i], rs.rcp, MAGIC);
      const float d = __builtin_fmaf(x[i], rs.rcp, -(tf - MAGIC));
      em = fminf(em, fabsf(fabsf(d) - 0.5f));
      t[i] = __float_as_uint(tf);
    }
    if (__builtin_expect(!(em < QTraits<BITS>::NEAR), 1)) {
      // bytes [b0 of t0, t2, t4, t6] and [b0 of t1, t3, t5, t7]
      const uint32_t e = __builtin_amdgcn_perm(t[2], t[0], 0x0c0c0400u) | __builtin_amdgcn_perm(t[6], t[4], 0x04000c0cu);
      const uint32_t o = __builtin_amdgcn_perm(t[3], t[1], 0x0c0c0400u) | __builtin_amdgcn_perm(t[7], t[5], 0x04000c0cu);
      return uint2{e, o};
    }
  }
  int c[8];
  quant8_exact<BITS>(x, rs.s, c);
  return codes_int8(c);
}
// 8 codes -> 8 int8 bytes.
__device__ __forceinline__ uint2 pack_bytes(const int (&c)[8]) {
  uint2 p;
  p.x = ((uint32_t)c[0] & 0xFFu) | (((uint32_t)c[1] & 0xFFu) << 8) | (((uint32_t)c[2] & 0xFFu) << 16) |
        ((uint32_t)c[3] << 24);
  p.y = ((uint32_t)c[4] & 0xFFu) | (((uint32_t)c[5] & 0xFFu) << 8) | (((uint32_t)c[6] & 0xFFu) << 16) |
        ((uint32_t)c[7] << 24);
  return p;
}

// ---------------------------------------------------------------------------
// Direct HBM -> LDS loads (gfx950 buffer_load ... lds).
// ---------------------------------------------------------------------------
// Raw (stride 0) buffer resource over [base, base + bytes); loads at offsets
// at or past `bytes` return zeros.  Word 3 is the gfx9-family dword format.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)((uint32_t)(a >> 32) & 0xFFFFu);
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}
constexpr int kOutOfRange = (int)0x80000000;  // voffset that no buffer here reaches

// 16 bytes per lane from buffer offset voff + soff into LDS at lds + 16 x lane
// (buffer_load_dwordx4 ... lds, LDS base in M0).  Written as asm so that the
// compiler does not track it: its own tracking would wait for every
// outstanding direct load before any LDS read.  Completion is waited for
// explicitly (wait_vmcnt); the data goes to LDS, so no VGPR is written.
__device__ __forceinline__ void load_lds16(i32x4 rsrc, uint32_t lds, int voff, int soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "m0");
}
// load_lds16 at agent scope (sc1: past the XCD's L2), for words that other
// blocks write during the launch
__device__ __forceinline__ void load_lds16_sc1(i32x4 rsrc, uint32_t lds, int voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen sc1 lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}
// 4 bytes per lane into LDS at lds + 4 x lane; sc1: read at agent scope (past
// the XCD's L2), for words that other blocks or earlier launches write
__device__ __forceinline__ void load_lds4_sc1(i32x4 rsrc, uint32_t lds, int voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dword %1, %2, 0 offen sc1 lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}
__device__ __forceinline__ void load_lds4(i32x4 rsrc, uint32_t lds, int voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}
// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------------------
// INT4 -> INT8 for the int8 MFMA: the nibble of every byte is moved to the
// byte's high half, so each int8 lane holds 16 * code exactly.  Both operands
// are scaled the same way, so products carry a factor 256 that the epilogue
// removes with an exact arithmetic shift (|acc| <= 256 * 64 * K < 2^31 for
// K <= 2^17).  lo gets the even-index codes, hi the odd-index codes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t nib_lo(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t nib_hi(uint32_t w) { return w & 0xF0F0F0F0u; }

// Two packed dwords (16 codes) -> one int8 MFMA operand of 16 lanes.
__device__ __forceinline__ i32x4 unpack16(uint32_t w0, uint32_t w1) {
  i32x4 r;
  r[0] = (int)nib_lo(w0);
  r[1] = (int)nib_hi(w0);
  r[2] = (int)nib_lo(w1);
  r[3] = (int)nib_hi(w1);
  return r;
}

// Maximum of non-negative floats over the 64 lanes of a wave, returned in
// every lane.  Non-negative floats order like their bit patterns as signed
// ints.  DPP steps inside each 16-lane row (swap neighbours, swap pairs,
// mirror half-rows, mirror rows) leave the row maximum in every lane of the
// row; the four row maxima are then read as scalars.
__device__ __forceinline__ float wave_max(float v) {
  int x = __float_as_int(v);
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  x = max(x, __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false));  // row_mirror
  const int m = max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
                    max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
  return __int_as_float(m);
}

// One token row (nch chunks of 8 values, chunk lane + 64 i in slot i) quantised
// at 4 bits by one wave with the whole row in registers: the codes go to
// `codes` as int8 in the tile GEMM's order (PK: nibble-packed, even k in the
// low nibble, d / 2 bytes) and, when `copy` is not null, to `copy` as int8
// in the tile GEMM's order; returns s_x.
template <typename T, int CH, bool PK = false>
__device__ __forceinline__ float quant_row_i8_wave(const T* x, int nch, int lane, uint8_t* codes, uint8_t* copy) {
  Row8<T> r[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int ch = lane + 64 * i;
    if (ch < nch) r[i].load(x + 8 * ch);
  }
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
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int ch = lane + 64 * i;
    if (ch < nch) {
      float v[8];
      r[i].get(v);
      const uint2 c = quant8_int8(v, rs);
      if constexpr (PK)  // byte j: code 2 j (even k, low nibble) and code 2 j + 1
        *reinterpret_cast<uint32_t*>(codes + 4 * ch) = (c.x & 0x0F0F0F0Fu) | ((c.y & 0x0F0F0F0Fu) << 4);
      else
        *reinterpret_cast<uint2*>(codes + 8 * ch) = c;
      if (copy) *reinterpret_cast<uint2*>(copy + 8 * ch) = c;
    }
  }
  return rs.s;
}

// ---------------------------------------------------------------------------
// Per-token asymmetric quantisation (CoQuant Eq. 1 with a zero-point): the
// row's z = min and s = fl32(fl32(max - min) / (2^N - 1)); the code of x is
// u = rne(fl32(fl32(x - z) / s)) in [0, 2^N - 1], returned as u - 2^(N-1).
// ---------------------------------------------------------------------------
// Maximum of any floats over the 64 lanes (DPP inside rows, then the four
// row results as scalars).
template <int CTRL>
__device__ __forceinline__ float dpp_fmax(float x) {
  const int y = __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF, 0xF, false);
  return fmaxf(x, __int_as_float(y));
}
__device__ __forceinline__ float wave_fmax(float v) {
  v = dpp_fmax<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_fmax<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_fmax<0x141>(v);  // row_half_mirror
  v = dpp_fmax<0x140>(v);  // row_mirror
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float e = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, e));
}

struct AsymScale {
  float s, z, rcp;
  bool fast;
};

template <int BITS>
__device__ __forceinline__ AsymScale asym_scale(float mn, float mx) {
  AsymScale a;
  a.z = mn;
  a.s = (mx - mn) / (float)((1 << BITS) - 1);  // correctly rounded fp32 subtraction and division
  a.fast = (a.s >= 0x1p-125f) && (a.s <= 0x1p+125f);
  a.rcp = a.fast ? 1.0f / a.s : 0.0f;
  return a;
}

// u - 2^(N-1) for v = fl32(x - z): the fast path rounds v * fl32(1 / s) with
// the magic-number add and falls back to the IEEE division when the
// product lies within NEAR of a half-integer (|v / s| <= 2^N - 1, so the
// product's error stays far below NEAR: the same decision as the division).
template <int BITS>
__device__ __forceinline__ int code_asym(float v, const AsymScale& a) {
  constexpr int QM = (1 << BITS) - 1, OFF = 1 << (BITS - 1);
  if (a.fast) {
    constexpr float MAGIC = 12582912.0f;  // 1.5 * 2^23
    const float t = __builtin_fmaf(v, a.rcp, MAGIC);
    const float dd = __builtin_fmaf(v, a.rcp, -(t - MAGIC));
    if (!(fabsf(fabsf(dd) - 0.5f) < QTraits<BITS>::NEAR))
      return min((int)(__float_as_uint(t) - 0x4B400000u), QM) - OFF;
  }
  if (!(a.s > 0.0f)) return -OFF;
  return min(max((int)rintf(v / a.s), 0), QM) - OFF;
}

}  // namespace tq
