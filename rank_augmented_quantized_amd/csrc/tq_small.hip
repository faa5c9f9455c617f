// One- or two-token rank-augmented layer (decode) in one launch.
//
// At decode sizes the layer is a stream over the INT4 weight codes; the
// activation quantisation and the first low-rank stage T = X L1 are small but
// sit on its critical path (TwinQuant notes, "TwinQuant: Learnable Subspace
// Decomposition for W4A4 LLM Quantization", section 04.C: the activations
// are quantised while the residual GEMM runs, and both components meet in one
// epilogue).  Here they share the grid with the weight stream:
//
//   blocks [0, nt)     fp32 partial of X L1 over k-chunk c for column group
//                      qg (producers);
//   blocks [nt, ...)   16 output channels each (consumers): issue the weight
//                      loads, quantise the (one or two) token rows themselves
//                      into LDS -- the rows are a few KB of L2-resident input,
//                      cheaper to re-read than to hand over -- run the integer
//                      product (v_mfma_i32_16x16x64_i8, exact), then wait for
//                      the producers, sum T (k-chunk partials in a fixed order,
//                      rounded to bf16), add T L2 (v_mfma_f32_16x16x32_bf16)
//                      and store Y.
//
// Producers are the lowest block indices, which are dispatched before any
// consumer, so a consumer only ever waits for blocks that already hold their
// resources; consumers wait only after their weight stream, by which time the
// producers are normally done.  The hand-off uses agent-scope atomic stores
// and loads (coherent across the XCDs' L2s without cache flushes) and one
// agent-scope counter of finished producers; consumers count themselves in
// sharded counters, and the last one resets everything for the next call.
// The wait is bounded: past the limit the consumer raises a flag in the
// workspace and carries on, so a broken hand-off cannot hang the GPU.

#include "tq_kernels.h"

namespace tq {

namespace {

__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent_u64(const void* p) {
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint4 ld_agent_u128(const void* p) {
  const uint64_t a = ld_agent_u64(p), b = ld_agent_u64(reinterpret_cast<const uint8_t*>(p) + 8);
  return uint4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
}

constexpr unsigned kSpinLimit = 1u << 18;  // well under a second of polling before giving up
// Hand-off words (uint32, in the workspace): [0] producers done, [2] wait-limit
// flag, [16] completed consumer shards, [32 + 16 s] consumers done in shard s.
// Consumers count themselves in kShards counters 64 bytes apart, so no single
// word takes one atomic per block.
constexpr int kShards = 32;
constexpr int kTop = 16, kShard0 = 32, kShardStride = 16;

}  // namespace

// Producer side: every thread's stores are complete, then one counter bump.
__device__ __forceinline__ void signal_done(unsigned* ctr) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// DBG: the test-hook instance, which also stores the exact int32 sums of the
// residual product to a.acc (n x m); its code is this template's, with those
// stores added.
template <typename T, int WAVES, int NR, bool DBG = false>
__global__ __launch_bounds__(WAVES * 64, (WAVES == 4) ? 4 : 2) void k_linear_small(SmallArgs a) {
  constexpr int NT = WAVES * 64;
  constexpr int U = (WAVES == 4) ? 8 : 16;  // 64-byte weight steps per wave per batch
  constexpr int UT = 4;                     // 32-k steps per wave per batch in the T role
  constexpr int CHX = (WAVES == 4) ? 2 : 8;  // most 8-value chunks of a row per thread
  constexpr int KB_MAX = CHX * NT * 4;       // most code bytes per row
  // LDS of a consumer: red | sT | sL | sPart | sX; of a producer: sP
  constexpr int RED_B = WAVES * 4 * 64 * 4;
  constexpr int ST_B = 16 * 256 * 2, SL_B = 16 * 256 * 2, SP_B = NT * 32, SX_B = 2 * KB_MAX;
  constexpr int C_B = RED_B + ST_B + SL_B + SP_B + SX_B + 64;
  constexpr int T_B = 16 * 65 * 4;
  constexpr int SMEM = C_B > T_B ? C_B : T_B;
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  const int nA = a.nt;
  const T* X = reinterpret_cast<const T*>(a.X);
  const int d = a.d, n = a.n;
  const int lr = lane & 15, lg = lane >> 4;

  // ---------------------------------------------------------------- T = X L1
  if (b < nA) {
    // block (c, qg): token rows 0..n-1, k-chunk c, columns 16 qs qg .. 16 qs (qg + 1) - 1
    float* sP = reinterpret_cast<float*>(smem);  // 16 x 65
    const int c = b / a.nqg, qg = b % a.nqg, qs = a.qs;
    const int s0 = c * (a.kc >> 5), s1 = min(d >> 5, s0 + (a.kc >> 5));
    const T* xr = X + (size_t)min(lr, n - 1) * d;
    const bf16_t* lp = a.L1t + (size_t)(16 * qg * qs + lr) * d;
    f32x4 acc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sb = s0 + wave; sb < s1; sb += WAVES * UT) {
      uint4 xa[UT], lb[UT][4];
#pragma unroll
      for (int u = 0; u < UT; ++u) {
        const int s = sb + WAVES * u;
        if (s < s1) {
          const int k = 32 * s + 8 * lg;
          float v[8];
          Load8<T>::load(xr + k, v, xa[u]);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q < qs) lb[u][q] = *reinterpret_cast<const uint4*>(lp + (size_t)16 * q * d + k);
        }
      }
#pragma unroll
      for (int u = 0; u < UT; ++u) {
        if (sb + WAVES * u < s1) {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (q < qs)
              acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[u]), as_bf16x8(lb[u][q]), acc[q], 0, 0, 0);
        }
      }
    }
    // waves' partials summed in wave order; 16x16 layout: lane l, element i -> row 4 (l / 16) + i, col l % 16
    for (int ww = 0; ww < WAVES; ++ww) {
      if (wave == ww) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (q < qs)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float& dst = sP[(4 * lg + i) * 65 + 16 * q + lr];
              dst = (ww == 0) ? acc[q][i] : dst + acc[q][i];
            }
      }
      __syncthreads();
    }
    const int cols = 16 * qs, col0 = 16 * qg * qs;
    for (int e = tid; e < n * cols; e += NT) {
      const int rr = e / cols, cc = e % cols;
      st_agent(a.P + ((size_t)c * n + rr) * a.ldt + col0 + cc, sP[rr * 65 + cc]);
    }
    signal_done(a.sync);
    return;
  }

  // ------------------------------------------------------------- consumers
  int* red = reinterpret_cast<int*>(smem);                                         // [WAVES][4][64]
  bf16_t* sT = reinterpret_cast<bf16_t*>(smem + RED_B);                            // 16 x rp
  bf16_t* sL = reinterpret_cast<bf16_t*>(smem + RED_B + ST_B);                     // 16 x rp
  float4* sPart = reinterpret_cast<float4*>(smem + RED_B + ST_B + SL_B);           // NT x 2
  uint8_t* sX = smem + RED_B + ST_B + SL_B + SP_B;                                 // n x Kb codes
  float* sRed = reinterpret_cast<float*>(smem + RED_B + ST_B + SL_B + SP_B + SX_B);  // WAVES maxima + 2 scales
  const int n0 = (b - nA) * 16;
  const int m = a.m, Kb = d >> 1;
  const uint8_t* bp = a.wc + (size_t)min(n0 + lr, m - 1) * Kb + 16 * lg;
  const int KS = (Kb + 63) / 64;
  const int per = (KS + WAVES - 1) / WAVES;
  const int sbeg = wave * per, send = min(KS, sbeg + per);
  const int rp = a.r_pad, rq = rp / 8;
  const int grp0 = group_of(a.groups, n0);
  const int toff = grp0 * rp;                           // this block's layer in the partials and T
  const bool tfirst = n0 == a.groups.start[grp0];      // first consumer of its layer writes T
  const int NP = n * rq;
  const int G = max(1, min(NT / max(NP, 1), max(a.nchunk, 1)));

  // Loads are unconditional, from clamped (always valid) addresses, and
  // masked where used: conditional loads become branches whose register
  // merges force early waits on every load in flight.
  const int kb_last = max(0, min((max(send, sbeg + 1) - 1) * 64, Kb - 16 - 16 * lg));
  uint4 bv[U];
  auto load_w = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      bv[u] = *reinterpret_cast<const uint4*>(bp + min((s0 + u) * 64, kb_last));
  };
  i32x4 acc = {0, 0, 0, 0};
  const uint8_t* xrow = sX + min(lr, n - 1) * Kb + 16 * lg;
  auto mma = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (s0 + u >= send) continue;
      const int kb = (s0 + u) * 64;
      const bool ok = kb + 16 * lg < Kb;  // this lane group's 16 bytes lie inside the row
      const uint4 xv = ok ? *reinterpret_cast<const uint4*>(xrow + kb) : uint4{0, 0, 0, 0};
      const uint4 w = ok ? bv[u] : uint4{0, 0, 0, 0};
      const i32x4 b0 = unpack16(w.x, w.y), b1 = unpack16(w.z, w.w);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16(xv.x, xv.y), b0, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16(xv.z, xv.w), b1, acc, 0, 0, 0);
    }
  };

  // 1. inputs: the token rows first (short L2 latency: their quantisation
  //    then overlaps the weight stream, memory counters being in order), the
  //    weight codes, scales and L2^T
  const int nch = d >> 3;
  Row8<T> r8[NR][CHX];  // NR = n: one or two token rows
#pragma unroll
  for (int i = 0; i < CHX; ++i) {
    const int ch = min(tid + NT * i, nch - 1);
#pragma unroll
    for (int row = 0; row < NR; ++row) r8[row][i].load(X + (size_t)row * d + 8 * ch);
  }
  load_w(sbeg);
  const float swv = a.sw[min(n0 + lr, m - 1)];
  uint4 lv;
  if (rp > 0) {
    const int el = min(tid, 16 * rq - 1);
    lv = *reinterpret_cast<const uint4*>(a.L2t + (size_t)min(n0 + el / rq, m - 1) * rp + 8 * (el % rq));
  }

  // 2. quantise the token rows into LDS (each consumer on its own: a row is a
  //    few KB of L2-resident input); the first consumer also writes s_x and
  //    the codes out
#pragma unroll
  for (int row = 0; row < NR; ++row) {
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < CHX; ++i) {
      if (tid + NT * i < nch) {
        float v[8];
        r8[row][i].get(v);
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[e]));
      }
    }
    mx = wave_max(mx);
    if (lane == 0) sRed[wave] = mx;
    __syncthreads();
    mx = 0.0f;
#pragma unroll
    for (int i = 0; i < WAVES; ++i) mx = fmaxf(mx, sRed[i]);
    const RowScale rs = row_scale<4>(mx);
    if (tid == 0) sRed[WAVES + row] = rs.s;
    const bool fast = __builtin_amdgcn_readfirstlane(rs.fast ? 1 : 0);
    uint32_t* cx = reinterpret_cast<uint32_t*>(sX + row * Kb);
#pragma unroll
    for (int i = 0; i < CHX; ++i) {
      const int ch = tid + NT * i;
      if (ch < nch) {
        float v[8];
        int q[8];
        r8[row][i].get(v);
        if (fast)
          quant8_fast<4>(v, rs, q);
        else
          quant8_exact<4>(v, rs.s, q);
        const uint32_t p = pack_nibbles(q);
        cx[ch] = p;
        if (b == nA) reinterpret_cast<uint32_t*>(a.xc + (size_t)row * Kb)[ch] = p;
      }
    }
    if (b == nA && tid == 0) a.sx[row] = rs.s;
    __syncthreads();  // sRed reused by the next row; codes visible to all waves
  }

  // 3. integer product
  mma(sbeg);
  for (int s0 = sbeg + U; s0 < send; s0 += U) {
    load_w(s0);
    mma(s0);
  }

  // 4. T from the producers: wait (normally already done), then the partials
  if (rp > 0) {
    if (tid == 0) {
      unsigned it = 0;
      while (__hip_atomic_load(a.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (unsigned)nA) {
        if (++it == kSpinLimit) {
          __hip_atomic_fetch_or(a.sync + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
    if (tid < 16 * rq) *reinterpret_cast<uint4*>(sL + tid * 8) = (n0 + tid / rq < m) ? lv : uint4{0, 0, 0, 0};
    for (int e = tid + NT; e < 16 * rq; e += NT) {
      const int cc = e / rq, q = e % rq;
      uint4 v = uint4{0, 0, 0, 0};
      if (n0 + cc < m) v = *reinterpret_cast<const uint4*>(a.L2t + (size_t)(n0 + cc) * rp + 8 * q);
      *reinterpret_cast<uint4*>(sL + e * 8) = v;
    }
    if (tid < NP * G) {
      // thread (piece pc, group grp): chunks grp and grp + G, in that order
      const int pc = tid % NP, grp = tid / NP;
      const int row = pc / rq, q = pc % rq;
      float4 t0 = float4{0.f, 0.f, 0.f, 0.f}, t1 = float4{0.f, 0.f, 0.f, 0.f};
      uint4 pv[2][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float* pp = a.P + ((size_t)min(grp + G * j, a.nchunk - 1) * n + row) * a.ldt + toff + 8 * q;
        pv[j][0] = ld_agent_u128(pp);
        pv[j][1] = ld_agent_u128(pp + 4);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        if (grp + G * j < a.nchunk) {
          t0.x += __uint_as_float(pv[j][0].x); t0.y += __uint_as_float(pv[j][0].y);
          t0.z += __uint_as_float(pv[j][0].z); t0.w += __uint_as_float(pv[j][0].w);
          t1.x += __uint_as_float(pv[j][1].x); t1.y += __uint_as_float(pv[j][1].y);
          t1.z += __uint_as_float(pv[j][1].z); t1.w += __uint_as_float(pv[j][1].w);
        }
      }
      sPart[2 * tid] = t0;
      sPart[2 * tid + 1] = t1;
    }
    __syncthreads();
    for (int pc = tid; pc < 16 * rq; pc += NT) {
      const int row = pc / rq, q = pc % rq;
      uint4 v = uint4{0, 0, 0, 0};
      if (row < n) {
        float t[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (pc < NT) {
          for (int gi = 0; gi < G; ++gi) {
            const float4 x0 = sPart[2 * (gi * NP + pc)], x1 = sPart[2 * (gi * NP + pc) + 1];
            t[0] += x0.x; t[1] += x0.y; t[2] += x0.z; t[3] += x0.w;
            t[4] += x1.x; t[5] += x1.y; t[6] += x1.z; t[7] += x1.w;
          }
        } else {  // pieces beyond the block's threads (G == 1): all chunks here
          for (int k = 0; k < a.nchunk; ++k) {
            const float* pp = a.P + ((size_t)k * n + row) * a.ldt + toff + 8 * q;
            const uint4 x0 = ld_agent_u128(pp), x1 = ld_agent_u128(pp + 4);
            t[0] += __uint_as_float(x0.x); t[1] += __uint_as_float(x0.y);
            t[2] += __uint_as_float(x0.z); t[3] += __uint_as_float(x0.w);
            t[4] += __uint_as_float(x1.x); t[5] += __uint_as_float(x1.y);
            t[6] += __uint_as_float(x1.z); t[7] += __uint_as_float(x1.w);
          }
        }
        v = uint4{pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3]), pack_bf16x2(t[4], t[5]), pack_bf16x2(t[6], t[7])};
        if (tfirst && a.Tout) *reinterpret_cast<uint4*>(a.Tout + (size_t)row * a.ldt + toff + 8 * q) = v;
      }
      *reinterpret_cast<uint4*>(sT + pc * 8) = v;
    }
  }

  // 5. waves' int32 partials summed in wave order; wave 0 finishes the tile
#pragma unroll
  for (int i = 0; i < 4; ++i) red[(wave * 4 + i) * 64 + lane] = acc[i];
  __syncthreads();
  if (wave == 0) {
    int s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int v = 0;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) v += red[(w * 4 + i) * 64 + lane];
      s[i] = v >> 8;  // int8 lanes carry 16 x code: 256 x the code product
    }
    f32x4 lrv = {0.f, 0.f, 0.f, 0.f};
    for (int t0 = 0; t0 < rp; t0 += 32) {
      const uint4 a8 = *reinterpret_cast<const uint4*>(sT + lr * rp + t0 + 8 * lg);
      const uint4 b8 = *reinterpret_cast<const uint4*>(sL + lr * rp + t0 + 8 * lg);
      lrv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a8), as_bf16x8(b8), lrv, 0, 0, 0);
    }
    const int col = n0 + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * lg + i;
      if (row >= n || col >= m) continue;
      if constexpr (DBG) a.acc[(size_t)row * m + col] = s[i];
      const float y = (float)s[i] * (sRed[WAVES + row] * swv) + lrv[i];
      if (a.y_bf16)
        reinterpret_cast<bf16_t*>(a.Y)[(size_t)row * m + col] = (bf16_t)f32_to_bf16_bits(y);
      else
        reinterpret_cast<float*>(a.Y)[(size_t)row * m + col] = y;
    }
  }

  // 6. the last consumer of the last shard to complete resets the counters
  //    for the next call (every consumer has passed its wait by then)
  if (nA > 0 && tid == 0) {
    const int nB = (int)gridDim.x - nA, cb = b - nA;
    const int sh = cb % kShards;
    const unsigned in_shard = (unsigned)(nB / kShards + (sh < nB % kShards ? 1 : 0));
    unsigned* shard = a.sync + kShard0 + kShardStride * sh;
    const unsigned done = __hip_atomic_fetch_add(shard, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == in_shard - 1) {
      __hip_atomic_store(shard, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned shards = (unsigned)min(nB, kShards);
      const unsigned top = __hip_atomic_fetch_add(a.sync + kTop, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (top == shards - 1) {
        __hip_atomic_store(a.sync + kTop, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.sync, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Plan and launch.
// ---------------------------------------------------------------------------
static int small_waves(int d) { return (d / 2 > 2048) ? 8 : 4; }

// The one-launch path pays off where a consumer is a light 4-wave block
// (d <= 4096): then the producers and all consumers share one dispatch round.
// With longer rows a consumer needs 8 waves and about 200 registers, one
// block per CU, and the producers push the grid into a second round; the
// two-launch path is faster there (measured on MI355X: 15.4 us against 20.3 us
// for d = 14336, m = 4096, n = 1).
bool small_fused_ok(int n, int d, int r_pad) {
  const int waves = small_waves(d);
  const int chx = waves == 4 ? 2 : 8;
  return waves == 4 && n >= 1 && n <= 2 && d % 32 == 0 && (d / 8) <= chx * waves * 64 && r_pad <= 256;
}

SmallPlan plan_small(int n, int d, int r_pad) {
  SmallPlan p{};
  const int steps = d / 32;
  const int nq = r_pad / 16;
  if (nq == 0) {
    p.qs = 1;
    p.nqg = 0;
    p.nchunk = 0;
    p.kc = d;
    p.nt = 0;
    return p;
  }
  p.qs = std::min(nq, 4);
  p.nqg = nq / p.qs;
  // chunks: at least 16 k-steps each, no more than the consumers sum in one pass
  const int nthr = small_waves(d) * 64;
  const int np = n * (r_pad / 8);
  const int max_chunks = 2 * std::max(1, nthr / std::max(np, 1));
  const int nch = std::max(1, std::min((steps + 15) / 16, max_chunks));
  const int chunk_steps = (steps + nch - 1) / nch;
  p.kc = 32 * chunk_steps;
  p.nchunk = (steps + chunk_steps - 1) / chunk_steps;
  p.nt = p.nchunk * p.nqg;
  return p;
}

template <typename T>
static hipError_t launch_small_t(const SmallArgs& a, hipStream_t st) {
  if (!small_fused_ok(a.n, a.d, a.r_pad)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(a.nt + (a.m + 15) / 16));
  if (a.acc) {  // the accumulator-export instance (test hook)
    if (a.n == 1)
      hipLaunchKernelGGL((k_linear_small<T, 4, 1, true>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((k_linear_small<T, 4, 2, true>), grid, dim3(256), 0, st, a);
  } else if (a.n == 1) {
    hipLaunchKernelGGL((k_linear_small<T, 4, 1>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((k_linear_small<T, 4, 2>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_linear_small(const SmallArgs& a, bool x_bf16, hipStream_t st) {
  return x_bf16 ? launch_small_t<bf16_t>(a, st) : launch_small_t<float>(a, st);
}

}  // namespace tq
