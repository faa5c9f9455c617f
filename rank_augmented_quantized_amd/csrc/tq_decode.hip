// Few-token layer (decode: one or two tokens) in one launch: the per-token
// quantiser, the first low-rank stage T = X L1, the stream over the INT4
// weight codes with its exact integer product, and the shared epilogue
// (dequantisation, T L2, one store of Y) share one grid (TwinQuant notes,
// "TwinQuant: Learnable Subspace Decomposition for W4A4 LLM Quantization",
// section 04.C: the activations are quantised while the residual GEMM runs,
// and both components meet in one epilogue).
//
// At these sizes the call is a stream of the weight codes (m x d / 2 bytes)
// from HBM; everything else must stay off its path.  Blocks have 7 stream
// waves and one control wave.
//
//  * Blocks [0, nt) each compute one fp32 partial of T (16 columns of T over
//    a 512-k chunk) on v_mfma_f32_16x16x32_bf16 and store it as tagged words
//    (below).  They stream no weights, so their few loads are not queued
//    behind the weight stream.
//  * Every other block owns gpb (1 .. 4) groups of 16 output channels, about
//    112 .. 128 steps of 64 bytes of weight codes, so that there is about one
//    such block per CU at the layer shapes of interest: the token rows are
//    loaded and quantised once per CU, and no block's early phase waits
//    behind another block's weight stream.  It loads the rows (direct HBM to
//    LDS), quantises them (absmax over the block), and only then issues the
//    weight loads -- every step of 64 bytes a 16-byte load per lane, the
//    block's steps split evenly between the stream waves -- and runs the
//    exact integer product on v_mfma_i32_16x16x64_i8 as they arrive, adding
//    it to the groups' sums in LDS (exact integer additions, so the order in
//    which the waves add does not matter).  Issued any earlier, the weights
//    queue ahead of everything the block still has to fetch and the early
//    phase stretches over the whole stream.
//  * Its control wave loads the channels' scales and rows of L2^T at the
//    start and the partials of T as the weights are issued, sums them in
//    chunk order (fixed: every call gives the same bits) and forms T L2 of
//    every group, then releases the groups' stores.
//  * The last stream wave to add to a group stores its Y = s_x s_w acc +
//    T L2 (no barrier after the stream: the other waves may still be
//    streaming).
//
// Hand-off.  Memory latency, not bandwidth, bounds every cross-block step
// here (a load, a write-through store or an atomic each take the order of a
// microsecond while the weight stream saturates HBM), so partials cross
// blocks in one step: they are stored as 64-bit words {value, tag}, the tag
// being this call's epoch, and the consumers read the words themselves, with
// no separate counter.  The epoch is a word of the workspace that every
// block reads at its start; the last channel block to finish (a counter)
// advances it, after every block of the call has read it (a channel block
// finishes only after the partials it reads were stored, and their blocks
// read the epoch before storing them; every layer has channel blocks).
// Every load and store of a hand-off word is performed at agent scope, at
// the device's point of coherence past the XCDs' separate L2s, so a word
// that carries the expected tag was written by this call and holds its
// value.
//
// Waits are bounded.  A block whose wait reaches the limit sets a flag word
// (sticky), writes NaN to its outputs and finishes; a later call that finds
// the flag set writes NaN everywhere until the workspace is zero-filled again.

#include "tq_kernels.h"

namespace tq {
namespace {

// hand-off words of the sync region (uint32 indices, 64 bytes apart): the
// epoch, the finished channel blocks' counter, the wait-limit flag
constexpr int kWEpoch = 0, kWCons = 16, kWFlag = 32;
constexpr int kSW = 7, kNW = kSW + 1, kNT = kNW * 64;  // stream waves, waves, threads per block
constexpr int kU = 19;    // most 64-byte weight steps per stream wave (7 x 19 >= 128 steps of a 16384-code row)
constexpr int kGmax = 4;  // most 16-channel groups per channel block

__device__ __forceinline__ uint32_t ld32(const unsigned* p) {
  return __hip_atomic_load(const_cast<unsigned*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st32(unsigned* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld64(const void* p) {
  return __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st64(void* p, uint64_t v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t tag_word(float v, uint32_t tag) {
  return (uint64_t)__float_as_uint(v) | ((uint64_t)tag << 32);
}
// Workgroup barrier without the fences of __syncthreads (which would wait for
// the stream waves' outstanding weight loads); a wave that wrote LDS for
// others first waits for its LDS operations (lds_done).
__device__ __forceinline__ void bar() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void lds_done() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)

// ---------------------------------------------------------------------------
// The kernel.  NR: token rows (1 or 2); DBG: the test-hook instance that also
// stores the exact int32 sums to a.acc; HP: the control wave runs at raised
// priority (chosen by the launcher for T of 16 or more chunks).
// ---------------------------------------------------------------------------
template <typename T, int NR, bool DBG, bool HP>
__global__ __launch_bounds__(kNT) void k_decode(DecodeArgs a) {
  constexpr int SW = kSW, NW = kNW, NT = kNT, U = kU;
  constexpr int CHX = (kDecodeMaxD / 8 + NT - 1) / NT;  // 8-value chunks per thread per row
  constexpr int UP = kDecodeSteps;                      // 32-k steps per wave of a T partial
  constexpr int LS = UP * NW * 64;                      // bytes of a chunk's k range in one row of L1^T
  static_assert(LS == 1024, "one row of L1^T per direct-load instruction");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x;
  const int d = a.d, n = a.n, m = a.m, Kb = d >> 1, nch = d >> 3;
  const int l16 = lane & 15, lg = lane >> 4;
  const bool prod = b < a.nt;  // blocks [0, nt) compute one partial of T each
  const bool cons = !prod;     // the others own G groups of 16 output channels
  const int G = a.gpb, S = (Kb + 63) >> 6;  // S: 64-byte steps of a weight row
  const int c0 = prod ? 0 : 16 * G * (b - a.nt);
  const int rp = a.r_pad;
  const int grp = group_of(a.groups, min(c0, m - 1)), toff = grp * rp;
  const bool tfirst = cons && c0 == a.groups.start[grp];  // the first block of its layer writes T out
  // stream items i = g S + s (group g, step s); stream wave w takes [ib, ie),
  // which reach at most groups gf and gf + 1 (per <= S as G <= 4 < 7)
  const int items = G * S, per = (items + SW - 1) / SW;
  const int ib = min(wave, SW - 1) * per, ie = min(items, ib + per);
  const int gf = ib / S;

  // LDS.  Region A (lds_a bytes) holds, in a channel block, the token rows
  // as they arrive (sXr: row i at i XR, XR = the row's bytes rounded up to
  // 1 KB); in a partial block, the rows' 512-k chunk of the partial (sXr:
  // row i at i XR, XR = 512 values) and its 16 rows of L1^T (sL1: [16][LS]).  Then sW [n r_pad nchunk]
  // (the layer's 64-bit hand-off words, a whole number of KB) | sL [16 G][rp]
  // bf16 (the block's rows of L2^T, SL bytes) | sSw [64] | sSync [64] (the
  // hand-off words) | red [4][4][64] int (the groups' integer sums) |
  // sLR [4][4][64] fp32 (the groups' T L2) | sT [16][rp] bf16 |
  // sP [NW][16][17] fp32 | sX [NR][Kb] codes | sSx [16] | sRed [NR][NW] |
  // sCtl [4] | sCnt [4] (stream waves done per group).
  const int xrow = d * (int)sizeof(T), XS = (xrow + 1023) & ~1023;
  const int XR = prod ? 512 * (int)sizeof(T) : XS;
  const int ne = n * rp, nck = a.nchunk, nwords = ne * nck;  // the layer's hand-off words
  const int SWB = (8 * nwords + 1023) & ~1023, SL = rp ? (32 * G * rp + 1023) & ~1023 : 0;
  const int oW = a.lds_a, oL = oW + SWB, oSw = oL + SL, oSync = oSw + 256, oRed = oSync + 256;
  uint8_t* sXr = lds;
  const uint8_t* sL1 = lds + NR * XR;
  uint64_t* sW = reinterpret_cast<uint64_t*>(lds + oW);
  const bf16_t* sL = reinterpret_cast<const bf16_t*>(lds + oL);
  const float* sSw = reinterpret_cast<const float*>(lds + oSw);
  const unsigned* sSync = reinterpret_cast<const unsigned*>(lds + oSync);
  int* red = reinterpret_cast<int*>(lds + oRed);
  float* sLR = reinterpret_cast<float*>(lds + oRed + 4096);
  bf16_t* sT = reinterpret_cast<bf16_t*>(lds + oRed + 8192);
  float* sP = reinterpret_cast<float*>(lds + oRed + 8192 + 32 * rp);
  uint8_t* sX = reinterpret_cast<uint8_t*>(sP + NW * 16 * 17);
  float* sSx = reinterpret_cast<float*>(sX + NR * Kb);
  float* sRed = sSx + 16;
  unsigned* sCtl = reinterpret_cast<unsigned*>(sRed + 16);  // [0] failed wait, [1] epoch, [2] sLR ready
  unsigned* sCnt = sCtl + 4;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;

  // 1. Early loads, all direct HBM -> LDS.  The stream waves issue, 1 KB a
  //    wave-instruction (instruction j of the list to stream wave j mod SW):
  //    the hand-off words (wave 0, first), then the token rows (in a partial
  //    block only their chunk of the partial) and in the partial blocks the
  //    16 rows of L1^T of their partial (columns 16 q .. 16 q + 15 of T over
  //    the 32-k steps [c kcs, (c + 1) kcs) of chunk c).  The control wave of a channel block loads the channels'
  //    scales and rows of L2^T (rows past m read as zeros), which only the
  //    epilogue uses.
  const int pc = prod ? b / a.nqg : 0, pq = prod ? b % a.nqg : 0;  // chunk, 16-column group
  const int ps0 = pc * a.kcs, ps1 = min(d >> 5, ps0 + a.kcs);
  if (wave < SW) {
    if (wave == 0) load_lds4_sc1(buffer_rsrc(a.sync, kSyncBytes), lds0 + oSync, 4 * lane);
    const int xi = XR >> 10, nxi = NR * xi;  // instructions of the token rows
    const int nli = prod ? 16 : 0;           // of the L1^T rows
    const int kx0 = prod ? 32 * ps0 * (int)sizeof(T) : 0;  // first byte of a row loaded
    const i32x4 rX = buffer_rsrc(a.X, (uint32_t)(n * xrow));
    const i32x4 rL = buffer_rsrc(a.L1t, (uint32_t)((size_t)a.ldt * d * 2));
    for (int j = wave; j < nxi + nli; j += SW) {
      if (j < nxi) {
        const int row = NR == 2 && j >= xi ? 1 : 0, off = kx0 + 1024 * (j - row * xi) + 16 * lane;
        load_lds16(rX, lds0 + 1024 * j, off < xrow ? row * xrow + off : kOutOfRange, 0);
      } else {
        const int row = j - nxi, kb = 16 * lane;  // kb: byte in the chunk
        const bool ok = 64 * ps0 + kb < 2 * d;
        load_lds16(rL, lds0 + NR * XR + 1024 * row, ok ? (16 * pq + row) * 2 * d + 64 * ps0 + kb : kOutOfRange, 0);
      }
    }
    wait_vmcnt<0>();
  } else if (cons) {
    load_lds4(buffer_rsrc(a.sw, (uint32_t)(4 * m)), lds0 + oSw,
              lane < 16 * G && c0 + lane < m ? 4 * (c0 + lane) : kOutOfRange);
    if (rp) {
      const i32x4 r2 = buffer_rsrc(a.L2t, (uint32_t)((size_t)m * rp * 2));
      const int base = c0 * rp * 2;  // the block's rows of L2^T are contiguous
      for (int j = 0; j < SL / 1024; ++j) {
        const int off = 1024 * j + 16 * lane;
        load_lds16(r2, lds0 + oL + 1024 * j, off < 32 * G * rp ? base + off : kOutOfRange, 0);
      }
    }
  }
  bar();  // hand-off words, token rows and L1^T rows in LDS

  // 2. channel blocks: the rows' absmax over every thread's chunks; partial
  //    blocks: their MFMA terms of this wave (32-k steps c kcs + wave + NW u;
  //    A: token rows 0 .. 15, rows >= n repeating the last, whose results
  //    are dropped)
  if (cons) {
#pragma unroll
    for (int row = 0; row < NR; ++row) {
      const T* xr = reinterpret_cast<const T*>(sXr + row * XS);
      float mx = 0.0f;
#pragma unroll
      for (int i = 0; i < CHX; ++i) {
        if (tid + NT * i < nch) {
          Row8<T> r8;
          float v[8];
          r8.load(xr + 8 * (tid + NT * i));
          r8.get(v);
#pragma unroll
          for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[e]));
        }
      }
      mx = wave_max(mx);
      if (lane == 0) sRed[row * NW + wave] = mx;
    }
  } else {
    const T* xr = reinterpret_cast<const T*>(sXr + min(l16, n - 1) * XR);
    f32x4 pacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < UP; ++u) {
      const int ls = wave + NW * u;
      if (ps0 + ls < ps1) {
        Row8<T> r8;
        r8.load(xr + 32 * ls + 8 * lg);  // the chunk starts at k = 32 ps0
        const uint4 lb = *reinterpret_cast<const uint4*>(sL1 + l16 * LS + 64 * ls + 16 * lg);
        pacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(r8.bf16()), as_bf16x8(lb), pacc, 0, 0, 0);
      }
    }
    // 16x16 result layout: lane l, element i -> row 4 (l / 16) + i, column l % 16
#pragma unroll
    for (int i = 0; i < 4; ++i) sP[(wave * 16 + 4 * lg + i) * 17 + l16] = pacc[i];
  }
  lds_done();
  bar();  // maxima or the partial's wave terms in LDS

  // 3. control wave: the call's words to LDS; a partial block sums its
  //    partial in wave order and stores it as tagged words {value, tag}:
  //    element (row, column g r_pad + j) of chunk c at word
  //    (g n r_pad + row r_pad + j) nchunk + c, so that a layer's words are
  //    contiguous and an element's chunks adjacent
  if (wave == SW) {
    const uint32_t epoch = sSync[kWEpoch];
    if (lane == 0) {
      sCtl[0] = sSync[kWFlag] != 0 ? 1u : 0u;  // a wait of an earlier call gave up
      sCtl[1] = epoch;
      sCtl[2] = 0u;
    }
    if (cons) {  // the groups' sums and counters start at zero
      for (int j = 0; j < 4 * G; ++j) red[j * 64 + lane] = 0;
      if (lane < 4) sCnt[lane] = 0u;
    }
    if (prod && lane < 16 * n) {
      const uint32_t tag = epoch + 1 - (a.silent ? 1u : 0u);
      const int row = lane >> 4, j16 = lane & 15, col = 16 * pq + j16;
      float v = sP[row * 17 + j16];
#pragma unroll
      for (int w = 1; w < NW; ++w) v += sP[(w * 16 + row) * 17 + j16];
      const int g = col >> a.lrp, j = col & (rp - 1);
      st64(reinterpret_cast<uint64_t*>(a.P) + (((size_t)g * n + row) * rp + j) * a.nchunk + pc, tag_word(v, tag));
    }
    wait_vmcnt<0>();  // a channel block's scales and L2^T rows are in LDS
  }
  if (prod) return;

  // 4. codes of the rows to sX (the first channel block also writes them out)
#pragma unroll
  for (int row = 0; row < NR; ++row) {
    float mx = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, sRed[row * NW + w]);
    const RowScale rs = row_scale<4>(mx);
    if (tid == 0) sSx[row] = rs.s;
    const T* xr = reinterpret_cast<const T*>(sXr + row * XS);
    uint32_t* cx = reinterpret_cast<uint32_t*>(sX + row * Kb);
#pragma unroll
    for (int i = 0; i < CHX; ++i) {
      const int ch = tid + NT * i;
      if (ch < nch) {
        Row8<T> r8;
        float v[8];
        int c8[8];
        r8.load(xr + 8 * ch);
        r8.get(v);
        quant8<4>(v, rs, c8);
        const uint32_t p = pack_nibbles(c8);
        cx[ch] = p;
        if (b == a.nt) reinterpret_cast<uint32_t*>(a.xc + (size_t)row * Kb)[ch] = p;
      }
    }
    if (b == a.nt && tid == 0) a.sx[row] = rs.s;
  }
  lds_done();
  bar();  // codes and scales in LDS; region A free

  // 5. Stream waves: the weight codes of items [ib, ie) (lane: channel
  //    l % 16 of the item's group, bytes 16 (l / 16) of its 64-byte step;
  //    loads past ie repeat the last item and are not used), the exact
  //    integer product, and its addition to the groups' sums in LDS (integer
  //    additions: any order gives the same bits).  The last stream wave to
  //    add to a group stores the group's Y (no barrier: every other wave may
  //    still be streaming).
  //    Control wave: the layer's partials of T, T, and T L2 of every group.
  const uint64_t* lay = reinterpret_cast<const uint64_t*>(a.P) + (size_t)grp * nwords;
  if (wave < SW) {
    if (ib >= ie) return;  // no items (tiny rows)
    i32x4 bv[U];
    const int ilast = ie - 1;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = min(ib + u, ilast);
      const int hi = i >= (gf + 1) * S ? 1 : 0;
      const int s = i - (gf + hi) * S;
      const int ch = min(c0 + 16 * (gf + hi) + l16, m - 1);
      const int kb = min(64 * s + 16 * lg, Kb - 16);
      bv[u] = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(a.wc + (size_t)ch * Kb + kb));
    }
    // one running sum, moved to acc0 where the items cross into group gf + 1
    // (local item ub)
    i32x4 acc = {0, 0, 0, 0}, acc0 = {0, 0, 0, 0};
    const int ub = (gf + 1) * S - ib;
    const uint8_t* xrow = sX + min(l16, n - 1) * Kb + 16 * lg;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ib + u >= ie) continue;
      if (u == ub) {
        acc0 = acc;
        acc = i32x4{0, 0, 0, 0};
      }
      const int s = ib + u - (u < ub ? gf : gf + 1) * S;
      const bool ok = 64 * s + 16 * lg < Kb;  // this lane group's 16 bytes lie inside the row
      const uint4 xv = ok ? *reinterpret_cast<const uint4*>(xrow + 64 * s) : uint4{0, 0, 0, 0};
      const i32x4 w = ok ? bv[u] : i32x4{0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16(xv.x, xv.y), unpack16((uint32_t)w[0], (uint32_t)w[1]), acc,
                                                  0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(unpack16(xv.z, xv.w), unpack16((uint32_t)w[2], (uint32_t)w[3]), acc,
                                                  0, 0, 0);
    }
    const bool two = ub < ie - ib;  // the items reach group gf + 1
    if (two) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __hip_atomic_fetch_add(&red[(gf * 4 + i) * 64 + lane], acc0[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_add(&red[((gf + 1) * 4 + i) * 64 + lane], acc[i], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        __hip_atomic_fetch_add(&red[(gf * 4 + i) * 64 + lane], acc[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    lds_done();  // this wave's additions are done before it counts itself in
    for (int g = gf; g <= gf + (two ? 1 : 0); ++g) {
      const int w0 = (g * S) / per, w1 = min(SW - 1, ((g + 1) * S - 1) / per);  // the waves adding to group g
      unsigned prev = 0;
      if (lane == 0) prev = __hip_atomic_fetch_add(&sCnt[g], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if (__builtin_amdgcn_readfirstlane(prev) != (unsigned)(w1 - w0)) continue;
      // the last wave of group g: wait until the control wave has T L2 (its
      // own waits are bounded, and it always sets the word), then store Y
      while (__hip_atomic_load(&sCtl[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0u)
        __builtin_amdgcn_s_sleep(2);
      const bool bad = sCtl[0] != 0;
      const int col = c0 + 16 * g + l16;
      const float swv = sSw[16 * g + l16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * lg + i;
        const int sum = red[(g * 4 + i) * 64 + lane] >> 8;  // both operands carry 16 x code: 256 x the code product
        if (row >= n || col >= m) continue;
        if constexpr (DBG) a.acc[(size_t)row * m + col] = sum;
        const float y = bad ? __builtin_nanf("") : (float)sum * (sSx[row] * swv) + sLR[(g * 4 + i) * 64 + lane];
        if (a.y_bf16)
          reinterpret_cast<bf16_t*>(a.Y)[(size_t)row * m + col] = (bf16_t)f32_to_bf16_bits(y);
        else
          reinterpret_cast<float*>(a.Y)[(size_t)row * m + col] = y;
      }
    }
    return;
  }

  // control wave.  Its T check, chunk sum and T L2 sit on the path to every
  // store of Y; with many chunks (long rows: 28 at d = 14336) they take long
  // enough that its instructions go first (the stream waves mostly wait on
  // memory meanwhile): 17.2 -> 15.3 us at d = 14336, while at 8 chunks
  // (d = 4096) the raised priority costs 0.5 us, so it stays at the default.
  if constexpr (HP) __builtin_amdgcn_s_setprio(3);
  if (rp > 0) {
    // T rows 0 .. n - 1 of this layer, element e = (row e / rp, column e % rp):
    // the layer's nchunk words per element are contiguous.  One batch of
    // direct loads brings them all to sW as the weight stream starts;
    // normally every partial was stored long before (the partial blocks
    // stream no weights) and every tag matches.  Otherwise poll one word per
    // partial block of this layer (chunk c, column group q: its element
    // (0, 16 q)) until all carry the tag, and read the words again.
    const uint32_t tag = sCtl[1] + 1;
    {
      const i32x4 rP = buffer_rsrc(lay, (uint32_t)(8 * nwords));
      for (int j = 0; j < SWB >> 10; ++j) {
        const int off = 1024 * j + 16 * lane;
        load_lds16_sc1(rP, lds0 + oW + 1024 * j, off < 8 * nwords ? off : kOutOfRange);
      }
      wait_vmcnt<0>();
    }
    const int nprod = nck * (rp >> 4);  // at most 128: two sentinels per lane
    bool bad = sCtl[0] != 0;
    unsigned it = 0;  // polls so far (bounded by a.spin)
    while (!bad) {
      bool mine = true;
      for (int e = lane; e < nwords; e += 64) mine &= (uint32_t)(sW[e] >> 32) == tag;
      if (__builtin_amdgcn_ballot_w64(!mine) == 0) break;
      for (;;) {  // wait on the sentinels (every round counts, so the re-reads are bounded too)
        if (it++ >= a.spin) {
          bad = true;
          break;
        }
        __builtin_amdgcn_s_sleep(4);
        bool done = true;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int pi = min(lane + 64 * i, nprod - 1);  // partial (c, q) = (pi % nck, pi / nck)
          done &= (uint32_t)(ld64(lay + (size_t)16 * (pi / nck) * nck + pi % nck) >> 32) == tag;
        }
        if (__builtin_amdgcn_ballot_w64(!done) == 0) break;
      }
      if (bad) break;
      for (int e = lane; e < nwords; e += 64) sW[e] = ld64(lay + e);
      lds_done();
    }
    if (bad && sCtl[0] == 0 && lane == 0) {
      sCtl[0] = 1u;
      __hip_atomic_fetch_or(a.sync + kWFlag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int e = lane; e < ne; e += 64) {
      float t = 0.0f;
      for (int k = 0; k < nck; ++k) t += __uint_as_float((uint32_t)sW[e * nck + k]);
      const bf16_t h = (bf16_t)f32_to_bf16_bits(t);
      sT[e] = h;  // sT is [16][rp]: element e is row e / rp, column e % rp
      if (tfirst && a.Tout) a.Tout[(size_t)(e >> a.lrp) * a.ldt + toff + (e & (rp - 1))] = h;
    }
    for (int e = ne + lane; e < 16 * rp; e += 64) sT[e] = 0;  // rows n .. 15 of the operand
    lds_done();
    // T L2 of every group on the bf16 MFMA, in the integer sums' layout
    for (int g = 0; g < G; ++g) {
      f32x4 lrv = {0.f, 0.f, 0.f, 0.f};
      for (int t0 = 0; t0 < rp; t0 += 32) {
        const uint4 a8 = *reinterpret_cast<const uint4*>(sT + l16 * rp + t0 + 8 * lg);
        const uint4 b8 = *reinterpret_cast<const uint4*>(sL + (16 * g + l16) * rp + t0 + 8 * lg);
        lrv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a8), as_bf16x8(b8), lrv, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sLR[(g * 4 + i) * 64 + lane] = lrv[i];
    }
  } else {
    for (int j = 0; j < 4 * G; ++j) sLR[j * 64 + lane] = 0.0f;
  }
  lds_done();
  if (lane == 0) {
    __hip_atomic_store(&sCtl[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    // the last channel block to be done with the hand-off words advances the epoch
    if (__hip_atomic_fetch_add(a.sync + kWCons, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        (unsigned)a.ncons - 1) {
      st32(a.sync + kWCons, 0u);
      st32(a.sync + kWEpoch, sCtl[1] + 1);
    }
  }
}

template <typename T, int NR, bool HP>
hipError_t launch_hp(const DecodeArgs& a, const DecodePlan& p, hipStream_t st) {
  const dim3 grid((unsigned)p.blocks), block(kNT);
  if (a.acc)
    hipLaunchKernelGGL((k_decode<T, NR, true, HP>), grid, block, p.lds, st, a);
  else
    launch_kernel(k_decode<T, NR, false, HP>, grid, block, p.lds, st, a);
  return hipGetLastError();
}

// Chunks of T from which the control wave runs at raised priority.
constexpr int kDecodeHpChunks = 16;

template <typename T, int NR>
hipError_t launch_nr(const DecodeArgs& a, const DecodePlan& p, hipStream_t st) {
  return a.nchunk >= kDecodeHpChunks ? launch_hp<T, NR, true>(a, p, st) : launch_hp<T, NR, false>(a, p, st);
}

}  // namespace

// The partial blocks (the grid's lowest indices, dispatched first) never
// wait; at most kDecodeMaxNt of them keep the partials' words few enough for
// one batch of loads per channel block.
constexpr int kDecodeMaxNt = 128;

static int decode_nt(int d, int ldt) {
  if (ldt <= 0) return 0;
  const int kcs = kDecodeSteps * kNW;
  return ((d / 32 + kcs - 1) / kcs) * (ldt / 16);
}

bool decode_ok(int n, int d, int ldt) {
  return n >= 1 && n <= kDecodeMaxN && d >= 32 && d % 32 == 0 && d <= kDecodeMaxD && n * d <= 16384 && ldt <= 256 &&
         decode_nt(d, ldt) <= kDecodeMaxNt;
}

DecodePlan plan_decode(int n, int d, int m, int r_pad, int ldt, bool x_bf16) {
  DecodePlan p{};
  const int S = (d / 2 + 63) / 64;  // 64-byte steps of a weight row
  p.gpb = std::max(1, std::min(kGmax, 128 / S));
  if (ldt > 0) {
    p.nqg = ldt / 16;
    p.kcs = kDecodeSteps * kNW;  // every wave of a partial block takes kDecodeSteps 32-k steps
    p.nchunk = (d / 32 + p.kcs - 1) / p.kcs;
    p.nt = p.nchunk * p.nqg;
  }
  p.ncons = (m + 16 * p.gpb - 1) / (16 * p.gpb);
  p.blocks = p.nt + p.ncons;
  // region A: the token rows (channel blocks) or their chunk and the L1^T
  // rows (partial blocks); then the partials' words (a
  // whole number of KB: their direct loads write whole KB), L2^T rows,
  // scales, hand-off words, the groups' sums and T L2, T, sP, codes, maxima,
  // flags and counters
  const int xs = (d * (x_bf16 ? 2 : 4) + 1023) & ~1023, ls = kDecodeSteps * kNW * 64;
  const int xc = 512 * (x_bf16 ? 2 : 4);  // a partial block's chunk of a row
  p.lds_a = (unsigned)std::max(n * xs, ldt > 0 ? n * xc + 16 * ls : 0);
  const int swb = (8 * n * r_pad * p.nchunk + 1023) & ~1023;
  const int sl = r_pad ? (32 * p.gpb * r_pad + 1023) & ~1023 : 0;
  p.lds = p.lds_a + (unsigned)(swb + sl + 512 + 8192 + 32 * r_pad + kNW * 16 * 17 * 4 + n * (d / 2) + 64 + 64 + 16 + 16);
  return p;
}

// the layer's words (nchunk n ldt), with 8 KB of slack
size_t decode_partials_bytes(const DecodePlan& p, int n, int ldt) { return ((size_t)p.nchunk * n * ldt + 1024) * 8; }

hipError_t launch_decode(const DecodeArgs& args, const DecodePlan& p, bool x_bf16, hipStream_t st) {
  if (!decode_ok(args.n, args.d, args.ldt)) return hipErrorInvalidValue;
  const DecodePlan q = plan_decode(args.n, args.d, args.m, args.r_pad, args.ldt, x_bf16);  // LDS for this X type
  if (q.blocks != p.blocks || q.nt != p.nt || q.lds > 160 * 1024) return hipErrorInvalidValue;
  DecodeArgs a = args;
  a.lds_a = (int)q.lds_a;
  a.gpb = q.gpb;
  a.ncons = q.ncons;
  if (x_bf16) return a.n == 1 ? launch_nr<bf16_t, 1>(a, q, st) : launch_nr<bf16_t, 2>(a, q, st);
  return a.n == 1 ? launch_nr<float, 1>(a, q, st) : launch_nr<float, 2>(a, q, st);
}

// ---------------------------------------------------------------------------
// The streaming-read ceiling that bounds the decode kernel: `bytes` read once
// with the same 16-byte non-temporal loads, 8 in flight per lane, each block
// a contiguous slab; every block XORs what it read and writes one word, so
// the loads cannot be dropped.
// ---------------------------------------------------------------------------
namespace {
__global__ __launch_bounds__(256) void k_stream_read(const i32x4* __restrict__ p, size_t n16, uint32_t* out) {
  __shared__ uint32_t acc_s;
  if (threadIdx.x == 0) acc_s = 0;
  __syncthreads();
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t beg = (size_t)blockIdx.x * per, end = n16 < beg + per ? n16 : beg + per;
  i32x4 acc = {0, 0, 0, 0};
  for (size_t i = beg + threadIdx.x; i < end; i += 256 * 8) {
    i32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const size_t j = i + 256 * (size_t)u;
      v[u] = j < end ? __builtin_nontemporal_load(p + j) : i32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  atomicXor(&acc_s, (uint32_t)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]));
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = acc_s;
}
}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* out, int blocks, hipStream_t st) {
  if (bytes % 16 || blocks < 1) return hipErrorInvalidValue;
  launch_kernel(k_stream_read, dim3((unsigned)blocks), dim3(256), 0, st, reinterpret_cast<const i32x4*>(buf), bytes / 16,
                out);
  return hipGetLastError();
}

}  // namespace tq
