// C ABI of the rank-augmented W4A4 layer: argument checking, workspace
// layout, kernel selection and optional per-kernel event timing.  Every
// check runs before any HIP call, so a failing check enqueues nothing.

#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/tq.h"
#include "tq_prologue.h"

namespace {

using tq::GemmArgs;

constexpr int kSmallN = 32;       // n <= kSmallN takes the memory-bound small-n path
constexpr int64_t kMaxDim = (int64_t)1 << 30;
// Longest reduction: |sum of k code products| <= 128 * 128 * k (8-bit) or, in
// the 4-bit GEMM whose operands carry 16 x code, 256 * 64 * k; both stay below
// 2^31 (exact int32) for k <= 2^16.
constexpr int64_t kMaxK = (int64_t)1 << 16;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// r rounded up to the padded width of the packed low-rank factors.
int64_t r_padded(int64_t r) {
  if (r <= 0) return 0;
  int64_t p = 32;
  while (p < r) p <<= 1;
  return p;
}

// ---------------------------------------------------------------------------
// profiling
// ---------------------------------------------------------------------------
struct ProfRecord {
  std::string name;
  hipEvent_t e0, e1;
};
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<ProfRecord> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};
Profiler& prof() {
  static Profiler p;
  return p;
}

}  // namespace

namespace tq {
LaunchEvents& launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}
}  // namespace tq

namespace {

// Wraps one kernel launch; returns the launcher's error.  Stream events are
// recorded around the launch; a launcher that takes the dispatch-timestamp
// events (tq::launch_kernel) makes those the record instead.
template <typename F>
hipError_t timed(const char* name, hipStream_t st, F&& launch) {
  Profiler& p = prof();
  std::unique_lock<std::mutex> lk(p.mu);
  if (!p.on) {
    lk.unlock();
    return launch();
  }
  hipEvent_t e0 = p.get(), e1 = p.get(), x0 = p.get(), x1 = p.get();
  tq::LaunchEvents& ev = tq::launch_events();
  ev = tq::LaunchEvents{x0, x1, false};
  if (e0) (void)hipEventRecord(e0, st);
  hipError_t err = launch();
  if (e1) (void)hipEventRecord(e1, st);
  const bool used = ev.used;
  ev = tq::LaunchEvents{};
  if (used) {
    p.recs.push_back({name, x0, x1});
    if (e0) p.pool.push_back(e0);
    if (e1) p.pool.push_back(e1);
  } else {
    if (e0 && e1) p.recs.push_back({name, e0, e1});
    if (x0) p.pool.push_back(x0);
    if (x1) p.pool.push_back(x1);
  }
  return err;
}

#define TQ_RUN(name, st, expr)                                  \
  do {                                                           \
    hipError_t _e = timed(name, st, [&]() { return (expr); });  \
    if (_e != hipSuccess) return TQ_ERR_HIP;                     \
  } while (0)

// Fixed counter region after the hand-off words (see linear_ws).
constexpr size_t kCtrBytes = 4096;

struct LinearWs {
  size_t sync, ctr, sx, xc, t, p, total;
  int r_pad;  // columns of T
  bool small, decode;
  bool fused;     // tq_linear: the one-launch few-token layer (fplan), when its grid fits
  bool fusable;   // the shape has a one-launch plan (fplan; the asymmetric layer too)
  tq::ProloguePlan plan, fplan;
  tq::DecodePlan dplan;
};

// tcols: columns of T (r_pad of one layer; a power of two covering all the
// layers of a group); rp: one layer's r_pad (0: tcols)
// two_launch: never the one-launch few-token kernel (the asymmetric layer)
LinearWs linear_ws(int64_t n, int64_t d, int64_t m, int64_t tcols, bool two_launch = false, int64_t rp = -1) {
  LinearWs w{};
  w.small = n <= kSmallN;
  w.r_pad = (int)tcols;
  w.decode = !two_launch && n > 0 && tq::decode_ok((int)n, (int)d, w.r_pad);
  size_t psize = 0;
  if (w.decode) {
    w.dplan = tq::plan_decode((int)n, (int)d, (int)m, (int)(rp < 0 ? tcols : rp), w.r_pad, false);
    psize = tq::decode_partials_bytes(w.dplan, (int)n, w.r_pad);
  } else {
    w.plan = tq::plan_prologue((int)n, (int)d, w.r_pad, w.small,
                               w.small ? tq::gemv_max_chunks((int)n, (int)(d / 2), w.r_pad) : 1);
    if (w.plan.ntb > 0 && (w.plan.nchunk > 1 || w.plan.partial))
      psize = (size_t)w.plan.nchunk * (size_t)n * (size_t)w.r_pad * 4;
    // one launch up to 16 tokens; for 17 .. 32 (two 16-token tiles per
    // block, twice the producers) the two launches measured faster
    w.fusable = n > 0 && n <= 16 && d <= 16384 && w.r_pad % 32 == 0;
    w.fused = !two_launch && w.fusable;
    if (w.fusable) {
      w.fplan = tq::plan_prologue_fused((int)n, (int)d, w.r_pad, tq::gemv_max_chunks((int)n, (int)(d / 2), w.r_pad));
      if (w.fplan.ntb > 0)
        psize = std::max(psize, (size_t)w.fplan.nchunk * (size_t)n * (size_t)w.r_pad * 4);
    }
  }
  // The counters sit at fixed offsets, whatever the shape, so that a
  // workspace zero-filled once serves calls of any shape in turn: the
  // hand-off words of the one-launch paths, then kCtrBytes holding the
  // prologue's counters (fewer than 128).
  size_t o = 0;
  w.sync = o;  // hand-off counters of the few-token launch
  o = tq::kSyncBytes;
  w.ctr = o;
  o += kCtrBytes;
  w.sx = o;
  o = align256(o + (size_t)n * 4);
  w.xc = o;  // activation codes: int8 (d bytes per row) for the tile GEMM, else packed
  o = align256(o + (size_t)n * (size_t)(w.small ? d / 2 : d));
  w.t = o;
  o = align256(o + (size_t)n * (size_t)w.r_pad * 2);
  w.p = o;
  o = align256(o + psize);
  w.total = o;
  return w;
}

struct MpWs {
  size_t sxl, sxh, xl, xh, total;
};

MpWs mp_ws(int64_t n, int64_t d, int64_t d_hi) {
  MpWs w{};
  const int64_t dl = d - d_hi;
  size_t o = 0;
  w.sxl = o;
  o = align256(o + (size_t)n * 4);
  w.sxh = o;
  o = align256(o + (size_t)n * 4);
  w.xl = o;  // 4-bit codes as int8 in the order of the tile GEMM
  o = align256(o + (size_t)n * (size_t)dl);
  w.xh = o;
  o = align256(o + (size_t)n * (size_t)d_hi);
  w.total = o;
  return w;
}

bool valid_dtype(tq_dtype t) { return t == TQ_F32 || t == TQ_BF16; }

// Workspace of tq_linear_mp_asym: the two-subspace workspace, then the two
// zero-point vectors.
struct MpAsymWs {
  MpWs mp;
  size_t zl, zh, total;
};
MpAsymWs mp_asym_ws(int64_t n, int64_t d, int64_t d_hi) {
  MpAsymWs w{};
  w.mp = mp_ws(n, d, d_hi);
  size_t o = w.mp.total;
  w.zl = o;
  o = align256(o + (size_t)n * 4);
  w.zh = o;
  o = align256(o + (size_t)n * 4);
  w.total = o;
  return w;
}

// Packed quantised low-rank factors: U^T codes (r_pad rows of d / 2 bytes),
// s_u (r_pad), V^T codes (m rows of r_pad / 2 bytes), s_v (m).
struct QlrPack {
  size_t uc, su, vc, sv, total;
};
QlrPack qlr_pack(int64_t d, int64_t m, int64_t r_pad) {
  QlrPack p{};
  size_t o = 0;
  p.uc = o;
  o = align256(o + (size_t)r_pad * (size_t)d / 2);
  p.su = o;
  o = align256(o + (size_t)r_pad * 4);
  p.vc = o;
  o = align256(o + (size_t)m * (size_t)r_pad / 2);
  p.sv = o;
  o = align256(o + (size_t)m * 4);
  p.total = o;
  return p;
}

// Workspace of tq_linear_qlr: s_x, the int8-order activation codes, s_t and
// the first stage's codes (r_pad int8 bytes per token).
struct QlrWs {
  size_t sx, xc, st, tc, total;
};
QlrWs qlr_ws(int64_t n, int64_t d, int64_t r_pad) {
  QlrWs w{};
  size_t o = 0;
  w.sx = o;
  o = align256(o + (size_t)n * 4);
  w.xc = o;
  o = align256(o + (size_t)n * (size_t)d);
  w.st = o;
  o = align256(o + (size_t)n * 4);
  w.tc = o;
  o = align256(o + (size_t)n * (size_t)r_pad);
  w.total = o;
  return w;
}

}  // namespace

extern "C" {

const char* tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "TQ_OK";
    case TQ_ERR_NULL: return "TQ_ERR_NULL: a required pointer is NULL";
    case TQ_ERR_SHAPE: return "TQ_ERR_SHAPE: a size is out of range";
    case TQ_ERR_DTYPE: return "TQ_ERR_DTYPE: unsupported element type";
    case TQ_ERR_BITS: return "TQ_ERR_BITS: unsupported bit width";
    case TQ_ERR_ALIGN: return "TQ_ERR_ALIGN: pointer not 16-byte aligned";
    case TQ_ERR_WORKSPACE: return "TQ_ERR_WORKSPACE: workspace too small";
    case TQ_ERR_HIP: return "TQ_ERR_HIP: HIP runtime error";
  }
  return "unknown tq_status";
}

int tq_version(void) { return 106; }

size_t tq_codes_bytes(int64_t rows, int64_t k, int bits) {
  if (rows < 0 || k < 0 || (bits != 3 && bits != 4 && bits != 6 && bits != 8) || (bits <= 4 && (k & 1))) return 0;
  return (size_t)rows * (size_t)k * (size_t)(bits <= 4 ? 4 : 8) / 8;  // 3 / 6 bits stored like 4 / 8
}

tq_status tq_pack_weight(const void* W, tq_dtype w_dt, int64_t d, int64_t m, int bits, void* w_codes, float* s_w,
                         hipStream_t stream) {
  if (bits != 3 && bits != 4 && bits != 6 && bits != 8) return TQ_ERR_BITS;
  if (!valid_dtype(w_dt)) return TQ_ERR_DTYPE;
  if (d <= 0 || m <= 0 || d > kMaxDim || m > kMaxDim || d % (bits <= 4 ? 32 : 16)) return TQ_ERR_SHAPE;
  if (!W || !w_codes || !s_w) return TQ_ERR_NULL;
  if (!aligned16(W) || !aligned16(w_codes) || !aligned16(s_w)) return TQ_ERR_ALIGN;
  TQ_RUN("pack_weight", stream, tq::launch_pack_weight(W, w_dt == TQ_BF16, (int)d, (int)m, bits, w_codes, s_w, stream));
  return TQ_OK;
}

// T columns of G layers of rank r: G r_pad rounded up to a power of two.
int64_t group_tcols(int64_t G, int64_t r) { return G <= 1 ? r_padded(r) : r_padded(G * r_padded(r)); }

size_t tq_lowrank_bytes(int64_t d, int64_t m, int64_t r) {
  if (d <= 0 || m <= 0 || r < 0 || r > 256) return 0;
  const int64_t rp = r_padded(r);
  return (size_t)(rp * d + m * rp) * 2;
}

tq_status tq_pack_lowrank(const void* L1, const void* L2, tq_dtype dt, int64_t d, int64_t m, int64_t r,
                          void* lowrank, hipStream_t stream) {
  if (!valid_dtype(dt)) return TQ_ERR_DTYPE;
  if (d <= 0 || m <= 0 || d > kMaxDim || m > kMaxDim || d % 32 || r < 1 || r > 256) return TQ_ERR_SHAPE;
  if (!L1 || !L2 || !lowrank) return TQ_ERR_NULL;
  if (!aligned16(lowrank)) return TQ_ERR_ALIGN;
  const int rp = (int)r_padded(r);
  TQ_RUN("pack_lowrank", stream,
         tq::launch_pack_lowrank(L1, L2, dt == TQ_BF16, (int)d, (int)m, (int)r, rp, rp, lowrank,
                                 (uint8_t*)lowrank + (size_t)rp * d * 2, stream));
  return TQ_OK;
}

tq_status tq_quantize_act(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int bits, void* x_codes, float* s_x,
                          hipStream_t stream) {
  if (bits != 4 && bits != 8) return TQ_ERR_BITS;
  if (!valid_dtype(x_dt)) return TQ_ERR_DTYPE;
  if (n < 0 || n > kMaxDim || d <= 0 || d > kMaxDim || d % (bits == 4 ? 32 : 16)) return TQ_ERR_SHAPE;
  if (n == 0) return TQ_OK;
  if (!X || !x_codes || !s_x) return TQ_ERR_NULL;
  if (!aligned16(X) || !aligned16(x_codes) || !aligned16(s_x)) return TQ_ERR_ALIGN;
  TQ_RUN("quant_rows", stream,
         tq::launch_quant_rows_fast(X, x_dt == TQ_BF16, (int)n, (int)d, (int)d, bits, bits, x_codes, s_x, nullptr, nullptr,
                               stream));
  return TQ_OK;
}

size_t tq_linear_workspace_bytes(int64_t n, int64_t d, int64_t m, int64_t r) {
  if (n < 0 || n > kMaxDim || d <= 0 || d > kMaxK || d % 32 || m <= 0 || m > kMaxDim || r < 0 || r > 256) return 0;
  return linear_ws(n, d, m, r_padded(r)).total;
}

}  // extern "C"

namespace {

// The layer (or G layers stacked along the channels, sharing X) once the
// arguments are checked: ms[g] channels per layer, m = their sum.
// acc: when not null, the kernels' exact int32 residual sums (n x m) are
// also stored there (test hook).
// Test hook of the one-launch few-token path: its polls' limit, and producers
// that tag their partials with the previous call's epoch.
struct HandoffDebug {
  unsigned spin;
  int silent;
};
// Polls of a wait before it gives up: each is a memory round trip, so this
// is a fraction of a second.
constexpr unsigned kDecodeSpin = 1u << 18;

tq_status linear_run(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r, int G,
                     const int64_t* ms, const void* w_codes, const float* s_w, const void* lowrank, void* Y,
                     tq_dtype y_dt, void* ws, size_t ws_bytes, hipStream_t stream, int32_t* acc = nullptr,
                     const HandoffDebug* dbg = nullptr) {
  const int rp = (int)r_padded(r);
  const LinearWs L = linear_ws(n, d, m, group_tcols(G, r), false, rp);
  if (ws_bytes < L.total) return TQ_ERR_WORKSPACE;
  // the fixed counter region holds every counter this shape uses
  if ((size_t)L.plan.counters * 4 > kCtrBytes) return TQ_ERR_SHAPE;

  uint8_t* base = (uint8_t*)ws;
  unsigned* ctr = (unsigned*)(base + L.ctr);
  float* sx = (float*)(base + L.sx);
  uint8_t* xc = base + L.xc;
  tq::bf16_t* T = (tq::bf16_t*)(base + L.t);
  float* P = (float*)(base + L.p);
  const tq::bf16_t* L1t = (const tq::bf16_t*)lowrank;
  const tq::bf16_t* L2t = lowrank ? L1t + (size_t)L.r_pad * d : nullptr;
  const bool xb = x_dt == TQ_BF16;
  tq::Groups groups{};
  groups.n = G;
  for (int g = 0; g < G; ++g) groups.start[g + 1] = groups.start[g] + (int)ms[g];

  if (L.decode) {
    tq::DecodeArgs a{};
    a.X = X;
    a.n = (int)n;
    a.d = (int)d;
    a.m = (int)m;
    a.wc = (const uint8_t*)w_codes;
    a.sw = s_w;
    a.L1t = L1t;
    a.L2t = L2t;
    a.r_pad = rp;
    a.lrp = 0;
    while ((1 << a.lrp) < rp) ++a.lrp;
    a.ldt = L.r_pad;
    a.groups = groups;
    a.nt = L.dplan.nt;
    a.nqg = L.dplan.nqg;
    a.kcs = L.dplan.kcs;
    a.nchunk = L.dplan.nchunk;
    a.xc = xc;
    a.sx = sx;
    a.P = P;
    a.Tout = L.r_pad ? T : nullptr;
    a.sync = (unsigned*)(base + L.sync);
    a.Y = Y;
    a.y_bf16 = y_dt == TQ_BF16;
    a.acc = acc;
    a.spin = dbg ? dbg->spin : kDecodeSpin;
    a.silent = dbg ? dbg->silent : 0;
    TQ_RUN("decode", stream, tq::launch_decode(a, L.dplan, xb, stream));
    return TQ_OK;
  }

  GemmArgs g{};
  g.A = xc;
  g.lda = d / 2;
  g.B = (const uint8_t*)w_codes;
  g.ldb = d / 2;
  g.M = (int)n;
  g.N = (int)m;
  g.Kb = (int)(d / 2);
  g.sx = sx;
  g.sw = s_w;
  g.T = L.r_pad ? T : nullptr;
  g.L2t = L2t;
  g.r_pad = rp;
  g.ldt = L.r_pad;
  g.groups = groups;
  if (L.r_pad && (L.plan.partial || L.plan.sum_to_p0)) {
    g.P = P;
    g.nchunk = L.plan.partial ? L.plan.nchunk : 1;
    g.Tout = T;
  }
  g.Y = Y;
  g.ldy = m;
  g.y_bf16 = y_dt == TQ_BF16;
  g.acc = acc;

  if (L.fused && tq::gemv_fused_fits((int)n, (int)(d / 2), (int)m, L.fplan.nqb + L.fplan.ntb, xb, acc != nullptr)) {
    // one launch: the quantiser and the partials of T run in the GEMM's grid
    const tq::ProloguePlan& fp = L.fplan;
    tq::SmallFuse f{};
    f.pa = tq::PrologueArgs{X,      (int)n,    (int)d, L1t, L.r_pad, fp.kc, fp.nchunk, fp.qs, fp.nqg,
                            fp.nqb, 1,         1,      0,   xc,      sx,    P,         T,     ctr};
    f.nprod = fp.nqb + fp.ntb;
    f.sync = (unsigned*)(base + L.sync);
    f.spin = dbg ? dbg->spin : kDecodeSpin;
    f.silent = dbg ? dbg->silent : 0;
    g.P = L.r_pad ? P : nullptr;
    g.nchunk = fp.nchunk;
    g.Tout = L.r_pad ? T : nullptr;
    TQ_RUN("small_fused", stream, tq::launch_gemv_fused(g, f, xb, stream));
    return TQ_OK;
  }
  TQ_RUN("prologue", stream,
         tq::launch_prologue(X, xb, (int)n, (int)d, L1t, L.r_pad, L.plan, xc, sx, P, T, ctr, stream));
  if (L.small) {
    TQ_RUN("gemm_small_n", stream, tq::launch_gemv(g, 4, tq::EPI_LINEAR, stream));
  } else {
    g.lda = d;  // int8 activation codes
    TQ_RUN("gemm_w4a4", stream, tq::launch_gemm8(g, tq::EPI_LINEAR, true, 4, stream));
  }
  return TQ_OK;
}

// Checks shared by tq_linear and tq_linear_group.
tq_status linear_check(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r, const void* w_codes,
                       const float* s_w, const void* lowrank, void* Y, tq_dtype y_dt, void* ws) {
  if (!valid_dtype(x_dt) || !valid_dtype(y_dt)) return TQ_ERR_DTYPE;
  if (n < 0 || n > kMaxDim || d <= 0 || d > kMaxK || m <= 0 || m > kMaxDim || d % 32 || r < 0 || r > 256)
    return TQ_ERR_SHAPE;
  if (n == 0) return TQ_OK;
  if (!X || !w_codes || !s_w || !Y || !ws || (r > 0 && !lowrank)) return TQ_ERR_NULL;
  if (!aligned16(X) || !aligned16(w_codes) || !aligned16(s_w) || !aligned16(Y) || !aligned16(ws) ||
      (r > 0 && !aligned16(lowrank)))
    return TQ_ERR_ALIGN;
  return TQ_OK;
}

// Group shapes: 1 <= G <= 8 layers, each but the last a whole number of
// 256-channel tiles, G r_pad <= 256; m_total = their sum.
tq_status group_check(const int64_t* ms, int64_t G, int64_t r, int64_t* m_total) {
  if (!ms) return TQ_ERR_NULL;
  if (G < 1 || G > tq::kMaxGroups || r < 0 || r > 256 || G * r_padded(r) > 256) return TQ_ERR_SHAPE;
  int64_t t = 0;
  for (int64_t g = 0; g < G; ++g) {
    if (ms[g] <= 0 || (g + 1 < G && ms[g] % 256)) return TQ_ERR_SHAPE;
    t += ms[g];
  }
  if (t > kMaxDim) return TQ_ERR_SHAPE;
  *m_total = t;
  return TQ_OK;
}

}  // namespace

extern "C" {

tq_status tq_linear(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r, const void* w_codes,
                    const float* s_w, const void* lowrank, void* Y, tq_dtype y_dt, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  const tq_status st = linear_check(X, x_dt, n, d, m, r, w_codes, s_w, lowrank, Y, y_dt, ws);
  if (st != TQ_OK || n == 0) return st;
  const int64_t ms[1] = {m};
  return linear_run(X, x_dt, n, d, m, r, 1, ms, w_codes, s_w, lowrank, Y, y_dt, ws, ws_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free variant of tq_linear: its workspace is a file-scope device
// array, so a caller that cannot allocate (code under graph capture, a tight
// serving loop) passes only inputs and outputs.
// ---------------------------------------------------------------------------
namespace {

// One array per device (each device that the library runs on holds its own
// copy until the process ends).  In host code `noalloc_scratch` names a
// host-side stand-in, not the device memory: the kernels are given the
// address hipGetSymbolAddress returns for the current device, never the name.
__device__ __attribute__((aligned(256))) uint8_t noalloc_scratch[TQ_NOALLOC_SCRATCH_BYTES];

// Leading bytes of the scratch that hold the hand-off words and counters of
// the layer's kernels (they must be zero before a call; every call leaves
// them zero again).
constexpr size_t kNoallocZeroBytes = 64 * 1024;
constexpr int kMaxDevices = 64;

__global__ void k_zero16(uint4* p, int n16) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) p[i] = uint4{0, 0, 0, 0};
}

struct NoallocTable {
  std::mutex mu;
  void* ptr[kMaxDevices] = {};
};
NoallocTable& noalloc_table() {
  static NoallocTable t;
  return t;
}

// The scratch of the current device; on its first use on that device, its
// address (hipGetSymbolAddress, with the device current) and one clear of its
// counter bytes by a fill kernel on `stream` (a kernel, not a memset node,
// so that a first call under graph capture records a plain kernel node).
tq_status noalloc_scratch_ptr(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TQ_ERR_HIP;
  NoallocTable& t = noalloc_table();
  std::lock_guard<std::mutex> lk(t.mu);
  if (!t.ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch)) != hipSuccess || !p) return TQ_ERR_HIP;
    const int n16 = (int)(kNoallocZeroBytes / 16);
    hipLaunchKernelGGL(k_zero16, dim3((n16 + 255) / 256), dim3(256), 0, stream, (uint4*)p, n16);
    if (hipGetLastError() != hipSuccess) return TQ_ERR_HIP;
    t.ptr[dev] = p;
  }
  *out = t.ptr[dev];
  return TQ_OK;
}

}  // namespace

extern "C" {

tq_status tq_linear_noalloc(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r,
                            const void* w_codes, const float* s_w, const void* lowrank, void* Y, tq_dtype y_dt,
                            hipStream_t stream) {
  // the checks of tq_linear, with a stand-in workspace pointer (never used)
  const tq_status st = linear_check(X, x_dt, n, d, m, r, w_codes, s_w, lowrank, Y, y_dt, (void*)X);
  if (st != TQ_OK || n == 0) return st;
  const size_t need = linear_ws(n, d, m, r_padded(r)).total;
  if (need > (size_t)TQ_NOALLOC_SCRATCH_BYTES) return TQ_ERR_WORKSPACE;
  void* ws = nullptr;
  const tq_status sp = noalloc_scratch_ptr(stream, &ws);
  if (sp != TQ_OK) return sp;
  const int64_t ms[1] = {m};
  return linear_run(X, x_dt, n, d, m, r, 1, ms, w_codes, s_w, lowrank, Y, y_dt, ws, need, stream);
}

tq_status tq_debug_linear_handoff(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r,
                                  const void* w_codes, const float* s_w, const void* lowrank, void* Y, tq_dtype y_dt,
                                  void* ws, size_t ws_bytes, unsigned spin, int silent, hipStream_t stream) {
  const tq_status st = linear_check(X, x_dt, n, d, m, r, w_codes, s_w, lowrank, Y, y_dt, ws);
  if (st != TQ_OK || n == 0) return st;
  const LinearWs L = linear_ws(n, d, m, r_padded(r));
  const bool fused =
      L.fused && tq::gemv_fused_fits((int)n, (int)(d / 2), (int)m, L.fplan.nqb + L.fplan.ntb, x_dt == TQ_BF16, false);
  if (r == 0 || !(L.decode || fused)) return TQ_ERR_SHAPE;  // no hand-off on this path
  const int64_t ms[1] = {m};
  const HandoffDebug dbg{spin, silent};
  return linear_run(X, x_dt, n, d, m, r, 1, ms, w_codes, s_w, lowrank, Y, y_dt, ws, ws_bytes, stream, nullptr, &dbg);
}

tq_status tq_debug_stream_read(const void* buf, size_t bytes, uint32_t* out, int blocks, hipStream_t stream) {
  if (!buf || !out) return TQ_ERR_NULL;
  if (!aligned16(buf) || bytes % 16) return TQ_ERR_ALIGN;
  if (blocks < 1 || blocks > 65536) return TQ_ERR_SHAPE;
  TQ_RUN("stream_read", stream, tq::launch_stream_read(buf, bytes, out, blocks, stream));
  return TQ_OK;
}

tq_status tq_debug_mfma_ceiling(int iters, int blocks, int32_t* out, hipStream_t stream) {
  if (!out) return TQ_ERR_NULL;
  if (iters < 1 || iters > (1 << 20) || blocks < 1 || blocks > 65536) return TQ_ERR_SHAPE;
  TQ_RUN("mfma_ceiling", stream, tq::launch_mfma_ceiling(iters, blocks, out, stream));
  return TQ_OK;
}

tq_status tq_linear_debug(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r,
                          const void* w_codes, const float* s_w, const void* lowrank, void* Y, tq_dtype y_dt, void* ws,
                          size_t ws_bytes, int32_t* acc, hipStream_t stream) {
  const tq_status st = linear_check(X, x_dt, n, d, m, r, w_codes, s_w, lowrank, Y, y_dt, ws);
  if (st != TQ_OK || n == 0) return st;
  if (!acc) return TQ_ERR_NULL;
  if (!aligned16(acc)) return TQ_ERR_ALIGN;
  const int64_t ms[1] = {m};
  return linear_run(X, x_dt, n, d, m, r, 1, ms, w_codes, s_w, lowrank, Y, y_dt, ws, ws_bytes, stream, acc);
}

size_t tq_lowrank_group_bytes(int64_t d, const int64_t* m, int64_t G, int64_t r) {
  int64_t mt = 0;
  if (d <= 0 || r < 1 || group_check(m, G, r, &mt) != TQ_OK) return 0;
  return (size_t)(group_tcols(G, r) * d + mt * r_padded(r)) * 2;
}

tq_status tq_pack_lowrank_group(const void* const* L1, const void* const* L2, tq_dtype dt, int64_t d,
                                const int64_t* m, int64_t G, int64_t r, void* lowrank, hipStream_t stream) {
  if (!valid_dtype(dt)) return TQ_ERR_DTYPE;
  int64_t mt = 0;
  const tq_status gs = group_check(m, G, r, &mt);
  if (gs != TQ_OK) return gs;
  if (d <= 0 || d > kMaxDim || d % 32 || r < 1) return TQ_ERR_SHAPE;
  if (!L1 || !L2 || !lowrank) return TQ_ERR_NULL;
  for (int64_t g = 0; g < G; ++g)
    if (!L1[g] || !L2[g]) return TQ_ERR_NULL;
  if (!aligned16(lowrank)) return TQ_ERR_ALIGN;
  const int rp = (int)r_padded(r), tc = (int)group_tcols(G, r);
  uint8_t* l1 = (uint8_t*)lowrank;
  uint8_t* l2 = l1 + (size_t)tc * d * 2;
  for (int64_t g = 0; g < G; ++g) {
    // the last layer also zero-fills the rows of T past G r_pad
    const int rows1 = g + 1 < G ? rp : tc - (int)(G - 1) * rp;
    TQ_RUN("pack_lowrank", stream,
           tq::launch_pack_lowrank(L1[g], L2[g], dt == TQ_BF16, (int)d, (int)m[g], (int)r, rp, rows1,
                                   l1 + (size_t)g * rp * d * 2, l2, stream));
    l2 += (size_t)m[g] * rp * 2;
  }
  return TQ_OK;
}

size_t tq_linear_group_workspace_bytes(int64_t n, int64_t d, const int64_t* m, int64_t G, int64_t r) {
  int64_t mt = 0;
  if (n < 0 || d <= 0 || group_check(m, G, r, &mt) != TQ_OK) return 0;
  return linear_ws(n, d, mt, group_tcols(G, r)).total;
}

tq_status tq_linear_group(const void* X, tq_dtype x_dt, int64_t n, int64_t d, const int64_t* m, int64_t G,
                          int64_t r, const void* w_codes, const float* s_w, const void* lowrank, void* Y,
                          tq_dtype y_dt, void* ws, size_t ws_bytes, hipStream_t stream) {
  int64_t mt = 0;
  const tq_status gs = group_check(m, G, r, &mt);
  if (gs != TQ_OK) return gs;
  const tq_status st = linear_check(X, x_dt, n, d, mt, r, w_codes, s_w, lowrank, Y, y_dt, ws);
  if (st != TQ_OK || n == 0) return st;
  return linear_run(X, x_dt, n, d, mt, r, (int)G, m, w_codes, s_w, lowrank, Y, y_dt, ws, ws_bytes, stream);
}

tq_status tq_linear_workspace_offsets(int64_t n, int64_t d, int64_t m, int64_t r, size_t off[4]) {
  if (n < 0 || d <= 0 || m <= 0 || r < 0 || r > 256 || d % 32) return TQ_ERR_SHAPE;
  if (!off) return TQ_ERR_NULL;
  const LinearWs L = linear_ws(n, d, m, r_padded(r));
  off[0] = L.sx;
  off[1] = L.xc;
  off[2] = L.t;
  off[3] = L.sync;
  return TQ_OK;
}

size_t tq_linear_mp_workspace_bytes(int64_t n, int64_t d, int64_t d_hi) {
  if (n < 0 || d <= 0 || d_hi < 0 || d_hi > d) return 0;
  return mp_ws(n, d, d_hi).total;
}

}  // extern "C"

namespace {

// Checks of the two-subspace layer (X is Xrot, or unrotated X with rot).
tq_status mp_check(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t d_hi, int64_t m, const void* wl_codes,
                   const float* s_wl, const void* wh_codes, const float* s_wh, void* Y, tq_dtype y_dt, void* ws) {
  if (!valid_dtype(x_dt) || !valid_dtype(y_dt)) return TQ_ERR_DTYPE;
  const int64_t dl = d - d_hi;
  if (n < 0 || n > kMaxDim || d <= 0 || d > kMaxK || m <= 0 || m > kMaxDim || d_hi < 0 || d_hi > d || dl % 32 ||
      d_hi % 16)
    return TQ_ERR_SHAPE;
  if (n == 0) return TQ_OK;
  if (!X || !Y || !ws || (dl > 0 && (!wl_codes || !s_wl)) || (d_hi > 0 && (!wh_codes || !s_wh))) return TQ_ERR_NULL;
  if (!aligned16(X) || !aligned16(Y) || !aligned16(ws) || (dl > 0 && (!aligned16(wl_codes) || !aligned16(s_wl))) ||
      (d_hi > 0 && (!aligned16(wh_codes) || !aligned16(s_wh))))
    return TQ_ERR_ALIGN;
  return TQ_OK;
}

// Accumulator-export buffers of the test-hook entry points: the residual (or
// 4-bit) product always, the second product when it is not empty.
tq_status debug_check(const int32_t* acc, const int32_t* acc2, bool need2) {
  if (!acc || (need2 && !acc2)) return TQ_ERR_NULL;
  if (!aligned16(acc) || (need2 && !aligned16(acc2))) return TQ_ERR_ALIGN;
  return TQ_OK;
}

// The two-subspace GEMM on the codes and scales in the workspace (with the
// zero-points and weight code sums of asymmetric activations when zl / zh
// are not null).
tq_status mp_gemm(int64_t n, int64_t d, int64_t d_hi, int64_t m, const void* wl_codes, const float* s_wl,
                  const void* wh_codes, const float* s_wh, void* Y, tq_dtype y_dt, const MpWs& W, uint8_t* base,
                  hipStream_t stream, const float* zl = nullptr, const float* zh = nullptr,
                  const int32_t* csl = nullptr, const int32_t* csh = nullptr, int32_t* acc_l = nullptr,
                  int32_t* acc_h = nullptr) {
  const int64_t dl = d - d_hi;
  float* sxl = (float*)(base + W.sxl);
  float* sxh = (float*)(base + W.sxh);
  uint8_t* xl = base + W.xl;
  uint8_t* xh = base + W.xh;
  GemmArgs g{};
  g.M = (int)n;
  g.N = (int)m;
  g.Y = Y;
  g.ldy = m;
  g.y_bf16 = y_dt == TQ_BF16;
  // low subspace is the main (4-bit) segment, the high subspace the second (8-bit) segment
  g.A = dl > 0 ? xl : xh;
  g.lda = dl > 0 ? dl : 16;  // int8 activation codes
  g.B = dl > 0 ? (const uint8_t*)wl_codes : (const uint8_t*)wh_codes;
  g.ldb = dl > 0 ? dl / 2 : 16;
  g.Kb = (int)(dl / 2);
  g.sx = dl > 0 ? sxl : sxh;
  g.sw = dl > 0 ? s_wl : s_wh;
  g.A2 = xh;
  g.lda2 = d_hi;
  g.B2 = (const uint8_t*)wh_codes;
  g.ldb2 = d_hi;
  g.Kb2 = (int)d_hi;
  g.sx2 = sxh;
  g.sw2 = s_wh;
  g.zx = dl > 0 ? zl : nullptr;
  g.csw = csl;
  g.zx2 = d_hi > 0 ? zh : nullptr;
  g.csw2 = csh;
  g.acc = acc_l;
  g.acc2 = acc_h;
  TQ_RUN("gemm_mp", stream, tq::launch_gemm8(g, tq::EPI_MP, true, 4, stream));
  return TQ_OK;
}

tq_status mp_bits_run(const void* Xrot, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t d_hi, int bits_lo,
                      int bits_hi, const void* wl_codes, const float* s_wl, const void* wh_codes, const float* s_wh,
                      void* Y, tq_dtype y_dt, void* ws, size_t ws_bytes, hipStream_t stream, int32_t* acc_l,
                      int32_t* acc_h) {
  const int64_t dl = d - d_hi;
  const MpWs W = mp_ws(n, d, d_hi);
  if (ws_bytes < W.total) return TQ_ERR_WORKSPACE;
  uint8_t* base = (uint8_t*)ws;
  float* sxl = (float*)(base + W.sxl);
  float* sxh = (float*)(base + W.sxh);
  uint8_t* xl = base + W.xl;
  uint8_t* xh = base + W.xh;
  const bool xb = x_dt == TQ_BF16;
  if (dl > 0 && d_hi > 0) {
    TQ_RUN("quant_rows_mp", stream,
           tq::launch_quant_rows_i8_bits(Xrot, xb, (int)n, (int)d, (int)dl, bits_lo, bits_hi, xl, sxl, xh, sxh,
                                         stream));
  } else if (dl > 0) {
    TQ_RUN("quant_rows_mp", stream,
           tq::launch_quant_rows_i8_bits(Xrot, xb, (int)n, (int)d, (int)d, bits_lo, bits_lo, xl, sxl, nullptr,
                                         nullptr, stream));
  } else {
    TQ_RUN("quant_rows_mp", stream,
           tq::launch_quant_rows_fast(Xrot, xb, (int)n, (int)d, (int)d, bits_hi, bits_hi, xh, sxh, nullptr, nullptr,
                                      stream));
  }
  return mp_gemm(n, d, d_hi, m, wl_codes, s_wl, wh_codes, s_wh, Y, y_dt, W, base, stream, nullptr, nullptr, nullptr,
                 nullptr, acc_l, acc_h);
}

}  // namespace

extern "C" {

tq_status tq_linear_mp_bits(const void* Xrot, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t d_hi,
                            int bits_lo, int bits_hi, const void* wl_codes, const float* s_wl, const void* wh_codes,
                            const float* s_wh, void* Y, tq_dtype y_dt, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  if (!((bits_lo == 4 && bits_hi == 8) || (bits_lo == 3 && bits_hi == 6))) return TQ_ERR_BITS;
  const tq_status st = mp_check(Xrot, x_dt, n, d, d_hi, m, wl_codes, s_wl, wh_codes, s_wh, Y, y_dt, ws);
  if (st != TQ_OK || n == 0) return st;
  return mp_bits_run(Xrot, x_dt, n, d, m, d_hi, bits_lo, bits_hi, wl_codes, s_wl, wh_codes, s_wh, Y, y_dt, ws,
                     ws_bytes, stream, nullptr, nullptr);
}

tq_status tq_linear_mp_bits_debug(const void* Xrot, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t d_hi,
                                  int bits_lo, int bits_hi, const void* wl_codes, const float* s_wl,
                                  const void* wh_codes, const float* s_wh, void* Y, tq_dtype y_dt, void* ws,
                                  size_t ws_bytes, int32_t* acc_l, int32_t* acc_h, hipStream_t stream) {
  if (!((bits_lo == 4 && bits_hi == 8) || (bits_lo == 3 && bits_hi == 6))) return TQ_ERR_BITS;
  const tq_status st = mp_check(Xrot, x_dt, n, d, d_hi, m, wl_codes, s_wl, wh_codes, s_wh, Y, y_dt, ws);
  if (st != TQ_OK || n == 0) return st;
  const tq_status sd = debug_check(acc_l, acc_h, d_hi > 0);
  if (sd != TQ_OK) return sd;
  return mp_bits_run(Xrot, x_dt, n, d, m, d_hi, bits_lo, bits_hi, wl_codes, s_wl, wh_codes, s_wh, Y, y_dt, ws,
                     ws_bytes, stream, acc_l, acc_h);
}

tq_status tq_linear_mp(const void* Xrot, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t d_hi,
                       const void* wl_codes, const float* s_wl, const void* wh_codes, const float* s_wh, void* Y,
                       tq_dtype y_dt, void* ws, size_t ws_bytes, hipStream_t stream) {
  return tq_linear_mp_bits(Xrot, x_dt, n, d, m, d_hi, 4, 8, wl_codes, s_wl, wh_codes, s_wh, Y, y_dt, ws, ws_bytes,
                           stream);
}

tq_status tq_linear_mp_workspace_offsets(int64_t n, int64_t d, int64_t d_hi, size_t off[4]) {
  if (n < 0 || d <= 0 || d_hi < 0 || d_hi > d) return TQ_ERR_SHAPE;
  if (!off) return TQ_ERR_NULL;
  const MpWs W = mp_ws(n, d, d_hi);
  off[0] = W.sxl;
  off[1] = W.sxh;
  off[2] = W.xl;
  off[3] = W.xh;
  return TQ_OK;
}

tq_status tq_weight_colsum(const void* w_codes, int64_t m, int64_t k, int bits, int32_t* colsum, hipStream_t stream) {
  if (bits != 4 && bits != 8) return TQ_ERR_BITS;
  if (m <= 0 || k <= 0 || m > kMaxDim || k > kMaxK || k % (bits == 4 ? 32 : 16)) return TQ_ERR_SHAPE;
  if (!w_codes || !colsum) return TQ_ERR_NULL;
  if (!aligned16(w_codes) || !aligned16(colsum)) return TQ_ERR_ALIGN;
  TQ_RUN("weight_colsum", stream, tq::launch_weight_colsum(w_codes, bits, (int)m, (int)k, colsum, stream));
  return TQ_OK;
}

size_t tq_linear_mp_asym_workspace_bytes(int64_t n, int64_t d, int64_t d_hi) {
  if (n < 0 || d <= 0 || d_hi < 0 || d_hi > d) return 0;
  return mp_asym_ws(n, d, d_hi).total;
}

tq_status tq_linear_mp_asym_workspace_offsets(int64_t n, int64_t d, int64_t d_hi, size_t off[6]) {
  if (n < 0 || d <= 0 || d_hi < 0 || d_hi > d) return TQ_ERR_SHAPE;
  if (!off) return TQ_ERR_NULL;
  const MpAsymWs W = mp_asym_ws(n, d, d_hi);
  off[0] = W.mp.sxl;
  off[1] = W.mp.sxh;
  off[2] = W.mp.xl;
  off[3] = W.mp.xh;
  off[4] = W.zl;
  off[5] = W.zh;
  return TQ_OK;
}

}  // extern "C"

namespace {

tq_status mp_asym_run(const void* Xrot, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t d_hi,
                      const void* wl_codes, const float* s_wl, const int32_t* colsum_l, const void* wh_codes,
                      const float* s_wh, const int32_t* colsum_h, void* Y, tq_dtype y_dt, void* ws, size_t ws_bytes,
                      hipStream_t stream, int32_t* acc_l, int32_t* acc_h) {
  const tq_status st = mp_check(Xrot, x_dt, n, d, d_hi, m, wl_codes, s_wl, wh_codes, s_wh, Y, y_dt, ws);
  if (st != TQ_OK) return st;
  if (d > tq::kAsymMaxD) return TQ_ERR_SHAPE;
  if (n == 0) return TQ_OK;
  const int64_t dl = d - d_hi;
  if ((dl > 0 && !colsum_l) || (d_hi > 0 && !colsum_h)) return TQ_ERR_NULL;
  if ((dl > 0 && !aligned16(colsum_l)) || (d_hi > 0 && !aligned16(colsum_h))) return TQ_ERR_ALIGN;
  const MpAsymWs W = mp_asym_ws(n, d, d_hi);
  if (ws_bytes < W.total) return TQ_ERR_WORKSPACE;
  uint8_t* base = (uint8_t*)ws;
  float* zl = (float*)(base + W.zl);
  float* zh = (float*)(base + W.zh);
  TQ_RUN("quant_rows_asym", stream,
         tq::launch_quant_rows_asym(Xrot, x_dt == TQ_BF16, (int)n, (int)d, (int)dl, base + W.mp.xl,
                                    (float*)(base + W.mp.sxl), zl, base + W.mp.xh, (float*)(base + W.mp.sxh), zh,
                                    stream));
  return mp_gemm(n, d, d_hi, m, wl_codes, s_wl, wh_codes, s_wh, Y, y_dt, W.mp, base, stream, zl, zh, colsum_l,
                 colsum_h, acc_l, acc_h);
}

}  // namespace

extern "C" {

tq_status tq_linear_mp_asym(const void* Xrot, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t d_hi,
                            const void* wl_codes, const float* s_wl, const int32_t* colsum_l, const void* wh_codes,
                            const float* s_wh, const int32_t* colsum_h, void* Y, tq_dtype y_dt, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  return mp_asym_run(Xrot, x_dt, n, d, m, d_hi, wl_codes, s_wl, colsum_l, wh_codes, s_wh, colsum_h, Y, y_dt, ws,
                     ws_bytes, stream, nullptr, nullptr);
}

tq_status tq_linear_mp_asym_debug(const void* Xrot, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t d_hi,
                                  const void* wl_codes, const float* s_wl, const int32_t* colsum_l,
                                  const void* wh_codes, const float* s_wh, const int32_t* colsum_h, void* Y,
                                  tq_dtype y_dt, void* ws, size_t ws_bytes, int32_t* acc_l, int32_t* acc_h,
                                  hipStream_t stream) {
  if (n > 0) {
    const tq_status sd = debug_check(acc_l, acc_h, d_hi > 0);
    if (sd != TQ_OK) return sd;
  }
  return mp_asym_run(Xrot, x_dt, n, d, m, d_hi, wl_codes, s_wl, colsum_l, wh_codes, s_wh, colsum_h, Y, y_dt, ws,
                     ws_bytes, stream, acc_l, acc_h);
}

size_t tq_rht_bytes(int64_t d) {
  if (d <= 0 || d % 128 || d > tq::kRhtMaxD) return 0;
  return tq::rht_bytes((int)d);
}

tq_status tq_pack_rht(const float* signs, const int32_t* perm, int64_t d, void* rot, hipStream_t stream) {
  if (d <= 0 || d % 128 || d > tq::kRhtMaxD) return TQ_ERR_SHAPE;
  if (!signs || !perm || !rot) return TQ_ERR_NULL;
  if (!aligned16(rot)) return TQ_ERR_ALIGN;
  TQ_RUN("pack_rht", stream, tq::launch_pack_rht(signs, perm, (int)d, rot, stream));
  return TQ_OK;
}

tq_status tq_linear_mp_rht(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t d_hi,
                           const void* rot, const void* wl_codes, const float* s_wl, const void* wh_codes,
                           const float* s_wh, void* Y, tq_dtype y_dt, void* ws, size_t ws_bytes, hipStream_t stream) {
  const tq_status st = mp_check(X, x_dt, n, d, d_hi, m, wl_codes, s_wl, wh_codes, s_wh, Y, y_dt, ws);
  if (st != TQ_OK) return st;
  if (d % 128 || d > tq::kRhtMaxD) return TQ_ERR_SHAPE;
  if (n == 0) return TQ_OK;
  if (!rot) return TQ_ERR_NULL;
  if (!aligned16(rot)) return TQ_ERR_ALIGN;
  const MpWs W = mp_ws(n, d, d_hi);
  if (ws_bytes < W.total) return TQ_ERR_WORKSPACE;
  uint8_t* base = (uint8_t*)ws;
  TQ_RUN("quant_rows_rht", stream,
         tq::launch_quant_rows_rht(X, x_dt == TQ_BF16, (int)n, (int)d, (int)(d - d_hi), rot, base + W.xl,
                                   (float*)(base + W.sxl), base + W.xh, (float*)(base + W.sxh), stream));
  return mp_gemm(n, d, d_hi, m, wl_codes, s_wl, wh_codes, s_wh, Y, y_dt, W, base, stream);
}

// Workspace of tq_linear_asym: the two-launch layout of tq_linear, then the
// zero-points.
size_t asym_zx_offset(const LinearWs& L) { return L.total; }
size_t asym_total(const LinearWs& L, int64_t n) { return align256(L.total + (size_t)n * 4); }

size_t tq_linear_asym_workspace_bytes(int64_t n, int64_t d, int64_t m, int64_t r) {
  if (n < 0 || d <= 0 || m <= 0 || r < 0 || r > 256) return 0;
  return asym_total(linear_ws(n, d, m, r_padded(r), true), n);  // two-launch layout
}

tq_status tq_linear_asym_workspace_offsets(int64_t n, int64_t d, int64_t m, int64_t r, size_t off[4]) {
  if (n < 0 || d <= 0 || m <= 0 || r < 0 || r > 256) return TQ_ERR_SHAPE;
  if (!off) return TQ_ERR_NULL;
  const LinearWs L = linear_ws(n, d, m, r_padded(r), true);
  off[0] = L.sx;
  off[1] = L.xc;
  off[2] = asym_zx_offset(L);
  off[3] = L.t;
  return TQ_OK;
}

}  // extern "C"

namespace {

tq_status asym_run(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r, const void* w_codes,
                   const float* s_w, const int32_t* colsum, const void* lowrank, void* Y, tq_dtype y_dt, void* ws,
                   size_t ws_bytes, hipStream_t stream, int32_t* acc) {
  const tq_status st = linear_check(X, x_dt, n, d, m, r, w_codes, s_w, lowrank, Y, y_dt, ws);
  if (st != TQ_OK || n == 0) return st;
  if (d > tq::kAsymMaxD) return TQ_ERR_SHAPE;
  if (!colsum) return TQ_ERR_NULL;
  if (!aligned16(colsum)) return TQ_ERR_ALIGN;
  const int rp = (int)r_padded(r);
  const LinearWs L = linear_ws(n, d, m, rp, true);
  if (ws_bytes < asym_total(L, n)) return TQ_ERR_WORKSPACE;
  uint8_t* base = (uint8_t*)ws;
  float* sx = (float*)(base + L.sx);
  float* zx = (float*)(base + asym_zx_offset(L));
  uint8_t* xc = base + L.xc;
  tq::bf16_t* T = (tq::bf16_t*)(base + L.t);
  const tq::bf16_t* L1t = (const tq::bf16_t*)lowrank;
  float* P = (float*)(base + L.p);
  GemmArgs g{};
  g.A = xc;
  g.lda = L.small ? d / 2 : d;  // codes u - 8: nibble-packed for the small-n GEMM, else int8
  g.B = (const uint8_t*)w_codes;
  g.ldb = d / 2;
  g.M = (int)n;
  g.N = (int)m;
  g.Kb = (int)(d / 2);
  g.sx = sx;
  g.sw = s_w;
  g.T = rp ? T : nullptr;
  g.L2t = lowrank ? L1t + (size_t)rp * d : nullptr;
  g.r_pad = rp;
  g.ldt = rp;
  g.groups.n = 1;
  g.groups.start[1] = (int)m;
  g.zx = zx;
  g.csw = colsum;
  g.Y = Y;
  g.ldy = m;
  g.y_bf16 = y_dt == TQ_BF16;
  g.acc = acc;
  const bool xb = x_dt == TQ_BF16;
  if (L.fusable && tq::gemv_fused_fits((int)n, (int)(d / 2), (int)m, L.fplan.nqb + L.fplan.ntb, xb, acc != nullptr)) {
    // one launch, as tq_linear's few-token layer, with the asymmetric quantiser in the producers
    const tq::ProloguePlan& fp = L.fplan;
    tq::SmallFuse f{};
    f.pa = tq::PrologueArgs{X, (int)n, (int)d, L1t, rp, fp.kc, fp.nchunk, fp.qs, fp.nqg, fp.nqb, 1, 1, 0, xc, sx, P,
                            rp ? T : nullptr, (unsigned*)(base + L.ctr)};
    f.zx = zx;
    f.nprod = fp.nqb + fp.ntb;
    f.sync = (unsigned*)(base + L.sync);
    f.spin = kDecodeSpin;
    g.P = rp ? P : nullptr;
    g.nchunk = fp.nchunk;
    g.Tout = rp ? T : nullptr;
    TQ_RUN("small_fused_asym", stream, tq::launch_gemv_fused(g, f, xb, stream));
    return TQ_OK;
  }
  TQ_RUN("prologue_asym", stream,
         tq::launch_prologue_asym(X, xb, (int)n, (int)d, L1t, rp, L.plan, xc, sx, zx, P, rp ? T : nullptr,
                                  (unsigned*)(base + L.ctr), stream));
  if (L.small) {
    if (rp && (L.plan.partial || L.plan.sum_to_p0)) {
      g.P = P;
      g.nchunk = L.plan.partial ? L.plan.nchunk : 1;
      g.Tout = T;
    }
    TQ_RUN("gemm_small_n_asym", stream, tq::launch_gemv(g, 4, tq::EPI_LINEAR, stream));
  } else {
    TQ_RUN("gemm_asym", stream, tq::launch_gemm8(g, tq::EPI_LINEAR, true, 4, stream));
  }
  return TQ_OK;
}

}  // namespace

extern "C" {

tq_status tq_linear_asym(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r,
                         const void* w_codes, const float* s_w, const int32_t* colsum, const void* lowrank, void* Y,
                         tq_dtype y_dt, void* ws, size_t ws_bytes, hipStream_t stream) {
  return asym_run(X, x_dt, n, d, m, r, w_codes, s_w, colsum, lowrank, Y, y_dt, ws, ws_bytes, stream, nullptr);
}

tq_status tq_linear_asym_debug(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r,
                               const void* w_codes, const float* s_w, const int32_t* colsum, const void* lowrank,
                               void* Y, tq_dtype y_dt, void* ws, size_t ws_bytes, int32_t* acc, hipStream_t stream) {
  if (n > 0) {
    const tq_status sd = debug_check(acc, nullptr, false);
    if (sd != TQ_OK) return sd;
  }
  return asym_run(X, x_dt, n, d, m, r, w_codes, s_w, colsum, lowrank, Y, y_dt, ws, ws_bytes, stream, acc);
}

size_t tq_lowrank_q_bytes(int64_t d, int64_t m, int64_t r) {
  if (d <= 0 || m <= 0 || r < 1 || r > 256) return 0;
  return qlr_pack(d, m, r_padded(r)).total;
}

tq_status tq_pack_lowrank_q(const void* U, const void* V, tq_dtype dt, int64_t d, int64_t m, int64_t r,
                            void* lowrank_q, hipStream_t stream) {
  if (!valid_dtype(dt)) return TQ_ERR_DTYPE;
  if (d <= 0 || m <= 0 || d > kMaxDim || m > kMaxDim || d % 32 || r < 1 || r > 256) return TQ_ERR_SHAPE;
  if (!U || !V || !lowrank_q) return TQ_ERR_NULL;
  if (!aligned16(lowrank_q)) return TQ_ERR_ALIGN;
  const int rp = (int)r_padded(r);
  const QlrPack P = qlr_pack(d, m, rp);
  uint8_t* b = (uint8_t*)lowrank_q;
  const bool bf = dt == TQ_BF16;
  // U (d x r) per column -> r_pad code rows of d; V (r x m) per column -> m code rows of r_pad
  TQ_RUN("pack_lowrank_q_u", stream,
         tq::launch_pack_weight_padded(U, bf, (int)d, rp, (int)r, (int)d, (int)r, 4, b + P.uc, (float*)(b + P.su),
                                       stream));
  TQ_RUN("pack_lowrank_q_v", stream,
         tq::launch_pack_weight_padded(V, bf, rp, (int)m, (int)m, (int)r, (int)m, 4, b + P.vc, (float*)(b + P.sv),
                                       stream));
  return TQ_OK;
}

size_t tq_linear_qlr_workspace_bytes(int64_t n, int64_t d, int64_t r) {
  if (n < 0 || d <= 0 || r < 1 || r > 256) return 0;
  return qlr_ws(n, d, r_padded(r)).total;
}

tq_status tq_linear_qlr_workspace_offsets(int64_t n, int64_t d, int64_t r, size_t off[4]) {
  if (n < 0 || d <= 0 || r < 1 || r > 256) return TQ_ERR_SHAPE;
  if (!off) return TQ_ERR_NULL;
  const QlrWs W = qlr_ws(n, d, r_padded(r));
  off[0] = W.sx;
  off[1] = W.xc;
  off[2] = W.st;
  off[3] = W.tc;
  return TQ_OK;
}

}  // extern "C"

namespace {

tq_status qlr_run(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r, const void* w_codes,
                  const float* s_w, const void* lowrank_q, void* Y, tq_dtype y_dt, void* ws, size_t ws_bytes,
                  hipStream_t stream, int32_t* acc, int32_t* acc2) {
  if (r < 1) return TQ_ERR_SHAPE;
  const tq_status st = linear_check(X, x_dt, n, d, m, r, w_codes, s_w, lowrank_q, Y, y_dt, ws);
  if (st != TQ_OK || n == 0) return st;
  const int64_t rp = r_padded(r);
  const QlrWs W = qlr_ws(n, d, rp);
  if (ws_bytes < W.total) return TQ_ERR_WORKSPACE;
  const QlrPack P = qlr_pack(d, m, rp);
  uint8_t* base = (uint8_t*)ws;
  const uint8_t* lq = (const uint8_t*)lowrank_q;
  float* sx = (float*)(base + W.sx);
  uint8_t* xc = base + W.xc;
  float* stt = (float*)(base + W.st);
  uint8_t* tc = base + W.tc;
  // few tokens: nibble-packed activation codes for the weight-streaming
  // small-n GEMM; otherwise int8 codes for the tile GEMM
  const bool small = n <= kSmallN;
  const bool xb = x_dt == TQ_BF16;
  if (tq::qlr_fused_ok((int)d, (int)rp)) {
    TQ_RUN("qlr_prologue", stream,
           tq::launch_qlr_prologue(X, xb, (int)n, (int)d, lq + P.uc, (const float*)(lq + P.su), (int)rp, xc, sx, tc,
                                   stt, small, stream));
  } else {
    if (small)
      TQ_RUN("quant_rows_qlr", stream,
             tq::launch_quant_rows_fast(X, xb, (int)n, (int)d, (int)d, 4, 4, xc, sx, nullptr, nullptr, stream));
    else
      TQ_RUN("quant_rows_qlr", stream,
             tq::launch_quant_rows_i8(X, xb, (int)n, (int)d, (int)d, 4, xc, sx, nullptr, nullptr, stream));
    TQ_RUN("qlr_stage1", stream,
           tq::launch_qlr_stage1(xc, (int)n, (int)d, lq + P.uc, (const float*)(lq + P.su), (int)rp, tc, stt, small,
                                 stream));
  }
  GemmArgs g{};
  g.A = xc;
  g.lda = small ? d / 2 : d;
  g.B = (const uint8_t*)w_codes;
  g.ldb = d / 2;
  g.M = (int)n;
  g.N = (int)m;
  g.Kb = (int)(d / 2);
  g.sx = sx;
  g.sw = s_w;
  g.r_pad = (int)rp;
  g.Vq = lq + P.vc;
  g.sv = (const float*)(lq + P.sv);
  g.Tq = tc;
  g.st = stt;
  g.Y = Y;
  g.ldy = m;
  g.y_bf16 = y_dt == TQ_BF16;
  g.acc = acc;
  g.acc2 = acc2;
  if (small)
    TQ_RUN("gemm_small_n_qlr", stream, tq::launch_gemv(g, 4, tq::EPI_QLR, stream));
  else
    TQ_RUN("gemm_qlr", stream, tq::launch_gemm8(g, tq::EPI_QLR, true, 4, stream));
  return TQ_OK;
}

}  // namespace

extern "C" {

tq_status tq_linear_qlr(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r, const void* w_codes,
                        const float* s_w, const void* lowrank_q, void* Y, tq_dtype y_dt, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  return qlr_run(X, x_dt, n, d, m, r, w_codes, s_w, lowrank_q, Y, y_dt, ws, ws_bytes, stream, nullptr, nullptr);
}

tq_status tq_linear_qlr_debug(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r,
                              const void* w_codes, const float* s_w, const void* lowrank_q, void* Y, tq_dtype y_dt,
                              void* ws, size_t ws_bytes, int32_t* acc, int32_t* acc2, hipStream_t stream) {
  if (n > 0) {
    const tq_status sd = debug_check(acc, acc2, true);
    if (sd != TQ_OK) return sd;
  }
  return qlr_run(X, x_dt, n, d, m, r, w_codes, s_w, lowrank_q, Y, y_dt, ws, ws_bytes, stream, acc, acc2);
}

tq_status tq_debug_accumulate(const void* x_codes, const void* w_codes, int64_t n, int64_t k, int64_t m, int bits,
                              int32_t* acc, hipStream_t stream) {
  if (bits != 4 && bits != 8) return TQ_ERR_BITS;
  if (n < 0 || n > kMaxDim || k <= 0 || k > kMaxK || m <= 0 || m > kMaxDim || k % (bits == 4 ? 32 : 16))
    return TQ_ERR_SHAPE;
  if (n == 0) return TQ_OK;
  if (!x_codes || !w_codes || !acc) return TQ_ERR_NULL;
  if (!aligned16(x_codes) || !aligned16(w_codes) || !aligned16(acc)) return TQ_ERR_ALIGN;
  GemmArgs g{};
  g.A = (const uint8_t*)x_codes;
  g.B = (const uint8_t*)w_codes;
  g.lda = g.ldb = k * bits / 8;
  g.M = (int)n;
  g.N = (int)m;
  g.Kb = (int)(k * bits / 8);
  g.acc = acc;
  if (n <= kSmallN)
    TQ_RUN("gemm_small_n_acc", stream, tq::launch_gemv(g, bits, tq::EPI_ACC, stream));
  else  // the main loop of tq_linear's tile GEMM (4-bit: on packed activation codes)
    TQ_RUN("gemm_acc", stream, tq::launch_gemm8(g, tq::EPI_ACC, bits == 8, bits, stream));
  return TQ_OK;
}

tq_status tq_debug_accumulate_i8(const void* x_codes, const void* w_codes, int64_t n, int64_t k, int64_t m,
                                 int32_t* acc, hipStream_t stream) {
  if (n < 0 || n > kMaxDim || k <= 0 || k > kMaxK || m <= 0 || m > kMaxDim || k % 32) return TQ_ERR_SHAPE;
  if (n == 0) return TQ_OK;
  if (!x_codes || !w_codes || !acc) return TQ_ERR_NULL;
  if (!aligned16(x_codes) || !aligned16(w_codes) || !aligned16(acc)) return TQ_ERR_ALIGN;
  GemmArgs g{};
  g.A = (const uint8_t*)x_codes;
  g.lda = k;  // one int8 byte per code
  g.B = (const uint8_t*)w_codes;
  g.ldb = k / 2;
  g.M = (int)n;
  g.N = (int)m;
  g.Kb = (int)(k / 2);
  g.acc = acc;
  TQ_RUN("gemm_acc_i8", stream, tq::launch_gemm8(g, tq::EPI_ACC, true, 4, stream));
  return TQ_OK;
}

tq_status tq_debug_gemm_w4a4(const void* x_codes, int x_packed, const float* s_x, const void* w_codes,
                             const float* s_w, int64_t n, int64_t k, int64_t m, void* Y, hipStream_t stream) {
  if (n < 0 || n > kMaxDim || k <= 0 || k > kMaxK || m <= 0 || m > kMaxDim || k % 32) return TQ_ERR_SHAPE;
  if (n == 0) return TQ_OK;
  if (!x_codes || !s_x || !w_codes || !s_w || !Y) return TQ_ERR_NULL;
  if (!aligned16(x_codes) || !aligned16(w_codes) || !aligned16(Y)) return TQ_ERR_ALIGN;
  GemmArgs g{};
  g.A = (const uint8_t*)x_codes;
  g.lda = x_packed ? k / 2 : k;
  g.B = (const uint8_t*)w_codes;
  g.ldb = k / 2;
  g.M = (int)n;
  g.N = (int)m;
  g.Kb = (int)(k / 2);
  g.sx = s_x;
  g.sw = s_w;
  g.groups.n = 1;
  g.groups.start[1] = (int)m;
  g.Y = Y;
  g.ldy = m;
  g.y_bf16 = 1;
  TQ_RUN(x_packed ? "gemm_w4a4_packed_x" : "gemm_w4a4_int8_x", stream,
         tq::launch_gemm8(g, tq::EPI_LINEAR, !x_packed, 4, stream));
  return TQ_OK;
}

tq_status tq_profile_enable(int on) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  p.on = on != 0;
  return TQ_OK;
}

int tq_profile_read(tq_kernel_stat* out, int max) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  std::vector<tq_kernel_stat> stats;
  for (const ProfRecord& r : p.recs) {
    if (hipEventSynchronize(r.e1) != hipSuccess) return TQ_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess) return TQ_ERR_HIP;
    tq_kernel_stat* s = nullptr;
    for (auto& x : stats)
      if (r.name == x.name) s = &x;
    if (!s) {
      tq_kernel_stat z{};
      strncpy(z.name, r.name.c_str(), sizeof(z.name) - 1);
      stats.push_back(z);
      s = &stats.back();
    }
    s->launches += 1;
    s->total_ms += ms;
  }
  const int k = (int)stats.size();
  if (out)
    for (int i = 0; i < k && i < max; ++i) out[i] = stats[i];
  return k;
}

tq_status tq_profile_reset(void) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  for (const ProfRecord& r : p.recs) {
    p.pool.push_back(r.e0);
    p.pool.push_back(r.e1);
  }
  p.recs.clear();
  return TQ_OK;
}

}  // extern "C"
