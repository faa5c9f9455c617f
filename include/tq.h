/*
 * tq.h -- C ABI of the rank-augmented W4A4 linear layer for MI355X (gfx950).
 *
 * The layer computes, for activations X (n x d) and a weight split into a
 * residual R (d x m) and low-rank factors L1 (d x r), L2 (r x m),
 *
 *     Y = s_x s_w^T (.) (Q4(X) Q4(R)) + (X L1) L2                           (1)
 *
 * the low-rank + residual form of the SVDQuant/TwinQuant line of work
 * ("TwinQuant: Learnable Subspace Decomposition for W4A4 LLM Quantization",
 * section 02.A; one shared epilogue as in section 04.C, Figure 4), and the
 * two-subspace mixed-precision form
 *
 *     Y = Q_l(X_l) Q_l(W_l) + Q_h(X_h) Q_h(W_h)                             (2)
 *
 * of "CoQuant: Joint Weight-Activation Subspace Projection for
 * Mixed-Precision LLMs", Eq. 9, on activations and weights already rotated by
 * an orthogonal U (CoQuant Eq. 3, 6, 7).
 *
 * Quantiser (TwinQuant notes section 02, quantization formula; CoQuant Eq. 1
 * with zero-point 0): per row of X (token) and per output channel of the
 * weight, amax = max|v|, s = fl32(amax / q_max) with q_max = 2^(bits-1) - 1,
 * code = clamp(rne(fl32(v / s)), -2^(bits-1), q_max); rne rounds half to
 * even, fl32 is an IEEE fp32 division; a row whose s is 0 gets codes 0.
 * Codes and their integer products are exact; the integer product of the
 * residual is accumulated exactly in int32 (TwinQuant notes section 02 and
 * Figure 4).
 *
 * Conventions for every entry point:
 *  - Every pointer is a DEVICE pointer (memory of the current HIP device),
 *    except where stated.  The caller owns all memory; the library never
 *    allocates device memory and keeps no state between calls except the
 *    optional profiling record (tq_profile_*, guarded by a lock) and the
 *    file-scope scratch array of tq_linear_noalloc.
 *  - Every call is asynchronous on `stream` (0 = the null stream).  A status
 *    other than TQ_OK from argument checking means nothing was enqueued.
 *    TQ_ERR_HIP reports a launch failure (hipGetLastError after the launch);
 *    faults during execution surface at the caller's next synchronisation.
 *  - Matrices are row-major and densely packed.  Device pointers must be
 *    16-byte aligned (TQ_ERR_ALIGN otherwise).
 *  - Codes: 4-bit codes are two's-complement nibbles, two per byte, the even
 *    index of each pair in the low nibble; 8-bit codes are int8.  A code
 *    matrix of `rows` x `k` therefore occupies rows * k * bits / 8 bytes, the
 *    k dimension contiguous ("K-contiguous").
 *  - Shapes: n == 0 is a valid no-op.  d must be a positive multiple of 32 and
 *    m positive; any n and m are handled (no tile multiple needed).  r may be
 *    0..256.  Reduction lengths (d of tq_linear and tq_linear_mp, k of
 *    tq_debug_accumulate) are at most 65536, which keeps every int32
 *    accumulator exact.  Non-finite inputs are outside the contract (codes unspecified).
 *  - Calls that share a workspace must not overlap in time.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_NULL = -1,      /* a required pointer is NULL */
  TQ_ERR_SHAPE = -2,     /* a size is out of range or breaks a multiple-of rule */
  TQ_ERR_DTYPE = -3,     /* unsupported element type */
  TQ_ERR_BITS = -4,      /* unsupported bit width */
  TQ_ERR_ALIGN = -5,     /* a pointer is not 16-byte aligned */
  TQ_ERR_WORKSPACE = -6, /* workspace smaller than the queried size */
  TQ_ERR_HIP = -7        /* the HIP runtime reported an error */
} tq_status;

typedef enum { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;

/* Human-readable name of a status (static string, never NULL). */
const char* tq_status_string(tq_status s);

/* ABI version of this header (major * 100 + minor). */
int tq_version(void);

/* Bytes of a code matrix: rows * k * bits / 8, with 3- and 6-bit codes stored
 * like 4- and 8-bit ones (0 for invalid arguments). */
size_t tq_codes_bytes(int64_t rows, int64_t k, int bits);

/*
 * tq_pack_weight -- offline per-output-channel symmetric quantisation.
 *   W       d x m weight (Y = X W), element type w_dt (TQ_F32 or TQ_BF16).
 *   bits    4 or 8; or 3 or 6 (the 6/3-bit two-subspace layer: q_max 3 or
 *           31, stored like 4 or 8 bits).
 *   w_codes out: m x tq_codes_bytes(1, d, bits) bytes; row j holds output
 *           channel j (column j of W) with k contiguous.
 *   s_w     out: m fp32 scales.
 * Per-channel symmetric weights follow CoQuant's experimental protocol (the
 * ResQ setting: per-channel symmetric weight quantisation).
 */
tq_status tq_pack_weight(const void* W, tq_dtype w_dt, int64_t d, int64_t m, int bits,
                         void* w_codes, float* s_w, hipStream_t stream);

/* Bytes of the packed low-rank factors of tq_pack_lowrank. */
size_t tq_lowrank_bytes(int64_t d, int64_t m, int64_t r);

/*
 * tq_pack_lowrank -- lays out the low-rank factors for tq_linear (offline).
 *   L1      d x r, L2 r x m, element type dt (TQ_F32 values are rounded to
 *           bf16, ties to even; TQ_BF16 values are copied).
 *   lowrank out: tq_lowrank_bytes(d, m, r) bytes, an opaque bf16 layout
 *           (L1 and L2 transposed, r padded with zeros to a multiple of 32).
 * The factors U, V of TwinQuant notes section 02.A (L1 = U, L2 = V).
 */
tq_status tq_pack_lowrank(const void* L1, const void* L2, tq_dtype dt, int64_t d, int64_t m,
                          int64_t r, void* lowrank, hipStream_t stream);

/*
 * Layers that share one input (CoQuant notes, "CoQuant: Joint Weight-
 * Activation Subspace Projection for Mixed-Precision LLMs", the grouping of
 * linear layers with identical input activations around Eq. 14: Q/K/V, and
 * gate/up).  G layers of m[0..G-1] output channels and a common rank r are
 * stacked along the output channels: one quantisation of X and one T for
 * all of them, then one integer GEMM over m_total = sum m[g] channels.
 * Shapes: 1 <= G <= 8; every m[g] but the last a multiple of 256;
 * G * r_pad <= 256 (r_pad = r rounded up to a power of two, at least 32).
 */

/* Bytes of the packed low-rank factors of tq_pack_lowrank_group (0 for invalid shapes). */
size_t tq_lowrank_group_bytes(int64_t d, const int64_t* m, int64_t G, int64_t r);

/*
 * tq_pack_lowrank_group -- lays out the G layers' low-rank factors (offline).
 *   L1[g]   d x r, L2[g] r x m[g] (host array of G device pointers each),
 *           element type dt, rounded or copied to bf16 as in tq_pack_lowrank.
 *   m       host array of G channel counts.
 *   lowrank out: tq_lowrank_group_bytes(d, m, G, r) bytes, an opaque bf16
 *           layout (all L1 transposed and stacked, then all L2 transposed and
 *           stacked in channel order, zero-padded).
 */
tq_status tq_pack_lowrank_group(const void* const* L1, const void* const* L2, tq_dtype dt, int64_t d,
                                const int64_t* m, int64_t G, int64_t r, void* lowrank,
                                hipStream_t stream);

/* Workspace bytes tq_linear_group needs for these sizes (0 for invalid shapes). */
size_t tq_linear_group_workspace_bytes(int64_t n, int64_t d, const int64_t* m, int64_t G,
                                       int64_t r);

/*
 * tq_linear_group -- G layers on one input X (n x d, x_dt):
 *   Y[:, M_g + j] = layer g's tq_linear output, channel j (M_g = sum of m[h], h < g).
 *   w_codes  m_total x d/2 bytes: the G layers' tq_pack_weight codes stacked in
 *            channel order (layer g at row M_g); s_w m_total fp32 likewise.
 *   lowrank  from tq_pack_lowrank_group, or NULL iff r == 0.
 *   Y        out, n x m_total row-major, y_dt.
 *   ws       device workspace of at least tq_linear_group_workspace_bytes,
 *            zero-filled once before first use (as for tq_linear).
 * Every layer's codes, scales and Y are those tq_linear gives for it alone.
 * Errors as tq_linear, plus TQ_ERR_SHAPE for group shapes outside the above.
 */
tq_status tq_linear_group(const void* X, tq_dtype x_dt, int64_t n, int64_t d, const int64_t* m,
                          int64_t G, int64_t r, const void* w_codes, const float* s_w,
                          const void* lowrank, void* Y, tq_dtype y_dt, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * tq_quantize_act -- per-token symmetric quantisation of activations.
 *   X       n x d, element type x_dt.  bits 4 or 8.
 *   x_codes out: n x (d*bits/8) bytes.   s_x out: n fp32 scales.
 * In the fused layer the activations are quantised inside the residual
 * GEMM's launch sequence (TwinQuant notes section 04.C); the scales are per
 * token (CoQuant, experimental protocol).
 */
tq_status tq_quantize_act(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int bits,
                          void* x_codes, float* s_x, hipStream_t stream);

/* Workspace bytes tq_linear needs for these sizes (0 for shapes tq_linear rejects). */
size_t tq_linear_workspace_bytes(int64_t n, int64_t d, int64_t m, int64_t r);

/*
 * tq_linear -- the rank-augmented quantised linear layer, equation (1).
 *   X        n x d activations (x_dt), quantised per token at 4 bits inside
 *            the call; the low-rank branch takes X itself (as bf16).
 *   w_codes, s_w   the residual from tq_pack_weight(R, ..., bits = 4).
 *   lowrank  from tq_pack_lowrank(L1, L2, ...), or NULL iff r == 0.
 *   Y        out: n x m, element type y_dt (TQ_BF16 or TQ_F32), rounded to
 *            nearest even from the fp32 epilogue.
 *   ws       device workspace of at least tq_linear_workspace_bytes(n,d,m,r)
 *            bytes.  It starts with completion counters (of the low-rank
 *            stage, and of the hand-off inside the few-token launch):
 *            zero-fill the workspace once before its first use (e.g.
 *            hipMemset after allocating it); every call leaves the counters
 *            zero again, and the rest is scratch whose contents on entry are
 *            ignored.  Calls that share a workspace must be ordered (one
 *            stream, or synchronised streams).
 * For n <= 32 the call runs a memory-bound path (weight codes streamed once).
 * It is one launch for n <= 2, d <= 16384 and n d <= 16384 (and at most 128
 * partial blocks of T: ceil(d / 512) r_pad / 16 <= 128: the decode kernel),
 * and for any other n <= 16 with d <= 16384 whose grid is at most a
 * quarter larger than what the GPU holds at once (the few-token GEMM, whose
 * first blocks quantise X and compute partials of T; on MI355X 1024 blocks of
 * 16 output channels for d <= 4096, 256 above); otherwise two launches.  In a one-launch path, weight-streaming blocks read what other
 * blocks of the same launch store; their waits are bounded: a wait that gives
 * up sets word 32 of the hand-off words (off[3] of
 * tq_linear_workspace_offsets), writes NaN to the block's outputs, and every
 * later call on that workspace writes NaN everywhere until it is zero-filled
 * again.  For n > 32 a tiled MFMA path.  All paths produce bit-identical
 * integer accumulators.
 */
tq_status tq_linear(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r,
                    const void* w_codes, const float* s_w, const void* lowrank,
                    void* Y, tq_dtype y_dt, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * tq_linear_noalloc -- tq_linear for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and the same Y, bit for bit.  The workspace is a file-scope device
 * array of TQ_NOALLOC_SCRATCH_BYTES, one per device, which the library keeps
 * until the process ends; its first use on a device looks up its address and
 * clears its counters with one small kernel on `stream`.  No call allocates
 * or frees memory.  Returns TQ_ERR_WORKSPACE when
 * tq_linear_workspace_bytes(n, d, m, r) exceeds TQ_NOALLOC_SCRATCH_BYTES
 * (nothing enqueued); other errors as tq_linear.  Every call on a device
 * shares that device's array: calls that overlap in time on one device
 * (different streams without ordering, or several host threads) race and
 * give undefined results.
 */
#define TQ_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
tq_status tq_linear_noalloc(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r,
                            const void* w_codes, const float* s_w, const void* lowrank, void* Y, tq_dtype y_dt,
                            hipStream_t stream);

/*
 * tq_linear_workspace_offsets -- where tq_linear keeps its intermediate
 * results inside the workspace, for inspection after a call:
 *   off[0] s_x (n fp32), off[1] activation codes: nibble-packed (n x d/2
 *   bytes) for n <= 32; for n > 32 one int8 byte per code, each row of d
 *   bytes listing, for every 8 consecutive k, the 4 even-k codes and then
 *   the 4 odd-k codes (the order in which the tile GEMM consumes them),
 *   off[2] T = X L1 (n x r_pad bf16, r_pad = r rounded up to a power of two
 *   >= 32; absent when r == 0), off[3] the 4 KiB of uint32 hand-off words:
 *   word 0 the call counter of the decode kernel (advanced by one per call),
 *   word 32 the wait-limit flag (zero unless a wait gave up), every other
 *   word a counter that is zero between calls.
 *   Returns TQ_ERR_SHAPE for invalid sizes.
 */
tq_status tq_linear_workspace_offsets(int64_t n, int64_t d, int64_t m, int64_t r, size_t off[4]);

/* Workspace bytes tq_linear_mp needs for these sizes. */
size_t tq_linear_mp_workspace_bytes(int64_t n, int64_t d, int64_t d_hi);

/*
 * tq_linear_mp -- the two-subspace mixed-precision layer.
 *   Xrot     n x d rotated activations (x_dt).  The first d - d_hi columns
 *            are the low-precision subspace (4 bits), the last d_hi columns
 *            the high-precision subspace (8 bits); each subspace has its own
 *            per-token scale.  d - d_hi must be a multiple of 32 and d_hi a
 *            multiple of 16 (either may be 0).
 *   wl_codes, s_wl  tq_pack_weight of the first d - d_hi rows of the rotated
 *            weight at bits = 4;  wh_codes, s_wh  of the last d_hi rows at
 *            bits = 8 (NULL allowed when d_hi == 0).
 *   Y, y_dt, ws, ws_bytes as in tq_linear (workspace from
 *            tq_linear_mp_workspace_bytes).
 * CoQuant Eq. 9 with 8-bit high-precision and 4-bit low-precision subspaces
 * (CoQuant experimental protocol).
 */
tq_status tq_linear_mp(const void* Xrot, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t d_hi,
                       const void* wl_codes, const float* s_wl, const void* wh_codes,
                       const float* s_wh, void* Y, tq_dtype y_dt, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/*
 * tq_linear_mp_bits -- tq_linear_mp at other bit widths: (bits_lo, bits_hi) =
 * (4, 8), or (3, 6), the other pair of CoQuant's experimental protocol (1/8 of
 * the channels at 6 bits, the rest at 3); the weights packed by
 * tq_pack_weight at those widths.  Codes keep the 4- and 8-bit storage, so the
 * same kernels run.  TQ_ERR_BITS for other pairs; otherwise as tq_linear_mp.
 */
tq_status tq_linear_mp_bits(const void* Xrot, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t d_hi,
                            int bits_lo, int bits_hi, const void* wl_codes, const float* s_wl,
                            const void* wh_codes, const float* s_wh, void* Y, tq_dtype y_dt, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * Byte offsets inside the tq_linear_mp (and tq_linear_mp_rht) workspace:
 *   off[0] s_x of the 4-bit subspace (n fp32), off[1] s_x of the 8-bit
 *   subspace (n fp32), off[2] the 4-bit codes (n x (d - d_hi) bytes, one int8
 *   per code, per 8 columns the 4 even then the 4 odd ones), off[3] the
 *   8-bit codes (n x d_hi int8).  TQ_ERR_SHAPE / TQ_ERR_NULL on bad arguments.
 */
tq_status tq_linear_mp_workspace_offsets(int64_t n, int64_t d, int64_t d_hi, size_t off[4]);

/*
 * Online rotation (CoQuant notes, the randomised block-Hadamard rotation after
 * Eq. 3; "Quantizing With Randomized Hadamard Transforms: Efficient
 * Heuristic Now Proven"): U = diag(signs) . blockdiag(H_128) / sqrt(128) . P,
 * X' = X U with X'[:, j] = (X diag(signs) blockdiag(H_128) / sqrt(128))[:, perm[j]].
 * d must be a multiple of 128 and at most 8192.
 */

/* Bytes of the packed rotation of tq_pack_rht (0 for unsupported d). */
size_t tq_rht_bytes(int64_t d);

/*
 * tq_pack_rht -- lays out a rotation for tq_linear_mp_rht (offline).
 *   signs  d fp32 values, +-1 (negative means -1).
 *   perm   d int32: a permutation of 0 .. d-1 (position j takes rotated
 *          coordinate perm[j]); for anything else the layer's output is
 *          unspecified (no access leaves the buffers).
 *   rot    out: tq_rht_bytes(d) bytes.
 */
tq_status tq_pack_rht(const float* signs, const int32_t* perm, int64_t d, void* rot, hipStream_t stream);

/*
 * tq_linear_mp_rht -- tq_linear_mp on unrotated X (n x d, x_dt): the rotation
 * (from tq_pack_rht) is applied to every token row in fp32 inside the
 * quantiser -- butterflies of increasing span, each (a + b, a - b), then one
 * multiply by fl32(1 / sqrt(128)) -- and X' is never stored.  The weights are
 * those of tq_linear_mp for the rotated weight U^T W.  Workspace and errors as
 * tq_linear_mp, plus TQ_ERR_SHAPE for d outside the rotation's range.
 */
tq_status tq_linear_mp_rht(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t d_hi,
                           const void* rot, const void* wl_codes, const float* s_wl, const void* wh_codes,
                           const float* s_wh, void* Y, tq_dtype y_dt, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * Per-token asymmetric activations for the two-subspace layer (CoQuant notes,
 * "CoQuant: Joint Weight-Activation Subspace Projection for Mixed-Precision
 * LLMs", Eq. 1 with a zero-point, and the experimental protocol: per-token
 * asymmetric activations, per-channel symmetric weights).  Each subspace of
 * each token row gets z = min and s = fl32(fl32(max - min) / (2^N - 1)), and
 * each value the code u = rne(fl32(fl32(x - z) / s)) in [0, 2^N - 1] (a
 * constant row: s = 0, u = 0); the subspace contributes
 * s_x s_w (U C_w^T) + z_x s_w colsum(C_w).
 *
 * tq_weight_colsum -- colsum[j] = sum over k of the codes of row j (m rows of
 * k codes, bits 4 or 8, as written by tq_pack_weight); int32, exact.  Offline.
 */
tq_status tq_weight_colsum(const void* w_codes, int64_t m, int64_t k, int bits, int32_t* colsum,
                           hipStream_t stream);

/*
 * tq_linear_mp_asym -- tq_linear_mp with asymmetric activations; colsum_l /
 * colsum_h: tq_weight_colsum of wl_codes / wh_codes (m int32 each, needed when
 * that subspace is not empty).  d <= 16384.  ws:
 * tq_linear_mp_asym_workspace_bytes(n, d, d_hi) bytes.  Two launches: the
 * quantiser (one wave per token row, the row read once) and the two-subspace
 * GEMM, whose epilogue adds each subspace's zero-point term.  Errors as
 * tq_linear_mp, plus TQ_ERR_SHAPE for d > 16384.
 */
size_t tq_linear_mp_asym_workspace_bytes(int64_t n, int64_t d, int64_t d_hi);
tq_status tq_linear_mp_asym(const void* Xrot, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t d_hi,
                            const void* wl_codes, const float* s_wl, const int32_t* colsum_l,
                            const void* wh_codes, const float* s_wh, const int32_t* colsum_h, void* Y,
                            tq_dtype y_dt, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Byte offsets inside the tq_linear_mp_asym workspace: off[0..3] as
 * tq_linear_mp_workspace_offsets, but the stored codes are u - 8 (4-bit
 * subspace, int8 in the tile GEMM's order) and u - 128 (8-bit subspace, int8,
 * natural order); off[4] z of the 4-bit subspace, off[5] z of the 8-bit
 * subspace (n fp32 each).  For tests.
 */
tq_status tq_linear_mp_asym_workspace_offsets(int64_t n, int64_t d, int64_t d_hi, size_t off[6]);

/*
 * tq_linear_asym -- tq_linear with per-token asymmetric 4-bit activations
 * (same z, s and codes as tq_linear_mp_asym's 4-bit subspace):
 *   Y = s_x s_w (.) (U C_w^T) + z_x (s_w (.) colsum(C_w)) + (X L1) L2,
 * colsum = tq_weight_colsum(w_codes, m, d, 4) (m int32).  d <= 16384.  Up to
 * 16 tokens one launch, as tq_linear's few-token GEMM (its first blocks
 * quantise with the zero-point and compute partials of T, under the same
 * grid-size rule); otherwise two launches: the quantiser with T = X L1, then
 * the GEMM (the tile GEMM, or for n <= 32 the weight-streaming small-n GEMM).
 * The GEMM's epilogue adds the zero-point term.  The one-launch form's waits
 * are bounded as tq_linear's (word 32 of the hand-off words at the start of
 * the workspace, NaN outputs).  ws:
 * tq_linear_asym_workspace_bytes(n, d, m, r) bytes, zero-filled once before
 * its first use (as tq_linear's).  Errors as tq_linear, plus TQ_ERR_SHAPE for
 * d > 16384.
 */
size_t tq_linear_asym_workspace_bytes(int64_t n, int64_t d, int64_t m, int64_t r);
tq_status tq_linear_asym(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r,
                         const void* w_codes, const float* s_w, const int32_t* colsum, const void* lowrank,
                         void* Y, tq_dtype y_dt, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Byte offsets inside the tq_linear_asym workspace: off[0] s_x (n fp32),
 * off[1] activation codes (u - 8: n x d int8 in the tile GEMM's order, or
 * for n <= 32 nibble-packed, n x d / 2 bytes), off[2] z_x (n fp32), off[3] T
 * (n x r_pad bf16).  For tests.
 */
tq_status tq_linear_asym_workspace_offsets(int64_t n, int64_t d, int64_t m, int64_t r, size_t off[4]);

/*
 * Fully quantised low-rank branch (TwinQuant notes, "TwinQuant: Learnable
 * Subspace Decomposition for W4A4 LLM Quantization", section 04.A error
 * expression Q(X)[Q(U)Q(V) + Q(R)] and section 04.C, Figure 4: the low-rank
 * product is taken on integer codes in two stages, the first stage's int32
 * result re-quantised per token on-chip, and both branches meet in one
 * epilogue):
 *
 *   acc  = C_x C_w^T,  acc1 = C_x C_u^T                       (exact, int32)
 *   t    = fl32(fl32(acc1) * s_u)   per token; C_t, s_t = 4-bit absmax codes of t
 *   Y    = s_x s_w (.) acc + (s_x s_t) s_v (.) (C_t C_v^T)
 *
 * U (d x r) and V (r x m) are quantised per column at 4 bits (symmetric, as
 * the weight R); the token scale s_x is common to a row of t and is kept
 * outside it.
 *
 * tq_lowrank_q_bytes -- size of the packed factors (0 for invalid shapes):
 * r_pad = r rounded up to 32, 64, 128 or 256; U's codes as r_pad rows of
 * d / 2 bytes (nibble-packed like tq_pack_weight, rows r .. r_pad - 1 zero),
 * its r_pad scales, V's codes as m rows of r_pad / 2 bytes (ranks past r
 * zero) and its m scales, each part 256-byte aligned.
 */
size_t tq_lowrank_q_bytes(int64_t d, int64_t m, int64_t r);

/*
 * tq_pack_lowrank_q -- quantises and packs U (d x r) and V (r x m), row-major
 * device arrays of dtype dt, into lowrank_q (tq_lowrank_q_bytes bytes, caller
 * owned, 16-byte aligned).  1 <= r <= 256, d % 32 == 0.  Offline.
 */
tq_status tq_pack_lowrank_q(const void* U, const void* V, tq_dtype dt, int64_t d, int64_t m, int64_t r,
                            void* lowrank_q, hipStream_t stream);

/*
 * tq_linear_qlr -- the layer above on X (n x d, x_dt) with R packed by
 * tq_pack_weight (4 bits) and the factors by tq_pack_lowrank_q; Y (n x m,
 * y_dt).  Launches on `stream`: the per-token quantiser together with the
 * first low-rank stage and its re-quantisation (one launch for d <= 4096 and
 * r <= 128, else two; only the r_pad code bytes and s_t of each token are
 * written), then the integer GEMM -- the tile GEMM, or for n <= 32 the
 * weight-streaming small-n GEMM -- whose epilogue adds the second stage on
 * the int8 MFMA.  ws: tq_linear_qlr_workspace_bytes(n, d, r) bytes of device
 * memory.  Errors as tq_linear (r < 1 is TQ_ERR_SHAPE).
 */
size_t tq_linear_qlr_workspace_bytes(int64_t n, int64_t d, int64_t r);
tq_status tq_linear_qlr(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r,
                        const void* w_codes, const float* s_w, const void* lowrank_q, void* Y,
                        tq_dtype y_dt, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Byte offsets inside the tq_linear_qlr workspace: off[0] s_x (n fp32),
 * off[1] activation codes (n x d int8, per 8 k the 4 even-k codes then the 4
 * odd-k codes; for n <= 32 nibble-packed, n x d / 2 bytes), off[2] s_t
 * (n fp32), off[3] first-stage codes (n x r_pad int8 in the int8 order over
 * the ranks).  For tests.
 */
tq_status tq_linear_qlr_workspace_offsets(int64_t n, int64_t d, int64_t r, size_t off[4]);

/*
 * tq_debug_accumulate -- exact integer product of two code matrices, exported.
 *   x_codes  n x k codes, w_codes m x k codes (both bits wide, K-contiguous).
 *   acc      out: n x m int32, acc[i][j] = sum_t x[i][t] * w[j][t], exactly.
 * The integer GEMM on caller codes (the tile GEMM's main loop for n > 32 on
 * nibble-packed or int8 codes, the small-n loop otherwise).  The layers'
 * own kernels export their sums through the *_debug entry points below.
 * k must be a multiple of 32 (bits = 4) or 16 (bits = 8).
 */
tq_status tq_debug_accumulate(const void* x_codes, const void* w_codes, int64_t n, int64_t k,
                              int64_t m, int bits, int32_t* acc, hipStream_t stream);

/*
 * tq_debug_accumulate_i8 -- the same exact product with the activation codes
 * as the rank-augmented layer's tile GEMM takes them (TwinQuant notes,
 * section 04.C and Figure 4: the 4-bit residual product with int32
 * accumulation): one int8 byte per 4-bit code, and within every 8
 * consecutive k the 4 codes of even k, then the 4 codes of odd k.
 *   x_codes  n x k int8 bytes in that order; w_codes m x k nibble-packed
 *            (as tq_pack_weight writes them); acc out: n x m int32.
 * Always the tile GEMM (any n), with the integer-export epilogue that
 * tq_debug_accumulate uses on nibble-packed activations, so the two time
 * the two activation formats through the same main loop and epilogue.
 * k a multiple of 32; device buffers, 16-byte aligned, caller-owned.
 * Kernel timing names it "gemm_acc_i8".
 */
tq_status tq_debug_accumulate_i8(const void* x_codes, const void* w_codes, int64_t n, int64_t k, int64_t m,
                                 int32_t* acc, hipStream_t stream);

/*
 * tq_debug_gemm_w4a4 -- the residual W4A4 product with its dequantising
 * epilogue and bf16 store, Y[i][j] = s_x[i] s_w[j] sum_t x[i][t] w[j][t]
 * (TwinQuant notes, section 04.C and Figure 4, without the low-rank term),
 * on either activation-code format: x_packed = 1, nibble-packed codes as
 * tq_quantize_act writes them (n x k/2 bytes); 0, one int8 byte per code in
 * the order of tq_debug_accumulate_i8 (n x k bytes), the format tq_linear's
 * tile GEMM reads.  w_codes / s_w as tq_pack_weight writes them; s_x n
 * floats; Y n x m bf16 (device, 16-byte aligned, caller-owned).  Always the
 * tile GEMM, so the two formats are timed through the same kernel and
 * epilogue; both give the same Y bit for bit (the scale absorbs the factor
 * of 16 between the two expanded forms exactly).  k a multiple of 32.
 * Kernel timing names it "gemm_w4a4_packed_x" or "gemm_w4a4_int8_x".
 */
tq_status tq_debug_gemm_w4a4(const void* x_codes, int x_packed, const float* s_x, const void* w_codes,
                             const float* s_w, int64_t n, int64_t k, int64_t m, void* Y, hipStream_t stream);

/*
 * Accumulator export (test hooks).  Each runs the layer exactly as the entry
 * point it is named after -- same checks, workspace, launches, kernel
 * templates and Y -- through the kernels' export instance, which also stores
 * the exact int32 sums of its integer products before they are dequantised:
 *   acc    n x m int32, acc[i][j] = sum_k C_x[i][k] C_w[j][k] (the residual,
 *          or the 4-bit subspace; asymmetric layers: the stored codes u - 8);
 *   acc_h  n x m int32, the 8-bit subspace's sums (u - 128 when asymmetric);
 *          may be NULL when d_hi == 0;
 *   acc2   n x m int32, the quantised branch's second stage sum_t C_t C_v.
 * Caller-owned device buffers, 16-byte aligned; TQ_ERR_NULL / TQ_ERR_ALIGN
 * otherwise.  Slower than the plain entry points (extra stores); meant for
 * checking the accumulators bit for bit, not for production use.
 */
tq_status tq_linear_debug(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r,
                          const void* w_codes, const float* s_w, const void* lowrank, void* Y, tq_dtype y_dt, void* ws,
                          size_t ws_bytes, int32_t* acc, hipStream_t stream);
tq_status tq_linear_mp_bits_debug(const void* Xrot, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t d_hi,
                                  int bits_lo, int bits_hi, const void* wl_codes, const float* s_wl,
                                  const void* wh_codes, const float* s_wh, void* Y, tq_dtype y_dt, void* ws,
                                  size_t ws_bytes, int32_t* acc_l, int32_t* acc_h, hipStream_t stream);
tq_status tq_linear_asym_debug(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r,
                               const void* w_codes, const float* s_w, const int32_t* colsum, const void* lowrank,
                               void* Y, tq_dtype y_dt, void* ws, size_t ws_bytes, int32_t* acc, hipStream_t stream);
tq_status tq_linear_mp_asym_debug(const void* Xrot, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t d_hi,
                                  const void* wl_codes, const float* s_wl, const int32_t* colsum_l,
                                  const void* wh_codes, const float* s_wh, const int32_t* colsum_h, void* Y,
                                  tq_dtype y_dt, void* ws, size_t ws_bytes, int32_t* acc_l, int32_t* acc_h,
                                  hipStream_t stream);
tq_status tq_linear_qlr_debug(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r,
                              const void* w_codes, const float* s_w, const void* lowrank_q, void* Y, tq_dtype y_dt,
                              void* ws, size_t ws_bytes, int32_t* acc, int32_t* acc2, hipStream_t stream);

/*
 * tq_debug_linear_handoff -- test hook of the one-launch few-token paths:
 * runs tq_linear (same checks and workspace) with its waits limited to
 * `spin` polls and, when `silent` is non-zero, with the producer blocks never
 * delivering (the decode kernel's tag their partials of T with the previous
 * call's tag, the few-token GEMM's never signal), so that every wait gives up
 * and the failure path runs (Y all NaN, the flag word set).  Every kernel
 * still exits.  TQ_ERR_SHAPE when the shape does not take a one-launch path,
 * or r == 0.
 */
tq_status tq_debug_linear_handoff(const void* X, tq_dtype x_dt, int64_t n, int64_t d, int64_t m, int64_t r,
                                  const void* w_codes, const float* s_w, const void* lowrank, void* Y, tq_dtype y_dt,
                                  void* ws, size_t ws_bytes, unsigned spin, int silent, hipStream_t stream);

/*
 * tq_debug_stream_read -- the streaming-read ceiling that bounds the
 * few-token (decode) kernel (TwinQuant notes, section 04.C: at decode sizes
 * the layer streams the INT4 weight codes once): reads `bytes` of device
 * memory at `buf` (16-byte aligned, bytes a multiple of 16) exactly once with
 * the decode kernel's 16-byte non-temporal loads, `blocks` blocks of 256
 * threads each reading a contiguous slab, and writes one XOR of what each
 * block read to out[0 .. blocks - 1] (device, caller-owned).  Kernel timing
 * names it "stream_read".  TQ_ERR_NULL / TQ_ERR_ALIGN / TQ_ERR_SHAPE (blocks
 * outside 1 .. 65536) before anything is enqueued.
 */
tq_status tq_debug_stream_read(const void* buf, size_t bytes, uint32_t* out, int blocks, hipStream_t stream);

/*
 * tq_debug_mfma_ceiling -- the int8 matrix-core ceiling that bounds the tile
 * GEMM (TwinQuant notes, section 04.C and Figure 4: the residual product on
 * the integer matrix units with int32 accumulation): `blocks` blocks of 512
 * threads, each wave chaining `iters` rounds of 8 independent
 * v_mfma_i32_32x32x32_i8 (2 x 32^3 operations each) on register operands,
 * with no memory traffic inside the loop; every thread then writes one int
 * to out[0 .. 512 blocks - 1] (device, caller-owned), so the work cannot be
 * dropped.  Kernel timing names it "mfma_ceiling".  TQ_ERR_NULL /
 * TQ_ERR_SHAPE (iters outside 1 .. 2^20, blocks outside 1 .. 65536) before
 * anything is enqueued.
 */
tq_status tq_debug_mfma_ceiling(int iters, int blocks, int32_t* out, hipStream_t stream);

/*
 * Kernel timing.  While enabled, every kernel the library launches is
 * bracketed by a pair of HIP events recorded on the launch stream (where a
 * step takes several dispatches under one name, the pair spans the first
 * one's start to the last one's end).  tq_profile_read synchronises on the
 * recorded events and returns, per kernel name, the number of launches (one
 * per step so bracketed) and their summed duration in milliseconds
 * (host arrays of `max` entries; returns the number of kernel names, or a
 * negative tq_status).  tq_profile_reset drops the record.  The record is
 * process-wide (one lock guards it); calls from several threads interleave
 * their entries.
 */
typedef struct {
  char name[48];
  int64_t launches;
  double total_ms;
} tq_kernel_stat;

tq_status tq_profile_enable(int on);
int tq_profile_read(tq_kernel_stat* out, int max);
tq_status tq_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
