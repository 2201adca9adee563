/*
 * macaq.h -- C ABI of the MACaQ online W4A4 linear layer for AMD Instinct
 * MI355X (gfx950).
 *
 * The method ("MACaQ: Fast, Model Agnostic Calibrated Quantization for
 * Low-Precision Weights and Activations", paper card, Abstract; restated in
 * "MACaQ - Huawei open-sources a 4-bit quantizer for GGUF, vLLM and
 * Diffusers", How it works): every linear layer is handled on its own. At
 * inference a per-channel scale D and a block-Hadamard transform H are applied
 * to the layer's activations, which are then quantized to MXFP4; the inverse
 * transforms are absorbed offline into the same layer's MXFP4 weights:
 *
 *     W' = MXFP4_RTN(W D^-1 H^T),   y = W' . MXFP4(H D x)  (~= W x).
 *
 * Conventions used by every call (readings where the pages are silent):
 *   - D = diag(1/s) with s_k = sqrt(max |x_k|) over calibration rows;
 *     H = S_b / sqrt(b), S_b the Sylvester (natural-order) Hadamard matrix,
 *     on contiguous aligned b-blocks of K, b in {32, 64, 128}; b = 0 means no
 *     Hadamard. The 1/sqrt(b) is folded into the per-channel multipliers:
 *     activations use a_k = RN32(c_b / s_k), weights r_k = RN32(c_b * s_k),
 *     c_b = RN32(1/sqrt(b)) (1 when b = 0).
 *   - The transform runs in fp32: t_k = RN32(v_k * m_k), then butterflies of
 *     span 1, 2, 4, ..., b/2 in that order, (u, v) -> (u + v, u - v).
 *   - MXFP4 (OCP MX v1.0): 32 consecutive elements along K share one E8M0
 *     scale 2^(floor(log2 amax) - 2), clamped to >= 2^-127; elements are E2M1
 *     codes (sign bit 3; magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6) rounded to
 *     nearest, ties to the even code, saturating at 6.
 *   - Packed operands come in one of two layouts. Codes hold element 2i in
 *     the low nibble and 2i+1 in the high nibble of a byte; scales are E8M0
 *     bytes (bias 127), one per 32 elements along K.
 *       MACAQ_ROW_MAJOR: codes uint8 [rows, K/2], scales uint8 [rows, K/32].
 *       MACAQ_GEMM_LAYOUT (what the GEMM reads): rows padded to RP =
 *         ceil(rows/32)*32 and K to KP = ceil(K/256)*256, the padding all
 *         zero bytes, cut into blocks of 32 rows x 256 elements ordered (row
 *         group, k block); with KB = KP/256 and, for row r and element k,
 *         blk = (r/32)*KB + k/256, chunk c = (k%256)/32, h = c/2, j = c%2:
 *           code byte of (r, k): blk*4096 + h*1024 + (32j + r%32)*16 + (k%32)/2
 *           scale of (r, k):     blk*256 + (32j + r%32)*4 + h
 *         so each 1 KiB of codes is the operand of one 32x32x64 scaled-FP4
 *         MFMA (lane 32j + r) and one dword per lane holds its 4 scale bytes
 *         of the block. Sizes: macaq_packed_codes_bytes /
 *         macaq_packed_scales_bytes; each packed operand must stay under
 *         2 GiB.
 *   - Activations X are bf16 [M, ldx] row-major. Outputs Y are [M, ldy]
 *     row-major, fp32 or bf16 (round-to-nearest-even).
 *
 * Ownership and execution: every pointer marked "device" is device memory
 * owned by the caller; host pointers are marked "host". The library allocates
 * nothing, keeps no per-call state, never synchronizes, and enqueues its work
 * on `stream` (NULL = the default stream). Calls are reentrant. Scratch that
 * a call needs is the caller's `workspace`, whose size the matching
 * *_workspace_size call gives.
 *
 * Errors: arguments are checked on the host before anything is enqueued; on a
 * check failure nothing is written and the status says why. MACAQ_EHIP means
 * the HIP runtime refused a launch; macaq_last_error() has the text. Inputs
 * must be finite: NaN or Inf in X or W give unspecified codes.
 */
#ifndef MACAQ_H
#define MACAQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t. */
typedef struct ihipStream_t* macaq_stream_t;

/* Status, element type and layout are plain 32-bit integers with the named
   values below, so that any value a caller passes is defined behaviour: an
   unknown dtype or layout is rejected with MACAQ_EINVAL, an unknown status
   has the text "unknown status". */
typedef int32_t macaq_status;
enum {
  MACAQ_OK = 0,
  MACAQ_EINVAL = 1,       /* null pointer, bad size, block or leading dimension */
  MACAQ_EALIGN = 2,       /* pointer or leading dimension not aligned as documented */
  MACAQ_EWORKSPACE = 3,   /* workspace smaller than the *_workspace_size result */
  MACAQ_EUNSUPPORTED = 4, /* current device is not gfx950 */
  MACAQ_EHIP = 5          /* a HIP runtime call failed; see macaq_last_error() */
};

typedef int32_t macaq_dtype;
enum { MACAQ_BF16 = 0, MACAQ_F32 = 1 };

typedef int32_t macaq_layout;
enum { MACAQ_ROW_MAJOR = 0, MACAQ_GEMM_LAYOUT = 1 };

/* Bytes of the codes / scales of a rows x K operand in MACAQ_GEMM_LAYOUT
   (0 for an empty operand). */
size_t macaq_packed_codes_bytes(int64_t rows, int64_t K);
size_t macaq_packed_scales_bytes(int64_t rows, int64_t K);

/* Text for a status code (static storage). */
const char* macaq_status_string(macaq_status s);

/* Detail of the last failure on the calling thread (static, thread-local). */
const char* macaq_last_error(void);

/*
 * Test hook for the device check that every enqueuing call makes: with arch
 * non-NULL, the check takes that architecture name (e.g. "gfx942") instead
 * of querying the HIP runtime, so the MACAQ_EUNSUPPORTED path can be
 * exercised on any host; NULL restores the real query. Process-wide; not for
 * use while other threads call the library.
 */
void macaq_debug_override_arch(const char* arch);

/*
 * Stress hook for the persistent GEMM launches (macaq_linear, macaq_gemm,
 * the grouped layer and the MoE calls): with n > 0 each such launch uses at
 * most n workgroups, so every workgroup walks more tiles, in another order
 * and another interleaving with the rest; n <= 0 restores the planned grid.
 * Each output tile is still computed whole by one workgroup in a fixed
 * order, so results must stay bit-identical: a difference exposes a race
 * between consecutive tiles of one workgroup. Process-wide, read at each
 * launch; slower, not for production.
 */
void macaq_debug_limit_workgroups(int32_t n);

/*
 * Measurement probes, not part of the layer: the ceilings that the GEMM and
 * the bandwidth-bound kernels are compared with on the device at hand (the
 * nominal peaks are the chip's published figures).
 *
 * macaq_debug_mfma_probe: `workgroups` workgroups of 256 threads (96 KiB of
 * LDS each, so one per CU) each run `iters` rounds of 8 independent scaled
 * FP4 MFMAs (32x32x64, E2M1 x E2M1, every scale 2^0) per wave on register
 * operands, nothing else in the loop. Thread t reads its 6 operands of 16
 * bytes once, from bytes [96 t, 96 t + 96) of `operands` (device, at least
 * 24576 bytes, shared by every workgroup; random bytes make the matrix
 * cores' inputs change from one MFMA to the next). out: device fp32
 * [workgroups * 256], written (a sum of each thread's accumulators, so the
 * work is kept). Work: workgroups * 4 * iters * 8 * 131072 flops.
 *
 * macaq_debug_read_probe: reads `bytes` of device memory at `src` with
 * `workgroups` workgroups of 256 threads, each thread with 8 loads of 16
 * bytes in flight along a grid-stride walk. out: device uint32
 * [workgroups * 256], written (a fold of what each thread read).
 *
 * Both: MACAQ_EINVAL for NULL pointers, workgroups outside [1, 65536],
 * iters < 1 or bytes < 16; MACAQ_EALIGN unless operands and src are 16-byte
 * aligned and bytes is a multiple of 16; enqueued on `stream`, nothing
 * allocated.
 */
macaq_status macaq_debug_mfma_probe(const void* operands, int32_t workgroups, int32_t iters, float* out,
                                    macaq_stream_t stream);
macaq_status macaq_debug_read_probe(const void* src, int64_t bytes, int32_t workgroups, uint32_t* out,
                                    macaq_stream_t stream);

/*
 * Per-channel scale from calibration activations (the "calibrated
 * per-channel scale" of the paper card's title and Abstract):
 *   s[k] = RN32(sqrt(max_r |xcal[r, k]|)), or 1 when that maximum is 0.
 * xcal: device bf16 [R, ldx]; s: device fp32 [K] (written).
 * Requires R >= 1, K >= 1, ldx >= K.
 */
macaq_status macaq_calibrate(const void* xcal, int64_t R, int64_t K, int64_t ldx, float* s,
                             macaq_stream_t stream);

/*
 * Calibration variants (the paper card's title calls the method calibrated;
 * the form of the scale is a reading): s[k] = (max_r |xcal[r, k]|)^(q/4) for
 * q = quarters in {0, 1, 2, 4}: 0 gives s = 1 (no per-channel scale), 1 two
 * correctly rounded square roots in turn, 2 is macaq_calibrate, 4 the maximum
 * itself (the whole range moved into the weights); 1 for an all-zero column.
 */
macaq_status macaq_calibrate_pow(const void* xcal, int64_t R, int64_t K, int64_t ldx, int32_t quarters, float* s,
                                 macaq_stream_t stream);

/*
 * Folded multipliers for one layer. "MACaQ: Fast, Model Agnostic Calibrated
 * Quantization ..." (paper card, Abstract) scales the activations per channel
 * and absorbs the inverse into the same layer's weights; with D = diag(1/s)
 * and the orthonormal H = S_b / sqrt(b) (both readings), the activations take
 * a[k] = RN32(c_b / s[k]) and the weights r[k] = RN32(c_b * s[k]), c_b =
 * RN32(1/sqrt(b)) (1 when b = 0), so that (r .* w) . (a .* x) = w . x before
 * rounding.
 *
 * Host-only and pure: s, a, r are host fp32 [K]; a or r may be NULL to skip
 * it; IEEE single-precision divide and multiply, no device, no stream, no
 * state. b in {0, 32, 64, 128}. Every s[k] must be positive and finite
 * (MACAQ_EINVAL otherwise, with nothing written).
 */
macaq_status macaq_make_multipliers(const float* s, int64_t K, int32_t b, float* a, float* r);

/*
 * The same multipliers computed on the device, for a scale s that already
 * lives there (macaq_calibrate's output): s, a, r are device fp32 [K], the
 * work is enqueued on `stream`, and the results are bit-identical to
 * macaq_make_multipliers (correctly rounded divide and multiply). s[k] must
 * be positive and finite (not checked: it lives on the device).
 */
macaq_status macaq_make_multipliers_device(const float* s, int64_t K, int32_t b, float* a, float* r,
                                           macaq_stream_t stream);

/*
 * Offline half (paper card, Abstract: inverse transforms absorbed into the
 * weights; round-to-nearest MXFP4): W' = MXFP4(rows of S_b (r .* W[n, :])).
 * W: device [N, ldw] of w_dtype (bf16 or fp32), row n = output channel n.
 * r: device fp32 [K] (macaq_make_multipliers, copied to the device, or
 * macaq_make_multipliers_device), or NULL with b = 0 for plain MXFP4
 * weights. w_codes / w_scales: device, in `layout`:
 *   MACAQ_ROW_MAJOR:   [N, K/2] codes and [N, K/32] scales (N*K/2 and
 *                      N*K/32 bytes; an interchange form);
 *   MACAQ_GEMM_LAYOUT: macaq_packed_codes_bytes(N, K) /
 *                      macaq_packed_scales_bytes(N, K) bytes, padding zero:
 *                      what macaq_linear, macaq_gemm and the grouped and MoE
 *                      calls read.
 * Requires K % 32 == 0, K % b == 0, ldw >= K; W, w_codes and w_scales 16-byte
 * aligned and rows of W a multiple of 16 bytes.
 */
macaq_status macaq_prepare_weights(const void* W, macaq_dtype w_dtype, int64_t N, int64_t K, int64_t ldw,
                                   const float* r, int32_t b, macaq_layout layout, uint8_t* w_codes,
                                   uint8_t* w_scales, macaq_stream_t stream);

/*
 * Online activation transform on its own (paper card, Abstract: per-channel
 * scale and block-Hadamard applied online to the activations, then MXFP4):
 * a_codes/a_scales = MXFP4(rows of S_b (a .* X[m, :])).
 * X: device bf16 [M, ldx]; a: device fp32 [K] or NULL (no scale); b in
 * {0, 32, 64, 128}. a_codes / a_scales: device, in `layout` (row-major
 * [M, K/2] / [M, K/32], or the GEMM layout). Alignment as
 * macaq_prepare_weights. M = 0 does nothing (pointers are not checked).
 */
macaq_status macaq_quant_act(const void* X, int64_t M, int64_t K, int64_t ldx, const float* a, int32_t b,
                             macaq_layout layout, uint8_t* a_codes, uint8_t* a_scales, macaq_stream_t stream);

/* Bytes of workspace that macaq_linear needs for these sizes. */
size_t macaq_linear_workspace_size(int64_t M, int64_t K, int64_t N);

/*
 * The layer (paper card, Abstract: W4A4 with the activation transforms run at
 * inference): Y[m, n] = sum_k dq(Q(S_b (a .* X[m, :]))_k) dq(W'[n, k]),
 * accumulated in fp32 on the scaled-FP4 matrix cores.
 * X: device bf16 [M, ldx]; a, b as macaq_quant_act (a = NULL, b = 0 is plain
 * MXFP4); w_codes/w_scales: device, from macaq_prepare_weights with the
 * matching r and b; Y: device [M, ldy] of y_dtype; workspace: device, at least
 * macaq_linear_workspace_size(M, K, N) bytes, 256-byte aligned.
 * Requires ldy >= N and Y aligned to its element size. M = 0 does nothing.
 */
macaq_status macaq_linear(const void* X, int64_t M, int64_t K, int64_t ldx, const float* a, int32_t b,
                          const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, void* Y,
                          macaq_dtype y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes,
                          macaq_stream_t stream);

/*
 * macaq_linear for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the same computation and kernels, with the
 * quantized activations and split-K partial sums in a scratch array the
 * library owns, 128 MiB on each GPU it runs on, held until the process ends
 * (its address is looked up on the first call on a device). Arguments as
 * macaq_linear without the workspace. A call whose scratch need,
 * macaq_linear_workspace_size(M, K, N), exceeds 128 MiB returns
 * MACAQ_EWORKSPACE before anything is enqueued. Every call on one GPU uses
 * the same scratch: calls that may overlap on one GPU (different streams
 * without ordering between them) race and give wrong results; calls on one
 * stream are ordered and safe. Nothing in the scratch needs clearing
 * between calls.
 */
macaq_status macaq_linear_noalloc(const void* X, int64_t M, int64_t K, int64_t ldx, const float* a, int32_t b,
                                  const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, void* Y,
                                  macaq_dtype y_dtype, int64_t ldy, macaq_stream_t stream);

/*
 * The GEMM alone on operands already in MXFP4 (the contraction step of
 * macaq_linear; also the baseline for the cost of the activation transform):
 * Y[m, n] = sum_k dq(A[m, k]) dq(W'[n, k]).
 * a_codes/a_scales: device, MACAQ_GEMM_LAYOUT for M rows (macaq_quant_act
 * with that layout); w_codes/w_scales as macaq_linear; other arguments as
 * macaq_linear.
 */
size_t macaq_gemm_workspace_size(int64_t M, int64_t K, int64_t N);
macaq_status macaq_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int64_t M, int64_t K,
                        const uint8_t* w_codes, const uint8_t* w_scales, int64_t N, void* Y,
                        macaq_dtype y_dtype, int64_t ldy, void* workspace, size_t workspace_bytes,
                        macaq_stream_t stream);

/* Bytes of workspace that macaq_linear_grouped needs. */
size_t macaq_linear_grouped_workspace_size(int64_t T, int32_t E, int64_t K, int64_t N);

/*
 * The layer for E experts of a mixture-of-experts block. "MACaQ - Huawei
 * open-sources a 4-bit quantizer for GGUF, vLLM and Diffusers" (What it is)
 * lists MoE models among those one recipe covers, and its How it works
 * section handles every linear layer on its own; so each expert's linear
 * layer is a MACaQ layer with its own D and absorbed weights: rows
 * [offsets[e], offsets[e+1]) of X belong to expert e and go through a[e, :]
 * and W'_e.
 * X: device bf16 [T, K] (contiguous, expert-major); offsets: device int32
 * [E+1], non-decreasing, offsets[0] = 0, offsets[E] = T (not checked on the
 * host: it lives on the device); a: device fp32 [E, K] or NULL with b = 0;
 * w_codes / w_scales: E prepared weights one after another, expert e at
 * e * macaq_packed_codes_bytes(N, K) / e * macaq_packed_scales_bytes(N, K);
 * Y: device [T, N] of y_dtype (row t is written for every t < T).
 */
macaq_status macaq_linear_grouped(const void* X, const int32_t* offsets, int32_t E, int64_t T, int64_t K,
                                  const float* a, int32_t b, const uint8_t* w_codes, const uint8_t* w_scales,
                                  int64_t N, void* Y, macaq_dtype y_dtype, void* workspace,
                                  size_t workspace_bytes, macaq_stream_t stream);

/*
 * ---- MoE block around macaq_linear_grouped --------------------------------
 *
 * "MACaQ - Huawei open-sources a 4-bit quantizer ..." (What it is) lists MoE
 * models among those the method covers, and "Huawei's MACaQ-R beats
 * Unsloth's ..." ("Changed tensors") names each routed expert's gate, up and
 * down projections; every one of them is a MACaQ layer with its own D and
 * absorbed weights. The block computes, for T tokens with top-k experts
 * ids[t, j] and routing weights w[t, j]:
 *
 *     y[t] = sum_j w[t, j] * bf16( Down_e( Q_dn( SiLU(Gate_e x_t) * Up_e x_t ) ) ),  e = ids[t, j]
 *
 * where Gate_e / Up_e / Down_e are MACaQ layers (Q_dn = the down layer's
 * transform and MXFP4 with a_dn[e]). Readings where the pages are silent:
 *   - the expert FFN is the gated one, SiLU(g) = g / (1 + exp(-g)), h in fp32;
 *   - rows: the (t, j) entries sorted by expert, ties by i = t*k + j; an id
 *     outside [0, E) takes no row and adds nothing to y;
 *   - gate and up are one stacked weight [2F, H] per expert whose rows
 *     alternate blocks of 32: rows 64c .. 64c+31 are gate channels 32c ..
 *     32c+31, rows 64c+32 .. 64c+63 the matching up channels (prepare W_gate
 *     and W_up with the same r, then interleave, or interleave the bf16 rows
 *     and prepare once: row preparation is per row);
 *   - each expert output row is rounded to bf16, and the combine sums over
 *     j = 0 .. k-1 in fp32.
 * Limits: 1 <= E <= 4096, 1 <= k, H and F multiples of 32 (and of b), T*k
 * rows fit every packed operand under 2 GiB.
 */

/* Bytes of workspace that each MoE call below needs (the same figure serves
   macaq_moe_gate_up, macaq_moe_down_combine and macaq_moe_block). */
size_t macaq_moe_workspace_size(int64_t T, int32_t k, int32_t E, int64_t H, int64_t F);

/* Bytes of workspace macaq_moe_route needs (0 for arguments it rejects). */
size_t macaq_moe_route_workspace_size(int64_t T, int32_t k, int32_t E);

/*
 * Routing: the stable sort of the T*k entries of ids by expert.
 * ids: device int32 [T, k], 16-byte aligned (may be NULL when T == 0); offsets: device int32 [E+1]
 * (rows of expert e are [offsets[e], offsets[e+1])); row_token: device int32
 * [T*k], the token of each row (rows past offsets[E] get token 0); pos:
 * device int32 [T*k], the row of entry i = t*k + j, or -1 for an id outside
 * [0, E). workspace: macaq_moe_route_workspace_size bytes, 256-byte aligned
 * (per-chunk expert counts; contents need not be cleared).
 */
macaq_status macaq_moe_route(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t* offsets,
                             int32_t* row_token, int32_t* pos, void* workspace, size_t workspace_bytes,
                             macaq_stream_t stream);

/*
 * Gate/up of every routed row and the down projection's quantized input:
 * row r gathers token row_token[r] of X, goes through expert e's a_gu[e] and
 * stacked weights, and h = SiLU(gate) * up goes through a_dn[e] and the
 * block-Hadamard of size b into MXFP4.
 * X: device bf16 [T, ldx]; row_token, offsets: from macaq_moe_route (R = T*k
 * rows); a_gu: device fp32 [E, H] or NULL (with b = 0); wgu_codes/scales: E
 * prepared stacked weights [2F, H] one after another (MACAQ_GEMM_LAYOUT,
 * expert e at e * macaq_packed_codes_bytes(2F, H)); a_dn: device fp32 [E, F]
 * or NULL (with b = 0); dn_codes/dn_scales: device outputs, MACAQ_GEMM_LAYOUT
 * of R rows x F (macaq_packed_*_bytes(R, F)); rows past offsets[E] are left
 * alone. workspace: macaq_moe_workspace_size bytes, 256-byte aligned.
 */
macaq_status macaq_moe_gate_up(const void* X, int64_t T, int64_t H, int64_t ldx, int32_t k, const int32_t* row_token,
                               const int32_t* offsets, int32_t E, const float* a_gu, int32_t b,
                               const uint8_t* wgu_codes, const uint8_t* wgu_scales, int64_t F, const float* a_dn,
                               uint8_t* dn_codes, uint8_t* dn_scales, void* workspace, size_t workspace_bytes,
                               macaq_stream_t stream);

/*
 * Down projection of every routed row (bf16 rows in the workspace) and the
 * weighted combine: y[t] = sum_j w[t, j] * row(pos[t*k + j]).
 * dn_codes/dn_scales, offsets, pos: as above (R = T*k rows); wdn_codes/scales:
 * E prepared down weights [H, F] one after another; w: device fp32 [T, k];
 * Y: device [T, ldy] of y_dtype.
 */
macaq_status macaq_moe_down_combine(const uint8_t* dn_codes, const uint8_t* dn_scales, const int32_t* offsets,
                                    const int32_t* pos, const float* w, int64_t T, int32_t k, int32_t E,
                                    const uint8_t* wdn_codes, const uint8_t* wdn_scales, int64_t H, int64_t F,
                                    void* Y, macaq_dtype y_dtype, int64_t ldy, void* workspace,
                                    size_t workspace_bytes, macaq_stream_t stream);

/*
 * The whole block: macaq_moe_route, macaq_moe_gate_up and
 * macaq_moe_down_combine in one call, their intermediates in the workspace.
 * ids: device int32 [T, k], 16-byte aligned; w: device fp32 [T, k]; other
 * arguments as in those calls.
 */
macaq_status macaq_moe_block(const void* X, int64_t T, int64_t H, int64_t ldx, const int32_t* ids, const float* w,
                             int32_t k, int32_t E, const float* a_gu, const uint8_t* wgu_codes,
                             const uint8_t* wgu_scales, const float* a_dn, const uint8_t* wdn_codes,
                             const uint8_t* wdn_scales, int64_t F, int32_t b, void* Y, macaq_dtype y_dtype,
                             int64_t ldy, void* workspace, size_t workspace_bytes, macaq_stream_t stream);

/*
 * ---- Flip-Refinement of prepared weights (offline) -------------------------
 *
 * "MACaQ ..." (paper card, Abstract) improves on round-to-nearest weights
 * with Flip-Refinement, a Hessian-aware coordinate descent that greedily moves
 * single FP4 codes to adjacent representable values; "Huawei's MACaQ-R beats
 * Unsloth's ..." (What we found when we compared the files) sees only codes
 * change, the block scales kept. Readings where the pages are silent:
 *   - row n of the layer minimises e^T H e, e = w~ - q: w~ = S_b (r .* W[n, :])
 *     in fp32 (what macaq_prepare_weights quantizes), q its dequantized codes,
 *     H = X~^T X~ with x~ = S_b (a .* x) of calibration rows (w~.x~ = w.x, so
 *     e.x~ is the row's output error on a calibration row);
 *   - a move takes one element's signed E2M1 index m (-7 .. 7) to m - 1 or
 *     m + 1 at its group's scale, changing the objective by
 *     d*d*H[k][k] - 2*d*g[k] with g = H e; each step takes the most negative
 *     change (ties: lowest k, then the downward move) until none is negative
 *     or max_flips moves are made;
 *   - everything in fp64 with sums in index order, one fused multiply-add
 *     per term, so the result is reproducible bit for bit; moved elements
 *     get the canonical code of their index, the others keep their bits.
 */

/* Bytes of workspace for macaq_hessian: R x K fp32. */
size_t macaq_hessian_workspace_size(int64_t R, int64_t K);

/*
 * H = X~^T X~ (fp64 [K, K], row-major) of R bf16 calibration rows X [R, ldx]
 * through the activation multiplier a (device fp32 [K], or NULL with b = 0)
 * and the block-Hadamard of size b. H: device, K*K doubles, 16-byte aligned.
 */
macaq_status macaq_hessian(const void* Xcal, int64_t R, int64_t K, int64_t ldx, const float* a, int32_t b, double* H,
                           void* workspace, size_t workspace_bytes, macaq_stream_t stream);

/* Bytes of workspace for macaq_flip_refine: 2 x N x K fp64 + K fp64. */
size_t macaq_flip_refine_workspace_size(int64_t N, int64_t K);

/*
 * Flip-Refinement of prepared weights in place: W [N, ldw] (bf16 or fp32, the
 * rows given to macaq_prepare_weights with the same r and b), H from
 * macaq_hessian with the matching a, w_codes / w_scales from
 * macaq_prepare_weights (MACAQ_GEMM_LAYOUT; codes rewritten, scales read
 * only). flips: device int32 [N] receiving each row's number of moves, or
 * NULL. max_flips >= 0 caps the moves per row (0 leaves the codes as they
 * are). Limits: K <= 32768, K a multiple of 32 and of b.
 */
macaq_status macaq_flip_refine(const void* W, macaq_dtype w_dtype, int64_t N, int64_t K, int64_t ldw, const float* r,
                               int32_t b, const double* H, int32_t max_flips, uint8_t* w_codes, const uint8_t* w_scales,
                               int32_t* flips, void* workspace, size_t workspace_bytes, macaq_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MACAQ_H */
