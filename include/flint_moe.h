/*
 * flint_moe.h -- C ABI of the MI355X (gfx950) W4A16 MoE decode library.
 *
 * The library runs the MoE sublayer of a Flint-shaped model: a router GEMV,
 * sigmoid top-k over the routed experts, SwiGLU expert GEMVs that read only
 * the selected experts' 4-bit weights, an always-on shared expert and a
 * weighted combine, with BF16 activations and NVFP4 (or BF16) weights.
 *
 * Sources for what is computed (cited by page title and section):
 *  [D0]  "Day-0 Support for Flint on vLLM" (wpnews.pro), sections
 *        "Model architecture" and "Optimizations".
 *  [AR]  "vLLM 宣布首日支持 Recursive 的 Flint：单张 GB200 上达约 500 tokens/s，
 *        每层内核启动从 22 次降至 7 次" (arex-research.com), sections
 *        "Flint 是什么" and "七个内核的依赖链：低延迟路径、无损重排与参考舍入".
 *
 * Conventions shared by every entry point
 *  - Pointers marked (device) are device addresses on the current HIP
 *    device; (host) pointers are read during the call only.  The caller owns
 *    all memory; the library never allocates, frees, or keeps per-call state.
 *  - Every device pointer must be 16-byte aligned (FLINT_ERR_ALIGNMENT),
 *    except the top-k outputs of decode and prefill (4-byte aligned).
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    work: the return value covers argument checks and launch errors, and
 *    results are valid after the stream is synchronised.  No call blocks or
 *    synchronises, so every call can be captured in a HIP graph.
 *  - Arguments are validated before anything is enqueued; on error nothing
 *    is enqueued.  No call prints or throws.
 *  - BF16 is IEEE binary32's top 16 bits; rounding to BF16 is to nearest,
 *    ties to even.
 *
 * Packed NVFP4 layout (the gfx950 layout written by flint_moe_repack)
 *  A matrix of R rows by C columns (C = reduction dimension, multiple of 64)
 *  becomes two planes:
 *    codes : uint8 [R][C/2]   two E2M1 codes per byte, column 2i in the low
 *                             nibble, column 2i+1 in the high nibble
 *    scales: uint8 [R][C/16]  the UE4M3 scale of columns 16j..16j+15
 *  A GEMV wave reads 16 bytes of codes (32 columns) per lane and the two
 *  matching scale bytes, so every load is a coalesced 128-bit row segment.
 *  Several matrices are stored back to back (matrix m at m*R*C/2 bytes of the
 *  code plane, m*R*C/16 of the scale plane).  Expert e's gate/up pair is
 *  matrices 2e (gate) and 2e+1 (up) of one [E][2][I][H] array.
 */
#ifndef FLINT_MOE_H
#define FLINT_MOE_H

#include <stdint.h>

/* Exported symbols keep default visibility; the library builds with
 * -fvisibility=hidden so nothing else leaks out of it. */
#define FLINT_API __attribute__((visibility("default")))

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status -- */
#define FLINT_OK                0
#define FLINT_ERR_INVALID_ARG   1   /* NULL where required, negative or zero size */
#define FLINT_ERR_ALIGNMENT     2   /* a device pointer is not 16-byte aligned */
#define FLINT_ERR_UNSUPPORTED   3   /* shape, batch or flag outside the envelope:
                                       the caller falls back (e.g. to prefill) */
#define FLINT_ERR_WORKSPACE     4   /* workspace NULL or smaller than required */
#define FLINT_ERR_DEVICE        5   /* a HIP launch reported an error */

/* ----------------------------------------------------------------- flags -- */
#define FLINT_RENORM       0x1u  /* combine weight = s_k / sum of selected s
                                    (default: the raw sigmoid score s_k) */
#define FLINT_W_BF16       0x2u  /* weights are BF16 (W16A16), not NVFP4 */
#define FLINT_PRE_RMSNORM  0x4u  /* input is the residual x: the layer first
                                    computes xn = RMSNorm(x) * gamma */
#define FLINT_RESIDUAL     0x8u  /* out = BF16(x + BF16(layer(xn))) */
#define FLINT_SPLIT        0x10u /* decode: always run the three-kernel path
                                    (by default a batch-1 NVFP4 call with
                                    hidden 2048 or 4096 runs as one launch; see
                                    flint_moe_decode_path) */

/* decode paths reported by flint_moe_decode_path */
#define FLINT_PATH_SPLIT        0  /* three kernels: route, gate/up, down    */
#define FLINT_PATH_SINGLE_ONE   1  /* one launch, batch 1                    */
#define FLINT_PATH_SINGLE_BATCH 2  /* one launch, batch 2..8 (Flint shape)   */

/* source NVFP4 super-block byte orders accepted by the repack */
#define FLINT_SRC_INTERLEAVED   0  /* 4 x [scale byte, 8 code bytes]          */
#define FLINT_SRC_SCALES_FIRST  1  /* 4 scale bytes, then 32 code bytes       */

/* dense GEMV epilogues */
#define FLINT_EPI_NONE     0   /* y = BF16(g * W x)                              */
#define FLINT_EPI_SWIGLU   1   /* W = [gate; up]: y = BF16(BF16(SiLU(BF16(g0 Wg x)))
                                  * BF16(g1 Wu x))                               */
#define FLINT_EPI_RESIDUAL 2   /* y = BF16(aux + BF16(g * W x))                  */

#define FLINT_MAX_DECODE_BATCH 8

/* Workspace header (byte offsets into the caller's workspace; each field is
 * one uint32):
 *   FLINT_WS_ERROR_OFFSET       the hand-off error word: 0 normally; set to 1
 *                               by a single-launch or route kernel whose
 *                               bounded wait for another workgroup's word
 *                               gave up.  That can only happen when the grid
 *                               of a single-launch call is not resident all
 *                               at once (another kernel holding compute units
 *                               meanwhile).  The kernel still exits, but the
 *                               results of that call are undefined and so are
 *                               those of later calls on the workspace until
 *                               it is zero-filled again.  Read it with
 *                               flint_moe_workspace_error.
 *   FLINT_WS_WAIT_LIMIT_OFFSET  bound of each such wait, in reloads of the
 *                               awaited words; 0 (the zero-filled default)
 *                               means 2^20.  A caller may store a smaller
 *                               value to bound how long a call can wait. */
#define FLINT_WS_ERROR_OFFSET      512
#define FLINT_WS_WAIT_LIMIT_OFFSET 768
#define FLINT_WS_HEADER_BYTES      1024

#define FLINT_MAX_TOP_K        8
#define FLINT_MAX_EXPERTS      256

/* Shape of one MoE layer.
 *   hidden        H, multiple of 64, at most 4096
 *   n_experts     E, routed experts, 1..256
 *   inter         I, routed expert intermediate, multiple of 64
 *   shared_inter  SI, shared expert intermediate, multiple of 64; 0 = none
 *   top_k         K, 1..min(8, E)
 *   flags         FLINT_RENORM | FLINT_W_BF16 | FLINT_PRE_RMSNORM | FLINT_RESIDUAL |
 *                 FLINT_SPLIT
 *   rms_eps       RMSNorm epsilon (used with FLINT_PRE_RMSNORM)
 * Sizes: [D0] "Model architecture" (hidden 2048; 256 experts, sigmoid top-6,
 * one shared expert); the expert intermediate is not printed on the pages. */
typedef struct flint_moe_shape {
  int32_t hidden;
  int32_t n_experts;
  int32_t inter;
  int32_t shared_inter;
  int32_t top_k;
  uint32_t flags;
  float rms_eps;
} flint_moe_shape;

/* Weights of one MoE layer (all device pointers, read-only).
 *   router        BF16 [E][H]
 * NVFP4 (flags without FLINT_W_BF16; packed layout above):
 *   gu_codes      [E][2][I][H/2]     gu_scales  [E][2][I][H/16]
 *   d_codes       [E][H][I/2]        d_scales   [E][H][I/16]
 *   gscale        float [E][3]       FP32 tensor scale of (gate, up, down)
 *                                    per expert ([AR] "七个内核的依赖链",
 *                                    second paragraph)
 *   sh_gu_codes   [2][SI][H/2]       sh_gu_scales [2][SI][H/16]
 *   sh_d_codes    [H][SI/2]          sh_d_scales  [H][SI/16]
 *   sh_gscale     float [3]
 * BF16 (FLINT_W_BF16; the scale fields are ignored):
 *   gu_bf16 [E][2][I][H], d_bf16 [E][H][I], sh_gu_bf16 [2][SI][H], sh_d_bf16 [H][SI]
 * Shared-expert fields may be NULL when shared_inter is 0. */
typedef struct flint_moe_weights {
  const void* router;
  const void* gu_codes;
  const void* gu_scales;
  const void* d_codes;
  const void* d_scales;
  const float* gscale;
  const void* sh_gu_codes;
  const void* sh_gu_scales;
  const void* sh_d_codes;
  const void* sh_d_scales;
  const float* sh_gscale;
  const void* gu_bf16;
  const void* d_bf16;
  const void* sh_gu_bf16;
  const void* sh_d_bf16;
} flint_moe_weights;

/* ---------------------------------------------------------------- helpers -- */

/* Library version string (static storage). */
FLINT_API const char* flint_version(void);

/* Text of a status code (static storage; unknown codes give "unknown"). */
FLINT_API const char* flint_status_string(int32_t status);

/* Bytes of the packed planes of n_mats matrices of rows x cols (cols a
 * multiple of 64).  Writes *code_bytes = n_mats*rows*cols/2 and
 * *scale_bytes = n_mats*rows*cols/16.  Host pointers. */
FLINT_API int32_t flint_nvfp4_packed_bytes(int64_t n_mats, int64_t rows, int64_t cols,
                                 int64_t* code_bytes, int64_t* scale_bytes);

/* Workspace bytes that flint_moe_decode (max_tokens <= 8) and
 * flint_moe_prefill (up to max_tokens tokens) need for this shape; negative
 * = a FLINT_ERR_* code negated.  The decode part (header, launch counters,
 * hand-off words) comes first and the prefill part after it, so decode and
 * prefill calls may share one workspace.  The workspace must be zero-filled
 * once after allocation (it carries a launch counter from call to call);
 * calls that share one workspace must be ordered on one stream. */
FLINT_API int64_t flint_moe_workspace_bytes(const flint_moe_shape* shape, int32_t max_tokens);

/* Enqueues a copy of the workspace's hand-off error word (see
 * FLINT_WS_ERROR_OFFSET) into dst (device or pinned host memory, 4 bytes) on
 * `stream`, after the calls already enqueued there. */
FLINT_API int32_t flint_moe_workspace_error(const void* ws, int64_t ws_bytes, uint32_t* dst, void* stream);

/* ------------------------------------------------------------------ repack -- */

/* Lossless load-time repack of source NVFP4 super-blocks into the packed
 * planes ([D0] "Model architecture", paragraph after the bullets: the
 * checkpoint's NVFP4 blocks come in another byte order and are repacked
 * without loss at load; [AR] "七个内核的依赖链", second paragraph: a 64-value
 * super-block is four groups of one UE4M3 scale and 16 E2M1 codes).
 *   src          (device) uint8 [n_mats][rows][cols/64][36] in `src_layout`
 *   dst_codes    (device) packed code plane; matrix m is written at matrix
 *                index m*dst_mat_stride of the plane (stride 2 writes every
 *                other matrix, e.g. gate into the even and up into the odd
 *                slots of a [E][2] array)
 *   dst_scales   (device) packed scale plane, same matrix indexing
 * A pure byte permutation: every byte is copied, NaN and sign-bit scale
 * bytes included.  Source and destination must not overlap. */
FLINT_API int32_t flint_moe_repack(const void* src, int64_t n_mats, int32_t rows, int32_t cols,
                         int32_t src_layout, void* dst_codes, void* dst_scales,
                         int64_t dst_mat_stride, void* stream);

/* Exact inverse of flint_moe_repack (for round-trip checks and export):
 * reads matrices m*src_mat_stride of the packed planes and writes
 * dst uint8 [n_mats][rows][cols/64][36] in `src_layout`. */
FLINT_API int32_t flint_moe_unpack(const void* codes, const void* scales, int64_t n_mats,
                         int32_t rows, int32_t cols, int32_t src_layout,
                         int64_t src_mat_stride, void* dst, void* stream);

/* Dequantise packed matrices to float32, the same E2M1 x UE4M3 decode the
 * GEMV kernels use: out[m][r][c] = E2M1 * UE4M3 * tensor_scale[m]
 * (tensor_scale (device) float [n_mats] or NULL for 1.0).  A verification
 * aid: it exposes the kernels' decode so it can be compared bit for bit. */
FLINT_API int32_t flint_nvfp4_dequant(const void* codes, const void* scales, int64_t n_mats,
                            int32_t rows, int32_t cols, const float* tensor_scale,
                            float* out, void* stream);

/* ------------------------------------------------------------------ decode -- */

/* The small-batch decode MoE layer ([D0] "Optimizations": router and
 * expert GEMVs that read only the selected experts' weights, with routing
 * and the expert combine fused into the neighbouring GEMV kernels, for up
 * to 8 concurrent requests).  Per token t of the batch:
 *   xn    = x, or BF16(BF16(x / sqrt(mean(x^2) + eps)) * gamma) with
 *           FLINT_PRE_RMSNORM
 *   s_e   = sigmoid(router[e] . xn)              logits accumulated in fp32
 *   idx   = top_k experts by descending s, ties to the lower index
 *   w_k   = s_idx[k]  (or s_idx[k] / sum_k s_idx[k] with FLINT_RENORM)
 *   E(z)  = W_d (BF16(BF16(SiLU(BF16(W_g z))) * BF16(W_u z)))
 *   out   = BF16(sum_k w_k E_idx[k](xn) + E_shared(xn))
 *   with FLINT_RESIDUAL: out = BF16(x + out)
 * Each selected expert's weights are read once per call, for all tokens
 * routed to it.
 *   x         (device) BF16 [batch][H]
 *   batch     1..8, else FLINT_ERR_UNSUPPORTED (use flint_moe_prefill)
 *   out       (device) BF16 [batch][H]; may equal x only with FLINT_RESIDUAL
 *   topk_idx  (device) int32 [batch][K] or NULL; ordered by descending score
 *   topk_w    (device) float [batch][K] or NULL; the combine weights
 *   gamma     (device) BF16 [H], required with FLINT_PRE_RMSNORM
 *   ws        (device) workspace of at least flint_moe_workspace_bytes(shape, batch)
 * With NVFP4 weights and hidden 2048 or 4096 (I, SI <= 2048), and with BF16
 * weights at the Flint shape (hidden 2048, 256 experts, I = SI = 512), a
 * batch-1 call is one launch of a persistent grid (at most one workgroup per compute
 * unit) whose phases hand data over through epoch-tagged words in the
 * workspace.  That grid relies on all of its workgroups running at once:
 * the call checks at launch that the device can hold the whole grid (and
 * runs the three kernels instead when it cannot), and the caller must not
 * run other kernels on the device concurrently (on other streams or in
 * other processes) while it runs; a caller that does should set
 * FLINT_SPLIT.  At the Flint shape (hidden 2048, 256 experts, I = SI = 512,
 * NVFP4) a call of batch 2..8 is one launch of the same kind, on a device
 * with at least 256 compute units.  Every other call enqueues three kernels: route (RMSNorm,
 * router GEMV, top-k, expert set), gate/up (+SiLU*up), down (weighted
 * combine, shared expert, residual).  flint_moe_decode_path tells which.
 * All paths give the same result up to fp32 summation order. */
FLINT_API int32_t flint_moe_decode(const flint_moe_shape* shape, const flint_moe_weights* weights,
                         const void* x, int32_t batch, void* out, int32_t* topk_idx,
                         float* topk_w, const void* gamma, void* ws, int64_t ws_bytes,
                         void* stream);

/* One stage of the three-kernel path, same arguments as flint_moe_decode:
 * stage 0 = route (router GEMV and top-k), 1 = gate/up, 2 = down + combine.
 * Enqueuing stages 0, 1, 2 in order on one stream with the same workspace is
 * exactly flint_moe_decode with FLINT_SPLIT; a stage reads what the previous
 * one left in the workspace.  For per-kernel timing and for callers that
 * interleave other work between stages. */
FLINT_API int32_t flint_moe_decode_stage(int32_t stage, const flint_moe_shape* shape,
                               const flint_moe_weights* weights, const void* x, int32_t batch,
                               void* out, int32_t* topk_idx, float* topk_w, const void* gamma,
                               void* ws, int64_t ws_bytes, void* stream);

/* A stack of MoE sublayers for one token in one launch (the decode step's
 * MoE part: [AR] "Flint 是什么" -- 47 MoE layers; [D0] "Model architecture"
 * and "Optimizations" -- pre-norm residual sublayers, the low-latency path
 * with each kernel's weight loads overlapping the previous step).  With x_0
 * = x, for l = 0 .. n_layers-1:
 *   x_{l+1} = BF16(x_l + flint_moe_decode(layer l, x_l)) with PRE_RMSNORM
 *             and RESIDUAL (gamma_l; rms_eps from the shape)
 * and out = x_{n_layers}.  Each layer's result equals one flint_moe_decode
 * call bit for bit; only the launches between layers are gone (the
 * residual is handed from layer to layer in the workspace).
 *   shape      as flint_moe_decode; flags: FLINT_RENORM only (PRE_RMSNORM
 *              and RESIDUAL are implied); the batch-1 single-launch envelope
 *              (NVFP4, hidden 2048 or 4096, I and SI <= 2048), else
 *              FLINT_ERR_UNSUPPORTED
 *   layers     (device) flint_moe_weights [n_layers], NVFP4 fields used
 *   n_layers   1 .. FLINT_MAX_STACK_LAYERS
 *   gammas     (device) BF16 [n_layers][H]
 *   x, out     (device) BF16 [H]; out may equal x
 *   topk_idx   (device) int32 [n_layers][K], topk_w float [n_layers][K]:
 *              every layer's selection (required)
 *   layer_out  (device) BF16 [n_layers][H] or NULL: x_{l+1} of every layer
 *   ws         as flint_moe_decode (the same workspace size)
 * One launch; a batch-1 flint_moe_decode may share the workspace. */
#define FLINT_MAX_STACK_LAYERS 4096
FLINT_API int32_t flint_moe_decode_stack(const flint_moe_shape* shape, const flint_moe_weights* layers,
                                         int32_t n_layers, const void* gammas, const void* x, void* out,
                                         int32_t* topk_idx, float* topk_w, void* layer_out, void* ws,
                                         int64_t ws_bytes, void* stream);

/* Which kernels flint_moe_decode runs for this shape (flags included) and
 * batch: FLINT_PATH_SPLIT, FLINT_PATH_SINGLE_ONE or FLINT_PATH_SINGLE_BATCH.
 * Reads only the shape; enqueues nothing.  Returns -status for an invalid
 * shape (-FLINT_ERR_INVALID_ARG, -FLINT_ERR_UNSUPPORTED) or a batch outside
 * 1..8 (-FLINT_ERR_UNSUPPORTED). */
FLINT_API int32_t flint_moe_decode_path(const flint_moe_shape* shape, int32_t batch);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation:
 * flint_moe_decode with the library's own device scratch (a static array of
 * FLINT_NOALLOC_SCRATCH_BYTES per device, zero at load and held until the
 * process ends) in place of the caller's workspace.  Same kernels, same
 * results, same arguments otherwise; nothing is allocated or freed.
 *   Returns FLINT_ERR_WORKSPACE when the shape's decode workspace
 *   (flint_moe_workspace_bytes(shape, 1) minus its prefill part) exceeds the
 *   scratch -- every shape with hidden <= 4096 and I, SI <= 2048 fits --
 *   and FLINT_ERR_DEVICE if the scratch's device address cannot be found.
 *   Every call on a device shares that device's scratch, which keeps the
 *   last call's state: calls that may overlap on one device (other streams,
 *   other host threads without ordering) race and must not be made; calls
 *   ordered on one stream are fine.  The scratch's error word is not
 *   readable through this entry point; a wait that gives up leaves it set
 *   for the rest of the process. */
#define FLINT_NOALLOC_SCRATCH_BYTES (4 << 20)
FLINT_API int32_t flint_moe_decode_noalloc(const flint_moe_shape* shape, const flint_moe_weights* weights,
                                           const void* x, int32_t batch, void* out, int32_t* topk_idx,
                                           float* topk_w, const void* gamma, void* stream);

/* ----------------------------------------------------------------- prefill -- */

/* The same layer for any number of tokens ([D0] "Optimizations": the
 * small-batch MoE change also gives the largest gain on an 8,192-token
 * prefill, on the same packed weights as the large-batch kernel).  The
 * result per token equals flint_moe_decode's definition.  Tokens are
 * grouped by expert (histogram, scan, stable permutation by expert then
 * token), run through grouped GEMMs on MFMA, and un-permuted into the
 * weighted combine with the shared expert.
 *   n_tokens  >= 1; ws at least flint_moe_workspace_bytes(shape, n_tokens)
 * Other arguments as flint_moe_decode. */
FLINT_API int32_t flint_moe_prefill(const flint_moe_shape* shape, const flint_moe_weights* weights,
                          const void* x, int32_t n_tokens, void* out, int32_t* topk_idx,
                          float* topk_w, const void* gamma, void* ws, int64_t ws_bytes,
                          void* stream);

/* Prefill layout of packed NVFP4 weights, for the grouped GEMMs of the
 * 8,192-token prefill ([D0] "Optimizations": the prefill runs on the same
 * NVFP4 weights).  Row by row, a GEMM step of 128 columns reads 64 bytes of
 * each of 32 rows, so every load instruction touches 32 rows; in this
 * layout it reads 1 KB in one piece.  The same bytes, regrouped (lossless):
 * the matrices of a set become blocks of 32 (virtual) rows x 128 columns;
 * block (vb, kb) of set m starts at code byte 2048 (m nb + vb (cols/128) +
 * kb) and scale byte 256 (m nb + vb (cols/128) + kb), nb the blocks per
 * set.  Inside a block, bytes 32 h + 16 p .. + 15 of row n's 64 code bytes
 * sit at 1024 p + 16 (2 n + h), and bytes 4 h .. 4 h + 3 of its 8 scale
 * bytes at 4 (2 n + h) (h, p in {0, 1}, n < 32).
 *   codes, scales  (device) packed planes of n_mats matrices [rows][cols],
 *                  flint_moe_repack's layout, 16-byte aligned
 *   interleave     0: a set is one matrix, virtual row r = row r;
 *                  1: a set is a (gate, up) pair of consecutive matrices
 *                  and virtual row 2 i + u is row i of matrix u, the order
 *                  in which the fused gate/up GEMM pairs them (n_mats even)
 *   rows, cols     rows (1 + interleave) a multiple of 32, cols of 128
 *   out_codes, out_scales  (device) as many bytes as the inputs, 16-byte
 *                  aligned; they must not overlap the inputs
 * Returns FLINT_ERR_INVALID_ARG for null pointers, bad sizes or overlap,
 * FLINT_ERR_ALIGNMENT for misaligned planes. */
FLINT_API int32_t flint_moe_prefill_layout(const void* codes, const void* scales, int64_t n_mats,
                                           int32_t rows, int32_t cols, int32_t interleave,
                                           void* out_codes, void* out_scales, void* stream);

/* One layer's weights in the prefill layout (device pointers): routed
 * gate/up (interleave 1 over the [E][2] matrices), routed down (interleave
 * 0 over [E]), and the shared expert's the same way (NULL when
 * shared_inter is 0). */
typedef struct flint_moe_prefill_planes {
  const void* gu_codes;
  const void* gu_scales;
  const void* d_codes;
  const void* d_scales;
  const void* sh_gu_codes;
  const void* sh_gu_scales;
  const void* sh_d_codes;
  const void* sh_d_scales;
} flint_moe_prefill_planes;

/* flint_moe_prefill with the NVFP4 weights also in the prefill layout.  The
 * grouped GEMMs read `planes` at hidden 2048 with routed and shared
 * intermediate 512 (the shapes they are specialised for) and ignore it
 * otherwise; the result is bit-identical to flint_moe_prefill's either way.
 * planes == NULL is flint_moe_prefill; a non-null planes with a missing
 * plane gives FLINT_ERR_INVALID_ARG, one not 16-byte aligned
 * FLINT_ERR_ALIGNMENT.  Other arguments as flint_moe_prefill. */
FLINT_API int32_t flint_moe_prefill_tiled(const flint_moe_shape* shape, const flint_moe_weights* weights,
                                          const flint_moe_prefill_planes* planes, const void* x,
                                          int32_t n_tokens, void* out, int32_t* topk_idx, float* topk_w,
                                          const void* gamma, void* ws, int64_t ws_bytes, void* stream);

/* --------------------------------------------------------------- dense GEMV -- */

/* Small-batch dense GEMV on the same packed NVFP4 weights ([D0]
 * "Optimizations", third bullet), used for the dense MLP layers.
 *   codes, scales  (device) packed matrix [rows][cols] (FLINT_EPI_SWIGLU:
 *                  two matrices [2][rows][cols], gate then up)
 *   gscale         (device) float [1] (FLINT_EPI_SWIGLU: [2]) tensor scales
 *   w_bf16         (device) BF16 weights of the same shape, used instead of
 *                  codes/scales/gscale when flags has FLINT_W_BF16
 *   flags          FLINT_W_BF16 and/or FLINT_PRE_RMSNORM (then x is the
 *                  residual and the GEMV input is RMSNorm(x) * gamma)
 *   x              (device) BF16 [batch][cols];  batch 1..8
 *   y              (device) BF16 [batch][rows]
 *   epilogue       FLINT_EPI_NONE | FLINT_EPI_SWIGLU | FLINT_EPI_RESIDUAL
 *   aux            (device) BF16 [batch][rows], the residual for
 *                  FLINT_EPI_RESIDUAL (y may equal aux), else NULL
 *   gamma, rms_eps RMSNorm weight (device, BF16 [cols]) and epsilon with
 *                  FLINT_PRE_RMSNORM */
FLINT_API int32_t flint_dense_gemv(const void* codes, const void* scales, const float* gscale,
                         const void* w_bf16, int32_t rows, int32_t cols, uint32_t flags,
                         const void* x, int32_t batch, void* y, int32_t epilogue,
                         const void* aux, const void* gamma, float rms_eps, void* stream);

/* ------------------------------------------------------------------------
 * Attention-side step of the same layers: per-head Q/K RMSNorm, rotary
 * position embedding and the BF16 KV-cache write, fused into one kernel
 * ([D0] "Optimizations", first bullet: one kernel instead of three;
 * "Model architecture": GQA, 32 query and 4 KV heads of dimension 128,
 * per-head Q/K RMSNorm, RoPE on the 35 sliding-window layers and none on
 * the 14 full-context layers, BF16 KV cache).
 * ---------------------------------------------------------------------- */
#define FLINT_ATTN_ROPE  0x1u   /* rotate Q and K (sliding-window layers); without it
                                   the heads are only normalised (NoPE layers) */

typedef struct flint_attn_shape {
  int32_t n_q_heads;    /* query heads (32), a multiple of n_kv_heads      */
  int32_t n_kv_heads;   /* KV heads (4)                                    */
  int32_t head_dim;     /* 128, the only value supported                   */
  uint32_t flags;       /* FLINT_ATTN_ROPE or 0                            */
  float rms_eps;        /* RMSNorm epsilon of the per-head norms (1e-6)    */
} flint_attn_shape;

/* For each of n_tokens tokens, from its projection row
 *   qkv        (device) BF16 [n_tokens][(n_q + 2 n_kv) * 128]: the q heads,
 *              then the k heads, then the v heads
 * computes, per q and k head h, y = BF16(BF16(x_h / sqrt(mean(x_h^2) + eps))
 * * gamma) and, with FLINT_ATTN_ROPE, the rotate-half rotation of the pairs
 * (y_i, y_{i+64}), i < 64, by the angles of table row positions[t]:
 * (y_i c_i - y_{i+64} s_i, y_{i+64} c_i + y_i s_i), rounded to BF16 once.
 *   positions  (device) int32 [n_tokens], with FLINT_ATTN_ROPE (else unused,
 *              may be NULL); a position outside 0..n_positions-1 is an error
 *   cos_sin    (device) float32 [n_positions][128]: row p holds cos of the
 *              64 angles of position p, then their sines (the caller's
 *              rotary table); with FLINT_ATTN_ROPE, else may be NULL
 *   slots      (device) int32 [n_tokens]: the KV-cache row of each token; a
 *              negative slot writes no K or V (a padding token); a slot >=
 *              n_slots is an error
 *   k_cache, v_cache (device) BF16 [n_slots][n_kv][128]: row slots[t] gets
 *              the token's normalised (and rotated) k heads and its v heads
 *              unchanged; other rows are not touched
 *   gamma_q, gamma_k (device) BF16 [128], shared by the heads of each role
 *   q_out      (device) BF16 [n_tokens][n_q][128], must not overlap qkv
 *   error      (device) int32 [1] or NULL: set to 1 when a token's position or
 *              slot is out of range; nothing of that token is written
 * Pointers 16-byte aligned (positions, slots, error: 4-byte).  Returns
 * FLINT_ERR_INVALID_ARG / _UNSUPPORTED / _ALIGNMENT before enqueuing
 * anything, FLINT_ERR_DEVICE on a launch error.  Asynchronous on `stream`. */
FLINT_API int32_t flint_qk_norm_rope_kv(const flint_attn_shape* shape, const void* qkv, int32_t n_tokens,
                                        const int32_t* positions, const float* cos_sin, int32_t n_positions,
                                        const int32_t* slots, void* k_cache, void* v_cache, int32_t n_slots,
                                        const void* gamma_q, const void* gamma_k, void* q_out, int32_t* error,
                                        void* stream);

/* Decode attention with learned sinks ("Day-0 Support for Flint on vLLM",
 * "Model architecture", first two bullets: 35 layers attend to a 513-token
 * sliding window (the current token and the 512 before it), 14 to the whole
 * context; GQA with 32 query and 4 KV heads of dimension 128; learned
 * attention sinks.  "Optimizations", fifth bullet: a decode attention kernel
 * with sinks and sliding windows).  One query token per sequence b:
 *   out[b][h] = sum_p w_p V[row(p)][g],  w_p = exp(s_p) / (sum_p' exp(s_p') +
 *   exp(sinks[h])),  s_p = scale * (q[b][h] . K[row(p)][g]),  g = h / (n_q / n_kv)
 * over the positions p = max(0, L - window) .. L - 1 (0 .. L - 1 when window
 * is 0), L = seq_len[b], row(p) = seq_base[b] + (p mod ring).
 *   shape      n_q_heads, n_kv_heads (n_q / n_kv in 1..16), head_dim 128,
 *              flags 0; rms_eps unused
 *   window     0 (whole context) or the window length (513 on Flint)
 *   ring       cache rows per sequence: at least the attended span (a ring
 *              of `window` rows for a window layer, the context for a
 *              full layer); else the sequence is an error
 *   scale      the score scale (1/sqrt(128)), finite and > 0
 *   q          (device) BF16 [batch][n_q][128], after the Q norm and RoPE
 *   k_cache, v_cache (device) BF16 [n_rows][n_kv][128] (the layout
 *              flint_qk_norm_rope_kv writes); n_rows * n_kv * 128 < 2^32
 *   seq_base, seq_len (device) int32 [batch]: first row and context length
 *              (newest token included, its K/V already in the cache) of each
 *              sequence; a length outside 1..max_len, base < 0, or base + ring
 *              > n_rows is an error
 *   max_len    (host) the largest seq_len of the call: sizes the split of the
 *              context over workgroups
 *   sinks      (device) float32 [n_q], one logit per query head (-inf: none)
 *   out        (device) BF16 [batch][n_q][128]
 *   workspace  (device) flint_decode_attention_workspace_bytes(...) bytes (0
 *              when the split has one chunk: NULL allowed); caller-owned,
 *              needs no initialisation
 *   error      (device) int32 [1] or NULL: set to 1 for an invalid sequence,
 *              whose output is all zeros
 * Scores and the softmax are float32 (base-2 exponentials of pre-scaled
 * scores); the weights enter the V product as BF16; output rounded to BF16
 * once.  Returns FLINT_OK or a FLINT_ERR_* code (host-side checks only). */
FLINT_API int64_t flint_decode_attention_workspace_bytes(const flint_attn_shape* shape, int32_t window,
                                                         int32_t batch, int32_t max_len);
FLINT_API int32_t flint_decode_attention(const flint_attn_shape* shape, int32_t window, int32_t ring,
                                         float scale, const void* q, int32_t batch, const void* k_cache,
                                         const void* v_cache, int32_t n_rows, const int32_t* seq_base,
                                         const int32_t* seq_len, int32_t max_len, const float* sinks, void* out,
                                         void* workspace, int64_t workspace_bytes, int32_t* error, void* stream);

/* Measurement utility (not part of the layer computation): a plain read of
 * `bytes` of device memory at `src`, for the achievable HBM read rate of a
 * transfer of that size, against which the decode kernels' rates are
 * compared.  Each of blocks x threads threads reads `loads` 16-byte words
 * per pass of a grid-stride loop, all issued before any is used.
 *   src      (device) 16-byte aligned; bytes > 0, a multiple of 16
 *   threads  64..1024, a multiple of 64;  loads 4, 8, 16 or 27;  blocks >= 1
 *   sink     (device) uint32 [1]: written only if the fold of the data equals
 *            0x9e3779b9 (so the reads are not dropped)
 * Returns FLINT_ERR_INVALID_ARG / _ALIGNMENT / _UNSUPPORTED for bad
 * arguments (nothing enqueued), FLINT_ERR_DEVICE on a launch error. */
FLINT_API int32_t flint_stream_read(const void* src, int64_t bytes, int32_t threads, int32_t loads,
                                    int32_t blocks, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FLINT_MOE_H */
