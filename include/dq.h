/*
 * dq.h -- C ABI of the delta-W4A4 linear layer for AMD Instinct MI355X (gfx950).
 *
 * The layer is the one of the DeltaQuant notes ("DeltaQuant: 4-bit Video
 * Diffusion Models with Spatiotemporal Delta Smoothing", papernotes.org,
 * CVPR 2026), section 方法详解:
 *
 *   Y = X L1 L2  +  bcast_k( Q8(core_k) Q4(R) )  +  Q4(delta) Q4(R)
 *
 * with X in R^{N x Ci} the flattened (T, H, W) token grid, W = L1 L2 + R an
 * SVD split of the weight (关键设计 4, the three-term equation), core_k the
 * mean token of the t x h x w cube k (关键设计 2 and 3, the core/delta
 * equation), delta = X - core, Q8 = MX-FP8 (E4M3) and Q4 = MX-FP4 (E2M1),
 * both with one power-of-two E8M0 scale per 32 consecutive channels (关键设计
 * 4, the quantizer definition, q_max = 6 for FP4 and 448 for FP8).  The core
 * term is computed once per cube and broadcast to the cube's tokens (the
 * "dynamic token bias" of 关键设计 4).
 *
 * Conventions
 *  - Pointers named *_host are host memory; *_dev are device memory of the
 *    handle's device.  Caller-owned buffers are never freed or kept by the
 *    library beyond the call (device buffers may be read asynchronously by
 *    work enqueued on the given stream, so keep them alive until it completes).
 *  - Matrices are dense and row-major.  The weight is given as W^T, i.e. the
 *    nn.Linear layout [Co][Ci]; token n of X is (t, h, w) with
 *    n = (t*H + h)*W + w.
 *  - FP4 codes are packed two per byte, the even channel in the low nibble.
 *    E8M0 scale codes are e + 127 for a scale of 2^e.
 *  - Every function validates its arguments first and returns a status; on
 *    failure nothing has been enqueued and outputs are untouched.  Device
 *    faults of enqueued work surface at the caller's next synchronisation.
 *    dq_last_error() gives a message for the last failure on this thread.
 *  - Streams are hipStream_t values passed as void*; NULL is the null stream.
 *  - All allocation happens in dq_prepare_weights* and dq_qact_create; the
 *    hot calls (dq_quantize_act, dq_linear_forward, dq_linear) allocate
 *    nothing.
 *  - A dq_weights is read-only after preparation and may be shared by
 *    streams; a dq_qact must not be used by two streams at once.
 */
#ifndef DQ_H
#define DQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DQ_OK = 0,
    DQ_ERR_INVALID_ARG = 1,   /* null pointer, unknown dtype, bad rank, ... */
    DQ_ERR_SHAPE = 2,         /* Ci % 32 != 0, cube larger than the grid, size overflow */
    DQ_ERR_UNSUPPORTED = 3,   /* device is not gfx950 */
    DQ_ERR_OUT_OF_MEMORY = 4, /* device or host allocation failed */
    DQ_ERR_DEVICE = 5         /* a HIP runtime call failed */
} dq_status;

typedef enum { DQ_F32 = 0, DQ_BF16 = 1 } dq_dtype;

/* Token grid T x H x W and cube t x h x w (1 <= t <= T, 1 <= h <= H,
 * 1 <= w <= W).  Cubes tile the grid from the origin; cubes at the high end
 * of an axis that does not divide evenly are clipped, and their core is the
 * mean of the tokens they hold.  t = T, h = H, w = W is one global cube. */
typedef struct {
    int32_t T, H, W;
    int32_t t, h, w;
} dq_geom;

typedef struct dq_weights dq_weights;   /* prepared weight: Q4(R), L1, L2 on one device */
typedef struct dq_qact dq_qact;         /* per-geometry activation workspace on one device */

/* Message for the last failed call on this thread ("" if none). */
const char* dq_last_error(void);
const char* dq_status_str(dq_status s);

/* Low-rank factors of W by a truncated SVD on the host (关键设计 4: the split
 * W = L1 L2 + R borrowed from SVDQuant).  Randomized subspace iteration with
 * a Gaussian test matrix drawn from `seed`; L1 = U_r sqrt(S_r) and
 * L2 = sqrt(S_r) V_r^T, each rounded to bf16 (nearest, ties to even).
 *   w_host   [Co][Ci] W^T, dtype dt
 *   l1_host  out, [Ci][rank] bf16 bits;  l2_host  out, [rank][Co] bf16 bits
 * rank 0 is allowed (no low-rank branch; nothing written).  Host only: no
 * device is touched.  Errors: DQ_ERR_INVALID_ARG for null pointers or
 * rank > min(Ci, Co); DQ_ERR_SHAPE for Ci or Co < 1. */
dq_status dq_lowrank_factors(const void* w_host, dq_dtype dt, int64_t Ci, int64_t Co, int32_t rank,
                             uint64_t seed, uint16_t* l1_host, uint16_t* l2_host);

/* Prepare a weight from given bf16 factors.  On `device` it forms
 * R^T = fl32(W^T - (L1 L2)^T), the product of every entry summed in fp64 in
 * rank order, then MX-FP4-encodes each output channel of R along Ci.
 *   w_host   [Co][Ci] W^T (dtype dt);  l1_host [Ci][rank], l2_host [rank][Co]
 *            bf16 bits (may be NULL when rank == 0)
 * Requires Ci % 32 == 0, 32 <= Ci <= 2^24, 1 <= Co <= 2^24 and
 * 0 <= rank <= min(Ci, Co, 128) (the activation pass keeps U's rank tiles
 * on chip; DQ_ERR_INVALID_ARG above 128).  l1_host and l2_host must hold
 * Ci*rank and rank*Co values: the library cannot check their sizes.
 * The handle owns every device buffer it allocates; free it with
 * dq_weights_destroy.  Synchronous (returns when the weight is ready). */
dq_status dq_prepare_weights_lowrank(const void* w_host, dq_dtype dt, int64_t Ci, int64_t Co, int32_t rank,
                                     const uint16_t* l1_host, const uint16_t* l2_host, int32_t device,
                                     dq_weights** out);

/* dq_lowrank_factors followed by dq_prepare_weights_lowrank (so rank <= 128). */
dq_status dq_prepare_weights(const void* w_host, dq_dtype dt, int64_t Ci, int64_t Co, int32_t rank,
                             uint64_t seed, int32_t device, dq_weights** out);

void dq_weights_destroy(dq_weights* w);

/* Sizes of a prepared weight (any pointer may be NULL). */
dq_status dq_weights_info(const dq_weights* w, int64_t* Ci, int64_t* Co, int32_t* rank, int32_t* device);

/* Copy the prepared weight to the host in canonical layout (any pointer may
 * be NULL): L1 [Ci][rank] and L2 [rank][Co] bf16 bits, R^T [Co][Ci] fp32,
 * Q4(R) codes [Co][Ci/2] and scale codes [Co][Ci/32].  Synchronous. */
dq_status dq_weights_export(const dq_weights* w, uint16_t* l1_host, uint16_t* l2_host, float* r_host,
                            uint8_t* rcodes_host, uint8_t* rscales_host);

/* Workspace for activations of one geometry: delta codes and scales, core
 * codes and scales, U = bf16(bf16(X) L1), and (for cube shapes that need it)
 * the per-cube core term.  Owns its device buffers (sized from the geometry,
 * Ci, Co and the rank of `w`); free with dq_qact_destroy.  When t does not
 * divide T, the cubes of the last, clipped frame group (T % t frames) are laid
 * out as a grid of their own: the same cubes, tokens, sums and codes, without
 * rows for the missing frames, so the forward does no work for them.  Errors:
 * DQ_ERR_SHAPE for an invalid geometry or size overflow. */
dq_status dq_qact_create(const dq_weights* w, dq_geom geom, dq_qact** out);

/* dq_qact_create with a choice of how cores are quantized.
 *   core_group = 32: one E8M0 scale per 32-channel MX block (as
 *     dq_qact_create); 64: the pages' per-group core with group size 64
 *     (DeltaQuant notes, 损失函数/训练策略): one exponent from the maximum
 *     over 64 consecutive channels, stored as the scale code of both of its
 *     32-channel blocks.
 *   core_bits = 8: MX-FP8 (E4M3) cores, the pages' choice; 4: MX-FP4 (E2M1)
 *     cores, the 4-bit point of the pages' core-precision ablation (消融实验);
 *     the core GEMM then runs FP4 x FP4; 16: bf16 cores (round to nearest
 *     even, no scales; core_group is then unused), the ablation's 16-bit
 *     point: the core term is a bf16 x bf16 MFMA GEMM (fp32 accumulation) of
 *     the bf16 cores against Q4(R) decoded to bf16 (exact), which the
 *     workspace holds (Co x Ci x 2 bytes more).
 * Deltas keep MX-FP4 with groups of 32.  dq_qact_export reports core codes one
 * per byte for 8 and 4 bits; for 16 bits it writes the bf16 bits (2 bytes per
 * value, so ccodes needs K x Ci x 2 bytes) and leaves cscales untouched.
 * Errors: DQ_ERR_INVALID_ARG for another core_group or core_bits, DQ_ERR_SHAPE
 * when core_group does not divide Ci, and those of dq_qact_create. */
dq_status dq_qact_create_ex(const dq_weights* w, dq_geom geom, int32_t core_group, int32_t core_bits,
                            dq_qact** out);
void dq_qact_destroy(dq_qact* q);

/* Sizes of a workspace (any pointer may be NULL): tokens N, cubes K, and the
 * device bytes it holds. */
dq_status dq_qact_info(const dq_qact* q, int64_t* N, int64_t* K, int64_t* device_bytes);

/* The activation pass (关键设计 2-4, and the implementation paragraph of
 * 损失函数/训练策略, which fuses core generation into activation
 * quantization): for every cube, core = fl32(fp32 sum of its tokens in
 * lexicographic (dt, dh, dw) order, in blocks of 64, / count); for every
 * token, delta = fl32(x - core); cores -> MX-FP8, deltas -> MX-FP4 (smallest
 * power-of-two scale with max|v| <= q_max 2^e, round to nearest even); and
 * U = bf16(bf16(X) L1) with fp32 accumulation.
 *   x_dev  [N][Ci] of dtype dt, N = T*H*W of the workspace's geometry (the
 *          geometry is the one given to dq_qact_create, held by `q`),
 *          contiguous and 16-byte aligned (DQ_ERR_INVALID_ARG otherwise).
 *          Its size cannot be checked here: a shorter buffer is read out of
 *          bounds.
 * Asynchronous on `stream`. */
dq_status dq_quantize_act(const dq_weights* w, const void* x_dev, dq_dtype dt, dq_qact* q, void* stream);

/* The GEMMs (关键设计 4, the three-term equation): for every token n of cube
 * k, y[n] = U[n] L2 + Q8(core_k) Q4(R) + Q4(delta_n) Q4(R), fp32 accumulation,
 * written to y_dev [N][Co] fp32 (every element written; contiguous, 4-byte
 * aligned, else DQ_ERR_INVALID_ARG; a shorter buffer is written out of
 * bounds, which the library cannot detect).  Uses the state left in `q` by
 * the last dq_quantize_act.  Asynchronous on `stream`.  It runs
 * dq_core_term then dq_delta_term, or, for small layers of 4-token cubes, the
 * one-kernel form dq_linear_forward_fused (dq_forward_form tells which); the
 * per-cube term in `q` is then not written. */
dq_status dq_linear_forward(const dq_weights* w, dq_qact* q, float* y_dev, void* stream);

/* The two halves of dq_linear_forward, in its order, for callers that time
 * or schedule them separately.
 * dq_core_term: the per-cube core term Q8(core_k) Q4(R) (the pages'
 *   "dynamic token bias", one row per cube, 关键设计 4), fp32, into the
 *   workspace `q`.
 * dq_delta_term: Q4(delta_n) Q4(R) + U[n] L2, plus the core term of token
 *   n's cube as left in `q` by the last dq_core_term, written to y_dev
 *   [N][Co] fp32 in token order (every element written).
 * Same arguments, errors and asynchrony as dq_linear_forward; calling
 * dq_delta_term without dq_core_term after a dq_quantize_act reads a stale
 * core term (not detected).
 * Cubes of one token (t = h = w = 1): every delta is exactly zero, so
 * dq_delta_term alone computes y = Q8(x_n) Q4(R) + U[n] L2 in one FP8 GEMM
 * and dq_core_term does nothing. */
dq_status dq_core_term(const dq_weights* w, dq_qact* q, void* stream);
dq_status dq_delta_term(const dq_weights* w, dq_qact* q, float* y_dev, void* stream);

/* dq_linear_forward in one kernel, the form of the pages' implementation
 * (DeltaQuant notes, 损失函数/训练策略: the core partial sums accumulated in
 * the W4A4 GEMM): each 256-slot x 256-channel tile accumulates the delta term
 * of its slots and the core term of its 64 cubes in the same K loop, sharing
 * the Q4(R) operand, and adds them in its epilogue, so the per-cube term is
 * never written to memory.  Same y as dq_linear_forward (bit-identical where
 * the core GEMM walks every tile forwards along K; otherwise the core sums
 * differ only in the order of their fp32 additions).  Only for cubes of 4
 * tokens (t h w = 4) with FP8 cores in one frame segment, rank 32, Co a
 * multiple of 256, Ci >= 512 and y_dev 16-byte aligned; other workspaces
 * return DQ_ERR_INVALID_ARG.  Arguments, ownership and asynchrony as
 * dq_linear_forward.  dq_linear_forward (and so dq_linear and
 * dq_linear_noalloc) runs this form itself where it applies and the layer has
 * at most 16 rounds of 256 x 256 output tiles per compute unit: on MI355X it
 * measured faster on such small layers and slower on larger ones (the fused
 * K loop also carries the cores' operand steps and is bound by operand
 * delivery). */
dq_status dq_linear_forward_fused(const dq_weights* w, dq_qact* q, float* y_dev, void* stream);

/* Which form dq_linear_forward takes for this weight and workspace, for a
 * 16-byte aligned y_dev: *one_kernel = 1 for the one-kernel form above, 0 for
 * dq_core_term followed by dq_delta_term.  Host only (queries the device's
 * compute-unit count); DQ_ERR_INVALID_ARG for a NULL or mismatched handle or
 * a NULL one_kernel. */
dq_status dq_forward_form(const dq_weights* w, const dq_qact* q, int* one_kernel);

/* dq_quantize_act followed by dq_linear_forward on the same stream. */
dq_status dq_linear(const dq_weights* w, const void* x_dev, dq_dtype dt, dq_qact* q, float* y_dev, void* stream);

/* Copy the state of the last dq_quantize_act to the host in canonical token
 * order (any pointer may be NULL): delta codes [N][Ci/2], delta scale codes
 * [N][Ci/32], core codes [K][Ci] (FP8 E4M3), core scale codes [K][Ci/32],
 * U [N][rank] bf16 bits.  Synchronises `stream` first.  With one-token
 * cubes (t = h = w = 1) every delta is exactly zero: its codes and scale
 * codes are reported as 0 (the activation pass does not store them). */
dq_status dq_qact_export(const dq_qact* q, uint8_t* dcodes_host, uint8_t* dscales_host, uint8_t* ccodes_host,
                         uint8_t* cscales_host, uint16_t* u_host, void* stream);

/* ---- 6-bit layers on text tokens ------------------------------------------
 * The pages quantize every linear layer to 4 bits except the cross-attention
 * K and V projections, which act only on the text tokens and are kept at 6
 * bits (DeltaQuant notes, 损失函数/训练策略).  Text tokens have no (T, H, W)
 * grid, so these layers have no cubes: for token n,
 *     y_n = U_n L2 + Q6(x_n) Q6(R),   W = L1 L2 + R,  U = bf16(bf16(X) L1)
 * with Q6 an MX 6-bit float (one E8M0 scale per 32 channels, the quantizer of
 * 关键设计 4 with q_max the format's largest value, round to nearest even)
 * and fp32 accumulation (E2M3 x E2M3 exactly per 64-term block; E3M2 x E3M2
 * keeps fewer bits, like FP8 x FP4).  6-bit codes are exported packed in
 * order, code i of a row at bits [6 i, 6 i + 6) of its byte string (24 bytes
 * per 32 channels). */
typedef enum { DQ_FP6_E2M3 = 2, DQ_FP6_E3M2 = 3 } dq_fp6_format;
typedef struct dq_act6 dq_act6;         /* workspace of a 6-bit layer for N text tokens */

/* dq_prepare_weights_lowrank with R quantized to MX-FP6 (`fp6_format`), for
 * the 6-bit entry points below only (the 4-bit ones reject it).
 * dq_weights_export then writes rcodes as [Co][3 Ci/4] packed 6-bit codes.
 * Same requirements and errors, and DQ_ERR_INVALID_ARG for another format. */
dq_status dq_prepare_weights_w6(const void* w_host, dq_dtype dt, int64_t Ci, int64_t Co, int32_t rank,
                                const uint16_t* l1_host, const uint16_t* l2_host, int32_t fp6_format, int32_t device,
                                dq_weights** out);

/* Workspace for N text tokens (1 <= N <= 2^31 - 256) of a 6-bit weight: the
 * codes and scales of Q6(X), U.  Owns its device buffers. */
dq_status dq_act6_create(const dq_weights* w, int64_t N, dq_act6** out);
void dq_act6_destroy(dq_act6* a);

/* Q6(X) per token and U = bf16(bf16(X) L1) (fp32 accumulation).
 *   x_dev [N][Ci] of dtype dt, contiguous, 16-byte aligned.
 * Asynchronous on `stream`. */
dq_status dq_quantize_act6(const dq_weights* w, const void* x_dev, dq_dtype dt, dq_act6* a, void* stream);
/* y_dev [N][Co] fp32 (every element written, 4-byte aligned) = U L2 +
 * Q6(X) Q6(R) from the state of the last dq_quantize_act6.  Asynchronous. */
dq_status dq_linear6_forward(const dq_weights* w, dq_act6* a, float* y_dev, void* stream);
/* dq_quantize_act6 followed by dq_linear6_forward. */
dq_status dq_linear6(const dq_weights* w, const void* x_dev, dq_dtype dt, dq_act6* a, float* y_dev, void* stream);
/* Host copies (any pointer may be NULL): codes [N][3 Ci/4], scale codes
 * [N][Ci/32], U [N][rank] bf16 bits.  Synchronises `stream` first. */
dq_status dq_act6_export(const dq_act6* a, uint8_t* codes_host, uint8_t* scales_host, uint16_t* u_host, void* stream);

/* ---- rotated-basis W4A4 layers (OrbitQuant notes: 方法, 离线的权重量化, 在线的激活量化)
 * Rows (tokens, and output channels of the weight) are rotated by a random
 * permuted block Hadamard transform, x' = blockdiag(H_256 / 16) x[perm],
 * divided by their RMS s = sqrt(sum x'^2 / Ci) (fp32; squares summed per
 * 256-channel block in channel order, then over the blocks), and each
 * coordinate is coded as its nearest level of the Lloyd-Max quantizer of
 * N(0, 1) with 2^bits levels, each level rounded to bf16 (exact ties to the
 * even index).  Weights are coded offline with the same permutation, so the
 * rotation cancels: y[n][j] = (sum_c lvl(x'_nc) lvl(w'_jc)) s_x[n] s_w[j],
 * the sum by bf16 MFMAs over the decoded levels with fp32 accumulation. */
typedef struct dq_orbit dq_orbit;           /* rotated, coded weight on one device */
typedef struct dq_orbit_act dq_orbit_act;   /* workspace for N tokens */

/* w_host [Co][Ci] (W^T, dtype dt); perm_host [Ci] a permutation of
 * 0 .. Ci - 1 (the caller draws it; DQ_ERR_INVALID_ARG otherwise);
 * wbits, abits in {2, 3, 4} (codebooks of 4, 8 or 16 levels).  Requires
 * Ci a multiple of 256 with Ci <= 15360 (one row in LDS), 1 <= Co <= 2^24.
 * Synchronous; the handle owns its device buffers. */
dq_status dq_orbit_prepare(const void* w_host, dq_dtype dt, int64_t Ci, int64_t Co, const int32_t* perm_host,
                           int32_t wbits, int32_t abits, int32_t device, dq_orbit** out);
void dq_orbit_destroy(dq_orbit* o);
/* Host copies (any pointer may be NULL): the bf16 levels of the weight and
 * activation codebooks (2^wbits and 2^abits entries, ascending), the weight's
 * level indices [Co][Ci/2] (two per byte, even channel in the low nibble) and
 * row scales [Co]. */
dq_status dq_orbit_export(const dq_orbit* o, uint16_t* wlev_host, uint16_t* alev_host, uint8_t* wcodes_host,
                          float* wscale_host);
/* Workspace for N tokens (1 <= N <= 2^31 - 256). */
dq_status dq_orbit_act_create(const dq_orbit* o, int64_t N, dq_orbit_act** out);
void dq_orbit_act_destroy(dq_orbit_act* a);
/* Rotate, normalize and code x_dev [N][Ci] (dtype dt, 16-byte aligned).
 * Asynchronous on `stream`. */
dq_status dq_orbit_quantize_act(const dq_orbit* o, const void* x_dev, dq_dtype dt, dq_orbit_act* a, void* stream);
/* y_dev [N][Co] fp32 (every element written) from the last
 * dq_orbit_quantize_act.  Asynchronous on `stream`. */
dq_status dq_orbit_forward(const dq_orbit* o, dq_orbit_act* a, float* y_dev, void* stream);
dq_status dq_orbit_linear(const dq_orbit* o, const void* x_dev, dq_dtype dt, dq_orbit_act* a, float* y_dev, void* stream);
/* Host copies: level indices [N][Ci/2] and row scales [N].  Synchronises
 * `stream` first. */
dq_status dq_orbit_act_export(const dq_orbit_act* a, uint8_t* codes_host, float* scale_host, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): dq_linear
 * for the geometry `geom` with MX-FP8 cores in groups of 32, without a
 * dq_qact.  The activation state (codes, scales, U, per-cube core term, slot
 * table, and the fp32 partial sums of launches split over more workgroups)
 * lives in a fixed per-device array of 128 MiB that the library holds
 * on every GPU it runs on until the process ends; the call allocates nothing
 * and calls no allocating routine.  Same arguments and layouts as
 * dq_quantize_act and dq_linear_forward (x_dev [N][Ci] 16-byte aligned,
 * y_dev [N][Co] fp32 4-byte aligned, every element written), with the same
 * results as dq_linear bit for bit.  Errors: those of dq_qact_create and
 * dq_linear, and DQ_ERR_SHAPE (with the bytes needed) when the layer does
 * not fit the array.  Every call on a GPU shares that GPU's array: calls that
 * overlap on one GPU (two streams, or two threads) race and give wrong
 * results; serialize them.  Asynchronous on `stream`. */
dq_status dq_linear_noalloc(const dq_weights* w, const void* x_dev, dq_dtype dt, dq_geom geom, float* y_dev,
                            void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DQ_H */
