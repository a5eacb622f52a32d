/*
 * gift.h -- C ABI of the GIFT FP8 gradient round trip on MI355X (gfx950).
 *
 * GIFT (GIFT review: pith.science review of arXiv 2607.07494, "GIFT:
 * Geometry-Informed Low-precision Gradient Communication for LLM
 * Pretraining") sends each selected layer's weight gradient G through FP8 in
 * whitened coordinates: G is right-multiplied by the inverse square root of a
 * rank-32 approximation of the input-side K-FAC factor A = X^T X / N before
 * quantization, and by its square root after dequantization ("What carries
 * the argument", "Core claim"; rank 32 and the 50-step refresh in the
 * free-parameter ledger).  Layers not selected use plain ("Euclidean") FP8
 * with one scale per tensor ("The pith").
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Tensor pointers inside gift_factor / gift_layer, and X, sketch, A_out,
 *   dev_flags, dev_out and ws, are DEVICE pointers on the current HIP device,
 *   allocated and owned by the caller.  The library allocates and frees
 *   nothing and keeps no state between calls.
 * - The gift_layer / gift_factor arrays themselves are HOST memory, read
 *   during the call only.
 * - All matrices are dense, row-major, with leading dimension = row length.
 *   Every device pointer must be 16-byte aligned.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   Calls only enqueue work on it and return; results are visible to later
 *   work on that stream.  No host synchronisation happens inside a call.
 * - `ws` is a device workspace of at least the size the matching
 *   gift_*_workspace_bytes() query returns.  Its contents on entry are
 *   ignored; on return they are scratch.  Two calls in flight at the same
 *   time (different streams) need different workspaces.
 * - Argument errors are reported synchronously, before anything is
 *   enqueued: the call returns a gift_status other than GIFT_OK and
 *   gift_last_error() holds a one-line explanation.  Errors raised by the
 *   HIP runtime while enqueueing return GIFT_ERR_HIP.
 * - Data-dependent conditions (a non-finite value met while computing an
 *   amax, an all-zero tensor) are not errors: the call OR-s the GIFT_FLAG_*
 *   bits into *dev_flags (when dev_flags is not NULL); the caller zeroes it.
 */
#ifndef GIFT_H
#define GIFT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GIFT_ABI_VERSION 4

/* Rank of the factor (GIFT review, free-parameter ledger: rank 32), and the
 * columns of one rank block: a factor of rank up to 32 stores 32 columns,
 * one of rank 33..64 (the rank sweep's largest) two blocks, 64 columns. */
#define GIFT_RANK 32
#define GIFT_MAX_RANK 64
/* Largest subspace width of the refresh eigensolve (rank + oversampling). */
#define GIFT_MAX_SKETCH 96
/* Row-segment length of 1x128 block scaling. */
#define GIFT_BLOCK 128

typedef enum gift_status {
    GIFT_OK = 0,
    GIFT_ERR_INVALID_ARG = 1,        /* NULL pointer, bad enum, misalignment */
    GIFT_ERR_UNSUPPORTED_SHAPE = 2,  /* a size outside what the kernels take */
    GIFT_ERR_WORKSPACE_TOO_SMALL = 3,
    GIFT_ERR_HIP = 4                 /* HIP runtime error while enqueueing */
} gift_status;

/* Activation dtype for the factor refresh. */
enum { GIFT_DTYPE_F32 = 0, GIFT_DTYPE_BF16 = 1 };

/* Damping reading of the factor (the pages fix neither damping nor scaling):
 *  FLOOR:           lambda_iso = eps * tr(A) / d_in
 *  FLOOR_PLUS_TAIL: lambda_iso = eps * tr(A) / d_in + mean discarded eigenvalue
 *                   (t - sum theta) / (d_in - rank), clamped at 0. */
enum { GIFT_DAMP_FLOOR = 0, GIFT_DAMP_FLOOR_PLUS_TAIL = 1 };

/* Payload format and scaling granularity.
 *  GIFT_SCALE_TENSOR:   E4M3 codes (d_out x d_in bytes), one fp32 inverse
 *                       scale per tensor.
 *  GIFT_SCALE_BLOCK128: E4M3 codes, one fp32 inverse scale per 128
 *                       consecutive elements of a row (d_in % 128 == 0):
 *                       inv_scale is d_out x d_in/128 floats.
 *  GIFT_SCALE_MXFP4:    OCP MXFP4 (OCP Microscaling Formats v1.0): E2M1
 *                       codes, two per byte with the lower-indexed element in
 *                       the low nibble (q is d_out x d_in/2 bytes), and one
 *                       E8M0 scale byte per 32 consecutive elements of a row
 *                       (d_in % 32 == 0): inv_scale points to d_out x d_in/32
 *                       bytes, code c standing for 2^(c - 127), 0xFF for NaN.
 *                       Scale: floor(log2 amax) - 2, clamped to [-127, 127];
 *                       elements round to nearest even and saturate at +-6;
 *                       an all-zero block gets 2^0, a block whose amax is NaN
 *                       or inf the NaN scale (and its NaN elements code 0).
 *                       The FP4 payload is this library's extension of the
 *                       pages' FP8 round trip (GIFT review, "Core claim":
 *                       larger gains expected at lower bit-widths). */
enum { GIFT_SCALE_TENSOR = 0, GIFT_SCALE_BLOCK128 = 1, GIFT_SCALE_MXFP4 = 2 };

/* Bits OR-ed into *dev_flags. */
#define GIFT_FLAG_NONFINITE 1u  /* an amax was NaN or +inf; or (refresh) the
                                   trace of A was, i.e. X held a NaN or an
                                   infinity, or a square overflowed fp32     */
#define GIFT_FLAG_ZERO_AMAX 2u  /* a tensor / block was all zero: scale = 1 */

/* Layout of gift_factor.coef (fp32, GIFT_COEF_COUNT entries) for a factor of
 * 32 storage columns; a factor of 64 columns (rank above 32) has D_w at 8
 * and D_u at 8 + 64, GIFT_COEF_COUNT_64 entries in all. */
enum {
    GIFT_COEF_ALPHA = 0,        /* lambda_iso^-1/2                            */
    GIFT_COEF_BETA = 1,         /* lambda_iso^+1/2                            */
    GIFT_COEF_LAMBDA_ISO = 2,
    GIFT_COEF_LAMBDA_FLOOR = 3,
    GIFT_COEF_TRACE = 4,        /* tr(A)                                      */
    GIFT_COEF_SIGMA2_TAIL = 5,  /* mean discarded eigenvalue                  */
    GIFT_COEF_DW = 8,           /* D_w[32] = (theta+lambda)^-1/2 - lambda^-1/2 */
    GIFT_COEF_DU = 8 + GIFT_RANK, /* D_u[32] = (theta+lambda)^1/2 - lambda^1/2 */
    GIFT_COEF_COUNT = 8 + 2 * GIFT_RANK,
    GIFT_COEF_DU_64 = 8 + GIFT_MAX_RANK,
    GIFT_COEF_COUNT_64 = 8 + 2 * GIFT_MAX_RANK
};

/*
 * Rank-r input-side factor A_r = U diag(theta) U^T + lambda_iso I of one
 * distinct layer input (r = 32 in the review's configuration; its
 * round-trip error table compares ranks, which is why r may be lower).  Its
 * inverse square root is
 *     A_r^-1/2 = alpha I + U diag(D_w) U^T
 * and its square root A_r^1/2 = beta I + U diag(D_u) U^T (U orthonormal).
 * The storage holds C = 32 columns for r <= 32 and C = 64 for 32 < r <= 64:
 * U is d_in x C, theta C floats, coef 8 + 2 C floats (D_w at 8, D_u at
 * 8 + C); the columns of U and the entries of theta, D_w and D_u from r on
 * are zero, so every kernel works on whole 32-column rank blocks and the
 * zero ones add exact zeros.
 * Written by gift_refresh_factor; a caller may also fill it itself.
 *
 * block = 32 or 64 makes it a block-diagonal factor instead ("block-A-b",
 * named in the review's round-trip error table; reading: A is replaced by
 * its d_in/b diagonal b x b blocks A_i, each damped by lambda_floor and
 * used in full): W[:, block i] = G[:, block i] S_i with
 * S_i = (A_i + lambda_floor I)^-1/2, and G^[:, block i] = W^[:, block i]
 * (A_i + lambda_floor I)^1/2.  Then
 *   U     is d_in x 2b: row b i + a holds row a of S_i, then row a of S_i^-1;
 *   theta is d_in floats: each block's eigenvalues, descending, >= 0;
 *   coef  holds LAMBDA_ISO (= lambda_floor), LAMBDA_FLOOR and TRACE, the
 *         rest 0;
 *   packs is required: gift_block_factor_pack_bytes(d_in, b) bytes, S and
 *         S^-1 in the kernels' operand layout;
 *   rank  is not used.
 * d_in % b == 0.  Block factors take per-tensor and 1x128 scaling (not
 * MXFP4) and are not taken by gift_unwhiten_f32.
 */
typedef struct gift_factor {
    int32_t d_in;     /* rows of U; 64 <= d_in, % 16 == 0 (% 32 to whiten)    */
    int32_t rank;     /* effective rank r, 1 <= r <= GIFT_MAX_RANK; the
                         refresh keeps the top r Ritz pairs and damps with
                         d_in - r                                             */
    float *U;         /* device, d_in x C, row-major (C above)                */
    float *theta;     /* device, C: Ritz values, descending, >= 0             */
    float *coef;      /* device, 8 + 2 C floats (layout above)                */
    void *packs;      /* optional device buffer of
                         gift_factor_pack_bytes_rank(d_in, rank) bytes: U
                         split into the bf16 operand layouts of the whitening
                         kernels.  Written by gift_refresh_factor(s) and
                         gift_prepare_factor; it must be rewritten after U
                         changes.  NULL: every grouped call re-packs U into
                         its workspace.                                     */
    int32_t block;    /* 0: the rank-r factor; 32 or 64: block-diagonal
                         factor of that block size (see above)                 */
} gift_factor;

/* Size of gift_factor.packs for a factor with d_in rows (d_in % 32 == 0) of
 * rank up to 32; gift_factor_pack_bytes_rank gives it for any rank (twice
 * that above rank 32), 0 for a rank outside [1, 64]. */
size_t gift_factor_pack_bytes(int64_t d_in);
size_t gift_factor_pack_bytes_rank(int64_t d_in, int rank);

/* Size of gift_factor.packs for a block-diagonal factor (block 32 or 64,
 * d_in % block == 0); 0 for other arguments. */
size_t gift_block_factor_pack_bytes(int64_t d_in, int block);

/* Rewrite f->packs from f->U (for callers that fill U themselves). */
gift_status gift_prepare_factor(const gift_factor *f, void *stream);

/*
 * One layer of a grouped call.  factor == NULL marks a Euclidean layer (plain
 * FP8 of G), otherwise the layer is whitened with *factor (factor->d_in must
 * equal d_in).  Which pointers an entry point reads or writes is listed at
 * the entry point; the others may be NULL.
 */
typedef struct gift_layer {
    int64_t d_out;               /* rows of G, >= 1                            */
    int64_t d_in;                /* columns of G, >= 1; % 4 == 0; % 32 == 0 and
                                    >= 64 when factor != NULL; % 128 == 0 for
                                    block scaling                              */
    const float *G;              /* device, d_out x d_in fp32 gradient         */
    uint8_t *q;                  /* device, d_out x d_in OCP E4M3 codes        */
    float *inv_scale;            /* device: 1 float (tensor scaling) or
                                    d_out x (d_in/128) (block scaling)         */
    float *G_hat;                /* device, d_out x d_in fp32 reconstruction   */
    const gift_factor *factor;   /* HOST pointer or NULL                       */
    float *W_out;                /* optional device d_out x d_in: the whitened
                                    fp32 tensor before scaling (or G itself for
                                    a Euclidean layer); NULL = not written     */
} gift_layer;

/*
 * gift_refresh_factor -- rebuild one factor from a batch of layer inputs
 * (GIFT review, "Load-bearing premise": the factor is refreshed every 50
 * steps; referee report major comment 2: the input-side factor A = E[a a^T]).
 *
 *   A       = X^T X / N                  (bf16 or fp32 X, fp32 accumulation)
 *   t       = tr(A), lambda_floor = damp_eps * t / d_in
 *   Omega   = sketch (device, d_in x sketch_width fp32) or, when sketch is
 *             NULL, a standard Gaussian drawn from Philox4x32-10 with key
 *             `seed` and Box-Muller (element n = i*width + j uses counter
 *             n/4, lanes (0,1) -> pair 1, (2,3) -> pair 2)
 *   Q       = orth(A Omega); power_steps times Q = orth(A Q)
 *   B       = Q^T A Q; theta, V = top-rank eigenpairs of B; U = Q V
 *   lambda_iso, alpha, beta, D_w, D_u per damping_mode (see above).
 *
 * X: device, n_tokens x f->d_in, x_dtype.  f: host struct with device
 * buffers, written.  A_out: optional device d_in x d_in fp32, receives A.
 * sketch_width: 32 <= width <= 96, multiple of 16, at least the rank (the
 * rank sweep's reading: width = rank + 32, i.e. 64 for rank <= 32 and 96
 * for rank 64).  power_steps >= 0.
 * dev_flags: optional device word (4-byte aligned); GIFT_FLAG_NONFINITE is
 * OR-ed into it when tr(A) is not finite (a NaN or infinity in X reaches
 * the diagonal of A).  The factor written in that case is not meaningful;
 * the caller checks the flag before using it.
 */
gift_status gift_refresh_factor(const void *X, int x_dtype, int64_t n_tokens,
                                const gift_factor *f, float damp_eps,
                                int damping_mode, int sketch_width,
                                int power_steps, uint64_t seed,
                                const float *sketch, float *A_out,
                                uint32_t *dev_flags,
                                void *ws, size_t ws_bytes, void *stream);

size_t gift_refresh_workspace_bytes(int64_t d_in, int64_t n_tokens,
                                    int x_dtype, int sketch_width);

/*
 * gift_refresh_factors -- gift_refresh_factor for n inputs in one grouped
 * pass: the covariance runs in launches of up to 16 inputs (in call order),
 * every later launch covers all inputs (up to 1024 at a time), so the small
 * serial steps of the eigensolve of different inputs run concurrently and
 * their latency is paid once per call.  Per input: X (device,
 * n_tokens x factor->d_in, x_dtype), factor (host struct, device buffers
 * written), sketch / A_out optional as above, seed of its Philox sketch.
 * The scalar arguments apply to every input; all factors of one call are of
 * one kind (rank-r or the same block size); dev_flags (optional) collects
 * GIFT_FLAG_NONFINITE over all inputs as in gift_refresh_factor.  The
 * workspace holds, for n > 16, the inputs' launch descriptors, then each
 * input's own area in order (A, the covariance partial tiles unless the
 * input is bf16 with one token range per tile, the subspace-iteration
 * buffers); query it with gift_refresh_group_workspace_bytes.
 */
typedef struct gift_refresh_input {
    const void *X;
    int32_t x_dtype;
    int64_t n_tokens;
    const gift_factor *factor;   /* HOST pointer                              */
    const float *sketch;         /* device d_in x sketch_width, or NULL       */
    float *A_out;                /* device d_in x d_in, or NULL               */
    uint64_t seed;
} gift_refresh_input;

gift_status gift_refresh_factors(const gift_refresh_input *inputs, int n,
                                 float damp_eps, int damping_mode,
                                 int sketch_width, int power_steps,
                                 uint32_t *dev_flags,
                                 void *ws, size_t ws_bytes, void *stream);

size_t gift_refresh_group_workspace_bytes(const gift_refresh_input *inputs,
                                          int n, int sketch_width);

/*
 * gift_draw_sketch -- the Gaussian sketch gift_refresh_factor draws when it
 * is given none: out (device, d_in x width fp32, row-major) element
 * n = i*width + j is normal number n of the Philox4x32-10 stream with key
 * (seed low word, seed high word) (Salmon et al., SC'11): counter
 * (n/4, 0, 0, 0) gives words w0..w3; (w0, w1) and (w2, w3) each make one
 * Box-Muller pair r cos(2 pi u2), r sin(2 pi u2) with r = sqrt(-2 ln u1),
 * u1 = (w + 1) 2^-32, u2 = w 2^-32, evaluated in fp64 and rounded to fp32.
 */
gift_status gift_draw_sketch(float *out, int64_t d_in, int width, uint64_t seed,
                             void *stream);

/*
 * gift_whiten_quantize -- the send side, grouped over n_layers layers.
 * For each layer: W = G A_r^-1/2 (factor != NULL) or W = G (factor == NULL);
 * amax = max |W| per tensor (or per 128-element row segment); scale =
 * 448 / amax, inv = amax / 448 (scale = inv = 1 when amax == 0); q =
 * E4M3(W * scale) rounded to nearest even, saturated to +-448, NaN -> 0x7F.
 * Reads G (and the factor); writes q, inv_scale, and W_out when given.
 * The FP8 format and the scaling rule are this library's reading of
 * "a single FP8 scale factor" ("The pith") and of reference [28].
 */
gift_status gift_whiten_quantize(const gift_layer *layers, int n_layers,
                                 int scaling, uint32_t *dev_flags,
                                 void *ws, size_t ws_bytes, void *stream);

/*
 * gift_whiten_quantize_static -- gift_whiten_quantize for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture
 * that may not call hipMalloc, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, results and flags as gift_whiten_quantize;
 * its scratch (the partial row coefficients, the split c' operands, the tile
 * and layer amax words, the operand packs of factors without packs) lives
 * in a static device array of gift_static_scratch_bytes() bytes (16 MiB)
 * compiled into the library, one per GPU, held until the process ends.  A
 * call whose gift_group_workspace_bytes(GIFT_OP_WHITEN_QUANTIZE, ...) exceeds
 * that size returns GIFT_ERR_WORKSPACE_TOO_SMALL before enqueueing anything
 * (split the group).  The call allocates nothing; its first call on a device
 * looks up that device's copy of the array (hipGetSymbolAddress).  Every
 * call on one GPU uses the same array: calls that overlap in time on one GPU
 * (different streams, or threads) race and must be serialised by the
 * caller.  Nothing in the array needs to start zeroed.
 */
gift_status gift_whiten_quantize_static(const gift_layer *layers, int n_layers,
                                        int scaling, uint32_t *dev_flags,
                                        void *stream);
size_t gift_static_scratch_bytes(void);

/*
 * gift_dequant_unwhiten -- the receive side ("maps the result back", "The
 * pith"): W^ = decode(q) * inv; G_hat = W^ A_r^1/2 (factor != NULL) or
 * G_hat = W^ (factor == NULL).  Reads q, inv_scale (and the factor); writes
 * G_hat.
 */
gift_status gift_dequant_unwhiten(const gift_layer *layers, int n_layers,
                                  int scaling, void *ws, size_t ws_bytes,
                                  void *stream);

/*
 * gift_euclid_fp8_roundtrip -- the Euclidean baseline ("Core claim": the
 * comparison GIFT is measured against): q = E4M3(G * scale), G_hat =
 * decode(q) * inv, ignoring layer.factor.  Reads G; writes q, inv_scale,
 * G_hat.
 */
gift_status gift_euclid_fp8_roundtrip(const gift_layer *layers, int n_layers,
                                      int scaling, uint32_t *dev_flags,
                                      void *ws, size_t ws_bytes, void *stream);

/*
 * gift_roundtrip_error -- per layer l: dev_out[2l] = sum (G_hat - G)^2 and
 * dev_out[2l+1] = sum G^2, accumulated in fp64 in a fixed order (relative
 * reconstruction error, "Core claim").  Reads G and G_hat.
 */
gift_status gift_roundtrip_error(const gift_layer *layers, int n_layers,
                                 double *dev_out, void *ws, size_t ws_bytes,
                                 void *stream);

/*
 * The receive side of a data-parallel reduction of FP8 (or MXFP4) payloads,
 * simulated on one GPU.  In the review's data-parallel setting every rank
 * holds its own gradient and the ranks' quantized whitened gradients are
 * summed in the collective ("Core claim": FP8 communication of the whitened
 * gradients); whitening is linear and the factor is shared, so the sum of
 * the ranks' whitened gradients un-whitens to the sum of their gradients.
 * This library's reading of the sum: fp32 additions of the dequantized
 * payloads, rank by rank in call order, each rank with its own scales.
 *
 * gift_dequant_accumulate -- per layer: G_hat = decode(q) * inv (first != 0)
 * or G_hat = fl32(G_hat + decode(q) * inv), element by element, with the
 * dequantized value formed exactly as gift_dequant_unwhiten forms it.
 * Reads q, inv_scale, G_hat (unless first); writes G_hat.  Ignores factor.
 * Needs no workspace.
 *
 * gift_unwhiten_f32 -- per whitened layer (factor != NULL): G_hat = G_hat
 * A_r^{1/2} in place; other layers are left alone.  Reads and writes G_hat.
 */
gift_status gift_dequant_accumulate(const gift_layer *layers, int n_layers,
                                    int scaling, int first, void *stream);
gift_status gift_unwhiten_f32(const gift_layer *layers, int n_layers,
                              void *ws, size_t ws_bytes, void *stream);

/* Workspace query for the grouped calls.  op: 0 whiten_quantize,
 * 1 dequant_unwhiten, 2 euclid_fp8_roundtrip, 3 roundtrip_error,
 * 4 unwhiten_f32. */
enum { GIFT_OP_WHITEN_QUANTIZE = 0, GIFT_OP_DEQUANT_UNWHITEN = 1,
       GIFT_OP_EUCLID_ROUNDTRIP = 2, GIFT_OP_ROUNDTRIP_ERROR = 3,
       GIFT_OP_UNWHITEN_F32 = 4 };
size_t gift_group_workspace_bytes(int op, const gift_layer *layers,
                                  int n_layers, int scaling);

const char *gift_status_string(int status);
/* Thread-local detail of the last failing call on this thread. */
const char *gift_last_error(void);
int gift_abi_version(void);
/* Hash of the sources the library was built from (16 hex digits), so that a
 * measurement can name the kernels it ran; "unknown" if not set by the build. */
const char *gift_build_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* GIFT_H */
