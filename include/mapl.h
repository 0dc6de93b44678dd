/*
 * mapl.h -- C ABI of the MAPL pipeline-boundary activation codec for AMD
 * Instinct MI355X (gfx950).
 *
 * The method is that of "Learned Subspace Compression for Communication-
 * Efficient Pipeline Parallelism" (MAPL).  A boundary activation X (B x T x d,
 * flattened to N = B*T rows) is compressed on the sending stage to
 * Z = (X - E_small[tids] P) A  (Section 3.2, Eq. (1)) and rebuilt on the
 * receiving stage as Xhat = Z A^T + E_small'[tids] P'  (Eq. (2)), with
 * A in St(d, r) (A^T A = I_r), E_small in R^{V x r} trainable and
 * P in R^{r x d} a frozen random orthonormal matrix (Eq. (3)).  The projector
 * is updated once per optimizer step by SPEL (Section 3.3, Eq. (4)-(7),
 * Algorithm 1), and Z may further be vector-quantised over G groups and R
 * residual rounds (Section 3.5) with streamed codebook sync (Appendix F).
 *
 * Conventions shared by every entry point
 *  - Every tensor argument is a caller-owned, contiguous, row-major DEVICE
 *    pointer.  The library never allocates, frees or keeps a pointer.
 *  - Work is enqueued on `stream` (NULL = the default stream) and the call
 *    returns without synchronising; outputs are valid once the stream is.
 *  - Outputs must not alias inputs, except where an argument is documented as
 *    updated in place.
 *  - Each call returns MAPL_OK (0) or a negative status.  Arguments are
 *    validated on the host before anything is enqueued; on a validation error
 *    nothing is enqueued and no output is touched.  A failed launch is
 *    reported as MAPL_ERR_HIP (no synchronisation is done to detect it).
 *  - `dt` selects the storage type of every floating-point tensor of a codec
 *    call (X, Xhat, Z, gZ, gX, gXhat, E_small, P, A): MAPL_BF16 (bf16 storage,
 *    fp32 accumulation, one round-to-nearest-even on output) or MAPL_F32.
 *    gA is always fp32.
 *  - Token ids are int32.  A token id outside [0, V) is a caller error; the
 *    kernels never read out of bounds for it (its anchor row is taken as
 *    zero), and mapl_check_tids counts such ids on the device (the Python
 *    binding, with MAPL_CHECK=1 in the environment, runs it before every map
 *    that reads ids and raises MAPL_ERR_TID).
 *  - Before its first launch on a device every entry point raises the
 *    dynamic-LDS limit of the kernels that use more than 64 KB (mapl_init);
 *    if the runtime refuses, the call returns MAPL_ERR_HIP and enqueues
 *    nothing.
 *  - Shape limits of the bf16 codec path: d % 128 == 0, r a power of two
 *    with 32 <= r <= 512, r <= d.  The fp32 path needs 1 <= r <= d <= 4096.
 *  - The library holds no state between calls and is reentrant; calls on
 *    different streams may overlap when their outputs and workspaces differ.
 */
#ifndef MAPL_H
#define MAPL_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MAPL_F32 = 0, MAPL_BF16 = 1 } mapl_dtype;

enum {
  MAPL_OK = 0,
  MAPL_ERR_NULL = -1,      /* a required pointer is NULL                       */
  MAPL_ERR_SHAPE = -2,     /* a size is out of range or breaks an alignment    */
  MAPL_ERR_DTYPE = -3,     /* unsupported dtype                                */
  MAPL_ERR_ARG = -4,       /* a scalar argument is out of range                */
  MAPL_ERR_WORKSPACE = -5, /* workspace or pack buffer too small               */
  MAPL_ERR_HIP = -6,       /* the HIP runtime reported an error (device set-up  *
                            * or launch)                                        */
  MAPL_ERR_TID = -7        /* a token id is outside [0, V) (raised by the       *
                            * binding's MAPL_CHECK=1 mode from mapl_check_tids) */
};

/* Human-readable text for a status code (static storage, never NULL). */
const char* mapl_status_string(int status);

/* Library version string (static storage). */
const char* mapl_version(void);

/* Prepare the current device: raise the dynamic-LDS limit of every kernel
 * that needs more than the default 64 KB (at most 160 KB, the LDS of one
 * gfx950 workgroup).  Every entry point does this itself, once per device,
 * before its first launch; calling it first only moves that cost.  Returns
 * MAPL_OK, or MAPL_ERR_HIP when there is no usable device or the runtime
 * refuses a limit. */
int mapl_init(void);

/* ------------------------------------------------------------------------
 * Packed weights.
 *
 * Anchor rank.  Every codec entry point takes ra, the rank of the anchor
 * E_small [V][ra] P [ra][d].  Eq. (3) and Table 8 use ra = r; Appendix G's
 * Table 6 ablates the anchor: ra = 0 is "no anchor" (tids, E_small and P are
 * then ignored and may be NULL), and ra = d with P = I is the full trainable
 * anchor E [V][d] (also the first stage's subtraction of the token embedding,
 * Figure 2).  For that one, pass P = NULL with ra == d: the maps then subtract
 * or add the rows E[t] themselves (no d x d product; a dense identity P gives
 * the same result through the general path, at the cost of that product).
 * bf16 takes ra == 0, ra == r, or ra a multiple of 64 with r a multiple of 64;
 * every path takes 0 <= ra <= d.
 *
 * The bf16 codec kernels read A and P through a packed copy laid out for the
 * matrix cores: the operands A^T (r x d), A (d x r), P^T (d x ra), P (ra x d)
 * and -(P A)^T (r x ra, formed with fp32 accumulation and rounded once), all bf16
 * and stored in fragment order, i.e. as the 64-lane x 16-byte pieces one
 * v_mfma_f32_32x32x16_bf16 consumes, so that every weight load of a wave is
 * one contiguous kilobyte.  In training A changes once per optimizer step
 * (SPEL) and P never, so one pack serves every micro-batch of a step.
 * Every bf16 codec entry point takes (pk, pk_bytes, pk_ready): with
 * pk_ready == 0 the call first rebuilds the pack from its own P and A
 * arguments (mapl_reconstruct_bwd, which has no P, rebuilds only the A^T
 * part; mapl_anchor_grad, which has no A, only the P part); with
 * pk_ready == 1 the caller guarantees that pk holds
 * mapl_pack(P, A) of exactly these matrices (and this ra).  For
 * dt == MAPL_F32 no pack is used (pk may be NULL and mapl_pack_bytes returns 0).
 * ---------------------------------------------------------------------- */
size_t mapl_pack_bytes(int64_t d, int64_t r, int64_t ra, mapl_dtype dt);

/* Build the whole pack from P [ra][d] and A [d][r] (bf16; P unused when ra == 0). */
int mapl_pack(const void* P, const void* A, void* pk, size_t pk_bytes,
              int64_t d, int64_t r, int64_t ra, mapl_dtype dt, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Forward codec (Section 3.2, Eq. (1)-(3); Algorithm 1 steps 1 and 3).
 * ---------------------------------------------------------------------- */

/* Eq. (1): Z[N][r] = (X[N][d] - E_small[tids] P) A,  N = B*T.
 * X [N][d], tids [N], E_small [V][ra], P [ra][d], A [d][r] -> Z [N][r].
 * The bf16 path evaluates the exact re-association X A - E_small[tids] (P A). */
int mapl_compress(const void* X, const int32_t* tids, const void* E_small,
                  const void* P, const void* A, void* Z,
                  int64_t B, int64_t T, int64_t d, int64_t r, int64_t ra, int64_t V,
                  mapl_dtype dt, void* pk, size_t pk_bytes, int pk_ready,
                  hipStream_t stream);

/* Instrumentation for benchmarks (not part of the method): arms the calling
 * thread so that the compress kernel of its next mapl_compress call is
 * launched with hipExtLaunchKernelGGL carrying `start` and `stop`
 * (hipEvent_t, created by the caller with timing enabled and owned by it).
 * The events then take that kernel's own begin and end time stamps, which
 * hipEventRecord markers around the call cannot give (each marker is a packet
 * of its own on the queue).  The next mapl_compress call on the thread takes
 * the arming whatever its outcome; one that cannot be timed this way (dt !=
 * MAPL_BF16, r >= 512, or B * T == 0) returns MAPL_ERR_ARG and launches
 * nothing.  The events bracket the compress kernel only, not the pack kernel
 * of a call with pk_ready == 0.  Both NULL disarms; exactly one NULL returns
 * MAPL_ERR_NULL. */
int mapl_time_next_compress_kernel(void* start, void* stop);

/* Eq. (2): Xhat[N][d] = Z A^T + E_small[tids] P.  Pass the RECEIVING stage's
 * anchor (E_{p+1}, P_{p+1}) and the sender's projector A. */
int mapl_reconstruct(const void* Z, const int32_t* tids, const void* E_small,
                     const void* P, const void* A, void* Xhat,
                     int64_t B, int64_t T, int64_t d, int64_t r, int64_t ra, int64_t V,
                     mapl_dtype dt, void* pk, size_t pk_bytes, int pk_ready,
                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * Backward of both maps (Section 3.1 "Setup": the backward pass sends the
 * gradient across the same boundary; Section 3.2: it is routed through the
 * same projector).  gA is fp32 [d][r]; accumulate == 0 overwrites it,
 * accumulate == 1 adds into it (to sum both maps' terms and micro-batches).
 * The reduction over tokens is deterministic (fixed split and order, no
 * floating-point atomics); it uses `ws` of mapl_bwd_workspace_bytes(), which
 * serves both maps.
 * ---------------------------------------------------------------------- */
size_t mapl_bwd_workspace_bytes(int64_t B, int64_t T, int64_t d, int64_t r, int64_t ra, mapl_dtype dt);

/* Receiver side, given gXhat = dL/dXhat [N][d]:
 *   gZ[N][r] = gXhat A ;   gA (+)= gXhat^T Z.
 * Uses the A^T part of the pack (rebuilt from A when pk_ready == 0). */
int mapl_reconstruct_bwd(const void* gXhat, const void* Z, const void* A,
                         void* gZ, float* gA, int accumulate,
                         int64_t B, int64_t T, int64_t d, int64_t r,
                         mapl_dtype dt, void* pk, size_t pk_bytes, int pk_ready,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* Sender side, given gZ = dL/dZ [N][r]:
 *   gX[N][d] = gZ A^T ;   gA (+)= (X - E_small[tids] P)^T gZ.
 * The bf16 path evaluates the exact re-association
 *   X^T gZ - P^T (E_small[tids]^T gZ). */
int mapl_compress_bwd(const void* gZ, const void* X, const int32_t* tids,
                      const void* E_small, const void* P, const void* A,
                      void* gX, float* gA, int accumulate,
                      int64_t B, int64_t T, int64_t d, int64_t r, int64_t ra, int64_t V,
                      mapl_dtype dt, void* pk, size_t pk_bytes, int pk_ready,
                      void* ws, size_t ws_bytes, hipStream_t stream);

/* Anchor-table gradient (Section 3.2 and Eq. (3): E_small is trainable; its
 * row t_n enters Eq. (1) as -E[t_n] P A and Eq. (2) as +E'[t_n] P').  For a
 * d-wide token gradient Y [N][d]:
 *   gE[v] (+)= alpha * sum over the tokens n with tids[n] == v of Y[n] P^T
 * - receiver's table (Eq. (2)): Y = gXhat, alpha = +1, P = the receiver's P;
 * - sender's table (Eq. (1)):   Y = gX = gZ A^T (the gX output of
 *   mapl_compress_bwd), alpha = -1, since gZ (P A)^T = (gZ A^T) P^T;
 * - a table shared by both sides: two calls, the second with accumulate = 1.
 * Y and P [ra][d] use `dt`; gE is fp32 [V][ra] (accumulate == 0 overwrites all
 * V rows, 1 adds); r is the projector's rank, on which the pack's layout
 * depends.  P = NULL with ra == d is the full-rank anchor (P = I: the rows
 * alpha Y[n] themselves; no pack is read).  Tokens whose id is outside
 * [0, V) contribute nothing.  The sums
 * are exact 64-bit fixed-point accumulations at one power-of-two scale chosen
 * from max |alpha Y[n] P^T| (every sum fits; each term is rounded once, by
 * at most 2^-30 times that maximum), so the result does not depend on the
 * order of the additions: it is bitwise repeatable.  If any projected value
 * alpha Y[n] P^T is not finite (Y holds NaN or Inf, or the product
 * overflows), no such scale exists and every row of gE is set to NaN
 * (accumulate == 1 included), so a diverging gradient is never silently lost
 * or clipped (alpha non-finite: MAPL_ERR_ARG).  bf16 reads P through the pack (pk,
 * pk_bytes, pk_ready as for the codec; pk_ready == 0 rebuilds only its P
 * part from this P, so a receiver passes the pack of its own P').  Uses a
 * 16-byte aligned `ws` of mapl_anchor_grad_workspace_bytes() (MAPL_ERR_ARG if
 * misaligned): N*ra fp32 projected rows and partial maxima.  Shapes follow
 * the codec rules (bf16: d % 128 == 0, r a power of two in [32, 512], and the
 * anchor-rank rules above with 1 <= ra); V <= 2^22, N < 2^24, N*ra <= 2^38. */
size_t mapl_anchor_grad_workspace_bytes(int64_t B, int64_t T, int64_t ra, int64_t V);
int mapl_anchor_grad(const void* Y, const int32_t* tids, const void* P, float* gE, float alpha,
                     int accumulate, int64_t B, int64_t T, int64_t d, int64_t r, int64_t ra, int64_t V,
                     mapl_dtype dt, void* pk, size_t pk_bytes, int pk_ready,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Count token ids outside [0, V) into *bad_count (device int32, overwritten). */
int mapl_check_tids(const int32_t* tids, int64_t N, int64_t V, int32_t* bad_count,
                    hipStream_t stream);

/* ------------------------------------------------------------------------
 * Residual multi-codebook VQ of Z (Section 3.5; Appendix E.4, Appendix F).
 *
 * Z [N][r] is split into G groups of width w = r/G (group g = columns
 * [g w, (g+1) w)).  Codebooks are fp32; codeword k of group g used in round
 * rho starts at C + rho*C_round_stride + (g*K + k)*w.  C_round_stride = 0
 * shares one codebook across all rounds (the paper's single per-stage C_p);
 * C_round_stride >= r*K gives each round its own.  Codes are uint8
 * [N][R][G] at codes[(n*R + rho)*G + g], so K <= 256.
 * Limits: w in {2, 4, 8, 16, 32, 64}, 1 <= K <= 256, 1 <= R <= 64;
 * C 16-byte aligned and C_round_stride a multiple of 4 (codeword rows move as
 * 16-byte vectors; MAPL_ERR_ARG otherwise); rvq_encode also needs Z 16-byte
 * aligned.
 * ---------------------------------------------------------------------- */

/* Encode: for rho = 0..R-1 and each group, code = argmin_k ||res - c_k||^2
 * (squared Euclidean; exact ties go to the lowest k; a NaN distance never
 * wins; a group whose distances are all NaN gets code 0), then res -= c_code.
 * res starts as Z (z_dt: MAPL_BF16 or MAPL_F32) and is kept in fp64, which
 * holds z - c_1 - ... exactly for inputs of ordinary range, so the codes are
 * those of exact arithmetic.  The K codewords are first scored on the matrix
 * cores (bf16 for w >= 16, fp32 below) with a proven bound on the scoring
 * error, and every codeword that can still be the argmin is then scored
 * exactly as sum_j (res_j - c_kj)^2 in fp64. */
int rvq_encode(const void* Z, mapl_dtype z_dt, const float* C, int64_t C_round_stride,
               uint8_t* codes, int64_t N, int64_t r, int64_t G, int64_t K, int64_t R,
               hipStream_t stream);

/* Decode: Zq[n][g*w + j] = sum over rho (in order) of codeword codes[n][rho][g]
 * of round rho, accumulated in fp32 and stored as out_dt. */
int rvq_decode(const uint8_t* codes, const float* C, int64_t C_round_stride,
               void* Zq, mapl_dtype out_dt, int64_t N, int64_t r, int64_t G,
               int64_t K, int64_t R, hipStream_t stream);

/* Streaming codebook sync on the receiver (Section 3.5 "Codebook
 * Synchronization", Appendix F): overwrite n whole codewords.  idx [n] holds
 * flat codeword indices q in [0, R_c*G*K) where codeword q starts at C + q*w;
 * vals [n][w] holds the sender's values, copied bit-exactly.  Out-of-range
 * indices are skipped.  Duplicate indices in one call: the last one wins. */
int rvq_stream_apply(float* C, const int32_t* idx, const float* vals, int64_t n,
                     int64_t r, int64_t G, int64_t K, int64_t R_c, hipStream_t stream);

/* The receiver's codebook sync followed by its decode (Section 3.5 "Codebook
 * Synchronization" and the decode above), in one launch: bit for bit the
 * effect of rvq_stream_apply(C, idx, vals, n, r, G, K, R_c) and then
 * rvq_decode(codes, C, C_round_stride, Zq, out_dt, N, r, G, K, R), with every
 * argument meaning what it means there (C updated in place, R_c books for the
 * sync, R rounds for the decode).  One launch covers packets of up to 64
 * codewords with w >= 8, w % 4 == 0, vals 16-byte aligned and C_round_stride
 * a multiple of w; other calls run the two launches in that order.
 * Errors: those of the two calls (shape, null, dtype, alignment of C). */
int rvq_stream_decode(float* C, int64_t C_round_stride, int64_t R_c, const int32_t* idx,
                      const float* vals, int64_t n, const uint8_t* codes, void* Zq,
                      mapl_dtype out_dt, int64_t N, int64_t r, int64_t G, int64_t K, int64_t R,
                      hipStream_t stream);

/* ------------------------------------------------------------------------
 * SPEL projector update (Section 3.3, Eq. (4)-(7), Algorithm 1 step 4).
 *
 * On fp32 A [d][r] (updated in place) and momentum m [d][r] (updated in
 * place), given the Euclidean gradient g [d][r]:
 *   g_R = g - A sym(A^T g),  sym(M) = (M + M^T)/2          (Eq. 4)
 *   m   = beta m + (1 - beta) g_R                            (Eq. 5)
 *   D   = NS(m / ||m||_F)   (D = 0 when m == 0)              (Eq. 6)
 *   A   = NS(A - alpha D)   (input not rescaled)             (Eq. 7)
 * with NS the cubic Newton-Schulz polar iteration X <- 1.5 X - 0.5 X (X^T X)
 * run ns_iters times (the method uses 8).  If D_out is not NULL the
 * direction D [d][r] is also written there.  A, g, m, D_out and ws must be
 * 16-byte aligned (MAPL_ERR_ARG otherwise) and no buffer may overlap another.
 * The workspace needs no initial contents; consecutive calls on one stream
 * may share it, calls that overlap in time may not.
 * For r <= 256 both polar maps run as iterations on r x r matrices (every
 * iterate is the input times a polynomial in its Gram matrix, so the result is
 * the same up to rounding): each map is one launch of 2r (r <= 128) or r
 * workgroups that wait for one another through counters in the workspace.
 * They need to be resident together; the library checks once per device that
 * the device can hold them all (an MI355X can), and otherwise -- or for
 * r > 256, or with the environment variable MAPL_SPEL_GRAM_SPACE=0 -- runs
 * every Newton-Schulz step on the d x r iterate, with no waits.  Should a wait
 * last beyond about a second (a device kept full by other work), the step is
 * abandoned rather than the call hanging.
 * The step is transactional: the new m and A are formed in the workspace and
 * the last launch writes both only if no wait timed out; an abandoned step
 * leaves A and m exactly as they were (D_out, if given, is then unspecified).
 * `status`, if not NULL, is a device int32 set to 0 when the step was applied
 * and to 1 when it was abandoned.
 * Limits: r % 32 == 0, d % 32 == 0, r <= d, r <= 1024, 0 <= beta < 1,
 * 0 <= alpha <= 0.7, 1 <= ns_iters <= 64; status 4-byte aligned.
 * ---------------------------------------------------------------------- */
size_t spel_workspace_bytes(int64_t d, int64_t r);

int spel_step(float* A, const float* g, float* m, float alpha, float beta, int ns_iters,
              float* D_out, int32_t* status, int64_t d, int64_t r, void* ws, size_t ws_bytes,
              hipStream_t stream);

/* For callers that cannot allocate -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc: spel_step with no `ws`
 * argument.  Its workspace is a static device array of the library,
 * MAPL_STATIC_SCRATCH_BYTES long, of which each GPU the library runs on holds
 * its own copy until the process ends; its address is looked up once per
 * device when the device is set up (mapl_init, or the first call on that
 * device).  The call allocates nothing (no hipMalloc, hipFree or allocating
 * library routine).  Shapes whose spel_workspace_bytes(d, r) exceeds
 * MAPL_STATIC_SCRATCH_BYTES (e.g. d x r = 2048 x 256 fits, 4096 x 256 does
 * not) are rejected with MAPL_ERR_WORKSPACE.  The array keeps the last call's
 * contents, and everything the step needs cleared it clears itself, in a
 * kernel.  Every call on one GPU shares that GPU's array: calls that overlap
 * in time on one GPU (different streams, or several threads) race and give
 * wrong results; calls on one stream are ordered and safe.  Arguments,
 * results, status and errors otherwise as for spel_step. */
#define MAPL_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
int spel_step_static(float* A, const float* g, float* m, float alpha, float beta, int ns_iters,
                     float* D_out, int32_t* status, int64_t d, int64_t r, hipStream_t stream);

/* The same SPEL step with the Polar Express polar map that Section 3.3 and
 * Table 8 name (5 LMO steps, 7 retraction steps; the pages print no
 * coefficients).  Step t multiplies X on the right by a I + b S + c S^2,
 * S = X^T X: the odd quintic a x + b x^3 + c x^5 of the singular values that
 * best approximates 1, uniformly, on the interval [l_t, u_t] the values are
 * known to lie in (Remez exchange); [l_1, u_1] = [ell, 1] and
 * [l_{t+1}, u_{t+1}] = [1 - E_t, 1 + E_t], E_t the step's maximum error;
 * intervals narrower than 1e-4 take the limit quintic (15 x - 10 x^3 +
 * 3 x^5) / 8.  Both polar inputs, m and A - alpha D, are scaled by their
 * Frobenius norms first (D = 0 when m == 0).  The schedule is computed on the
 * host in double and rounded to fp32.  Buffers, workspace
 * (spel_workspace_bytes), status and the other limits as for spel_step (this
 * form has no waits between workgroups, so the step is always applied);
 * 1 <= lmo_steps, ret_steps <= 32, 0 < ell < 1 (MAPL_ERR_ARG otherwise). */
int spel_step_polar_express(float* A, const float* g, float* m, float alpha, float beta, int lmo_steps,
                            int ret_steps, float ell, float* D_out, int32_t* status, int64_t d, int64_t r,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Host only: the Polar Express schedule above from [ell, 1]: coef [steps][3]
 * = (a, b, c) of each step and, if err is not NULL, err [steps] = E_t.
 * 0 < ell < 1, 1 <= steps <= 32 (MAPL_ERR_ARG otherwise). */
int spel_polar_express_coefficients(double ell, int steps, double* coef, double* err);

#ifdef __cplusplus
}
#endif

#endif /* MAPL_H */
