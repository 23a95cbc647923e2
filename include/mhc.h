/*
 * mhc.h -- C ABI of the fused mHC pre-mapping forward, and of the MhcPre backward, for
 * AMD Instinct MI355X (gfx950).
 *
 * What one call computes, per token t (x viewed as xFlat of length K = n*D):
 *   invRms = (mean(xFlat^2) + normEps)^(-1/2)
 *   hMix   = (xFlat (.) gammaFlat) . phi^T            (gamma optional)
 *   w      = hMix * invRms, split [n, n, n*n] (alpha has 3 entries) or [n, n] (2 entries)
 *   hPre   = sigmoid(alpha0 * wPre + biasPre) + hcEps
 *   hPost  = 2 sigmoid(alpha1 * wPost + biasPost)   (+ hcEps when alpha has 2 entries)
 *   hRes   = Sinkhorn(alpha2 * wRes + biasRes)       (0 when alpha has 2 entries)
 *   hIn[d] = sum_i weight_i * x[i][d], weight = pre_mix[t] if given, else hPre
 * Sources:
 *   - aclnnMhcPreV2 guide (kwkr.cn/news/422178), section 3 (math semantics) and
 *     section 5 (inputs/outputs, optional outputs, shapes);
 *   - aclnnMhcPreSinkhorn guide (m.mzlw.cn/news/197063), section 3.2 (Sinkhorn steps:
 *     a row softmax + hcEps, then alternating column/row normalisations with + hcEps on
 *     every sum, 2*numIters steps, hRes = normOut[2*numIters-1]), section 4 (two-phase
 *     call), section 5.1 (needBackward outputs and their shapes), section 6 (error codes);
 *   - HcPre guide (mhpn.cn/news/2282827), function prototype (pre_mix, hc_pre output)
 *     and parameter defaults (numIters 20, normEps = hcEps = 1e-6).
 *
 * Layout and ownership. Every tensor is a caller-owned, contiguous, row-major device
 * buffer in the TND layout (a [B, S, n, D] input is the same bytes as [B*S, n, D]).
 * bf16 and fp16 tensors are passed as raw 16-bit patterns. The library allocates nothing
 * (the no-allocation entry point's array is static), never synchronises the stream except
 * where an entry point says so (mhc_pre_wait_status), and keeps between calls only what a
 * caller's workspace holds (call counters, which mhc_pre_workspace_size's buffer carries)
 * and, per device, facts it queries once (compute units, which kernels fit).
 *
 * Errors. Every entry point validates on the host before any HIP call and returns:
 *   MHC_OK                 success (also for T == 0: nothing is launched);
 *   MHC_ERR_NULLPTR        a required pointer is NULL;
 *   MHC_ERR_PARAM_INVALID  unsupported size or attribute, inconsistent output set,
 *                          misaligned pointer, or a buffer smaller than required;
 *   MHC_ERR_RUNTIME        a HIP call (kernel launch) failed.
 * The three codes have the values the aclnnMhcPreSinkhorn guide (section 6) lists for
 * the same three classes. Kernel faults surface at the caller's next synchronisation.
 */
#ifndef MHC_H
#define MHC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mhc_status;

#define MHC_OK 0
#define MHC_ERR_NULLPTR 161001
#define MHC_ERR_PARAM_INVALID 161002
#define MHC_ERR_RUNTIME 361001

/* Problem description (host memory; read during the call only).
 *   T              tokens, >= 0
 *   n              hyper-streams (hcMult): 4, 6 or 8 (the aclnnMhcPreV2 guide, section 7.3,
 *                  allows these three; the MhcPreBackward guide, section 5, the same
 *                  three for the backward)
 *   D              hidden size per stream: a multiple of 8 in [8, 16384]; with n == 8 and
 *                  n_alpha == 3 at most 8192
 *   n_alpha        3 (pre/post/res branches, phi has n*n+2n rows) or
 *                  2 (pre/post only, phi has 2n rows, hRes = 0)
 *   num_iters      Sinkhorn iterations, >= 1 (ignored when n_alpha == 2)
 *   norm_eps       > 0 (RMS guard);  hc_eps >= 0 (gate / Sinkhorn guard)
 *   need_backward  0 or 1; with 1 the backward intermediates are mandatory outputs
 *   x_dtype        MHC_DTYPE_BF16 (0) or MHC_DTYPE_F16 (1): the 16-bit format of x and hIn
 *                  (the aclnnMhcPreSinkhorn and aclnnMhcPreV2 guides, section 5.1, list
 *                  BF16 and FLOAT16). With fp16 the weights are packed as three fp16 terms
 *                  scaled by 1, 2^11, 2^22 (phi * gamma must stay within 65504 in
 *                  magnitude); every forward path takes it, and the standalone stages
 *                  read and write fp16 too. hc_post takes either format (its own
 *                  x_dtype), and so does the backward (mhc_pre_bwd_params.x_f16). */
typedef struct mhc_pre_params {
    int64_t T;
    int32_t n;
    int32_t D;
    int32_t n_alpha;
    int32_t num_iters;
    double norm_eps;
    double hc_eps;
    int32_t need_backward;
    int32_t x_dtype;
} mhc_pre_params;

#define MHC_DTYPE_BF16 0
#define MHC_DTYPE_F16 1

/* Device pointers. M = n*n + 2n (n_alpha == 3) or 2n (n_alpha == 2); it = num_iters.
 * Inputs:
 *   x          x_dtype [T, n, D], 16-byte aligned                        required
 *   phi        f32  [M, n*D]                          required unless phi_packed is given
 *   alpha      f32  [n_alpha]                                            required
 *   bias       f32  [M]                                                  required
 *   gamma      f32  [n, D]          scales the projection input only     optional
 *   pre_mix    f32  [T, n]          hIn weights instead of hPre          optional
 *   phi_packed from mhc_pre_prepack for these (n, D, n_alpha, gamma)     optional; when
 *              given, phi and gamma are not read
 * Outputs (must not alias inputs or each other):
 *   h_in       x_dtype [T, D], 16-byte aligned                           required
 *   h_post     f32  [T, n]                                               required
 *   h_res      f32  [T, n, n]    required when n_alpha == 3; with n_alpha == 2 it may be
 *                                NULL, else it is filled with zeros
 *   inv_rms    f32  [T]          optional (required with need_backward)
 *   h_mix      f32  [T, M]       un-normalised projection; optional (required with need_backward)
 *   h_pre      f32  [T, n]       optional (required with need_backward)
 *   sum_out    f32  [2*it, T, n]       step-major Sinkhorn sums; only with n_alpha == 3;
 *                                optional (required with need_backward and n_alpha == 3);
 *                                plane 0 holds the row softmax denominators
 *   norm_out   f32  [2*it, T, n, n]    step-major Sinkhorn matrices; same rules as sum_out */
typedef struct mhc_pre_tensors {
    const uint16_t* x;
    const float* phi;
    const float* alpha;
    const float* bias;
    const float* gamma;
    const float* pre_mix;
    const void* phi_packed;
    uint16_t* h_in;
    float* h_post;
    float* h_res;
    float* inv_rms;
    float* h_mix;
    float* h_pre;
    float* sum_out;
    float* norm_out;
} mhc_pre_tensors;

/* Library version as major*10000 + minor*100 + patch. */
int mhc_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char* mhc_status_string(mhc_status status);

/* Bytes of the packed projection weights for this problem (phi with gamma folded in,
 * split into three bf16 terms and ordered for the matrix cores). Host only; T is
 * ignored. Errors: NULLPTR, PARAM_INVALID. */
mhc_status mhc_pre_packed_size(const mhc_pre_params* params, size_t* bytes);

/* Bytes of device workspace mhc_pre_forward needs for this problem. Host only.
 * The workspace holds per-call intermediate results (partial sums, the hIn weights, the
 * values workgroups of the single-read kernel exchange) and, in its first 256 bytes, a
 * call counter that tags those exchanged values with the call that wrote them. Zero-fill
 * it once after allocating it and then leave it to the library; it may serve calls of
 * any size that fit it, one at a time. Concurrent calls need distinct workspaces.
 * Errors: NULLPTR, PARAM_INVALID. */
mhc_status mhc_pre_workspace_size(const mhc_pre_params* params, size_t* bytes);

/* Packs phi (f32 [M, n*D]) and the optional gamma (f32 [n, D]) into phi_packed
 * (device, >= mhc_pre_packed_size bytes, 16-byte aligned) asynchronously on `stream`
 * (a hipStream_t; NULL = the default stream). Weights are static across calls, so a
 * caller can pack once and pass phi_packed to every forward. T is ignored.
 * Errors: NULLPTR, PARAM_INVALID, RUNTIME. */
mhc_status mhc_pre_prepack(const mhc_pre_params* params, const float* phi, const float* gamma,
                           void* phi_packed, size_t packed_bytes, void* stream);

/* The forward, asynchronous on `stream` (a hipStream_t; NULL = default stream). Emits
 * every non-NULL output listed in mhc_pre_tensors. `workspace` is device memory of at
 * least mhc_pre_workspace_size bytes, 256-byte aligned, zero-filled before its first use.
 * When tensors->phi_packed is NULL the weights are packed from phi (and gamma): by a pack
 * kernel into the workspace on the classic path, inside the kernel on the streaming,
 * single-read and one-launch paths. Then one of four kernel sequences
 * (mhc_pre_forward_path tells which):
 *   classic path: a projection kernel (which with pre_mix also writes hIn) and a
 *     per-token epilogue, which without pre_mix also writes hIn (x is read twice);
 *   streaming path (no pre_mix, D a multiple of 32, n == 4 with either alpha length or
 *     n == 6 or 8 with n_alpha == 2, where neither kernel below serves): the same
 *     epilogue (writing hIn) after a projection by persistent workgroups (one per
 *     compute unit) that keep their slice of the packed weights in LDS, read x in
 *     contiguous 1 KB runs of each token's row and load the next task's x while the
 *     current one is on the matrix cores;
 *   single-read path (n == 4, n_alpha == 3, no pre_mix, 992 < D <= 7168 (32 to 224
 *     blocks of 32 positions), T >= 8192, a device of 8 XCDs with 32 compute units each):
 *     one kernel computes the projection, hPre and hIn, x read once, then the per-token
 *     epilogue. Its workgroups (one per compute unit, in one group of 32 per XCD) wait on
 *     each other, each wait bounded: it needs every compute unit of an XCD at once, as an
 *     otherwise idle device gives; a wait that times out (other work holding compute
 *     units that long) leaves NaN in hIn for the tokens concerned, which
 *     mhc_pre_wait_status reports;
 *   one-launch path (n == 4, n_alpha == 3, no pre_mix, T <= 64, the device able to hold
 *     ceil(D / 32) workgroups of 256 threads at once): the whole forward in one kernel,
 *     one workgroup per block of 32 positions, which exchange their partial sums and hPre
 *     through the workspace (bounded waits, as above: a time-out leaves the token's
 *     outputs NaN, or only hIn when it comes at hPre, and mhc_pre_wait_status reports it).
 *   Every path takes bf16 or fp16 x.
 * Every path can be captured into a HIP graph.
 * The paths sum the projection's partial products in different groupings, so their
 * outputs may differ in the last bits; each meets the same accuracy. Within a call, hIn
 * uses exactly the hPre it emits. Results are bitwise reproducible for the same inputs,
 * parameters and path. The environment variable MHC_FORWARD_PATH = "classic" or
 * "fused" (for tests) overrides the choice: "classic" the classic path, "fused" the
 * single-read kernel where its geometry allows it (neither then takes the one-launch path;
 * "fused" falls back to the streaming or classic path elsewhere).
 * Errors: NULLPTR, PARAM_INVALID, RUNTIME. */
mhc_status mhc_pre_forward(const mhc_pre_params* params, const mhc_pre_tensors* tensors,
                           void* workspace, size_t workspace_bytes, void* stream);

/* mhc_pre_forward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation,
 * outputs and errors, without a workspace argument. The workspace is a device array of
 * 64 MiB that the library holds on every GPU it runs on, from the first such call on that
 * GPU (whose device must be current) to the end of the process; it is zero-filled when the
 * library is loaded and keeps the last call's contents. The call itself allocates nothing.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (different
 * streams, other host threads) race and must not be made. A problem whose
 * mhc_pre_workspace_size exceeds 64 MiB is rejected with MHC_ERR_PARAM_INVALID (it fits
 * up to 7808 tokens at n = 4, D = 7168; 12544 at D = 4096; 25216 at n = 8, D = 2048). The
 * wait-time-out flag of this workspace is not readable through mhc_pre_wait_status.
 * Errors: NULLPTR, PARAM_INVALID, RUNTIME (also when the array's address cannot be
 * obtained on the current device). */
mhc_status mhc_pre_forward_noalloc(const mhc_pre_params* params, const mhc_pre_tensors* tensors,
                                   void* stream);

/* Whether a single-read or one-launch forward that used `workspace` has given up one of
 * its waits since the last report. The single-read kernel's workgroups wait for values
 * other workgroups of their group publish, the one-launch kernel's for every workgroup at
 * its two barriers; each wait is bounded (about 0.3 s of polling), and one that gives up
 * leaves NaN in outputs of the tokens concerned (mhc_pre_forward has already
 * returned MHC_OK by then: it is asynchronous). This call synchronises `stream` (the stream
 * those forwards ran on; NULL = the default stream), then sets *timed_out to 1 if the
 * workspace's time-out flag is set, else 0, and clears the flag. In normal operation the
 * waits end by construction and the flag stays 0; it can be set when the workgroups that
 * wait for each other cannot all run at once (another workload holding compute units for
 * that long).
 *   workspace        the forward's workspace (>= 256 bytes, 256-byte aligned)
 *   workspace_bytes  its size
 * Errors: NULLPTR (workspace or timed_out), PARAM_INVALID (workspace too small or
 * misaligned), RUNTIME (a HIP call failed). */
mhc_status mhc_pre_wait_status(void* workspace, size_t workspace_bytes, void* stream, int32_t* timed_out);

/* Which path mhc_pre_forward would take for these parameters on the current device:
 * *path = 3 the streaming projection, 2 the one-launch kernel, 1 the single-read kernel,
 * 0 the classic path
 * (has_pre_mix: whether pre_mix
 * will be given). Errors: NULLPTR, PARAM_INVALID. */
mhc_status mhc_pre_forward_path(const mhc_pre_params* params, int32_t has_pre_mix, int32_t* path);

/* Events mhc_pre_forward_timed records: one before the first kernel and one after each
 * of the forward's four stages (weight pack, projection, epilogue, hIn). */
#define MHC_FORWARD_EVENTS 5

/* mhc_pre_forward, plus per-kernel timing: also records the caller's events (hipEvent_t
 * handles, created by the caller, who keeps ownership) on `stream`, in this order:
 *   events[0] before the weight-pack kernel,
 *   events[1] after it, before the projection kernel,
 *   events[2] after the projection kernel,
 *   events[3] after the per-token epilogue kernel,
 *   events[4] after the hIn stage, which launches no kernel on any forward path (the
 *     projection writes hIn with pre_mix and on the single-read path, the epilogue
 *     otherwise).
 * A stage the call does not launch a kernel for (the pack when phi_packed is given or on
 * the streaming, single-read and one-launch paths, which pack inside their kernel; the
 * epilogue on the one-launch path; the hIn stage always) has its two events recorded
 * back to back, so elapsed time between events[i] and events[i+1] is kernel i's duration
 * (plus the launch gap) whatever the inputs; with T == 0 all five are recorded back to
 * back. A NULL entry is not recorded: a caller that only wants some boundaries (each
 * record costs a few microseconds on the stream) passes NULL for the others. Computes
 * exactly what mhc_pre_forward computes.
 * Errors: as mhc_pre_forward; NULLPTR also for a NULL events array; PARAM_INVALID when
 * num_events != MHC_FORWARD_EVENTS. */
mhc_status mhc_pre_forward_timed(const mhc_pre_params* params, const mhc_pre_tensors* tensors,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* events, int32_t num_events);

/* ------------------------------------------------------------------ MhcPre backward
 *
 * The gradient of the MhcPre forward (aclnnMhcPreV2 guide, section 3: the same invRms,
 * hMix, gates and hIn as above, with hRes = alpha2 * wRes + biasRes, no Sinkhorn) with
 * respect to x, phi, alpha, bias and gamma, for the scalar whose gradients with respect to
 * hIn, hPost and hRes are given. Source: MhcPreBackward guide (0539edu.com/news/4871844),
 * section 3 (stages 3.1-3.8), section 6.1 (inputs and outputs), section 8.2 (shapes and
 * types: gradX takes gradHIn's type, the other gradients are float32, gradAlpha has 3
 * entries). Per token t, with s = hPre - hcEps and w = hMix * invRms:
 *   gHPre_i = sum_d gradHIn[d] x[i][d]
 *   gW      = [gHPre s(1-s) alpha0 | gradHPost hPost(1-hPost/2) alpha1 | gradHRes alpha2]
 *   gMix    = gW invRms;  gInv = sum_m gW[m] hMix[m]
 *   gradX   = gradHIn[d] hPre_i + (gMix . phi)[k] gamma[k] - gInv invRms^3 x[k] / (n D)
 *             + gradXPost[k]                                   (k = i D + d)
 *   gradPhi[m][k] = sum_t gMix[t][m] x[t][k] gamma[k];  gradGamma[k] = sum_t x[t][k] (gMix[t] . phi)[k]
 *   gradAlpha = sums over t of (gate term * w) per branch;  gradBias = sums of the gate terms
 * The RMS term uses raw x (invRms is defined on raw x); the guide writes x_rs there,
 * which is the same value when gamma is absent. Only the three-entry alpha (n*n + 2n phi
 * rows) has a backward (section 5 of the guide).
 *
 * With num_iters >= 1 the same call is the MhcPreSinkhorn backward: the forward's hRes
 * is then Sinkhorn(alpha2 * wRes + biasRes) (2 num_iters steps, as mhc_pre_forward
 * computes it), and the residual logits' gradient comes back through the forward's saved
 * sum_out / norm_out planes (the aclnnMhcPreSinkhorn guide, section 1, names that
 * backward and those inputs; it gives no formula). With G = gradHRes, for k = 2 it - 1
 * down to 1: a column step (k odd) passes back (G[r][c] - sum_r' G[r'][c] A_k[r'][c]) /
 * s_k[c], a row step (k even) the same along rows, with A_k = norm_out[k] and s_k =
 * sum_out[k]; the first step (row softmax + hcEps) passes back P (G - rowsum(G P)),
 * P = norm_out[0] - hcEps. That logit gradient takes gradHRes's place above.
 *
 * Problem description (host memory):
 *   T          tokens, >= 0
 *   n          4, 6 or 8;  D  a multiple of 8 in [8, 16384]
 *   hc_eps     >= 0: the hcEps the forward used (hPre = sigmoid(...) + hcEps)
 *   num_iters  0: MhcPre backward (affine hRes); 1 .. 1000: MhcPreSinkhorn backward with
 *              that many Sinkhorn iterations
 *   x_f16      0: x, grad_h_in, grad_x_post and grad_x hold bf16; 1: all four hold fp16
 *              (IEEE binary16). The guide's section 8.2 gives gradX gradHIn's type, BF16
 *              or FP16. Other values: PARAM_INVALID. */
typedef struct mhc_pre_bwd_params {
    int64_t T;
    int32_t n;
    int32_t D;
    double hc_eps;
    int32_t num_iters;
    int32_t x_f16;
} mhc_pre_bwd_params;

/* Device pointers, M = n*n + 2n, K = n*D. Inputs (x, grad_h_in and grad_x_post 16-bit
 * values in the format x_f16 names, the rest float32):
 *   x            [T, n, D], 16-byte aligned                            required
 *   phi          [M, K]                                                required
 *   alpha        [3]                                                   required
 *   grad_h_in    [T, D], 16-byte aligned                               required
 *   grad_h_post  [T, n]                                                required
 *   grad_h_res   [T, n, n]                                             required
 *   inv_rms      [T]        the forward's saved invRms                  required
 *   h_mix        [T, M]     the forward's saved (un-normalised) hMix    required
 *   h_pre        [T, n]     the forward's saved hPre                    required
 *   h_post       [T, n]     the forward's saved hPost                   required
 *   gamma        [n, D]                                                optional
 *   grad_x_post  [T, n, D], 16-byte aligned: added to gradX            optional
 * Outputs (must not alias inputs or each other):
 *   grad_x       [T, n, D] in x's format, 16-byte aligned              required
 *   grad_phi     [M, K]                                                required
 *   grad_alpha   [3]                                                   required
 *   grad_bias    [M]                                                   required
 *   grad_gamma   [n, D]     required when gamma is given, else ignored
 * Saved Sinkhorn planes (inputs; required when num_iters >= 1, else ignored):
 *   sum_out      [2 it, T, n]       the forward's sum_out (step-major)
 *   norm_out     [2 it, T, n, n]    the forward's norm_out (step-major)
 * With T == 0 the per-token tensors (x, grad_h_in, grad_h_post, grad_h_res, inv_rms,
 * h_mix, h_pre, h_post, grad_x_post, grad_x, sum_out, norm_out) are empty and may be
 * NULL. */
typedef struct mhc_pre_bwd_tensors {
    const uint16_t* x;
    const float* phi;
    const float* alpha;
    const uint16_t* grad_h_in;
    const float* grad_h_post;
    const float* grad_h_res;
    const float* inv_rms;
    const float* h_mix;
    const float* h_pre;
    const float* h_post;
    const float* gamma;
    const uint16_t* grad_x_post;
    uint16_t* grad_x;
    float* grad_phi;
    float* grad_alpha;
    float* grad_bias;
    float* grad_gamma;
    const float* sum_out;
    const float* norm_out;
} mhc_pre_bwd_tensors;

/* Bytes of device workspace mhc_pre_backward needs. Host only. The workspace holds
 * per-call intermediates only (packed phi, per-token gradients, per-group partial sums)
 * and needs no initialisation. Errors: NULLPTR, PARAM_INVALID. */
mhc_status mhc_pre_backward_workspace_size(const mhc_pre_bwd_params* params, size_t* bytes);

/* The backward, asynchronous on `stream` (a hipStream_t; NULL = default stream).
 * `workspace`: device memory of at least mhc_pre_backward_workspace_size bytes, 256-byte
 * aligned. Every cross-token sum runs in a fixed order, so results are bitwise
 * reproducible for the same inputs. With T == 0, gradPhi, gradAlpha, gradBias and
 * gradGamma are set to zero. Errors: NULLPTR, PARAM_INVALID, RUNTIME. */
mhc_status mhc_pre_backward(const mhc_pre_bwd_params* params, const mhc_pre_bwd_tensors* tensors,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------ standalone stages
 *
 * The HcPre guide (mhpn.cn/news/2282827, "功能说明") splits the pre-mapping into
 * invRms, the mixing projection and the Sinkhorn stage, and names invRms and the Sinkhorn
 * stage as operators of their own; the Sinkhorn operator takes the mixes and the rsqrt as
 * inputs instead of computing them. These two entry points run those stages alone, on
 * the same per-token arithmetic as mhc_pre_forward; they serve callers that already hold
 * the mixes (a projection of their own) and tests that check one stage at a time.
 *
 * mhc_pre_inv_rms: inv_rms[t] = 1 / sqrt(mean over the n*D entries of x[t]^2 + norm_eps)
 * (the same reading of the mean as mhc_pre_forward; aclnnMhcPreV2 guide, section 3).
 * Squares and sums in fp64, one rounding to f32.
 *   params     validated as for mhc_pre_forward (T, n, D and norm_eps are used)
 *   x          x_dtype [T, n, D], 16-byte aligned
 *   inv_rms    f32  [T]
 * Pointers may be NULL only when T == 0. Asynchronous on `stream`, no workspace, no
 * allocation. Errors: NULLPTR, PARAM_INVALID, RUNTIME. */
mhc_status mhc_pre_inv_rms(const mhc_pre_params* params, const uint16_t* x, float* inv_rms,
                           void* stream);

/* mhc_pre_sinkhorn: from the mixes hMix (the un-normalised projection, mhc_pre_forward's
 * h_mix) and invRms, everything the forward derives from them: hPre, hPost, the Sinkhorn
 * of the res logits with its planes, and hIn (aclnnMhcPreSinkhorn guide, m.mzlw.cn/news/
 * 197063, sections 3.1 and 3.2; aclnnMhcPreV2 guide, section 3). Outputs follow the rules
 * of mhc_pre_tensors, except that h_pre is always required (it carries the hIn weights
 * when pre_mix is not given).
 *   params     as for mhc_pre_forward; need_backward makes sum_out / norm_out mandatory
 *              (n_alpha == 3)
 * Inputs:  x x_dtype [T, n, D] (16-byte aligned), h_mix f32 [T, M], inv_rms f32 [T],
 *          alpha f32 [n_alpha], bias f32 [M], pre_mix f32 [T, n] (optional)
 * Outputs: h_in x_dtype [T, D] (16-byte aligned), h_pre, h_post f32 [T, n], h_res f32 [T, n, n]
 *          (required when n_alpha == 3), sum_out / norm_out as in mhc_pre_tensors
 * Pointers may be NULL only when T == 0. Asynchronous on `stream`, no workspace, no
 * allocation. Errors: NULLPTR, PARAM_INVALID, RUNTIME. */
typedef struct mhc_pre_sinkhorn_tensors {
    const uint16_t* x;
    const float* h_mix;
    const float* inv_rms;
    const float* alpha;
    const float* bias;
    const float* pre_mix;
    uint16_t* h_in;
    float* h_pre;
    float* h_post;
    float* h_res;
    float* sum_out;
    float* norm_out;
} mhc_pre_sinkhorn_tensors;

mhc_status mhc_pre_sinkhorn(const mhc_pre_params* params, const mhc_pre_sinkhorn_tensors* tensors,
                            void* stream);

/* ------------------------------------------------------------------ hc_post
 *
 * The mHC post-mapping (HcPre guide, mhpn.cn/news/2282827, section "mHC 架构与 HcPre 的
 * 定位"): the layer output x is expanded back into the n streams by post (the forward's
 * hPost) and added to the streams fused across streams by comb (the forward's hRes):
 *     out[t][j][d] = post[t][j] x[t][d] + sum_i comb[t][i][j] residual[t][i][d]
 * This is the guide's printed broadcast expression evaluated on the [b, s, n, n] comb_frag
 * its section "返回值说明" documents: the sum runs over comb's first index, so output
 * stream j takes column j of comb (comb transposed times the residual streams). fp32 fused
 * multiply-adds (post term first, then i in order), one rounding to the 16-bit format.
 *   T >= 0; n: 4, 6 or 8; D: a multiple of 8 in [8, 16384]
 *   x        x_dtype [T, D]       16-byte aligned    (the attention / MLP output)
 *   residual x_dtype [T, n, D]    16-byte aligned    (the n streams)
 *   post     f32     [T, n]
 *   comb     f32     [T, n, n]
 *   out      x_dtype [T, n, D]    16-byte aligned; must not alias the inputs
 * Pointers may be NULL only when T == 0 (nothing is launched). Asynchronous on `stream`,
 * no workspace, no allocation. Errors: NULLPTR, PARAM_INVALID, RUNTIME. */
typedef struct mhc_post_params {
    int64_t T;
    int32_t n;
    int32_t D;
    int32_t x_dtype;    /* MHC_DTYPE_BF16 or MHC_DTYPE_F16: the format of x, residual and out */
    int32_t reserved;   /* must be 0 */
} mhc_post_params;

typedef struct mhc_post_tensors {
    const uint16_t* x;
    const uint16_t* residual;
    const float* post;
    const float* comb;
    uint16_t* out;
} mhc_post_tensors;

mhc_status mhc_post(const mhc_post_params* params, const mhc_post_tensors* tensors, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MHC_H */
