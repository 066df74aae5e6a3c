/*
 * gdnrt -- gated delta-rule recurrent state update on AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels. Every pointer argument is device memory
 * owned by the caller (except the leapq_state struct itself, which is read on the
 * host during the call). The library allocates no device memory and keeps no
 * state between calls. Work is enqueued on `stream` (a hipStream_t; NULL means the
 * null stream) and is complete when that stream is synchronised.
 *
 * Orientation: every recurrent state is stored [d_v][d_k] row-major fp32: one row
 * per value channel, contiguous along the key channels. The pages that define the
 * method write d_k x d_v; their formulas apply transposed.
 *
 * Errors: arguments are validated on the host before anything is launched; on a
 * failed check nothing is launched and a gdnrt_status is returned. Nothing throws
 * across the ABI and no call aborts. gdnrt_last_error() returns a message for
 * the calling thread's last non-OK status.
 *
 * Shapes supported by this build: d_k = d_v = 128, chunk = 64, window <= 16,
 * rank <= 8. Anything else returns GDNRT_ESHAPE. Empty work (N == 0 or T == 0)
 * returns GDNRT_OK and launches nothing.
 *
 * Precision: accumulation is fp32. Inputs q, k, v and the output o have the dtype
 * `io` (GDNRT_F32 or GDNRT_BF16); gates and states are fp32. q and k are used as
 * given: the library does not normalise them and applies no 1/sqrt(d) scale.
 */
#ifndef GDNRT_H
#define GDNRT_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define GDNRT_API __attribute__((visibility("default")))
#else
#define GDNRT_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDNRT_OK = 0,
  GDNRT_EINVAL = 1,  /* null pointer, bad enum, overlapping buffers            */
  GDNRT_ESHAPE = 2,  /* unsupported or negative size                           */
  GDNRT_EALIGN = 3,  /* a pointer is not 16-byte aligned                       */
  GDNRT_EDTYPE = 4,  /* io is not GDNRT_F32 / GDNRT_BF16                       */
  GDNRT_ESTATE = 5,  /* window position out of range                           */
  GDNRT_ELAUNCH = 6  /* the HIP runtime reported an error at launch            */
} gdnrt_status;

typedef enum { GDNRT_F32 = 0, GDNRT_BF16 = 1 } gdnrt_dtype;

/* Flag or-ed into gla_chunk_fwd's io: also leave in the workspace what the
 * sequence-parallel shard calls below read (gla_shard_decay, gla_shard_output_correct). */
enum { GDNRT_GLA_SHARD = 0x100 };

/*
 * Gated DeltaNet recurrent step ("LeapQuant: an 8-bit recurrent state that stops
 * rounding every token", section "The state, from the update rule up": the delta
 * rule with a scalar per-token decay; section "Why a decode step is a memory
 * copy"). For each of N independent heads and each of T consecutive tokens:
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t.
 *
 *   S      [N][dv][dk] fp32, read and updated in place (initial -> final state).
 *   q, k   [N][T][dk]  io dtype.       v, o  [N][T][dv] io dtype.
 *   alpha, beta [N][T] fp32.
 * o must not overlap any input. Decode is T = 1 per call; T > 1 runs the tokens
 * back to back with the state held on chip.
 */
GDNRT_API int gdn_decode_step(float* S, const void* q, const void* k, const void* v,
                    const float* alpha, const float* beta, void* o,
                    int N, int T, int dk, int dv, int io, void* stream);

/*
 * Kimi Delta Attention recurrent step: the same delta rule with the decay a vector,
 * one factor per key channel ("LeapQuant: an 8-bit recurrent state that stops
 * rounding every token", section "The state, from the update rule up", eq. 1 and
 * eq. 3). In the [d_v][d_k] layout, per head and token:
 *
 *     u_t = beta_t (v_t - S_{t-1} (alpha_t o k_t)),
 *     S_t = S_{t-1} Diag(alpha_t) + u_t k_t^T,   o_t = S_t q_t.
 *
 * Arguments as gdn_decode_step except alpha: [N][T][dk] fp32, 16-byte aligned.
 */
GDNRT_API int kda_decode_step(float* S, const void* q, const void* k, const void* v,
                    const float* alpha, const float* beta, void* o,
                    int N, int T, int dk, int dv, int io, void* stream);

/*
 * Gated linear attention, chunkwise forward of one sequence shard that starts
 * from an incoming state ("ZeCO: Zero Communication Overhead Sequence Parallelism
 * for Linear Attention", section "Gated Linear Attention (GLA) Formulation" for
 * the per-token and chunk forms, section "Global State Update Formula", eq. 6, for
 * the incoming state). Per token, with per-key-channel log-gates g_t:
 *
 *     S_t[v,k] = exp(g_t[k]) S_{t-1}[v,k] + v_t[v] k_t[k],   o_t = S_t q_t.
 *
 *   q, k   [N][T][dk] bf16.   v, o [N][T][dv] bf16.   log_g [N][T][dk] fp32 (<= 0).
 *   S0     [N][dv][dk] fp32 incoming state, or NULL for zero.
 *   ST     [N][dv][dk] fp32 final state (may equal S0: read before written).
 *   io     GDNRT_BF16, or GDNRT_BF16 | GDNRT_GLA_SHARD for a shard of the
 *          sequence-parallel calls below.
 *   workspace: caller-owned device memory of gla_chunk_fwd_workspace_bytes() bytes,
 *   16-byte aligned, overwritten: 16,896 bytes per chunk that GDNRT_GLA_SHARD fills
 *   (Q o e^b in bf16, in the order the output correction reads it as matrix-core
 *   operands, and e^{b_C} in fp32; b the cumulative log-gate within the chunk), then
 *   the call's own segment buffers (the chunks of each sequence are
 *   cut into segments run in parallel: their end states and decays, and start states).
 *   May be NULL when T = 0.
 * T must be a multiple of chunk (64).
 */
GDNRT_API int gla_chunk_fwd(const void* q, const void* k, const void* v, const float* log_g,
                  const float* S0, float* ST, void* o,
                  int N, int T, int dk, int dv, int chunk, int io,
                  void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes gla_chunk_fwd needs for this shape (0 if the shape is unsupported
 * or empty). */
GDNRT_API size_t gla_chunk_fwd_workspace_bytes(int N, int T, int dk, int dv, int chunk);

/*
 * Sequence parallelism for GLA, the per-device calls ("ZeCO: Zero Communication
 * Overhead Sequence Parallelism for Linear Attention", sections "Local State
 * Computation", "Global State Update Formula" (eq. 6), "All-Scan Collective
 * Communication" and "The Complete Forward Algorithm"). The sequence is cut into
 * contiguous shards of whole chunks, one per device. A device:
 *   1. runs gla_chunk_fwd on its shard from a zero state (S0 = NULL) with
 *      io = GDNRT_BF16 | GDNRT_GLA_SHARD: local outputs o, local final state S_[N] (its
 *      ST), and a workspace holding per chunk Q o e^b and the chunk decay gamma = e^{b_C};
 *   2. gla_shard_decay: the cumulative decays gamma~ from that workspace;
 *   3. gla_all_scan_step, block by block along d_k: receives block k of the state
 *      from the previous device and forms the block to send to the next one;
 *   4. gla_shard_output_correct: adds the received state's share to its outputs.
 * o and the last device's sent state then equal one gla_chunk_fwd over the whole
 * sequence. Moving the state blocks between devices is the caller's (one
 * point-to-point send/receive per block); nothing here communicates.
 *
 * Between steps 1 and 4 the workspace must hold what gla_chunk_fwd left in it
 * (same N, T; not reused meanwhile).
 */

/* gamma [N][T/chunk + 1][dk] fp32, 16-byte aligned: gamma[n][c][k] is the product of
 * the chunk decays e^{b_C}[k] of chunks 0..c-1 of sequence n (gamma~_[c] of the page;
 * gamma[n][0] = 1 and gamma[n][T/chunk] is the shard's total decay). workspace,
 * ws_bytes: as passed to gla_chunk_fwd for this shard (N, T). T = 0 writes the ones. */
GDNRT_API int gla_shard_decay(const void* workspace, size_t ws_bytes, float* gamma,
                    int N, int T, int dk, int chunk, void* stream);

/* All-Scan update of key channels [k0, k1) (0 <= k0 <= k1 <= dk):
 *     S_send[n][v][k] = gamma_n[k] S_recv[n][v][k] + S_local[n][v][k],
 * gamma_n = gamma + n * gamma_stride (floats, >= dk): the shard's total decay, e.g.
 * gla_shard_decay's output with offset (T/chunk) * dk and stride (T/chunk + 1) * dk.
 * S_recv NULL (the first device): S_send = S_local, and gamma may be NULL. States
 * [N][dv][dk] fp32, 4-byte aligned; S_send may equal S_local or S_recv, other overlaps
 * are rejected. Channels outside [k0, k1) of S_send are not touched. */
GDNRT_API int gla_all_scan_step(const float* S_recv, const float* gamma, size_t gamma_stride,
                      const float* S_local, float* S_send, int N, int dk, int dv, int k0, int k1,
                      void* stream);

/* Adds to the outputs o [N][T][dv] (bf16, those of gla_chunk_fwd from a zero state)
 * the share of the received state S_in [N][dv][dk] (fp32):
 *     o_t += S_in (q_t o e^{b_t} o gamma~_[c]),   token t in chunk c,
 * b the inclusive cumulative log-gate within the chunk; gamma from gla_shard_decay.
 * The scaled query is formed in bf16 (from the workspace's bf16 Q o e^b), the state
 * is rounded to bf16 for the matrix cores, accumulation is fp32 and o is rounded
 * once. S_in NULL (the first device, or a zero incoming state) does nothing.
 * workspace, gamma, S_in, o: 16-byte aligned; o must not overlap the others.
 * io must be GDNRT_BF16. */
GDNRT_API int gla_shard_output_correct(const void* workspace, size_t ws_bytes, const float* gamma,
                             const float* S_in, void* o, int N, int T, int dk, int dv, int chunk,
                             int io, void* stream);

/*
 * Gated linear attention, chunkwise backward of one sequence shard ("ZeCO: Zero
 * Communication Overhead Sequence Parallelism for Linear Attention", section "The
 * Backward Algorithm and Gradient Flow": the state gradient flows backward over the
 * chunks, dS <- gamma o dS + Q~^T dO, and each chunk combines its intra-chunk and
 * inter-chunk gradients). For the forward of gla_chunk_fwd from S0 and the scalar
 * L = sum(dO o o) + sum(dST o S_T), writes
 *   dq, dk [N][T][dk], dv [N][T][dv] (bf16), dlog_g [N][T][dk] (fp32) and dS0
 *   [N][dv][dk] (fp32, the gradient with respect to the incoming state).
 *   q, k, v, dO [N][T][d] bf16 and log_g fp32: 16-byte aligned. S0, dST may be NULL
 *   (zero). workspace: gla_chunk_bwd_workspace_bytes() bytes, 16-byte aligned,
 *   overwritten (per chunk the scaled operands, the state before the chunk and the
 *   state gradient after it, in bf16: 132,608 bytes). May be NULL when T = 0.
 * The gate gradient is the reverse cumulative sum of q o dq - k o dk (plus dST o S_T
 * summed over value channels at the last token). T must be a multiple of 64.
 */
GDNRT_API int gla_chunk_bwd(const void* q, const void* k, const void* v, const float* log_g,
                            const float* S0, const void* dO, const float* dST,
                            void* dq, void* dk, void* dv, float* dlog_g, float* dS0,
                            int N, int T, int dk_, int dv_, int chunk, int io,
                            void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes gla_chunk_bwd needs for this shape (0 if unsupported or empty). */
GDNRT_API size_t gla_chunk_bwd_workspace_bytes(int N, int T, int dk, int dv, int chunk);

/*
 * ZeCO's backward on one device of a sequence-parallel GLA run ("ZeCO: Zero
 * Communication Overhead Sequence Parallelism for Linear Attention", section "The
 * Backward Algorithm and Gradient Flow"), phase 1: the gradient with respect to the
 * state the shard starts from, counting only the shard's own outputs,
 *     dS <- gamma o dS + dO^T (Q o e^b)   over the chunks in reverse, from dS = 0,
 * written to dS0 [N][dv][dk] fp32. With it a device:
 *   1. gla_shard_bwd_state: its local dS_[0];
 *   2. gla_all_scan_step(S_recv = the state gradient received from the next device,
 *      gamma = the shard's total decay, S_local = dS_[0]): the state gradient to send
 *      to the previous device (the backward All-Scan, block by block along d_k);
 *   3. gla_chunk_bwd (or gla_shard_bwd_grads, which reuses step 1's workspace) from
 *      the shard's incoming state with dST = the received state gradient: every
 *      gradient of the shard (its dS0 equals what step 2 sent).
 * q, k, dO [N][T][128] bf16, log_g fp32, 16-byte aligned (k is read by the shared
 * per-chunk preparation). workspace: at least N * (T/chunk) * 132,608 bytes (e.g. the
 * gla_chunk_bwd workspace), 16-byte aligned, overwritten; may be NULL when T = 0.
 */
GDNRT_API int gla_shard_bwd_state(const void* q, const void* k, const float* log_g, const void* dO,
                        float* dS0, int N, int T, int dk, int dv, int chunk, int io,
                        void* workspace, size_t ws_bytes, void* stream);

/* Step 3 above without repeating the per-chunk preparation: gla_chunk_bwd (same
 * arguments and results) for a workspace of gla_chunk_bwd_workspace_bytes() bytes in
 * which gla_shard_bwd_state has just run on the same q, k, log_g, N, T (and that
 * nothing has used since). */
GDNRT_API int gla_shard_bwd_grads(const void* q, const void* k, const void* v, const float* log_g,
                        const float* S0, const void* dO, const float* dST, void* dq, void* dk,
                        void* dv, float* dlog_g, float* dS0, int N, int T, int dk_, int dv_,
                        int chunk, int io, void* workspace, size_t ws_bytes, void* stream);

/*
 * Gated DeltaNet chunkwise forward (prefill): the same recurrence as
 * gdn_decode_step over T tokens, computed per chunk of 64 tokens through the
 * UT / WY form of the intra-chunk delta rule (derived from eq. 3 of the LeapQuant
 * page's section "The state, from the update rule up" by unrolling within a
 * chunk; the pages print no chunk form for the delta rule):
 *   (I + L) U = diag(beta) V - diag(beta g) K S_0^T, L[r,j] = beta_r (g_r/g_j) k_r.k_j (j < r),
 *   O = diag(g) Q S_0^T + A U, A[r,j] = (g_r/g_j) q_r.k_j (j <= r),
 *   S_C = g_C S_0 + U^T diag(g_C/g) K,  g_r = prod_{i<=r} alpha_i within the chunk.
 *
 *   q, k [N][T][dk] bf16 (q, k as given).   v, o [N][T][dv] bf16.
 *   alpha (in (0,1)), beta [N][T] fp32.   S0 [N][dv][dk] fp32 or NULL (zero).
 *   ST [N][dv][dk] fp32 final state (may equal S0).
 *   workspace: caller-owned device memory of gdn_chunk_fwd_workspace_bytes() bytes,
 *   16-byte aligned, overwritten (the per-chunk state-independent operands in bf16:
 *   W, U~, Q' = diag(g) Q - A W, O~ = A U~ and diag(g_C/g) K, plus g_C; 81,984 bytes
 *   per chunk).
 * T must be a multiple of chunk (64).
 */
GDNRT_API int gdn_chunk_fwd(const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta,
                            const float* S0, float* ST, void* o,
                            int N, int T, int dk, int dv, int chunk, int io,
                            void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes gdn_chunk_fwd needs for this shape (0 if the shape is unsupported
 * or empty). */
GDNRT_API size_t gdn_chunk_fwd_workspace_bytes(int N, int T, int dk, int dv, int chunk);

/*
 * gdn_chunk_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments and
 * results as gdn_chunk_fwd without the workspace: the per-chunk operands go to a
 * scratch array of gdn_chunk_fwd_noalloc_max_bytes() bytes (128 MiB: 1,637 chunks of 64
 * tokens, e.g. 32 heads x 3,264 tokens) that the library holds on each GPU it runs on
 * until the process ends. Nothing is allocated or freed by the call. A shape whose
 * operands exceed the scratch (gdn_chunk_fwd_workspace_bytes > the maximum) returns
 * GDNRT_ESHAPE and launches nothing. Every call on one GPU shares that GPU's scratch,
 * so calls that overlap in time on one GPU (different streams, or threads) race: the
 * caller orders them. The scratch keeps the last call's contents; nothing in it needs
 * to start at zero.
 */
GDNRT_API int gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                    const float* alpha, const float* beta,
                                    const float* S0, float* ST, void* o,
                                    int N, int T, int dk, int dv, int chunk, int io, void* stream);

/* Bytes of the scratch array gdn_chunk_fwd_noalloc uses (its size limit). */
GDNRT_API size_t gdn_chunk_fwd_noalloc_max_bytes(void);

/*
 * Gated DeltaNet chunkwise backward of one sequence shard: for the forward of
 * gdn_chunk_fwd from S0 and the scalar L = sum(dO o o) + sum(dST o S_T), writes
 *   dq, dk [N][T][dk], dv [N][T][dv] (bf16), dalpha, dbeta [N][T] (fp32) and dS0
 *   [N][dv][dk] (fp32, the gradient with respect to the incoming state).
 * The pages print no backward for the delta rule; this one differentiates the
 * forward's chunk form (above): the state gradient runs backward over the chunks,
 *   dS_b = g_C dS_a + dO^T Q' - (diag(g_C/g) K dS_a^T)^T W,
 * each chunk's gradients go through U = U~ - W S_b^T, A and the WY factors
 * (T = (I + L)^-1, W, U~), and the decay gradient follows from the cumulative
 * log-decay B_t entering only as q_t e^{B_t} and v_t e^{-B_t} once the state is
 * divided by e^{B_t}: d log alpha_t = sum_{s >= t} (q_s.dq_s - v_s.dv_s), plus
 * sum(dST o S_T), and dalpha = d log alpha / alpha.
 *   q, k, v, dO [N][T][d] bf16, 16-byte aligned; alpha (in (0,1)), beta [N][T] fp32.
 *   S0, dST [N][dv][dk] fp32 or NULL (zero). Outputs must not overlap inputs.
 *   workspace: gdn_chunk_bwd_workspace_bytes() bytes, 16-byte aligned, overwritten
 *   (per chunk the forward's operands, (I + L)^-1, the state before the chunk and the
 *   state gradient after it, dU and a partial dk in bf16, q.dq and the chunk's
 *   sum(dS o S): 188,740 bytes). May be NULL when T = 0.
 * T must be a multiple of 64 (chunk).
 */
GDNRT_API int gdn_chunk_bwd(const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta, const float* S0,
                            const void* dO, const float* dST,
                            void* dq, void* dk, void* dv, float* dalpha, float* dbeta, float* dS0,
                            int N, int T, int dk_, int dv_, int chunk, int io,
                            void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes gdn_chunk_bwd needs for this shape (0 if unsupported or empty). */
GDNRT_API size_t gdn_chunk_bwd_workspace_bytes(int N, int T, int dk, int dv, int chunk);

/*
 * Kimi Delta Attention chunkwise forward (prefill): the recurrence of
 * kda_decode_step (one decay per key channel; LeapQuant page, section "The state,
 * from the update rule up", eq. 1 / eq. 3) over T tokens, per chunk of 64 tokens
 * through the UT form of gdn_chunk_fwd with the decay inside the key and query
 * products (derived by unrolling eq. 3 within a chunk; the pages print no chunk
 * form). With b_r the cumulative log-decay per key channel within the chunk and
 * Gamma_r = exp(b_r):
 *   (I + L) U = diag(beta) V - diag(beta) (K o Gamma) S_0^T,
 *       L[r,j] = beta_r sum_c k_r[c] k_j[c] exp(b_r[c] - b_j[c]) (j < r),
 *   O = (Q o Gamma) S_0^T + A U,  A[r,j] = sum_c q_r[c] k_j[c] exp(b_r[c] - b_j[c]) (j <= r),
 *   S_C = S_0 Diag(Gamma_C) + U^T (K o exp(b_C - b)).
 *
 *   q, k [N][T][dk] bf16, v, o [N][T][dv] bf16 (as gdn_chunk_fwd).
 *   alpha [N][T][dk] fp32 in (0, 1), 16-byte aligned; beta [N][T] fp32.
 *   S0, ST, workspace as gdn_chunk_fwd, workspace of kda_chunk_fwd_workspace_bytes()
 *   bytes (82,432 per chunk: the per-channel chunk decay Gamma_C takes 512 bytes).
 * The products are formed relative to the chunk's middle token, so exp(|b_r - b_m|)
 * must stay within fp32 range: the log-decays of any 32 consecutive tokens of a
 * channel must sum to more than -88 (e.g. every alpha above 0.064).
 * T must be a multiple of chunk (64).
 */
GDNRT_API int kda_chunk_fwd(const void* q, const void* k, const void* v,
                            const float* alpha, const float* beta,
                            const float* S0, float* ST, void* o,
                            int N, int T, int dk, int dv, int chunk, int io,
                            void* workspace, size_t ws_bytes, void* stream);

/* Workspace bytes kda_chunk_fwd needs for this shape (0 if unsupported or empty). */
GDNRT_API size_t kda_chunk_fwd_workspace_bytes(int N, int T, int dk, int dv, int chunk);

/*
 * Per-step low-precision state baselines ("LeapQuant: an 8-bit recurrent state that
 * stops rounding every token", section "Rounding every token", eq. 2): gdn_decode_step
 * with the state stored in a narrow format and re-rounded after every token. Each token
 * computes u, o and the next state in fp32 from the stored state, then rounds it:
 *
 *   gdn_decode_step_bf16_state: S [N][dv][dk] bf16 (16-byte aligned), rounded to
 *     nearest even per entry.
 *   gdn_decode_step_int_state: codes [N][dv][dk] int8 in [-Q, Q], Q = 2^(bits-1) - 1
 *     (bits in 2..8), and rowmax [N][dv] fp32, the value row's largest magnitude; the
 *     state is rowmax[v] * codes[v,k] / Q; after each token rowmax <- max_k |S[v,k]| and
 *     codes <- clamp(rint(S * (Q / rowmax)), -Q, Q) (fp32, nearest even). No smoothing
 *     and no compensator tokens.
 *
 * q, k [N][T][dk] (16-byte aligned), v, o [N][T][dv] in the io dtype; alpha, beta [N][T]
 * fp32. Outputs o_t = S_t q_t from the unrounded S_t. Errors as gdn_decode_step.
 */
GDNRT_API int gdn_decode_step_bf16_state(uint16_t* S, const void* q, const void* k, const void* v,
                                         const float* alpha, const float* beta, void* o,
                                         int N, int T, int dk, int dv, int io, void* stream);
GDNRT_API int gdn_decode_step_int_state(int8_t* codes, float* rowmax, int bits,
                                        const void* q, const void* k, const void* v,
                                        const float* alpha, const float* beta, void* o,
                                        int N, int T, int dk, int dv, int io, void* stream);

/*
 * LeapQuant windowed 8-bit state ("LeapQuant: an 8-bit recurrent state that stops
 * rounding every token": section "Fix one: leap over a window" eq. 4 and eq. 10,
 * section "Fix two: pull the outliers out as tokens" eq. 5, section "Fix three:
 * smooth what is left" eq. 7, layout from section "What 1.19 bytes buys").
 * A host struct of caller-owned device pointers, per head n of N:
 *
 *   codes   [N][dv][RB] bytes  residual codes Z in [-Q, Q], Q = 2^(bits-1) - 1 (127 at 8
 *                              bits), one value row of dk = 128 codes in RB bytes.
 *                              bits = 6 or 4 (the narrower widths of section "Fix two",
 *                              which pairs them with 6 compensator tokens) are packed:
 *                              RB = 16 * bits; at 4 bits byte j holds codes 2j (low
 *                              nibble) and 2j+1 (high nibble); at 6 bits every 3 bytes
 *                              hold 4 codes, code 4c+i in bits [6i, 6i+6) of the
 *                              little-endian 24-bit group c; codes are two's complement
 *                              in their width. Any other width takes one int8 per code
 *                              (RB = 128).
 *   vscale  [N][dv]     fp32   one scale per value channel (row): its largest
 *                              smoothed residual magnitude
 *   ksmooth [N][dk]     fp32   one smoothing factor per key channel (column)
 *   ct_k    [N][rank][dk] fp16 compensator-token keys (unit norm before rounding)
 *   ct_u    [N][rank][dv] fp16 compensator-token values
 *   buf_k   [N][window][dk] fp32, buf_u [N][window][dv] fp32, buf_a [N][window] fp32:
 *                              the open window's records (k_t, u_t, alpha_t)
 *
 * Alignment: codes, ksmooth, ct_k, ct_u, buf_k, buf_u 16 bytes; vscale, buf_a 4
 * bytes (GDNRT_EALIGN otherwise).
 *
 * The stored state is S_hat[v,k] = vscale[v] * codes[v,k] / Q * ksmooth[k]
 *                                   + sum_r ct_u[r][v] ct_k[r][k].
 * The compensator tokens enter the window ahead of the real tokens with decay 1,
 * so they decay together with the residual.
 */
typedef struct {
  int8_t* codes;
  float* vscale;
  float* ksmooth;
  uint16_t* ct_k;
  uint16_t* ct_u;
  float* buf_k;
  float* buf_u;
  float* buf_a;
  int N, dk, dv, rank, window;
  int bits;   /* code width: codes on [-Q, Q], Q = 2^(bits-1) - 1; 2..8, or 0 for 8 */
} leapq_state;

/*
 * One decode token per head inside a window. `pos` real tokens (0 <= pos < window)
 * are already buffered. Reads the stored state and the buffer, and with
 * x -> S_pos x evaluated by eq. 10,
 *
 *     u_t = beta_t (v_t - alpha_t S_pos k_t),   o_t = alpha_t S_pos q_t + u_t (k_t . q_t),
 *
 * then appends (k_t, u_t, alpha_t) at buffer slot pos. Writes no state.
 *   q, k [N][dk], v, o [N][dv] io dtype; alpha, beta [N] fp32. q and k are read 16
 *   bytes at a time and must be 16-byte aligned; v, o, alpha, beta 4-byte aligned.
 * pos outside [0, window) returns GDNRT_ESTATE.
 */
GDNRT_API int leapq_decode_step(const leapq_state* st, int pos,
                      const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta, void* o,
                      int io, void* stream);

/*
 * Window flush: rebuild the dense state S_pos (eq. 4) from the stored state and
 * the first `pos` buffered records -- or take `dense` ([N][dv][dk] fp32) instead
 * when it is not NULL, to encode an initial state -- then
 *   1. fit `rank` compensator tokens: `iters` rounds of Q <- orth(S^T (S Q)) from
 *      the start block q0 ([dk][rank] fp32, device), each orthonormalised by two
 *      CholeskyQR passes whose Gram matrix is shifted by 1e-6 * trace + 1e-30;
 *      ct_k = fp16(Q^T), ct_u = fp16((S Q)^T) (round to nearest even);
 *   2. R = S - sum_r ct_u[r] ct_k[r]^T (the rounded pieces);
 *   3. smoothing per key channel k: smooth_mode 0: sqrt(mean_v |R[v,k]|),
 *      1: sqrt(mean_v R[v,k]^2), 2: none (1); clamped below at 1e-12;
 *   4. vscale[v] = max_k |R[v,k] / ksmooth[k]|;
 *   5. x = (R[v,k] / ksmooth[k]) * (Q / vscale[v]) in fp32 (0 when vscale is 0),
 *      codes = clamp(rint(x), -Q, Q), round half to even (Q = 127 at 8 bits).
 * The stored state is overwritten; the buffer is then empty (next pos = 0).
 * pre_round, when not NULL ([N][dv][dk] fp32), receives x.
 * pos outside [0, window] returns GDNRT_ESTATE.
 */
GDNRT_API int leapq_window_flush(const leapq_state* st, int pos, const float* dense,
                       const float* q0, int iters, int smooth_mode,
                       float* pre_round, void* stream);

/*
 * Kimi Delta Attention (one decay per key channel) in the windowed 8-bit state:
 * "LeapQuant: an 8-bit recurrent state that stops rounding every token", section
 * "The state, from the update rule up" for the update, section "Fix one: leap over a
 * window" (eq. 4 and eq. 10 with diagonal decays, which accumulate per channel) and
 * section "What 1.19 bytes buys" for the buffered per-channel decays. Same stored
 * state and buffer as leapq_decode_step except buf_a: [N][window][dk] fp32, 16-byte
 * aligned, one decay vector per buffered token. With Gamma_{a:b} = Diag(alpha_a ...
 * alpha_b) and S_pos y = S_hat_0 (Gamma_{1:pos} y) + sum_j u_j (k_j . Gamma_{j+1:pos} y)
 * (the compensator tokens decay with the residual by Gamma_{1:pos}),
 *
 *     u_t = beta_t (v_t - S_pos (alpha_t o k_t)),   o_t = S_pos (alpha_t o q_t) + u_t (k_t . q_t),
 *
 * then appends (k_t, u_t, alpha_t) at slot pos. alpha [N][dk] fp32 (16-byte aligned).
 * Errors as leapq_decode_step.
 */
GDNRT_API int kda_leapq_decode_step(const leapq_state* st, int pos,
                      const void* q, const void* k, const void* v,
                      const float* alpha, const float* beta, void* o,
                      int io, void* stream);

/*
 * Window flush of the KDA windowed state: as leapq_window_flush, with the rebuild
 * S_pos = S_hat_0 Gamma_{1:pos} + sum_j u_j k_j^T Gamma_{j+1:pos} (eq. 4 with diagonal
 * decays) from buf_a [N][window][dk]. The fit, subtraction, smoothing and rounding are
 * those of leapq_window_flush; with `dense` the two are the same operation.
 */
GDNRT_API int kda_leapq_window_flush(const leapq_state* st, int pos, const float* dense,
                       const float* q0, int iters, int smooth_mode,
                       float* pre_round, void* stream);

/*
 * The last token of a window and the flush that closes it, in one launch: the same
 * results as leapq_decode_step at pos = window - 1 followed by leapq_window_flush at
 * pos = window with dense = pre_round = NULL, up to fp32 rounding order ("LeapQuant",
 * section "Fix one: leap over a window": the token after window - 1 buffered ones
 * ends the window, eq. 4 rebuilds S_{window-1}, the token's update is applied to it
 * in fp32, and steps 1-5 of leapq_window_flush encode the result). The token's
 * record is not appended: the flush consumes it. window - 1 records must be
 * buffered. q, k, v, o [N][dk|dv] io dtype, alpha [N] fp32 (kda_: [N][dk]), beta [N]
 * fp32, all 4-byte aligned; q0, iters, smooth_mode as in leapq_window_flush. o must
 * not overlap an input or the state. Errors as the two calls it replaces.
 */
GDNRT_API int leapq_decode_flush(const leapq_state* st, const void* q, const void* k,
                      const void* v, const float* alpha, const float* beta, void* o,
                      int io, const float* q0, int iters, int smooth_mode, void* stream);

/* KDA form of leapq_decode_flush (the kda_leapq_decode_step token, then kda_leapq_window_flush). */
GDNRT_API int kda_leapq_decode_flush(const leapq_state* st, const void* q, const void* k,
                      const void* v, const float* alpha, const float* beta, void* o,
                      int io, const float* q0, int iters, int smooth_mode, void* stream);

/*
 * Measurement aid, not a step of the method: one streaming read and write of n fp32
 * values, dst[i] = scale * src[i] (dst may equal src: an in-place pass, as the decode
 * updates its state), with 16-byte non-temporal loads and stores, vec (1, 2 or 4)
 * pieces per thread and 256-thread blocks. Its rate is the HBM ceiling measured on the
 * device, reported beside the published peak. dst, src 16-byte aligned; n a multiple
 * of 4; partial overlap returns GDNRT_EINVAL.
 */
GDNRT_API int gdnrt_hbm_stream(float* dst, const float* src, size_t n, int vec, float scale,
                               void* stream);

/* Message for the calling thread's last non-OK status ("" if none). */
GDNRT_API const char* gdnrt_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDNRT_H */
