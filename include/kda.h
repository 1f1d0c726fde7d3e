/*
 * kda.h -- C ABI of libkda: the chunkwise forward pass of gated delta-rule
 * linear attention on AMD Instinct MI355X (gfx950).
 *
 * Two operations:
 *   kda_fwd  Kimi Delta Attention: per-channel decay computed from a
 *            pre-activation gate, beta given as logits.
 *   gdn_fwd  Gated DeltaNet: one scalar log decay per (token, head), beta
 *            given as probabilities.
 *
 * Both compute, for every sequence and head, with the state S in [K, V] layout:
 *   q^_t = q_t / sqrt(|q_t|^2 + 1e-6),  k^_t likewise
 *   S_t  = (I - beta_t k^_t k^_t^T) Diag(alpha_t) S_{t-1} + beta_t k^_t v_t^T
 *   o_t  = scale * S_t^T q^_t
 * KDA: log alpha_t[c] = max(lower_bound, -exp(A_log[h]) * softplus(g_t[c] + dt_bias[h, c]))
 *      beta_t = sigmoid(beta_t logit)
 * GDN: log alpha_t[c] = g_t (the same for every channel), beta_t as given.
 *
 * Sources: the KDA parameter table of the FlashKDA summary on
 * discuss.pytorch.kr (section "FlashKDA의 KDA 연산 구조": q, k, v, g, beta
 * logits with the sigmoid inside, A_log, dt_bias [H, K], lower_bound in
 * [-5, 0], optional initial/final state, fused q/k L2 norm and gate); the
 * cuLA README's KDA example (section "KDA (Kimi Delta Attention) --
 * Blackwell (SM10X)": fp32 [B, H, K, V] states, int32 cu_seqlens); the
 * QwenLM/FlashQLA summary (section "간단한 사용 예시": the GDN call with g,
 * beta, scale, initial_state and cu_seqlens).  The pages name the operations
 * but print no equation; the formulas above are the reading this library
 * implements.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers to contiguous row-major arrays.
 *    bf16 tensors are passed as uint16_t bit patterns.
 *  - Shapes: q, k [B, T, H, K]; v, o [B, T, H, V]; KDA g [B, T, H, K] bf16;
 *    GDN g [B, T, H] fp32; beta [B, T, H] bf16; A_log [H] fp32; dt_bias
 *    [H, K] fp32 (the same memory as a flat [H * K]); states [N, H, K, V]
 *    fp32, where N = B for fixed-length batches and N = num_seqs when
 *    cu_seqlens is given.
 *  - Variable length: cu_seqlens (device, int32, num_seqs + 1 entries) packs
 *    the sequences along T of a B = 1 batch: sequence i is tokens
 *    [cu_seqlens[i], cu_seqlens[i+1]).  Expected: cu_seqlens[0] = 0,
 *    non-decreasing, cu_seqlens[num_seqs] = T.  This is not checked (the
 *    library never reads device memory on the host); the kernels clamp the
 *    offsets into a non-decreasing sequence within [0, T], so a malformed
 *    array gives unspecified results but no out-of-bounds access.  The
 *    state restarts at every sequence boundary.
 *  - initial_state may be NULL (zero state); final_state may be NULL (not
 *    written).  An empty sequence returns its initial state.
 *  - Only K, V in {64, 128} are supported.  B * T must be < 2^31.  Token
 *    tensors (q, k, v, g, beta, o) may be NULL only when T == 0.
 *  - Alignment: q, k, v, g (KDA), dt_bias 16 bytes; o 16 bytes for
 *    kda_fwd / gdn_fwd, 8 bytes elsewhere; workspace 256 bytes.
 *  - Ownership: the caller allocates and frees every buffer, including the
 *    workspace (at least *_workspace_size() bytes).  The library allocates
 *    nothing, keeps no pointer after it returns and never synchronises.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *    stream); results are valid once the stream reaches that point.  Outputs
 *    must not alias inputs; concurrent calls must use distinct workspaces.
 *  - Errors: every argument check runs on the host before any HIP call and a
 *    failed check returns a KDA_ERR_* code with nothing enqueued.  A failed
 *    launch returns KDA_ERR_LAUNCH.  No C++ exception crosses this ABI.
 */
#ifndef LIBKDA_KDA_H
#define LIBKDA_KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* null pointer, bad size, lower_bound, alignment */
    KDA_ERR_UNSUPPORTED = 2, /* K or V outside {64, 128} */
    KDA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    KDA_ERR_LAUNCH = 4       /* a kernel launch failed */
};

/* Bytes of device workspace that kda_fwd needs: the packed-sequence and
 * segment tables when cu_seqlens is given (one alignment unit otherwise; a
 * fixed-length call reads no workspace and accepts NULL).  num_seqs: the
 * number of packed sequences when cu_seqlens will be passed, else B.  Pure
 * host function; returns 0 for invalid sizes. */
size_t kda_fwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                              int32_t num_seqs);

/* KDA forward.  beta holds logits (sigmoid applied inside); lower_bound must
 * be finite and in [-5, 0]; scale must be finite (K^-0.5 is customary).
 * num_seqs is read only when cu_seqlens is non-NULL (then B must be 1).
 *
 * One launch computes the whole pass: a workgroup per (sequence segment,
 * head) forms each 32-token chunk's decayed operands, intra-chunk matrices
 * and (I + A)^-1 in LDS and runs the recurrence over them, so HBM sees the
 * inputs and states read once and the outputs written once.  The FlashKDA
 * summary (discuss.pytorch.kr, section "커널 퓨전(Kernel Fusion) 전략의 분리")
 * describes the same two computations as a token-parallel and a sequential
 * kernel; here they are wave roles of one workgroup.  When the (sequence,
 * head) pairs are fewer than the compute units, sequences are cut into
 * segments that run in parallel; a segment that starts mid-sequence begins
 * one chunk early from a zero state and keeps that start only if that
 * chunk's transitions provably scale the true entering state by less than
 * 2^-24, the fp32 rounding of the state (for one token
 * ||(I - b k^ k^T) Diag(a)||_2 <= max_c a_c); else it tries four chunks
 * early, and else it restarts from the sequence start: the result is the
 * unsplit one up to rounding and that bound.  The FlashQLA summary (section "핵심 기능")
 * describes intra-card parallelism switched on when the gate's decay allows
 * it.  o must be 16-byte aligned. */
int kda_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
            const uint16_t* beta, const float* A_log, const float* dt_bias, float lower_bound,
            float scale, const float* initial_state, float* final_state,
            const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
            int32_t K, int32_t V, uint16_t* o, void* workspace, size_t workspace_bytes,
            void* stream);

/* Bytes of device workspace that gdn_fwd needs (same arguments). */
size_t gdn_fwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                              int32_t num_seqs);

/* GDN forward.  g is the fp32 log decay [B, T, H] and must be <= 0 (any
 * magnitude: the scalar gate forms its in-chunk decays as exp(G_r - G_j) <= 1);
 * beta holds probabilities in [0, 1], used as given. */
int gdn_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
            const uint16_t* beta, float scale, const float* initial_state, float* final_state,
            const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
            int32_t K, int32_t V, uint16_t* o, void* workspace, size_t workspace_bytes,
            void* stream);

/* kda_fwd / gdn_fwd with explicit segments: segment_chunks > 0 cuts every
 * sequence into segments of that many 32-token chunks, < 0 keeps whole
 * sequences, 0 is kda_fwd's automatic choice.  The workspace must hold
 * kda_fwd_segmented_workspace_size(..., segment_chunks) bytes; everything
 * else is as for kda_fwd / gdn_fwd. */
size_t kda_fwd_segmented_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                        int32_t num_seqs, int32_t segment_chunks);

int kda_fwd_segmented(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const uint16_t* g, const uint16_t* beta, const float* A_log,
                      const float* dt_bias, float lower_bound, float scale,
                      const float* initial_state, float* final_state, const int32_t* cu_seqlens,
                      int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                      uint16_t* o, void* workspace, size_t workspace_bytes,
                      int32_t segment_chunks, void* stream);

int gdn_fwd_segmented(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                      const uint16_t* beta, float scale, const float* initial_state,
                      float* final_state, const int32_t* cu_seqlens, int32_t num_seqs,
                      int32_t B, int32_t T, int32_t H, int32_t K, int32_t V, uint16_t* o,
                      void* workspace, size_t workspace_bytes, int32_t segment_chunks,
                      void* stream);

/* Measurement forms of kda_fwd / gdn_fwd: the same call, plus two events
 * (hipEvent_t handles created with timing enabled) into which the forward
 * kernel's own start and end are recorded on the GPU (it is launched with
 * hipExtLaunchKernel), so hipEventElapsedTime gives its execution time
 * without the dispatch gap of events recorded between kernels.  Both NULL:
 * the plain call; exactly one NULL: KDA_ERR_INVALID_ARG. */
int kda_fwd_timed(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
                  const uint16_t* beta, const float* A_log, const float* dt_bias,
                  float lower_bound, float scale, const float* initial_state,
                  float* final_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                  int32_t T, int32_t H, int32_t K, int32_t V, uint16_t* o, void* workspace,
                  size_t workspace_bytes, void* stream, void* start_event, void* stop_event);

/* kda_fwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same pass and results as kda_fwd, with no workspace argument.  A packed
 * batch keeps its sequence and segment tables (what kda_fwd puts in the
 * workspace) in a device array of the library, KDA_NOALLOC_SCRATCH_BYTES per
 * GPU, held until the process ends; a fixed-length batch needs none.  The
 * call allocates nothing; the caller passes every input and output.
 * Errors: those of kda_fwd, and KDA_ERR_WORKSPACE (before any HIP call) for
 * a packed batch whose tables need more than the array: about 28 bytes per
 * sequence (the size kda_fwd_workspace_size gives), so up to about 149,000
 * packed sequences of any lengths.
 * The array is shared by every call on a GPU: calls that overlap in time on
 * one GPU (other streams, other host threads) race on it and must be
 * serialised by the caller; calls in stream order are safe. */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
int kda_fwd_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
                    const uint16_t* beta, const float* A_log, const float* dt_bias,
                    float lower_bound, float scale, const float* initial_state,
                    float* final_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                    int32_t T, int32_t H, int32_t K, int32_t V, uint16_t* o, void* stream);

int gdn_fwd_timed(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                  const uint16_t* beta, float scale, const float* initial_state,
                  float* final_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                  int32_t T, int32_t H, int32_t K, int32_t V, uint16_t* o, void* workspace,
                  size_t workspace_bytes, void* stream, void* start_event, void* stop_event);

/* The two-stage form of kda_fwd / gdn_fwd (kda_prep then kda_recur, with the
 * chunk records in the workspace), with explicit control of its sequence
 * splitting.
 *
 * A sequence is one chain of dependent chunk steps, so a batch of few long
 * sequences leaves most of the GPU idle.  Splitting cuts every sequence into
 * segments of segment_chunks chunks that run in parallel: a first pass runs
 * each segment from a zero state (and, when its bound says the entering
 * state is not forgotten, its K x K transition from an identity start), a
 * scan over the segments gives each segment its true entering state, and a
 * second pass recomputes the segments with outputs.  The result equals the
 * unsplit pass up to rounding.  This is context parallelism inside one
 * card: the cuLA README (section "Benchmarks") reports it for FlashKDA on
 * long sequences, the FlashQLA summary (section "핵심 기능") switches it on
 * from the gate's decay.
 *
 * segment_chunks: < 0 never split; 0 automatic (only when the sequences are
 * long and the (sequence, head, 32-column) workgroups too few to fill the
 * GPU); > 0 segments of that many 32-token chunks.  The workspace must hold
 * kda_fwd_split_workspace_size(..., segment_chunks) bytes (with -1, also the
 * workspace of kda_prep / kda_recur); the other arguments, layouts and
 * errors are those of kda_fwd / gdn_fwd (o 8-byte aligned). */
size_t kda_fwd_split_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                                    int32_t num_seqs, int32_t segment_chunks);

int kda_fwd_split(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
                  const uint16_t* beta, const float* A_log, const float* dt_bias,
                  float lower_bound, float scale, const float* initial_state,
                  float* final_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                  int32_t T, int32_t H, int32_t K, int32_t V, uint16_t* o, void* workspace,
                  size_t workspace_bytes, int32_t segment_chunks, void* stream);

int gdn_fwd_split(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                  const uint16_t* beta, float scale, const float* initial_state,
                  float* final_state, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                  int32_t T, int32_t H, int32_t K, int32_t V, uint16_t* o, void* workspace,
                  size_t workspace_bytes, int32_t segment_chunks, void* stream);

/* The two stages of the two-stage form, callable on their own (same
 * conventions; kda_fwd_split with segment_chunks = -1 is exactly kda_prep
 * followed by kda_recur).  Workspace: kda_fwd_split_workspace_size(...,
 * -1) bytes.
 *
 * kda_prep / gdn_prep: the token-parallel stage.  Gate activation, sigmoid
 * of beta (KDA), in-chunk cumulative decay, q/k L2 norm, the intra-chunk
 * matrices and the exact inverse of (I + A); writes the sequence table and
 * one record per (32-token chunk, head) into the workspace.  The FlashKDA
 * summary (discuss.pytorch.kr, section "커널 퓨전(Kernel Fusion) 전략의 분리")
 * puts exactly these operations in its first, token-parallel kernel.
 *
 * kda_recur: the head-parallel stage.  The sequential inter-chunk state
 * update and the output, reading the workspace that the preceding prep call
 * filled on the same stream with the same B, T, H, K, V and sequence
 * packing (varlen != 0 when that call received cu_seqlens, with the same
 * num_seqs).  The same page assigns the chunked delta recurrence and the
 * output projection to its second, head-parallel kernel.  It serves both
 * KDA and GDN workspaces. */
int kda_prep(const uint16_t* q, const uint16_t* k, const uint16_t* g, const uint16_t* beta,
             const float* A_log, const float* dt_bias, float lower_bound,
             const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
             int32_t K, int32_t V, void* workspace, size_t workspace_bytes, void* stream);

int gdn_prep(const uint16_t* q, const uint16_t* k, const float* g, const uint16_t* beta,
             const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
             int32_t K, int32_t V, void* workspace, size_t workspace_bytes, void* stream);

int kda_recur(const uint16_t* v, float scale, const float* initial_state, float* final_state,
              int32_t varlen, int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K,
              int32_t V, uint16_t* o, void* workspace, size_t workspace_bytes, void* stream);

/* Measurement forms of the two stages: exactly kda_prep and kda_recur (same
 * arguments, same work, same results), plus two events.  start_event and
 * stop_event are hipEvent_t handles the caller created with timing enabled
 * (for instance those of torch.cuda.Event(enable_timing=True) after a first
 * record()); the stage's main kernel (the record kernel; the recurrence
 * kernel) is launched with hipExtLaunchKernel, which records that kernel's
 * own start and end on the GPU into them, so hipEventElapsedTime gives its
 * execution time without the dispatch gap that events recorded between
 * kernels include.  With no token (no kernel) both events are recorded at
 * that point of the stream.  Both NULL: the plain stage.  Exactly one NULL:
 * KDA_ERR_INVALID_ARG.  The events are only written, never owned or freed. */
int kda_prep_timed(const uint16_t* q, const uint16_t* k, const uint16_t* g,
                   const uint16_t* beta, const float* A_log, const float* dt_bias,
                   float lower_bound, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                   int32_t T, int32_t H, int32_t K, int32_t V, void* workspace,
                   size_t workspace_bytes, void* stream, void* start_event, void* stop_event);

int kda_recur_timed(const uint16_t* v, float scale, const float* initial_state,
                    float* final_state, int32_t varlen, int32_t num_seqs, int32_t B, int32_t T,
                    int32_t H, int32_t K, int32_t V, uint16_t* o, void* workspace,
                    size_t workspace_bytes, void* stream, void* start_event, void* stop_event);

/* One recurrent step per sequence: the single-token form of the same
 * recurrence, for decoding after a prefill (the cuLA pages list decode
 * kernels on their inference roadmap: cuLA blog, section "Status &
 * Roadmap"; the gate, beta and norm are those of FlashKDA's parameter table,
 * discuss.pytorch.kr, section "FlashKDA의 KDA 연산 구조").  For each of the
 * N sequences and H heads, with S the [K, V] state:
 *   S' = (I - beta k^ k^T) Diag(alpha) S + beta k^ v^T,   o = scale S'^T q^
 * where alpha, beta and the normalised q^, k^ are formed exactly as in
 * kda_fwd / gdn_fwd for one token.  Running it T times from a state gives the
 * same states and outputs (up to rounding) as the forward pass over those T
 * tokens.
 *
 * Layouts (device pointers, contiguous): q, k [N, H, K] bf16; v, o [N, H, V]
 * bf16; KDA g [N, H, K] bf16 and GDN g [N, H] fp32 (log decay <= 0); beta
 * [N, H] bf16 (KDA logits, GDN probabilities); A_log [H], dt_bias [H, K]
 * fp32; state_in, state_out [N, H, K, V] fp32.  state_in may be NULL (zero
 * state) and may equal state_out (update in place); state_out is required.
 * No workspace.  Alignment: q, k, state_in, state_out 16 bytes; v, o 8 bytes.
 * Errors as for the forward pass (lower_bound in [-5, 0], finite scale,
 * K and V in {64, 128}); nothing is enqueued when a check fails. */
int kda_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
               const uint16_t* beta, const float* A_log, const float* dt_bias, float lower_bound,
               float scale, const float* state_in, float* state_out, int32_t N, int32_t H,
               int32_t K, int32_t V, uint16_t* o, void* stream);

int gdn_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
               const uint16_t* beta, float scale, const float* state_in, float* state_out,
               int32_t N, int32_t H, int32_t K, int32_t V, uint16_t* o, void* stream);

/* Backward pass: the gradients of a scalar loss L with respect to every input
 * of kda_fwd / gdn_fwd, given dL/do and, optionally, dL/d(final state).  The
 * pages show the backward only as autograd over the forward call (cuLA
 * README mirror, section "Usage": q, k, v with requires_grad and
 * o.backward(do)); the cuLA roadmap lists backward kernels for training and
 * the FlashQLA summary (section "핵심 기능") a backward path beside the forward
 * one.  The result is the exact derivative of the forward recurrence above,
 * computed chunkwise (recomputing the forward states; no state of a forward
 * call is needed).  The floor max(lower_bound, x) passes the gradient where
 * x >= lower_bound and blocks it where the floor is active.
 *
 * Inputs: the forward inputs (same layouts and conventions as kda_fwd /
 * gdn_fwd), d_o [B, T, H, V] bf16 (dL/do), d_final [N, H, K, V] fp32 or NULL
 * (dL/d final state; NULL = zero).
 * Outputs (caller-allocated, every element written):
 *   dq, dk [B, T, H, K] bf16;  dv [B, T, H, V] bf16;
 *   KDA: dg [B, T, H, K] bf16 (w.r.t. the pre-activation gate), dbeta
 *        [B, T, H] bf16 (w.r.t. the logits), dA_log [H] fp32, ddt_bias [H, K]
 *        fp32 (sums over all tokens, in a fixed order: reproducible);
 *   GDN: dg [B, T, H] fp32 (w.r.t. the log decay), dbeta [B, T, H] bf16
 *        (w.r.t. the probabilities);
 *   dh0 [N, H, K, V] fp32 or NULL (dL/d initial state; not written if NULL).
 * Workspace: at least *_bwd_workspace_size() bytes, 256-byte aligned (it holds
 * bf16 copies of the state entering every chunk and of its gradient, about
 * 4 (K + C) V bytes per chunk and head, C = 32).  Alignment: d_o, dq, dk, dv,
 * dg (KDA), d_final, dh0 16 bytes.  Errors and stream semantics as for the
 * forward pass.  There is no sequence splitting in the backward pass. */
size_t kda_bwd_workspace_size(int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
                              int32_t num_seqs);

int kda_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
            const uint16_t* beta, const float* A_log, const float* dt_bias, float lower_bound,
            float scale, const float* initial_state, const int32_t* cu_seqlens,
            int32_t num_seqs, int32_t B, int32_t T, int32_t H, int32_t K, int32_t V,
            const uint16_t* d_o, const float* d_final, uint16_t* dq, uint16_t* dk, uint16_t* dv,
            uint16_t* dg, uint16_t* dbeta, float* dA_log, float* ddt_bias, float* dh0,
            void* workspace, size_t workspace_bytes, void* stream);

int gdn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
            const uint16_t* beta, float scale, const float* initial_state,
            const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
            int32_t K, int32_t V, const uint16_t* d_o, const float* d_final, uint16_t* dq,
            uint16_t* dk, uint16_t* dv, float* dg, uint16_t* dbeta, float* dh0, void* workspace,
            size_t workspace_bytes, void* stream);

/* Training pair: a forward pass that keeps what its backward pass would
 * recompute, and that backward pass.  Same computation as the two-stage
 * forward pass (kda_fwd_split / gdn_fwd_split with no splitting) and
 * kda_bwd / gdn_bwd (results bit for bit equal to theirs); the single-launch
 * kda_fwd / gdn_fwd forms the same function in another rounding order.  The
 * pages' training use (cuLA README mirror, section "Usage": o.backward(do)
 * after the forward call) runs the two back to back on the same inputs.
 *
 * *_fwd_save: arguments and outputs as kda_fwd / gdn_fwd (no sequence
 * splitting), but the workspace must hold *_bwd_workspace_size() bytes: it is
 * left holding the chunk records, the reverse-pass records and the bf16 state
 * entering every chunk with V - KG S.
 * *_bwd_saved: arguments and outputs as kda_bwd / gdn_bwd; the workspace must
 * be the one a *_fwd_save call on the same inputs, sizes and cu_seqlens filled,
 * unchanged since, on the same stream (or synchronised with it).  It then runs
 * only the reverse sweep, the chunk gradients and the gate-parameter sums.
 * With any other workspace contents the gradients are meaningless, but every
 * access stays in bounds: the sequence table that indexes the workspace is
 * rebuilt from cu_seqlens. */
int kda_fwd_save(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
                 const uint16_t* beta, const float* A_log, const float* dt_bias,
                 float lower_bound, float scale, const float* initial_state, float* final_state,
                 const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                 int32_t K, int32_t V, uint16_t* o, void* workspace, size_t workspace_bytes,
                 void* stream);

int gdn_fwd_save(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                 const uint16_t* beta, float scale, const float* initial_state, float* final_state,
                 const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                 int32_t K, int32_t V, uint16_t* o, void* workspace, size_t workspace_bytes,
                 void* stream);

int kda_bwd_saved(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* g,
                  const uint16_t* beta, const float* A_log, const float* dt_bias,
                  float lower_bound, float scale, const float* initial_state,
                  const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                  int32_t K, int32_t V, const uint16_t* d_o, const float* d_final, uint16_t* dq,
                  uint16_t* dk, uint16_t* dv, uint16_t* dg, uint16_t* dbeta, float* dA_log,
                  float* ddt_bias, float* dh0, void* workspace, size_t workspace_bytes,
                  void* stream);

int gdn_bwd_saved(const uint16_t* q, const uint16_t* k, const uint16_t* v, const float* g,
                  const uint16_t* beta, float scale, const float* initial_state,
                  const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                  int32_t K, int32_t V, const uint16_t* d_o, const float* d_final, uint16_t* dq,
                  uint16_t* dk, uint16_t* dv, float* dg, uint16_t* dbeta, float* dh0,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code (never NULL). */
const char* kda_status_str(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBKDA_KDA_H */
