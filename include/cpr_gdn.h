/*
 * cpr_gdn.h -- C ABI of libcpr_gdn: chunkwise-parallel recurrent (CPR) evaluation of the
 * Gated DeltaNet gated delta rule on AMD Instinct MI355X (gfx950).
 *
 * Source of the method: the IsoExec articles (alphasignal.ai, "NovaSky's IsoExec Fixes the Hidden
 * Math Bug Corrupting AI Training Runs"), section "Solving the linear-attention headache": CPR
 * makes the per-token recurrence the reference computation; one pass finds the state at the
 * start of every chunk, a second pass (parallel over chunks) computes each chunk's outputs from
 * that state, and decode advances one token at a time, re-basing its state at every chunk start
 * so that its rounding agrees with prefill and training.  Section "The execution contract" fixes what an
 * implementation must pin (accumulation and boundary dtypes, reduction decomposition) and the use
 * of SHA-256 digests to refuse mismatched numerical policies.  Section "Making kernels
 * parallelism-invariant" requires identical bits however the work is split.
 *
 * The recurrence, per (sequence, value head h), key head g = h / (H_v / H_k), fp32 state S
 * (d_k x d_v):
 *     u_t = S_{t-1}^T k_t,   S_t = a_t S_{t-1} + b_t k_t (v_t - a_t u_t)^T,   o_t = S_t^T q_t.
 *
 * Every entry point evaluates each token with the same pinned fp32 arithmetic schedule
 * (schedule 1, described at gdn_policy.schedule), so prefill, trainer forward and decode give
 * bitwise-identical o and S for any batch composition, packing, chunk size or launch shape.
 *
 * Conventions shared by every call
 *   Return value   GDN_OK (0) or one of the GDN_E* codes; gdn_last_error() gives a message
 *                  (per host thread).  No C++ exception crosses this interface.
 *   Memory         all tensor pointers are DEVICE pointers owned by the caller and must stay
 *                  valid until the stream work completes.  Except in gdn_state_alloc's
 *                  self-allocating mode, the library allocates no device memory and never frees
 *                  caller memory; calls never synchronise the host.
 *   Streams        `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is
 *                  asynchronous; device-side faults surface at the caller's next synchronisation.
 *   Layouts        contiguous, row-major:
 *                    q, k  [N][H_k][d_k]     v, o  [N][H_v][d_v]     a, b  [N][H_v] (fp32)
 *                    state [num_slots][H_v][d_v][d_k] fp32  (S transposed: each d_v column of S
 *                          is d_k contiguous floats)
 *                    pos   [num_slots] int64  (tokens absorbed by each slot so far)
 *                  N is the total number of tokens of the call; sequences are packed back to
 *                  back as described by cu_seqlens (int32, [num_seqs + 1], cu[0] = 0,
 *                  non-decreasing, cu[num_seqs] = N).
 *   Dtypes         q, k, v and o share the policy's io dtype (fp32 or bf16); a, b, the state and
 *                  chunk states are always fp32.  bf16 outputs are rounded to nearest even.
 *   Chunks         chunk c of a sequence covers absolute positions [cC, (c+1)C), positions being
 *                  counted from the sequence's first token across prefill and decode calls.
 *   Device-side    kernels never read or write outside the sizes given; a sequence whose
 *   robustness     cu_seqlens entries are out of order or out of range, or whose slot id is out
 *                  of range, is skipped (its outputs are left unwritten).  Use
 *                  gdn_check_cu_seqlens on a host copy to reject such input up front.
 */
#ifndef CPR_GDN_H
#define CPR_GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes -------------------------------------------------------------------------- */
#define GDN_OK 0
#define GDN_EINVAL 1       /* malformed argument (null pointer, bad size, inconsistent shapes) */
#define GDN_EUNSUPPORTED 2 /* valid but not built: head dims, dtypes or schedule not compiled in */
#define GDN_EHIP 3         /* a HIP runtime call or kernel launch failed */
#define GDN_EPOLICY 4      /* numerical-policy digests differ (see gdn_policy_check) */

/* ---- dtypes -------------------------------------------------------------------------------- */
#define GDN_F32 0
#define GDN_BF16 1

/* The numerical policy of a state pool ("The execution contract": the constants an
 * implementation pins).  h_k, h_v: key and value heads (h_v a multiple of h_k; value head h reads
 * key head h / (h_v / h_k)).  dk, dv: head dims; builds support dk = dv in {16, 32, 64, 128}.
 * chunk: boundary spacing C >= 1.  io_dtype: GDN_F32 or GDN_BF16.
 * state_dtype: the boundary dtype.  The state is always stored and updated in fp32; at every
 * chunk start (just before the token at a position that is a multiple of C is applied) it is
 * resynchronised to the boundary dtype: GDN_F32 changes nothing, GDN_BF16 rounds every element
 * to the nearest bf16 (ties to even).  Every path applies the same rounding at the same
 * positions; the state after a call's last token is left unrounded.
 * schedule: 1, the pinned per-token schedule:
 *   for every value column j independently, in fp32 with IEEE denormals and round-to-nearest-even,
 *   (1) leaf partials over consecutive 8-row leaves of the d_k rows: p = S[r0][j]*k[r0], then
 *       p = fma(S[r][j], k[r], p) for r = r0+1 .. r0+7;
 *   (2) u_j = balanced pairwise sum of the d_k/8 leaf partials (leaf 2m with 2m+1, then pairs of
 *       those, ...);
 *   (3) w_j = fma(-a, u_j, v_j);  c_j = b * w_j;
 *   (4) S[r][j] = fma(k[r], c_j, a * S[r][j]) for every row r;
 *   (5) o_j = steps (1)-(2) applied to the updated S and q.
 * With fp32 boundaries chunk is a deployment setting (it decides which states are materialised,
 * never a value) and is left out of the policy digest; with bf16 boundaries it is numerical. */
typedef struct gdn_policy {
  int32_t h_k;
  int32_t h_v;
  int32_t dk;
  int32_t dv;
  int32_t chunk;
  int32_t io_dtype;
  int32_t state_dtype;
  int32_t schedule;
} gdn_policy;

/* Opaque host handle describing a pool of recurrent states ("slots") on one device. */
typedef struct gdn_state gdn_state;

/* Message for the last failing call on this host thread ("" if none).  Never NULL; the buffer is
 * owned by the library and valid until the next call on this thread. */
const char* gdn_last_error(void);

/* SHA-256 (FIPS 180-4) of the policy's canonical bytes: the ASCII tag "cpr-gdn-policy-v1"
 * followed by h_k, h_v, dk, dv, io_dtype, state_dtype, schedule, chunk (0 when state_dtype is
 * GDN_F32), the leaf size (8) and the GQA rule (0 = repeat-interleave) as little-endian int32.
 * Writes 32 bytes.
 * ("The execution contract": digests exchanged at start-up.)  Host-only; needs no GPU. */
int gdn_policy_digest(const gdn_policy* policy, uint8_t out[32]);

/* The other two digests of "The execution contract", same form (SHA-256 of an ASCII tag and
 * little-endian int32 fields):
 *   semantic    what is computed: tag "cpr-gdn-semantic-v1", recurrence id (1), h_k, h_v, dk, dv,
 *               GQA rule (0).  Equal semantic digests mean the same mathematical function.
 *   deployment  settings that provably move no bit: tag "cpr-gdn-deploy-v1", chunk (0 when the
 *               boundary dtype is bf16, where chunk is numerical policy), and the kernels' work-
 *               mapping version.  Peers may differ here and still agree bitwise.
 * Host-only. */
int gdn_semantic_digest(const gdn_policy* policy, uint8_t out[32]);
int gdn_deployment_digest(const gdn_policy* policy, uint8_t out[32]);

/* SHA-256 (FIPS 180-4) of n host bytes into out[32]; the primitive behind the policy digest and
 * the identity digests of outputs ("The execution contract": SHA-256 identity digests).
 * Host-only. */
int gdn_sha256(const void* data, size_t n, uint8_t out[32]);

/* Compare two 32-byte policy digests: GDN_OK when equal, GDN_EPOLICY otherwise (the caller must
 * then refuse to run, as the execution contract prescribes).  Host-only. */
int gdn_policy_check(const uint8_t mine[32], const uint8_t theirs[32]);

/* Validate a policy against what the library was compiled with: GDN_OK, GDN_EINVAL or
 * GDN_EUNSUPPORTED.  Host-only. */
int gdn_policy_validate(const gdn_policy* policy);

/* Bytes of a state array for num_slots slots: num_slots * h_v * dv * dk * 4 (0 on bad input).
 * The state is the fp32 matrix the recurrence carries per (sequence, value head) (section "Solving
 * the linear-attention headache": decode keeps it between tokens and re-bases it every chunk). */
size_t gdn_state_bytes(const gdn_policy* policy, int32_t num_slots);

/* Create a state pool handle for num_slots slots: the recurrent states decode carries from token
 * to token and prefill starts from or leaves behind (section "Solving the linear-attention
 * headache"), with the policy that pins their arithmetic (section "The execution contract").
 *   state, pos:     caller-owned device arrays (layouts above; state_bytes must equal
 *                   gdn_state_bytes).  The caller initialises them (normally to zero).  If both
 *                   are NULL the library allocates and zero-fills them itself (hipMalloc,
 *                   synchronous) and frees them in gdn_state_free.
 *   boundary, boundary_pos:  optional (both NULL or both set) caller-owned device arrays with the
 *                   layouts of state and pos.  When present, every resynchronisation records the
 *                   slot's chunk-start state and its position there.
 * The handle itself is host memory; free it with gdn_state_free.  On error *out is set to NULL. */
int gdn_state_alloc(const gdn_policy* policy, int32_t num_slots, float* state, int64_t* pos,
                    size_t state_bytes, float* boundary, int64_t* boundary_pos,
                    gdn_state** out);

/* Release a handle made by gdn_state_alloc (and the device arrays if the library allocated them);
 * caller-owned arrays are left untouched.  NULL is a no-op. */
int gdn_state_free(gdn_state* st);

/* Device pointers of a pool (for callers that let the library allocate).  Host-only. */
float* gdn_state_data(gdn_state* st);
int64_t* gdn_state_positions(gdn_state* st);

/* Launch shape of later calls on this pool (section "Making kernels parallelism-invariant":
 * identical bits however the work is split).  max_workgroups = 0, the default, launches one
 * workgroup per work item.  A positive value caps the workgroups of the compute kernels at that
 * number, and each workgroup takes work items in turn.  The capped kernels are the two prefill
 * passes, the one-pass and overlapped prefill and the decode step.  No output or state changes
 * by a bit; a small cap only runs the work with less parallelism.  The position-update, resync,
 * chunkwise and backward kernels keep their natural shapes.  GDN_EINVAL for a NULL handle, a
 * negative value or one of 2^31 or more.  Host-only. */
int gdn_state_set_max_workgroups(gdn_state* st, int64_t max_workgroups);

/* Bound of each wait in the overlapped prefill's later calls on this pool: the number of polls
 * (about 50 ns each) after which a wave stops waiting for another wave of its workgroup.
 * 0, the default, is 2^22 polls (about 0.2 s), far beyond any wait of a working kernel.  A small
 * value makes waits give up, which is reported by gdn_device_status; it exists so that the error
 * path can be exercised with every kernel still ending normally.  GDN_EINVAL for a NULL handle.
 * Host-only. */
int gdn_state_set_wait_limit(gdn_state* st, uint32_t polls);

/* Outcome of the overlapped prefills run on the current device since the last call (section "The
 * execution contract": refuse to run, rather than run mismatched numerics).  Each wave of the
 * overlapped kernel waits for others of its workgroup only for a bounded time; a wave whose wait
 * gives up touches no shared buffer afterwards, leaves its work item and sets a flag in a
 * per-device status word.  This call synchronises `stream`, reads that word and clears it:
 * GDN_OK when no wait gave up, GDN_EHIP otherwise (gdn_last_error names which waits), in which
 * case the outputs, final states, positions and chunk-start rows of those calls are not valid.
 * Unlike every other call it synchronises the host (with `stream`).  The word is shared by every
 * pool on the device: any give-up since the last check is reported. */
int gdn_device_status(void* stream);

/* Host-side check of a cu_seqlens array (host copy): GDN_OK if cu[0] == 0, non-decreasing and
 * cu[num_seqs] == total_tokens; GDN_EINVAL otherwise. */
int gdn_check_cu_seqlens(const int32_t* cu_seqlens_host, int32_t num_seqs, int64_t total_tokens);

/* Upper bound on the chunk-state rows any prefill over total_tokens tokens in num_seqs sequences
 * can need: floor(total_tokens / chunk) + 2 * num_seqs.  Returns -1 on bad input. */
int64_t gdn_chunk_rows_bound(int64_t total_tokens, int32_t num_seqs, int32_t chunk);

/* Exact chunk-state row layout of a prefill, from host copies.  For sequence i of length L_i
 * starting at absolute position p_i (0, or the slot's pos when continuing), the rows are the
 * states entering position p_i and every chunk start strictly inside [p_i, p_i + L_i); there are
 * R_i = 1 + floor((p_i + L_i - 1)/C) - floor(p_i/C) of them (0 if L_i = 0), stored consecutively
 * from row_offsets[i]; row_offsets has num_seqs + 1 entries, the last being the total.
 * pos0_host may be NULL (all zero). */
int gdn_chunk_rows(const int32_t* cu_seqlens_host, const int64_t* pos0_host, int32_t num_seqs,
                   int32_t chunk, int64_t* row_offsets);

/* Prefill / trainer forward over a packed batch ("Solving the linear-attention headache": first
 * pass to the chunk boundaries, then the chunk-parallel output pass).
 *   cu_seqlens   device int32 [num_seqs + 1]; total_tokens = N.
 *   slot_ids     device int32 [num_seqs]: sequence i starts from and ends in slot slot_ids[i]
 *                (distinct slots; num_seqs may be 0).
 *   from_state   0: start from the zero state at position 0 (slot contents ignored);
 *                1: continue from the slot's state at position pos[slot].
 *   q, k, v, o   io dtype; a, b fp32 (layouts above).  o receives every token's output.
 *   chunk_states device fp32 [chunk_state_rows][H_v][d_v][d_k]: the chunk-boundary states, in the
 *                layout gdn_chunk_rows describes (row 0 of a sequence is its initial state).
 *                For engine prefill this is scratch; for the trainer forward it is the stash the
 *                caller keeps.  chunk_state_rows must be >= gdn_chunk_rows_bound(N, num_seqs, C).
 *   c_stash      NULL, or device fp32 scratch [N][H_v][d_v] (16-byte aligned).  When given, the
 *                boundary pass runs every token (not only up to the last chunk start) and keeps
 *                each token's write value c_t = b_t w_t there, and the output pass applies the
 *                kept c_t instead of computing the prediction S^T k_t again: about a quarter less
 *                arithmetic in the output pass for N*H_v*d_v*8 more bytes of traffic.  The
 *                update is fed the very value it would compute, so o, final states and chunk
 *                states are bit for bit the same with or without it.  Contents on return: c.
 * On return (stream order) each slot holds its sequence's final state and pos[slot] = p_i + L_i.
 * Launches the boundary pass, the output pass and a position update on `stream`.
 * events: NULL, or 3 hipEvent_t (as void*) recorded on `stream` before the boundary pass, between
 * the two passes and after the output pass, so a caller can time each pass. */
int gdn_prefill(gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                const int32_t* slot_ids, int32_t from_state,
                const void* q, const void* k, const void* v, const float* a, const float* b,
                void* o, float* chunk_states, int64_t chunk_state_rows, float* c_stash, void* stream,
                void* const* events);

/* gdn_prefill without any device memory from the caller or the allocator, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * The chunk-start states the two passes hand over, and the c stash when it fits as well, live in a
 * library-owned static device buffer of GDN_STATIC_SCRATCH_BYTES (256 MiB), which every device the
 * library runs on holds from its first use of this call until the process ends.  The call itself
 * allocates nothing and frees nothing.
 *   Arguments as gdn_prefill, without chunk_states and c_stash.  The results (o, final states,
 *   positions) are gdn_prefill's bits.
 *   Limit: gdn_chunk_rows_bound(total_tokens, num_seqs, chunk) * h_v * dv * dk * 4 bytes (rounded
 *   up to 256) must fit the buffer -- 128 rows at 32 value heads of 128 x 128, e.g. 7,680 tokens in
 *   4 sequences at chunk 64; larger batches return GDN_EINVAL with a message naming the sizes
 *   (split them, or use gdn_prefill).  The c stash is used when the rows and N * h_v * dv * 4 bytes
 *   both fit; otherwise the output pass recomputes c (the same bits).
 *   Nothing in the buffer needs clearing: every row or c a call reads was written earlier in the
 *   same call.  The buffer is shared by every call on the device and keeps the last call's
 *   contents: calls that overlap on one device (on different streams, or from different host
 *   threads) race on it and must be ordered by the caller.
 * events: as gdn_prefill. */
#define GDN_STATIC_SCRATCH_BYTES (256u << 20)
int gdn_prefill_static(gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                       const int32_t* slot_ids, int32_t from_state,
                       const void* q, const void* k, const void* v, const float* a, const float* b,
                       void* o, void* stream, void* const* events);

/* The trainer forward (the "trainer_fwd" case of section "The execution contract", whose per-layer
 * table in section "Solving the linear-attention headache" times CPR for the trainer's forward and
 * backward): gdn_prefill, bit for bit in o, final states
 * and chunk states, that also keeps what the backward would otherwise recompute:
 *   cw  device fp32 [2][N][H_v][d_v]: every token's c_t = b_t w_t (block 0) and
 *       w_t = v_t - a_t S_{t-1}^T k_t (block 1), as the pinned step computed them.  Block 0
 *       serves as gdn_prefill's c_stash: the boundary pass writes both blocks and the output
 *       pass applies block 0.
 * Pass it to gdn_backward.  events as gdn_prefill. */
int gdn_trainer_forward(gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                        const int32_t* slot_ids, int32_t from_state,
                        const void* q, const void* k, const void* v, const float* a, const float* b,
                        void* o, float* chunk_states, int64_t chunk_state_rows, float* cw, void* stream,
                        void* const* events);

/* One-pass prefill: the same recurrence and the same outputs, final states and chunk-start rows
 * as gdn_prefill, bit for bit, evaluated by a single kernel that runs every token of a sequence
 * in order (the per-layer table of section "Solving the linear-attention headache" calls this
 * evaluation "recurrent everywhere").  It does no second pass, so it suits batches whose
 * (sequence, value head, column) chains already fill the GPU; gdn_prefill's chunk-parallel
 * pass suits few long sequences.  Arguments as gdn_prefill, except that there is no c_stash and
 * chunk_states may be NULL (no stash is written; chunk_state_rows is then ignored).
 * events: NULL, or 2 hipEvent_t recorded before and after the kernel. */
int gdn_prefill_fused(gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                      const int32_t* slot_ids, int32_t from_state,
                      const void* q, const void* k, const void* v, const float* a, const float* b,
                      void* o, float* chunk_states, int64_t chunk_state_rows, void* stream,
                      void* const* events);

/* Overlapped prefill: the same results as gdn_prefill, bit for bit, from a single launch in
 * which each (sequence, value head, column group) workgroup runs pass 1 on some of its waves and
 * produces the outputs of every chunk pass 1 has finished on other waves of the same workgroup,
 * while pass 1 goes on (section "Solving the linear-attention headache": the parallel fill-in of
 * a chunk's outputs needs only the state at its start).  It suits a few long sequences, where
 * pass 1 alone cannot fill the GPU and pass 2 would otherwise run after it.  The state entering
 * each chunk and its tokens' write values c_t pass between the waves through LDS, so nothing is
 * written to HBM for the hand-off.  Each workgroup (one per sequence, value head and group of
 * 16 columns at d = 16 or 128, 32 at d = 32 or 64) needs a CU of its own: when there are more
 * workgroups than the device has CUs, or a chunk exceeds 64 tokens, the call runs the one-pass
 * kernel instead (the same bits).  Arguments as gdn_prefill_fused.  events: NULL, or 2 hipEvent_t recorded before and
 * after the kernel. */
int gdn_prefill_overlapped(gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                           const int32_t* slot_ids, int32_t from_state,
                           const void* q, const void* k, const void* v, const float* a, const float* b,
                           void* o, float* chunk_states, int64_t chunk_state_rows, void* stream,
                           void* const* events);

/* One decode step: one token for each of `batch` slots (section "Solving the linear-attention
 * headache": decode applies the recurrence one token at a time).
 *   slot_ids device int32 [batch] (distinct); q, k [batch][H_k][d_k]; v, o [batch][H_v][d_v];
 *   a, b [batch][H_v].
 * For a slot whose position is a multiple of C the incoming state is a chunk-start state: it is
 * resynchronised first (see gdn_state_resync) and then the token is applied with the same pinned
 * step as prefill.  Afterwards pos[slot] += 1.  With the fp32 boundary dtype and no boundary
 * record the step needs no position and advances it itself (one kernel launch); otherwise a
 * second kernel advances it after the step (two launches).  batch may be 0.
 * events: NULL, or 2 hipEvent_t (as void*) recorded on `stream` before the step and after its last
 * launch. */
int gdn_decode_step(gdn_state* st, const int32_t* slot_ids, int32_t batch,
                    const void* q, const void* k, const void* v, const float* a, const float* b,
                    void* o, void* stream, void* const* events);

/* Resynchronise listed slots (same section: decode re-bases its state once per chunk).  For a
 * slot at a chunk start (pos % C == 0) the state is re-based on the boundary state in the
 * policy's boundary dtype (fp32: no change; bf16: the state is rounded in place, as a decode step
 * would do before applying the token) and committed: copied, with pos, into the pool's boundary
 * record if it has one.  Slots that are not at a chunk start are left alone.  Rounding is
 * idempotent, so a decode step after an explicit resync changes nothing further.
 * slot_ids device int32 [n]. */
int gdn_state_resync(gdn_state* st, const int32_t* slot_ids, int32_t n, void* stream);

/* ---- chunkwise evaluation on matrix cores --------------------------------------------------
 * The per-layer table of section "Solving the linear-attention headache" compares CPR with a
 * "native" evaluation: the chunkwise (WY/UT) form of the gated delta rule on matrix units.  Per
 * chunk of L tokens with gate products G_t = a_1...a_t and entering state S_0, the write vectors
 * c_t solve (I + A) C = diag(b) V - diag(b G) K S_0 with A[s][r] = b_s (G_s/G_r) k_s.k_r (r < s);
 * with T = (I + A)^{-1}, W = T diag(b G) K and U = T diag(b) V:  C = U - W S_0,
 * S_L = G_L S_0 + K^T diag(G_L/G) C  and  O = diag(G) Q S_0 + (M . Q K^T) C, M[t][s] = G_t/G_s
 * (s <= t).  The products run on bf16 matrix cores with fp32 accumulation, operands that are not
 * exact bf16 split into a high and a low bf16 part.  Results agree with the recurrence to the
 * bf16 output tolerance, not bit for bit with the CPR entry points.
 *   outputs GDN_CHUNKED_NATIVE  o and the final states from the chunk form;
 *   outputs GDN_CHUNKED_R2      the chunk form gives only the states at chunk starts; o and the
 *                               final state come from the pinned per-token step started at those
 *                               states (the other reading of CPR's first pass: its boundary states
 *                               differ from the per-token ones, so resynchronisation changes
 *                               values).
 * Requirements: bf16 io, fp32 boundary dtype, chunk <= 64, dk = dv in {32, 64, 128}, every gate
 * a_t > 0 (GDN_EUNSUPPORTED otherwise).  Arguments as gdn_prefill, plus a caller-owned device
 * workspace (16-byte aligned) of gdn_prefill_chunked_workspace_bytes().  chunk_states receives
 * the states entering every chunk, in gdn_chunk_rows' layout.
 * events: NULL, or 4 hipEvent_t recorded before and between the three stages and at the end. */
#define GDN_CHUNKED_NATIVE 0
#define GDN_CHUNKED_R2 1

/* ---- R2 resynchronisation in decode ---------------------------------------------------------
 * Under the R2 reading of CPR's first pass (GDN_CHUNKED_R2 above), the state at every chunk start
 * is the chunk form's, and decode, which the section "Solving the linear-attention headache" has
 * bring its state back in line once every chunk of tokens, does so by recomputing it with the chunk
 * form.  A pool with R2
 * attached keeps, per slot, the chunk-start state of the chunk its last token fell in (in its
 * boundary record, with that chunk start as boundary_pos) and the chunk's tokens so far (a
 * caller-owned ring, indexed by position mod C).  Then:
 *   gdn_prefill_chunked(GDN_CHUNKED_R2) also fills each sequence's ring with the tokens from the
 *     start of its last chunk on, and its boundary record with the state entering that chunk;
 *   gdn_decode_step, for each listed slot whose position is a chunk start p > 0, first replaces
 *     the slot's state by the chunk form's state at p, computed from the recorded state over the
 *     ring's C tokens by the same kernels as gdn_prefill_chunked (so with its bits), then applies
 *     the token with the pinned step (recording the new chunk-start state) and appends it to the
 *     ring.
 * Decoding a prompt's continuation this way gives the bits of one gdn_prefill_chunked(R2) over
 * prompt and generated tokens, when each R2 prefill of the slot started at a chunk start (such as
 * position 0).  R2 pools refuse the R1 prefills, gdn_state_resync and native chunked outputs, which
 * would leave the ring behind.
 * Requirements: as gdn_prefill_chunked, and a pool with a boundary record.
 *   gdn_r2_ring_bytes       num_slots * C token positions of q, k (bf16 [H_k][dk]), v (bf16
 *                           [H_v][dv]), a and b (fp32 [H_v]); -1 on bad input.
 *   gdn_r2_workspace_bytes  the chunk form's workspace for one chunk per slot plus small tables.
 *   gdn_state_attach_r2     binds caller-owned device memory (16-byte aligned, at least those
 *                           sizes); both NULL detaches.  The first attach also creates, on the
 *                           current device (the pool's), a second HIP stream at the default
 *                           priority and two events: gdn_decode_step runs the listed slots'
 *                           resynchronisation and step on it, forked from and joined back into
 *                           the caller's stream (graph capture follows the fork), beside the
 *                           other slots' step.  Where they cannot be created (no device), the
 *                           step runs in sequence on the caller's stream, with the same bits.
 *                           Detaching or gdn_state_free releases them.  No device work. */
int64_t gdn_r2_ring_bytes(const gdn_policy* policy, int32_t num_slots);
int64_t gdn_r2_workspace_bytes(const gdn_policy* policy, int32_t num_slots);
int gdn_state_attach_r2(gdn_state* st, void* ring, size_t ring_bytes, void* workspace, size_t workspace_bytes);
int64_t gdn_prefill_chunked_workspace_bytes(const gdn_policy* policy, int64_t total_tokens, int32_t num_seqs);
int gdn_prefill_chunked(gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                        const int32_t* slot_ids, int32_t from_state,
                        const void* q, const void* k, const void* v, const float* a, const float* b,
                        void* o, float* chunk_states, int64_t chunk_state_rows, int32_t outputs,
                        void* workspace, size_t workspace_bytes, void* stream, void* const* events);

/* ---- trainer backward ------------------------------------------------------------------------
 * The per-layer table of section "Solving the linear-attention headache" times CPR for the
 * trainer's forward and backward.  The gradients are those of the recurrence above for a loss L,
 * given dO = dL/do and, optionally, dL/dS_T of every sequence's final state:
 *   G = dL/dS_t runs backward in time; per token, with Gh = G + q_t dO_t^T,
 *   dq_t = S_t dO_t,  dc = Gh^T k_t,  dw = b_t dc,  du = -a_t dw,  dv_t = dw,  db_t = <dc, w_t>,
 *   dk_t = Gh c_t + S_{t-1} du,  da_t = <Gh, S_{t-1}> - <dw, u_t>,  G <- a_t Gh + k_t du^T,
 * and dL/dS_0 is G after the first token; dq and dk of a key head sum its value heads'.
 * Four kernels evaluate it: an adjoint pass walks each sequence backward (G needs no forward
 * state) and keeps dc for every token, G at every chunk boundary and <G, S> at every chunk start;
 * a replay pass re-runs the pinned forward step of every chunk from the stash and keeps c and w
 * (skipped when the trainer forward kept them); a per-token pass forms dv and db; a
 * chunk-gradient pass, one workgroup per (chunk, key head), forms dq and dk on fp32 matrix cores
 * from the chunk-form expansion of S_t and G_t (chunk-start or chunk-end matrix plus
 * decay-weighted rank-one terms), and da from a_t da_t = <G_{t-1}, S_{t-1}>, carried along the
 * chunk in fp64.  Every sum has a fixed order, so the gradients are bitwise reproducible for any
 * batch composition or packing. */

/* Workspace bytes gdn_backward needs for total_tokens tokens in num_seqs sequences (-1 on bad
 * input): dL/dS at every boundary of the gradient chunks (total_tokens / C' + 2 num_seqs states;
 * C' = 64 with fp32 boundaries, min(C, 64) with bf16 boundaries), three fp32 per-token arrays
 * of N * H_v * d_v (dc, c, w), per boundary and value head the parts of <dL/dS, S> (fp64:
 * 32 at d = 128, 8 at 64, 2 at 32, 1 at 16), and one fp32 v_t . dv_t per token and value head;
 * with fp32 boundaries and C != 64 also a rebuilt 64-token stash
 * (total_tokens / 64 + num_seqs states), one int32 per sequence and one int64 per row of the
 * forward's stash.  Each part is padded to 256 bytes. */
int64_t gdn_backward_workspace_bytes(const gdn_policy* policy, int64_t total_tokens, int32_t num_seqs);

/* Gradients of a trainer forward (gdn_trainer_forward, gdn_prefill or gdn_prefill_fused over the
 * same packed batch, every sequence starting at position 0: from_state 0, or 1 from slots at
 * position 0).
 *   policy        the forward's policy.  The chunk-gradient kernel's tile is 64 tokens.  With fp32
 *                 boundaries the gradients are always taken at chunk 64: for a forward at any
 *                 other chunk C a fourth kernel first rebuilds the 64-token stash with the
 *                 boundary pass, from each sequence's row 0 of `chunk_states`.  A chunk-start
 *                 state does not depend on C there, so that stash holds the bits a 64-token
 *                 forward would have stored, and the gradients are the same bits for every C
 *                 (C is a deployment setting, as the policy digest says; section "The execution
 *                 contract": equal policy digests, equal bits).  With bf16 boundaries C is part of
 *                 the policy: the gradients run at chunk C on the forward's own rounded rows, and
 *                 C > 64 is GDN_EUNSUPPORTED.
 *                 With the bf16 boundary dtype the rounding at chunk starts is read as the
 *                 identity (straight-through): the gradients are those of the trajectory the
 *                 forward took (from its rounded chunk-start states), with dL/dS passed through
 *                 each rounding unchanged.  Every gate a_t must be positive (da_t is obtained by
 *                 dividing by a_t); the gate form exp(-softplus(x)) always is.
 *   cu_seqlens, total_tokens, q, k, v, a, b   the forward's inputs (device, layouts above).
 *   chunk_states  the forward's stash, chunk_state_rows >= total_tokens / C + num_seqs (any
 *                 forward stash qualifies): row 0 of a sequence is its initial state S_0.
 *   cw            NULL, or gdn_trainer_forward's c and w: then the replay of the forward is
 *                 skipped (the gradients are the same bits either way).
 *   d_o           device, io dtype, [N][H_v][d_v]: dL/do.
 *   d_state       device fp32 [num_seqs][H_v][d_v][d_k] (state layout) or NULL (zero): dL/dS_T.
 *   dq, dk        device fp32 [N][H_k][d_k];  dv  fp32 [N][H_v][d_v];  da, db  fp32 [N][H_v].
 *   d_state0      device fp32 [num_seqs][H_v][d_v][d_k] or NULL: dL/dS_0 (for a forward that
 *                 continued from slots).
 *   workspace     device, 16-byte aligned, workspace_bytes >= gdn_backward_workspace_bytes().
 * Outputs are fully overwritten for every token of every well-formed sequence.  Up to four kernels
 * on `stream` (after the stash rebuild when C != 64 with fp32 boundaries); events: NULL, or 4
 * hipEvent_t recorded before the adjoint, after it, after the replay and per-token pass, and at
 * the end. */
int gdn_backward(const gdn_policy* policy, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                 const void* q, const void* k, const void* v, const float* a, const float* b,
                 const float* chunk_states, int64_t chunk_state_rows, const float* cw, const void* d_o,
                 const float* d_state,
                 float* dq, float* dk, float* dv, float* da, float* db, float* d_state0,
                 void* workspace, size_t workspace_bytes, void* stream, void* const* events);

/* ---- chunkwise trainer: forward and backward on matrix cores ----------------------------------
 * The "native" trainer column of the per-layer table in section "Solving the linear-attention
 * headache": the chunkwise evaluation above for the forward, and the chunk form of the adjoint
 * recurrence for the backward.  Per chunk (notation of the chunkwise block above), with J the
 * gradient dL/dS at the chunk's end, the gradients reaching the write vectors solve the transposed
 * system, dC = T^T R with R = (M . Q K^T)^T dO + diag(G_L/G) K J, and dL/dS at the chunk start is
 * G_L J + Q^T diag(G) dO - W^T R; the forward's w = v - a S^T k is V - diag(G) K S_0 - (N . K K^T) C
 * (N[t][s] = G_t/G_s, s < t).  A parallel pass forms w and the part of R without G_L, a pass per (sequence, value head,
 * 32 columns) walks the chunks last to first, and dq, dk, dv, da and db then come from the same
 * per-token and chunk-gradient kernels as gdn_backward.  The gradients agree with the recurrence's
 * to the backward tolerance; they are deterministic (fixed summation orders) but not the bits of
 * gdn_backward, and they depend on C, as the chunkwise forward does.
 * Requirements: as gdn_prefill_chunked; every sequence starts at position 0 (from_state 0, or 1
 * from slots at position 0).
 *   gdn_trainer_forward_chunked_stash_bytes  bytes of the stash the forward keeps for the backward:
 *       the chunk form's workspace, T^T and W^T per chunk row and value head (fp32), and every
 *       token's c (fp32 [N][H_v][d_v]), each part padded to 256 bytes; -1 on bad input.
 *   gdn_trainer_forward_chunked  gdn_prefill_chunked(GDN_CHUNKED_NATIVE) that also fills the
 *       caller-owned stash (device, 16-byte aligned); chunk_states keeps the chunk-start states.
 *       events: as gdn_prefill_chunked.
 *   gdn_backward_chunked_workspace_bytes  dL/dS at every chunk boundary (total_tokens / C +
 *       2 num_seqs states), dc and w (fp32 [N][H_v][d_v] each), 4 fp64 parts of <dL/dS, S> per
 *       32 value columns per boundary and value head, and v . dv per token and value head.
 *   gdn_backward_chunked  arguments as gdn_backward, with the forward's stash in place of cw;
 *       d_state0 (nullable) receives dL/dS_0.  Events: NULL, or 4 hipEvent_t recorded before the
 *       chunk-form passes, after them, after the per-token gradients and at the end. */
int64_t gdn_trainer_forward_chunked_stash_bytes(const gdn_policy* policy, int64_t total_tokens, int32_t num_seqs);
int gdn_trainer_forward_chunked(gdn_state* st, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                                const int32_t* slot_ids, int32_t from_state,
                                const void* q, const void* k, const void* v, const float* a, const float* b,
                                void* o, float* chunk_states, int64_t chunk_state_rows,
                                void* stash, size_t stash_bytes, void* stream, void* const* events);
int64_t gdn_backward_chunked_workspace_bytes(const gdn_policy* policy, int64_t total_tokens, int32_t num_seqs);
int gdn_backward_chunked(const gdn_policy* policy, const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                         const void* q, const void* k, const void* v, const float* a, const float* b,
                         const float* chunk_states, int64_t chunk_state_rows, const void* stash, size_t stash_bytes,
                         const void* d_o, const float* d_state,
                         float* dq, float* dk, float* dv, float* da, float* db, float* d_state0,
                         void* workspace, size_t workspace_bytes, void* stream, void* const* events);

#ifdef __cplusplus
}
#endif

#endif /* CPR_GDN_H */
