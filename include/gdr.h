/*
 * gdr.h -- C ABI of libgdr, the gated delta-rule hot path for MI355X (gfx950).
 *
 * The operation.  "Super Apriel: One Checkpoint, Many Speeds" (arXiv
 * 2604.19877) builds every decoder layer with four mixer choices: full
 * attention, sliding-window attention, Kimi Delta Attention (KDA) and Gated
 * DeltaNet (GDN) (abstract; gist.science technical summary, section 2a).  The
 * summary describes KDA as recurrent with a gate per key channel and GDN as
 * recurrent with one scalar gate per head.  The pages print no formula; this
 * library implements the standard gated delta rule, per sequence and head:
 *
 *     S_t = S_{t-1} Diag(a_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = scale * S_t q_t          (the state after the token's update)
 *
 * S is Dv x Dk, fp32, stored row-major with the key index contiguous
 * (state[..., i, j], i < Dv, j < Dk).  The gate is passed as its logarithm
 * g = ln a <= 0 (fp32): GDR_GATE_SCALAR takes one value per token and head,
 * GDR_GATE_CHANNEL takes Dk values.  beta is one fp32 per token and head.
 * A placement assigns one mixer per layer and can change between requests
 * (abstract; summary section 2d); gdr_decode_placement steps only the layers
 * it tags GDN or KDA.
 *
 * Conventions for every entry point.
 *   - Pointers are DEVICE pointers unless marked "host".  Tensors are dense,
 *     row-major, in the layouts given per function, and 16-byte aligned.
 *   - The caller owns every buffer and the stream.  The library never
 *     allocates, frees or synchronises; work is enqueued on `stream`
 *     (a hipStream_t; NULL = the default stream) and the call returns.
 *   - Every argument is checked on the host before any HIP call.  A bad
 *     argument returns GDR_EINVAL or GDR_EUNSUPPORTED, launches nothing and
 *     writes nothing.  A failed launch returns GDR_EHIP.  Faults during
 *     execution surface at the caller's next synchronisation.
 *   - gdr_last_error() returns a thread-local description of the last
 *     non-OK status.  No C++ exception crosses this interface; all entry
 *     points are reentrant.
 *   - Supported shapes: Dk == Dv, Dk in {64, 128}; chunk == 64 (prefill);
 *     per prefill call fewer than 2^40 elements in q and at most 2^28
 *     (sequence, head) pairs, per decode call fewer than 2^31 stepped
 *     (layer, b, h) slots (GDR_EUNSUPPORTED otherwise).
 *     q, k, v and o share one dtype (GDR_F32 or GDR_BF16); g, beta, states
 *     are always fp32.  bf16 outputs are rounded to nearest-even.
 *   - Setting the environment variable GDR_DEBUG=1 makes each call
 *     synchronise its stream and check for errors (for tests only).
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int gdr_status;
enum { GDR_OK = 0, GDR_EINVAL = 1, GDR_EUNSUPPORTED = 2, GDR_EHIP = 3 };

/* dtype of q, k, v and o */
enum gdr_dtype { GDR_F32 = 0, GDR_BF16 = 1 };

/* GDN: g[..., H]   KDA: g[..., H, Dk] */
enum gdr_gate { GDR_GATE_SCALAR = 0, GDR_GATE_CHANNEL = 1 };

/* placement codes, one mixer per layer */
enum gdr_mixer { GDR_FA = 0, GDR_SWA = 1, GDR_GDN = 2, GDR_KDA = 3 };

/*
 * Device workspace (bytes) that a prefill call over N sequences of `tokens`
 * tokens in all (B and B*T for gdr_prefill_chunked, N and T_total for
 * gdr_prefill_chunked_varlen) and H heads needs with this dtype and gate
 * kind: the varlen schedule and chunk offsets (N and N+1 int32, each rounded
 * up to 256 bytes); for bf16 with the channel gate, one int32 per (sequence,
 * head) (rounded up to 256 bytes: the pairs that the second pass redoes,
 * see gdr_prefill_chunked); for bf16 with the scalar gate, a record of
 * every chunk and head (the chunk-local inverse T, the gate's prefix sums
 * and the chunk's decay factors, 5888 bytes) for tokens / 64 + N chunks, an
 * upper bound.  Returns 0 for N <= 0, tokens < 0 or H <= 0.  A buffer of
 * this size serves either call with these sizes.
 */
size_t gdr_prefill_workspace_bytes(enum gdr_dtype dt, enum gdr_gate gk, int N,
                                   long long tokens, int H);

/*
 * Chunked prefill over a fixed-length batch: the recurrence above for every
 * (b, h), all T tokens, returning every output and (optionally) the final
 * states.
 *
 *   dt, gk      dtype of q/k/v/o; gate kind
 *   B, T, H     batch, tokens per sequence (T >= 0), heads
 *   Dk, Dv      key and value widths (equal, 64 or 128)
 *   chunk       64
 *   scale       multiplies o only
 *   q, k        [B, T, H, Dk]   dt
 *   v           [B, T, H, Dv]   dt
 *   g           [B, T, H] (scalar) or [B, T, H, Dk] (channel), fp32, <= 0
 *   beta        [B, T, H] fp32
 *   h0          [B, H, Dv, Dk] fp32 initial states, or NULL for zeros
 *   o           [B, T, H, Dv]   dt (written)
 *   ht          [B, H, Dv, Dk] fp32 final states (written), or NULL.
 *               ht == h0 is allowed (in-place resume); no other aliasing.
 *   workspace   device buffer, 16-byte aligned, of at least
 *               gdr_prefill_workspace_bytes(dt, gk, B, B*T, H) bytes, used
 *               for bf16 inputs (fp32 inputs need none: it is ignored and
 *               may be NULL); scratch for the duration of the call, not to
 *               be shared with a concurrent call
 *   ws_bytes    its size
 *   stream      hipStream_t
 *
 * bf16 inputs run the chunked form on MFMA (chunk of 64 tokens, WY/UT
 * transform inside the chunk, state carried between chunks in fp32).  fp32
 * inputs run the recurrent form token by token in fp32 on the vector ALUs.
 * With T == 0 nothing is written to o and ht = h0 (zeros if h0 is NULL).
 * Every gate g in [-inf, 0] is taken, for both gate kinds: the chunked
 * form never forms a decay factor from a difference of infinite prefix sums
 * or a factor above 1 from the chunk's whole decay.  It raises g below -30
 * to -30 (a gate under 9.4e-14 becomes 9.4e-14, a change far below fp32
 * rounding of the states).  The scalar gate forms each in-chunk factor as
 * e^{b_r - b_s}, s <= r.  The channel gate runs two passes: the first
 * factors each chunk from its first token, which is exact while no channel
 * decays by more than e^80 over the chunk, and marks any (sequence, head)
 * where one does; the second redoes only the marked pairs with references at
 * every 16th token (all factors at most 1), and forms a 16-token diagonal
 * block entry by entry where a channel decays by more than e^70 inside it.
 */
gdr_status gdr_prefill_chunked(enum gdr_dtype dt, enum gdr_gate gk, int B, int T,
                               int H, int Dk, int Dv, int chunk, float scale,
                               const void *q, const void *k, const void *v,
                               const float *g, const float *beta, const float *h0,
                               void *o, float *ht, void *workspace, size_t ws_bytes,
                               void *stream);

/*
 * gdr_prefill_chunked without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The library keeps its own workspace:
 * one array of GDR_NOALLOC_MAX_BYTES per GPU, held from the first call on
 * that GPU until the process ends.  The call allocates and frees nothing.
 *
 *   all arguments as gdr_prefill_chunked, without workspace and ws_bytes
 *
 * Calls whose workspace (gdr_prefill_workspace_bytes(dt, gk, B, B*T, H))
 * would exceed GDR_NOALLOC_MAX_BYTES return GDR_EUNSUPPORTED and launch
 * nothing; GDN B=4 H=16 T=4096 needs 25 MB.  Every call on one GPU uses that
 * GPU's one array: calls that overlap on one GPU (two streams, two threads)
 * race and must be ordered by the caller.  Nothing in the array needs
 * clearing between calls: each call writes every byte it reads.  The device
 * address of the array is taken once per GPU, on the call's current device,
 * which must be the device of `stream`.
 */
#define GDR_NOALLOC_MAX_BYTES ((size_t)32 << 20)
gdr_status gdr_prefill_chunked_noalloc(enum gdr_dtype dt, enum gdr_gate gk, int B, int T,
                                       int H, int Dk, int Dv, int chunk, float scale,
                                       const void *q, const void *k, const void *v,
                                       const float *g, const float *beta, const float *h0,
                                       void *o, float *ht, void *stream);

/*
 * Chunked prefill over a packed variable-length batch.  Sequence n owns
 * tokens [cu_seqlens[n], cu_seqlens[n+1]) of the packed axis; its state
 * starts at h0[n] (zeros if h0 is NULL) and nothing crosses a boundary.
 * Chunks start at each sequence's own first token.
 *
 *   N                 number of sequences (>= 0)
 *   T_total           packed tokens (== cu_seqlens[N])
 *   cu_seqlens        device int32 [N+1], non-decreasing, cu_seqlens[0] == 0
 *   cu_seqlens_host   host copy of cu_seqlens, optional (NULL): when given
 *                     it is validated on the host before launching
 *   q, k              [T_total, H, Dk]   v, o [T_total, H, Dv]
 *   g                 [T_total, H] or [T_total, H, Dk] fp32;  beta [T_total, H]
 *   h0, ht            [N, H, Dv, Dk] fp32 (h0 may be NULL, ht may be NULL)
 *   workspace         device buffer, 16-byte aligned, of at least
 *                     gdr_prefill_workspace_bytes(dt, gk, N, T_total, H)
 *                     bytes; the call writes its schedule (longest sequence
 *                     first), the chunk offsets and (bf16, scalar gate) the
 *                     chunk-local matrices there; it must not be shared with
 *                     a concurrent call
 * Other arguments as gdr_prefill_chunked.  Only bf16 runs chunked; fp32
 * runs the recurrent form.  Without cu_seqlens_host, device offsets that
 * violate the rules above give undefined results.
 */
gdr_status gdr_prefill_chunked_varlen(enum gdr_dtype dt, enum gdr_gate gk, int N,
                                      int T_total, int H, int Dk, int Dv, int chunk,
                                      float scale, const int32_t *cu_seqlens,
                                      const int32_t *cu_seqlens_host,
                                      const void *q, const void *k, const void *v,
                                      const float *g, const float *beta,
                                      const float *h0, void *o, float *ht,
                                      void *workspace, size_t ws_bytes, void *stream);

/*
 * One decode token for B sequences and H heads: the fused state update.
 * Each (b, h) state is read from HBM once and written once.
 *
 *   q, k   [B, H, Dk] dt;   v [B, H, Dv] dt
 *   g      [B, H] (scalar) or [B, H, Dk] (channel) fp32;  beta [B, H] fp32
 *   state  [B, H, Dv, Dk] fp32, updated in place
 *   o      [B, H, Dv] dt (written)
 */
gdr_status gdr_decode_step(enum gdr_dtype dt, enum gdr_gate gk, int B, int H,
                           int Dk, int Dv, float scale, const void *q,
                           const void *k, const void *v, const float *g,
                           const float *beta, float *state, void *o, void *stream);

/*
 * One decode token through a stack of L layers under a placement: every
 * layer tagged GDR_GDN (scalar gate: reads g[l, b, h, 0]) or GDR_KDA
 * (channel gate: reads g[l, b, h, :]) is stepped with gdr_decode_step's
 * update, all in one launch.  Layers tagged GDR_FA or GDR_SWA are not
 * touched: their slots of state_pool and o keep their bytes.
 *
 *   placement   host uint8 [L], codes gdr_mixer (0..3)
 *   L           layers (1..1024)
 *   q, k        [L, B, H, Dk] dt;  v [L, B, H, Dv] dt
 *   g           [L, B, H, Dk] fp32;  beta [L, B, H] fp32
 *   state_pool  [L, B, H, Dv, Dk] fp32, updated in place for GDN/KDA layers
 *   o           [L, B, H, Dv] dt (written for GDN/KDA layers only)
 */
gdr_status gdr_decode_placement(const uint8_t *placement, int L, enum gdr_dtype dt,
                                int B, int H, int Dk, int Dv, float scale,
                                const void *q, const void *k, const void *v,
                                const float *g, const float *beta,
                                float *state_pool, void *o, void *stream);

/*
 * Serving forms.  A serving loop keeps every live request's states in one
 * pool and refers to them by slot; a placement can change from one request
 * to the next (abstract; summary section 2d), so a request's layers are
 * addressed per call.  The shared checkpoint also drafts tokens for
 * speculative decoding with a cheaper placement (abstract; summary section
 * 2d; "Component-Aware Self-Speculative Decoding in Hybrid Language Models",
 * abstract, on linear-attention layers as the draft): the verifier needs
 * the state after each drafted token so that the state after the accepted
 * prefix can be kept.
 */

/*
 * Packed-batch prefill whose initial and final states live in a
 * slot-indexed pool: sequence n starts from state_pool[h0_slot[n]] and its
 * final state is written to state_pool[ht_slot[n]].  Slot -1 (any value
 * outside 0..pool_slots-1) means: start from zeros / do not store.
 * h0_slot[n] == ht_slot[n] continues a request in place.
 *
 *   pool_slots        slots in the pool (>= 0)
 *   state_pool        [pool_slots, H, Dv, Dk] fp32
 *   h0_slot, ht_slot  device int32 [N], both required
 *   h0_slot_host, ht_slot_host
 *                     host copies, optional (NULL): when both are given
 *                     they are validated first -- values in -1..pool_slots-1,
 *                     no slot written by two sequences, no slot read by one
 *                     sequence and written by another (such calls race;
 *                     without the host copies their result is undefined)
 * Other arguments, the workspace and the numerics as
 * gdr_prefill_chunked_varlen.
 */
gdr_status gdr_prefill_varlen_pool(enum gdr_dtype dt, enum gdr_gate gk, int N,
                                   int T_total, int H, int Dk, int Dv, int chunk,
                                   float scale, const int32_t *cu_seqlens,
                                   const int32_t *cu_seqlens_host,
                                   const void *q, const void *k, const void *v,
                                   const float *g, const float *beta, int pool_slots,
                                   float *state_pool, const int32_t *h0_slot,
                                   const int32_t *ht_slot, const int32_t *h0_slot_host,
                                   const int32_t *ht_slot_host, void *o,
                                   void *workspace, size_t ws_bytes, void *stream);

/*
 * n_tok decode tokens for each of B sequences in one launch: gdr_decode_step's
 * update applied to tokens 0 .. n_tok-1 in order, with each state read from
 * HBM once.  Sequence b's state is state_pool[slot[b]] (slot[b] = b when
 * slot is NULL); a slot outside 0..pool_slots-1 marks an idle sequence:
 * nothing of it is read or written.
 *
 *   q, k          [B, n_tok, H, Dk] dt;  v, o [B, n_tok, H, Dv] dt
 *   g             [B, n_tok, H] (scalar) or [B, n_tok, H, Dk] (channel) fp32
 *   beta          [B, n_tok, H] fp32
 *   slot          device int32 [B] or NULL (then pool_slots >= B)
 *   slot_host     host copy of slot, optional: validated first (values in
 *                 -1..pool_slots-1, no slot used twice; two sequences on one
 *                 slot race, and without the host copy the result is
 *                 undefined)
 *   state_pool    [pool_slots, H, Dv, Dk] fp32
 *   checkpoints   [B, n_tok, H, Dv, Dk] fp32 or NULL.  NULL: the state after
 *                 the last token replaces the pool's.  Given: the state after
 *                 token t is written to checkpoints[b, t] and the pool keeps
 *                 its bytes (see gdr_decode_commit).  Must not overlap the
 *                 pool.
 */
gdr_status gdr_decode_tokens(enum gdr_dtype dt, enum gdr_gate gk, int B, int n_tok, int H,
                             int Dk, int Dv, float scale, const void *q, const void *k,
                             const void *v, const float *g, const float *beta,
                             const int32_t *slot, const int32_t *slot_host,
                             int pool_slots, float *state_pool, float *checkpoints,
                             void *o, void *stream);

/*
 * Keep the state after the accepted prefix of a checkpointed
 * gdr_decode_tokens call: for 1 <= accepted[b] <= n_tok the pool slot of
 * sequence b receives checkpoints[b, accepted[b] - 1]; any other count (0:
 * every drafted token rejected) leaves it unchanged.  slot, pool_slots,
 * B, n_tok, H, Dk, Dv as in that call; accepted is device int32 [B].
 */
gdr_status gdr_decode_commit(int B, int n_tok, int H, int Dk, int Dv, const int32_t *slot,
                             int pool_slots, const int32_t *accepted,
                             const float *checkpoints, float *state_pool, void *stream);

/*
 * Fused input preprocessing.  A layer's projections reach the mixer raw: q
 * and k before their L2 normalisation, and logits for beta and the gate.
 * These calls take them as they are and form the recurrence inputs inside
 * the kernels, per token and head, in fp32:
 *
 *     q <- q / sqrt(|q|^2 + 1e-6),   k likewise,
 *     beta = 1 / (1 + exp(-beta_logit)),
 *     g = ln a = -gate_scale * ln(1 + exp(gate_logit)).
 *
 * gate_logit and beta_logit are in the dtype of q (bf16 or fp32), laid out as
 * g and beta of the plain calls (gate_logit [.., H] for GDR_GATE_SCALAR,
 * [.., H, Dk] for GDR_GATE_CHANNEL).  gate_scale >= 0 (GDR_EINVAL
 * otherwise).  The pages give no preprocessing; these three are the usual
 * forms of the operations, and taking them inside the kernels saves the
 * separate passes over q, k and the gate, and halves the gate bytes of a
 * bf16 caller.  Everything else -- layouts, h0/ht, aliasing, numerics of the
 * recurrence, errors -- is as in the plain call named.
 */

/* Workspace of the fused prefill calls: as gdr_prefill_workspace_bytes, with
 * 6144-byte chunk records (the key norms folded into two more factor rows). */
size_t gdr_prefill_fused_workspace_bytes(enum gdr_dtype dt, enum gdr_gate gk, int N,
                                         long long tokens, int H);

/* gdr_prefill_chunked on raw projections (workspace: the size above). */
gdr_status gdr_prefill_chunked_fused(enum gdr_dtype dt, enum gdr_gate gk, int B, int T,
                                     int H, int Dk, int Dv, int chunk, float scale,
                                     const void *q, const void *k, const void *v,
                                     const void *gate_logit, const void *beta_logit,
                                     float gate_scale, const float *h0, void *o, float *ht,
                                     void *workspace, size_t ws_bytes, void *stream);

/* gdr_prefill_chunked_varlen on raw projections (workspace: the size above). */
gdr_status gdr_prefill_varlen_fused(enum gdr_dtype dt, enum gdr_gate gk, int N,
                                    int T_total, int H, int Dk, int Dv, int chunk,
                                    float scale, const int32_t *cu_seqlens,
                                    const int32_t *cu_seqlens_host, const void *q,
                                    const void *k, const void *v, const void *gate_logit,
                                    const void *beta_logit, float gate_scale,
                                    const float *h0, void *o, float *ht, void *workspace,
                                    size_t ws_bytes, void *stream);

/* gdr_decode_tokens on raw projections. */
gdr_status gdr_decode_tokens_fused(enum gdr_dtype dt, enum gdr_gate gk, int B, int n_tok,
                                   int H, int Dk, int Dv, float scale, const void *q,
                                   const void *k, const void *v, const void *gate_logit,
                                   const void *beta_logit, float gate_scale,
                                   const int32_t *slot, const int32_t *slot_host,
                                   int pool_slots, float *state_pool, float *checkpoints,
                                   void *o, void *stream);

/*
 * Backward of the chunked prefill, for training (the pages train the
 * supernet by distillation and then fine-tuning, summary section 2b).  For a
 * fixed-length batch and the upstream gradients d_o (of o) and dht (of the
 * final states), returns the gradients of every input of gdr_prefill_chunked:
 * the vector-Jacobian product of the recurrence stated at the top of this
 * header.
 *
 *   dt, gk, B, T, H, Dk, Dv, chunk, scale, q, k, v, g, beta, h0
 *                as gdr_prefill_chunked (dt must be GDR_BF16)
 *   d_o          [B, T, H, Dv] bf16: gradient of o
 *   dht          [B, H, Dv, Dk] fp32 or NULL (zero)
 *   dq, dk       [B, T, H, Dk] fp32 (written)
 *   dv           [B, T, H, Dv] fp32 (written)
 *   dg           like g, fp32 (written);  dbeta [B, T, H] fp32 (written)
 *   dh0          [B, H, Dv, Dk] fp32 (written) or NULL
 *   workspace    device buffer of gdr_backward_workspace_bytes(gk, B, T, H,
 *                Dk, Dv) bytes (the state entering and the state gradient
 *                leaving every chunk of 64 tokens in fp32, the forward's
 *                workspace -- the forward stores no outputs -- and per chunk
 *                the bf16 matrices of the state gradient's recurrence),
 *                16-byte aligned
 *
 * Three stages: the chunked forward storing the state that enters every
 * chunk; the state gradient's recurrence over chunks in reverse (its
 * chunk-local matrices first, all chunks in parallel), storing each chunk's
 * state gradient and dh0; and one MFMA workgroup per (chunk, head) for the
 * chunk-local gradients.  fp32 inputs are GDR_EUNSUPPORTED.
 * Numerics: bf16 operands with fp32 accumulation, as the forward.
 * Range: every gate g in [-inf, 0]; g is raised to -30 as in the forward.
 * The chunk-local gradients factor each chunk from its first token, which
 * holds while every gate channel decays by at most e^80 over the chunk; the
 * forward marks each (sequence, head) with a chunk that decays further, and
 * all gradients of the marked pairs are then recomputed by the adjoint of
 * the token recurrence in fp32 from the stored chunk-entering states (about
 * 11 to 12 times the in-range cost for a batch where every pair is marked).  The
 * results are the same bits on every run except dg and dbeta of in-range
 * pairs, which are summed in LDS float atomics (equal to fp32 rounding).
 */
size_t gdr_backward_workspace_bytes(enum gdr_gate gk, int B, int T, int H, int Dk, int Dv);

gdr_status gdr_backward_chunked(enum gdr_dtype dt, enum gdr_gate gk, int B, int T, int H,
                                int Dk, int Dv, int chunk, float scale, const void *q,
                                const void *k, const void *v, const float *g,
                                const float *beta, const float *h0, const void *d_o,
                                const float *dht, float *dq, float *dk, float *dv, float *dg,
                                float *dbeta, float *dh0, void *workspace, size_t ws_bytes,
                                void *stream);

/*
 * The same backward for a packed batch of N variable-length sequences (the
 * layout of gdr_prefill_chunked_varlen): the gradients of every input of
 * that call.
 *
 *   dt, gk, N, T_total, H, Dk, Dv, chunk, scale, cu_seqlens,
 *   cu_seqlens_host, q, k, v, g, beta, h0
 *                as gdr_prefill_chunked_varlen (dt must be GDR_BF16)
 *   d_o          [T_total, H, Dv] bf16: gradient of o
 *   dht          [N, H, Dv, Dk] fp32 or NULL (zero)
 *   dq, dk, dv   [T_total, H, D] fp32 (written)
 *   dg, dbeta    like g and beta, fp32 (written)
 *   dh0          [N, H, Dv, Dk] fp32 (written) or NULL; an empty sequence's
 *                dh0 is its dht
 *   workspace    device buffer of gdr_backward_varlen_workspace_bytes(gk, N,
 *                T_total, H, Dk, Dv) bytes (as the fixed-length form's, sized
 *                for T_total / 64 + N chunks), 16-byte aligned
 *
 * The sequences' chunks are numbered one after the other on the device
 * (from cu_seqlens); the forward runs longest sequence first, the state
 * gradient's recurrence walks each (sequence, head) in reverse, and the
 * chunk-local gradients take one workgroup per (chunk, head) as in the
 * fixed-length form.
 */
size_t gdr_backward_varlen_workspace_bytes(enum gdr_gate gk, int N, long long tokens, int H,
                                           int Dk, int Dv);

gdr_status gdr_backward_chunked_varlen(enum gdr_dtype dt, enum gdr_gate gk, int N, int T_total,
                                       int H, int Dk, int Dv, int chunk, float scale,
                                       const int32_t *cu_seqlens, const int32_t *cu_seqlens_host,
                                       const void *q, const void *k, const void *v,
                                       const float *g, const float *beta, const float *h0,
                                       const void *d_o, const float *dht, float *dq, float *dk,
                                       float *dv, float *dg, float *dbeta, float *dh0,
                                       void *workspace, size_t ws_bytes, void *stream);

/* Thread-local text describing the last non-OK status of this thread. */
const char *gdr_last_error(void);

/* Library version string. */
const char *gdr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
