/*
 * attn.h - C ABI of the exact tiled-softmax attention library (libattn.so)
 * for AMD Instinct MI355X (gfx950).
 *
 * Every entry point computes exact softmax attention (no approximation):
 *
 *   S = scale * Q K^T,  P = row-softmax(S with blocked keys removed),
 *   O = P V,            LSE_i = log(sum_j exp(S_ij))   (natural log)
 *
 * as defined in "The Hidden Recurrence in Softmax Attention: A Path to Flash
 * Attention", section "Standard Attention / Forward Pass", and "attention
 * backprop", section "Forward Pass" (the 1/sqrt(head_dim) scale is the caller's
 * `scale` argument here).  The forward kernels never build S: they visit K/V
 * block by block and keep, per query row, a running max m, a running sum l and
 * an accumulator a that are rescaled whenever the max grows ("The Hidden
 * Recurrence in Softmax Attention", section "Chunk-wise Mode with Online
 * Softmax Re-scale"; "Tiled attention with an online softmax", section
 * "Task").  The backward kernels recompute P from the stored LSE instead of
 * storing it ("The Hidden Recurrence in Softmax Attention", section "Flash
 * Attention Backward Pass", closing comment) and apply the gradients of
 * "attention backprop", sections "Gradient of V and P", "Gradient of S" and
 * "Gradient of Q and K".
 *
 * Conventions shared by all entry points
 * --------------------------------------
 * Layout.   Tensors are contiguous, row-major [B, H, T, dim] ("attention
 *           backprop", section "Forward Pass": batch, heads, sequence, head
 *           dim): q [B,H,Tq,d], k [B,H,Tk,d], v [B,H,Tk,dv], o/dout
 *           [B,H,Tq,dv], lse [B,H,Tq] (fp32 in every variant).
 * Pointers. Device pointers (memory of the GPU that is current on the calling
 *           thread).  The caller owns every buffer.  Inputs are const and never
 *           written ("Tiled attention with an online softmax", section
 *           "Constraints": inputs are not changed).  Outputs are overwritten in
 *           full, never accumulated into.  Outputs must not alias inputs.
 * Mask.     causal != 0 blocks key j for query i when j > i, on global row
 *           indices ("Tiled attention with an online softmax", section
 *           "Task"); with Tq != Tk this is top-left alignment.  causal == 0
 *           blocks nothing.  A blocked key contributes exactly zero, like a
 *           score of -infinity.
 * Scale.    `scale` multiplies Q K^T; callers normally pass 1/sqrt(d).  It
 *           must be finite and >= 0.
 * Values.   Every element of q, k, v and dout (and o, lse, dlse passed to a
 *           backward, as a forward returned them) must be finite.  A score of
 *           -infinity arises only from the mask, where a blocked key counts
 *           as a score of -infinity ("Tiled attention with an online
 *           softmax", section "Task").  NaN or infinite inputs are outside the
 *           domain: the bf16 forward kernels are compiled without NaN
 *           semantics (a row maximum may then ignore a NaN score), so such
 *           inputs give unspecified outputs, never an error code.  Nothing
 *           reads the inputs on the host to check this.
 * Sizes.    B, H, Tq, Tk, d, dv >= 1, with B*H <= 2^31/8 - 1 and B*H*Tq and
 *           B*H*Tk each <= 2^31 - 1 (row counts, not element counts: element
 *           offsets are 64-bit inside); otherwise ATTN_ERR_INVALID_ARG.
 * Empty rows. A query row with no allowed key gets O = 0 and LSE = -inf
 *           (the page's step leaves such a row at m = -inf, l = 0, a = 0).
 *           With causal top-left masking and Tk >= 1 this never happens.
 * Stream.   `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *           enqueue work on it and never synchronise; kernel faults surface at
 *           the caller's next synchronisation on that stream.
 * Workspace. Some calls need scratch memory (row statistics of the
 *           backward, split partial states).  The library takes it with
 *           hipMallocFromPoolAsync on `stream` from a memory pool of its own
 *           (one per device, created at the first such call, kept until the
 *           process ends, caching up to 256 MiB of freed memory across
 *           synchronisations) and returns it with hipFreeAsync on the same
 *           stream, so its lifetime is stream-ordered and no data persists
 *           between calls.
 * Errors.   Return 0 on success or a negative ATTN_ERR_* code.  Argument
 *           checks happen before any HIP call, so an invalid call has no
 *           effect.  No C++ exception crosses this interface.
 * Threads.  Calls on different streams may run concurrently.
 */
#ifndef EXACT_TILED_SOFTMAX_ATTN_H
#define EXACT_TILED_SOFTMAX_ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_OK 0
#define ATTN_ERR_INVALID_ARG (-1) /* null pointer, dimension < 1, bad scale, bad block size */
#define ATTN_ERR_UNSUPPORTED (-2) /* head dims the bf16 kernels are not built for */
#define ATTN_ERR_HIP (-3)         /* a HIP launch or allocation failed */
#define ATTN_ERR_TOO_LARGE (-4)   /* attn_bwd_noalloc: workspace larger than its static scratch */

/*
 * attn_fwd - bf16 forward.
 *   q, k, v : bf16 inputs (layout above).
 *   o       : bf16 output [B,H,Tq,dv], O = P V rounded to nearest even.
 *   lse     : fp32 output [B,H,Tq], natural-log log-sum-exp of the scaled,
 *             masked scores ("Tiled attention with an online softmax",
 *             section "Task": log-sum-exp = m + log l).
 * Arithmetic: bf16 MFMA products with fp32 accumulation; the online softmax
 * statistics are fp32; P is rounded to bf16 before the P V product.
 * Supported: d == dv, d in {64, 128}; otherwise ATTN_ERR_UNSUPPORTED.
 * B, H, Tq, Tk >= 1 within the size limits above; ragged tails are masked.
 * Workspace: none, except the partial states when the key range is split
 * (num_splits*B*H*Tq*(dv+2) floats).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Tq, int Tk, int d, int dv, float scale, int causal,
             void* stream);

/*
 * attn_fwd_splits - attn_fwd with an explicit number of key-range splits.
 *   num_splits: 0 lets the library choose (what attn_fwd does); n >= 1 splits
 *   each row's key range into n contiguous chunks processed by separate
 *   workgroups whose partial states (m, l, a) are merged afterwards with the
 *   same rescale rule ("The Hidden Recurrence in Softmax Attention", section
 *   "Chunk-wise Mode with Online Softmax Re-scale").  Values above the number
 *   of 64-key blocks are clamped.  Other arguments as attn_fwd.
 */
int attn_fwd_splits(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Tq, int Tk, int d, int dv, float scale, int causal,
                    int num_splits, void* stream);

/*
 * attn_bwd - bf16 backward.
 *   q, k, v, o, lse : the forward's inputs and outputs (o bf16, lse fp32).
 *   dout            : bf16 gradient of the loss with respect to O.
 *   dq, dk, dv_grad : bf16 outputs with the shapes of q, k, v.
 * Computes, per (b, h), with P recomputed as exp(S - LSE):
 *   D_i = sum_c dout_ic o_ic            ("attention backprop", "Gradient of S")
 *   dV  = P^T dout                      ("attention backprop", "Gradient of V and P")
 *   dS  = P o (dout V^T - D)            ("attention backprop", "Gradient of S")
 *   dQ  = scale dS K,  dK = scale dS^T Q ("attention backprop", "Gradient of Q and K",
 *                                         with the chain-rule factor of `scale`)
 * dK, dV come from one kernel that walks the queries of each key block and
 * dQ from another that walks the keys of each query block, so every output
 * element is summed in a fixed order by one workgroup: results are
 * deterministic.  Workspace (row statistics, about B*H*Tq*8 bytes, and,
 * when the dQ kernel splits the key range because there are few query
 * blocks, fp32 partial dQ of splits*B*H*Tq*d*4 bytes) comes from the
 * library's workspace pool on `stream` (see Workspace above).
 * Supported: d == dv, d in {64, 128}; otherwise ATTN_ERR_UNSUPPORTED.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv_grad,
             int B, int H, int Tq, int Tk, int d, int dv, float scale, int causal,
             void* stream);

/*
 * attn_bwd_noalloc - attn_bwd that allocates nothing: for callers that cannot
 * allocate device memory during the call (code under HIP graph capture,
 * tight training or serving loops, harnesses that forbid hipMalloc).
 *   Arguments, layouts, results and supported sizes as attn_bwd.  Its
 *   workspace (row statistics and, for few query blocks against many keys,
 *   fp32 partial dQ of the key-range splits) lives in a static scratch array
 *   of ATTN_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU
 *   it runs on until the process ends; nothing in it needs clearing (every
 *   call overwrites what it reads).  The split count is attn_bwd's when its
 *   partials fit, else the largest that fits (the summation order of dQ, and
 *   so its last bits, can then differ from attn_bwd's).
 *   ATTN_ERR_TOO_LARGE (checked before any HIP call) when not even the row
 *   statistics fit: about B*H*Tq*8 bytes, i.e. B*H*Tq above about 8.4 million
 *   rows.  The first call on a device looks up the device address of that
 *   device's copy (hipGetSymbolAddress) and keeps it.
 *   Calls on one GPU share its scratch: two calls whose work overlaps in time
 *   on one GPU (different streams, or host threads) race and corrupt each
 *   other's gradients; serialise them on one stream.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv_grad,
                     int B, int H, int Tq, int Tk, int d, int dv, float scale, int causal,
                     void* stream);

/*
 * attn_bwd_dlse - attn_bwd with an upstream gradient on the LSE output.
 *   dlse : fp32 [B,H,Tq], d(loss)/d(LSE_i) (required; NULL is
 *          ATTN_ERR_INVALID_ARG).  Other arguments as attn_bwd.
 * LSE_i = m_i + log l_i, and gradients flow through the row sum l ("The
 * Hidden Recurrence in Softmax Attention", sections "Flash Attention Backward
 * Pass" and "Gradient at the Output"); with d LSE_i / d S_ij = P_ij the
 * gradient of the scores becomes dS = P o (dP - D + dlse): D_i is replaced by
 * D_i - dlse_i.
 * This lets a caller that merged key-range states (attn_merge_states)
 * propagate a gradient through the merged LSE.
 */
int attn_bwd_dlse(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const float* dlse, const void* dout, void* dq, void* dk, void* dv_grad,
                  int B, int H, int Tq, int Tk, int d, int dv, float scale, int causal,
                  void* stream);

/*
 * attn_fwd_state - the unnormalised online-softmax state of one key range
 * ("Tiled attention with an online softmax", section "Task": a row's state is
 * its running max m, running sum l and accumulator a; "The Hidden Recurrence
 * in Softmax Attention", section "Chunk-wise Mode with Online Softmax
 * Re-scale": states of separate key chunks combine by rescaling to a common
 * max, see attn_merge_states).
 *   q [B,H,Tq,d], k [B,H,Tk,d], v [B,H,Tk,dv] : bf16, this call's queries and
 *             this key range (layout as above).
 *   acc       : fp32 output [B,H,Tq,dv], a_i = sum_j exp(s_ij - m_i) v_j over
 *               the allowed keys j (exp(s - m) rounded to bf16 in the product
 *               with v, as in attn_fwd).
 *   m         : fp32 output [B,H,Tq], natural-log units: a reference value at
 *               most 8 ln 2 (about 5.55) below the largest allowed scaled
 *               score s_ij = scale q_i.k_j of row i and not above it (the
 *               library moves its reference lazily); -inf if row i has no
 *               allowed key in this range.
 *   l         : fp32 output [B,H,Tq], l_i = sum_j exp(s_ij - m_i) (0 if none).
 *   a_i / l_i and m_i + ln l_i do not depend on which reference m_i is used.
 *   q_offset, k_offset : >= 0, global positions of this call's first query and
 *               first key; with causal != 0, key j is blocked for query i when
 *               k_offset + j > q_offset + i (the top-left rule of attn_fwd on
 *               global indices).  Ignored when causal == 0.
 * Supported: d == dv, d in {64, 128}.  Workspace: none, except without the
 * causal mask when the query tiles alone would leave the chip under-filled
 * (few queries, many keys): then the key range is computed in splits, as in
 * attn_fwd, whose partial states (splits*B*H*Tq*(dv+2) floats, from the
 * library's workspace pool on `stream`) are merged into acc, m, l by the rule
 * of attn_merge_states.
 */
int attn_fwd_state(const void* q, const void* k, const void* v, float* acc, float* m, float* l,
                   int B, int H, int Tq, int Tk, int d, int dv, float scale, int causal,
                   int q_offset, int k_offset, void* stream);

/*
 * attn_merge_states - O and LSE from n partial states of the same queries
 * (the rescale rule of "The Hidden Recurrence in Softmax Attention", section
 * "Chunk-wise Mode with Online Softmax Re-scale"):
 *   M = max_s m_s,  l = sum_s exp(m_s - M) l_s,  a = sum_s exp(m_s - M) a_s,
 *   O = a / l (bf16, 0 where l = 0),  LSE = M + ln l (-inf where l = 0).
 *   acc [n,B,H,Tq,dv], m [n,B,H,Tq], l [n,B,H,Tq] : fp32 inputs, state s at
 *               index s (as written by attn_fwd_state).
 *   o [B,H,Tq,dv] bf16 and lse [B,H,Tq] fp32 : outputs.
 *   n >= 1; dv in {64, 128} (else ATTN_ERR_UNSUPPORTED).
 */
int attn_merge_states(const float* acc, const float* m, const float* l, int n, void* o, float* lse,
                      int B, int H, int Tq, int dv, void* stream);

/*
 * attn_fwd_standard - standard attention with the score matrix materialised
 * in HBM ("The Hidden Recurrence in Softmax Attention", section "Standard
 * Attention / Forward Pass"): S = scale Q K^T (fp32, blocked keys -inf), the
 * row softmax P (bf16) with LSE, then O = P V, each step a kernel of its own.
 * Same arguments, outputs and supported sizes as attn_fwd; the results agree
 * with attn_fwd to bf16 rounding.  For measuring what the tiled method saves:
 * it takes a workspace of about B*H*Tq*Tk*6 bytes (S in fp32 and P in bf16)
 * from the library's workspace pool on `stream` (ATTN_ERR_HIP if that
 * fails) and moves
 * Tq*Tk*12 bytes per head through HBM.
 */
int attn_fwd_standard(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Tq, int Tk, int d, int dv, float scale, int causal, void* stream);

/*
 * attn_decode - the newest Tq queries of each sequence against its key/value
 * cache (the recurrent mode of "The Hidden Recurrence in Softmax Attention",
 * section "Recurrent mode": the query of step t attends to the keys of steps
 * up to t; computed as the exact softmax with a running max, "Tiled attention
 * with an online softmax", section "Task").
 *   q       : bf16 [B,H,Tq,d], the Tq newest queries of each sequence.
 *   k, v    : bf16 [B,H,Tk,d] and [B,H,Tk,dv], Tk cache slots per (b, h);
 *             sequence b uses slots 0 .. L_b-1.
 *   kv_lens : device int32 [B] holding L_b, or NULL for L_b = Tk.  Values are
 *             read on the device and clamped to [0, Tk]; slots at L_b and
 *             beyond are never read.
 *   o, lse  : bf16 [B,H,Tq,dv] and fp32 [B,H,Tq] outputs.
 * Query i of sequence b sits at position L_b - Tq + i.  causal != 0: key j is
 * blocked for it when j > L_b - Tq + i (so the newest query sees every cached
 * key and query i the keys up to its own position); causal == 0: every key
 * j < L_b is allowed.  A query with no allowed key gets o = 0, lse = -inf.
 * 1 <= Tq <= ATTN_DECODE_MAX_QUERIES and d == dv in {64, 128}, else
 * ATTN_ERR_UNSUPPORTED.  The key range is split over workgroups; with more
 * than one split the partial states are merged with the rescale rule
 * ("Chunk-wise Mode with Online Softmax Re-scale"), using a workspace of
 * splits*B*H*Tq*(dv+2) floats from the library's workspace pool on `stream`.
 */
#define ATTN_DECODE_MAX_QUERIES 4
int attn_decode(const void* q, const void* k, const void* v, const int* kv_lens, void* o, float* lse,
                int B, int H, int Tq, int Tk, int d, int dv, float scale, int causal, void* stream);

/*
 * attn_decode_splits - attn_decode with an explicit number of key-range splits
 * (0: the library's choice, as attn_decode; values above the number of
 * row batches per sequence are clamped).  Other arguments as attn_decode.
 */
int attn_decode_splits(const void* q, const void* k, const void* v, const int* kv_lens, void* o, float* lse,
                       int B, int H, int Tq, int Tk, int d, int dv, float scale, int causal, int num_splits,
                       void* stream);

/*
 * attn_fwd_f32 - fp32 forward that follows the page's block loop literally:
 * keys are taken in blocks of `block_n` starting at 0, block_n, 2*block_n, ...
 * (the last may be shorter) and each block updates (m, l, a) with one online
 * softmax step ("Tiled attention with an online softmax", section "Task").
 *   block_n: 1..1024, or 0 for the default of 64.  Any block size gives the
 *   same result up to fp32 rounding (section "Constraints").
 * All tensors fp32.  1 <= d, dv <= 128.
 */
int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                 int B, int H, int Tq, int Tk, int d, int dv, float scale, int causal,
                 int block_n, void* stream);

/*
 * attn_fwd_f32_unrescaled - the chunk-wise mode of "The Hidden Recurrence in
 * Softmax Attention" (section "Chunk-wise Mode") before the rescale of the
 * following section: the block loop of attn_fwd_f32 with no running max,
 *   l += sum_j exp(s_ij),  a += sum_j exp(s_ij) v_j,  o = a / l,  lse = log l.
 * A NEGATIVE CONTROL, not a path to use: fp32 exp overflows once a score
 * exceeds about 88.7, and such rows come out inf or nan (attn_fwd_f32 stays
 * finite on the same input).  Arguments, layouts and errors as attn_fwd_f32.
 */
int attn_fwd_f32_unrescaled(const float* q, const float* k, const float* v, float* o, float* lse,
                            int B, int H, int Tq, int Tk, int d, int dv, float scale, int causal,
                            int block_n, void* stream);

/*
 * attn_bwd_f32 - fp32 backward (same formulas as attn_bwd, fp32 throughout,
 * deterministic, no workspace).  All tensors fp32.  1 <= d, dv <= 128.
 */
int attn_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* lse,
                 const float* dout, float* dq, float* dk, float* dv_grad,
                 int B, int H, int Tq, int Tk, int d, int dv, float scale, int causal,
                 void* stream);

/*
 * Kernel timing with HIP events (measurement support, not part of the math).
 * While profiling is on, every kernel the library launches is bracketed by a
 * pair of hipEvents recorded on the stream it is launched on; the elapsed
 * times are summed per kernel kind.  Recording adds two event records per
 * launch and no synchronisation.
 *   attn_profile_start()  clear the totals and turn recording on
 *   attn_profile_stop()   turn recording off (recorded pairs are kept)
 *   attn_profile_query(kind, &total_ms, &launches)
 *       wait for the recorded events of `kind` (ATTN_KERNEL_*), add their
 *       durations to the totals and return them.  ATTN_ERR_INVALID_ARG for
 *       an unknown kind or null pointers, ATTN_ERR_HIP if an event fails.
 */
#define ATTN_KERNEL_FWD 0            /* forward main kernel */
#define ATTN_KERNEL_FWD_AUX 1        /* forward: merge of key-split states (attn_fwd, attn_decode) */
#define ATTN_KERNEL_BWD_PREP 2       /* (no longer launched: the dQ kernel forms the row statistics) */
#define ATTN_KERNEL_BWD_DKDV 3       /* backward: dK and dV */
#define ATTN_KERNEL_BWD_DQ 4         /* backward: dQ */
#define ATTN_KERNEL_DECODE 5         /* decode main kernel (its split merge counts as ATTN_KERNEL_FWD_AUX) */
#define ATTN_KERNEL_STANDARD 6       /* attn_fwd_standard: its kernels together */
#define ATTN_KERNEL_KINDS 7
int attn_profile_start(void);
int attn_profile_stop(void);
int attn_profile_query(int kind, double* total_ms, int* launches);

/* attn_strerror - static description of a return code (never NULL). */
const char* attn_strerror(int code);

/* attn_last_hip_error - the hipError_t value behind the most recent
 * ATTN_ERR_HIP returned on the calling thread (0 if none). */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_TILED_SOFTMAX_ATTN_H */
