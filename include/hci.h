/*
 * hci.h -- C ABI of libhci: replay-free block verification for one hybrid
 * convolutional-recurrent-attention layer on AMD MI355X (gfx950).
 *
 * The method is the one summarised in "EvSpark: Lossless Speculative Decoding
 * for Hybrid DNA Foundation Models" (ai4snews digest): the target verifies the
 * old anchor and gamma drafts in ONE initial-state block forward
 * (Interpretation; Figure 1(c)), decides losslessly how many drafts to keep
 * (Figure 1(c): a sampled correction becomes the next anchor), and then
 * restores all three state classes -- finite FIR windows, modal IIR state,
 * attention KV cache -- by selecting retained intermediate values instead of
 * replaying the accepted tokens (Figure 1(d); Interpretation).  The acceptance
 * rules are the greedy rule of the ReaDy summary section 3.1 and the
 * speculative-sampling rule of its section D.2.
 *
 * General conventions (all calls):
 *  - Every pointer is a DEVICE pointer unless said otherwise, owned by the
 *    caller, and must stay valid until the work enqueued on `stream` has run.
 *    The library never allocates, frees or keeps a pointer after returning.
 *  - Every call is asynchronous on `stream` and never synchronises the host.
 *  - Return value: HCI_OK (0) or a negative HCI_E* code.  All argument checks
 *    run on the host before anything is enqueued, so a failed call enqueues
 *    nothing.  HCI_EDEVICE reports a launch error from the HIP runtime.
 *  - Sizes: nb sequences, nc candidate blocks per sequence, gamma drafts,
 *    P = gamma + 1 block positions (position 0 is the anchor), d channels,
 *    Ts / To short / outer FIR taps, N poles per channel, H heads of Dh,
 *    V vocabulary entries.  "act" is the activation dtype of the layer
 *    (HCI_F32 or HCI_BF16); bf16 values are raw 16-bit patterns.
 *  - Arrays are dense, row-major in the order their dimensions are listed.
 */
#ifndef HCI_H
#define HCI_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status */
#define HCI_OK            0
#define HCI_EINVAL       -1  /* null/misaligned pointer, bad dimension, bad mode */
#define HCI_ECAPACITY    -2  /* max_kv_len + gamma + 1 > kv_cap */
#define HCI_EUNSUPPORTED -3  /* dtype or shape this build has no kernel for */
#define HCI_EDEVICE      -4  /* HIP runtime reported an error at launch */
#define HCI_EWORKSPACE   -5  /* workspace missing or smaller than required */

#define HCI_F32  0
#define HCI_BF16 1

#define HCI_GREEDY 0
#define HCI_SAMPLE 1
#define HCI_SAMPLE_RECURSIVE 2

/* Rows of the KV cache are grouped in tiles of this many keys. */
#define HCI_KV_TILE 32

/* Writes the human-readable name of a status code into buf (at most n bytes,
 * always NUL-terminated when n > 0; truncated if it does not fit) and returns
 * the length of the full name without the NUL, as snprintf does, so a call with
 * n = 0 (buf may then be NULL) sizes the buffer.  HCI_EINVAL if buf is NULL
 * and n > 0.  Never touches the device. */
int hci_status_string(int status, char* buf, size_t n);

/* Library ABI version (major * 100 + minor). */
int hci_version(void);

/* ------------------------------------------------------ device status word
 *
 * Host checks cannot see values that live on the device (kv_len, the k and
 * c* that acceptance hands to slicing, the logits).  Kernels that find such a
 * value out of contract OR one of these bits into the caller's status word of
 * that sequence (uint32 per sequence, hci_state.status and the status argument
 * of hci_accept; a NULL pointer disables the reporting but not the guard), so
 * the caller sees it after its next synchronisation.  The bits accumulate until
 * the caller clears them (they are never cleared by the library).  Every kernel
 * still runs to completion; what the guard does instead is stated per bit. */
#define HCI_DS_NONFINITE     0x1u  /* accept: a logit it read is NaN or +Inf, or a row it read has no
                                      finite entry.  The block's n_accepted and next_token are set
                                      to -1 (and best_cand to -1 when no candidate of the sequence
                                      is valid), so slicing then commits nothing for it. */
#define HCI_DS_K_RANGE       0x2u  /* slice: n_accepted of the winning candidate outside [0, gamma];
                                      the sequence's state is left unchanged. */
#define HCI_DS_CAND_RANGE    0x4u  /* slice: best_cand outside [0, nc); state left unchanged. */
#define HCI_DS_KV_LEN        0x8u  /* verify / slice / prefill: kv_len[b] outside [0, max_kv_len].
                                      Verify attends to the clamped length; slice and prefill leave
                                      the sequence's state (windows, IIR state, cache, kv_len)
                                      unchanged. */
#define HCI_DS_DRAFT_ID      0x10u /* accept: a draft token id outside [0, V) (it counted as a
                                      mismatch / rejection, as documented; reported only). */
#define HCI_DS_TREE          0x20u /* token trees: a parent entry breaks 0 <= parent[m] < m
                                      (parent[0] = -1), or the path handed to slicing does not
                                      follow the tree.  Verify reads such an entry as m - 1;
                                      acceptance marks the sequence (n_accepted -1); slicing
                                      leaves it unchanged. */

/* Writes the names of the bits set in `bits` (a status word copied to the
 * host), separated by '|', into buf with the conventions of hci_status_string;
 * "none" when no bit is set. */
int hci_device_status_string(uint32_t bits, char* buf, size_t n);

/* -------------------------------------------------------------- structures */

/* Fixed per-layer parameters.  All weight arrays are fp32 on the device.
 *   w_short [Ts][d]   short depthwise FIR taps, w_short[j] multiplies lag j
 *   w_outer [To][d]   outer depthwise FIR taps, same convention
 *   lambda, beta, c [d][N]   modal IIR poles, input gains and readout gains:
 *       s_i = lambda * s_{i-1} + beta * g_i,   y_i = sum_n c * s_i
 * Limits: d >= 1, Ts >= 1, To >= 1, 1 <= N <= 64, 1 <= H <= 65535,
 *         Dh in {64, 128} (bf16) or Dh in {32, 64, 96, 128} (f32). */
typedef struct hci_layer {
    int d, taps_short, taps_outer, poles, heads, head_dim;
    int act_dtype;                 /* HCI_F32 or HCI_BF16 */
    const float* w_short;
    const float* w_outer;
    const float* lambda;
    const float* beta;
    const float* c;
} hci_layer;

/* Committed (per-sequence) state: the three state classes of the EvSpark
 * digest (Interpretation: finite convolution windows, modal IIR states,
 * attention caches).
 *   short_win [nb][Ts-1][d] act   last Ts-1 short-FIR inputs, oldest first
 *   outer_win [nb][To-1][d] fp32  last To-1 outer-FIR inputs (the u of
 *                                 Figure 1(d)), oldest first
 *   iir       [nb][d][N]    fp32  modal IIR state
 *   k_cache, v_cache              [nb][H][kv_cap/32][32*Dh] act, TILED layout:
 *                                 rows are grouped in tiles of 32 keys whose
 *                                 element order matches the matrix-core
 *                                 operand layout of the attention kernel.
 *                                 Read and write logical rows only through
 *                                 hci_kv_write / hci_kv_read.
 *   kv_len    [nb] int32          readable prefix length of each sequence
 *   kv_cap                        rows per (sequence, head); multiple of 32
 *   status    [nb] uint32         device status words (HCI_DS_* bits), may be
 *                                 NULL; the kernels only OR bits in. */
typedef struct hci_state {
    int kv_cap;
    void* short_win;
    float* outer_win;
    float* iir;
    void* k_cache;
    void* v_cache;
    int32_t* kv_len;
    uint32_t* status;              /* [nb] device status words (HCI_DS_*), or NULL */
} hci_state;

/* One verify round's block: inputs, retained intermediates, outputs.
 *   x [nb][nc][P][d] act            conv-path inputs of the block positions
 *   q, k, v [nb][nc][P][H][Dh] act  attention inputs of the block positions
 *   f [nb][nc][P][d] fp32           OUT of verify: short-FIR outputs
 *                                   (= outer-FIR inputs), read by slice
 *   s [nb][nc][P][d][N] fp32        OUT of verify: IIR state after each
 *                                   position (s_0..s_gamma), read by slice
 *   y [nb][nc][P][d] act            OUT of verify: IIR readout
 *   o [nb][nc][P][H][Dh] act        OUT of verify: attention output
 * x, k and v must stay unchanged between hci_verify_block and
 * hci_slice_state: slicing copies the accepted rows from them. */
typedef struct hci_block {
    const void* x;
    const void* q;
    const void* k;
    const void* v;
    float* f;
    float* s;
    void* y;
    void* o;
} hci_block;

/* ------------------------------------------------------------------ verify */

/* Bytes of workspace hci_verify_block needs for these sizes on the current
 * device: the prefix stream's job-queue counter (256 bytes, reset by the call
 * itself) and the split-K attention partials.  Returns 0 for invalid
 * arguments. */
size_t hci_verify_workspace_bytes(const hci_layer* L, int nb, int nc, int gamma, int max_kv_len);

/* One initial-state block forward over P = gamma + 1 positions for every
 * (sequence, candidate) -- EvSpark digest, Interpretation ("one initial-state
 * block forward") and Figure 1(c).  For each block position i:
 *   f_i = sum_j w_short[j] * xbar[i-j]   (xbar = short_win then x_0..x_i)
 *   g_i = sum_j w_outer[j] * fbar[i-j]   (fbar = outer_win then f_0..f_i)
 *   s_i = lambda * s_{i-1} + beta * g_i,  s_{-1} = iir;  y_i = sum_n c * s_i
 *   o_i[h] = softmax(q_i[h] . keys / sqrt(Dh)) . values over the sequence's
 *            kv_len committed rows followed by block rows 0..i (causal).
 * The candidates of a sequence share its committed state; the committed
 * prefix is read once per sequence for all nc*P queries.
 * Committed state is only read: a round abandoned after verify can be
 * verified again from the same state.
 *   max_kv_len  host-side upper bound on every kv_len[b] (sizes the grid);
 *               must satisfy max_kv_len + gamma + 1 <= kv_cap.  A kv_len[b]
 *               outside [0, max_kv_len] is read clamped into that range and
 *               reported as HCI_DS_KV_LEN in S->status.
 *   ws, ws_bytes  device workspace of at least
 *               hci_verify_workspace_bytes(...) bytes, 256-byte aligned; two
 *               calls in flight at once must not share a workspace.
 * q, k and v must be 16-byte aligned.
 * Limits: gamma >= 0; nc * P <= 64; the conv/IIR scan stages the outer
 * window, taps and block rows of 16 channels in LDS:
 * 16 * 4 * (2*To + 2*Ts + 3*nc*P - 2) bytes <= 160 KiB. */
int hci_verify_block(const hci_layer* L, const hci_state* S, const hci_block* blk,
                     int nb, int nc, int gamma, int max_kv_len,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* hci_verify_block that also records events[0..3] on `stream`: before the
 * first kernel (the set-up kernel: queue counter, work-list table), right
 * before the kernel that streams the KV prefix, right after it, and after the
 * finish kernel (conv/IIR scan, causal block part, merge of the partials), so
 * the caller can time the parts with hipEventElapsedTime -- events[1] to
 * events[2] spans the streaming kernel alone.  events must point at 4 events
 * created by the caller (entries may be NULL to skip one).  Errors as
 * hci_verify_block. */
int hci_verify_block_timed(const hci_layer* L, const hci_state* S, const hci_block* blk,
                           int nb, int nc, int gamma, int max_kv_len,
                           void* ws, size_t ws_bytes, hipStream_t stream, hipEvent_t* events);

/* hci_verify_block for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, results and errors as hci_verify_block, but the workspace is
 * a library-owned device array of HCI_NOALLOC_SCRATCH_BYTES bytes (one per
 * GPU, held until the process ends; its address is looked up once per device).
 * Nothing is allocated or freed by the call.
 *  - HCI_EWORKSPACE (nothing enqueued) when hci_verify_workspace_bytes for
 *    these sizes exceeds HCI_NOALLOC_SCRATCH_BYTES (e.g. one sequence of up to
 *    262144 prefix tokens at 32 or 64 heads of 128 and gamma <= 12 fits; four
 *    sequences of four candidate blocks at 64k tokens do not).
 *  - Every call on a GPU shares that GPU's array: calls whose work overlaps
 *    on one GPU (two streams, or two threads) race and must be ordered by the
 *    caller.  Each call re-initialises the parts it reads first (the queue
 *    counter and the work list), whatever an earlier call left there.
 *  - HCI_EDEVICE if the device's array cannot be located. */
#define HCI_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int hci_verify_block_noalloc(const hci_layer* L, const hci_state* S, const hci_block* blk,
                             int nb, int nc, int gamma, int max_kv_len, hipStream_t stream);

/* ------------------------------------------------------------------ accept */

/* Lossless acceptance for every candidate block, and the best candidate.
 * Row i of target_logits (i = 0..gamma) is the target's prediction for the
 * token after block position i; draft_tokens[..][m-1] is draft t_m.
 *   mode HCI_GREEDY (ReaDy summary, section 3.1): accept the longest prefix
 *     of drafts equal to the target argmax (ties -> lowest id); next token =
 *     argmax of row k (a correction if k < gamma, the bonus if k == gamma).
 *   mode HCI_SAMPLE (ReaDy summary, section D.2; EvSpark Figure 1(c)):
 *     p_m = softmax(target row m / T), q_m = softmax(draft row m-1 / T), both
 *     in fp64; draft t_m is kept iff r_m * q_m(t_m) < p_{m-1}(t_m), checked
 *     left to right, stopping at the first rejection; after a rejection at
 *     m = k+1 the correction is drawn from max(0, p_k - q_{k+1}), after full
 *     acceptance the bonus from p_gamma; a draw takes the smallest token id
 *     whose running sum exceeds r* x (total running sum), else the last
 *     token with positive weight.
 *   mode HCI_SAMPLE_RECURSIVE (lossless over several candidates; the pages
 *     report C = 1/2/4 candidate blocks (EvSpark digest, Interpretation) but
 *     no rule, so this is the published recursive rejection scheme for
 *     multiple drafts): the candidates of a sequence share the anchor; at
 *     depth k the alive candidates (drafts t_1..t_k equal to the accepted
 *     prefix) are tried in index order with the rows p, q of the lowest-index
 *     alive candidate and the running residual w / z (w = p, z = 1 at the
 *     start of a depth): draft t is kept iff r * q(t) * z < w(t), a rejection
 *     sets w <- max(0, w - z q), z <- sum w.  The first kept draft extends
 *     the prefix (candidates holding it stay alive); if all are rejected the
 *     next token is drawn from w, after gamma kept drafts from p_gamma; the
 *     draw uses r* = uniforms[b][0][gamma].  Candidate c's depth-k test uses
 *     uniforms[b][c][k].  With nc = 1 it equals HCI_SAMPLE bit for bit.  The
 *     caller supplies equal rows for candidates that share a prefix, and the
 *     drafts of such candidates are independent draws from q.
 *   Inputs: target_logits [nb][nc][P][V] fp32; draft_logits [nb][nc][gamma][V]
 *     fp32 (the distribution each draft was actually sampled from; NULL in
 *     greedy mode); draft_tokens [nb][nc][gamma] int32 (an id outside [0, V)
 *     counts as a mismatch / rejection); uniforms [nb][nc][P] fp64 in [0, 1):
 *     r_1..r_gamma then r* (NULL in greedy mode).
 *   Outputs: n_accepted [nb][nc] int32 = k; next_token [nb][nc] int32;
 *     best_cand [nb] int32 = candidate with the largest k (lowest index on
 *     ties); in recursive mode n_accepted[b][c] = how many of candidate c's
 *     leading drafts are in the accepted sequence, next_token[b][c] = the one
 *     emitted token, best_cand[b] = the lowest-index candidate alive at the
 *     end (n_accepted[b][best] = k); margin [nb][nc] fp64 = smallest relative distance of any
 *     decision from its threshold (greedy: smallest top-1 logit gap of the
 *     rows read); may be NULL.
 *   status [nb] uint32 (may be NULL): HCI_DS_NONFINITE when a logit read is
 *     NaN or +Inf or a row read has no finite entry (-Inf entries are valid,
 *     probability 0); the block's n_accepted and next_token are then -1 and it
 *     cannot win best_cand (best_cand = -1 if no candidate of the sequence is
 *     valid; in the recursive mode every candidate of the sequence is marked).
 *     HCI_DS_DRAFT_ID when a draft id read is outside [0, V).
 * Limits: 1 <= V <= 65536; temperature > 0 in the sampling modes; nc <= 64. */
int hci_accept(int mode, int nb, int nc, int gamma, int vocab, float temperature,
               const float* target_logits, const float* draft_logits,
               const int32_t* draft_tokens, const double* uniforms,
               int32_t* n_accepted, int32_t* next_token, int32_t* best_cand,
               double* margin, uint32_t* status, hipStream_t stream);

/* ------------------------------------------------------------------- slice */

/* Commit block positions 0..k of the winning candidate c* = best_cand[b]
 * (k = n_accepted[b][c*]) -- EvSpark digest, Figure 1(d) and Interpretation
 * (state slicing, no replay):
 *   kv rows kv_len..kv_len+k  <- block k/v rows 0..k of c*;  kv_len += k+1
 *   short_win <- last Ts-1 rows of [short_win ; x_0..x_k]
 *   outer_win <- last To-1 rows of [outer_win ; f_0..f_k]
 *   iir       <- s_k
 * k and c* are read on the device (no host synchronisation).  best_cand may
 * be NULL when nc == 1.  max_kv_len is the same host bound as for verify.
 * A sequence whose c* is outside [0, nc), whose k is outside [0, gamma] or
 * whose kv_len is outside [0, max_kv_len] is left unchanged, and the matching
 * HCI_DS_* bit is set in S->status (nothing is clamped into range). */
int hci_slice_state(const hci_layer* L, const hci_state* S, const hci_block* blk,
                    int nb, int nc, int gamma, int max_kv_len,
                    const int32_t* n_accepted, const int32_t* best_cand,
                    hipStream_t stream);

/* ------------------------------------------------------------- token trees */

/* Several candidate blocks that share prefixes, verified as one token tree
 * (EvSpark digest, Interpretation: C = 1/2/4 candidate blocks per step; ReaDy
 * summary, section 5: tree verification with recovery of recurrent state).
 * Per sequence a tree of n nodes: node 0 is the anchor, node m > 0 holds a
 * drafted token and has a parent parent[b][m] < m (parent[b][0] = -1).  Node m
 * stands for the positions along the path root -> m, so shared prefixes are
 * computed once.  Arrays are per node, nodes in index order:
 *   parent [nb][n] int32
 *   x [nb][n][d] act; q, k, v [nb][n][H][Dh] act (16-byte aligned q)
 *   f [nb][n][d] fp32, s [nb][n][d][N] fp32, y [nb][n][d] act, o [nb][n][H][Dh] act: OUT of verify
 * parent, x, k, v, f and s must stay unchanged between hci_verify_tree and
 * hci_slice_tree. */
typedef struct hci_tree {
    const int32_t* parent;
    const void* x;
    const void* q;
    const void* k;
    const void* v;
    float* f;
    float* s;
    void* y;
    void* o;
} hci_tree;

/* One block forward over every node of every tree from the committed state
 * (only read).  Each output at node m equals the chain block forward
 * (hci_verify_block) over the path root -> m at its last position: the FIR
 * windows read m's ancestors, newest first, then the committed window; the IIR
 * state starts from the parent's state; the query attends to the committed
 * prefix and to the block keys of m's ancestors and m itself.  f, s and y are
 * computed with the chain kernel's summation orders, so they carry the same
 * bits as the chain forward over the path.
 *   ws, ws_bytes  hci_verify_workspace_bytes(L, nb, 1, n - 1, max_kv_len) bytes.
 * Limits: 1 <= n <= 64; N <= 16 poles.  Errors as hci_verify_block; an invalid
 * parent entry is reported (HCI_DS_TREE in S->status) and read as m - 1. */
int hci_verify_tree(const hci_layer* L, const hci_state* S, const hci_tree* tree,
                    int nb, int n, int max_kv_len, void* ws, size_t ws_bytes, hipStream_t stream);

/* Acceptance over each sequence's tree, walking from the anchor:
 *   HCI_GREEDY: at node m the argmax of target row m (ties -> lowest id) is
 *     compared with m's children in index order; the first child holding it
 *     becomes the current node, otherwise the argmax is the next token.
 *   HCI_SAMPLE: m's children are tried in index order against the running
 *     residual w / z of p = softmax(target row m / T) (w = p, z = 1): child c
 *     with token t, drawn from q_c = softmax(draft row c / T), is kept iff
 *     r_c * q_c(t) * z < w(t); a rejection sets w <- max(0, w - z q_c),
 *     z <- sum(w).  A kept child becomes the current node; if all are
 *     rejected the next token is drawn from w, at a node without children from
 *     p (inverse CDF with r*, as hci_accept).  Lossless when every child's
 *     token is an independent draw from its q_c (multi-step speculative
 *     sampling with one draft distribution per child).
 *   Inputs: parent [nb][n]; tokens [nb][n] int32 (entry 0 unused);
 *     target_logits [nb][n][V] fp32 (row m: the token after node m);
 *     draft_logits [nb][n][V] fp32 (row c: the distribution node c's token was
 *     drawn from; row 0 unused; NULL in greedy mode); uniforms [nb][n] fp64:
 *     r_c of node c, entry 0 = r* (NULL in greedy mode).
 *   Outputs: n_accepted [nb] = depth k of the accepted node; path [nb][n] =
 *     its nodes from the anchor (path[b][0] = 0, entries past k = -1);
 *     next_token [nb]; margin [nb] fp64 or NULL (as hci_accept); status [nb]
 *     or NULL (HCI_DS_NONFINITE and HCI_DS_TREE mark the sequence with
 *     n_accepted = next_token = -1; HCI_DS_DRAFT_ID is reported only).
 * Limits: 1 <= n <= 64, 1 <= V <= 65536, temperature > 0 when sampling. */
int hci_accept_tree(int mode, int nb, int n, int vocab, float temperature, const int32_t* parent,
                    const int32_t* tokens, const float* target_logits, const float* draft_logits,
                    const double* uniforms, int32_t* n_accepted, int32_t* path, int32_t* next_token,
                    double* margin, uint32_t* status, hipStream_t stream);

/* Commit the accepted path of each sequence's tree: its nodes path[b][0..k]
 * (k = n_accepted[b]) play the role of block rows 0..k in hci_slice_state
 * (KV rows appended, windows <- their last rows, IIR <- s of the accepted
 * node, kv_len += k + 1).  A sequence whose k is outside [0, n - 1], whose
 * kv_len is outside [0, max_kv_len] or whose path does not start at node 0 and
 * follow the tree is left unchanged (HCI_DS_K_RANGE / HCI_DS_KV_LEN /
 * HCI_DS_TREE in S->status). */
int hci_slice_tree(const hci_layer* L, const hci_state* S, const hci_tree* tree, int nb, int n, int max_kv_len,
                   const int32_t* n_accepted, const int32_t* path, hipStream_t stream);

/* ----------------------------------------------------------------- prefill */

/* Bytes of workspace hci_prefill needs (want_y: whether y is requested). */
size_t hci_prefill_workspace_bytes(const hci_layer* L, int nb, int T, int want_y);

/* Prefill a prompt of T positions into the committed state -- the step
 * before the verify hot path.  By the block-forward contract of the EvSpark
 * digest (Interpretation) this equals T sequential single-position steps
 * restricted to the state:
 *   short_win <- last Ts-1 rows of [short_win ; x_0..x_{T-1}]
 *   outer_win <- last To-1 rows of [outer_win ; f_0..f_{T-1}]
 *   iir       <- s_{T-1}   (s_t = lambda * s_{t-1} + beta * g_t from iir)
 *   kv rows kv_len..kv_len+T-1 <- k, v;   kv_len += T
 * and, if y is not NULL, y_t = sum_n c * s_t for every prompt position.  The
 * prompt's attention outputs are not computed (they are not state).
 *   x [nb][T][d] act;  k, v [nb][T][H][Dh] act;  y [nb][T][d] act or NULL;
 *   all four 16-byte aligned (HCI_EINVAL otherwise).
 *   max_kv_len  host bound on every kv_len[b]; max_kv_len + T <= kv_cap.
 *   ws, ws_bytes  workspace of hci_prefill_workspace_bytes(...), 256-aligned.
 * A sequence whose kv_len is outside [0, max_kv_len] keeps its committed state
 * (windows, IIR state, cache rows, kv_len) and gets HCI_DS_KV_LEN in S->status;
 * its outputs y are still written.
 * Limits: N <= 16 poles; T <= 16776960.  The IIR runs as a chunked parallel
 * scan, so the state equals the sequential recurrence up to fp32 rounding.
 * With bf16 activations (d % 8 == 0, T >= To, Ts <= 4, To <= 144) the outputs
 * y come from matrix-core products whose fp32 operands are split into two
 * bf16 terms: each sum carries a relative error of about 2^-14 of the
 * magnitudes of its terms before y is rounded to bf16. */
int hci_prefill(const hci_layer* L, const hci_state* S, int nb, int T, int max_kv_len,
                const void* x, const void* k, const void* v, void* y,
                void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------ dense projections */

/* The projections around the mixers of a full hybrid layer (input / output
 * projections of the Hyena and attention blocks; StripedHyena2-style layers
 * as described by the EvSpark digest, Figure 1(a)).  The weight W [K][N]
 * (y = x W) is packed once, in matrix-core operand order: tiles of 32 (K) x
 * 16 (N), the K/32 tiles of each 16-column strip consecutive, and inside a
 * tile element [g<4][n<16][e<8] = W[32 kt + 8 g + e][16 nt + n].
 * Limits: K % 32 == 0, N % 16 == 0, K, N <= 65536 x 16; bf16 data. */
size_t hci_linear_packed_elems(int K, int N);          /* 0 if K, N unsupported */

/* w [K][N] bf16 row-major -> w_packed (hci_linear_packed_elems bf16 elements). */
int hci_linear_pack(int K, int N, const void* w, void* w_packed, hipStream_t stream);

/* y [M][N] = x [M][K] w (+ residual [M][N]), bf16 inputs, fp32 accumulation;
 * y is bf16 (round to nearest even) or fp32 (out_f32 != 0).  residual may be
 * NULL (bf16 when given).  x, w_packed, residual and y are 16-byte aligned.
 * Every weight byte is read once per call; sums over K run in a fixed order. */
int hci_linear(int M, int K, int N, const void* x, const void* w_packed, const void* residual, void* y,
               int out_f32, hipStream_t stream);

/* y [M][K] = bf16( x * gamma / sqrt(mean_k(x^2) + eps) ) per row; x, y bf16,
 * gamma fp32 [K]. */
int hci_rmsnorm(int M, int K, const void* x, const float* gamma, float eps, void* y, hipStream_t stream);

/* ------------------------------------------------------- full layer stack */

/* A stack of full hybrid layers around the mixers above: the StripedHyena2
 * target of the EvSpark digest (Synopsis, Figure 1(a)) interleaves Hyena
 * layers (short-explicit and medium-regularised explicit filters, long
 * implicit modal filters) with attention, and each state class of Figure
 * 1(d) then lives in its own layer.  The pages print no layer equations;
 * the plain reading implemented here, per layer on the residual stream x:
 *   a = bf16( RMSNorm(x) * g )
 *   Hyena (HCI_MIX_FIR / HCI_MIX_IIR):
 *     z = a W_in (fp32), three streams z_q, z_k, z_v of d channels;
 *     zhat = short depthwise FIR (Ts taps) of each of the 3d channels;
 *     u = zhat_k * zhat_v;
 *     h = explicit FIR of Tl taps over u (HCI_MIX_FIR) or the modal IIR
 *         s_i = lambda s_{i-1} + beta u_i, h_i = sum_n c s_i (HCI_MIX_IIR);
 *     y = bf16( zhat_q * h )
 *   attention (HCI_MIX_ATTN): (q, k, v) = bf16( a W_in ), H heads of Dh,
 *     y = causal block attention over the layer's KV cache (as hci_verify_block)
 *   x <- bf16( x + y W_out )
 * The feature buffer (the drafter's window of target states, Figure 1(b);
 * it commits the same consumed prefix, Figure 1(d)) holds the residual
 * stream after layer feature_layer for the last feature_window positions.
 * Limits: d % 32 == 0, d = H * Dh, Dh in {64, 128}, Ts <= 8, Tl <= 256,
 * N <= 16, nc * P <= 64, nb * nc * P <= 65535. */
#define HCI_MIX_FIR  0
#define HCI_MIX_IIR  1
#define HCI_MIX_ATTN 2

typedef struct hci_mixer {
    int kind;                      /* HCI_MIX_* */
    int taps_short, taps_long, poles;
    const float* norm;             /* [d] RMSNorm gain g */
    const void* w_in;              /* packed (hci_linear_pack) bf16 [d][3d] */
    const void* w_out;             /* packed bf16 [d][d] */
    const float* w_short;          /* [Ts][3d] (Hyena) */
    const float* w_long;           /* [Tl][d]  (HCI_MIX_FIR) */
    const float* lambda;           /* [d][N]   (HCI_MIX_IIR) */
    const float* beta;
    const float* c;
} hci_mixer;

typedef struct hci_model {
    int n_layers, d, heads, head_dim;
    int feature_layer, feature_window;
    float eps;                     /* RMSNorm epsilon */
    const hci_mixer* layers;       /* host array of n_layers */
} hci_model;

/* Committed state of one layer for nb sequences (all fp32 except the caches):
 *   short_win [nb][Ts-1][3d]  last Ts-1 rows of z, oldest first (Hyena)
 *   long_win  [nb][Tl-1][d]   last Tl-1 values of u (HCI_MIX_FIR)
 *   iir       [nb][d][N]      (HCI_MIX_IIR)
 *   k_cache, v_cache          tiled bf16 caches as in hci_state (HCI_MIX_ATTN) */
typedef struct hci_layer_state {
    float* short_win;
    float* long_win;
    float* iir;
    void* k_cache;
    void* v_cache;
} hci_layer_state;

typedef struct hci_model_state {
    int kv_cap;
    int32_t* kv_len;               /* [nb], shared by every attention layer */
    void* feature;                 /* [nb][feature_window][d] bf16, oldest first */
    const hci_layer_state* layers; /* host array of n_layers */
} hci_model_state;

/* Block tensors of one verify, retained for the slice (rows = nb * nc * P,
 * row (b, c, i) at (b * nc + c) * P + i):
 *   x [n_layers+1][rows][d] bf16: x[0] is the block input (caller-filled),
 *     x[l+1] the residual stream after layer l (OUT); x[n_layers] is the output
 *   per layer: z [3][rows][d] (fp32 for Hyena, bf16 for attention), u [rows][d]
 *     fp32 (HCI_MIX_FIR), s [rows][d][N] fp32 (HCI_MIX_IIR). */
typedef struct hci_layer_block {
    void* z;
    float* u;
    float* s;
} hci_layer_block;

typedef struct hci_model_block {
    void* x;
    const hci_layer_block* layers; /* host array of n_layers */
} hci_model_block;

size_t hci_model_workspace_bytes(const hci_model* M, int nb, int nc, int gamma, int max_kv_len);

/* One block forward through every layer from the committed state (state is
 * only read).  Same block conventions as hci_verify_block. */
int hci_model_verify(const hci_model* M, const hci_model_state* S, const hci_model_block* blk,
                     int nb, int nc, int gamma, int max_kv_len, void* ws, size_t ws_bytes, hipStream_t stream);

/* Commit rows 0..k of candidate c* of every sequence in every layer (EvSpark
 * digest, Figure 1(d), layer by layer): Hyena windows <- their last rows,
 * IIR state <- s_k, attention rows appended at kv_len, feature buffer <- its
 * last rows, then kv_len += k + 1.  k = n_accepted[b][c*], c* = best_cand[b]
 * (NULL when nc == 1), read on the device. */
int hci_model_slice(const hci_model* M, const hci_model_state* S, const hci_model_block* blk,
                    int nb, int nc, int gamma, int max_kv_len,
                    const int32_t* n_accepted, const int32_t* best_cand, hipStream_t stream);

/* ----------------------------------------------------------------- drafter */

/* The drafter of the EvSpark digest (Figure 1(b); Interpretation): a
 * projected window of W target states (the feature buffer) forms the K/V
 * prefix of each of two causal attention layers of width d; the anchor's
 * embedding followed by gamma-1 mask embeddings gives all gamma draft logits
 * in one trunk pass (input and output embeddings tied); a previous-token
 * Markov bias then supports serial sampling.  The pages print no equations;
 * the reading implemented:
 *   hw = bf16(window W_proj);   block rows h = [E[anchor]; mask x (gamma-1)]
 *   per layer: a = bf16(RMSNorm(h) g1); (q,k,v) = bf16(a W_qkv) for the block
 *     rows and (k,v) of bf16(RMSNorm(hw) g1) W_qkv for the window rows; causal
 *     block attention with the window as prefix -> o (bf16); h = bf16(h + o W_o);
 *     h = bf16(h + bf16(SiLU(bf16(RMSNorm(h) g2) W_up)) W_down)
 *   z = bf16(RMSNorm(h) g_f) E^T  (fp32)
 * Sizes: d % 32 == 0, d = H * 128, d_target % 32 == 0, ffn % 32 == 0,
 * vocab % 16 == 0, 1 <= window <= 64, 1 <= gamma <= 32. */
typedef struct hci_drafter_layer {
    const float* g1;               /* [d] */
    const void* w_qkv;             /* packed bf16 [d][3d] */
    const void* w_o;               /* packed bf16 [d][d] */
    const float* g2;               /* [d] */
    const void* w_up;              /* packed bf16 [d][ffn] */
    const void* w_down;            /* packed bf16 [ffn][d] */
} hci_drafter_layer;

typedef struct hci_drafter {
    int d_target, d, heads, head_dim, ffn, vocab, window, n_layers;
    float eps;
    const void* w_proj;            /* packed bf16 [d_target][d] */
    const void* emb;               /* [vocab][d] bf16 row-major (input embedding) */
    const void* emb_t;             /* packed bf16 [d][vocab] (the tied output embedding) */
    const void* mask;              /* [d] bf16 */
    const float* g_f;              /* [d] final RMSNorm gain */
    const hci_drafter_layer* layers;   /* host array of n_layers */
} hci_drafter;

size_t hci_draft_workspace_bytes(const hci_drafter* D, int nb, int gamma);

/* Trunk pass: z [nb][gamma][vocab] fp32 = the draft logits before the bias.
 * window [nb][W][d_target] bf16 (e.g. the feature buffer of hci_model_state),
 * anchor [nb] int32 (ids outside [0, vocab) are clamped). */
int hci_draft_logits(const hci_drafter* D, int nb, int gamma, const void* window, const int32_t* anchor,
                     float* z, void* ws, size_t ws_bytes, hipStream_t stream);

/* Serial sampling with the previous-token bias (prev = anchor, then each
 * draft): draft m draws from softmax(l / T) with the fp32 logits
 * l = z[m] + markov[prev][.] (markov [vocab][vocab] fp32), by inverse CDF
 * with uniforms[b][m] under the acceptance rule's conventions (fp64
 * probabilities; the smallest id whose running sum exceeds u x total).
 * Writes drafts [nb][gamma] int32 and draft_logits [nb][gamma][vocab] = l,
 * the distribution each draft was drawn from (what hci_accept needs as
 * draft_logits); margin [nb][gamma] fp64 (or NULL) as in hci_accept.
 * Limits: 1 <= vocab <= 4096. */
int hci_draft_sample(int nb, int gamma, int vocab, float temperature, const float* z, const float* markov,
                     const int32_t* anchor, const double* uniforms, int32_t* drafts, float* draft_logits,
                     double* margin, hipStream_t stream);

/* -------------------------------------------------------------- KV access */

/* Elements (not bytes) of ONE of k_cache / v_cache for nb sequences. */
size_t hci_kv_cache_elems(const hci_layer* L, int nb, int kv_cap);

/* Write logical rows [row0, row0+nrows) of sequence b (0 <= b < nb) into the
 * tiled caches.  k_rows, v_rows: [H][nrows][Dh] act, 16-byte aligned
 * (HCI_EINVAL otherwise).  Does not touch kv_len.
 * HCI_ECAPACITY if row0 + nrows > kv_cap. */
int hci_kv_write(const hci_layer* L, const hci_state* S, int nb, int b, int row0, int nrows,
                 const void* k_rows, const void* v_rows, hipStream_t stream);

/* Read logical rows [row0, row0+nrows) of sequence b: [H][nrows][Dh] act. */
int hci_kv_read(const hci_layer* L, const hci_state* S, int nb, int b, int row0, int nrows,
                void* k_rows, void* v_rows, hipStream_t stream);

/* ------------------------------------------------------------------ probes */

/* Stream `bytes` (multiple of 16) from src; one word per workgroup is written
 * to sink[0..blocks) so the reads cannot be elided.  sink must hold
 * hci_probe_sink_words() floats.  Measures the practical HBM read ceiling. */
int hci_probe_read(const void* src, size_t bytes, float* sink, hipStream_t stream);
int hci_probe_sink_words(void);

/* Plain device copy of `bytes` (multiple of 16): the known-size kernel that
 * hardware byte counters are calibrated against. */
int hci_probe_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* HCI_H */
