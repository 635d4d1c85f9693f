/*
 * jev.h — shared-prefix candidate scoring on MI355X (gfx950).
 *
 * The operation (from the pages this library follows):
 *   A vision-language decoder reads one image and text prefix.  The prefix is
 *   run through the decoder ONCE and its key/value cache kept resident
 *   ("How to Deploy Visual Jev ...", Step 2; "Ochevid Jev-VL 2B", intro).
 *   Many independent question suffixes are then run as rows of ONE batched
 *   forward over that cache, and candidate answers are scored straight from
 *   the logits at each question's last position, with no generation
 *   (Step 3; Ochevid "Run": one encoding, one shared prefill, one branch call).
 *   Multi-token candidates of one question share their common history in a
 *   prefix tree and are scored by the sum of their tokens' log-probabilities
 *   ("FastJEV", §3.3 Candidate Prefix Sharing).
 *
 * Conventions for every call:
 *   - Every function returns a jev_status; no C++ exception crosses the ABI.
 *   - All arguments are validated before anything is enqueued.  On an error
 *     nothing is launched, outputs are untouched and jev_last_error() says why.
 *   - "dev" pointers are device memory on the current HIP device; "host"
 *     pointers are ordinary host memory read during the call only.
 *   - The caller owns every device buffer (weights, prefix KV store,
 *     workspace, outputs).  Handles keep pointers only; keep buffers alive
 *     while a handle that names them is used.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream).  Outputs are valid once the stream has synchronised.
 *     Hot-path calls allocate no device memory and never synchronise the
 *     stream themselves.  Their one host->device copy (the call's packed
 *     metadata) goes through a ring of pinned host slots that the model
 *     creates on its first staging call (8 x 1 MiB of pinned host memory,
 *     freed by jev_model_destroy); a slot is refilled only once the copy that
 *     last read it has completed, so the caller's host arrays may be reused as
 *     soon as a call returns.  A host that runs more than eight staging calls
 *     ahead of the device waits for the oldest copy at that point.
 *   - A model or prefix may be used from several host threads or streams at
 *     once provided each call has its own workspace and output buffers.
 */
#ifndef JEV_H
#define JEV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t jev_status;
#define JEV_OK             0
#define JEV_E_INVALID     -1   /* bad argument: null pointer, out-of-range id/length/count   */
#define JEV_E_UNSUPPORTED -2   /* well-formed but outside what the kernels implement          */
#define JEV_E_WORKSPACE   -3   /* workspace or prefix buffer smaller than required            */
#define JEV_E_HIP         -4   /* a HIP runtime call or kernel launch failed                  */

/* Storage type of weights, embeddings and prefix inputs. */
#define JEV_F32  0   /* float32 everywhere; the KV store is float32                          */
#define JEV_BF16 1   /* bfloat16 weights; KV store float16; residual/norm/softmax in float32 */

/* Decoder shape.  Pre-norm layers: RMSNorm -> q/k/v (rotate-half RoPE) ->
 * grouped-query attention -> o-proj + residual -> RMSNorm -> SwiGLU MLP +
 * residual; final RMSNorm; untied LM head.  No biases. */
typedef struct {
    int32_t n_layers;     /* >= 0                                                       */
    int32_t hidden;       /* H; multiple of 64 and <= 8192 for JEV_BF16                 */
    int32_t n_q_heads;    /* Hq                                                         */
    int32_t n_kv_heads;   /* Hkv; Hq % Hkv == 0; q head h reads kv head h / (Hq/Hkv)    */
    int32_t head_dim;     /* D; 64 or 128                                               */
    int32_t mlp;          /* I; multiple of 64 for JEV_BF16                             */
    int32_t vocab;        /* V                                                          */
    float   rope_theta;   /* angle of pair t at position p: p * theta^(-2t/D)           */
    float   rms_eps;      /* RMSNorm(x; g) = g * x / sqrt(mean(x^2) + eps)              */
    int32_t dtype;        /* JEV_F32 or JEV_BF16                                        */
} jev_config;

/* One layer's parameters, dev pointers of type `dtype`, row-major [out, in]. */
typedef struct {
    const void *attn_norm;  /* [H]                    */
    const void *wq;         /* [Hq*D, H]              */
    const void *wk;         /* [Hkv*D, H]             */
    const void *wv;         /* [Hkv*D, H]             */
    const void *wo;         /* [H, Hq*D]              */
    const void *mlp_norm;   /* [H]                    */
    const void *w_gate;     /* [I, H]                 */
    const void *w_up;       /* [I, H]                 */
    const void *w_down;     /* [H, I]                 */
} jev_layer;

typedef struct {
    const void      *embed;       /* dev [V, H]                              */
    const void      *final_norm;  /* dev [H]                                 */
    const void      *lm_head;     /* dev [V, H]                              */
    const jev_layer *layers;      /* host array [n_layers]; copied at create */
} jev_weights;

typedef struct jev_model  jev_model;
typedef struct jev_prefix jev_prefix;

typedef struct {
    uint64_t prefills;   /* jev_prefill_prefix calls that launched work            */
    uint64_t forwards;   /* jev_score_suffixes + jev_score_tree calls that launched */
    uint64_t rows;       /* decoder rows run by those forwards                      */
    uint64_t launches;   /* kernels launched by this model, all calls               */
} jev_stats;

/* ---- model ------------------------------------------------------------------ */
/* Validates the shape and records the weight pointers.  Makes no HIP call. */
jev_status jev_model_create(const jev_config *cfg, const jev_weights *w, jev_model **out);
void       jev_model_destroy(jev_model *m);
jev_status jev_get_stats(const jev_model *m, jev_stats *out);

/* ---- float16 weight mirror (JEV_BF16 models) ----------------------------------
 * The pages fix no arithmetic precision below the model's own; the decoder's
 * matrix products may run in any precision that keeps the scores within the
 * tolerance of the plain float32 forward.  By default a bf16 model's GEMMs take
 * each float32 activation as two bfloat16 terms (hi + lo, two matrix-core
 * passes).  For a mirrored group of matrices they take it as ONE float16 term
 * against a float16 copy of the weights (one pass, half the matrix-core work):
 * bfloat16 weights are exact in float16 except below 2^-17 in magnitude
 * (rounded to float16's subnormal grid) and above 65504 (rejected).
 * Activations entering a mirrored GEMM must then stay below 65504 in magnitude.
 *
 * groups: any OR of JEV_F16_GATE_UP (w_gate, w_up), JEV_F16_QKV (wq, wk, wv),
 *   JEV_F16_DOWN (w_down) and JEV_F16_O (wo), each used by every call, and of
 *   JEV_F16_GATE_UP_PREFILL, JEV_F16_QKV_PREFILL and JEV_F16_O_PREFILL, which
 *   mirror the same matrices but use the single f16 pass in prefills only:
 *   the prefix rows feed nothing but the float16 KV store, while the rows of
 *   scoring calls, whose logits are read, keep the two bfloat16 terms.
 *   JEV_F16_QKV_PREFILL applies to prefills whose longest segment is at most
 *   2048 rows; longer prefixes keep q|k|v on two terms (the rounding of K and
 *   V reaches every query's scores, and its error grows with the keys a query
 *   sees, as for the q terms in jev_model_set_attn_q_terms).
 *   JEV_F16_GATE_UP_SCORE extends the single f16 pass of gate|up from prefills
 *   to the suffix-scoring calls, whose every candidate log-probability is read
 *   from one row ("How to Deploy Visual Jev", Step 3: two logits of the last
 *   position); tree calls keep two terms, since a candidate's tree score sums the
 *   log-probabilities of up to four rows and their rounding errors with them.
 * jev_model_f16_bytes: size of the mirror buffer for those groups (0 for JEV_F32
 *   models or unknown bits).
 * jev_model_attach_f16: buf dev [bytes >= jev_model_f16_bytes(m, groups)],
 *   caller-owned and kept alive while the model is used.  Converts the groups'
 *   matrices of every layer into it on `stream`, then synchronises the stream to
 *   read the range check: JEV_E_UNSUPPORTED if a weight exceeds the float16
 *   range, JEV_E_WORKSPACE if bytes is too small (nothing changes then).  Any
 *   failure after the conversion has begun (a range error, a HIP error) leaves
 *   the model detached, every GEMM on the two-term path: a mirror attached
 *   earlier is dropped, since the buffer may hold it and is being rewritten.
 *   Each call replaces the previous mirror; its groups alone decide which
 *   GEMMs run on the float16 pass.  buf == NULL or groups == 0 detaches the mirror.  Not a hot-path
 *   call (it blocks); do not call it while another call on this model is in
 *   flight.  The LM head and embeddings are never mirrored. */
#define JEV_F16_GATE_UP 1
#define JEV_F16_QKV     2
#define JEV_F16_DOWN    4
#define JEV_F16_O       8
#define JEV_F16_GATE_UP_PREFILL 16  /* w_gate, w_up mirrored, the f16 pass used by prefills only */
#define JEV_F16_QKV_PREFILL     32  /* wq, wk, wv mirrored, used by prefills of <= 2048 rows  */
#define JEV_F16_O_PREFILL       64  /* wo mirrored, used by prefills only                    */
#define JEV_F16_GATE_UP_SCORE  128  /* w_gate, w_up mirrored, used by prefills and by
                                       jev_score_suffixes / jev_score_segments, not by trees  */
size_t     jev_model_f16_bytes(const jev_model *m, int32_t groups);
jev_status jev_model_attach_f16(jev_model *m, int32_t groups, void *buf, size_t bytes, void *stream);
/* The groups whose float16 pass is in effect (0: none; a prefill-only bit is
 * reported only when its every-call bit is not set). */
int32_t    jev_model_f16_groups(const jev_model *m);

/* ---- decision-guided block skipping ("FastJEV", §2.3 and §3.4) -----------------
 * The candidate rows of jev_score_suffixes and jev_score_tree bypass the decoder
 * blocks whose skip[l] is non-zero (x leaves block l as it entered it), while the
 * shared context keeps every block: jev_prefill_prefix ignores the mask.  The
 * same blocks apply to shared histories and their continuations (every row of a
 * scoring call).  Ranking the blocks (the pages calibrate on unlabeled inputs)
 * is the caller's business; this is the mechanism only.
 * skip: host [n], n == n_layers; NULL or n == 0 clears the mask.  The mask is
 * copied; it applies to calls enqueued after this returns (do not change it
 * while another call on this model is being enqueued). */
jev_status jev_model_set_skip(jev_model *m, const uint8_t *skip, int32_t n);

/* ---- attention precision ---------------------------------------------------------
 * The scores q.k of the attention run on float16 matrix cores.  q is rounded to
 * float16 once (terms = 1) or carried as two float16 terms, f16(q) and the rounding
 * remainder q - f16(q) (terms = 2, twice the matrix-core work of the score
 * product).  q's rounding moves every score of a row coherently; its weight grows
 * with the number of keys a row sees.  terms = 0 (the default) takes two terms when
 * a call's rows see more than 2048 prefix keys (the longest segment of the store),
 * one otherwise.  Applies to calls enqueued after this returns. */
jev_status jev_model_set_attn_q_terms(jev_model *m, int32_t terms);

/* ---- range flag of a call ---------------------------------------------------------
 * Float16 activation planes (q, k and v; the normalised input of a float16
 * mirrored GEMM; the SwiGLU output feeding a float16 down projection) hold
 * magnitudes up to 65504.  Every forward clears a flag word at the start of its
 * workspace and each kernel writing such a plane sets bit JEV_FLAG_F16_RANGE when
 * a value is out of range or not finite; the scores of that call are then not
 * reliable.  jev_workspace_flags enqueues a read of the word on `stream`,
 * synchronises the stream and returns it in *flags: it reports the last call that
 * used the workspace (not a hot-path call: it blocks). */
#define JEV_FLAG_F16_RANGE 1
jev_status jev_workspace_flags(const void *ws, int32_t *flags, void *stream);

/* ---- prefix KV store ---------------------------------------------------------
 * Layout per layer l (element type float16 for JEV_BF16, float32 for JEV_F32),
 * with Pc = prefix_len rounded up to a multiple of 64 and Dk the stored head
 * width (128 for JEV_BF16, whose float16 attention runs on 128-dim heads: a
 * 64-dim head is stored and computed zero-padded; D for JEV_F32):
 *     K  [Hkv][Pc][Dk]  rotated keys, row p = prefix position p
 *     Vt [Hkv][Dk][Pc]  values, transposed (position fastest)
 * and layers stacked: store = { K_0, Vt_0, K_1, Vt_1, ... }.  Columns
 * [prefix_len, Pc) are padding and never read as values.  The buffer is
 * written by jev_prefill_prefix and only read afterwards ("FastJEV", §3.2:
 * a read-only shared anchor with separate per-branch working state). */
size_t     jev_prefix_bytes(const jev_model *m, int32_t prefix_len);
/* prefix_len in [0, 32768]; kv_bytes >= jev_prefix_bytes(m, prefix_len). */
jev_status jev_prefix_create(jev_model *m, int32_t prefix_len, void *kv_buf, size_t kv_bytes,
                             jev_prefix **out);
void       jev_prefix_destroy(jev_prefix *p);

/* ---- workspace ----------------------------------------------------------------
 * Upper bound of the workspace bytes for one call on a prefix of prefix_len:
 *   prefill:          max_rows = prefix_len, max_seqs = 1,  max_targets = 0
 *   score_suffixes:   max_rows = sum of suffix lengths (<= B*S_max), max_seqs = B,
 *                     max_targets = B*C_max
 *   score_tree:       max_rows = rows of the chosen mode (<= Q*C_max*(S_max+K_max)),
 *                     max_seqs = Q*C_max, max_targets = Q*C_max*K_max
 * The workspace is scratch: any content on entry, undefined on exit. */
size_t     jev_workspace_bytes(const jev_model *m, int32_t prefix_len, int32_t max_rows,
                               int32_t max_seqs, int32_t max_targets);

/* ---- the hot path -------------------------------------------------------------- */

/* Prefill the prefix once ("How to Deploy Visual Jev ...", Step 2: encode the
 * shared visual prefix and cache its KV; Ochevid intro: decoder image-prefix
 * prefill happens once).  Rows 0..n_vis-1 are the given visual embeddings,
 * rows n_vis..P-1 the embedding rows of text_ids; positions 0..P-1; causal.
 * Writes every layer's rotated K and V into the prefix store.
 *   vis_embeds  dev  [n_vis, H] of the model dtype (may be NULL if n_vis == 0)
 *   text_ids    host [n_text], each in [0, V)
 *   n_vis + n_text must equal the prefix's prefix_len.
 * Errors: JEV_E_INVALID (counts, ids, pointers), JEV_E_WORKSPACE, JEV_E_HIP. */
jev_status jev_prefill_prefix(jev_prefix *p, const void *vis_embeds, int32_t n_vis,
                              const int32_t *text_ids, int32_t n_text,
                              void *ws, size_t ws_bytes, void *stream);

/* Score B question suffixes over the prefix in one batched forward
 * ("How to Deploy Visual Jev ...", Step 3; Ochevid "Run").  Suffix b is
 * ids[b, 0:lens[b]] at positions P..P+lens[b]-1; it sees every prefix row and
 * its own earlier rows, never another suffix's.  At its last valid row the
 * logits z of the n_cands[b] candidates cand_ids[b, :] are read and
 *     out_logp[b, c] = z_c - logsumexp_{c' < n_cands[b]} z_{c'}
 * i.e. the log-softmax over the candidate set (Step 3's softmax over the
 * candidate logits), which equals the full-vocabulary log-probability
 * renormalised over the candidates.  Slots c >= n_cands[b] are set to -inf.
 * Duplicate candidate ids are allowed and score equally.
 *   ids       host [B, S_max] right-padded; pad slots are never read
 *   lens      host [B], each in [1, S_max]
 *   cand_ids  host [B, C_max], each used id in [0, V)
 *   n_cands   host [B], each in [1, C_max]
 *   out_logp  dev  [B, C_max] float32
 * B == 0 launches nothing and returns JEV_OK (Ochevid "Run": an all-skipped
 * request does no work).  Limits: S_max <= 256, C_max <= 64, sum of lens <= 65536.
 * Errors: JEV_E_INVALID, JEV_E_UNSUPPORTED, JEV_E_WORKSPACE, JEV_E_HIP. */
jev_status jev_score_suffixes(const jev_prefix *p,
                              const int32_t *ids, const int32_t *lens, int32_t B, int32_t S_max,
                              const int32_t *cand_ids, const int32_t *n_cands, int32_t C_max,
                              float *out_logp, void *ws, size_t ws_bytes, void *stream);

/* Scoring for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): jev_score_suffixes without a
 * workspace argument.  The workspace is a file-scope device array of
 * jev_static_scratch_bytes() bytes (256 MiB) inside the library, one copy per GPU,
 * held until the process ends.  The call allocates nothing: no device memory, no
 * pinned host memory.  Its metadata goes through the model's pinned staging ring
 * if an earlier call created it, otherwise it is copied and the stream
 * synchronised before the call returns.  A request whose workspace would exceed
 * the scratch returns JEV_E_WORKSPACE with the size it needs.  Every call on one
 * GPU shares that GPU's scratch: calls that overlap on one GPU (other streams or
 * host threads) race and must be serialised by the caller.  jev_workspace_flags
 * does not reach the scratch.  Otherwise as jev_score_suffixes. */
size_t     jev_static_scratch_bytes(void);
jev_status jev_score_suffixes_noalloc(const jev_prefix *p,
                                      const int32_t *ids, const int32_t *lens, int32_t B, int32_t S_max,
                                      const int32_t *cand_ids, const int32_t *n_cands, int32_t C_max,
                                      float *out_logp, void *stream);

/* Tree layouts of jev_score_tree. */
#define JEV_TREE_TRIE      0  /* stem + candidate tokens merged on (parent, token)   */
#define JEV_TREE_STEM_ONLY 1  /* stem shared, each candidate's tokens its own chain  */
#define JEV_TREE_FLAT      2  /* every candidate its own sequence stem ‖ tokens      */

/* Score multi-token candidates of Q questions ("FastJEV", §3.3).  Question q
 * has stem stem_ids[q, 0:stem_lens[q]] and candidates
 * w = cand_tok[q, c, 0:cand_lens[q, c]].  With l_r the full-vocabulary
 * log-probabilities at row r,
 *     out_score[q, c] = sum_k l_{row before w_k}[w_k]
 * over the history prefix ‖ stem ‖ w_0..w_{k-1} of each token, and
 *     out_norm[q, c]  = out_score[q, c] - logsumexp over the question's candidates.
 * All three layouts compute the same values; they differ only in how many
 * rows run.  In the trie layout, equal tokens are merged only when they
 * follow the same node, so equal tokens after different histories stay
 * separate, and a candidate's last token is never fed (no row needs it).
 *   stem_ids  host [Q, S_max], stem_lens host [Q] in [1, S_max]
 *   cand_tok  host [Q, C_max, K_max], cand_lens host [Q, C_max] in [1, K_max]
 *   n_cands   host [Q] in [1, C_max]
 *   out_score dev [Q, C_max] float32; out_norm dev [Q, C_max] float32 or NULL
 *   Slots c >= n_cands[q] are set to -inf.
 * Limits: the rows of one question's group (stem + fed candidate tokens) <= 64,
 * S_max <= 64, K_max <= 64, C_max <= 64.  Q == 0 launches nothing.
 * Errors: JEV_E_INVALID, JEV_E_UNSUPPORTED, JEV_E_WORKSPACE, JEV_E_HIP. */
jev_status jev_score_tree(const jev_prefix *p,
                          const int32_t *stem_ids, const int32_t *stem_lens, int32_t Q, int32_t S_max,
                          const int32_t *cand_tok, const int32_t *cand_lens, const int32_t *n_cands,
                          int32_t C_max, int32_t K_max, int32_t mode,
                          float *out_score, float *out_norm,
                          void *ws, size_t ws_bytes, void *stream);

/* ---- one question over several images ----------------------------------------
 * ("Ochevid Jev-VL 2B", One question, multiple images: a single typed
 * question asked of up to eight images, each image run through the model on
 * its own and answered separately, with nothing shared between the images'
 * rows.)  A segmented prefix
 * stores n_seg independent prefixes back to back in one KV store, segment i
 * occupying store rows [off_i, off_i + seg_lens[i]) with off_i the sum of the
 * earlier lengths.  One batched prefill runs all of them; each suffix of a
 * scoring call continues one segment and never sees another.
 *
 * jev_prefix_create_segments: as jev_prefix_create for prefix_len = the sum of
 *   seg_lens (each >= 0; n_seg in [1, 64]; the sum <= 32768); size kv_buf with
 *   jev_prefix_bytes(m, sum).  A plain prefix is the one-segment case.
 *   jev_prefill_prefix, jev_score_suffixes and jev_score_tree reject a prefix of
 *   more than one segment (JEV_E_INVALID).
 * jev_prefill_segments: segment i's rows are its n_vis[i] visual embeddings
 *   then the embedding rows of its n_text[i] text ids, at positions
 *   0..seg_lens[i]-1, causal within the segment only.  n_vis[i] + n_text[i] must
 *   equal seg_lens[i].
 *     vis_embeds  dev  [sum n_vis, H] of the model dtype, segment-major
 *     text_ids    host [sum n_text], segment-major, each in [0, V)
 *     n_vis, n_text host [n_seg]
 *   Workspace: jev_workspace_bytes(m, sum, sum, 1, 0).
 * jev_score_segments: jev_score_suffixes where suffix b continues segment
 *   seg[b] (host [B], each in [0, n_seg)): its token j sits at position
 *   seg_lens[seg[b]] + j and it sees that segment's rows and its own earlier
 *   rows only.  The one-question case passes the same question for every
 *   segment with seg[b] = b.  Suffixes of the same segment should be adjacent
 *   and segments in ascending order: the attention visits, for each block of
 *   rows, the keys between the first and the last segment its rows name.
 *   Workspace: jev_workspace_bytes(m, sum, sum of lens, B, B * C_max).
 * Errors: as jev_prefix_create / jev_prefill_prefix / jev_score_suffixes. */
jev_status jev_prefix_create_segments(jev_model *m, const int32_t *seg_lens, int32_t n_seg,
                                      void *kv_buf, size_t kv_bytes, jev_prefix **out);
jev_status jev_prefill_segments(jev_prefix *p, const void *vis_embeds, const int32_t *n_vis,
                                const int32_t *text_ids, const int32_t *n_text,
                                void *ws, size_t ws_bytes, void *stream);
jev_status jev_score_segments(const jev_prefix *p, const int32_t *seg,
                              const int32_t *ids, const int32_t *lens, int32_t B, int32_t S_max,
                              const int32_t *cand_ids, const int32_t *n_cands, int32_t C_max,
                              float *out_logp, void *ws, size_t ws_bytes, void *stream);

/* ---- launch-only scoring (HIP graph capture) -----------------------------------
 * jev_score_suffixes_launch and jev_score_tree_launch take the arguments of
 * jev_score_suffixes and jev_score_tree, make the same checks and build the
 * same plan on the host, but do not copy the plan's metadata (row tokens,
 * positions, sequence starts, masks, readout tables) into the workspace: the
 * workspace must still hold what the last staging call on this model (any
 * hot-path call other than these two) put into it, for identical arguments,
 * and no call on another model may have used the workspace since.
 * The library keeps, per model and workspace address (up to 1024 addresses;
 * beyond that the remembered digests are dropped), a 64-bit digest of the
 * metadata it last staged there; a mismatch (other arguments,
 * another call in between, no staging call yet) returns JEV_E_INVALID and
 * launches nothing.  Everything these calls enqueue is a kernel launch (no
 * copy, memset, allocation or synchronisation), so a caller can capture them
 * on a stream into a HIP graph and replay it; each replay recomputes the
 * outputs from the prefix store and the workspace as they are when it runs.
 * Calls that share a workspace must not overlap.
 * Errors: as the staging calls. */
jev_status jev_score_suffixes_launch(const jev_prefix *p,
                                     const int32_t *ids, const int32_t *lens, int32_t B, int32_t S_max,
                                     const int32_t *cand_ids, const int32_t *n_cands, int32_t C_max,
                                     float *out_logp, void *ws, size_t ws_bytes, void *stream);
jev_status jev_score_tree_launch(const jev_prefix *p,
                                 const int32_t *stem_ids, const int32_t *stem_lens, int32_t Q, int32_t S_max,
                                 const int32_t *cand_tok, const int32_t *cand_lens, const int32_t *n_cands,
                                 int32_t C_max, int32_t K_max, int32_t mode,
                                 float *out_score, float *out_norm,
                                 void *ws, size_t ws_bytes, void *stream);

/* Rows the tree layout `mode` runs for this request (host-only planning; no
 * HIP call).  Useful to size the workspace exactly.  Returns JEV_OK and sets
 * *rows, *seqs and *targets, or an error as jev_score_tree would. */
jev_status jev_tree_plan_size(const int32_t *stem_ids, const int32_t *stem_lens, int32_t Q,
                              int32_t S_max, const int32_t *cand_tok, const int32_t *cand_lens,
                              const int32_t *n_cands, int32_t C_max, int32_t K_max, int32_t mode,
                              int32_t *rows, int32_t *seqs, int32_t *targets);

/* Host-only introspection of a tree plan (no HIP call), for tests of the
 * packing: per row its token, its depth below the prefix, its group and its
 * 64-bit visibility mask over the group's rows; per target (q, c, k) the row
 * that predicts it.  Arrays are caller-allocated with the sizes reported by
 * jev_tree_plan_size.  row_mask bit j set means the row sees row
 * (group start + j). */
jev_status jev_tree_plan_rows(const int32_t *stem_ids, const int32_t *stem_lens, int32_t Q,
                              int32_t S_max, const int32_t *cand_tok, const int32_t *cand_lens,
                              const int32_t *n_cands, int32_t C_max, int32_t K_max, int32_t mode,
                              int32_t *row_tok, int32_t *row_depth, int32_t *row_group,
                              uint64_t *row_mask, int32_t *target_row);

/* Host-only introspection of the attention's segment table (no HIP call), for
 * tests: pseg host [T][2] holds each row's prefix key range [x, y); for every
 * 128-row block of the G*T query rows (row r = t*G + g) ptile host
 * [ceil(G*T/128)][4] receives the block's prefix key tiles [x, y) of 64 keys
 * (the hull of its rows' ranges; 0, 0 when they are all empty) and the keys
 * [z, w) every one of its rows sees (z >= w when there are none); *max_tiles
 * the largest tile count.  JEV_E_INVALID for negative or reversed ranges. */
jev_status jev_segment_plan_tiles(const int32_t *pseg, int32_t T, int32_t G, int32_t *ptile,
                                  int32_t *max_tiles);

/* Host-only introspection of the bf16 attention's work split (no HIP call), for tests.
 * For T query tokens with G q heads per KV head, Hkv KV heads, P prefix keys, own_tiles
 * own-key tiles of 64 keys (the largest any 128-row tile needs) and segmented != 0 for
 * segmented prefixes, *n_split, *chunk and *blocks receive the schedule of the shared-prefix
 * attention (FastJEV, §3.2: every question's rows read the shared prefix keys): chunk 0 means
 * n_split equal key splits per 128-row tile, chunk > 0 the balanced schedule (chunk key
 * tiles per block, n_split partial slots).  Under the balanced schedule, with spans
 * non-null, spans [cap][7] receives block by block every run the kernel processes:
 * (block, item, slot, first tile, end tile, last, the item's slot count as the merge
 * reads it), the item being KV head item / n_rt and row tile n_rt - 1 - item % n_rt
 * (n_rt = ceil(G*T/128)); *n_spans their count.
 * JEV_E_INVALID for sizes out of range or a short cap. */
jev_status jev_attn_schedule(int32_t T, int32_t G, int32_t Hkv, int32_t P, int32_t own_tiles, int32_t segmented,
                             int32_t *n_split, int32_t *chunk, int32_t *blocks, int32_t *spans, int32_t cap,
                             int32_t *n_spans);

/* ---- diagnostics ----------------------------------------------------------------
 * Per-kernel timing with HIP events recorded on the call's stream around every
 * launch, plus the algorithmic work of each launch (flops counted once, i.e.
 * without the second pass of the split bf16 activations; bytes = operands
 * read once and results written once).  While enabled, calls on the model
 * must come from one host thread; events add a small gap between launches.
 * jev_profile_stop synchronises on the last recorded event, fills up to
 * max_out entries (one per kernel kind that ran) and sets *n_out to the
 * number of kinds. */
typedef struct {
    char     name[32];
    uint64_t launches;
    double   ms;       /* summed launch durations        */
    double   flops;    /* summed algorithmic flops       */
    double   bytes;    /* summed algorithmic bytes       */
} jev_kernel_stat;
jev_status jev_profile_start(jev_model *m);
jev_status jev_profile_stop(jev_model *m, jev_kernel_stat *out, int32_t max_out, int32_t *n_out);

/* Thread-local text of the last error on this thread ("" if none). */
const char *jev_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* JEV_H */
