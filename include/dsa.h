/*
 * dsa.h -- C ABI of libdsa, the MI355X (gfx950) hot path of DeepSeek Sparse
 * Attention (DSA): lightning indexer -> top-k selector -> attention over the
 * selected KV rows.
 *
 * The operation is the one described in "DeepSeek-V3.2-Exp 稀疏注意力机制(DSA)
 * 技术深度解析：从原理到 TaoToken API 实测效率提升" (sheratonhq.com), section 1:
 * a light indexer with few heads, index_head_dim 128, ReLU instead of softmax
 * and FP8 arithmetic scores every history token of each query; a top-k
 * selector keeps the k highest-scoring KV; the main attention then looks only
 * at that subset, so its cost falls from O(n^2) to O(n*k).  "DeepSeek-V4 百万
 * token 上下文的工程实现" (blog.hotdry.top), section "从 O(N²) 到 O(N・k)", names the
 * same two stages (Lightning Indexer, then a fine-grained selector).
 *
 * Definitions used by every entry point (per sequence b, query row t):
 *   pos(t)   last visible key: q_pos[b*n_q+t] if q_pos is given, else
 *            n_k - n_q + t (queries are the last n_q tokens of the sequence,
 *            the query's own position included).  Keys s > pos(t) are history
 *            of no one and never scored or selected.
 *   I[t,s] = sum_h w[t,h] * ReLU( q_I[t,h] . k_I[s] )   for s <= pos(t).
 *            With FP8 inputs q_I = sq[t]*code, k_I = sk[s]*code, so
 *            I = sq*sk * sum_h w*ReLU(code.code) exactly (scales are > 0).
 *   top-k    m = min(top_k, pos(t)+1) keys with the highest I; among equal I
 *            the lower position wins; -0.0 equals +0.0.
 *   backbone optional forced keys: the first sink_tokens keys and the last
 *            local_window visible keys of each row are always kept, and the
 *            top-k runs over the visible keys between them (m = min(top_k,
 *            their count)); the selection is the union.  This is the local
 *            window + global tokens + salience-chosen far tokens of "DeepSeek
 *            Sparse Attention" (sider.ai essay "sparse-attention-that-isn-t-
 *            sparse-thinking", section "DSA 可能如何選擇保留內容"), and the recent-
 *            window KV of "DeepSeek-V4 百万 token 上下文的工程实现", section
 *            "滑动窗口 KV Cache 与混合策略".  A selection row has W = top_k +
 *            sink_tokens + local_window entries.
 *   attn     for each query head h (kv head g = h / (q_heads/kv_heads)):
 *            z_j = softmax_scale * q[t,h].k[s_j,g] over the kept rows s_j,
 *            out = sum_j softmax(z)_j * v[s_j,g], lse = log sum_j exp(z_j).
 *            In latent mode (kv_latent = 1, kv_heads = 1) the value is the
 *            first d_v entries of the key row.
 *   cache    the main k and v may be stored in FP8 (kv_dtype = DSA_FP8_E4M3),
 *            the cache format "DeepSeek-V4 百万 token 上下文的工程实现" names
 *            in its section on the sliding-window KV cache and mixed strategy
 *            (FP8 instead of FP16, half the memory).  Each (token, kv head) row
 *            is its E4M3 codes times one fp32 scale: k[s,g] = ks[s,g] * code,
 *            v[s,g] = vs[s,g] * code; a latent value row is part of its key
 *            row and takes ks.  The attention above runs on those decoded
 *            values.  The pages fix no layout for the scales; here each
 *            token's scales sit right after its codes in one record (see
 *            DSA_FP8_KV_RECORD_BYTES below), so a gathered token's scale comes
 *            from the same memory page as its codes.
 *
 * Memory and ownership.  Every pointer inside dsa_problem_t and every output
 * pointer is DEVICE memory owned by the caller, contiguous and row-major in
 * the layouts given below; the library keeps no pointer after a call returns,
 * never allocates, frees or copies between host and device, and never
 * synchronises.  All work is enqueued on `stream` (0 = the null stream); the
 * call returns once it is enqueued.  The dsa_problem_t struct itself is host
 * memory, read only during the call.
 *
 * Errors.  Arguments are validated on the host before anything is enqueued;
 * an invalid call returns a negative status and enqueues nothing.
 * DSA_E_DEVICE reports a failed launch (the HIP error text is in
 * dsa_last_error()).  Data-dependent cases are defined, not errors: an idx
 * entry that is negative, > pos(t) or >= n_k is skipped by dsa_sparse_attn,
 * and a row with no valid entry gets out = 0 and lse = -inf.  The library
 * never prints and never aborts.  Calls are thread-safe as long as concurrent
 * calls do not share output or workspace memory; dsa_last_error() is
 * per-thread.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same typedef as HIP's own header, so both may be included together. */
typedef struct ihipStream_t *hipStream_t;

#define DSA_ABI_VERSION 4

/* Bytes of one token's record in an FP8 (DSA_FP8_E4M3) k or v cache with
 * `heads` kv heads of `dim` entries: bytes [0, heads*dim) are the E4M3 codes,
 * head g at g*dim; then `heads` little-endian fp32 scales, head g's at
 * heads*dim + 4*g; then zero padding to a multiple of 16 bytes.  Records of a
 * sequence are contiguous: token s of sequence b at (b*n_k + s) * record. */
#define DSA_FP8_KV_RECORD_BYTES(heads, dim) ((((heads) * (dim) + 4 * (heads)) + 15) / 16 * 16)

typedef enum {
    DSA_OK = 0,
    DSA_E_INVALID = -1,      /* null required pointer, non-positive size, bad combination */
    DSA_E_UNSUPPORTED = -2,  /* valid problem the library has no kernel for */
    DSA_E_WORKSPACE = -3,    /* workspace missing or smaller than dsa_workspace_bytes() */
    DSA_E_DEVICE = -4        /* a HIP launch failed; see dsa_last_error() */
} dsa_status_t;

typedef enum {
    DSA_F32 = 0,             /* IEEE binary32 */
    DSA_BF16 = 1,            /* bfloat16 */
    DSA_FP8_E4M3 = 2         /* OCP FP8 E4M3 (bias 7, max 448, no inf) + fp32 scale per token row */
} dsa_dtype_t;

typedef enum {
    DSA_OP_INDEX_SCORES = 0,
    DSA_OP_TOPK = 1,
    DSA_OP_SPARSE_ATTN = 2,
    DSA_OP_PREFILL = 3,
    DSA_OP_DECODE = 4,
    DSA_OP_DENSE_ATTN = 5,
    DSA_OP_COMPRESS_KV = 6
} dsa_op_t;

/* How the attention over the kept rows is computed; every mode gives the same
 * result up to fp32 rounding order.  "DeepSeek-V3.2-Exp 稀疏注意力机制(DSA)技术深度
 * 解析" (sheratonhq.com), section 1, says short sequences run DSA as masked MHA:
 * dense attention whose mask admits each query's selected keys. */
typedef enum {
    DSA_ATTN_AUTO = 0,       /* the library picks (the masked form for long prefill blocks
                                whose selections cover enough of each key tile) */
    DSA_ATTN_GATHER = 1,     /* gather each query's kept rows */
    DSA_ATTN_MASKED = 2      /* masked MHA: every key tile up to the block's last visible
                                key, the selection as a mask (bf16, d_qk = d_v = 128,
                                not latent, bf16 KV, n_k * Hkv * 256 B below 2 GiB;
                                else DSA_E_UNSUPPORTED) */
} dsa_attn_mode_t;

/* One problem: B sequences, each with n_q query rows and n_k key rows. */
typedef struct {
    int32_t batch;            /* B >= 1 */
    int32_t n_q;              /* query rows per sequence, 1 <= n_q <= n_k */
    int32_t n_k;              /* key rows per sequence, n_k <= 2^24 */
    const int32_t *q_pos;     /* [B*n_q] last visible key of each query, or NULL */

    /* lightning indexer */
    int32_t idx_heads;        /* H_I, 1..64 (16 in the pages' configuration) */
    int32_t idx_dim;          /* index_head_dim; must be 128 */
    int32_t idx_dtype;        /* dsa_dtype_t of iq and ik */
    const void *iq;           /* [B, n_q, H_I, idx_dim] */
    const float *iq_scale;    /* [B, n_q] one scale per query row (FP8 only, else NULL) */
    const void *ik;           /* [B, n_k, idx_dim] */
    const float *ik_scale;    /* [B, n_k] one scale per key row (FP8 only, else NULL) */
    const float *iw;          /* [B, n_q, H_I] fp32 head weights w[t,h] */

    /* main attention */
    int32_t q_heads;          /* Hq >= 1 */
    int32_t kv_heads;         /* Hkv >= 1, Hq % Hkv == 0 */
    int32_t d_qk;             /* 64, 128, or 576 (latent) */
    int32_t d_v;              /* 64, 128, or 512 (latent) */
    int32_t kv_latent;        /* 1: v is NULL, value = first d_v entries of the k row */
    int32_t attn_dtype;       /* DSA_F32 or DSA_BF16, for q and out */
    int32_t kv_dtype;         /* dtype of k and v: attn_dtype, or DSA_FP8_E4M3 when attn_dtype is DSA_BF16 */
    const void *q;            /* [B, n_q, Hq, d_qk] */
    const void *k;            /* [B, n_k, Hkv, d_qk]; FP8: [B, n_k] records of DSA_FP8_KV_RECORD_BYTES(Hkv, d_qk) */
    const void *v;            /* [B, n_k, Hkv, d_v]; FP8: [B, n_k] records of DSA_FP8_KV_RECORD_BYTES(Hkv, d_v);
                                 NULL when kv_latent */
    const float *k_scale;     /* reserved: must be NULL (FP8 scales live in the k records) */
    const float *v_scale;     /* reserved: must be NULL (FP8 scales live in the v records) */
    float softmax_scale;      /* > 0, e.g. 1/sqrt(d_qk) */

    int32_t top_k;            /* k, 1..8192 */
    int32_t attn_mode;        /* dsa_attn_mode_t */
    int32_t sink_tokens;      /* >= 0: the first sink_tokens keys are always kept (0 = none) */
    int32_t local_window;     /* >= 0: the last local_window visible keys are always kept (0 = none);
                                 top_k + sink_tokens + local_window <= 16384 */
} dsa_problem_t;

/* DSA_ABI_VERSION of the loaded library. */
int dsa_abi_version(void);

/* Workspace bytes that entry point `op` needs for problem `p` (0 if none).
 * Returns (size_t)-1 if the problem is invalid for that op; the reason is in
 * dsa_last_error(). */
size_t dsa_workspace_bytes(int op, const dsa_problem_t *p);

/* Indexer scores, unfused: scores[b][t][s] = I[t,s] (fp32) for s <= pos(t) and
 * -inf for s > pos(t).  scores: [B, n_q, n_k] fp32.  Uses the iq/ik/iw fields. */
dsa_status_t dsa_index_scores(const dsa_problem_t *p, float *scores, hipStream_t stream);

/* Top-k selector, unfused.  scores: [B, n_q, n_k] fp32 as written by
 * dsa_index_scores (entries past pos(t) are ignored whatever they hold);
 * idx: [B, n_q, W] int32 (W = top_k + sink_tokens + local_window), the kept
 * positions in ascending order, then -1: the m = min(top_k, pos(t)+1) best
 * keys, or with a backbone its forced keys and the best top_k between them.
 * Among equal scores the lower position wins. */
dsa_status_t dsa_topk(const dsa_problem_t *p, const float *scores, int32_t *idx,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Attention over the selected rows only, unfused.  idx: [B, n_q, W] int32 with
 * W = top_k + sink_tokens + local_window (any entries; invalid ones skipped);
 * out: [B, n_q, Hq, d_v] in attn_dtype; lse: [B, n_q, Hq] fp32 natural-log
 * sum-exp, or NULL. */
dsa_status_t dsa_sparse_attn(const dsa_problem_t *p, const int32_t *idx, void *out, float *lse,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Fused prefill: indexer, top-k and sparse attention for every query row.  The
 * full [n_q, n_k] score matrix is never held in memory: scores are produced
 * and consumed one bounded block of query rows at a time inside the
 * workspace.  idx_out: [B, n_q, W] (W = top_k + sink_tokens + local_window)
 * or NULL (then kept in the workspace).
 * A row with pos(t) + 1 <= W keeps every visible key whatever the scores,
 * so when q_pos is NULL, blocks of such rows skip the indexer and the top-k
 * (their selection is written as 0..pos(t) directly) and a problem made only
 * of such rows is dense causal attention. */
dsa_status_t dsa_prefill(const dsa_problem_t *p, void *out, float *lse, int32_t *idx_out,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Fused decode: as dsa_prefill for n_q == 1 (one new token per sequence whose
 * own key row is already the last cached row, unless q_pos says otherwise). */
dsa_status_t dsa_decode(const dsa_problem_t *p, void *out, float *lse, int32_t *idx_out,
                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Fused decode that allocates nothing and takes no workspace: for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Inputs, outputs and results are
 * those of dsa_decode (the same kernels run).  Its scratch is a static array
 * of DSA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; the kernels clear what must start at zero, and the
 * array keeps whatever the last call left.  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (other streams or other
 * threads) race and must not be made.  A problem whose scratch need (the
 * bytes dsa_workspace_bytes(DSA_OP_DECODE) reports, less the selection when
 * idx_out is given) exceeds DSA_NOALLOC_SCRATCH_BYTES returns
 * DSA_E_UNSUPPORTED before anything is enqueued.  The phase timer does not
 * record these calls. */
#define DSA_NOALLOC_SCRATCH_BYTES (64u << 20)
dsa_status_t dsa_decode_noalloc(const dsa_problem_t *p, void *out, float *lse, int32_t *idx_out,
                                hipStream_t stream);

/* Dense causal attention: every query row over all its visible keys, the
 * attention DSA reduces to when top_k >= pos(t) + 1 and the baseline the
 * pages measure DSA against.  Uses the main-attention fields only (q, k, v,
 * heads, dims, softmax_scale, q_pos); bf16, d_qk = d_v = 128, not latent,
 * bf16 KV, n_k * Hkv * 256 B below 2 GiB (else DSA_E_UNSUPPORTED).  out: [B, n_q, Hq, d_v] bf16; lse:
 * [B, n_q, Hq] fp32 or NULL; workspace: dsa_workspace_bytes(DSA_OP_DENSE_ATTN)
 * bytes (partial results when the key walk is split; may be 0). */
dsa_status_t dsa_dense_attn(const dsa_problem_t *p, void *out, float *lse,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Importance compression of the cached tokens, as "DeepSeek-V4 百万 token
 * 上下文的工程实现" (blog.hotdry.top), section "滑动窗口 KV Cache 与混合策略",
 * describes it: the most recent tokens keep their full K/V and the older ones
 * are cut down by an importance score to the ones that matter.  The pages give
 * no rule for the score or the cut; read here as a selection of whole tokens.
 * Per sequence b, with W = min(window, n_k) and n_old = n_k - W:
 *   - the last W tokens (positions n_old .. n_k-1) are kept;
 *   - of the old tokens 0 .. n_old-1, the min(keep_old, n_old) with the
 *     highest importance[b][s] are kept; among equal importance the lower
 *     position wins, and -0.0 equals +0.0 (NaN importance is unsupported:
 *     which of those tokens are kept is unspecified);
 *   - the kept tokens, in ascending position order, are written to slots
 *     0 .. n_keep-1 of the outputs, n_keep = dsa_compress_kept(n_k, window,
 *     keep_old) = W + min(keep_old, n_old), the same for every sequence.
 * Each kept token's rows are copied bit for bit: its k row (or FP8 record),
 * its v row (or record) unless kv_latent, its indexer key row ik and, for an
 * FP8 indexer, its ik_scale.  The outputs use the input layouts with n_k
 * replaced by n_keep, so a problem over the compressed cache (n_k = n_keep,
 * the same head counts and dtypes) runs through every other entry point.
 * importance: [B, n_k] fp32 device memory, any per-token score the caller
 * keeps (for example the indexer scores I of recent queries, or their sum).
 * Uses batch, n_k, kv_heads, d_qk, d_v, kv_latent, kv_dtype, k, v, idx_dim,
 * idx_dtype, ik and ik_scale of p (n_q and the query fields are ignored; ik
 * may be NULL, then no indexer rows are copied).  out->pos: [B, n_keep] int32,
 * the original positions.  Requires batch * n_k < 2^31 and a workspace of
 * dsa_workspace_bytes(DSA_OP_COMPRESS_KV, p) bytes.  Rows are copied 16 or 4
 * bytes at a time: each row size and its input and output pointers must be
 * multiples of 4 (else DSA_E_UNSUPPORTED).  When n_keep is 0 nothing is
 * enqueued. */
typedef struct {
    void *k;                  /* [B, n_keep] rows in p->k's layout and dtype */
    void *v;                  /* [B, n_keep] rows in p->v's layout; NULL when kv_latent */
    void *ik;                 /* [B, n_keep, idx_dim] in idx_dtype; NULL when p->ik is NULL */
    float *ik_scale;          /* [B, n_keep]; required when p->ik_scale is given, else NULL */
    int32_t *pos;             /* [B, n_keep] original positions, ascending per sequence */
} dsa_kv_compressed_t;
int32_t dsa_compress_kept(int32_t n_k, int32_t window, int32_t keep_old);
dsa_status_t dsa_compress_kv(const dsa_problem_t *p, const float *importance, int32_t window, int32_t keep_old,
                             const dsa_kv_compressed_t *out, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Phase timing of the fused entry points, for profiling.
 * dsa_phase_timing(1) makes every later dsa_prefill / dsa_decode call record
 * HIP events on its own stream: one before its first kernel and one after
 * each phase; dsa_phase_timing(0) stops it (the default).  While it is on, the
 * fused calls create HIP events the first time they need them (kept by the
 * library until the process ends), and the timer keeps only the latest call:
 * time one caller at a time.  dsa_phase_times() waits for that call's last
 * event and writes DSA_PHASE_COUNT floats to `us`, the GPU microseconds of
 * each phase summed over the call's row blocks (0 for a phase it did not
 * run).  Returns DSA_E_INVALID if us is NULL or no timed call was made. */
typedef enum {
    DSA_PHASE_PREP = 0,      /* threshold sample (decode) or histogram clear */
    DSA_PHASE_INDEX = 1,     /* indexer kernel */
    DSA_PHASE_TOPK = 2,      /* top-k selection */
    DSA_PHASE_ATTN = 3,      /* sparse attention */
    DSA_PHASE_COUNT = 4
} dsa_phase_t;
dsa_status_t dsa_phase_timing(int enable);
dsa_status_t dsa_phase_times(float *us);

/* Static text for a status code. */
const char *dsa_status_str(dsa_status_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char *dsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
