// dsa_kernels.h -- internal launch interface between the C ABI layer and the
// kernels.  Host-only structs of device pointers and sizes; not part of the
// public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

struct IndexArgs {
    int rows, row0;      // rows handled, absolute index of the first (b*n_q+t)
    int n_q, n_k, H;
    int k;               // top_k (candidate mode)
    int dtype;           // DType
    const void* iq;
    const float* iq_scale;
    const void* ik;
    const float* ik_scale;
    const float* iw;
    const int32_t* q_pos;
    float* scores;       // [rows, n_k], row 0 = absolute row row0
    uint32_t* hist;      // optional [rows][kTopkBins] top-k histogram to accumulate into
    bool visible_only;   // scores past pos(t) may be left unwritten (the top-k never reads them)
    // candidate mode (sampled top-k): per-row metadata and candidate lists
    uint32_t* meta;      // [rows][kTopkMeta]
    uint64_t* cand;      // [rows][cand_cap]
    int cand_cap;
    // backbone (candidate mode and the sampled top-k): only keys in
    // [sinks, pos + 1 - window) are ranked
    int sinks, window;
};

// Top-k workspace (device), per row r:
//   hist  [rows][2048] uint32  counts of digit 0 (key bits 31..21)
//   hist1 [rows][2048] uint32  counts of digit 1 (key bits 20..10) in the threshold bin
//   count [rows][8]    uint32  {kept above, candidates, digit-0 bin, count above it, unused}
//   cand  [rows][cap]  uint64  (low 21 key bits << 32 | ~position) candidates
// hist, hist1 and count are contiguous (zero_words words) and must start at 0.
constexpr int kTopkBins = 2048;
constexpr int kTopkMeta = 8;
// Candidates one decode-indexer workgroup (8192 keys) holds in LDS: about
// 2.5 times the most a workgroup expects when the row has 16 k keys (the
// shortest row the sampled top-k takes); more overflow the row to its exact
// recompute.
constexpr int kIdxCandBuf = 2048;
// Row metadata of the sampled top-k (TopkArgs::count / IndexArgs::meta).
// A row that falls back: S_DONE counts the finish workgroups that have
// finished their slice, S_NWIN the slice winners they appended.
enum { S_NCAND = 0, S_KLOW = 1, S_OVF = 2, S_FALLBACK = 3, S_DONE = 4, S_NWIN = 5 };
constexpr int kTopkCandCapMax = 12288;   // candidates per row kept for the LDS select
constexpr int kTopkMaxK = 8192;

struct TopkArgs {
    int rows, row0;        // rows handled, absolute index of the first (for pos)
    int n_q, n_k, k;
    const int32_t* q_pos;
    const float* scores;   // row stride n_k
    int32_t* idx;          // [rows, k]
    uint32_t* hist;
    uint32_t* hist1;
    uint32_t* count;
    size_t zero_words;
    uint64_t* cand;
    int cand_cap;
    bool hist_ready;       // hist..count were zeroed and the scores producer filled hist
    int sinks, window;     // backbone: the first `sinks` and last `window` visible keys rank as -inf
};

size_t topk_workspace_bytes(int rows, int n_k);
int topk_cand_cap(int n_k);
void topk_carve(void* ws, int rows, int n_k, TopkArgs& a);
hipError_t launch_topk(const TopkArgs& a, hipStream_t st);
// True when launch_topk selects through the digit-0 histograms (rows too long
// for the LDS select, too few for the sampled candidate lists); otherwise it
// neither reads nor clears them.
bool topk_uses_hist(const TopkArgs& a);
hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t st);
// idx[r][j] = j for j <= pos(row0 + r), else -1 (pos from n_k - n_q + t): the
// top-k result of a row that keeps every visible key.
hipError_t launch_fill_prefix_idx(int32_t* idx, int row0, int rows, int n_q, int n_k, int k, hipStream_t st);
// Backbone union: idx[r] (width k + sinks + window) = the first min(sinks,
// vis) keys, the picks[r] (width k, ascending) between the forced sets, the
// last window keys, then -1.
hipError_t launch_union_backbone(const int32_t* picks, int32_t* idx, int row0, int rows, int n_q, int n_k,
                                 const int32_t* q_pos, int k, int sinks, int window, hipStream_t st);

// Attention modes (dsa_attn_mode_t).
enum AttnMode { ATTN_AUTO = 0, ATTN_GATHER = 1, ATTN_MASKED = 2 };
constexpr int kMaskedMaxKeys = 1 << 18;  // keys of a selection bit row the masked path holds in LDS
// The masked kernels address one sequence's K and V rows (n_k x Hkv x 256
// bytes each) with 32-bit buffer offsets: the span must stay below 2^31.
inline bool masked_kv_fits(int n_k, int Hkv) {
    return static_cast<int64_t>(n_k) * Hkv * 256 < (static_cast<int64_t>(1) << 31);
}

struct AttnArgs {
    int rows, n_q, n_k, kk;
    int Hq, Hkv, dqk, dv, latent, dtype;
    int kv_dtype;          // dtype of k and v: dtype, or E4M3 (then dtype is BF16)
    const void* q;
    const void* k;         // E4M3: token records of k_rec bytes (codes of every kv head, then their scales)
    const void* v;         // E4M3: token records of v_rec bytes (latent rows: none, values use k's)
    int k_rec, v_rec;      // E4M3 record bytes (DSA_FP8_KV_RECORD_BYTES), else 0
    const int32_t* idx;    // [rows, kk]
    const int32_t* q_pos;
    float scale;
    void* out;             // [rows, Hq, dv]
    float* lse;            // [rows, Hq] or null
    int mode;              // AttnMode
    bool all_visible;      // every row keeps all keys 0..pos(t) (idx may then be ignored)
};

// Lets kernel `fn` take `bytes` of dynamic LDS on the current device.  The
// attribute is set once per (device, kernel, size reached so far): later
// launches that need no more LDS than an earlier one make no HIP call.
hipError_t allow_dyn_lds(const void* fn, size_t bytes);

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t st);
// True when launch_index_scores accumulates a.hist (the top-k's first-digit
// histogram) while it writes the scores.
bool index_fills_hist(const IndexArgs& a);
// True for the FP8 MFMA path (E4M3, <= 16 heads), which also has the
// candidate mode used by the sampled top-k.
bool index_fp8_path(const IndexArgs& a);
// Candidate mode of the FP8 indexer: no scores are written, only the keys at
// or above the row's sampled bound are appended to a.cand (see topk_sampled).
hipError_t launch_index_candidates(const IndexArgs& a, hipStream_t st);

// Sampled top-k for long rows (n_k >= 16 k): a sample of each row bounds the
// k-th score from below, the indexer keeps only keys above the bound, and an
// exact select runs over those candidates.  A row whose bound proves too high
// or whose candidates overflow is recomputed and selected in full.
struct SampledTopk {
    IndexArgs ix;          // the indexer inputs (ix.meta / ix.cand set from here)
    int32_t* idx;          // [rows, k]
    uint32_t* samples;     // [rows, kSampleKeys] order keys of the sampled scores
    float* scratch;        // [rows, n_k] fp32, used only by a recomputed row
    uint64_t* win;         // [rows, win_cap] the slice winners of a recomputed row
    int win_cap;
};
constexpr int kSampleKeys = 4096;       // keys sampled per row
constexpr int kSampleSplit = 16;        // workgroups scoring one row's sample
constexpr int kSampledCandCap = 12288;  // candidates per row
bool topk_sampled_eligible(int n_k, int k);
size_t topk_sampled_workspace_bytes(int rows, int n_k, int k);
void topk_sampled_carve(void* ws, int rows, int n_k, int k, SampledTopk& t);
hipError_t launch_topk_sample(const SampledTopk& t, hipStream_t st);
hipError_t launch_topk_finish_sampled(const SampledTopk& t, hipStream_t st);
// Attention over index sets; `ws` holds attn_workspace_bytes(a) bytes (the
// per-slice partials of the split kernel), possibly 0.
size_t attn_workspace_bytes(const AttnArgs& a);
hipError_t launch_sparse_attn(const AttnArgs& a, void* ws, hipStream_t st);
// Prefill rows as masked dense MFMA tiles (attn_masked.hip).  `ws` holds
// attn_masked_workspace_bytes(a): the selection bit rows (none with
// a.all_visible, where the mask is causal only), then the records of the
// key-range splits (none when the walk is not split).
bool attn_masked_eligible(const AttnArgs& a);
size_t attn_masked_workspace_bytes(const AttnArgs& a);
hipError_t launch_attn_masked(const AttnArgs& a, void* ws, hipStream_t st);
// Shared latent rows (576 wide, value = first 512), bf16: one workgroup per
// (row, 128 heads, slice of the index list) sharing each gathered tile in LDS
// (attn_latent.hip).
bool attn_latent_eligible(const AttnArgs& a);
size_t attn_latent_workspace_bytes(const AttnArgs& a);
hipError_t launch_attn_latent(const AttnArgs& a, float* part, hipStream_t st);
// MFMA kernel for wide rows / many heads per kv head (attn_wide.hip).
bool attn_wide_eligible(const AttnArgs& a);
size_t attn_wide_workspace_bytes(const AttnArgs& a);
hipError_t launch_attn_wide(const AttnArgs& a, float* part, hipStream_t st);
// Combine per-slice records part[(row*Hq + head)*nsplit + slice] = (max (base 2),
// sum, unnormalised O[dv]) into out and lse (bf16 out).
hipError_t launch_attn_merge(const AttnArgs& a, int nsplit, const float* part, hipStream_t st);

// Importance compression of cached tokens (compress.hip): per sequence the
// last `window` tokens and the `keep` older tokens of highest importance
// (lower position first among equal importance) are copied, in position
// order, into [B, n_keep] outputs.  Rows are opaque bytes (a multiple of 4).
struct CompressArgs {
    int B, n_k, window, keep, n_keep, nch;   // window <= n_k, keep <= n_k - window, n_keep = window + keep
    const float* imp;                        // [B, n_k]
    int nrow;                                // row arrays to copy (<= 4)
    const uint8_t* src[4];
    uint8_t* dst[4];
    int bytes[4];                            // bytes per token of each array
    int unit[4];                             // 16 or 4: bytes per vector load and store
    int32_t* pos_out;                        // [B, n_keep] original positions
    uint32_t* ws;                            // compress_workspace_bytes(B, n_k)
};
int compress_chunks(int n_k);
size_t compress_workspace_bytes(int batch, int n_k);
hipError_t launch_compress(const CompressArgs& a, hipStream_t st);

}  // namespace dsa
