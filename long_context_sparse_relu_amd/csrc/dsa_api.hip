// dsa_api.hip -- the C ABI declared in include/dsa.h: host-side validation,
// workspace layout and launch sequencing on the caller's stream.  Nothing here
// allocates device memory, copies or synchronises; only the opt-in phase timer
// creates HIP events and waits on them.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "dsa.h"
#include "dsa_kernels.h"

namespace {

thread_local std::string g_last_error;

dsa_status_t fail(dsa_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dsa_status_t fail(dsa_status_t st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

dsa_status_t device_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return DSA_OK;
    return fail(DSA_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// Opt-in phase timer: events recorded on the caller's stream between the
// phases of one fused call, reused by the next timed call.
struct PhaseTimer {
    std::mutex mu;
    bool on = false;
    int device = -1;
    std::vector<hipEvent_t> ev;   // ev[0] before the first kernel, ev[i] after a phase
    std::vector<int> phase;       // phase[i]: the phase ending at ev[i]
    int used = 0;
};
PhaseTimer g_timer;

hipError_t timer_mark(int ph, hipStream_t st) {
    std::lock_guard<std::mutex> lk(g_timer.mu);
    if (!g_timer.on) return hipSuccess;
    if (ph < 0) {                              // a new call
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        if (dev != g_timer.device) {           // events belong to the device current at creation
            for (hipEvent_t x : g_timer.ev) (void)hipEventDestroy(x);
            g_timer.ev.clear();
            g_timer.phase.clear();
            g_timer.device = dev;
        }
        g_timer.used = 0;
    }
    if (g_timer.used == static_cast<int>(g_timer.ev.size())) {
        hipEvent_t x;
        hipError_t e = hipEventCreate(&x);
        if (e != hipSuccess) return e;
        g_timer.ev.push_back(x);
        g_timer.phase.push_back(-1);
    }
    g_timer.phase[g_timer.used] = ph;
    return hipEventRecord(g_timer.ev[g_timer.used++], st);
}

constexpr int kMaxNk = 1 << 24;
constexpr int kMaxSelWidth = 16384;   // entries of a selection row (top_k + sinks + window)
constexpr size_t kAlign = 256;
// Query rows whose scores the fused prefill keeps at once (bounded scratch).
#ifndef DSA_PREFILL_SCORE_MB
#define DSA_PREFILL_SCORE_MB 256
#endif
constexpr size_t kPrefillScoreBytes = size_t(DSA_PREFILL_SCORE_MB) << 20;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

dsa_status_t check_common(const dsa_problem_t* p) {
    if (!p) return fail(DSA_E_INVALID, "problem pointer is NULL");
    if (p->batch < 1 || p->n_q < 1 || p->n_k < 1)
        return fail(DSA_E_INVALID, "batch, n_q and n_k must be >= 1 (got %d, %d, %d)", p->batch, p->n_q, p->n_k);
    if (p->n_q > p->n_k) return fail(DSA_E_INVALID, "n_q (%d) exceeds n_k (%d)", p->n_q, p->n_k);
    if (p->n_k > kMaxNk) return fail(DSA_E_UNSUPPORTED, "n_k %d exceeds %d", p->n_k, kMaxNk);
    if (static_cast<int64_t>(p->batch) * p->n_q > (int64_t(1) << 30))
        return fail(DSA_E_UNSUPPORTED, "batch*n_q too large");
    return DSA_OK;
}

dsa_status_t check_index(const dsa_problem_t* p) {
    if (p->idx_heads < 1 || p->idx_heads > 64)
        return fail(DSA_E_UNSUPPORTED, "idx_heads must be in 1..64 (got %d)", p->idx_heads);
    if (p->idx_dim != 128) return fail(DSA_E_UNSUPPORTED, "idx_dim must be 128 (got %d)", p->idx_dim);
    if (p->idx_dtype != DSA_F32 && p->idx_dtype != DSA_BF16 && p->idx_dtype != DSA_FP8_E4M3)
        return fail(DSA_E_INVALID, "idx_dtype %d is not a dsa_dtype_t", p->idx_dtype);
    if (!p->iq || !p->ik || !p->iw) return fail(DSA_E_INVALID, "iq, ik and iw are required");
    if (p->idx_dtype == DSA_FP8_E4M3 && (!p->iq_scale || !p->ik_scale))
        return fail(DSA_E_INVALID, "FP8 indexer inputs need iq_scale and ik_scale");
    return DSA_OK;
}

dsa_status_t check_topk(const dsa_problem_t* p) {
    if (p->top_k < 1 || p->top_k > dsa::kTopkMaxK)
        return fail(DSA_E_UNSUPPORTED, "top_k must be in 1..%d (got %d)", dsa::kTopkMaxK, p->top_k);
    if (p->sink_tokens < 0 || p->local_window < 0)
        return fail(DSA_E_INVALID, "sink_tokens and local_window must be >= 0 (got %d, %d)", p->sink_tokens,
                    p->local_window);
    if (static_cast<int64_t>(p->top_k) + p->sink_tokens + p->local_window > kMaxSelWidth)
        return fail(DSA_E_UNSUPPORTED, "top_k + sink_tokens + local_window must be <= %d", kMaxSelWidth);
    return DSA_OK;
}

static_assert(int(DSA_ATTN_AUTO) == int(dsa::ATTN_AUTO) && int(DSA_ATTN_GATHER) == int(dsa::ATTN_GATHER) &&
              int(DSA_ATTN_MASKED) == int(dsa::ATTN_MASKED), "attention modes");

// Shapes the masked (dense tile) kernels take.
bool masked_shape(const dsa_problem_t* p) {
    return p->attn_dtype == DSA_BF16 && p->kv_dtype == DSA_BF16 && !p->kv_latent && p->d_qk == 128 &&
           p->d_v == 128 && dsa::masked_kv_fits(p->n_k, p->kv_heads);
}

dsa_status_t check_attn(const dsa_problem_t* p) {
    if (p->q_heads < 1 || p->kv_heads < 1 || p->q_heads % p->kv_heads)
        return fail(DSA_E_INVALID, "q_heads (%d) must be a positive multiple of kv_heads (%d)", p->q_heads, p->kv_heads);
    if (p->attn_dtype != DSA_F32 && p->attn_dtype != DSA_BF16)
        return fail(DSA_E_UNSUPPORTED, "attn_dtype must be DSA_F32 or DSA_BF16 (got %d)", p->attn_dtype);
    if (p->kv_dtype == DSA_FP8_E4M3) {
        if (p->attn_dtype != DSA_BF16)
            return fail(DSA_E_UNSUPPORTED, "an FP8 KV cache needs attn_dtype DSA_BF16");
        if (p->k_scale || p->v_scale)
            return fail(DSA_E_INVALID, "k_scale and v_scale are reserved (NULL): an FP8 cache keeps its scales "
                                       "in its token records");
    } else if (p->kv_dtype != p->attn_dtype) {
        return fail(DSA_E_INVALID, "kv_dtype (%d) must equal attn_dtype (%d) or be DSA_FP8_E4M3",
                    p->kv_dtype, p->attn_dtype);
    }
    if (p->d_qk < 1 || p->d_qk > 576 || p->d_v < 1 || p->d_v > 512)
        return fail(DSA_E_UNSUPPORTED, "need 1 <= d_qk <= 576 and 1 <= d_v <= 512 (got %d, %d)", p->d_qk, p->d_v);
    if (p->kv_latent) {
        if (p->kv_heads != 1) return fail(DSA_E_INVALID, "latent rows need kv_heads == 1");
        if (p->d_v > p->d_qk) return fail(DSA_E_INVALID, "latent rows need d_v <= d_qk");
    } else if (!p->v) {
        return fail(DSA_E_INVALID, "v is required unless kv_latent");
    }
    if (!p->q || !p->k) return fail(DSA_E_INVALID, "q and k are required");
    if (!(p->softmax_scale > 0.0f) || !std::isfinite(p->softmax_scale))
        return fail(DSA_E_INVALID, "softmax_scale must be finite and > 0");
    if (p->attn_mode != DSA_ATTN_AUTO && p->attn_mode != DSA_ATTN_GATHER && p->attn_mode != DSA_ATTN_MASKED)
        return fail(DSA_E_INVALID, "attn_mode %d is not a dsa_attn_mode_t", p->attn_mode);
    if (p->attn_mode == DSA_ATTN_MASKED && (!masked_shape(p) || p->n_k > dsa::kMaskedMaxKeys))
        return fail(DSA_E_UNSUPPORTED, "masked attention needs bf16 q and KV, d_qk = d_v = 128, no latent rows, "
                    "n_k <= %d and n_k * kv_heads * 256 B below 2 GiB", dsa::kMaskedMaxKeys);
    return DSA_OK;
}

// The cached-token fields dsa_compress_kv reads.
dsa_status_t check_cache(const dsa_problem_t* p) {
    if (p->kv_heads < 1) return fail(DSA_E_INVALID, "kv_heads must be >= 1 (got %d)", p->kv_heads);
    if (p->kv_dtype != DSA_F32 && p->kv_dtype != DSA_BF16 && p->kv_dtype != DSA_FP8_E4M3)
        return fail(DSA_E_INVALID, "kv_dtype %d is not a dsa_dtype_t", p->kv_dtype);
    if (p->d_qk < 1 || p->d_qk > 576 || p->d_v < 1 || p->d_v > 512)
        return fail(DSA_E_UNSUPPORTED, "need 1 <= d_qk <= 576 and 1 <= d_v <= 512 (got %d, %d)", p->d_qk, p->d_v);
    if (!p->k) return fail(DSA_E_INVALID, "k is required");
    if (p->kv_latent ? p->kv_heads != 1 : !p->v)
        return fail(DSA_E_INVALID, "latent rows need kv_heads == 1; otherwise v is required");
    if (p->ik) {
        if (p->idx_dim != 128) return fail(DSA_E_UNSUPPORTED, "idx_dim must be 128 (got %d)", p->idx_dim);
        if (p->idx_dtype != DSA_F32 && p->idx_dtype != DSA_BF16 && p->idx_dtype != DSA_FP8_E4M3)
            return fail(DSA_E_INVALID, "idx_dtype %d is not a dsa_dtype_t", p->idx_dtype);
        if (p->idx_dtype == DSA_FP8_E4M3 && !p->ik_scale)
            return fail(DSA_E_INVALID, "FP8 indexer keys need ik_scale");
    }
    if (static_cast<int64_t>(p->batch) * p->n_k >= (int64_t(1) << 31))
        return fail(DSA_E_UNSUPPORTED, "batch * n_k must be below 2^31");
    return DSA_OK;
}

// Bytes per token of a k (or v) cache row of `dim` entries.
int cache_row_bytes(const dsa_problem_t* p, int dim) {
    if (p->kv_dtype == DSA_FP8_E4M3) return DSA_FP8_KV_RECORD_BYTES(p->kv_heads, dim);
    return p->kv_heads * dim * (p->kv_dtype == DSA_F32 ? 4 : 2);
}

int rows_of(const dsa_problem_t* p) { return p->batch * p->n_q; }

// Entries of a selection row: the k picks plus a backbone's forced keys.
int sel_width(const dsa_problem_t* p) { return p->top_k + p->sink_tokens + p->local_window; }
bool has_backbone(const dsa_problem_t* p) { return p->sink_tokens > 0 || p->local_window > 0; }

dsa::IndexArgs index_args(const dsa_problem_t* p, int row0, int rows, float* scores) {
    dsa::IndexArgs a{};
    a.rows = rows; a.row0 = row0;
    a.n_q = p->n_q; a.n_k = p->n_k; a.H = p->idx_heads; a.dtype = p->idx_dtype;
    a.iq = p->iq; a.iq_scale = p->iq_scale;
    a.ik = p->ik; a.ik_scale = p->ik_scale;
    a.iw = p->iw;
    a.q_pos = p->q_pos;
    a.scores = scores;
    a.sinks = p->sink_tokens; a.window = p->local_window;
    return a;
}

dsa::TopkArgs topk_args(const dsa_problem_t* p, int row0, int rows, const float* scores,
                        int32_t* idx, void* ws) {
    dsa::TopkArgs a{};
    a.rows = rows; a.row0 = row0;
    a.n_q = p->n_q; a.n_k = p->n_k; a.k = p->top_k;
    a.sinks = p->sink_tokens; a.window = p->local_window;
    a.q_pos = p->q_pos;
    a.scores = scores;
    a.idx = idx;
    dsa::topk_carve(ws, rows, p->n_k, a);
    a.hist_ready = false;
    return a;
}

dsa::AttnArgs attn_args(const dsa_problem_t* p, const int32_t* idx, void* out, float* lse) {
    dsa::AttnArgs a{};
    a.rows = rows_of(p); a.n_q = p->n_q; a.n_k = p->n_k; a.kk = sel_width(p);
    a.Hq = p->q_heads; a.Hkv = p->kv_heads; a.dqk = p->d_qk; a.dv = p->d_v;
    a.latent = p->kv_latent ? 1 : 0; a.dtype = p->attn_dtype; a.kv_dtype = p->kv_dtype;
    a.q = p->q; a.k = p->k; a.v = p->v; a.idx = idx; a.q_pos = p->q_pos;
    if (p->kv_dtype == DSA_FP8_E4M3) {
        a.k_rec = DSA_FP8_KV_RECORD_BYTES(p->kv_heads, p->d_qk);
        a.v_rec = p->kv_latent ? 0 : DSA_FP8_KV_RECORD_BYTES(p->kv_heads, p->d_v);
    }
    a.scale = p->softmax_scale; a.out = out; a.lse = lse;
    a.mode = p->attn_mode; a.all_visible = false;
    return a;
}

// Attention over every visible key (the causal-only masked kernels).
dsa::AttnArgs dense_args(const dsa_problem_t* p, void* out, float* lse) {
    dsa::AttnArgs a = attn_args(p, nullptr, out, lse);
    a.kk = 0;
    a.mode = dsa::ATTN_MASKED;
    a.all_visible = true;
    return a;
}

// Last visible key of the rows [r0, r0 + nr) at most, when q_pos is NULL
// (pos(t) = n_k - n_q + t); -1 ("unknown") when q_pos is given.
int block_max_pos(const dsa_problem_t* p, int r0, int nr) {
    if (p->q_pos) return -1;
    const int last = r0 + nr - 1;
    const int t_max = (r0 / p->n_q == last / p->n_q) ? last % p->n_q : p->n_q - 1;
    return p->n_k - p->n_q + t_max;
}

// Every row of the block keeps all its visible keys (top_k + sinks + window
// >= pos(t) + 1): the selection is 0..pos(t) whatever the scores.
bool block_keeps_all(const dsa_problem_t* p, int r0, int nr) {
    const int mp = block_max_pos(p, r0, nr);
    return mp >= 0 && mp + 1 <= sel_width(p);
}

// Rows of scores the fused paths produce per round.
int fused_block_rows(const dsa_problem_t* p) {
    size_t per_row = static_cast<size_t>(p->n_k) * sizeof(float);
    size_t r = kPrefillScoreBytes / per_row;
    if (r < 1) r = 1;
    if (r > static_cast<size_t>(rows_of(p))) r = rows_of(p);
    return static_cast<int>(r);
}

// The sampled top-k (no score rows in memory) serves decode-shaped problems
// with long FP8 rows; prefill (the tiled indexer) and other problems go
// through score blocks and the full radix select.
bool use_sampled(const dsa_problem_t* p) {
    dsa::IndexArgs probe{};
    probe.dtype = p->idx_dtype;
    probe.H = p->idx_heads;
    return p->n_q < 16 && dsa::index_fp8_path(probe) && dsa::topk_sampled_eligible(p->n_k, p->top_k);
}

struct FusedLayout {
    bool sampled;
    int block_rows;
    size_t scores_off, topk_off, picks_off, idx_off, attn_off, total;
};

FusedLayout fused_layout(const dsa_problem_t* p, bool need_idx) {
    FusedLayout L{};
    L.sampled = use_sampled(p);
    L.block_rows = fused_block_rows(p);
    L.scores_off = 0;
    if (L.sampled) {
        L.topk_off = 0;
        L.picks_off = align_up(dsa::topk_sampled_workspace_bytes(L.block_rows, p->n_k, p->top_k));
        L.idx_off = L.picks_off + (has_backbone(p) ? align_up(static_cast<size_t>(L.block_rows) * p->top_k *
                                                              sizeof(int32_t)) : 0);
    } else {
        L.topk_off = align_up(static_cast<size_t>(L.block_rows) * p->n_k * sizeof(float));
        L.picks_off = L.topk_off + align_up(dsa::topk_workspace_bytes(L.block_rows, p->n_k));
        // a backbone's top-k picks of one block, before the union
        L.idx_off = L.picks_off + (has_backbone(p) ? align_up(static_cast<size_t>(L.block_rows) * p->top_k *
                                                              sizeof(int32_t)) : 0);
    }
    L.attn_off = L.idx_off + (need_idx ? align_up(static_cast<size_t>(rows_of(p)) * sel_width(p) * sizeof(int32_t)) : 0);
    dsa::AttnArgs aa = attn_args(p, nullptr, nullptr, nullptr);
    aa.all_visible = block_keeps_all(p, 0, rows_of(p));
    L.total = L.attn_off + align_up(dsa::attn_workspace_bytes(aa));
    return L;
}

// dsa_topk's workspace: the select's own, then a backbone's picks.
size_t topk_ws_bytes(const dsa_problem_t* p) {
    const size_t sel = align_up(dsa::topk_workspace_bytes(rows_of(p), p->n_k));
    return sel + (has_backbone(p) ? static_cast<size_t>(rows_of(p)) * p->top_k * sizeof(int32_t) : 0);
}

// timed = false: the phase timer is bypassed (it creates HIP events).
dsa_status_t run_fused(const dsa_problem_t* p, void* out, float* lse, int32_t* idx_out,
                       void* ws, size_t ws_bytes, hipStream_t st, bool timed = true) {
    FusedLayout L = fused_layout(p, idx_out == nullptr);
    if (!ws || ws_bytes < L.total)
        return fail(DSA_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, L.total);
    unsigned char* base = static_cast<unsigned char*>(ws);
    int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(base + L.idx_off);
    const int rows = rows_of(p);
    dsa_status_t s = timed ? device_status(timer_mark(-1, st), "phase timer") : DSA_OK;
    if (s != DSA_OK) return s;
    auto mark = [&](int ph) { return timed ? device_status(timer_mark(ph, st), "phase timer") : DSA_OK; };
    for (int r0 = 0; r0 < rows; r0 += L.block_rows) {
        int nr = rows - r0 < L.block_rows ? rows - r0 : L.block_rows;
        if (block_keeps_all(p, r0, nr)) {
            // no indexer and no top-k: the selection of every row is 0..pos(t)
            s = device_status(dsa::launch_fill_prefix_idx(idx + static_cast<size_t>(r0) * sel_width(p), r0, nr,
                                                          p->n_q, p->n_k, sel_width(p), st), "selection fill");
            if (s != DSA_OK || (s = mark(DSA_PHASE_TOPK)) != DSA_OK) return s;
            continue;
        }
        if (L.sampled) {
            dsa::SampledTopk t{};
            t.ix = index_args(p, r0, nr, nullptr);
            t.ix.k = p->top_k;
            int32_t* picks = has_backbone(p) ? reinterpret_cast<int32_t*>(base + L.picks_off)
                                             : idx + static_cast<size_t>(r0) * p->top_k;
            t.idx = picks;
            dsa::topk_sampled_carve(base, nr, p->n_k, p->top_k, t);
            s = device_status(dsa::launch_topk_sample(t, st), "top-k sample launch");
            if (s != DSA_OK || (s = mark(DSA_PHASE_PREP)) != DSA_OK) return s;
            s = device_status(dsa::launch_index_candidates(t.ix, st), "indexer launch");
            if (s != DSA_OK || (s = mark(DSA_PHASE_INDEX)) != DSA_OK) return s;
            s = device_status(dsa::launch_topk_finish_sampled(t, st), "top-k launch");
            if (s == DSA_OK && has_backbone(p))
                s = device_status(dsa::launch_union_backbone(picks, idx + static_cast<size_t>(r0) * sel_width(p), r0,
                                                             nr, p->n_q, p->n_k, p->q_pos, p->top_k, p->sink_tokens,
                                                             p->local_window, st), "backbone union");
            if (s != DSA_OK || (s = mark(DSA_PHASE_TOPK)) != DSA_OK) return s;
            continue;
        }
        float* scores = reinterpret_cast<float*>(base + L.scores_off);
        dsa::IndexArgs ia = index_args(p, r0, nr, scores);
        ia.visible_only = true;
        int32_t* picks = has_backbone(p) ? reinterpret_cast<int32_t*>(base + L.picks_off)
                                         : idx + static_cast<size_t>(r0) * p->top_k;
        dsa::TopkArgs ta = topk_args(p, r0, nr, scores, picks, base + L.topk_off);
        // (the indexer's histogram counts the real scores; a backbone ranks its
        // forced keys as -inf, so the top-k builds its own)
        if (dsa::index_fills_hist(ia) && dsa::topk_uses_hist(ta) && !has_backbone(p)) {
            // the indexer builds the first-digit histogram as it writes the scores
            ia.hist = ta.hist;
            ta.hist_ready = true;
            s = device_status(dsa::launch_zero_u32(ta.hist, ta.zero_words, st), "workspace clear");
            if (s != DSA_OK || (s = mark(DSA_PHASE_PREP)) != DSA_OK) return s;
        }
        s = device_status(dsa::launch_index_scores(ia, st), "indexer launch");
        if (s != DSA_OK || (s = mark(DSA_PHASE_INDEX)) != DSA_OK) return s;
        s = device_status(dsa::launch_topk(ta, st), "top-k launch");
        if (s == DSA_OK && has_backbone(p))
            s = device_status(dsa::launch_union_backbone(picks, idx + static_cast<size_t>(r0) * sel_width(p), r0, nr,
                                                         p->n_q, p->n_k, p->q_pos, p->top_k, p->sink_tokens,
                                                         p->local_window, st), "backbone union");
        if (s != DSA_OK || (s = mark(DSA_PHASE_TOPK)) != DSA_OK) return s;
    }
    dsa::AttnArgs aa = attn_args(p, idx, out, lse);
    aa.all_visible = block_keeps_all(p, 0, rows);
    s = device_status(dsa::launch_sparse_attn(aa, base + L.attn_off, st), "attention launch");
    if (s != DSA_OK) return s;
    return mark(DSA_PHASE_ATTN);
}

// Scratch of dsa_decode_noalloc.  Each GPU the library runs on holds its own
// copy of this array until the process ends.  On the host its name is a
// stand-in, not a device address: host code uses only the address
// hipGetSymbolAddress returns for the current device (kept per device below).
__device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

constexpr int kScratchDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// The current device's copy of `scratch`, looked up once per device with that
// device current.
dsa_status_t scratch_ptr(void** out) {
    int dev = 0;
    dsa_status_t s = device_status(hipGetDevice(&dev), "hipGetDevice");
    if (s != DSA_OK) return s;
    if (dev < 0 || dev >= kScratchDevices)
        return fail(DSA_E_UNSUPPORTED, "device %d is beyond the %d devices the static scratch serves", dev,
                    kScratchDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        s = device_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (s != DSA_OK) return s;
        if (!ptr) return fail(DSA_E_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return DSA_OK;
}

}  // namespace

namespace dsa {

hipError_t allow_dyn_lds(const void* fn, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;             // below the default limit
    struct Entry { int device; const void* fn; size_t bytes; };
    static std::mutex mu;
    static std::vector<Entry> set;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lk(mu);
    for (Entry& x : set) {
        if (x.device != dev || x.fn != fn) continue;
        if (bytes <= x.bytes) return hipSuccess;
        if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes))) !=
            hipSuccess)
            return e;
        x.bytes = bytes;
        return hipSuccess;
    }
    if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes))) !=
        hipSuccess)
        return e;
    set.push_back(Entry{dev, fn, bytes});
    return hipSuccess;
}

}  // namespace dsa

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

size_t dsa_workspace_bytes(int op, const dsa_problem_t* p) {
    dsa_status_t s = check_common(p);
    if (s != DSA_OK) return static_cast<size_t>(-1);
    switch (op) {
        case DSA_OP_INDEX_SCORES: return 0;
        case DSA_OP_SPARSE_ATTN:
            if (check_topk(p) != DSA_OK || check_attn(p) != DSA_OK) return static_cast<size_t>(-1);
            return dsa::attn_workspace_bytes(attn_args(p, nullptr, nullptr, nullptr));
        case DSA_OP_TOPK:
            if (check_topk(p) != DSA_OK) return static_cast<size_t>(-1);
            return topk_ws_bytes(p);
        case DSA_OP_PREFILL:
        case DSA_OP_DECODE:
            // the same checks as the entry points: the layout divides by head counts
            if (check_index(p) != DSA_OK || check_topk(p) != DSA_OK || check_attn(p) != DSA_OK)
                return static_cast<size_t>(-1);
            if (op == DSA_OP_DECODE && p->n_q != 1) {
                fail(DSA_E_INVALID, "dsa_decode takes n_q == 1 (got %d)", p->n_q);
                return static_cast<size_t>(-1);
            }
            return fused_layout(p, true).total;
        case DSA_OP_COMPRESS_KV:
            if (check_cache(p) != DSA_OK) return static_cast<size_t>(-1);
            return dsa::compress_workspace_bytes(p->batch, p->n_k);
        case DSA_OP_DENSE_ATTN:
            if (check_attn(p) != DSA_OK) return static_cast<size_t>(-1);
            if (!masked_shape(p)) {
                fail(DSA_E_UNSUPPORTED, "dense attention needs bf16 q and KV, d_qk = d_v = 128, no latent rows "
                     "and n_k * kv_heads * 256 B below 2 GiB");
                return static_cast<size_t>(-1);
            }
            return dsa::attn_masked_workspace_bytes(dense_args(p, nullptr, nullptr));
        default:
            fail(DSA_E_INVALID, "unknown op %d", op);
            return static_cast<size_t>(-1);
    }
}

dsa_status_t dsa_index_scores(const dsa_problem_t* p, float* scores, hipStream_t stream) {
    g_last_error.clear();
    dsa_status_t s;
    if ((s = check_common(p)) != DSA_OK || (s = check_index(p)) != DSA_OK) return s;
    if (!scores) return fail(DSA_E_INVALID, "scores is NULL");
    dsa::IndexArgs a = index_args(p, 0, rows_of(p), scores);
    return device_status(dsa::launch_index_scores(a, stream), "indexer launch");
}

dsa_status_t dsa_topk(const dsa_problem_t* p, const float* scores, int32_t* idx,
                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
    g_last_error.clear();
    dsa_status_t s;
    if ((s = check_common(p)) != DSA_OK || (s = check_topk(p)) != DSA_OK) return s;
    if (!scores || !idx) return fail(DSA_E_INVALID, "scores and idx are required");
    size_t need = topk_ws_bytes(p);
    if (!workspace || workspace_bytes < need)
        return fail(DSA_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
    if (!has_backbone(p)) {
        dsa::TopkArgs a = topk_args(p, 0, rows_of(p), scores, idx, workspace);
        return device_status(dsa::launch_topk(a, stream), "top-k launch");
    }
    int32_t* picks = reinterpret_cast<int32_t*>(static_cast<unsigned char*>(workspace) +
                                                align_up(dsa::topk_workspace_bytes(rows_of(p), p->n_k)));
    dsa::TopkArgs a = topk_args(p, 0, rows_of(p), scores, picks, workspace);
    s = device_status(dsa::launch_topk(a, stream), "top-k launch");
    if (s != DSA_OK) return s;
    return device_status(dsa::launch_union_backbone(picks, idx, 0, rows_of(p), p->n_q, p->n_k, p->q_pos, p->top_k,
                                                    p->sink_tokens, p->local_window, stream), "backbone union");
}

dsa_status_t dsa_sparse_attn(const dsa_problem_t* p, const int32_t* idx, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    g_last_error.clear();
    dsa_status_t s;
    if ((s = check_common(p)) != DSA_OK || (s = check_topk(p)) != DSA_OK || (s = check_attn(p)) != DSA_OK)
        return s;
    if (!idx || !out) return fail(DSA_E_INVALID, "idx and out are required");
    dsa::AttnArgs a = attn_args(p, idx, out, lse);
    const size_t need = dsa::attn_workspace_bytes(a);
    if (need && (!workspace || workspace_bytes < need))
        return fail(DSA_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
    return device_status(dsa::launch_sparse_attn(a, workspace, stream), "attention launch");
}

dsa_status_t dsa_prefill(const dsa_problem_t* p, void* out, float* lse, int32_t* idx_out,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
    g_last_error.clear();
    dsa_status_t s;
    if ((s = check_common(p)) != DSA_OK || (s = check_index(p)) != DSA_OK ||
        (s = check_topk(p)) != DSA_OK || (s = check_attn(p)) != DSA_OK)
        return s;
    if (!out) return fail(DSA_E_INVALID, "out is required");
    return run_fused(p, out, lse, idx_out, workspace, workspace_bytes, stream);
}

dsa_status_t dsa_decode(const dsa_problem_t* p, void* out, float* lse, int32_t* idx_out,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
    g_last_error.clear();
    dsa_status_t s;
    if ((s = check_common(p)) != DSA_OK) return s;
    if (p->n_q != 1) return fail(DSA_E_INVALID, "dsa_decode takes n_q == 1 (got %d)", p->n_q);
    if ((s = check_index(p)) != DSA_OK || (s = check_topk(p)) != DSA_OK || (s = check_attn(p)) != DSA_OK)
        return s;
    if (!out) return fail(DSA_E_INVALID, "out is required");
    return run_fused(p, out, lse, idx_out, workspace, workspace_bytes, stream);
}

dsa_status_t dsa_decode_noalloc(const dsa_problem_t* p, void* out, float* lse, int32_t* idx_out,
                                hipStream_t stream) {
    g_last_error.clear();
    dsa_status_t s;
    if ((s = check_common(p)) != DSA_OK) return s;
    if (p->n_q != 1) return fail(DSA_E_INVALID, "dsa_decode_noalloc takes n_q == 1 (got %d)", p->n_q);
    if ((s = check_index(p)) != DSA_OK || (s = check_topk(p)) != DSA_OK || (s = check_attn(p)) != DSA_OK)
        return s;
    if (!out) return fail(DSA_E_INVALID, "out is required");
    const size_t need = fused_layout(p, idx_out == nullptr).total;
    if (need > static_cast<size_t>(DSA_NOALLOC_SCRATCH_BYTES))
        return fail(DSA_E_UNSUPPORTED, "dsa_decode_noalloc: this problem needs %zu bytes of scratch and the "
                    "static scratch holds %zu; call dsa_decode with a workspace instead", need,
                    static_cast<size_t>(DSA_NOALLOC_SCRATCH_BYTES));
    void* ws = nullptr;
    if ((s = scratch_ptr(&ws)) != DSA_OK) return s;
    return run_fused(p, out, lse, idx_out, ws, DSA_NOALLOC_SCRATCH_BYTES, stream, /*timed=*/false);
}

dsa_status_t dsa_dense_attn(const dsa_problem_t* p, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    g_last_error.clear();
    dsa_status_t s;
    if ((s = check_common(p)) != DSA_OK || (s = check_attn(p)) != DSA_OK) return s;
    if (!masked_shape(p))
        return fail(DSA_E_UNSUPPORTED, "dense attention needs bf16 q and KV, d_qk = d_v = 128, no latent rows "
                    "and n_k * kv_heads * 256 B below 2 GiB");
    if (!out) return fail(DSA_E_INVALID, "out is required");
    dsa::AttnArgs a = dense_args(p, out, lse);
    const size_t need = dsa::attn_masked_workspace_bytes(a);
    if (need && (!workspace || workspace_bytes < need))
        return fail(DSA_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
    return device_status(dsa::launch_attn_masked(a, workspace, stream), "attention launch");
}

dsa_status_t dsa_phase_timing(int enable) {
    g_last_error.clear();
    std::lock_guard<std::mutex> lk(g_timer.mu);
    g_timer.on = enable != 0;
    g_timer.used = 0;
    return DSA_OK;
}

dsa_status_t dsa_phase_times(float* us) {
    g_last_error.clear();
    if (!us) return fail(DSA_E_INVALID, "us is NULL");
    std::lock_guard<std::mutex> lk(g_timer.mu);
    if (g_timer.used < 2) return fail(DSA_E_INVALID, "no timed fused call");
    for (int i = 0; i < DSA_PHASE_COUNT; ++i) us[i] = 0.0f;
    dsa_status_t s = device_status(hipEventSynchronize(g_timer.ev[g_timer.used - 1]), "phase timer");
    if (s != DSA_OK) return s;
    for (int i = 1; i < g_timer.used; ++i) {
        float ms = 0.0f;
        s = device_status(hipEventElapsedTime(&ms, g_timer.ev[i - 1], g_timer.ev[i]), "phase timer");
        if (s != DSA_OK) return s;
        us[g_timer.phase[i]] += ms * 1000.0f;
    }
    return DSA_OK;
}

const char* dsa_status_str(dsa_status_t status) {
    switch (status) {
        case DSA_OK: return "DSA_OK";
        case DSA_E_INVALID: return "DSA_E_INVALID: invalid argument";
        case DSA_E_UNSUPPORTED: return "DSA_E_UNSUPPORTED: valid problem the library has no kernel for";
        case DSA_E_WORKSPACE: return "DSA_E_WORKSPACE: workspace missing or too small";
        case DSA_E_DEVICE: return "DSA_E_DEVICE: HIP launch failed";
        default: return "unknown dsa_status_t";
    }
}

const char* dsa_last_error(void) { return g_last_error.c_str(); }


int32_t dsa_compress_kept(int32_t n_k, int32_t window, int32_t keep_old) {
    if (n_k < 0 || window < 0 || keep_old < 0) return 0;
    const int32_t w = window < n_k ? window : n_k;
    const int32_t n_old = n_k - w;
    return w + (keep_old < n_old ? keep_old : n_old);
}

dsa_status_t dsa_compress_kv(const dsa_problem_t* p, const float* importance, int32_t window, int32_t keep_old,
                             const dsa_kv_compressed_t* out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
    if (!p) return fail(DSA_E_INVALID, "problem pointer is NULL");
    if (p->batch < 1 || p->n_k < 1)
        return fail(DSA_E_INVALID, "batch and n_k must be >= 1 (got %d, %d)", p->batch, p->n_k);
    if (p->n_k > kMaxNk) return fail(DSA_E_UNSUPPORTED, "n_k %d exceeds %d", p->n_k, kMaxNk);
    dsa_status_t s = check_cache(p);
    if (s != DSA_OK) return s;
    if (window < 0 || keep_old < 0)
        return fail(DSA_E_INVALID, "window and keep_old must be >= 0 (got %d, %d)", window, keep_old);
    if (!importance || !out || !out->k || !out->pos) return fail(DSA_E_INVALID, "importance, out, out->k and out->pos are required");
    if (!p->kv_latent && !out->v) return fail(DSA_E_INVALID, "out->v is required unless kv_latent");
    if (p->kv_latent && out->v) return fail(DSA_E_INVALID, "out->v must be NULL when kv_latent");
    if (!p->ik != !out->ik) return fail(DSA_E_INVALID, "out->ik must be given exactly when p->ik is");
    const bool with_scale = p->ik && p->idx_dtype == DSA_FP8_E4M3;
    if (with_scale != (out->ik_scale != nullptr))
        return fail(DSA_E_INVALID, "out->ik_scale must be given exactly when FP8 indexer keys are copied");
    const size_t need = dsa::compress_workspace_bytes(p->batch, p->n_k);
    if (!workspace || workspace_bytes < need)
        return fail(DSA_E_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    const int n_keep = dsa_compress_kept(p->n_k, window, keep_old);
    if (n_keep == 0) return DSA_OK;

    dsa::CompressArgs a{};
    a.B = p->batch;
    a.n_k = p->n_k;
    a.window = window < p->n_k ? window : p->n_k;
    a.keep = n_keep - a.window;
    a.n_keep = n_keep;
    a.nch = dsa::compress_chunks(p->n_k);
    a.imp = importance;
    // rows move 16 bytes at a time where the row size and both pointers allow
    // it, else 4; anything else is refused before a launch
    auto add = [&](const char* name, const void* src, void* dst, int bytes) -> bool {
        const uintptr_t al = reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst);
        const int unit = (bytes % 16 == 0 && al % 16 == 0) ? 16 : ((bytes % 4 == 0 && al % 4 == 0) ? 4 : 0);
        if (!unit) {
            fail(DSA_E_UNSUPPORTED, "%s rows of %d bytes (or their pointers) are not 4-byte aligned", name, bytes);
            return false;
        }
        a.src[a.nrow] = static_cast<const uint8_t*>(src);
        a.dst[a.nrow] = static_cast<uint8_t*>(dst);
        a.bytes[a.nrow] = bytes;
        a.unit[a.nrow] = unit;
        ++a.nrow;
        return true;
    };
    if (!add("k", p->k, out->k, cache_row_bytes(p, p->d_qk))) return DSA_E_UNSUPPORTED;
    if (!p->kv_latent && !add("v", p->v, out->v, cache_row_bytes(p, p->d_v))) return DSA_E_UNSUPPORTED;
    if (p->ik && !add("ik", p->ik, out->ik, 128 * (p->idx_dtype == DSA_F32 ? 4 : (p->idx_dtype == DSA_BF16 ? 2 : 1))))
        return DSA_E_UNSUPPORTED;
    if (with_scale && !add("ik_scale", p->ik_scale, out->ik_scale, 4)) return DSA_E_UNSUPPORTED;
    a.pos_out = out->pos;
    a.ws = static_cast<uint32_t*>(workspace);
    return device_status(dsa::launch_compress(a, stream), "compress launch");
}

}  // extern "C"
