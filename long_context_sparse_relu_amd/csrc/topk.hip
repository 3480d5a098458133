// topk.hip -- per-row top-k selector over fp32 score rows.
//
// The selector keeps the k highest-scoring keys of each query
// ("DeepSeek-V3.2-Exp 稀疏注意力机制(DSA)技术深度解析", sheratonhq.com,
// section 1; the fine-grained selector stage of "DeepSeek-V4 百万 token 上下文的
// 工程实现", blog.hotdry.top, section "从 O(N²) 到 O(N・k)").  Ties go to the
// lower position.
//
// Method: radix select on order-preserving uint32 keys, never a full sort.
// Digit 0 is key bits 31..21, digit 1 is key bits 20..10.
//   hist      the top-11-bit histogram of each row (or the indexer built it
//             while writing the scores);
//   threshold one workgroup per row finds the digit-0 bin d0 that holds the
//             k-th key and the count gt0 above it;
//   filter    every workgroup streams its slice of the row once: keys above
//             d0 go straight to the output row, keys in d0 are appended to
//             the row's candidate list and counted in a digit-1 histogram;
//   finish    one workgroup per row finds the digit-1 bin d1, keeps the
//             candidates above it, radix-selects the rest inside d1 on the
//             composite (low 21 key bits, ~position) -- so equal scores
//             resolve to the lower position -- and writes the kept positions
//             in ascending order (through an LDS bitmap of the row, or a
//             bitonic sort for rows too long for one).
// The score row is read twice (hist, filter) or once when the indexer built
// the histogram.  A row whose digit-0 bin overflows its candidate list (a
// mass of equal scores) is selected again in the finish from its whole score
// row.
#include "topk_common.h"

namespace dsa {

constexpr int kChunk = 2048;       // scores per workgroup in hist
constexpr int kFilterThreads = 256;
constexpr int kPerThread = kChunk / kFilterThreads;
constexpr int kFChunk = 8192;      // scores per workgroup in filter
constexpr int kFThreads = 512;
constexpr int kFPer = kFChunk / kFThreads;
constexpr int kFinishThreads = 512;

// Row metadata words in TopkArgs::count (kTopkMeta per row).
enum { M_SEL = 0, M_CAND = 1, M_D0 = 2, M_GT0 = 3 };

__global__ void k_zero_u32(uint32_t* p, size_t n) {
    size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (; i < n; i += stride) p[i] = 0u;
}

hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(k_zero_u32, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

// A row with top_k >= pos(t) + 1 keeps all its visible keys: positions
// 0..pos(t) in ascending order, then -1.  One workgroup per row.
__global__ void k_fill_prefix_idx(int32_t* idx, int row0, int n_q, int n_k, int k) {
    const int r = blockIdx.x;
    const int pos = row_pos(nullptr, row0 + r, n_q, n_k);
    int32_t* out = idx + static_cast<size_t>(r) * k;
    for (int j = threadIdx.x; j < k; j += blockDim.x) out[j] = j <= pos ? j : -1;
}

hipError_t launch_fill_prefix_idx(int32_t* idx, int row0, int rows, int n_q, int n_k, int k, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_prefix_idx, dim3(rows), dim3(256), 0, st, idx, row0, n_q, n_k, k);
    return hipGetLastError();
}

// The union of a backbone selection: row r of idx (width k + sinks + window)
// = the forced first keys 0..min(sinks, vis)-1, the picks that lie between
// the forced sets (ascending in picks; a row with fewer than k such keys also
// picked some forced ones, which are dropped), then the window keys
// max(sinks, vis - window)..vis-1, then -1.  All three parts are ascending
// and in that order, so the row is ascending.  One workgroup per row.
__global__ __launch_bounds__(256) void k_union_backbone(const int32_t* picks, int32_t* idx, int row0, int n_q,
                                                        int n_k, const int32_t* q_pos, int k, int sinks,
                                                        int window) {
    __shared__ int cnt[2][4];
    const int r = blockIdx.x;
    const int vis = row_pos(q_pos, row0 + r, n_q, n_k) + 1;
    const int v = vis > 0 ? vis : 0;
    const int ns = min(sinks, v);
    const int wlo = max(sinks, v - window);
    const int nw = max(0, v - wlo);
    const int32_t* pr = picks + static_cast<size_t>(r) * k;
    // picks below `sinks` come first and picks at or past v - window last
    int below = 0, inside = 0;
    for (int j = threadIdx.x; j < k; j += blockDim.x) {
        const int p = pr[j];
        below += p >= 0 && p < sinks;
        inside += p >= sinks && p < v - window;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        below += __shfl_xor(below, o);
        inside += __shfl_xor(inside, o);
    }
    if ((threadIdx.x & 63) == 0) { cnt[0][threadIdx.x >> 6] = below; cnt[1][threadIdx.x >> 6] = inside; }
    __syncthreads();
    const int a0 = cnt[0][0] + cnt[0][1] + cnt[0][2] + cnt[0][3];
    const int np = cnt[1][0] + cnt[1][1] + cnt[1][2] + cnt[1][3];
    const int width = k + sinks + window;
    int32_t* out = idx + static_cast<size_t>(r) * width;
    for (int j = threadIdx.x; j < width; j += blockDim.x) {
        int val = -1;
        if (j < ns) val = j;
        else if (j < ns + np) val = pr[a0 + (j - ns)];
        else if (j < ns + np + nw) val = wlo + (j - ns - np);
        out[j] = val;
    }
}

hipError_t launch_union_backbone(const int32_t* picks, int32_t* idx, int row0, int rows, int n_q, int n_k,
                                 const int32_t* q_pos, int k, int sinks, int window, hipStream_t st) {
    if (rows <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_union_backbone, dim3(rows), dim3(256), 0, st, picks, idx, row0, n_q, n_k, q_pos, k,
                       sinks, window);
    return hipGetLastError();
}

__device__ __forceinline__ int row_visible(const TopkArgs& a, int row) {
    return row_pos(a.q_pos, row, a.n_q, a.n_k) + 1;   // 0..n_k
}

// A score as the selection ranks it: with a backbone, the forced keys of the
// row (its first `sinks` and last `window` visible keys) rank as -inf, so the
// k picks come from the keys between them whenever there are k of those; the
// union step adds the forced keys and drops any forced key picked to fill k.
// The load is unconditional (no branch around it).
__device__ __forceinline__ float ranked(const TopkArgs& a, const float* sc, int s, int vis) {
    const float x = sc[s];
    return (s < a.sinks || s >= vis - a.window) ? -__builtin_inff() : x;
}

__device__ __forceinline__ uint64_t composite(uint32_t key, int s) {
    return (static_cast<uint64_t>(key & 0x1FFFFFu) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(s));
}

// Digit-0 histogram of every visible key.  Each thread issues all of its
// loads before it touches any of them.
__global__ __launch_bounds__(kFilterThreads) void k_topk_hist(TopkArgs a) {
    __shared__ uint32_t lh[kTopkBins];
    const int lrow = blockIdx.y, row = a.row0 + lrow;
    const int vis = row_visible(a, row);
    if (vis <= a.k) return;
    const int c0 = blockIdx.x * kChunk;
    if (c0 >= vis) return;
    const int c1 = min(c0 + kChunk, vis);
    const float* sc = a.scores + static_cast<size_t>(lrow) * a.n_k;
    float x[kPerThread];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
        int s = c0 + u * kFilterThreads + threadIdx.x;
        x[u] = s < c1 ? ranked(a, sc, s, vis) : 0.0f;
    }
    for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x) lh[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
        int s = c0 + u * kFilterThreads + threadIdx.x;
        if (s < c1) atomicAdd(&lh[order_key(x[u]) >> 21], 1u);
    }
    __syncthreads();
    uint32_t* gh = a.hist + static_cast<size_t>(lrow) * kTopkBins;
    for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x)
        if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// One workgroup per row: locate the digit-0 threshold bin once.
__global__ __launch_bounds__(kFilterThreads) void k_topk_threshold(TopkArgs a) {
    __shared__ uint32_t lh[kTopkBins];
    __shared__ uint32_t wsum[kFilterThreads / 64 + 2];
    const int lrow = blockIdx.x, row = a.row0 + lrow;
    if (row_visible(a, row) <= a.k) return;
    copy_to_lds(lh, a.hist + static_cast<size_t>(lrow) * kTopkBins, kTopkBins);
    __syncthreads();
    int d0; uint32_t gt0;
    find_threshold_bin(lh, kTopkBins, static_cast<uint32_t>(a.k), wsum, &d0, &gt0);
    if (threadIdx.x == 0) {
        uint32_t* meta = a.count + static_cast<size_t>(lrow) * kTopkMeta;
        meta[M_D0] = static_cast<uint32_t>(d0);
        meta[M_GT0] = gt0;
    }
}

// Keys above d0 go to the output row, keys in d0 become candidates and are
// counted in the digit-1 histogram.  Each thread classifies kFPer scores held
// in registers; a block scan of the packed (kept, candidate) counts gives
// every thread its output offsets, so nothing is staged in LDS.
__global__ __launch_bounds__(kFThreads) void k_topk_filter(TopkArgs a) {
    __shared__ uint32_t lh1[kTopkBins];
    __shared__ uint32_t wsum[kFThreads / 64];
    __shared__ uint32_t g_base[2];
    const int lrow = blockIdx.y, row = a.row0 + lrow;
    const int vis = row_visible(a, row);
    if (vis <= a.k) return;
    const int c0 = blockIdx.x * kFChunk;
    if (c0 >= vis) return;
    const int c1 = min(c0 + kFChunk, vis);
    const float* sc = a.scores + static_cast<size_t>(lrow) * a.n_k;
    float x[kFPer];
#pragma unroll
    for (int u = 0; u < kFPer; ++u) {
        int s = c0 + u * kFThreads + threadIdx.x;
        x[u] = s < c1 ? ranked(a, sc, s, vis) : 0.0f;
    }
    uint32_t* meta = a.count + static_cast<size_t>(lrow) * kTopkMeta;
    const int d0 = static_cast<int>(meta[M_D0]);
    for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x) lh1[i] = 0u;
    uint32_t key[kFPer];
    uint32_t nsel = 0, ncand = 0;
#pragma unroll
    for (int u = 0; u < kFPer; ++u) {
        int s = c0 + u * kFThreads + threadIdx.x;
        key[u] = order_key(x[u]);
        int dg = s < c1 ? static_cast<int>(key[u] >> 21) : -1;
        nsel += dg > d0;
        ncand += dg == d0;
    }
    uint32_t total;
    const uint32_t off = block_exclusive_scan((nsel << 16) | ncand, wsum, &total);
    if (threadIdx.x == 0) {
        uint32_t ts = total >> 16, tc = total & 0xFFFFu;
        g_base[0] = ts ? atomicAdd(&meta[M_SEL], ts) : 0u;
        g_base[1] = tc ? atomicAdd(&meta[M_CAND], tc) : 0u;
    }
    __syncthreads();
    uint32_t os = g_base[0] + (off >> 16);
    uint32_t oc = g_base[1] + (off & 0xFFFFu);
    int32_t* out = a.idx + static_cast<size_t>(lrow) * a.k;
    uint64_t* cd = a.cand + static_cast<size_t>(lrow) * a.cand_cap;
#pragma unroll
    for (int u = 0; u < kFPer; ++u) {
        int s = c0 + u * kFThreads + threadIdx.x;
        int dg = s < c1 ? static_cast<int>(key[u] >> 21) : -1;
        if (dg > d0) {
            if (os < static_cast<uint32_t>(a.k)) out[os] = s;
            ++os;
        } else if (dg == d0) {
            if (oc < static_cast<uint32_t>(a.cand_cap)) cd[oc] = composite(key[u], s);
            ++oc;
            atomicAdd(&lh1[(key[u] >> 10) & 0x7FFu], 1u);
        }
    }
    __syncthreads();
    if ((total & 0xFFFFu) != 0) {
        uint32_t* gh1 = a.hist1 + static_cast<size_t>(lrow) * kTopkBins;
        for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x)
            if (lh1[i]) atomicAdd(&gh1[i], lh1[i]);
    }
}

// The finishing select's candidates: a list in LDS or global memory.
struct CandList {
    const uint64_t* c; int n;
    __device__ int size() const { return n; }
    __device__ bool get(int i, uint64_t* out) const { *out = c[i]; return true; }
};
// Candidates whose top composite digit (key bits 20..10) is d1 share the
// first 22 key bits; radix-select the k_rem largest of them on the remaining
// digits and keep them.
template <class Src>
__device__ void select_in_bin(const Src& src, int d1, uint32_t k_rem, uint32_t* lh, uint32_t* wsum,
                              const Sink& sink)
{
    const int shifts[4] = {31, 20, 9, 0};
    const int widths[4] = {11, 11, 11, 9};
    radix_select(src, k_rem, shifts, widths, 4, static_cast<uint64_t>(d1), lh, wsum, sink);
}

// One workgroup per row: candidates above d1 are kept, the d1 bin is
// resolved exactly, then the row's k positions are written in ascending
// order.
__global__ __launch_bounds__(kFinishThreads) void k_topk_finish(TopkArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint64_t* grp = reinterpret_cast<uint64_t*>(smem);                      // [cand_cap]
    uint32_t* tail = reinterpret_cast<uint32_t*>(grp + a.cand_cap);          // bitmap or list
    __shared__ uint32_t lh[kTopkBins];
    __shared__ uint32_t wsum[kFinishThreads / 64 + 2];
    __shared__ uint32_t n_list, n_grp;
    const int lrow = blockIdx.x, row = a.row0 + lrow;
    const int vis = row_visible(a, row);
    int32_t* out = a.idx + static_cast<size_t>(lrow) * a.k;
    if (vis <= a.k) {                            // every visible key is kept
        for (int j = threadIdx.x; j < a.k; j += blockDim.x) out[j] = j < vis ? j : -1;
        return;
    }
    const bool use_bitmap = a.n_k <= kBitmapMaxKeys;
    const int nwords = (vis + 31) >> 5;
    int kpad = 1;
    while (kpad < a.k) kpad <<= 1;
    Sink sink{use_bitmap ? tail : nullptr, reinterpret_cast<int32_t*>(tail), &n_list,
              static_cast<uint32_t>(a.k)};
    if (use_bitmap) {
        for (int i = threadIdx.x; i < nwords; i += blockDim.x) tail[i] = 0u;
    } else {
        for (int i = threadIdx.x; i < kpad; i += blockDim.x) tail[i] = 0x7FFFFFFFu;
    }
    const uint32_t* meta = a.count + static_cast<size_t>(lrow) * kTopkMeta;
    const uint32_t gt0 = meta[M_GT0];
    const uint32_t n_cand = meta[M_CAND];
    copy_to_lds(lh, a.hist1 + static_cast<size_t>(lrow) * kTopkBins, kTopkBins);
    if (threadIdx.x == 0) { n_list = 0; n_grp = 0; }
    __syncthreads();
    for (int j = threadIdx.x; j < static_cast<int>(gt0); j += blockDim.x) sink.put(out[j]);
    const uint32_t k1 = static_cast<uint32_t>(a.k) - gt0;
    int d1; uint32_t gt1;
    find_threshold_bin(lh, kTopkBins, k1, wsum, &d1, &gt1);
    const uint32_t k2 = k1 - gt1;
    const bool whole_bin = lh[d1] == k2;
    __syncthreads();

    if (n_cand <= static_cast<uint32_t>(a.cand_cap)) {
        // keep what is above d1, gather the d1 bin into LDS
        CandList gl{a.cand + static_cast<size_t>(lrow) * a.cand_cap, static_cast<int>(n_cand)};
        for_each_candidate(gl, [&](uint64_t c) {
            int dg = static_cast<int>(c >> 42);
            if (dg > d1 || (dg == d1 && whole_bin)) sink.put_c(c);
            else if (dg == d1) grp[atomicAdd(&n_grp, 1u)] = c;
        });
        __syncthreads();
        if (!whole_bin) {
            CandList src{grp, static_cast<int>(n_grp)};
            select_in_bin(src, d1, k2, lh, wsum, sink);
        }
    } else {
        // the list overflowed (a mass of equal or nearly equal scores): select
        // the row again from all of its scores, on the composite bits that
        // vary among them, starting from an empty sink
        if (use_bitmap) {
            for (int i = threadIdx.x; i < nwords; i += blockDim.x) tail[i] = 0u;
        } else {
            for (int i = threadIdx.x; i < kpad; i += blockDim.x) tail[i] = 0x7FFFFFFFu;
        }
        if (threadIdx.x == 0) n_list = 0;
        ScoreRow64 row_src{a.scores + static_cast<size_t>(lrow) * a.n_k, vis, a.sinks, vis - a.window};
        radix_select_spread(row_src, static_cast<uint32_t>(a.k), lh, wsum, sink);
    }
    __syncthreads();
    write_ordered(sink, nwords, kpad, a.k, out, wsum);
}

// Dynamic LDS of the finish kernel: the candidate group plus the bitmap or list.
static size_t finish_lds_bytes(const TopkArgs& a) {
    int kpad = 1;
    while (kpad < a.k) kpad <<= 1;
    size_t tail = a.n_k <= kBitmapMaxKeys ? static_cast<size_t>((a.n_k + 31) >> 5) * 4
                                          : static_cast<size_t>(kpad) * 4;
    return static_cast<size_t>(a.cand_cap) * sizeof(uint64_t) + tail;
}

int topk_cand_cap(int n_k) {
    return n_k < kTopkCandCapMax ? n_k : kTopkCandCapMax;
}

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// ---------------------------------------------------------------------------
// Rows short enough for LDS (every prefill row up to 32K keys): one workgroup
// per row reads the row's visible scores once, as order keys, into LDS and
// radix-selects there on the composite ((key - row minimum) << 32 | ~position),
// whose first digit covers the top 11 bits of the row's key range, so the
// histogram passes spread over the bins and never re-read memory; the kept
// positions come out in ascending order through an LDS bitmap.
// ---------------------------------------------------------------------------
constexpr int kRowLdsMax = 32768;       // scores a row may hold in LDS (128 KiB)
constexpr int kRowThreads = 1024;


struct LdsRel {
    const uint32_t* key; int n; uint32_t base;
    __device__ int size() const { return n; }
    __device__ bool get(int i, uint64_t* out) const {
        *out = (static_cast<uint64_t>(key[i] - base) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(i));
        return true;
    }
};

// Radix select over a row's order keys in LDS and the ordered write of the
// kept positions (the whole block; vis > k; kmin, kmax: the keys' range).
__device__ __forceinline__ void select_lds_row(const TopkArgs& a, uint32_t* keys, int vis, uint32_t kmin, uint32_t kmax,
                               uint32_t* lh, uint32_t* bm, uint32_t* wsum, uint32_t* n_list, int32_t* out) {
    const int k = a.k;
    const uint32_t range = kmax - kmin;
    const int bits = range ? 32 - __clz(static_cast<int>(range)) : 0;
    const int sh = bits > 11 ? bits - 11 : 0;
    int shifts[6], widths[6], np = 1;
    shifts[0] = 32 + sh;
    widths[0] = 11;
    for (int below = 32 + sh; below > 0 && np < 6; ++np) {
        const int w = below < 11 ? below : 11;
        below -= w;
        shifts[np] = below;
        widths[np] = w;
    }
    const int nwords = (vis + 31) >> 5;
    Sink sink{bm, nullptr, n_list, static_cast<uint32_t>(k)};
    LdsRel src{keys, vis, kmin};
    radix_select(src, static_cast<uint32_t>(k), shifts, widths, np, 0ull, lh, wsum, sink);
    write_ordered(sink, nwords, 1, k, out, wsum);
}

// Keys of one bin that the comparison ranking below takes (they sit in the
// histogram's LDS once the bin is known: kTopkBins words = this many 64-bit
// entries).
constexpr int kLinListCap = kTopkBins / 2;

// Exact top k of a row whose scores (float bits; a backbone's forced keys
// already -inf) sit in LDS at sbits[0, vis), vis > k: the k largest by
// (score descending, position ascending), written in ascending order.
//   histogram  a digit linear in the score over the row's finite range
//              [smin, smax] (2048 bins; -inf and smin fall in bin 0): the
//              digit never decreases as the score grows, so the threshold bin
//              d0 and the count above it give the exact split;
//   split      keys of bins above d0 are kept (bitmap), keys of bin d0 go to
//              a list as (order key << 32 | ~position);
//   rank       each listed key counts the listed keys that beat it; the
//              k - (count above d0) best are kept.
// On rows whose scores are nearly equal (finite range 0, or more than
// kLinListCap keys in bin d0) the scores are turned into order keys in place
// and radix-selected instead.  Whole block; smin, smax block-uniform.
__device__ void select_lds_row_lin(const TopkArgs& a, uint32_t* sbits, int vis, float smin, float smax,
                                   uint32_t* lh, uint32_t* bm, uint32_t* wsum, uint32_t* n_list, int32_t* out) {
    const int k = a.k;
    const int T = blockDim.x;
    const int nwords = (vis + 31) >> 5;
    float scale = smax > smin && smin > -__builtin_inff() && smax < __builtin_inff()
                      ? static_cast<float>(kTopkBins) / (smax - smin) : 0.0f;
    const bool spread = scale > 0.0f && scale < __builtin_inff();
    auto digit = [&](float x) {
        return x <= smin ? 0 : min(kTopkBins - 1, static_cast<int>((x - smin) * scale));
    };
    int d0 = 0;
    uint32_t gt0 = 0, n0 = 0;
    if (spread) {
        for (int i = threadIdx.x; i < kTopkBins; i += T) lh[i] = 0u;
        __syncthreads();
        for (int i0 = threadIdx.x; i0 < vis; i0 += 8 * T) {      // eight reads in flight
            uint32_t x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = sbits[min(i0 + u * T, vis - 1)];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (i0 + u * T < vis) atomicAdd(&lh[digit(__uint_as_float(x[u]))], 1u);
        }
        __syncthreads();
        find_threshold_bin(lh, kTopkBins, static_cast<uint32_t>(k), wsum, &d0, &gt0);
        n0 = lh[d0];
        __syncthreads();                          // every thread has read lh[d0] (the list reuses lh)
    }
    if (!spread || n0 > static_cast<uint32_t>(kLinListCap)) {
        // nearly equal scores: radix select over order keys
        uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
        for (int i = threadIdx.x; i < vis; i += T) {
            const uint32_t kk = order_key(__uint_as_float(sbits[i]));
            sbits[i] = kk;
            kmin = min(kmin, kk);
            kmax = max(kmax, kk);
        }
        kmin = wave_allreduce(kmin, [](uint32_t p, uint32_t q) { return p < q ? p : q; });
        kmax = wave_allreduce(kmax, [](uint32_t p, uint32_t q) { return p > q ? p : q; });
        uint32_t* wred = lh;                      // free until the select clears it
        if ((threadIdx.x & 63) == 0) { wred[2 * (threadIdx.x >> 6)] = kmin; wred[2 * (threadIdx.x >> 6) + 1] = kmax; }
        __syncthreads();
        for (int w = 0; w < T / 64; ++w) { kmin = min(kmin, wred[2 * w]); kmax = max(kmax, wred[2 * w + 1]); }
        __syncthreads();
        select_lds_row(a, sbits, vis, kmin, kmax, lh, bm, wsum, n_list, out);
        return;
    }
    // split: bins above d0 kept, bin d0 listed
    uint64_t* list = reinterpret_cast<uint64_t*>(lh);
    const int lane = threadIdx.x & 63;
    for (int j0 = 0; j0 < vis; j0 += 4 * T) {    // uniform trip count (ballots below); four reads in flight
        uint32_t xs[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) xs[u] = sbits[min(j0 + u * T + static_cast<int>(threadIdx.x), vis - 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i0 = j0 + u * T;
            const int i = i0 + static_cast<int>(threadIdx.x);
            const float x = i < vis ? __uint_as_float(xs[u]) : -__builtin_inff();
            const int d = i < vis ? digit(x) : -1;
            // a wave covers 64 consecutive positions from a multiple of 64: two
            // whole bitmap words, which only this wave writes in this pass
            const uint64_t above = __ballot(d > d0);
            if ((lane & 31) == 0) {
                const uint32_t bits = static_cast<uint32_t>(lane == 0 ? above : above >> 32);
                if (bits) bm[i >> 5] = bits;
            }
            const bool take = d == d0;
            const uint64_t m = __ballot(take);
            if (m) {
                const int leader = __ffsll(static_cast<unsigned long long>(m)) - 1;
                uint32_t base = 0;
                if (lane == leader) base = atomicAdd(n_list, static_cast<uint32_t>(__popcll(m)));
                base = __shfl(base, leader);
                if (take) list[base + __popcll(m & ((1ull << lane) - 1ull))] = composite64(order_key(x), i);
            }
        }
    }
    __syncthreads();
    // rank: the k - gt0 best of the n0 listed keys (composites are distinct)
    const uint32_t k_rem = static_cast<uint32_t>(k) - gt0;
    for (uint32_t t = threadIdx.x; t < n0; t += T) {
        const uint64_t c = list[t];
        uint32_t beat = 0;
        uint32_t j = 0;
        for (; j + 8 <= n0; j += 8) {            // eight reads in flight
            uint64_t y[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) y[u] = list[j + u];
#pragma unroll
            for (int u = 0; u < 8; ++u) beat += y[u] > c ? 1u : 0u;
        }
        for (; j < n0; ++j) beat += list[j] > c ? 1u : 0u;
        if (beat < k_rem) {
            const int pos = static_cast<int>(~static_cast<uint32_t>(c & 0xFFFFFFFFull));
            atomicOr(&bm[pos >> 5], 1u << (pos & 31));
        }
    }
    __syncthreads();
    Sink sink{bm, nullptr, n_list, static_cast<uint32_t>(k)};
    write_ordered(sink, nwords, 1, k, out, wsum);
}

template <int T>
__global__ __launch_bounds__(T) void k_topk_row_lds(TopkArgs a) {
    extern __shared__ uint32_t keys[];                        // [min(n_k, kRowLdsMax)]
    __shared__ __align__(16) uint32_t lh[kTopkBins];          // (8-byte list entries in the select)
    __shared__ uint32_t bm[kRowLdsMax / 32];
    __shared__ uint32_t wsum[T / 64 + 2];
    __shared__ uint32_t n_list;
    const int lrow = blockIdx.x, row = a.row0 + lrow;
    const int vis = row_visible(a, row);
    const int k = a.k;
    int32_t* out = a.idx + static_cast<size_t>(lrow) * k;
    if (vis <= k) {
        for (int j = threadIdx.x; j < k; j += blockDim.x) out[j] = j < vis ? j : -1;
        return;
    }
    const float* sc = a.scores + static_cast<size_t>(lrow) * a.n_k;
    // the row's scores, eight loads in flight per thread (indices past vis
    // re-read the last score and are not stored), and their finite range
    float smin = __builtin_inff(), smax = -__builtin_inff();
    for (int i0 = threadIdx.x; i0 < vis; i0 += 8 * T) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = ranked(a, sc, min(i0 + u * T, vis - 1), vis);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * T;
            if (i < vis) {
                keys[i] = __float_as_uint(v[u]);
                if (v[u] > -__builtin_inff()) smin = fminf(smin, v[u]);
                smax = fmaxf(smax, v[u]);
            }
        }
    }
    const int nwords = (vis + 31) >> 5;
    for (int i = threadIdx.x; i < nwords; i += T) bm[i] = 0u;
    if (threadIdx.x == 0) n_list = 0;
    smin = wave_allmin(smin);
    smax = wave_allmax(smax);
    __shared__ float wmin[T / 64], wmax[T / 64];
    if ((threadIdx.x & 63) == 0) { wmin[threadIdx.x >> 6] = smin; wmax[threadIdx.x >> 6] = smax; }
    __syncthreads();
    for (int w = 0; w < T / 64; ++w) { smin = fminf(smin, wmin[w]); smax = fmaxf(smax, wmax[w]); }
    select_lds_row_lin(a, keys, vis, smin, smax, lh, bm, wsum, &n_list, out);
}

// Rows longer than half the LDS limit leave room for one workgroup per
// compute unit, so nothing hides a row's load behind another row's select.
// This persistent form does it inside the workgroup: workgroup w takes rows
// w, w + gridDim.x, ...; while it selects one row, the next row's scores
// (kRowPerThread per thread) are already in flight into registers.
constexpr int kRowPerThread = kRowLdsMax / kRowThreads;
__global__ __launch_bounds__(kRowThreads) void k_topk_row_lds_next(TopkArgs a) {
    extern __shared__ uint32_t keys[];                        // [kRowLdsMax]
    __shared__ __align__(16) uint32_t lh[kTopkBins];          // (8-byte list entries in the select)
    __shared__ uint32_t bm[kRowLdsMax / 32];
    __shared__ uint32_t wsum[kRowThreads / 64 + 2];
    __shared__ float wmin[kRowThreads / 64], wmax[kRowThreads / 64];
    __shared__ uint32_t n_list;
    float v[kRowPerThread];
    // issue the loads of row lrow's scores: entry u of thread t is key
    // t + u * kRowThreads; entries past vis re-read the last score and are not
    // stored.  The loads are unconditional and nothing reads them until the
    // next row's keys are stored, so no wait separates them.
    auto fetch = [&](int lrow, int vis) {
        const float* sc = a.scores + static_cast<size_t>(lrow) * a.n_k;
#pragma unroll
        for (int u = 0; u < kRowPerThread; ++u) v[u] = sc[min(static_cast<int>(threadIdx.x) + u * kRowThreads, vis - 1)];
    };
    int lrow = blockIdx.x;
    int vis = lrow < a.rows ? row_visible(a, a.row0 + lrow) : 0;
    if (lrow < a.rows && vis > a.k) fetch(lrow, vis);
    for (; lrow < a.rows; lrow += gridDim.x) {
        const int next = lrow + gridDim.x;
        const int vis_next = next < a.rows ? row_visible(a, a.row0 + next) : 0;
        int32_t* out = a.idx + static_cast<size_t>(lrow) * a.k;
        if (vis <= a.k) {
            for (int j = threadIdx.x; j < a.k; j += blockDim.x) out[j] = j < vis ? j : -1;
            if (next < a.rows && vis_next > a.k) fetch(next, vis_next);
        } else {
            float smin = __builtin_inff(), smax = -__builtin_inff();
#pragma unroll
            for (int u = 0; u < kRowPerThread; ++u) {
                const int i = static_cast<int>(threadIdx.x) + u * kRowThreads;
                if (i < vis) {
                    // a backbone's forced keys rank as -inf (as ranked() does)
                    const float x = (i < a.sinks || i >= vis - a.window) ? -__builtin_inff() : v[u];
                    keys[i] = __float_as_uint(x);
                    if (x > -__builtin_inff()) smin = fminf(smin, x);
                    smax = fmaxf(smax, x);
                }
            }
            const int nwords = (vis + 31) >> 5;
            for (int i = threadIdx.x; i < nwords; i += kRowThreads) bm[i] = 0u;
            if (threadIdx.x == 0) n_list = 0;
            smin = wave_allmin(smin);
            smax = wave_allmax(smax);
            if ((threadIdx.x & 63) == 0) { wmin[threadIdx.x >> 6] = smin; wmax[threadIdx.x >> 6] = smax; }
            __syncthreads();
            for (int w = 0; w < kRowThreads / 64; ++w) { smin = fminf(smin, wmin[w]); smax = fmaxf(smax, wmax[w]); }
            if (next < a.rows && vis_next > a.k) fetch(next, vis_next);   // lands during the select
            select_lds_row_lin(a, keys, vis, smin, smax, lh, bm, wsum, &n_list, out);
        }
        __syncthreads();                    // the next row's keys reuse the LDS
        vis = vis_next;
    }
}

// ---------------------------------------------------------------------------
// Rows of more than half the LDS limit (persistent, one workgroup per CU).
// A row's scores arrive in LDS straight from memory (global_load_lds), and the
// next row's are loaded while the current one finishes.  Per row:
//   sample    every eighth key (key t + (8m + (t mod 8)) * 1024 for thread t,
//             m < 4), up to 4096 scores; their finite range and a 2048-bin
//             histogram of g(x) = (x - min) * 2048 / range;
//   bracket   the bins d_hi >= d_lo holding the sample's r_hi-th and r_lo-th
//             largest score, r = k * samples / visible keys -/+ 4 standard
//             deviations (binomial) and 2;
//   classify  every key by the same map g: g >= d_hi + 1 -> above (bitmap
//             bit, one ballot per 64 keys), d_lo <= g < d_hi + 1 -> listed as
//             (score, position) in its wave's LDS region, below -> dropped;
//             the next row's chunks are loaded during it;
//   select    if fewer than k keys are above and at least k are above or
//             listed (which proves the bracket holds the k-th key), the k -
//             above best listed keys: a 256-bin histogram of a second map
//             linear over the bracket, and its threshold bin ranked exactly by
//             (order key << 32 | ~position).
// g and the second map never decrease as the score grows, so "above" keys beat
// every listed key and listed keys beat every dropped one: the result is the
// exact top k whatever the sample.  When the counts do not prove the bracket
// (or a wave's region overflows) the row, still in LDS, is selected in full
// there (select_lds_row_lin); a threshold bin too large to rank by comparison
// is radix-selected from the list.
// ---------------------------------------------------------------------------
#ifndef DSA_TOPK_ROW_REG
#define DSA_TOPK_ROW_REG 1
#endif
// launches whose longest row exceeds this many keys take k_topk_row_reg
#ifndef DSA_TOPK_ROW_REG_MIN
#define DSA_TOPK_ROW_REG_MIN (kRowLdsMax / 2)
#endif
constexpr int kRegThreads = 1024;
constexpr int kRegPer = kRowLdsMax / kRegThreads;   // 32 keys per thread
constexpr int kRegRegion = 128;     // list entries per wave
constexpr int kRegBins2 = 256;      // second-level bins over the bracket
constexpr int kRegTieCap = (kTopkBins - kRegBins2) / 2;   // threshold-bin entries ranked (8-byte entries in lh past the bins)

// The second-level digit of a listed score: linear over the bracket [lo2,
// d_hi + 1) of the first map t = x * scale + off, clamped to the bins.
__device__ __forceinline__ int reg_digit2(uint32_t bits, float scale, float off, float lo2, float scale2) {
    const float t = fmaf(__uint_as_float(bits), scale, off);
    return max(0, min(kRegBins2 - 1, static_cast<int>((t - lo2) * scale2)));
}
// The listed keys (wave regions of (score bits, position) pairs, wc1[w] in
// region w) whose second-level digit is d2, as composites (order key << 32 |
// ~position).
struct RegTieSrc {
    const uint32_t* lpair; const uint32_t* wc1; int region; int total;
    float scale, off, lo2, scale2; int d2;
    __device__ int size() const { return total; }
    __device__ bool get(int i, uint64_t* out) const {
        int w = 0;
        while (i >= static_cast<int>(wc1[w])) { i -= static_cast<int>(wc1[w]); ++w; }
        const uint32_t bits = lpair[2 * (w * region + i)];
        const int pos = static_cast<int>(lpair[2 * (w * region + i) + 1]);
        if (reg_digit2(bits, scale, off, lo2, scale2) != d2) return false;
        *out = composite64(order_key(__uint_as_float(bits)), pos);
        return true;
    }
};

__global__ __launch_bounds__(kRegThreads) void k_topk_row_reg(TopkArgs a) {
    // (static: the compiler then knows that no other LDS array overlaps the
    // loads in flight into keys and waits for them only where keys is read)
    __shared__ __align__(16) uint32_t keys[kRowLdsMax];        // the row's scores
    __shared__ __align__(16) uint32_t lh[kTopkBins];
    __shared__ uint32_t bm[kRowLdsMax / 32];
    constexpr int T = kRegThreads, P = kRegPer, NW = kRegThreads / 64;
    __shared__ uint32_t lpair[NW * kRegRegion * 2];            // per wave: (score bits, position) pairs
    __shared__ int fres[4];
    __shared__ uint32_t wsum[NW + 2];
    __shared__ float wmin[NW], wmax[NW];
    __shared__ uint32_t wc0[NW], wc1[NW];
    __shared__ uint32_t n_list;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float kNaN = __uint_as_float(0x7FC00000u);
    // The thread index through an empty asm, taken afresh for each use:
    // per-key positions are then recomputed where they are needed (one add
    // each) instead of being kept alive or hoisted out of the row loop.
    auto fresh_tid = [&]() {
        int t = tid;
        asm volatile("" : "+v"(t));
        return t;
    };
    // Row lrow's scores into keys[] (completion is awaited at the row's
    // start): instruction u of wave w copies keys [u * T + 64 w, +64), lane l
    // one key, through a buffer resource over the row's visible scores (a
    // position past vis reads 0 and is never used; the thread's offset is
    // fixed and the chunk's is a scalar, so a chunk costs no address
    // arithmetic).  Each wave reads only these slices of keys[] (the sample
    // and the classify below), so chunk u of the next row can follow as soon
    // as the wave has classified chunk u of the current one.
    auto row_rsrc = [&](int lr, int vis) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.scores + static_cast<size_t>(lr) * a.n_k), 0,
                                                 vis * 4, kBufferWord3);
    };
    auto load_chunk = [&](__amdgpu_buffer_rsrc_t rs, int u, int t0, int wbase) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(keys + u * T + wbase), 4,
                                                 static_cast<uint32_t>(t0) * 4u, static_cast<uint32_t>(u * T) * 4u, 0, 0);
    };
    auto prefetch = [&](int lrow, int vis) {
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(lrow, vis);
        const int t0 = fresh_tid();
        const int wbase = __builtin_amdgcn_readfirstlane(t0 & ~63);
#pragma unroll
        for (int u = 0; u < P; ++u) load_chunk(rs, u, t0, wbase);
    };
    int lrow = blockIdx.x;
    int vis = lrow < a.rows ? row_visible(a, a.row0 + lrow) : 0;
    if (lrow < a.rows && vis > a.k) prefetch(lrow, vis);
    for (; lrow < a.rows; lrow += gridDim.x) {
        const int next = lrow + gridDim.x;
        const int vis_next = next < a.rows ? row_visible(a, a.row0 + next) : 0;
        const bool fetch_next = next < a.rows && vis_next > a.k;
        int32_t* out = a.idx + static_cast<size_t>(lrow) * a.k;
        const uint32_t k = static_cast<uint32_t>(a.k);
        if (vis <= a.k) {
            for (int j = tid; j < a.k; j += T) out[j] = j < vis ? j : -1;
            if (fetch_next) prefetch(next, vis_next);
            vis = vis_next;
            continue;
        }
        // this row's scores have landed in keys[] (every wave's part)
        __builtin_amdgcn_s_waitcnt(kWaitVmem);
        lds_barrier();
        // a key as ranked: absent (past vis) NaN, a backbone's forced keys -inf
        auto key_at = [&](int i) {
            const float y = __uint_as_float(keys[i]);
            return i >= vis ? kNaN : (i < a.sinks || i >= vis - a.window) ? -__builtin_inff() : y;
        };
        const int nwords = (vis + 31) >> 5;

        // sample: key t + (8m + (t & 7)) * T of thread t
        float smp[4];
        float smin = __builtin_inff(), smax = -__builtin_inff();
        uint32_t ns_w = 0;
        {
            const int tr = fresh_tid();
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int i = tr + (8 * m + (tr & 7)) * T;
                const bool pres = i < vis;
                const float sv = key_at(min(i, kRowLdsMax - 1));
                smp[m] = pres ? sv : kNaN;
                ns_w += static_cast<uint32_t>(__popcll(__ballot(pres)));
                if (pres && sv > -__builtin_inff()) smin = fminf(smin, sv);
                if (pres) smax = fmaxf(smax, sv);
            }
        }
        smin = wave_allmin(smin);
        smax = wave_allmax(smax);
        if (lane == 0) { wmin[wave] = smin; wmax[wave] = smax; wc0[wave] = ns_w; }
        for (int i = tid; i < kTopkBins; i += T) lh[i] = 0u;
        if (tid == 0) n_list = 0;
        lds_barrier();
        uint32_t ns = 0;
        for (int w = 0; w < NW; ++w) { smin = fminf(smin, wmin[w]); smax = fmaxf(smax, wmax[w]); ns += wc0[w]; }
        const float scale = static_cast<float>(kTopkBins) / (smax - smin);
        const float off = -smin * scale;
        // block-uniform: the sampled path holds (else the whole-row select)
        bool fast = smax > smin && scale > 0.0f && scale < __builtin_inff();
        int d_hi = kTopkBins - 1, d_lo = 0;
        uint32_t above_all = 0, listed = 0;
        const bool classified = fast;          // the classify (and the next row's loads) ran
        if (fast) {
#pragma unroll
            for (int m = 0; m < 4; ++m)
                if (smp[m] == smp[m]) {
                    const float t = fmaf(smp[m], scale, off);
                    atomicAdd(&lh[max(0, min(kTopkBins - 1, static_cast<int>(t)))], 1u);
                }
            lds_barrier();
            // bracket
            const float ks = static_cast<float>(k) * static_cast<float>(ns) / static_cast<float>(vis);
            const float sd = sqrtf(ks);
            const int r_hi = static_cast<int>(floorf(ks - 4.0f * sd - 2.0f));
            const int r_lo = static_cast<int>(ceilf(ks + 4.0f * sd + 2.0f));
            float th = __builtin_inff(), tl = -__builtin_inff();
            if (wave == 0)
                wave_find_bins<kTopkBins>(lh, static_cast<uint32_t>(max(r_hi, 1)),
                                          static_cast<uint32_t>(min(r_lo, static_cast<int>(ns))), fres);
            lds_barrier();
            if (r_hi >= 1) {
                d_hi = fres[0];
                th = static_cast<float>(d_hi + 1);
            }
            if (r_lo <= static_cast<int>(ns)) {
                d_lo = fres[2];
                if (d_lo > 0) tl = static_cast<float>(d_lo);
            }
            // the second level's bins, cleared here (the first level is done
            // with lh; the barrier after the classify orders this)
            for (int i = tid; i < kRegBins2; i += T) lh[i] = 0u;
            // classify: lane 2u (2u + 1) of bw gathers the low (high) bitmap
            // word of this wave's 64 keys of chunk u
            uint32_t n_above = 0, cnt = 0;
            int bw = 0;
            const int tc = fresh_tid();
            uint32_t* lreg = lpair + 2 * (tc >> 6) * kRegRegion;   // this wave's region
            const __amdgpu_buffer_rsrc_t nrs = row_rsrc(fetch_next ? next : lrow, fetch_next ? vis_next : vis);
            const int wbase = __builtin_amdgcn_readfirstlane(tc & ~63);
            // each chunk's score is read one chunk ahead, so its LDS latency
            // overlaps the classify of the chunk before (the slots it reads
            // are not the ones that chunk's next-row load replaces)
            uint32_t ynext = keys[tc];
#pragma unroll
            for (int u = 0; u < P; ++u) {
                const uint32_t y = ynext;
                if (u + 1 < P && (u + 1) * T < vis) ynext = keys[tc + (u + 1) * T];
                if (u * T < vis) {
                    // (chunks holding no absent or forced key skip those tests)
                    float xv = __uint_as_float(y);
                    if (!(u * T >= a.sinks && (u + 1) * T <= vis - a.window)) {
                        const int i = tc + u * T;
                        xv = i >= vis ? kNaN : (i < a.sinks || i >= vis - a.window) ? -__builtin_inff() : xv;
                    }
                    // (the ballots take the compares' lane masks directly)
                    const float t = fmaf(xv, scale, off);
                    const bool ab = t >= th;
                    const bool ge = t >= tl;
                    const uint64_t above = __builtin_amdgcn_ballot_w64(ab);
                    asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(bw) : "s"(static_cast<uint32_t>(above)), "n"(2 * u));
                    asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(bw) : "s"(static_cast<uint32_t>(above >> 32)), "n"(2 * u + 1));
                    const uint64_t take = __builtin_amdgcn_ballot_w64(ge) & ~above;
                    if (take) {
                        if (ge && !ab) {
                            // (past the region's end every entry lands on its last slot;
                            // the count then exceeds the region and the row takes the
                            // fallback, so those entries are never read)
                            const uint32_t slot = min(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(take >> 32),
                                                          __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(take), cnt)),
                                                      static_cast<uint32_t>(kRegRegion - 1));
                            lreg[2 * slot] = __float_as_uint(xv);
                            lreg[2 * slot + 1] = static_cast<uint32_t>(tc + u * T);
                        }
                        cnt += static_cast<uint32_t>(__popcll(take));
                    }
                }
                // this wave is done with its slice of chunk u (the scores above
                // were used, so their reads have completed): the next row's
                // chunk u follows
                if (fetch_next) {
                    __builtin_amdgcn_sched_barrier(0);
                    load_chunk(nrs, u, tc, wbase);
                }
            }
            {
                // (the above-count is summed from the bitmap words after the
                // loop, not per chunk: the scalar unit is this loop's limit)
                const int nchunk = (vis + T - 1) / T;
                const bool mine = lane < 2 * nchunk;
                if (mine) bm[(lane >> 1) * (T / 32) + 2 * (tc >> 6) + (lane & 1)] = static_cast<uint32_t>(bw);
                n_above = wave_allreduce(mine ? static_cast<uint32_t>(__popc(static_cast<uint32_t>(bw))) : 0u,
                                         [](uint32_t x, uint32_t y) { return x + y; });
            }
            if (lane == 0) { wc0[wave] = n_above; wc1[wave] = cnt; }
            lds_barrier();
            // the waves' counts, one per lane, summed across the wave
            uint32_t c0 = lane < NW ? wc0[lane] : 0u, c1 = lane < NW ? wc1[lane] : 0u;
            uint32_t ovf = c1 > static_cast<uint32_t>(kRegRegion) ? 1u : 0u;
            const auto add = [](uint32_t x, uint32_t y) { return x + y; };
            c0 = wave_allreduce(c0, add);
            c1 = wave_allreduce(c1, add);
            ovf = wave_allreduce(ovf, [](uint32_t x, uint32_t y) { return x | y; });
            above_all = __builtin_amdgcn_readfirstlane(c0);
            listed = __builtin_amdgcn_readfirstlane(c1);
            fast = !__builtin_amdgcn_readfirstlane(ovf) && above_all <= k && above_all + listed >= k;
        }
        if (!fast) {
            // the whole row selected in LDS; if the classify ran, the next row's
            // loads have replaced it: they complete, the row is loaded again,
            // and the next row follows once more after the select
            if (classified && fetch_next) {
                __builtin_amdgcn_s_waitcnt(kWaitVmem);
                lds_barrier();
                prefetch(lrow, vis);
                __builtin_amdgcn_s_waitcnt(kWaitVmem);
                lds_barrier();
            }
            float rmin = __builtin_inff(), rmax = -__builtin_inff();
            {
                const int tf = fresh_tid();
                for (int u = 0; u < P; ++u) {
                    const int i = tf + u * T;
                    if (i < vis) {
                        const float xv = key_at(i);
                        if (xv != __uint_as_float(keys[i])) keys[i] = __float_as_uint(xv);   // forced keys
                        if (xv > -__builtin_inff()) rmin = fminf(rmin, xv);
                        rmax = fmaxf(rmax, xv);
                    }
                }
            }
            for (int i = tid; i < nwords; i += T) bm[i] = 0u;
            rmin = wave_allmin(rmin);
            rmax = wave_allmax(rmax);
            __syncthreads();                  // every thread has read the sample's range
            if (lane == 0) { wmin[wave] = rmin; wmax[wave] = rmax; }
            if (tid == 0) n_list = 0;
            __syncthreads();
            for (int w = 0; w < NW; ++w) { rmin = fminf(rmin, wmin[w]); rmax = fmaxf(rmax, wmax[w]); }
            select_lds_row_lin(a, keys, vis, rmin, rmax, lh, bm, wsum, &n_list, out);
            __syncthreads();                  // every wave is done with keys[]
            if (fetch_next) prefetch(next, vis_next);
            vis = vis_next;
            continue;
        }
        if (above_all < k) {
            // the k - above best listed keys; second map linear over [d_lo, d_hi + 1)
            const uint32_t k_rem = k - above_all;
            const float lo2 = static_cast<float>(d_lo);
            const float scale2 = static_cast<float>(kRegBins2) / (static_cast<float>(d_hi + 1) - lo2);
            auto digit2 = [&](uint32_t bits) { return reg_digit2(bits, scale, off, lo2, scale2); };
            // (the arrays indexed directly, not through pointers, so the
            // compiler sees that they do not overlap the loads in flight)
            const int lb = 2 * wave * kRegRegion;
            const int mine = static_cast<int>(wc1[wave]);     // this wave's region
            for (int j = lane; j < mine; j += 64) lds_add(&lh[digit2(lpair[lb + 2 * j])], 1u);
            lds_barrier();
            // every wave finds the threshold bin itself (no barrier to publish it)
            int d2;
            uint32_t gt2;
            wave_find_bin_reg<kRegBins2>(lh, k_rem, &d2, &gt2);
            // the threshold bin's keys: (order key, ~position) word pairs in lh past the bins
            constexpr int TB = kRegBins2;
            for (int j = lane; j < mine; j += 64) {
                const uint32_t bits = lpair[lb + 2 * j];
                const int pos = static_cast<int>(lpair[lb + 2 * j + 1]);
                const int d = digit2(bits);
                if (d > d2) {
                    lds_or(&bm[pos >> 5], 1u << (pos & 31));
                } else if (d == d2) {
                    const uint32_t sl = lds_add_rtn(&n_list, 1u);
                    if (sl < static_cast<uint32_t>(kRegTieCap)) {
                        lh[TB + 2 * sl] = order_key(__uint_as_float(bits));
                        lh[TB + 2 * sl + 1] = ~static_cast<uint32_t>(pos);
                    }
                }
            }
            lds_barrier();
            const uint32_t n_t = n_list;
            const uint32_t k_t = k_rem - gt2;
            if (n_t > static_cast<uint32_t>(kRegTieCap)) {
                // a mass of nearly equal scores in the threshold bin: its listed
                // keys radix-selected (on the composite bits that vary among them)
                RegTieSrc src{lpair, wc1, kRegRegion, static_cast<int>(listed), scale, off, lo2, scale2, d2};
                Sink tsink{bm, nullptr, &n_list, k_t};
                radix_select_spread(src, k_t, lh, wsum, tsink);
            } else {
                for (uint32_t j = tid; j < n_t; j += T) {
                    const uint64_t c = (static_cast<uint64_t>(lh[TB + 2 * j]) << 32) | lh[TB + 2 * j + 1];
                    uint32_t beat = 0;
                    for (uint32_t q = 0; q < n_t; ++q)
                        beat += ((static_cast<uint64_t>(lh[TB + 2 * q]) << 32) | lh[TB + 2 * q + 1]) > c ? 1u : 0u;
                    if (beat < k_t) {
                        const int pos = static_cast<int>(~static_cast<uint32_t>(c & 0xFFFFFFFFull));
                        lds_or(&bm[pos >> 5], 1u << (pos & 31));
                    }
                }
            }
            lds_barrier();                    // every thread has read n_list; the bits are set
        }
        Sink sink{bm, nullptr, &n_list, k};
        write_ordered(sink, nwords, 1, a.k, out, wsum);
        lds_barrier();                        // the next row reuses the LDS
        vis = vis_next;
    }
}

// ---------------------------------------------------------------------------
// Rows of scores in memory much longer than k (prefill rows past a few
// thousand keys; dsa_topk over many such rows).  One workgroup per row:
//   sample  kRcSample order keys of the row -- runs of 16 consecutive keys
//           spread evenly over it, so every load is one 64-byte piece -- and a
//           lower bound k_low of their r-th largest, r ~ 1.5 k * samples /
//           visible keys + 24, about the (1.5 k + 24 * visible / samples)-th
//           largest key of the row;
//   collect one pass over the row keeps the keys at or above k_low as
//           (order key << 32 | ~position) in an LDS list (wave ballots, one
//           LDS atomic per wave and load);
//   select  the exact k largest of the list, radix-selected on the keys
//           relative to k_low (ties to the lower position), written in
//           ascending order through an LDS bitmap of the row.
// A list with at least k entries holds the k largest keys whatever the
// sample was (any key left out is below k_low, and k listed keys are not).
// A row whose list came out shorter than k, or overflowed, is selected again
// from its scores in memory (radix passes over the whole row), so the result
// never depends on the sample.
// ---------------------------------------------------------------------------
constexpr int kRcThreads = 512;
constexpr int kRcSample = 4096;

__global__ __launch_bounds__(kRcThreads) void k_topk_row_cand(TopkArgs a, int cap) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint64_t* cl = reinterpret_cast<uint64_t*>(smem);              // [cap] candidates
    uint32_t* skey = reinterpret_cast<uint32_t*>(smem);            // [kRcSample] samples, dead before collection
    uint32_t* tail = reinterpret_cast<uint32_t*>(cl + cap);        // bitmap of the row, or the list of kept keys
    __shared__ __align__(16) uint32_t lh[kTopkBins];
    __shared__ uint32_t wsum[kRcThreads / 64 + 2];
    __shared__ uint32_t wmin[kRcThreads / 64], wmax[kRcThreads / 64];
    __shared__ uint32_t n_c, n_list, n_tie;
    const int lrow = blockIdx.x, row = a.row0 + lrow;
    const int vis = row_visible(a, row);
    const int k = a.k;
    const int lane = threadIdx.x & 63;
    int32_t* out = a.idx + static_cast<size_t>(lrow) * k;
    if (vis <= k) {                                                // every visible key is kept
        for (int j = threadIdx.x; j < k; j += blockDim.x) out[j] = j < vis ? j : -1;
        return;
    }
    const float* sc = a.scores + static_cast<size_t>(lrow) * a.n_k;

    // the sample (all visible keys when there are at most kRcSample)
    const int m = vis < kRcSample ? vis : kRcSample;
    const int gap = vis / ((m + 15) / 16);                         // >= 16 unless m == vis
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    {
        constexpr int kPer = kRcSample / kRcThreads;
        float v[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {                           // loads first (past m: sample m - 1, unused)
            const int j = min(static_cast<int>(threadIdx.x) + u * kRcThreads, m - 1);
            v[u] = ranked(a, sc, m == vis ? j : (j >> 4) * gap + (j & 15), vis);
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int j = threadIdx.x + u * kRcThreads;
            if (j < m) {
                const uint32_t kk = order_key(v[u]);
                skey[j] = kk;
                kmin = min(kmin, kk);
                kmax = max(kmax, kk);
            }
        }
    }
    kmin = wave_allreduce(kmin, [](uint32_t p, uint32_t q) { return p < q ? p : q; });
    kmax = wave_allreduce(kmax, [](uint32_t p, uint32_t q) { return p > q ? p : q; });
    if (lane == 0) { wmin[threadIdx.x >> 6] = kmin; wmax[threadIdx.x >> 6] = kmax; }
    __syncthreads();
    for (int w = 0; w < kRcThreads / 64; ++w) { kmin = min(kmin, wmin[w]); kmax = max(kmax, wmax[w]); }
    const int64_t want = (3 * static_cast<int64_t>(m) * k + 2 * static_cast<int64_t>(vis) - 1) /
                         (2 * static_cast<int64_t>(vis)) + 24;
    const uint32_t k_low = want < m ? lower_bound_rth(skey, m, static_cast<uint32_t>(want), kmin, kmax, lh, wsum)
                                    : 0u;
    __syncthreads();                                               // the samples are dead from here

    // collect the keys at or above k_low
    const bool use_bitmap = a.n_k <= kBitmapMaxKeys;
    const int nwords = (vis + 31) >> 5;
    int kpad = 1;
    while (kpad < k) kpad <<= 1;
    if (use_bitmap) {
        for (int i = threadIdx.x; i < nwords; i += blockDim.x) tail[i] = 0u;
    } else {
        for (int i = threadIdx.x; i < kpad; i += blockDim.x) tail[i] = 0x7FFFFFFFu;
    }
    if (threadIdx.x == 0) { n_c = 0u; n_list = 0u; }
    __syncthreads();
    const uint64_t below = (1ull << lane) - 1ull;
    // one wave-wide append of this lane's key s if it takes it
    auto append = [&](int s, float x) {
        const float r = (s < a.sinks || s >= vis - a.window) ? -__builtin_inff() : x;
        const uint32_t key = order_key(r);
        const bool take = s < vis && key >= k_low;
        const uint64_t msk = __ballot(take);
        if (msk) {
            uint32_t base_slot = 0;
            if (lane == 0) base_slot = atomicAdd(&n_c, static_cast<uint32_t>(__popcll(msk)));
            base_slot = __shfl(base_slot, 0);
            const uint32_t slot = base_slot + static_cast<uint32_t>(__popcll(msk & below));
            if (take && slot < static_cast<uint32_t>(cap)) cl[slot] = composite64(key, s);
        }
    };
    // (lane 0 of a wave has the wave's lowest index, so it is active whenever
    // any lane of the wave is; every load is issued before any key is used)
    if ((a.n_k & 3) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0) {
        // rows start 16-byte aligned: 16-byte loads of four keys; groups past
        // vis re-read the last group (inside the row: 4 * ceil(vis / 4) <= n_k)
        const int nv4 = (vis + 3) >> 2;
        for (int g0 = threadIdx.x; g0 < nv4; g0 += 8 * kRcThreads) {
            float4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = *reinterpret_cast<const float4*>(sc + 4 * min(g0 + u * kRcThreads, nv4 - 1));
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int s = 4 * (g0 + u * kRcThreads);
                append(s, v[u].x);
                append(s + 1, v[u].y);
                append(s + 2, v[u].z);
                append(s + 3, v[u].w);
            }
        }
    } else {
        for (int i0 = threadIdx.x; i0 < vis; i0 += 8 * kRcThreads) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = sc[min(i0 + u * kRcThreads, vis - 1)];
#pragma unroll
            for (int u = 0; u < 8; ++u) append(i0 + u * kRcThreads, v[u]);
        }
    }
    __syncthreads();
    const uint32_t n = n_c;
    Sink sink{use_bitmap ? tail : nullptr, reinterpret_cast<int32_t*>(tail), &n_list, static_cast<uint32_t>(k)};
    if (n >= static_cast<uint32_t>(k) && n <= static_cast<uint32_t>(cap)) {
        uint32_t cmax = 0u;
        for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) cmax = max(cmax, static_cast<uint32_t>(cl[i] >> 32));
        cmax = wave_allreduce(cmax, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
        if (lane == 0) wmax[threadIdx.x >> 6] = cmax;
        __syncthreads();
        for (int w = 0; w < kRcThreads / 64; ++w) cmax = max(cmax, wmax[w]);
        // digits of ((key - k_low) << 32 | ~position): the first over the top
        // 11 bits of the candidates' key range, then 11 bits at a time
        const uint32_t range = cmax - k_low;
        const int bits = range ? 32 - __clz(static_cast<int>(range)) : 0;
        const int sh = bits > 11 ? bits - 11 : 0;
        int shifts[6], widths[6], np = 1;
        shifts[0] = 32 + sh;
        widths[0] = 11;
        for (int rest = 32 + sh; rest > 0 && np < 6; ++np) {
            const int w = rest < 11 ? rest : 11;
            rest -= w;
            shifts[np] = rest;
            widths[np] = w;
        }
        select_candidates(cl, n, k_low, static_cast<uint32_t>(k), shifts, widths, np, lh, wsum, &n_tie, sink);
    } else {
        // the whole row, on the bits of the composite that vary
        ScoreRow64 src{sc, vis, a.sinks, vis - a.window};
        radix_select_spread(src, static_cast<uint32_t>(k), lh, wsum, sink);
    }
    __syncthreads();
    write_ordered(sink, nwords, kpad, k, out, wsum);
}

// Candidate list capacity for a launch whose rows have at most vis_max keys:
// about 1.6 x the expected list length, at least the sample's size.
static int row_cand_cap(int k, int vis_max) {
    const int64_t expect = (3 * static_cast<int64_t>(k)) / 2 + 24 * ((vis_max + kRcSample - 1) / kRcSample);
    int64_t cap = (expect * 8) / 5 + 512;
    cap = (cap + 255) & ~static_cast<int64_t>(255);
    if (cap < kRcSample / 2) cap = kRcSample / 2;                 // the samples alias the list
    if (cap > kTopkCandCapMax) cap = kTopkCandCapMax;
    return static_cast<int>(cap);
}

size_t topk_workspace_bytes(int rows, int n_k) {
    size_t r = static_cast<size_t>(rows);
    size_t zeroed = align256(r * (2 * kTopkBins + kTopkMeta) * sizeof(uint32_t));
    size_t cand = r * static_cast<size_t>(topk_cand_cap(n_k)) * sizeof(uint64_t);
    return zeroed + cand;
}

void topk_carve(void* ws, int rows, int n_k, TopkArgs& a) {
    unsigned char* p = static_cast<unsigned char*>(ws);
    size_t r = static_cast<size_t>(rows);
    a.hist = reinterpret_cast<uint32_t*>(p);
    a.hist1 = a.hist + r * kTopkBins;
    a.count = a.hist1 + r * kTopkBins;
    a.zero_words = r * (2 * kTopkBins + kTopkMeta);
    p += align256(a.zero_words * sizeof(uint32_t));
    a.cand = reinterpret_cast<uint64_t*>(p);
    a.cand_cap = topk_cand_cap(n_k);
}

// `a.rows` rows starting at absolute row a.row0; scores, idx and the
// workspace are indexed from the first of them.  Unless a.hist_ready, the
// workspace's counters are cleared and the digit-0 histogram built here.
// The longest visible prefix among the rows of a launch: known on the host
// when positions are implicit (pos = n_k - n_q + t), else n_k.
static int launch_vis_max(const TopkArgs& a) {
    int vis_max = a.n_k;
    if (!a.q_pos && a.rows > 0) {
        const int last = a.row0 + a.rows - 1;
        const int t_max = a.row0 / a.n_q == last / a.n_q ? last % a.n_q : a.n_q - 1;
        vis_max = min(a.n_k, a.n_k - a.n_q + t_max + 1);
        if (vis_max < 1) vis_max = 1;
    }
    return vis_max;
}


// Launches of many rows, some much longer than k, select through sampled
// candidate lists (k_topk_row_cand) when some row exceeds kRowLdsMax keys
// (measured: rows of up to 32K keys select faster whole in LDS, 1.92 against
// 2.21 ms on the 32K prefill; DSA_TOPK_ROWCAND_LDS = 1 sends them here too).
#ifndef DSA_TOPK_ROWCAND_LDS
#define DSA_TOPK_ROWCAND_LDS 0
#endif
constexpr int kRowCandMinRows = 128;
static bool use_row_cand(const TopkArgs& a, int vis_max) {
    if (a.rows < kRowCandMinRows || a.k > 4096) return false;
    if (static_cast<int64_t>(vis_max) < 4 * static_cast<int64_t>(a.k) || vis_max < 2 * kRcSample) return false;
    return DSA_TOPK_ROWCAND_LDS || vis_max > kRowLdsMax;
}

bool topk_uses_hist(const TopkArgs& a) {
    const int vis_max = launch_vis_max(a);
    return !use_row_cand(a, vis_max) && vis_max > kRowLdsMax;
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
    hipError_t e;
    const int vis_max = launch_vis_max(a);
    if (use_row_cand(a, vis_max)) {
        const int cap = row_cand_cap(a.k, vis_max);
        int kpad = 1;
        while (kpad < a.k) kpad <<= 1;
        const size_t tail = a.n_k <= kBitmapMaxKeys ? static_cast<size_t>((a.n_k + 31) >> 5) * 4
                                                    : static_cast<size_t>(kpad) * 4;
        const size_t smem = static_cast<size_t>(cap) * sizeof(uint64_t) + tail;
        if ((e = allow_dyn_lds(reinterpret_cast<const void*>(k_topk_row_cand), smem)) != hipSuccess) return e;
        hipLaunchKernelGGL(k_topk_row_cand, dim3(a.rows), dim3(kRcThreads), smem, st, a, cap);
        return hipGetLastError();
    }
    // rows of at most kRowLdsMax visible keys (all rows of a short prefill,
    // the early row blocks of a long one) are selected from LDS
    if (vis_max <= kRowLdsMax) {
        if (vis_max > (DSA_TOPK_ROW_REG ? DSA_TOPK_ROW_REG_MIN : kRowLdsMax / 2)) {
            const void* fn = DSA_TOPK_ROW_REG ? reinterpret_cast<const void*>(k_topk_row_reg)
                                              : reinterpret_cast<const void*>(k_topk_row_lds_next);
            // (the register select holds its row buffer in static LDS)
            const size_t smem = DSA_TOPK_ROW_REG ? 0 : static_cast<size_t>(kRowLdsMax) * sizeof(uint32_t);
            if ((e = allow_dyn_lds(fn, smem)) != hipSuccess) return e;
            // workgroups the chip holds at once (one per CU at this LDS size)
            static const int per_cu = [fn] {
                int nb = 0;
                return hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, DSA_TOPK_ROW_REG ? kRegThreads : kRowThreads, smem) == hipSuccess && nb > 0
                    ? nb : 1;
            }();
            int dev = 0, cus = 0;
            if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
            if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
            const long long slots = static_cast<long long>(per_cu) * (cus > 0 ? cus : 1);
            const dim3 grid(static_cast<unsigned>(a.rows < slots ? a.rows : slots));
            if (DSA_TOPK_ROW_REG)
                hipLaunchKernelGGL(k_topk_row_reg, grid, dim3(kRegThreads), smem, st, a);
            else
                hipLaunchKernelGGL(k_topk_row_lds_next, grid, dim3(kRowThreads), smem, st, a);
            return hipGetLastError();
        }
        const size_t smem = static_cast<size_t>(vis_max) * sizeof(uint32_t);
        // rows of up to 8K keys leave LDS for three workgroups per CU, which
        // 1024-thread workgroups cannot reach (two fill the CU's waves)
        if (vis_max <= kRowLdsMax / 4) {
            hipLaunchKernelGGL(k_topk_row_lds<512>, dim3(a.rows), dim3(512), smem, st, a);
            return hipGetLastError();
        }
        if ((e = allow_dyn_lds(reinterpret_cast<const void*>(k_topk_row_lds<kRowThreads>), smem)) != hipSuccess)
            return e;
        hipLaunchKernelGGL(k_topk_row_lds<kRowThreads>, dim3(a.rows), dim3(kRowThreads), smem, st, a);
        return hipGetLastError();
    }
    const dim3 grid((a.n_k + kChunk - 1) / kChunk, a.rows);
    if (!a.hist_ready) {
        if ((e = launch_zero_u32(a.hist, a.zero_words, st)) != hipSuccess) return e;
        hipLaunchKernelGGL(k_topk_hist, grid, dim3(kFilterThreads), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_topk_threshold, dim3(a.rows), dim3(kFilterThreads), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 fgrid((a.n_k + kFChunk - 1) / kFChunk, a.rows);
    hipLaunchKernelGGL(k_topk_filter, fgrid, dim3(kFThreads), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t smem = finish_lds_bytes(a);
    if ((e = allow_dyn_lds(reinterpret_cast<const void*>(k_topk_finish), smem)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_topk_finish, dim3(a.rows), dim3(kFinishThreads), smem, st, a);
    return hipGetLastError();
}

}  // namespace dsa
