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
// the histogram.
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

// Candidate sources for the finishing select: a list (LDS or global), or,
// when the digit-0 bin overflowed the list, the score row itself filtered to
// that bin.
struct CandList {
    const uint64_t* c; int n;
    __device__ int size() const { return n; }
    __device__ bool get(int i, uint64_t* out) const { *out = c[i]; return true; }
};
struct CandRow {
    const float* sc; int n; int d0;
    int lo, hi;                 // keys outside [lo, hi) rank as -inf (a backbone's forced keys)
    __device__ int size() const { return n; }
    __device__ bool get(int i, uint64_t* out) const {
        const float x = sc[i];
        uint32_t key = order_key(i < lo || i >= hi ? -__builtin_inff() : x);
        if (static_cast<int>(key >> 21) != d0) return false;
        *out = composite(key, i);
        return true;
    }
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
    const int d0 = static_cast<int>(meta[M_D0]);
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
        // the list overflowed: read the row again, filtered to the d0 bin
        CandRow row_src{a.scores + static_cast<size_t>(lrow) * a.n_k, vis, d0, a.sinks, vis - a.window};
        for_each_candidate(row_src, [&](uint64_t c) {
            int dg = static_cast<int>(c >> 42);
            if (dg > d1 || (dg == d1 && whole_bin)) sink.put_c(c);
        });
        __syncthreads();
        if (!whole_bin) select_in_bin(row_src, d1, k2, lh, wsum, sink);
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

bool topk_row_lds(int n_k) { return n_k <= kRowLdsMax; }

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

template <int T>
__global__ __launch_bounds__(T) void k_topk_row_lds(TopkArgs a) {
    extern __shared__ uint32_t keys[];                        // [min(n_k, kRowLdsMax)]
    __shared__ uint32_t lh[kTopkBins];
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
    // the row's keys, eight loads in flight per thread (indices past vis
    // re-read the last score and are not stored)
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    for (int i0 = threadIdx.x; i0 < vis; i0 += 8 * T) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = ranked(a, sc, min(i0 + u * T, vis - 1), vis);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * T;
            if (i < vis) {
                const uint32_t kk = order_key(v[u]);
                keys[i] = kk;
                kmin = min(kmin, kk);
                kmax = max(kmax, kk);
            }
        }
    }
    const int nwords = (vis + 31) >> 5;
    for (int i = threadIdx.x; i < nwords; i += T) bm[i] = 0u;
    if (threadIdx.x == 0) n_list = 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), o)));
        kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), o)));
    }
    __shared__ uint32_t wmin[T / 64], wmax[T / 64];
    if ((threadIdx.x & 63) == 0) { wmin[threadIdx.x >> 6] = kmin; wmax[threadIdx.x >> 6] = kmax; }
    __syncthreads();
    for (int w = 0; w < T / 64; ++w) { kmin = min(kmin, wmin[w]); kmax = max(kmax, wmax[w]); }
    select_lds_row(a, keys, vis, kmin, kmax, lh, bm, wsum, &n_list, out);
}

// Rows longer than half the LDS limit leave room for one workgroup per
// compute unit, so nothing hides a row's load behind another row's select.
// This persistent form does it inside the workgroup: workgroup w takes rows
// w, w + gridDim.x, ...; while it selects one row, the next row's scores
// (kRowPerThread per thread) are already in flight into registers.
constexpr int kRowPerThread = kRowLdsMax / kRowThreads;
__global__ __launch_bounds__(kRowThreads) void k_topk_row_lds_next(TopkArgs a) {
    extern __shared__ uint32_t keys[];                        // [kRowLdsMax]
    __shared__ uint32_t lh[kTopkBins];
    __shared__ uint32_t bm[kRowLdsMax / 32];
    __shared__ uint32_t wsum[kRowThreads / 64 + 2];
    __shared__ uint32_t wmin[kRowThreads / 64], wmax[kRowThreads / 64];
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
            uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
            for (int u = 0; u < kRowPerThread; ++u) {
                const int i = static_cast<int>(threadIdx.x) + u * kRowThreads;
                if (i < vis) {
                    // a backbone's forced keys rank as -inf (as ranked() does)
                    const float x = (i < a.sinks || i >= vis - a.window) ? -__builtin_inff() : v[u];
                    const uint32_t kk = order_key(x);
                    keys[i] = kk;
                    kmin = min(kmin, kk);
                    kmax = max(kmax, kk);
                }
            }
            const int nwords = (vis + 31) >> 5;
            for (int i = threadIdx.x; i < nwords; i += kRowThreads) bm[i] = 0u;
            if (threadIdx.x == 0) n_list = 0;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                kmin = min(kmin, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmin), o)));
                kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(static_cast<int>(kmax), o)));
            }
            if ((threadIdx.x & 63) == 0) { wmin[threadIdx.x >> 6] = kmin; wmax[threadIdx.x >> 6] = kmax; }
            __syncthreads();
            for (int w = 0; w < kRowThreads / 64; ++w) { kmin = min(kmin, wmin[w]); kmax = max(kmax, wmax[w]); }
            if (next < a.rows && vis_next > a.k) fetch(next, vis_next);   // lands during the select
            select_lds_row(a, keys, vis, kmin, kmax, lh, bm, wsum, &n_list, out);
        }
        __syncthreads();                    // the next row's keys reuse the LDS
        vis = vis_next;
    }
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
hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
    hipError_t e;
    if (topk_row_lds(a.n_k)) {
        // LDS for the longest visible prefix among the rows: known on the
        // host when positions are implicit (pos = n_k - n_q + t), else n_k
        int vis_max = a.n_k;
        if (!a.q_pos && a.rows > 0) {
            const int last = a.row0 + a.rows - 1;
            const int t_max = a.row0 / a.n_q == last / a.n_q ? last % a.n_q : a.n_q - 1;
            vis_max = min(a.n_k, a.n_k - a.n_q + t_max + 1);
            if (vis_max < 1) vis_max = 1;
        }
        if (vis_max > kRowLdsMax / 2) {
            const void* fn = reinterpret_cast<const void*>(k_topk_row_lds_next);
            const size_t smem = static_cast<size_t>(kRowLdsMax) * sizeof(uint32_t);
            if ((e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem))) !=
                hipSuccess)
                return e;
            // workgroups the chip holds at once (one per CU at this LDS size)
            static const int per_cu = [fn, smem] {
                int nb = 0;
                return hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kRowThreads, smem) == hipSuccess && nb > 0
                    ? nb : 1;
            }();
            int dev = 0, cus = 0;
            if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
            if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
            const long long slots = static_cast<long long>(per_cu) * (cus > 0 ? cus : 1);
            const dim3 grid(static_cast<unsigned>(a.rows < slots ? a.rows : slots));
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
        if (smem > 64 * 1024) {
            e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_topk_row_lds<kRowThreads>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
            if (e != hipSuccess) return e;
        }
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
    if (smem > 64 * 1024) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_topk_finish),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_topk_finish, dim3(a.rows), dim3(kFinishThreads), smem, st, a);
    return hipGetLastError();
}

}  // namespace dsa
