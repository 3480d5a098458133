// topk.hip -- per-row top-k selector over fp32 score rows.
//
// The selector keeps the k highest-scoring keys of each query
// ("DeepSeek-V3.2-Exp 稀疏注意力机制(DSA)技术深度解析", sheratonhq.com,
// section 1; the fine-grained selector stage of "DeepSeek-V4 百万 token 上下文的
// 工程实现", blog.hotdry.top, section "从 O(N²) 到 O(N・k)").  Ties go to the
// lower position.
//
// Method: radix select on order-preserving uint32 keys, never a full sort.
//   1. hist   every workgroup histograms the top 11 key bits of its slice of
//             the row into LDS and adds the non-empty bins to the row's global
//             histogram (or the score producer already did this).
//   2. filter every workgroup finds the bin holding the k-th key, writes the
//             positions above that bin straight into the output row and
//             appends the bin's own entries to a candidate list.
//   3. finish one workgroup per row radix-selects the remaining k' entries
//             among the candidates in LDS on the 53-bit composite
//             (low 21 key bits, ~position) -- so equal scores resolve to the
//             lower position -- then bitonic-sorts the row's k positions.
// The score row is read twice from memory (steps 1 and 2) and never sorted.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kChunk = 2048;       // scores per workgroup in hist/filter
constexpr int kFilterThreads = 256;
constexpr int kPerThread = kChunk / kFilterThreads;
constexpr int kFinishThreads = 512;

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

// Block-wide search of the threshold bin: the digit d with
//   count(bins > d) < k_rem <= count(bins >= d).
// `hist` (nbins entries) and `scan` (blockDim entries) are LDS.  Every thread
// returns the same d and count(bins > d).  Requires sum(hist) >= k_rem >= 1.
__device__ void find_threshold_bin(const uint32_t* hist, int nbins, uint32_t k_rem,
                                   uint32_t* scan, int* sh_digit, uint32_t* sh_gt,
                                   int* digit, uint32_t* gt)
{
    const int T = blockDim.x, tid = threadIdx.x;
    const int per = (nbins + T - 1) / T;
    uint32_t local = 0;
    for (int j = 0; j < per; ++j) {
        int bin = nbins - 1 - (tid * per + j);
        if (bin >= 0) local += hist[bin];
    }
    scan[tid] = local;
    __syncthreads();
    for (int off = 1; off < T; off <<= 1) {
        uint32_t v = tid >= off ? scan[tid - off] : 0u;
        __syncthreads();
        scan[tid] += v;
        __syncthreads();
    }
    uint32_t excl = scan[tid] - local;
    if (excl < k_rem && excl + local >= k_rem) {
        uint32_t run = excl;
        for (int j = 0; j < per; ++j) {
            int bin = nbins - 1 - (tid * per + j);
            if (bin < 0) break;
            if (run + hist[bin] >= k_rem) { *sh_digit = bin; *sh_gt = run; break; }
            run += hist[bin];
        }
    }
    __syncthreads();
    *digit = *sh_digit;
    *gt = *sh_gt;
    __syncthreads();
}

__device__ __forceinline__ int row_visible(const TopkArgs& a, int row) {
    return row_pos(a.q_pos, row, a.n_q, a.n_k) + 1;   // 0..n_k
}

// Step 1: histogram of the top 11 bits of every visible key.  Every thread
// issues all of its loads before it touches any of them.
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
        x[u] = s < c1 ? sc[s] : 0.0f;
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

// Step 2: keep everything above the threshold bin, collect the bin itself.
__global__ __launch_bounds__(kFilterThreads) void k_topk_filter(TopkArgs a) {
    __shared__ uint32_t lh[kTopkBins];
    __shared__ uint32_t scan[kFilterThreads];
    __shared__ int32_t sel_buf[kChunk];
    __shared__ uint64_t cand_buf[kChunk];
    __shared__ int sh_digit;
    __shared__ uint32_t sh_gt, n_sel, n_cand, g_sel, g_cand;
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
        x[u] = s < c1 ? sc[s] : 0.0f;
    }
    const uint32_t* gh = a.hist + static_cast<size_t>(lrow) * kTopkBins;
    for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x) lh[i] = gh[i];
    if (threadIdx.x == 0) { n_sel = 0; n_cand = 0; }
    __syncthreads();
    int d0; uint32_t gt0;
    find_threshold_bin(lh, kTopkBins, static_cast<uint32_t>(a.k), scan, &sh_digit, &sh_gt, &d0, &gt0);

    const int lane = threadIdx.x & 63;
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int u = 0; u < kPerThread; ++u) {
        int s = c0 + u * kFilterThreads + threadIdx.x;
        uint32_t key = s < c1 ? order_key(x[u]) : 0u;
        int dg = static_cast<int>(key >> 21);
        bool is_sel = s < c1 && dg > d0;
        bool is_cand = s < c1 && dg == d0;
        uint64_t ms = __ballot(is_sel);
        uint64_t mc = __ballot(is_cand);
        uint32_t bs = 0, bc = 0;
        if (lane == 0) {
            if (ms) bs = atomicAdd(&n_sel, static_cast<uint32_t>(__popcll(ms)));
            if (mc) bc = atomicAdd(&n_cand, static_cast<uint32_t>(__popcll(mc)));
        }
        bs = __shfl(bs, 0);
        bc = __shfl(bc, 0);
        if (is_sel) sel_buf[bs + __popcll(ms & below)] = s;
        if (is_cand)
            cand_buf[bc + __popcll(mc & below)] =
                (static_cast<uint64_t>(key & 0x1FFFFFu) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(s));
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t* cnt = a.count + static_cast<size_t>(lrow) * 2;
        g_sel = n_sel ? atomicAdd(&cnt[0], n_sel) : 0u;
        g_cand = n_cand ? atomicAdd(&cnt[1], n_cand) : 0u;
    }
    __syncthreads();
    int32_t* out = a.idx + static_cast<size_t>(lrow) * a.k;
    for (uint32_t i = threadIdx.x; i < n_sel; i += blockDim.x) {
        uint32_t slot = g_sel + i;
        if (slot < static_cast<uint32_t>(a.k)) out[slot] = sel_buf[i];
    }
    uint64_t* cd = a.cand + static_cast<size_t>(lrow) * a.cand_cap;
    for (uint32_t i = threadIdx.x; i < n_cand; i += blockDim.x) {
        uint32_t slot = g_cand + i;
        if (slot < static_cast<uint32_t>(a.cand_cap)) cd[slot] = cand_buf[i];
    }
}

// Candidate source for the finishing select: the compacted list in LDS, or,
// when the threshold bin overflowed the list, the score row itself filtered
// to that bin.
struct CandList {
    const uint64_t* c; int n;
    __device__ int size() const { return n; }
    __device__ bool get(int i, uint64_t* out) const { *out = c[i]; return true; }
};
struct CandRow {
    const float* sc; int n; int d0;
    __device__ int size() const { return n; }
    __device__ bool get(int i, uint64_t* out) const {
        uint32_t key = order_key(sc[i]);
        if (static_cast<int>(key >> 21) != d0) return false;
        *out = (static_cast<uint64_t>(key & 0x1FFFFFu) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(i));
        return true;
    }
};

// Visit every candidate of `src`, eight loads in flight per thread.
template <class Src, class F>
__device__ __forceinline__ void for_each_candidate(const Src& src, F&& f) {
    const int n = src.size();
    const int T = blockDim.x;
    int i = threadIdx.x;
    for (; i + 7 * T < n; i += 8 * T) {
        uint64_t c[8];
        bool ok[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) ok[u] = src.get(i + u * T, &c[u]);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (ok[u]) f(c[u]);
    }
    for (; i < n; i += T) {
        uint64_t c;
        if (src.get(i, &c)) f(c);
    }
}

// Radix-select the k_rem largest composites of `src` and append their
// positions to sorted[] at *n_out (an LDS counter).
template <class Src>
__device__ void select_candidates(const Src& src, uint32_t k_rem, uint32_t* lh, uint32_t* scan,
                                  int* sh_digit, uint32_t* sh_gt, int32_t* sorted, uint32_t* n_out,
                                  uint32_t cap)
{
    // Digits of the 53-bit composite, most significant first.
    const int shifts[5] = {42, 31, 20, 9, 0};
    const int widths[5] = {11, 11, 11, 11, 9};
    uint64_t prefix = 0;
    int done_shift = 0;
    for (int p = 0; p < 5; ++p) {
        const int sh = shifts[p], w = widths[p];
        const int nb = 1 << w;
        for (int i = threadIdx.x; i < nb; i += blockDim.x) lh[i] = 0u;
        __syncthreads();
        for_each_candidate(src, [&](uint64_t c) {
            if ((c >> (sh + w)) == prefix) atomicAdd(&lh[(c >> sh) & (nb - 1)], 1u);
        });
        __syncthreads();
        int d; uint32_t gt;
        find_threshold_bin(lh, nb, k_rem, scan, sh_digit, sh_gt, &d, &gt);
        k_rem -= gt;
        prefix = (prefix << w) | static_cast<uint64_t>(d);
        done_shift = sh;
        bool done = lh[d] == k_rem;
        __syncthreads();
        if (done) break;
    }
    for_each_candidate(src, [&](uint64_t c) {
        if ((c >> done_shift) >= prefix) {
            uint32_t slot = atomicAdd(n_out, 1u);
            if (slot < cap) sorted[slot] = static_cast<int32_t>(~static_cast<uint32_t>(c & 0xFFFFFFFFull));
        }
    });
    __syncthreads();
}

// Step 3: exact select inside the threshold bin, then sort the row's picks.
__global__ __launch_bounds__(kFinishThreads) void k_topk_finish(TopkArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    uint64_t* cl = reinterpret_cast<uint64_t*>(smem);                       // [cand_cap]
    int32_t* sorted = reinterpret_cast<int32_t*>(cl + a.cand_cap);           // [kpad]
    __shared__ uint32_t lh[kTopkBins];
    __shared__ uint32_t scan[kFinishThreads];
    __shared__ int sh_digit;
    __shared__ uint32_t sh_gt, n_out;
    const int lrow = blockIdx.x, row = a.row0 + lrow;
    const int vis = row_visible(a, row);
    int32_t* out = a.idx + static_cast<size_t>(lrow) * a.k;
    if (vis <= a.k) {                            // every visible key is kept
        for (int j = threadIdx.x; j < a.k; j += blockDim.x) out[j] = j < vis ? j : -1;
        return;
    }
    const uint32_t* gh = a.hist + static_cast<size_t>(lrow) * kTopkBins;
    for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x) lh[i] = gh[i];
    __syncthreads();
    int d0; uint32_t gt0;
    find_threshold_bin(lh, kTopkBins, static_cast<uint32_t>(a.k), scan, &sh_digit, &sh_gt, &d0, &gt0);
    int kpad = 1;
    while (kpad < a.k) kpad <<= 1;
    for (int j = threadIdx.x; j < kpad; j += blockDim.x)
        sorted[j] = j < static_cast<int>(gt0) ? out[j] : 0x7FFFFFFF;
    if (threadIdx.x == 0) n_out = gt0;
    const uint32_t n_cand = a.count[static_cast<size_t>(lrow) * 2 + 1];
    __syncthreads();
    const uint32_t k_rem = static_cast<uint32_t>(a.k) - gt0;
    if (n_cand <= static_cast<uint32_t>(a.cand_cap)) {
        const uint64_t* gc = a.cand + static_cast<size_t>(lrow) * a.cand_cap;
        for (uint32_t i = threadIdx.x; i < n_cand; i += blockDim.x) cl[i] = gc[i];
        __syncthreads();
        CandList src{cl, static_cast<int>(n_cand)};
        select_candidates(src, k_rem, lh, scan, &sh_digit, &sh_gt, sorted, &n_out, static_cast<uint32_t>(a.k));
    } else {
        CandRow src{a.scores + static_cast<size_t>(lrow) * a.n_k, vis, d0};
        select_candidates(src, k_rem, lh, scan, &sh_digit, &sh_gt, sorted, &n_out, static_cast<uint32_t>(a.k));
    }
    // Bitonic sort of the kpad entries, ascending.
    for (int size = 2; size <= kpad; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = threadIdx.x; i < (kpad >> 1); i += blockDim.x) {
                int lo = 2 * i - (i & (stride - 1));
                int hi = lo + stride;
                bool asc = (lo & size) == 0;
                int32_t x = sorted[lo], y = sorted[hi];
                if ((x > y) == asc) { sorted[lo] = y; sorted[hi] = x; }
            }
            __syncthreads();
        }
    }
    for (int j = threadIdx.x; j < a.k; j += blockDim.x) out[j] = sorted[j];
}

int topk_cand_cap(int n_k) {
    return n_k < kTopkCandCapMax ? n_k : kTopkCandCapMax;
}

size_t topk_workspace_bytes(int rows, int n_k) {
    size_t r = static_cast<size_t>(rows);
    size_t hist = r * kTopkBins * sizeof(uint32_t);
    size_t cnt = ((r * 2 * sizeof(uint32_t)) + 255) & ~static_cast<size_t>(255);
    size_t cand = r * static_cast<size_t>(topk_cand_cap(n_k)) * sizeof(uint64_t);
    return hist + cnt + cand;
}

void topk_carve(void* ws, int rows, int n_k, TopkArgs& a) {
    unsigned char* p = static_cast<unsigned char*>(ws);
    size_t r = static_cast<size_t>(rows);
    a.hist = reinterpret_cast<uint32_t*>(p);
    p += r * kTopkBins * sizeof(uint32_t);
    a.count = reinterpret_cast<uint32_t*>(p);
    p += ((r * 2 * sizeof(uint32_t)) + 255) & ~static_cast<size_t>(255);
    a.cand = reinterpret_cast<uint64_t*>(p);
    a.cand_cap = topk_cand_cap(n_k);
}

// `a.rows` rows starting at absolute row a.row0; scores, idx and the
// workspace are indexed from the first of them.
hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
    hipError_t e;
    const size_t r = static_cast<size_t>(a.rows);
    if (!a.hist_ready) {
        e = launch_zero_u32(a.hist, r * kTopkBins + r * 2, st);  // hist and count are adjacent
        if (e != hipSuccess) return e;
    }
    const dim3 grid((a.n_k + kChunk - 1) / kChunk, a.rows);
    if (!a.hist_ready) {
        hipLaunchKernelGGL(k_topk_hist, grid, dim3(kFilterThreads), 0, st, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_topk_filter, grid, dim3(kFilterThreads), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    int kpad = 1;
    while (kpad < a.k) kpad <<= 1;
    const size_t smem = static_cast<size_t>(a.cand_cap) * sizeof(uint64_t) + static_cast<size_t>(kpad) * sizeof(int32_t);
    if (smem > 64 * 1024) {
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_topk_finish),
                                hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_topk_finish, dim3(a.rows), dim3(kFinishThreads), smem, st, a);
    return hipGetLastError();
}

}  // namespace dsa
