// topk_common.h -- block-level building blocks of the radix top-k selectors
// (threshold-bin search, block scan, batched candidate visits, the sink that
// collects kept positions, a generic radix select and the ordered write-out).
#pragma once

#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kBitmapMaxKeys = 1 << 18;   // rows up to this long are ordered through a bitmap

// Block-wide search of the threshold bin: the digit d with
//   count(bins > d) < k_rem <= count(bins >= d).
// `hist` has nbins LDS entries (nbins and blockDim.x powers of two; with
// fewer bins than threads, the first nbins threads own one bin each); `wsum`
// is an LDS array of one slot per wave plus two result slots.  Every thread
// returns the same d and count(bins > d).  Requires sum(hist) >= k_rem >= 1.
__device__ inline void find_threshold_bin(const uint32_t* hist, int nbins, uint32_t k_rem,
                                   uint32_t* wsum, int* digit, uint32_t* gt)
{
    const int T = blockDim.x, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, nwaves = T >> 6;
    const int per = nbins >= T ? nbins / T : (tid < nbins ? 1 : 0);
    const int top = nbins - 1 - tid * per;      // this thread's bins: top, top-1, ...
    uint32_t local = 0;
    for (int j = 0; j < per; ++j) local += hist[top - j];
    uint32_t x = local;                          // inclusive scan inside the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const uint32_t excl = before + x - local;
    if (excl < k_rem && excl + local >= k_rem) {
        uint32_t run = excl;
        for (int j = 0; j < per; ++j) {
            uint32_t h = hist[top - j];
            if (run + h >= k_rem) { wsum[nwaves] = static_cast<uint32_t>(top - j); wsum[nwaves + 1] = run; break; }
            run += h;
        }
    }
    __syncthreads();
    *digit = static_cast<int>(wsum[nwaves]);
    *gt = wsum[nwaves + 1];
    __syncthreads();
}

// Block-wide exclusive scan of one value per thread (wave scans, then the
// wave totals); `wsum` holds one LDS slot per wave.  Returns the exclusive
// prefix; *total gets the block sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (int w = 0; w < nwaves; ++w) {
        uint32_t t = wsum[w];
        if (w < wave) before += t;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + x - v;
}

// dst[i] = src[i] for i < n (global -> LDS), eight loads in flight per thread.
template <class T>
__device__ __forceinline__ void copy_to_lds(T* dst, const T* src, int n) {
    const int T_ = blockDim.x;
    int i = threadIdx.x;
    for (; i + 7 * T_ < n; i += 8 * T_) {
        T v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = src[i + u * T_];
#pragma unroll
        for (int u = 0; u < 8; ++u) dst[i + u * T_] = v[u];
    }
    for (; i < n; i += T_) dst[i] = src[i];
}

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

// Where the finish puts kept positions: bits of an LDS bitmap over the row
// (rows up to kBitmapMaxKeys keys; read back in position order), or an LDS
// list sorted afterwards.
struct Sink {
    uint32_t* bitmap;      // null when the list is used
    int32_t* list;
    uint32_t* n_list;
    uint32_t cap;
    __device__ void put(int s) const {
        if (bitmap) {
            atomicOr(&bitmap[s >> 5], 1u << (s & 31));
        } else {
            uint32_t slot = atomicAdd(n_list, 1u);
            if (slot < cap) list[slot] = s;
        }
    }
    __device__ void put_c(uint64_t c) const {
        put(static_cast<int>(~static_cast<uint32_t>(c & 0xFFFFFFFFull)));
    }
};

// Radix-select the k_rem largest composites of `src` on the digits
// (shifts[p], widths[p]), p = 0..npass-1, most significant first, starting
// below an already fixed `prefix` (the bits above shifts[0]+widths[0]; pass
// prefix = 0 and top_bits = 64 when nothing is fixed), and keep them in
// `sink`.  Candidates whose fixed bits differ from `prefix` are ignored.
// Requires at least k_rem matching candidates and a unique composite per
// candidate (the position is part of it), so the last digit always resolves.
template <class Src>
__device__ void radix_select(const Src& src, uint32_t k_rem, const int* shifts, const int* widths, int npass,
                             uint64_t prefix, uint32_t* lh, uint32_t* wsum, const Sink& sink)
{
    int done_shift = shifts[0] + widths[0];
    for (int p = 0; p < npass; ++p) {
        const int sh = shifts[p], w = widths[p];
        const int nb = 1 << w;
        const int top = sh + w;
        for (int i = threadIdx.x; i < nb; i += blockDim.x) lh[i] = 0u;
        __syncthreads();
        for_each_candidate(src, [&](uint64_t c) {
            if (top >= 64 || (c >> top) == prefix) atomicAdd(&lh[(c >> sh) & (nb - 1)], 1u);
        });
        __syncthreads();
        int d; uint32_t gt;
        find_threshold_bin(lh, nb, k_rem, wsum, &d, &gt);
        k_rem -= gt;
        prefix = (top >= 64 ? 0ull : (prefix << w)) | static_cast<uint64_t>(d);
        done_shift = sh;
        bool done = lh[d] == k_rem;
        __syncthreads();
        if (done) break;
    }
    for_each_candidate(src, [&](uint64_t c) {
        if ((c >> done_shift) >= prefix) sink.put_c(c);
    });
    __syncthreads();
}

// Write the k kept positions of a row in ascending order from the sink's
// bitmap (nwords words) or its list (kpad entries, sorted here).
__device__ inline void write_ordered(const Sink& sink, int nwords, int kpad, int k, int32_t* out, uint32_t* wsum) {
    if (sink.bitmap) {
        // per-thread runs of words, block scan of their popcounts
        const uint32_t* bm = sink.bitmap;
        const int per = (nwords + blockDim.x - 1) / blockDim.x;
        const int w0 = threadIdx.x * per;
        const int w1 = min(w0 + per, nwords);
        uint32_t cnt = 0;
        for (int w = w0; w < w1; ++w) cnt += __popc(bm[w]);
        uint32_t total;
        uint32_t o = block_exclusive_scan(cnt, wsum, &total);
        for (int w = w0; w < w1; ++w) {
            uint32_t bits = bm[w];
            while (bits) {
                int b = __ffs(bits) - 1;
                bits &= bits - 1;
                if (o < static_cast<uint32_t>(k)) out[o] = (w << 5) + b;
                ++o;
            }
        }
        return;
    }
    // bitonic sort of the kpad list entries, ascending
    int32_t* sorted = sink.list;
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
    for (int j = threadIdx.x; j < k; j += blockDim.x) out[j] = sorted[j];
}

}  // namespace dsa
