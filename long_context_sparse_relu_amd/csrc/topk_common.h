// topk_common.h -- block-level building blocks of the radix top-k selectors
// (threshold-bin search, block scan, batched candidate visits, the sink that
// collects kept positions, a generic radix select and the ordered write-out).
#pragma once

#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int kBitmapMaxKeys = 1 << 18;   // rows up to this long are ordered through a bitmap
// s_waitcnt immediate that waits for every outstanding vector memory access
// of the wave (vmcnt = 0, the other counters unconstrained).
constexpr int kWaitVmem = 0x0F70;

// Workgroup barrier for LDS data: the wave's LDS accesses complete
// (lgkmcnt = 0), then s_barrier.  Unlike __syncthreads it does not wait for
// the wave's global loads, which may stay in flight across it (including
// loads straight into LDS, whose target the caller must not touch until it
// has waited for them).  Global stores made before it are not ordered for
// other waves.  The helpers below use it: they share only LDS data.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// x combined over the whole wave on the VALU: lanes l and l^1, then l^2
// (quad permutations), then the two halves of each 8-lane group and of each
// 16-lane row (mirrors), all by DPP, then rows 2r and 2r+1 and the two halves
// of the wave by v_permlane16/32_swap.  Each step pairs every lane with one
// lane of the other group, so any commutative and associative op works (sum,
// min, max, or); every lane gets the result.
template <class Op>
__device__ __forceinline__ uint32_t wave_allreduce(uint32_t x, Op op) {
    x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0xB1, 0xF, 0xF, false)));
    x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x4E, 0xF, 0xF, false)));
    x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x141, 0xF, 0xF, false)));
    x = op(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x140, 0xF, 0xF, false)));
    const auto r16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = op(r16[0], r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return op(r32[0], r32[1]);
}
__device__ __forceinline__ float wave_allmin(float x) {
    return __uint_as_float(wave_allreduce(__float_as_uint(x), [](uint32_t a, uint32_t b) {
        return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b)));
    }));
}
__device__ __forceinline__ float wave_allmax(float x) {
    return __uint_as_float(wave_allreduce(__float_as_uint(x), [](uint32_t a, uint32_t b) {
        return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
    }));
}

// Inclusive prefix sum over the wave's lanes on the VALU: lanes l - 1, l - 2,
// l - 4, l - 8 of the same 16-lane row by DPP row shifts (a lane shifted in
// from outside the row adds 0), which scans each row; then the last lane of
// row 0 (of row 2) is broadcast into row 1 (row 3) and the last lane of row 1
// into rows 2 and 3 (DPP row broadcasts, the other rows left unchanged).
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x111, 0xF, 0xF, false));
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x112, 0xF, 0xF, false));
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x114, 0xF, 0xF, false));
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x118, 0xF, 0xF, false));
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x142, 0xA, 0xF, false));
    x += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x143, 0xC, 0xF, false));
    return x;
}

// LDS atomics issued as plain instructions, for kernels that keep loads into
// LDS in flight: the compiler cannot tell an atomic's target from the loads'
// and would otherwise wait for all of them before it.  The caller's next
// lds_barrier completes them; lds_add_rtn waits for its own result.
__device__ __forceinline__ uint32_t lds_addr(const uint32_t* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint32_t*)p));
}
__device__ __forceinline__ void lds_add(uint32_t* p, uint32_t v) {
    asm volatile("ds_add_u32 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_or(uint32_t* p, uint32_t v) {
    asm volatile("ds_or_b32 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}
__device__ __forceinline__ uint32_t lds_add_rtn(uint32_t* p, uint32_t v) {
    uint32_t old;
    asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=v"(old) : "v"(lds_addr(p)), "v"(v) : "memory");
    return old;
}

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
    const uint32_t x = wave_inclusive_sum(local);   // inclusive scan inside the wave
    if (lane == 63) wsum[wave] = x;
    lds_barrier();
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
    lds_barrier();
    *digit = static_cast<int>(wsum[nwaves]);
    *gt = wsum[nwaves + 1];
    lds_barrier();
}

// The same search by one wave, for two ranks at once: for r = r1 and r = r2
// the bin d with count(bins > d) < r <= count(bins >= d), written to LDS as
// res = {d1, count above d1, d2, count above d2}.  Lane l holds the NB / 64
// bins from NB - 1 - (NB / 64) l downwards (the top bins in lane 0).  Call
// from one wave; the caller's barrier publishes res.  Requires
// 1 <= r <= sum(hist) for both ranks.
template <int NB>
__device__ __forceinline__ void wave_find_bins(const uint32_t* hist, uint32_t r1, uint32_t r2, int* res) {
    constexpr int PER = NB / 64;
    const int lane = threadIdx.x & 63;
    const int top = NB - 1 - lane * PER;
    uint32_t local = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) local += hist[top - j];
    const uint32_t x = wave_inclusive_sum(local);   // inclusive scan from the top lane
    const uint32_t excl = x - local;
    // the lane holding rank r; then its PER bins, one per lane, scanned again
    auto find = [&](uint32_t r, int slot) {
        const uint64_t hit = __ballot(excl < r && x >= r);
        const int src = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        const uint32_t base = static_cast<uint32_t>(__shfl(static_cast<int>(excl), src));
        const int btop = NB - 1 - src * PER;
        const uint32_t h = lane < PER ? hist[btop - lane] : 0u;
        const uint32_t y = wave_inclusive_sum(h);
        const uint32_t before = base + y - h;
        if (lane < PER && before < r && before + h >= r) {
            res[slot] = btop - lane;
            res[slot + 1] = static_cast<int>(before);
        }
    };
    find(r1, 0);
    find(r2, 2);
}

// The same search for one rank r, by every wave that calls it, with the
// result in registers (no LDS write and no barrier): the bin d with
// count(bins > d) < r <= count(bins >= d) and that count above it.  Lane l
// holds the NB / 64 bins from NB - 1 - (NB / 64) l downwards; the lane whose
// range holds rank r walks its own bins.  Requires 1 <= r <= sum(hist).
template <int NB>
__device__ __forceinline__ void wave_find_bin_reg(const uint32_t* hist, uint32_t r, int* d, uint32_t* gt) {
    constexpr int PER = NB / 64;
    const int lane = threadIdx.x & 63;
    const int top = NB - 1 - lane * PER;
    uint32_t h[PER], local = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) { h[j] = hist[top - j]; local += h[j]; }
    const uint32_t x = wave_inclusive_sum(local);
    const uint32_t excl = x - local;
    int dl = top;
    uint32_t gl = excl, run = excl;
    bool found = false;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (!found && run + h[j] >= r) { dl = top - j; gl = run; found = true; }
        run += h[j];
    }
    const uint64_t hit = __ballot(excl < r && x >= r);
    const int src = __ffsll(static_cast<unsigned long long>(hit)) - 1;
    *d = __builtin_amdgcn_readlane(dl, src);
    *gt = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(gl), src));
}

// Block-wide exclusive scan of one value per thread (wave scans, then the
// wave totals); `wsum` holds one LDS slot per wave.  Returns the exclusive
// prefix; *total gets the block sum.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    const uint32_t x = wave_inclusive_sum(v);
    if (lane == 63) wsum[wave] = x;
    lds_barrier();
    uint32_t before = 0, all = 0;
    for (int w = 0; w < nwaves; ++w) {
        uint32_t t = wsum[w];
        if (w < wave) before += t;
        all += t;
    }
    lds_barrier();
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

// Candidates relative to the row's bound: every candidate has key >= k_low,
// so subtracting (k_low << 32) keeps the order and leaves small keys whose
// top digit spreads the candidates over the histogram instead of piling them
// into the one or two bins just above the bound.
struct Cand64Rel {
    const uint64_t* c; int n; uint64_t base;
    __device__ int size() const { return n; }
    __device__ bool get(int i, uint64_t* out) const { *out = c[i] - base; return true; }
};
// A score row in memory as 64-bit composites (order key << 32 | ~position),
// visited over positions [first, n).
struct ScoreRow64 {
    const float* sc; int n;
    int lo, hi;                 // keys outside [lo, hi) rank as -inf (a backbone's forced keys)
    int first = 0;
    __device__ int size() const { return n; }
    __device__ bool get(int i, uint64_t* out) const {
        const float x = sc[i];
        *out = composite64(order_key(i < lo || i >= hi ? -__builtin_inff() : x), i);
        return true;
    }
};
// Score rows are visited four scores per load over their 16-byte aligned
// part (eight loads in flight per thread), the ends one by one.
template <class F>
__device__ __forceinline__ void for_each_candidate(const ScoreRow64& src, F&& f) {
    const int n = src.n, T = blockDim.x;
    auto one = [&](int i) {
        uint64_t c;
        src.get(i, &c);
        f(c);
    };
    if ((reinterpret_cast<uintptr_t>(src.sc) & 15) != 0) {
        for (int i = src.first + threadIdx.x; i < n; i += T) one(i);
        return;
    }
    const int g0 = (src.first + 3) >> 2, g1 = n >> 2;      // whole float4 groups
    if (g0 >= g1) {
        for (int i = src.first + threadIdx.x; i < n; i += T) one(i);
        return;
    }
    for (int i = src.first + threadIdx.x; i < 4 * g0; i += T) one(i);
    const float4* v = reinterpret_cast<const float4*>(src.sc);
    auto visit = [&](const float4& x, int i4) {
        const float e[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int s = 4 * i4 + c;
            f(composite64(order_key(s < src.lo || s >= src.hi ? -__builtin_inff() : e[c]), s));
        }
    };
    int i = g0 + threadIdx.x;
    for (; i + 7 * T < g1; i += 8 * T) {
        float4 x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = v[i + u * T];
#pragma unroll
        for (int u = 0; u < 8; ++u) visit(x[u], i + u * T);
    }
    for (; i < g1; i += T) visit(v[i], i);
    for (int j = 4 * g1 + threadIdx.x; j < n; j += T) one(j);
}

// One count per hit lane into the LDS histogram `lh`; when every hit lane of
// the wave falls in the same bin (rows of tied scores put all of them there)
// the first hit lane adds the wave's count in one atomic instead of up to 64
// serialised ones on one address.
__device__ __forceinline__ void lds_count(uint32_t* lh, bool hit, uint32_t bin) {
    const uint32_t lb = __builtin_amdgcn_readfirstlane(bin);
    const uint64_t hits = __ballot(hit);
    const uint64_t same = __ballot(hit && bin == lb);
    if (same == hits) {
        if (hit && (threadIdx.x & 63) == __ffsll(static_cast<unsigned long long>(hits)) - 1)
            atomicAdd(&lh[lb], static_cast<uint32_t>(__popcll(hits)));
    } else if (hit) {
        atomicAdd(&lh[bin], 1u);
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
    __device__ void put_if(bool take, uint64_t c) const {
        if (take) put_c(c);
    }
};
// A sink that appends the kept composites themselves to a list in global
// memory at out[0..cap): one LDS counter, bumped once per wave.
struct ListSink64 {
    uint64_t* out;
    uint32_t* n;       // LDS, starts at 0
    uint32_t cap;
    __device__ void put_if(bool take, uint64_t c) const {
        const uint64_t m = __ballot(take);
        if (!m) return;
        const int lane = threadIdx.x & 63;
        const int leader = __ffsll(static_cast<unsigned long long>(m)) - 1;
        uint32_t base = 0;
        if (lane == leader) base = atomicAdd(n, static_cast<uint32_t>(__popcll(m)));
        base = __shfl(base, leader);
        const uint32_t slot = base + static_cast<uint32_t>(__popcll(m & ((1ull << lane) - 1ull)));
        if (take && slot < cap) out[slot] = c;
    }
};

// Radix-select the k_rem largest composites of `src` on the digits
// (shifts[p], widths[p]), p = 0..npass-1, most significant first, starting
// below an already fixed `prefix` (the bits above shifts[0]+widths[0]; pass
// prefix = 0 and top_bits = 64 when nothing is fixed), and keep them in
// `sink`.  Candidates whose fixed bits differ from `prefix` are ignored.
// Requires at least k_rem matching candidates and a unique composite per
// candidate (the position is part of it), so the last digit always resolves.
// With AGG the histogram adds are aggregated per wave (lds_count): worth its
// extra instructions only where whole waves tend to hit one bin (whole rows
// of tied scores).
template <bool AGG = false, class Src, class SinkT>
__device__ void radix_select(const Src& src, uint32_t k_rem, const int* shifts, const int* widths, int npass,
                             uint64_t prefix, uint32_t* lh, uint32_t* wsum, const SinkT& sink)
{
    int done_shift = shifts[0] + widths[0];
    for (int p = 0; p < npass; ++p) {
        const int sh = shifts[p], w = widths[p];
        const int nb = 1 << w;
        const int top = sh + w;
        for (int i = threadIdx.x; i < nb; i += blockDim.x) lh[i] = 0u;
        lds_barrier();
        for_each_candidate(src, [&](uint64_t c) {
            const bool hit = top >= 64 || (c >> top) == prefix;
            const uint32_t bin = static_cast<uint32_t>((c >> sh) & (nb - 1));
            if constexpr (AGG) lds_count(lh, hit, bin);
            else if (hit) atomicAdd(&lh[bin], 1u);
        });
        lds_barrier();
        int d; uint32_t gt;
        find_threshold_bin(lh, nb, k_rem, wsum, &d, &gt);
        k_rem -= gt;
        prefix = (top >= 64 ? 0ull : (prefix << w)) | static_cast<uint64_t>(d);
        done_shift = sh;
        bool done = lh[d] == k_rem;
        lds_barrier();
        if (done) break;
    }
    for_each_candidate(src, [&](uint64_t c) { sink.put_if((c >> done_shift) >= prefix, c); });
    lds_barrier();
}

// radix_select over full 64-bit composites whose digits start below the
// highest bit in which the candidates differ: one pass finds their minimum
// and maximum, the bits above their first difference are fixed, and 11-bit
// digits cover the rest.  Rows of tied scores then take only the passes over
// the position bits.  `lh` (kTopkBins entries) and `wsum` as radix_select.
template <class Src, class SinkT>
__device__ void radix_select_spread(const Src& src, uint32_t k, uint32_t* lh, uint32_t* wsum, const SinkT& sink) {
    uint64_t lo = ~0ull, hi = 0ull;
    for_each_candidate(src, [&](uint64_t c) { lo = c < lo ? c : lo; hi = c > hi ? c : hi; });
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint64_t l2 = __shfl_xor(lo, o), h2 = __shfl_xor(hi, o);
        lo = l2 < lo ? l2 : lo;
        hi = h2 > hi ? h2 : hi;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    uint64_t* red = reinterpret_cast<uint64_t*>(lh);        // lh is free until the select
    if (lane == 0) { red[2 * wave] = lo; red[2 * wave + 1] = hi; }
    lds_barrier();
    for (int w = 0; w < nwaves; ++w) {
        const uint64_t l2 = red[2 * w], h2 = red[2 * w + 1];
        lo = l2 < lo ? l2 : lo;
        hi = h2 > hi ? h2 : hi;
    }
    lds_barrier();
    const uint64_t diff = lo ^ hi;
    const int bits = diff ? 64 - __clzll(static_cast<long long>(diff)) : 1;   // the bits that vary
    int shifts[6], widths[6], np = 0;
    for (int below = bits; below > 0 && np < 6; ++np) {
        const int w = below < 11 ? below : 11;
        below -= w;
        shifts[np] = below;
        widths[np] = w;
    }
    radix_select<true>(src, k, shifts, widths, np, bits >= 64 ? 0ull : hi >> bits, lh, wsum, sink);
}

// The k largest of the n candidate composites cl[0..n) (order key << 32 |
// ~position, every key at least k_low; LDS) into the sink, with the radix
// digits of ((key - k_low) << 32 | ~position) in shifts / widths (np of them).
// The first digit's histogram finds the threshold bin.  A bin of at most
// kTopkBins / 2 candidates (a few, when the candidates spread over the key
// range) is then ranked by direct comparison, the composites being distinct;
// a larger one takes the radix passes from the start.  `lh` (kTopkBins
// entries, 8-byte aligned), `wsum` and the LDS counter `n_tie` are scratch.
template <class SinkT>
__device__ void select_candidates(const uint64_t* cl, uint32_t n, uint32_t k_low, uint32_t k, const int* shifts,
                                  const int* widths, int np, uint32_t* lh, uint32_t* wsum, uint32_t* n_tie,
                                  const SinkT& sink) {
    const uint64_t base = static_cast<uint64_t>(k_low) << 32;
    const int sh0 = shifts[0];
    for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x) lh[i] = 0u;
    if (threadIdx.x == 0) *n_tie = 0u;
    lds_barrier();
    for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) atomicAdd(&lh[static_cast<uint32_t>((cl[i] - base) >> sh0)], 1u);
    lds_barrier();
    int d0;
    uint32_t gt0;
    find_threshold_bin(lh, kTopkBins, k, wsum, &d0, &gt0);
    const uint32_t n_t = lh[d0], k_t = k - gt0;
    lds_barrier();                               // every thread has read lh[d0]
    if (n_t <= static_cast<uint32_t>(kTopkBins / 2)) {
        uint64_t* tie = reinterpret_cast<uint64_t*>(lh);      // lh is free now
        for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
            const uint64_t c = cl[i] - base;
            const int dg = static_cast<int>(c >> sh0);
            if (dg > d0) sink.put_c(c);
            else if (dg == d0) tie[atomicAdd(n_tie, 1u)] = c;
        }
        lds_barrier();
        for (uint32_t j = threadIdx.x; j < n_t; j += blockDim.x) {
            const uint64_t c = tie[j];
            uint32_t beat = 0;
            for (uint32_t q = 0; q < n_t; ++q) beat += tie[q] > c ? 1u : 0u;
            if (beat < k_t) sink.put_c(c);
        }
        lds_barrier();
    } else {
        Cand64Rel src{cl, static_cast<int>(n), base};
        radix_select(src, k, shifts, widths, np, 0ull, lh, wsum, sink);
    }
}

// A lower bound on the r-th largest of the m order keys skey[0..m) (LDS),
// at two 11-bit digits of resolution: digit 0 spans the top 11 bits of the
// keys' range [kmin, kmax], digit 1 the next 11 below it; the result is kmin
// plus the r-th largest key's two digits (lower bits cleared), so at least r
// keys are >= it.  Whole block; requires 1 <= r <= m; `lh` has kTopkBins
// entries, `wsum` one slot per wave plus two.
__device__ inline uint32_t lower_bound_rth(const uint32_t* skey, int m, uint32_t r, uint32_t kmin, uint32_t kmax,
                                           uint32_t* lh, uint32_t* wsum) {
    const uint32_t range = kmax - kmin;
    const int bits = range ? 32 - __clz(static_cast<int>(range)) : 0;
    const int sh1 = bits > 11 ? bits - 11 : 0;
    for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x) lh[i] = 0u;
    lds_barrier();
    for (int j = threadIdx.x; j < m; j += blockDim.x) atomicAdd(&lh[(skey[j] - kmin) >> sh1], 1u);
    lds_barrier();
    int d0; uint32_t gt0;
    find_threshold_bin(lh, kTopkBins, r, wsum, &d0, &gt0);
    uint32_t k_low = kmin + (static_cast<uint32_t>(d0) << sh1);
    if (sh1 > 0) {
        const int sh2 = sh1 > 11 ? sh1 - 11 : 0;
        const uint32_t mask2 = (1u << (sh1 - sh2)) - 1u;
        for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x) lh[i] = 0u;
        lds_barrier();
        for (int j = threadIdx.x; j < m; j += blockDim.x) {
            const uint32_t rel = skey[j] - kmin;
            if (static_cast<int>(rel >> sh1) == d0) atomicAdd(&lh[(rel >> sh2) & mask2], 1u);
        }
        lds_barrier();
        int d1; uint32_t gt1;
        find_threshold_bin(lh, kTopkBins, r - gt0, wsum, &d1, &gt1);
        k_low += static_cast<uint32_t>(d1) << sh2;
    }
    return k_low;
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
            lds_barrier();
        }
    }
    for (int j = threadIdx.x; j < k; j += blockDim.x) out[j] = sorted[j];
}

}  // namespace dsa
