// topk_sampled.hip -- top-k for long rows without materialising the scores.
//
// The selector keeps the k highest-scoring keys of each query
// ("DeepSeek-V3.2-Exp 稀疏注意力机制(DSA)技术深度解析", sheratonhq.com,
// section 1; "DeepSeek-V4 百万 token 上下文的工程实现", blog.hotdry.top, section
// "从 O(N²) 到 O(N・k)", which recommends k = 256..512 over 1M tokens).  When a
// row holds many more keys than k, writing every score to memory and reading
// it back costs more than finding the k largest, so:
//   sample  kSampleSplit workgroups per row score kSampleKeys keys -- runs
//           of 16 consecutive keys spread evenly over the row, so every load
//           is a contiguous 2 KiB block -- with the same MFMA code as the
//           indexer; then one workgroup per row takes a lower bound of the
//           r-th largest sample, r ~ 1.5 k * samples / visible keys + 24: the
//           indexer then keeps about 1.5 k + 24 * visible / samples keys;
//   index   the FP8 indexer appends only scores at or above that bound to the
//           row's candidate list (indexer.hip, candidate mode);
//   finish  one workgroup per row radix-selects the exact k largest of the
//           candidates on (order key, ~position) -- ties go to the lower
//           position -- and writes the positions in ascending order.
// If a row ends with fewer than k candidates or more than the list holds, the
// finish recomputes that row's scores in full, spread over several
// workgroups that each keep the top k of their slice, and the last of them
// selects the row's k from those, so the result never depends on how good
// the sample was.
#include "fp8_index.h"
#include "topk_common.h"

namespace dsa {

constexpr int kSampleThreads = 512;
constexpr int kSFinishThreads = 1024;
// Workgroups per row of the finish: one selects from the candidates; a row
// that falls back is recomputed by all of them, a slice of at least
// kFinishSliceKeys keys each, up to kFinishPartsMax workgroups.
constexpr int kFinishSliceKeys = 16384;
constexpr int kFinishPartsMax = 64;
static int finish_parts(int n_k) {
    const int p = (n_k + kFinishSliceKeys - 1) / kFinishSliceKeys;
    return p < 1 ? 1 : p > kFinishPartsMax ? kFinishPartsMax : p;
}

bool topk_sampled_eligible(int n_k, int k) {
    return static_cast<int64_t>(n_k) >= 16 * static_cast<int64_t>(k) && n_k >= kSampleKeys;
}



// The ranked keys of a row: [lo, lo + cnt) = the visible keys outside a
// backbone's forced first `sinks` and last `window` ones (all visible keys
// without a backbone).
struct Ranked { int lo, cnt; };
__device__ __forceinline__ Ranked ranked_keys(const IndexArgs& x, int pos) {
    const int hi = pos + 1 - x.window;
    return Ranked{x.sinks, hi > x.sinks ? hi - x.sinks : 0};
}

// The sample: kSampleKeys keys per row as runs of 16 consecutive keys spread
// evenly over the ranked keys (all of them when there are fewer); sample j is
// ranked key j when m == cnt, else run j/16 starts at (j/16) * gap.
__device__ __forceinline__ int sample_key(int j, int m, int cnt, int gap) {
    return m == cnt ? j : (j >> 4) * gap + (j & 15);
}

// Score the row's samples: grid (kSampleSplit, rows), each workgroup scores
// kSampleKeys / kSampleSplit of them and stores their order keys.
__global__ __launch_bounds__(256) void k_topk_sample_score(SampledTopk t) {
    const IndexArgs& x = t.ix;
    const int lrow = blockIdx.y, row = x.row0 + lrow;
    const int pos = row_pos(x.q_pos, row, x.n_q, x.n_k);
    const Ranked rk = ranked_keys(x, pos);
    const int vis = rk.cnt;                  // keys the sample spreads over, from rk.lo
    if (vis <= x.k) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, kg = lane >> 4;
    const int m = vis < kSampleKeys ? vis : kSampleKeys;
    const int gap = vis / ((m + 15) / 16);   // >= 16 unless m == vis
    const int per = kSampleKeys / kSampleSplit;                 // samples per workgroup
    const int j0 = blockIdx.x * per;
    if (j0 >= m) return;
    const int b = row / x.n_q;
    const uint8_t* kb = static_cast<const uint8_t*>(x.ik) + (static_cast<size_t>(b) * x.n_k + rk.lo) * 128;
    const float* ksb = x.ik_scale + static_cast<size_t>(b) * x.n_k + rk.lo;
    uint32_t* skey = t.samples + static_cast<size_t>(lrow) * kSampleKeys;
    static_assert(kSampleKeys / kSampleSplit == 4 * 64, "one group of 64 samples per wave");
    // block u of this wave holds samples j0 + 64*wave + 16u + (0..15); lane l
    // scores sample j0 + 64*wave + l.  All loads go out before any wait:
    // samples past m read sample m-1 and are not stored.
    v8i bv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = min(j0 + wave * 64 + u * 16 + col, m - 1);
        bv[u] = load_split32(kb + static_cast<size_t>(sample_key(j, m, vis, gap)) * 128, kg);
    }
    const int j = j0 + wave * 64 + lane;
    const float sk = ksb[sample_key(min(j, m - 1), m, vis, gap)];
    const Fp8Query q = load_fp8_query(static_cast<const uint8_t*>(x.iq), x.iq_scale, x.iw, row, x.H, lane);
    __builtin_amdgcn_sched_barrier(0);    // keep every load above the first wait
    const float score = fp8_score4(q, bv, sk);
    if (j < m) skey[j] = order_key(score);
}

// Lower bound of each row's r-th largest sample score; clears the row's
// candidate counters.
__global__ __launch_bounds__(kSampleThreads) void k_topk_sample_bound(SampledTopk t) {
    __shared__ uint32_t skey[kSampleKeys];
    __shared__ uint32_t lh[kTopkBins];
    __shared__ uint32_t wsum[kSampleThreads / 64 + 2];
    const IndexArgs& x = t.ix;
    const int lrow = blockIdx.x, row = x.row0 + lrow;
    const int pos = row_pos(x.q_pos, row, x.n_q, x.n_k);
    const int vis = ranked_keys(x, pos).cnt;   // keys ranked (and sampled)
    uint32_t* meta = x.meta + static_cast<size_t>(lrow) * kTopkMeta;
    if (threadIdx.x == 0) { meta[S_NCAND] = 0u; meta[S_OVF] = 0u; meta[S_FALLBACK] = 0u; meta[S_DONE] = 0u; meta[S_NWIN] = 0u; }
    if (vis <= x.k) {                      // every ranked key is kept: nothing to bound
        if (threadIdx.x == 0) meta[S_KLOW] = 0xFFFFFFFFu;
        return;
    }
    const int m = vis < kSampleKeys ? vis : kSampleKeys;
    const uint32_t* src = t.samples + static_cast<size_t>(lrow) * kSampleKeys;
    // the whole sample buffer is read at once (entries past m are ignored)
    static_assert(kSampleKeys % kSampleThreads == 0, "sample buffer splits evenly");
    constexpr int kPer = kSampleKeys / kSampleThreads;
    uint32_t v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) v[u] = src[threadIdx.x + u * kSampleThreads];
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int j = threadIdx.x + u * kSampleThreads;
        if (j < m) { skey[j] = v[u]; kmin = min(kmin, v[u]); kmax = max(kmax, v[u]); }
    }
    kmin = wave_allreduce(kmin, [](uint32_t p, uint32_t q) { return p < q ? p : q; });
    kmax = wave_allreduce(kmax, [](uint32_t p, uint32_t q) { return p > q ? p : q; });
    __shared__ uint32_t wmin[kSampleThreads / 64], wmax[kSampleThreads / 64];
    if ((threadIdx.x & 63) == 0) { wmin[threadIdx.x >> 6] = kmin; wmax[threadIdx.x >> 6] = kmax; }
    __syncthreads();
    for (int w = 0; w < kSampleThreads / 64; ++w) { kmin = min(kmin, wmin[w]); kmax = max(kmax, wmax[w]); }
    const int64_t want = (3 * static_cast<int64_t>(m) * x.k + 2 * static_cast<int64_t>(vis) - 1) /
                         (2 * static_cast<int64_t>(vis)) + 24;
    // the floor of the r-th largest sample at two 11-bit digits of resolution
    // (every visible key a candidate when r reaches the sample size)
    const uint32_t k_low = want < m ? lower_bound_rth(skey, m, static_cast<uint32_t>(want), kmin, kmax, lh, wsum)
                                    : 0u;
    if (threadIdx.x == 0) meta[S_KLOW] = k_low;
}

// Exact top-k over the candidate list (or the recomputed row), then the
// positions in ascending order.  Grid (rows, parts): workgroup (r, 0)
// selects row r from its candidates; the others return at once unless the
// row falls back, and then all `parts` workgroups of the row recompute one
// slice of its scores each, and the last of them to finish selects from the
// whole row.
__global__ __launch_bounds__(kSFinishThreads) void k_topk_finish_sampled(SampledTopk t) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ __align__(16) uint32_t lh[kTopkBins];
    __shared__ uint32_t wsum[kSFinishThreads / 64 + 2];
    __shared__ uint32_t n_list, n_tie;
    __shared__ uint32_t last, win_base;
    const IndexArgs& x = t.ix;
    const int lrow = blockIdx.x, row = x.row0 + lrow;
    const int part = blockIdx.y, nparts = gridDim.y;
    const int pos = row_pos(x.q_pos, row, x.n_q, x.n_k);
    const int vis = pos + 1;
    const Ranked rk = ranked_keys(x, pos);
    const int k = x.k;
    int32_t* out = t.idx + static_cast<size_t>(lrow) * k;
    if (rk.cnt <= k) {                     // every ranked key is kept
        if (part == 0)
            for (int j = threadIdx.x; j < k; j += blockDim.x) out[j] = j < rk.cnt ? rk.lo + j : -1;
        return;
    }
    uint64_t* cl = reinterpret_cast<uint64_t*>(smem);                       // [cand_cap]
    uint32_t* tail = reinterpret_cast<uint32_t*>(cl + x.cand_cap);          // bitmap or list
    const bool use_bitmap = x.n_k <= kBitmapMaxKeys;
    const int nwords = (vis + 31) >> 5;
    int kpad = 1;
    while (kpad < k) kpad <<= 1;
    Sink sink{use_bitmap ? tail : nullptr, reinterpret_cast<int32_t*>(tail), &n_list, static_cast<uint32_t>(k)};
    // the sink starts empty (ordered before its first use by the select's
    // first barrier)
    auto clear_sink = [&]() {
        if (use_bitmap) {
            for (int i = threadIdx.x; i < nwords; i += blockDim.x) tail[i] = 0u;
        } else {
            for (int i = threadIdx.x; i < kpad; i += blockDim.x) tail[i] = 0x7FFFFFFFu;
        }
        if (threadIdx.x == 0) n_list = 0;
    };
    uint32_t* meta = x.meta + static_cast<size_t>(lrow) * kTopkMeta;
    // the first kSpecLoads*blockDim.x list entries are fetched together with the
    // counters, before the list's length is known (entries past it are ignored;
    // they lie inside the row's list, whose capacity is larger)
    constexpr int kSpecLoads = 8;
    static_assert(kSpecLoads * kSFinishThreads <= kSampledCandCap, "speculative reads stay inside the list");
    const uint64_t* cg = x.cand + static_cast<size_t>(lrow) * x.cand_cap;
    uint64_t spec[kSpecLoads];
    if (part == 0) {
#pragma unroll
        for (int u = 0; u < kSpecLoads; ++u) spec[u] = cg[threadIdx.x + u * kSFinishThreads];
    }
    const uint32_t n = meta[S_NCAND];
    const uint32_t k_low = meta[S_KLOW];
    const bool ok = meta[S_OVF] == 0u && n >= static_cast<uint32_t>(k) && n <= static_cast<uint32_t>(x.cand_cap);
    if (ok) {
        if (part != 0) return;
        clear_sink();
        uint32_t kmax = 0u;
#pragma unroll
        for (int u = 0; u < kSpecLoads; ++u) {
            const uint32_t i = threadIdx.x + u * kSFinishThreads;
            if (i < n) { cl[i] = spec[u]; kmax = max(kmax, static_cast<uint32_t>(spec[u] >> 32)); }
        }
        for (uint32_t i = threadIdx.x + kSpecLoads * kSFinishThreads; i < n; i += kSFinishThreads) {
            const uint64_t c = cg[i];
            cl[i] = c;
            kmax = max(kmax, static_cast<uint32_t>(c >> 32));
        }
        kmax = wave_allreduce(kmax, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
        if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = kmax;
        __syncthreads();
        for (int w = 0; w < kSFinishThreads / 64; ++w) kmax = max(kmax, wsum[w]);
        __syncthreads();                       // wsum is reused by the select
        // digits of the relative composite ((key - k_low) << 32 | ~position):
        // the first covers the top 11 bits of the candidates' key range, the
        // rest the remaining bits 11 at a time
        const uint32_t range = kmax - k_low;
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
        select_candidates(cl, n, k_low, static_cast<uint32_t>(k), shifts, widths, np, lh, wsum, &n_tie, sink);
    } else {
        // recompute this row's scores in full, slice `part` of nparts here:
        // each wave scores 128 keys per step with whole-line loads
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
        const int b = row / x.n_q;
        const Fp8Query q = load_fp8_query(static_cast<const uint8_t*>(x.iq), x.iq_scale, x.iw, row, x.H, lane);
        const uint8_t* kb = static_cast<const uint8_t*>(x.ik) + static_cast<size_t>(b) * x.n_k * 128;
        const float* ksb = x.ik_scale + static_cast<size_t>(b) * x.n_k;
        float* sc = t.scratch + static_cast<size_t>(lrow) * x.n_k;
        const int slice = (((vis + nparts - 1) / nparts) + 127) & ~127;
        const int s0 = part * slice, s1 = min(vis, s0 + slice);
        for (int base = s0 + wave * 128; base < s1; base += nwaves * 128) {   // uniform per wave
            v4i lines[16];
            float sk[2];
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                load_keys64_lines(kb, base + 64 * g, vis - 1, lane, lines + 8 * g);
                sk[g] = ksb[min(base + 64 * g + lane, vis - 1)];
            }
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                v8i bv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) bv[u] = keys_block_operand(lines + 8 * g, u, lane);
                const float score = fp8_score4(q, bv, sk[g]);
                const int s = base + 64 * g + lane;
                if (s < s1) sc[s] = score;
            }
        }
        __threadfence_block();
        __syncthreads();
        // this slice's top k (all of its ranked keys when it has no more) go
        // to the row's winner list; the top k of the row are among them
        const int r0 = max(s0, rk.lo), r1 = min(s1, rk.lo + rk.cnt);
        const int cnt = r1 > r0 ? r1 - r0 : 0;
        const uint32_t take = static_cast<uint32_t>(min(cnt, k));
        uint64_t* win = t.win + static_cast<size_t>(lrow) * t.win_cap;
        if (threadIdx.x == 0) {
            n_list = 0;
            win_base = take ? atomicAdd(&meta[S_NWIN], take) : 0u;
        }
        __syncthreads();
        if (cnt > k) {
            ScoreRow64 src{sc, r1, rk.lo, rk.lo + rk.cnt, r0};
            ListSink64 ls{win + win_base, &n_list, take};
            radix_select_spread(src, static_cast<uint32_t>(k), lh, wsum, ls);
        } else {
            for (int s = r0 + threadIdx.x; s < r1; s += blockDim.x)
                win[win_base + static_cast<uint32_t>(s - r0)] = composite64(order_key(sc[s]), s);
        }
        // publish the winners: every wave waits until its stores have reached
        // the L2, then one thread releases them at device scope (a device
        // fence writes back the whole L2, so one per workgroup, not one per
        // wave) and counts the workgroup in; the last of the row's
        // workgroups to arrive acquires and merges
        __builtin_amdgcn_s_waitcnt(kWaitVmem);
        __syncthreads();
        if (threadIdx.x == 0) {
            if (part == 0) meta[S_FALLBACK] = 1u;
            __threadfence();
            last = atomicAdd(&meta[S_DONE], 1u) == static_cast<uint32_t>(nparts - 1) ? 1u : 0u;
        }
        __syncthreads();
        if (!last) return;
        __threadfence();
        const uint32_t nw = __hip_atomic_load(&meta[S_NWIN], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        clear_sink();
        Cand64Rel src{win, static_cast<int>(nw), 0ull};
        radix_select_spread(src, static_cast<uint32_t>(k), lh, wsum, sink);
    }
    __syncthreads();
    write_ordered(sink, nwords, kpad, k, out, wsum);
}

static size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

size_t topk_sampled_workspace_bytes(int rows, int n_k, int k) {
    const size_t r = static_cast<size_t>(rows);
    return align256(r * kTopkMeta * sizeof(uint32_t)) +
           align256(r * kSampledCandCap * sizeof(uint64_t)) +
           align256(r * kSampleKeys * sizeof(uint32_t)) +
           align256(r * static_cast<size_t>(n_k) * sizeof(float)) +
           align256(r * static_cast<size_t>(finish_parts(n_k)) * k * sizeof(uint64_t));
}

void topk_sampled_carve(void* ws, int rows, int n_k, int k, SampledTopk& t) {
    unsigned char* p = static_cast<unsigned char*>(ws);
    const size_t r = static_cast<size_t>(rows);
    t.ix.meta = reinterpret_cast<uint32_t*>(p);
    p += align256(r * kTopkMeta * sizeof(uint32_t));
    t.ix.cand = reinterpret_cast<uint64_t*>(p);
    t.ix.cand_cap = kSampledCandCap;
    p += align256(r * kSampledCandCap * sizeof(uint64_t));
    t.samples = reinterpret_cast<uint32_t*>(p);
    p += align256(r * kSampleKeys * sizeof(uint32_t));
    t.scratch = reinterpret_cast<float*>(p);
    p += align256(r * static_cast<size_t>(n_k) * sizeof(float));
    t.win = reinterpret_cast<uint64_t*>(p);
    t.win_cap = finish_parts(n_k) * k;
}

hipError_t launch_topk_sample(const SampledTopk& t, hipStream_t st) {
    hipLaunchKernelGGL(k_topk_sample_score, dim3(kSampleSplit, t.ix.rows), dim3(256), 0, st, t);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_topk_sample_bound, dim3(t.ix.rows), dim3(kSampleThreads), 0, st, t);
    return hipGetLastError();
}

hipError_t launch_topk_finish_sampled(const SampledTopk& t, hipStream_t st) {
    int kpad = 1;
    while (kpad < t.ix.k) kpad <<= 1;
    const size_t tail = t.ix.n_k <= kBitmapMaxKeys ? static_cast<size_t>((t.ix.n_k + 31) >> 5) * 4
                                                   : static_cast<size_t>(kpad) * 4;
    const size_t smem = static_cast<size_t>(t.ix.cand_cap) * sizeof(uint64_t) + tail;
    {
        hipError_t e = allow_dyn_lds(reinterpret_cast<const void*>(k_topk_finish_sampled), smem);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_topk_finish_sampled, dim3(t.ix.rows, finish_parts(t.ix.n_k)), dim3(kSFinishThreads), smem, st, t);
    return hipGetLastError();
}

}  // namespace dsa
