// Importance compression of a sequence's cached tokens.
//
// "DeepSeek-V4 百万 token 上下文的工程实现" (blog.hotdry.top), section
// "滑动窗口 KV Cache 与混合策略": the most recent tokens keep their full K/V
// while older ones are compressed by an importance score and only the
// important ones survive (an 8K window plus that compression is said to cut
// the cache by 45-55 % at 1M tokens).  Read here as: per sequence the last
// `window` tokens are kept, and of the tokens before them the `keep` ones of
// highest importance (lower position first among equal importance, -0.0 equal
// to +0.0); the kept tokens' rows are written out in position order together
// with their original positions.
//
// Work per sequence, all on the device and HBM-bound:
//   1. a three-pass radix select over the old tokens' order keys finds the
//      keep-th largest key T and how many keys equal to T are kept (k_cmp_hist
//      over many workgroups, k_cmp_pick for the bin);
//   2. k_cmp_count counts, per 1024-token chunk, the keys above T, equal to T
//      and in the window; k_cmp_scan turns that into each chunk's first output
//      slot and the number of T-keys before it;
//   3. k_cmp_write ranks the chunk's kept tokens and copies their rows with
//      16-byte (or 4-byte) vector loads and stores.
#include <type_traits>

#include "dsa_kernels.h"

namespace dsa {
namespace {

constexpr int kCmpBins = 2048;          // 11-bit digits: passes over bits 31..21, 20..10, 9..0
constexpr int kCmpHistKeys = 16384;     // old tokens per histogram workgroup
// Tokens per count / write workgroup.  Chunks of the recent window keep every
// token and the others about half; 1024-token chunks give several workgroups
// per CU slot over a launch, so the heavier ones are spread as slots free up.
constexpr int kCmpChunk = 1024;
constexpr int kCmpThreads = 256;
constexpr int kCmpPer = kCmpChunk / kCmpThreads;   // tokens per thread
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;                         // -0.0 orders as +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // larger float -> larger key
}

__device__ __forceinline__ int digit_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t digit_mask(int pass) { return pass == 2 ? 0x3FFu : 0x7FFu; }
// bits already fixed before `pass`
__device__ __forceinline__ uint32_t fixed_mask(int pass) {
    return pass == 0 ? 0u : (pass == 1 ? 0xFFE00000u : 0xFFFFFC00u);
}

struct SeqWs {                          // per-sequence workspace view
    uint32_t* hist;                     // [3][kCmpBins]
    uint32_t* state;                    // [0] prefix of T, [1] keys equal to T still to keep
    uint32_t* fixed;                    // [nch] kept tokens of the chunk besides T-keys, then its first slot
    uint32_t* eq;                       // [nch] T-keys of the chunk, then T-keys before it
};

__device__ __forceinline__ SeqWs seq_ws(uint32_t* ws, int b, int nch) {
    uint32_t* base = ws + static_cast<size_t>(b) * (3 * kCmpBins + 4 + 2 * static_cast<size_t>(nch));
    return SeqWs{base, base + 3 * kCmpBins, base + 3 * kCmpBins + 4, base + 3 * kCmpBins + 4 + nch};
}

__global__ __launch_bounds__(kCmpThreads) void k_cmp_clear(CompressArgs a) {
    const SeqWs w = seq_ws(a.ws, blockIdx.x, a.nch);
    for (int i = threadIdx.x; i < 3 * kCmpBins; i += kCmpThreads) w.hist[i] = 0u;
    if (threadIdx.x == 0) {
        w.state[0] = 0u;
        w.state[1] = static_cast<uint32_t>(a.keep);
    }
}

// Histogram of the next digit over the old tokens whose fixed bits match T's.
__global__ __launch_bounds__(kCmpThreads) void k_cmp_hist(CompressArgs a, int pass) {
    __shared__ uint32_t h[kCmpBins];
    const int b = blockIdx.y;
    const SeqWs w = seq_ws(a.ws, b, a.nch);
    for (int i = threadIdx.x; i < kCmpBins; i += kCmpThreads) h[i] = 0u;
    __syncthreads();
    const uint32_t prefix = w.state[0], fm = fixed_mask(pass), dm = digit_mask(pass);
    const int sh = digit_shift(pass);
    const int n_old = a.n_k - a.window;
    const float* imp = a.imp + static_cast<size_t>(b) * a.n_k;
    const int s0 = blockIdx.x * kCmpHistKeys, s1 = min(n_old, s0 + kCmpHistKeys);
    for (int s = s0 + threadIdx.x; s < s1; s += kCmpThreads) {
        const uint32_t key = order_key(imp[s]);
        if (((key ^ prefix) & fm) == 0u) atomicAdd(&h[(key >> sh) & dm], 1u);
    }
    __syncthreads();
    uint32_t* g = w.hist + pass * kCmpBins;
    for (int i = threadIdx.x; i < kCmpBins; i += kCmpThreads)
        if (h[i]) atomicAdd(&g[i], h[i]);
}

// The bin holding the remaining-th largest key: fix its digit, subtract the
// keys of the bins above it.  One workgroup per sequence.
__global__ __launch_bounds__(kCmpThreads) void k_cmp_pick(CompressArgs a, int pass) {
    constexpr int PER = kCmpBins / kCmpThreads;         // 8 bins per thread, thread t: bins 8t..8t+7
    __shared__ uint32_t above[kCmpThreads];             // keys in the bins of higher threads
    const SeqWs w = seq_ws(a.ws, blockIdx.x, a.nch);
    const uint32_t* g = w.hist + pass * kCmpBins;
    const int t = threadIdx.x;
    uint32_t mine = 0u;
#pragma unroll
    for (int i = 0; i < PER; ++i) mine += g[PER * t + i];
    above[t] = mine;
    __syncthreads();
    // suffix sum: above[t] = keys in bins of threads > t (Hillis-Steele over 256 entries)
    uint32_t incl = mine;
    for (int o = 1; o < kCmpThreads; o <<= 1) {
        const uint32_t add = t + o < kCmpThreads ? above[t + o] : 0u;
        __syncthreads();
        incl += add;
        above[t] = incl;
        __syncthreads();
    }
    const uint32_t rem = w.state[1];
    uint32_t acc = incl - mine;                          // keys above this thread's bins
    __syncthreads();                                     // every thread has read state[1]
    if (acc < rem && rem <= incl) {                      // exactly one thread
        for (int i = PER - 1; i >= 0; --i) {
            const uint32_t c = g[PER * t + i];
            if (acc + c >= rem) {
                w.state[0] |= static_cast<uint32_t>(PER * t + i) << digit_shift(pass);
                w.state[1] = rem - acc;
                break;
            }
            acc += c;
        }
    }
}

__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
    // sh: kCmpThreads words of LDS
    const int t = threadIdx.x;
    sh[t] = v;
    __syncthreads();
    uint32_t incl = v;
    for (int o = 1; o < kCmpThreads; o <<= 1) {
        const uint32_t add = t >= o ? sh[t - o] : 0u;
        __syncthreads();
        incl += add;
        sh[t] = incl;
        __syncthreads();
    }
    total = sh[kCmpThreads - 1];
    __syncthreads();
    return incl - v;
}

// Which tokens of [s0, s0 + kCmpPer) the thread's flags describe.
struct Flags {
    uint32_t fixed;   // bit i: kept whatever the tie rank (window, key > T, or every old token kept)
    uint32_t eq;      // bit i: an old token with key == T (kept if its rank among them is small enough)
};

__device__ __forceinline__ Flags token_flags(const CompressArgs& a, const float* imp, uint32_t T, int s0) {
    const int n_old = a.n_k - a.window;
    Flags f{0u, 0u};
#pragma unroll
    for (int i = 0; i < kCmpPer; ++i) {
        const int s = s0 + i;
        if (s >= a.n_k) break;
        if (s >= n_old || a.keep == n_old) {
            f.fixed |= 1u << i;
        } else if (a.keep > 0) {
            const uint32_t key = order_key(imp[s]);
            if (key > T) f.fixed |= 1u << i;
            else if (key == T) f.eq |= 1u << i;
        }
    }
    return f;
}

__global__ __launch_bounds__(kCmpThreads) void k_cmp_count(CompressArgs a) {
    __shared__ uint32_t sh[kCmpThreads];
    const int b = blockIdx.y, c = blockIdx.x;
    const SeqWs w = seq_ws(a.ws, b, a.nch);
    const float* imp = a.imp + static_cast<size_t>(b) * a.n_k;
    const Flags f = token_flags(a, imp, w.state[0], c * kCmpChunk + kCmpPer * static_cast<int>(threadIdx.x));
    uint32_t nf = 0u, ne = 0u;
    block_excl_scan(static_cast<uint32_t>(__builtin_popcount(f.fixed)), sh, nf);
    block_excl_scan(static_cast<uint32_t>(__builtin_popcount(f.eq)), sh, ne);
    if (threadIdx.x == 0) {
        w.fixed[c] = nf;
        w.eq[c] = ne;
    }
}

// Per sequence: T-keys before each chunk and each chunk's first output slot.
__global__ __launch_bounds__(kCmpThreads) void k_cmp_scan(CompressArgs a) {
    __shared__ uint32_t sh[kCmpThreads];
    const SeqWs w = seq_ws(a.ws, blockIdx.x, a.nch);
    const uint32_t take = w.state[1];
    uint32_t eq_base = 0u, slot_base = 0u;
    for (int c0 = 0; c0 < a.nch; c0 += kCmpThreads) {
        const int c = c0 + threadIdx.x;
        const uint32_t e = c < a.nch ? w.eq[c] : 0u;
        const uint32_t fx = c < a.nch ? w.fixed[c] : 0u;
        uint32_t etot = 0u;
        const uint32_t ebefore = eq_base + block_excl_scan(e, sh, etot);
        // T-keys of this chunk that are kept: those ranked below `take`
        const uint32_t keq = ebefore >= take ? 0u : min(e, take - ebefore);
        uint32_t ktot = 0u;
        const uint32_t sbefore = slot_base + block_excl_scan(fx + keq, sh, ktot);
        if (c < a.nch) {
            w.eq[c] = ebefore;
            w.fixed[c] = sbefore;
        }
        eq_base += etot;
        slot_base += ktot;
    }
}

// Copies the chunk's nk kept rows of one array.  Their output slots are
// consecutive, so piece j of the chunk's output goes to dst + j * UNIT and the
// stores are contiguous.  A thread moves U pieces per step and loads the next
// step's pieces before it stores the current ones, so up to 2U loads are in
// flight.
template <int UNIT>
__device__ __forceinline__ void copy_rows(const uint8_t* src, uint8_t* dst, int bytes, const int* ls, int nk) {
    using V = typename std::conditional<UNIT == 16, v4u32, uint32_t>::type;
    constexpr int U = 8;
    constexpr int STEP = U * kCmpThreads;
    const int per = bytes / UNIT;
    const int total = nk * per;
    auto load = [&](int j0, V* x) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u * kCmpThreads;
            if (j < total) {
                const int r = j / per, piece = j - r * per;
                x[u] = *reinterpret_cast<const V*>(src + static_cast<size_t>(ls[r]) * bytes + piece * UNIT);
            }
        }
    };
    V cur[U];
    int j0 = threadIdx.x;
    if (j0 >= total) return;
    load(j0, cur);
    while (true) {
        V nxt[U];
        const bool more = j0 + STEP < total;
        if (more) load(j0 + STEP, nxt);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u * kCmpThreads;
            if (j < total) __builtin_nontemporal_store(cur[u], reinterpret_cast<V*>(dst + static_cast<size_t>(j) * UNIT));
        }
        if (!more) break;
#pragma unroll
        for (int u = 0; u < U; ++u) cur[u] = nxt[u];
        j0 += STEP;
    }
}

__global__ __launch_bounds__(kCmpThreads) void k_cmp_write(CompressArgs a) {
    __shared__ uint32_t sh[kCmpThreads];
    __shared__ int lsrc[kCmpChunk];
    const int b = blockIdx.y, c = blockIdx.x;
    const SeqWs w = seq_ws(a.ws, b, a.nch);
    const float* imp = a.imp + static_cast<size_t>(b) * a.n_k;
    const int s0 = c * kCmpChunk + kCmpPer * static_cast<int>(threadIdx.x);
    const Flags f = token_flags(a, imp, w.state[0], s0);
    const uint32_t take = w.state[1];
    uint32_t etot = 0u;
    const uint32_t erank0 = w.eq[c] + block_excl_scan(static_cast<uint32_t>(__builtin_popcount(f.eq)), sh, etot);
    // the thread's T-keys in order get ranks erank0, erank0 + 1, ...; kept below `take`
    uint32_t kept = f.fixed;
    {
        uint32_t r = erank0, m = f.eq;
        while (m) {
            const int i = __builtin_ctz(m);
            m &= m - 1u;
            if (r < take) kept |= 1u << i;
            ++r;
        }
    }
    uint32_t nk = 0u;
    const uint32_t local = block_excl_scan(static_cast<uint32_t>(__builtin_popcount(kept)), sh, nk);
    const uint32_t first = w.fixed[c];
    const size_t n_keep = static_cast<size_t>(a.n_keep);
    {
        uint32_t j = local, m = kept;
        while (m) {
            const int i = __builtin_ctz(m);
            m &= m - 1u;
            lsrc[j] = b * a.n_k + s0 + i;
            a.pos_out[b * n_keep + first + j] = s0 + i;
            ++j;
        }
    }
    __syncthreads();
    for (int r = 0; r < a.nrow; ++r) {
        uint8_t* d = a.dst[r] + (b * n_keep + first) * static_cast<size_t>(a.bytes[r]);
        if (a.unit[r] == 16) copy_rows<16>(a.src[r], d, a.bytes[r], lsrc, static_cast<int>(nk));
        else copy_rows<4>(a.src[r], d, a.bytes[r], lsrc, static_cast<int>(nk));
    }
}

}  // namespace

int compress_chunks(int n_k) { return (n_k + kCmpChunk - 1) / kCmpChunk; }

size_t compress_workspace_bytes(int batch, int n_k) {
    return static_cast<size_t>(batch) * (3 * kCmpBins + 4 + 2 * static_cast<size_t>(compress_chunks(n_k))) * 4;
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t st) {
    const int n_old = a.n_k - a.window;
    hipLaunchKernelGGL(k_cmp_clear, dim3(a.B), dim3(kCmpThreads), 0, st, a);
    if (a.keep > 0 && a.keep < n_old) {
        const dim3 hg((n_old + kCmpHistKeys - 1) / kCmpHistKeys, a.B);
        for (int pass = 0; pass < 3; ++pass) {
            hipLaunchKernelGGL(k_cmp_hist, hg, dim3(kCmpThreads), 0, st, a, pass);
            hipLaunchKernelGGL(k_cmp_pick, dim3(a.B), dim3(kCmpThreads), 0, st, a, pass);
        }
    }
    const dim3 cg(a.nch, a.B);
    hipLaunchKernelGGL(k_cmp_count, cg, dim3(kCmpThreads), 0, st, a);
    hipLaunchKernelGGL(k_cmp_scan, dim3(a.B), dim3(kCmpThreads), 0, st, a);
    hipLaunchKernelGGL(k_cmp_write, cg, dim3(kCmpThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace dsa
