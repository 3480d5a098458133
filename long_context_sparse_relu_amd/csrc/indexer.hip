// indexer.hip -- lightning-indexer score kernels.
//
// I[t,s] = sum_h w[t,h] * ReLU(q_I[t,h] . k_I[s]) for s <= pos(t), -inf after.
// The indexer uses few heads, index_head_dim 128, ReLU in place of softmax and
// FP8 arithmetic ("DeepSeek-V3.2-Exp 稀疏注意力机制(DSA)技术深度解析",
// sheratonhq.com, section 1).  With E4M3 inputs the per-token scales are
// positive, so they factor out of the ReLU: I = sq[t]*sk[s]*sum_h w*ReLU(c_q.c_k)
// where c are the decoded codes; the code products are exact in fp32.
#include <climits>
#include <type_traits>
#include "dsa_kernels.h"
#include "fp8_index.h"
#include "topk_common.h"

namespace dsa {

// ---------------------------------------------------------------------------
// Generic path: any storage type, 1..64 heads.  One thread per key; the query
// row (H x 128, decoded to fp32) and its head weights sit in LDS and are read
// as broadcasts.  Used for fp32/bf16 indexers and as the reference layout for
// shapes the MFMA kernels do not take.
// ---------------------------------------------------------------------------
template <int DT, int HMAX>
__global__ __launch_bounds__(256) void k_index_generic(
    const void* __restrict__ iq, const float* __restrict__ iq_scale,
    const void* __restrict__ ik, const float* __restrict__ ik_scale,
    const float* __restrict__ iw, const int32_t* __restrict__ q_pos,
    int row0, int n_q, int n_k, int H, float* __restrict__ scores)
{
    constexpr int D = 128;
    __shared__ float q_s[HMAX * D];
    __shared__ float w_s[HMAX];
    const int row = row0 + blockIdx.y;        // b * n_q + t
    const int b = row / n_q;
    const int pos = row_pos(q_pos, row, n_q, n_k);
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    float* out = scores + static_cast<size_t>(blockIdx.y) * n_k;
    const int first = blockIdx.x * blockDim.x;
    if (first > pos) {                        // whole block is in the future
        if (s < n_k) out[s] = -__builtin_inff();
        return;
    }
    for (int i = threadIdx.x; i < HMAX * D; i += blockDim.x) {
        int h = i / D;
        q_s[i] = h < H ? load_as_f32<DT>(iq, static_cast<size_t>(row) * H * D + i) : 0.0f;
    }
    for (int h = threadIdx.x; h < HMAX; h += blockDim.x)
        w_s[h] = h < H ? iw[static_cast<size_t>(row) * H + h] : 0.0f;
    __syncthreads();
    if (s >= n_k) return;
    if (s > pos) { out[s] = -__builtin_inff(); return; }

    float acc[HMAX];
#pragma unroll
    for (int h = 0; h < HMAX; ++h) acc[h] = 0.0f;
    const size_t kbase = (static_cast<size_t>(b) * n_k + s) * D;
    for (int d = 0; d < D; d += 4) {
        float k0 = load_as_f32<DT>(ik, kbase + d + 0);
        float k1 = load_as_f32<DT>(ik, kbase + d + 1);
        float k2 = load_as_f32<DT>(ik, kbase + d + 2);
        float k3 = load_as_f32<DT>(ik, kbase + d + 3);
#pragma unroll
        for (int h = 0; h < HMAX; ++h) {
            const float* qh = q_s + h * D + d;
            acc[h] = fmaf(qh[0], k0, acc[h]);
            acc[h] = fmaf(qh[1], k1, acc[h]);
            acc[h] = fmaf(qh[2], k2, acc[h]);
            acc[h] = fmaf(qh[3], k3, acc[h]);
        }
    }
    float score = 0.0f;
#pragma unroll
    for (int h = 0; h < HMAX; ++h) score = fmaf(w_s[h], fmaxf(acc[h], 0.0f), score);
    if (DT == E4M3) score *= iq_scale[row] * ik_scale[static_cast<size_t>(b) * n_k + s];
    out[s] = score;
}

// ---------------------------------------------------------------------------
// FP8 streaming path (decode and any row count): up to 16 heads, d = 128,
// 16 keys per MFMA (fp8_index.h).  Keys stream from HBM once; each wave keeps
// U blocks of 16 keys in flight.  Two output modes:
//   scores      every score is written; when `hist` is given the workgroup
//               also counts the top 11 bits of each visible score's order key
//               in LDS and adds its non-empty bins to the row's histogram,
//               which saves the top-k a pass;
//   candidates  nothing is written except the scores whose order key reaches
//               the row's sampled lower bound (meta[S_KLOW]); they are
//               gathered per workgroup in LDS and appended to the row's
//               candidate list as (key << 32 | ~position).
// ---------------------------------------------------------------------------
// Launch shape, measured on decode_128k and decode_1m with the whole-line
// loads: 8192 keys per workgroup of 4 waves with a 128-register budget
// (indexer 166 us) against 4096 keys at 64 registers (183 us); 16384 keys,
// 8 waves per workgroup, other budgets and register prefetch of the next
// batch were equal or slower.
#ifndef DSA_IDX_U
#define DSA_IDX_U 4          // blocks of 16 keys each wave loads per step
#endif
#ifndef DSA_IDX_KPB
#define DSA_IDX_KPB 8192     // keys per workgroup
#endif
#ifndef DSA_IDX_WAVES
#define DSA_IDX_WAVES 4      // waves per workgroup
#endif
#ifndef DSA_IDX_OCC
#define DSA_IDX_OCC 4        // waves per SIMD the register budget must allow
#endif

template <int U, bool CAND>
__global__ __launch_bounds__(DSA_IDX_WAVES * 64) __attribute__((amdgpu_waves_per_eu(DSA_IDX_OCC)))
void k_index_fp8_mfma(IndexArgs x, int keys_per_block) {
    static_assert(U % 4 == 0, "keys are scored 64 at a time");
    __shared__ uint32_t lh[CAND ? 1 : kTopkBins];
    __shared__ uint64_t cbuf[CAND ? kIdxCandBuf : 1];
    __shared__ uint32_t n_c, g_c;
    const int row = x.row0 + blockIdx.y;
    const int n_q = x.n_q, n_k = x.n_k, H = x.H;
    const int b = row / n_q;
    const int pos = row_pos(x.q_pos, row, n_q, n_k);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;
    const int kg = lane >> 4;
    uint32_t* hist = CAND ? nullptr : x.hist;
    uint32_t* meta = CAND ? x.meta + static_cast<size_t>(blockIdx.y) * kTopkMeta : nullptr;
    uint32_t k_low = 0;
    bool collect = false;
    if constexpr (CAND) {
        if (threadIdx.x == 0) n_c = 0;
        k_low = meta[S_KLOW];
        // rows that keep every ranked key need no candidates
        collect = pos + 1 - x.window - x.sinks > x.k;
    } else if (hist) {
        for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x) lh[i] = 0u;
    }
    const Fp8Query q = load_fp8_query(static_cast<const uint8_t*>(x.iq), x.iq_scale, x.iw, row, H, lane);
    const uint8_t* kb = static_cast<const uint8_t*>(x.ik) + static_cast<size_t>(b) * n_k * 128;
    const float* ksb = x.ik_scale + static_cast<size_t>(b) * n_k;
    float* out = x.scores + static_cast<size_t>(blockIdx.y) * n_k;
    if (CAND || hist) __syncthreads();

    const int nwaves = blockDim.x >> 6;
    const int s_begin = blockIdx.x * keys_per_block;
    const int s_end = min(s_begin + keys_per_block, n_k);
    const int step = nwaves * 16 * U;
    const uint64_t below = (1ull << lane) - 1ull;

    // a batch is U/4 groups of 64 keys; lane l scores key base + 64g + l of group g
    // Loads are issued unconditionally: a key past the chunk or past pos
    // reads the chunk's last visible key (key 0 when it has none) and its
    // score is discarded, so no branch separates a load from its use.
    const int lim = max(0, min(s_end, pos + 1) - 1);
    // whole-line loads of the batch's 64 U/4 keys and their scales
    auto load_batch = [&](int base, v4i* lines, float* sk) {
#pragma unroll
        for (int g = 0; g < U / 4; ++g) load_keys64_lines(kb, base + 64 * g, lim, lane, lines + 8 * g);
#pragma unroll
        for (int g = 0; g < U / 4; ++g) sk[g] = __builtin_nontemporal_load(ksb + min(base + g * 64 + lane, lim));
    };
    auto score_batch = [&](int base, const v4i* lines, const float* sk) {
#pragma unroll
        for (int g = 0; g < U / 4; ++g) {
            v8i bv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) bv[u] = keys_block_operand(lines + 8 * g, u, lane);
            const float part = fp8_score4(q, bv, sk[g]);
            const int s = base + g * 64 + lane;
            const bool mine = s < s_end;
            if constexpr (CAND) {
                const uint32_t key = order_key(part);
                const bool take = mine && collect && s >= x.sinks && s <= pos - x.window && key >= k_low;
                const uint64_t m = __ballot(take);
                if (m) {
                    uint32_t base_slot = 0;
                    if (lane == 0) base_slot = atomicAdd(&n_c, static_cast<uint32_t>(__popcll(m)));
                    base_slot = __shfl(base_slot, 0);
                    const uint32_t slot = base_slot + static_cast<uint32_t>(__popcll(m & below));
                    if (take && slot < static_cast<uint32_t>(kIdxCandBuf)) cbuf[slot] = composite64(key, s);
                }
            } else if (mine) {
                const float score = s <= pos ? part : -__builtin_inff();
                out[s] = score;
                if (hist && s <= pos) atomicAdd(&lh[order_key(score) >> 21], 1u);
            }
        }
    };

#ifndef DSA_IDX_PREFETCH
#define DSA_IDX_PREFETCH 0
#endif
    if (DSA_IDX_PREFETCH) {
        // the next batch's loads are in flight while this one is scored
        v4i lines[2 * U];
        float sk[U / 4];
        int base = s_begin + wave * 16 * U;
        load_batch(base, lines, sk);
        for (; base < s_end; base += step) {
            v4i nlines[2 * U];
            float nsk[U / 4];
            load_batch(base + step, nlines, nsk);          // clamped to lim past the chunk
            score_batch(base, lines, sk);
#pragma unroll
            for (int j = 0; j < 2 * U; ++j) lines[j] = nlines[j];
#pragma unroll
            for (int g = 0; g < U / 4; ++g) sk[g] = nsk[g];
        }
    } else {
        for (int base = s_begin + wave * 16 * U; base < s_end; base += step) {
            v4i lines[2 * U];
            float sk[U / 4];
            load_batch(base, lines, sk);
            score_batch(base, lines, sk);
        }
    }
    if constexpr (CAND) {
        __syncthreads();
        if (threadIdx.x == 0) {
            g_c = n_c ? atomicAdd(&meta[S_NCAND], n_c) : 0u;
            if (n_c > static_cast<uint32_t>(kIdxCandBuf)) atomicOr(&meta[S_OVF], 1u);
        }
        __syncthreads();
        const uint32_t nkeep = min(n_c, static_cast<uint32_t>(kIdxCandBuf));
        uint64_t* cd = x.cand + static_cast<size_t>(blockIdx.y) * x.cand_cap;
        for (uint32_t i = threadIdx.x; i < nkeep; i += blockDim.x)
            if (g_c + i < static_cast<uint32_t>(x.cand_cap)) cd[g_c + i] = cbuf[i];
    } else if (hist) {
        __syncthreads();
        uint32_t* gh = hist + static_cast<size_t>(blockIdx.y) * kTopkBins;
        for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x)
            if (lh[i]) atomicAdd(&gh[i], lh[i]);
    }
}

// ---------------------------------------------------------------------------
// Tiled path for prefill rows (FP8 E4M3 or bf16, up to 16 heads, d = 128).
// Query rows go in blocks of kTQ consecutive rows of one sequence (kQPW per
// wave).  A block scores the keys its rows see in tiles of 64, staged in LDS
// and shared by all kTQ queries, so every key row is fetched once per kTQ
// queries and each key operand read from LDS feeds kQPW MFMAs.  A launch
// with few query blocks (a fused row block) cuts its (block, tile) pairs,
// block-major, into equal runs, one per workgroup the chip holds at once, so
// every workgroup starts at once and all finish together; a run crosses at
// most one block boundary and loads a block's queries once.  A launch with
// many blocks (a whole sequence) cuts each block into pieces of kTiledPiece
// tiles, handed out longest blocks first over several rounds.  No workgroup
// is launched without work.  The next tile is fetched into registers while
// the current one is scored.  Per (query, 16 keys) the
// scores come from one v_mfma_scale_f32_16x16x128_f8f6f4 (FP8) or four
// v_mfma_f32_16x16x32_bf16 (bf16) with the heads as M; each lane folds its
// four heads with ReLU and the head weights, and one reduce-scatter over the
// four 16-key blocks of a tile finishes the head sums, leaving lane l with
// the score of key l of the tile (one coalesced 256-byte store per query and
// tile).  Keys past a query's last visible key are written as -inf only when
// `write_future` (the unfused entry point): inside the block's tiles by the
// scorer, past them by k_fill_future.
// ---------------------------------------------------------------------------
#ifndef DSA_TILED_TILE
#define DSA_TILED_TILE 64
#endif
constexpr int kTileKeys = DSA_TILED_TILE;   // keys per LDS tile (a multiple of 64)
static_assert(kTileKeys % 64 == 0, "tiles are scored 64 keys at a time");
// query rows per wave and waves per workgroup (measured best: FP8 4 x 8, bf16 2 x 4)
#ifndef DSA_TILED_F8_QPW
#define DSA_TILED_F8_QPW 4
#endif
#ifndef DSA_TILED_F8_TW
#define DSA_TILED_F8_TW 8
#endif
template <int DT> struct TiledShape {
    static constexpr int QPW = DT == E4M3 ? DSA_TILED_F8_QPW : 2, TW = DT == E4M3 ? DSA_TILED_F8_TW : 4;
};
// fewest tiles in a workgroup's run when a launch has few tiles, and the
// piece length when a launch has many query blocks
constexpr int kTiledMinRun = 4;
#ifndef DSA_TILED_PIECE
#define DSA_TILED_PIECE 64
#endif
constexpr int kTiledPiece = DSA_TILED_PIECE;

// 64-key tiles of query block j of a launch over nrows rows: the tiles that
// hold a key some row of the block sees.  base is the position of the
// launch's first row (n_k - n_q + its index in the sequence); with explicit
// positions (all_keys) every key counts as seen.
__host__ __device__ inline int tiled_block_tiles(int j, int nrows, int kTQ, long long base, int n_k, bool all_keys) {
    if (all_keys) return (n_k + 63) / 64;
    const int rows_upto = (j + 1) * kTQ < nrows ? (j + 1) * kTQ : nrows;
    long long vis = base + rows_upto;
    if (vis > n_k) vis = n_k;
    return vis > 0 ? static_cast<int>((vis + 63) / 64) : 0;
}

// This workgroup's share of a launch's (query block, key tile) pairs,
// block-major.  Runs (piece == 0): tiles [total*w/G, total*(w+1)/G), which
// cross at most one block boundary (the launcher checks that no block is
// shorter than a run): ta tiles of block qb from tile t0, then tb tiles of
// block qb + 1.  Pieces (piece > 0): block j's tiles cut into pieces of at
// most `piece` tiles, handed out in reverse block order (longest blocks
// first).  Either way the first block is found the same way: lane l sums the
// counts (tiles or pieces) of blocks [l*m, (l+1)*m), the lanes take an
// inclusive prefix, and the first lane whose prefix passes the target walks
// its own blocks.  Every wave does this and gets the same answer.  Returns
// false when the workgroup has no work.
// With PRO > 0 the runs are cut over a sequence in which every block with
// tiles starts with PRO units of no work, the cost of the prologue (query
// operands and weights) that a workgroup pays again when its run crosses
// into the next block: such a run then takes PRO fewer tiles, and the
// runs end together.
struct TiledWork { int qb, t0, tj, ta, tb, piece; };

template <int kTQ, int PRO = 0>
__device__ __forceinline__ bool tiled_work_start(int lane, int nrows, long long base, int n_k, bool all_keys,
                                                 int piece, long long total, TiledWork& w) {
    const int nqb = (nrows + kTQ - 1) / kTQ;
    const bool runs = piece == 0;
    const long long target = runs ? total * blockIdx.x / gridDim.x : static_cast<long long>(gridDim.x - 1 - blockIdx.x);
    const long long g_end = runs ? total * (blockIdx.x + 1) / gridDim.x : 0;
    if (runs && target >= g_end) return false;               // uniform over the workgroup
    auto units = [&](int j) {
        const int tj = tiled_block_tiles(j, nrows, kTQ, base, n_k, all_keys);
        return runs ? (tj > 0 ? tj + PRO : 0) : (tj + piece - 1) / piece;
    };
    // (a launch's units stay far below 2^31: the prefix scan is 32-bit, on DPP)
    const int m = (nqb + 63) / 64;
    uint32_t lsum = 0;
    for (int i = 0; i < m; ++i) {
        const int j = lane * m + i;
        if (j < nqb) lsum += static_cast<uint32_t>(units(j));
    }
    const uint32_t incl32 = wave_inclusive_sum(lsum);
    const long long incl = incl32;
    const int L = __ffsll(static_cast<long long>(__ballot(target < incl))) - 1;   // target < all units
    long long acc = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl32 - lsum), L));
    int j = L * m;
    int u = units(j);
    while (acc + u <= target) {
        acc += u;
        u = units(++j);
    }
    w.qb = __builtin_amdgcn_readfirstlane(j);
    w.tj = __builtin_amdgcn_readfirstlane(tiled_block_tiles(j, nrows, kTQ, base, n_k, all_keys));
    const int into = __builtin_amdgcn_readfirstlane(static_cast<int>(target - acc));
    w.piece = piece;
    w.ta = w.tb = 0;
    if (runs) {
        // the run's units: the block's prologue units it covers, then tiles
        // of block qb, then (prologue units and) tiles of block qb + 1
        const int skip = into < PRO ? PRO - into : 0;
        w.t0 = into < PRO ? 0 : into - PRO;
        const long long budget = g_end - target - skip;
        w.ta = static_cast<int>(max(0ll, min(static_cast<long long>(w.tj - w.t0), budget)));
        const long long rest = budget - w.ta - PRO;
        w.tb = rest > 0 ? static_cast<int>(min(rest, static_cast<long long>(
                              tiled_block_tiles(w.qb + 1, nrows, kTQ, base, n_k, all_keys))))
                        : 0;
    } else {
        w.t0 = into * piece;
    }
    return true;
}

template <int DT>
__global__ __launch_bounds__(TiledShape<DT>::TW * 64) void k_index_tiled(IndexArgs x, int t_first, int nrows,
                                                                        int piece, long long total, int write_future) {
    constexpr int kQPW = TiledShape<DT>::QPW, kTW = TiledShape<DT>::TW, kTQ = kQPW * kTW;
    constexpr int KROW = DT == E4M3 ? 128 : 256;           // bytes per key row
    constexpr int KSTR = KROW + 16;                         // padded LDS stride (conflict-free 16 B reads)
    constexpr int NC = DT == E4M3 ? 1 : 4;                  // MFMAs per 16 keys
    constexpr int LPT = kTileKeys * KROW / 16 / (kTW * 64); // 16-byte loads per thread per tile
    static_assert(LPT * kTW * 64 * 16 == kTileKeys * KROW, "a tile must split evenly over the threads");
    __shared__ __align__(16) uint8_t k_s[2][kTileKeys * KSTR];   // double-buffered key tile
    __shared__ float ks_s[2][kTileKeys];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: rows and positions in SGPRs
    const int col = lane & 15, kg = lane >> 4;
    const int n_k = x.n_k, H = x.H;

    const int b = t_first / x.n_q;                           // every row of the launch is in sequence b
    const long long base = static_cast<long long>(n_k) - x.n_q + t_first % x.n_q;
    const bool all_keys = x.q_pos != nullptr;

    // Score keys [c0, c1) of query block qb (c0 a multiple of 64).
    auto run_segment = [&](const int qb, const int c0, const int c1) {
        const int tid = static_cast<int>(threadIdx.x);
        // the block's last visible key: positions run with the rows unless
        // they are explicit (then a uniform pass over the block's rows)
        int last = -1;
        if (x.q_pos) {
            for (int r = 0; r < kTQ; ++r) {
                const int lr = qb * kTQ + r;
                if (lr < nrows) last = max(last, row_pos(x.q_pos, t_first + lr, x.n_q, n_k));
            }
        } else {
            last = row_pos(nullptr, t_first + min(qb * kTQ + kTQ, nrows) - 1, x.n_q, n_k);
        }
        last = __builtin_amdgcn_readfirstlane(last);
        const int cvis = min(c1, last + 1);                      // keys some query of the block sees
        // -inf for keys [from, c1) of this wave's rows (the unfused entry point
        // writes every key of a row)
        auto write_inf = [&](int from) {
            for (int q = 0; q < kQPW; ++q) {
                const int lr = qb * kTQ + wave * kQPW + q;
                if (lr >= nrows) continue;
                float* out = x.scores + static_cast<size_t>(t_first + lr - x.row0) * n_k;
                for (int s = from + lane; s < c1; s += 64) out[s] = -__builtin_inff();
            }
        };
        if (c0 >= cvis) {                                        // uniform over the workgroup
            if (write_future) write_inf(c0);
            return;
        }

        // this wave's query rows (absolute row index t_first + qb*kTQ + kQPW*wave + q)
        int rows[kQPW], pos[kQPW];
        float w[kQPW][4], sq[kQPW];
        v8i a8[DT == E4M3 ? kQPW : 1];
        v8bf a16[DT == E4M3 ? 1 : kQPW][4];
        unsigned livem = 0;                                      // bit q: row q exists
#pragma unroll
        for (int q = 0; q < kQPW; ++q) {
            const int lr = qb * kTQ + wave * kQPW + q;          // row within the launch
            const bool live = lr < nrows;
            livem |= live ? 1u << q : 0u;
            rows[q] = t_first + (live ? lr : 0);
            pos[q] = live ? row_pos(x.q_pos, rows[q], x.n_q, n_k) : -1;  // may be negative for a live row
        }
        // Every operand load is issued unconditionally (a missing row reads row
        // t_first, heads past H read head H - 1) and masked afterwards, so one
        // wait covers them all.
        const int hq = min(col, H - 1);
#pragma unroll
        for (int q = 0; q < kQPW; ++q) {
            sq[q] = DT == E4M3 ? x.iq_scale[rows[q]] : 1.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) w[q][i] = x.iw[static_cast<size_t>(rows[q]) * H + min(4 * kg + i, H - 1)];
            if constexpr (DT == E4M3) {
                a8[q] = load_split32(static_cast<const uint8_t*>(x.iq) + (static_cast<size_t>(rows[q]) * H + hq) * 128, kg);
            } else {
                const uint16_t* qrow = static_cast<const uint16_t*>(x.iq) + (static_cast<size_t>(rows[q]) * H + hq) * 128 + kg * 32;
#pragma unroll
                for (int c = 0; c < 4; ++c) a16[q][c] = *reinterpret_cast<const v8bf*>(qrow + c * 8);
            }
        }
#pragma unroll
        for (int q = 0; q < kQPW; ++q) {
            const bool live = livem >> q & 1u;
            // the query's scale rides on its head weights: a score is then
            // (sum over heads of (w * sq) * ReLU(q . k)) * sk
#pragma unroll
            for (int i = 0; i < 4; ++i) w[q][i] = (live && 4 * kg + i < H) ? w[q][i] * sq[q] : 0.0f;
            if constexpr (DT == E4M3) {
                if (!(live && col < H)) a8[q] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (!(live && col < H)) a16[q][c] = v8bf{};
            }
        }
        const uint8_t* kb = static_cast<const uint8_t*>(x.ik) + static_cast<size_t>(b) * n_k * KROW;
        const float* ksb = DT == E4M3 ? x.ik_scale + static_cast<size_t>(b) * n_k : nullptr;
        float* orow[kQPW];
#pragma unroll
        for (int q = 0; q < kQPW; ++q) orow[q] = x.scores + static_cast<size_t>(rows[q] - x.row0) * n_k;

        // Every tile load is issued unconditionally, from an address clamped to
        // the last key, so no branch separates a load from its wait and the loop's
        // one wait covers exactly the loads and stores of its own iteration.  Rows
        // past n_k hold copies of the last key; their scores are never stored.
        v4i pre[LPT];
        float pre_s = 0.0f;
        auto fetch = [&](int k0) {
#pragma unroll
            for (int u = 0; u < LPT; ++u) {
                const int i = tid + u * kTW * 64;
                const int kr = i / (KROW / 16), off = (i % (KROW / 16)) * 16;
                pre[u] = *reinterpret_cast<const v4i*>(kb + static_cast<size_t>(min(k0 + kr, n_k - 1)) * KROW + off);
            }
            if constexpr (DT == E4M3) pre_s = ksb[min(k0 + static_cast<int>(tid % kTileKeys), n_k - 1)];
        };
        auto stage = [&](int nb) {
#pragma unroll
            for (int u = 0; u < LPT; ++u) {
                const int i = tid + u * kTW * 64;
                const int kr = i / (KROW / 16), off = (i % (KROW / 16)) * 16;
                *reinterpret_cast<v4i*>(k_s[nb] + kr * KSTR + off) = pre[u];
            }
            if (DT == E4M3 && tid < kTileKeys) ks_s[nb][tid] = pre_s;
        };
        // Scores of the previous 64 keys, stored while the next 64 are scored.
        // Stores count against the same in-order counter as the tile loads, so
        // the four stores of a wave are issued unconditionally, after the loads
        // of the next tile: the wait for those loads then leaves the stores in
        // flight.  They are buffer stores, one resource per query row (no
        // records for a missing row); a lane with nothing to store gets an
        // offset past the row, which the hardware drops.
        constexpr uint32_t kNoStore = 0x7fffffffu;
        __amdgpu_buffer_rsrc_t orsrc[kQPW];
#pragma unroll
        for (int q = 0; q < kQPW; ++q)
            orsrc[q] = __builtin_amdgcn_make_buffer_rsrc(orow[q], 0, (livem >> q & 1u) ? n_k * 4 : 0, kBufferWord3);
        float held[kQPW] = {};
        uint32_t hoff[kQPW];                                     // byte offset of held[q] in its row, or kNoStore
#pragma unroll
        for (int q = 0; q < kQPW; ++q) hoff[q] = kNoStore;
        auto flush = [&]() {
#pragma unroll
            for (int q = 0; q < kQPW; ++q)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(held[q]), orsrc[q], static_cast<int>(hoff[q]), 0, 0);
        };
        int minpos = pos[0];
#pragma unroll
        for (int q = 1; q < kQPW; ++q) minpos = min(minpos, pos[q]);   // -1 when some row is missing

        fetch(c0);
        stage(0);
        // every prologue load (queries, weights, positions) has landed before the loop
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        int cur = 0;
        for (int k0 = c0; k0 < cvis; k0 += kTileKeys) {
            fetch(min(k0 + kTileKeys, cvis - 1));                // in flight while this tile is scored
            // Score 64 keys starting at k0 + 64*sub.  FAST: every query of the
            // wave sees all of them (the common case away from the diagonal), so
            // no per-key visibility test or -inf is needed.
            auto score64 = [&](int sub, auto fast_tag) {
                constexpr bool FAST = decltype(fast_tag)::value;
                // key k0 + 64*sub + g16*16 + col sits in LDS row 64*sub + g16*16 + col;
                // lane l scores key k0 + 64*sub + l
                v8i b8[4];
                v8bf b16[4][4];
#pragma unroll
                for (int g16 = 0; g16 < 4; ++g16) {
                    const uint8_t* kr = k_s[cur] + (sub * 64 + g16 * 16 + col) * KSTR;
                    if constexpr (DT == E4M3) {
                        b8[g16] = load_split32(kr, kg);
                    } else {
#pragma unroll
                        for (int c = 0; c < 4; ++c) b16[g16][c] = *reinterpret_cast<const v8bf*>(kr + kg * 64 + c * 16);
                    }
                }
                const int s = k0 + sub * 64 + lane;
                const float sk = DT == E4M3 ? ks_s[cur][sub * 64 + lane] : 1.0f;
                const uint32_t off = static_cast<uint32_t>(s) * 4u;
#pragma unroll
                for (int q = 0; q < kQPW; ++q) {
                    float p[4];
#pragma unroll
                    for (int g16 = 0; g16 < 4; ++g16) {
                        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
                        if constexpr (DT == E4M3) {
                            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8[q], b8[g16], acc, 0, 0, 0, 127, 0, 127);
                        } else {
#pragma unroll
                            for (int c = 0; c < NC; ++c)
                                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a16[q][c], b16[g16][c], acc, 0, 0, 0);
                        }
                        float part = w[q][0] * relu(acc[0]);
                        part = fmaf(w[q][1], relu(acc[1]), part);
                        part = fmaf(w[q][2], relu(acc[2]), part);
                        p[g16] = fmaf(w[q][3], relu(acc[3]), part);
                    }
                    const float part = reduce_scatter4(p[0], p[1], p[2], p[3]);
                    const float score = DT == E4M3 ? part * sk : part;
                    if constexpr (FAST) {
                        held[q] = score;
                        hoff[q] = off;
                    } else {
                        const bool vis = s <= pos[q];
                        held[q] = vis ? score : -__builtin_inff();
                        hoff[q] = (s < c1 && (vis || write_future)) ? off : kNoStore;
                    }
                }
#ifndef DSA_TILED_NO_PINGPONG
                // Ping-pong: each MFMA is issued before the ReLU-weight epilogue
                // of the one before it, so the matrix core works through one
                // product while the vector ALU folds the previous one (left to
                // itself the scheduler runs each product and its epilogue back
                // to back).
                __builtin_amdgcn_sched_group_barrier(0x100, 8 * NC, 0);   // the tile's LDS operand reads
                __builtin_amdgcn_sched_group_barrier(0x008, NC, 0);       // product 0
#pragma unroll
                for (int i = 1; i < 4 * kQPW; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, NC, 0);   // product i
                    __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);   // epilogue of product i - 1
                }
#endif
            };
#pragma unroll
            for (int sub = 0; sub < kTileKeys / 64; ++sub) {
                flush();                                         // on every path, so the tile wait can count past it
                if (k0 + sub * 64 + 63 <= minpos) score64(sub, std::true_type{});
                else score64(sub, std::false_type{});
            }
            // the next tile goes to the other buffer, which every wave finished
            // reading before the barrier that ended the previous iteration; the
            // scheduling barrier keeps the LDS writes (and the wait for the tile
            // loads in front of them) after this tile's MFMAs
            __builtin_amdgcn_sched_barrier(0);
            stage(cur ^ 1);
            __syncthreads();
            cur ^= 1;
        }
        flush();
        if (write_future) write_inf(cvis);                       // keys of this run no query of the block sees
    };

    TiledWork w;
    if (!tiled_work_start<kTQ>(lane, nrows, base, n_k, all_keys, piece, total, w)) return;
    if (w.piece > 0) {
        run_segment(w.qb, 64 * w.t0, min(64 * min(w.t0 + w.piece, w.tj), n_k));
        return;
    }
    // a run: the rest of this block, then (if the run is longer) the head of
    // the next block
    run_segment(w.qb, 64 * w.t0, min(64 * (w.t0 + w.ta), n_k));
    if (w.tb > 0) {
        __syncthreads();                                      // the second segment restages both LDS buffers
        run_segment(w.qb + 1, 0, min(64 * w.tb, n_k));
    }
}

// ---------------------------------------------------------------------------
// FP8 prefill path with the query rows as the rows of the MFMA.  A wave holds
// RG groups of 16 query rows with every head's operand in registers (16
// heads x 8 registers per group); per head and 16 keys one
// v_mfma_scale_f32_16x16x128_f8f6f4 gives that head's 16 x 16 dot products,
// lane l holding queries 4(l/16)..4(l/16)+3 of one key (column l%16 of key
// block u is key 4(l%16) + u of the 64-key tile).  Each lane folds its
// four products with ReLU and the head weight (one integer max and one FMA
// each) into four running sums, so the sum over heads needs no exchange
// between lanes and the only vector work per product is those two
// instructions.  The waves of a workgroup share each 64-key tile staged in
// LDS.  The head weights times the query scales sit in LDS ([head][query])
// and are read as one 16-byte broadcast per head and group.  Work split as
// in k_index_tiled; a lane stores four consecutive keys of a query at once.
// ---------------------------------------------------------------------------
#ifndef DSA_Q16_RG
#define DSA_Q16_RG 1
#endif
constexpr int kQ16RG = DSA_Q16_RG;                   // groups of 16 query rows per wave
constexpr int kQ16W = kQ16RG == 1 ? 8 : 4;           // waves per workgroup (one workgroup per CU)
constexpr int kQ16Q = 16 * kQ16RG * kQ16W;           // query rows per workgroup (block)
// a block's prologue (256 KiB of query operands and the weights, ~10 us)
// counted as this many tiles (~3.5 us each) when runs are cut
#ifndef DSA_Q16_PRO
#define DSA_Q16_PRO 3
#endif
constexpr int kQ16Pro = DSA_Q16_PRO;

__global__ __launch_bounds__(kQ16W * 64) __attribute__((amdgpu_waves_per_eu(kQ16W / 4)))
void k_index_fp8_q16(IndexArgs x, int t_first, int nrows, int piece, long long total, int write_future) {
    constexpr int RG = kQ16RG;
    constexpr int KSTR = 144;                                // padded LDS stride of a 128-byte key row
    constexpr int PIECES = 64 * 128 / 16 / (kQ16W * 64);     // 16-byte pieces of a key tile per thread
    __shared__ __align__(16) uint8_t k_s[2][64 * KSTR];      // double-buffered key tile
    __shared__ float ks_s[2][kQ16W * 64];                    // key scales (entries 64.. are never read)
    __shared__ __align__(16) float w_s[16 * kQ16Q];          // [head][query]: w * sq (0 past H or nrows)

    const int lane = threadIdx.x & 63;
    const int tid = static_cast<int>(threadIdx.x);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15, kg = lane >> 4;
    const int n_k = x.n_k, H = x.H;
    const int b = t_first / x.n_q;                           // every row of the launch is in sequence b
    const long long base = static_cast<long long>(n_k) - x.n_q + t_first % x.n_q;
    const bool all_keys = x.q_pos != nullptr;
    const uint8_t* kb = static_cast<const uint8_t*>(x.ik) + static_cast<size_t>(b) * n_k * 128;
    const float* ksb = x.ik_scale + static_cast<size_t>(b) * n_k;
    constexpr uint32_t kNoStore = 0x7FFFFFF0u;               // past any row range (<= 2^30 bytes): dropped
    const v4f zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

    auto run_segment = [&](const int qb, const int c0, const int c1) {
        // the block's last visible key (every wave computes it)
        int last = -1;
        for (int r = lane; r < kQ16Q; r += 64) {
            const int lr = qb * kQ16Q + r;
            if (lr < nrows) last = max(last, row_pos(x.q_pos, t_first + lr, x.n_q, n_k));
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) last = max(last, __shfl_xor(last, o));
        last = __builtin_amdgcn_readfirstlane(last);
        const int cvis = min(c1, last + 1);                  // keys some query of the block sees

        // row group g of this wave: block rows r0[g] .. r0[g] + nlive[g] - 1
        int r0[RG], nlive[RG], pos[RG][4], wmin = INT_MAX, wmax = -1;
        __amdgpu_buffer_rsrc_t orsrc[RG];
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            r0[g] = qb * kQ16Q + 16 * (wave * RG + g);
            nlive[g] = __builtin_amdgcn_readfirstlane(max(0, min(16, nrows - r0[g])));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = 4 * kg + i;
                pos[g][i] = q < nlive[g] ? row_pos(x.q_pos, t_first + r0[g] + q, x.n_q, n_k) : -1;
                if (q < nlive[g]) { wmin = min(wmin, pos[g][i]); wmax = max(wmax, pos[g][i]); }
            }
            // stores: one resource over the group's live rows (missing rows lie past its end)
            float* grow = x.scores + static_cast<size_t>(t_first + r0[g] - x.row0) * n_k;
            orsrc[g] = __builtin_amdgcn_make_buffer_rsrc(grow, 0, nlive[g] > 0 ? nlive[g] * n_k * 4 : 0, kBufferWord3);
        }
#pragma unroll
        for (int o = 16; o < 64; o <<= 1) {
            wmin = min(wmin, __shfl_xor(wmin, o));
            wmax = max(wmax, __shfl_xor(wmax, o));
        }
        wmin = __builtin_amdgcn_readfirstlane(wmin);         // first and last key every / any row of the wave sees
        wmax = __builtin_amdgcn_readfirstlane(wmax);
        uint32_t roff[4];                                    // lane's byte offset of output row 4kg + i
#pragma unroll
        for (int i = 0; i < 4; ++i) roff[i] = static_cast<uint32_t>(4 * kg + i) * static_cast<uint32_t>(n_k) * 4u;

        auto store_inf = [&](int from) {                     // -inf for keys [from, c1) of every row
#pragma unroll
            for (int g = 0; g < RG; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    for (int s0 = from; s0 < c1; s0 += 16)
                        if (s0 + col < c1)
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(-__builtin_inff()), orsrc[g],
                                                                  static_cast<int>(roff[i] + (s0 + col) * 4u), 0, 0);
        };
        if (c0 >= cvis) {                                    // uniform over the workgroup
            if (write_future) store_inf(c0);
            return;
        }


        // Tile loads: PIECES 16-byte pieces per thread, clamped to the last key.
        // Key r of a tile goes to LDS row 16 (r % 4) + r / 4, so that the MFMA
        // column c of key block u (LDS row 16 u + c) is key 4 c + u: each lane
        // then holds four consecutive keys of its queries and stores them with
        // one 16-byte store.
        v4i pre[PIECES];
        float pre_s = 0.0f;
        auto fetch = [&](int k0) {
#pragma unroll
            for (int p = 0; p < PIECES; ++p) {
                const int e = tid + p * kQ16W * 64, kr = e >> 3, off = (e & 7) * 16;
                pre[p] = *reinterpret_cast<const v4i*>(kb + static_cast<size_t>(min(k0 + kr, n_k - 1)) * 128 + off);
            }
            pre_s = ksb[min(k0 + (tid & 63), n_k - 1)];
        };
        auto stage = [&](int nb) {
#pragma unroll
            for (int p = 0; p < PIECES; ++p) {
                const int e = tid + p * kQ16W * 64, kr = e >> 3, off = (e & 7) * 16;
                *reinterpret_cast<v4i*>(k_s[nb] + (16 * (kr & 3) + (kr >> 2)) * KSTR + off) = pre[p];
            }
            // every thread writes (threads past the tile's 64 keys to unread
            // entries), so the scale load is never moved to a branch of its own
            ks_s[nb][tid < 64 ? 16 * (tid & 3) + (tid >> 2) : tid] = pre_s;
        };

        // scores of the previous tile, stored while the next is scored (16 per
        // group and lane: held[g][4u + i] is query 4 kg + i, key 4 col + u;
        // issued after the next tile's loads)
        float held[RG][16];
        uint32_t hbase = kNoStore;                           // (k0 + 4 col) * 4 of the held tile
        uint32_t hmask[RG];                                  // bit 4u + i: store held[g][4u + i]
        bool hall = false;                                   // uniform: store every held value
        // whole 16-byte stores need 16-byte aligned rows
        const bool vec_rows = (n_k & 3) == 0 && (reinterpret_cast<uintptr_t>(x.scores) & 15) == 0;
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            hmask[g] = 0u;
#pragma unroll
            for (int j = 0; j < 16; ++j) held[g][j] = 0.0f;
        }
        auto flush = [&]() {
#pragma unroll
            for (int g = 0; g < RG; ++g) {
                if (hall) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const v4i q4 = {__float_as_int(held[g][i]), __float_as_int(held[g][4 + i]),
                                        __float_as_int(held[g][8 + i]), __float_as_int(held[g][12 + i])};
                        __builtin_amdgcn_raw_buffer_store_b128(q4, orsrc[g], static_cast<int>(roff[i] + hbase), 0, 0);
                    }
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const uint32_t off = (hmask[g] >> (4 * u + i) & 1u) ? roff[i] + hbase + 4u * u : kNoStore;
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(held[g][4 * u + i]), orsrc[g],
                                                                  static_cast<int>(off), 0, 0);
                        }
                }
            }
        };

        fetch(c0);
        // The prologue's loads (the block's head weights and query scales, the
        // query operands, the first key tile) are all issued before any of them
        // is waited for, so the prologue costs one memory round trip.
        // Weights: entry e = tid + i * threads of the [head][query] table.
        constexpr int WPT = 16 * kQ16Q / (kQ16W * 64);
        static_assert(16 * kQ16Q % (kQ16W * 64) == 0, "whole weight entries per thread");
        float wl[WPT], sl[WPT];
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int e = tid + i * kQ16W * 64, h = e / kQ16Q, q = e % kQ16Q;
            const int row = t_first + min(qb * kQ16Q + q, nrows - 1);
            wl[i] = x.iw[static_cast<size_t>(row) * H + min(h, H - 1)];
            sl[i] = x.iq_scale[row];
        }
        // operands: head h of row r0[g] + col, loaded unconditionally from a
        // valid row.  A missing row's operand is never zeroed: its scores lie
        // past the end of the group's store resource and are dropped.  A head
        // past H repeats head H - 1 with weight 0, so it adds nothing (a NaN
        // code there is already in head H - 1's own term).
        v8i a[RG][16];
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const int arow = t_first + (nlive[g] > 0 ? r0[g] + min(col, nlive[g] - 1) : 0);
#pragma unroll
            for (int h = 0; h < 16; ++h)
                a[g][h] = load_split32(static_cast<const uint8_t*>(x.iq) + (static_cast<size_t>(arow) * H + min(h, H - 1)) * 128, kg);
        }
        __builtin_amdgcn_sched_barrier(0);                   // every load issued before the first wait
#pragma unroll
        for (int i = 0; i < WPT; ++i) {
            const int e = tid + i * kQ16W * 64, h = e / kQ16Q, q = e % kQ16Q;
            w_s[e] = (qb * kQ16Q + q < nrows && h < H) ? wl[i] * sl[i] : 0.0f;
        }
        stage(0);
        // The staged tile and weights are visible after this barrier, which
        // waits for LDS only: the query operands may still be in flight, and
        // the first tile's products wait for each one as they reach it (the
        // first tile stores nothing before its products, so those waits count
        // loads only).
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        int cur = 0;
        auto score_tile = [&](const int k0, auto first_tag) {
            fetch(min(k0 + 64, cvis - 1));                   // in flight while this tile is scored
            if constexpr (!decltype(first_tag)::value) flush();
            if (k0 <= wmax) {                                // uniform: some row of the wave sees the tile
                v8i bk[4];
                float sk[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    bk[u] = load_split32(k_s[cur] + (16 * u + col) * KSTR, kg);
                    sk[u] = ks_s[cur][16 * u + col];
                }
                float acc[RG][16];
#pragma unroll
                for (int g = 0; g < RG; ++g)
#pragma unroll
                    for (int j = 0; j < 16; ++j) acc[g][j] = 0.0f;
                // product j = (4h + u) * RG + g.  Software pipeline: product j + 1
                // is issued before the ReLU-weight fold of product j, so the
                // matrix core works through one product while the vector ALU
                // folds the one before; head h + 1's weights are read while head
                // h is folded.  One scheduling region per product.
                constexpr int NP = 64 * RG;
                const float* wrow = &w_s[16 * wave * RG + 4 * kg];
                v4f wv[RG], wn[RG];
#pragma unroll
                for (int g = 0; g < RG; ++g) wn[g] = wv[g] = *reinterpret_cast<const v4f*>(wrow + 16 * g);
                v4f dcur = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[0][0], bk[0], zero4, 0, 0, 0, 127, 0, 127);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 1; j <= NP; ++j) {
                    v4f dnext = zero4;
                    if (j < NP) {
                        const int g = j % RG, u = (j / RG) & 3, h = j / (4 * RG);
                        dnext = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[g][h], bk[u], zero4, 0, 0, 0,
                                                                                 127, 0, 127);
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    }
                    const int jp = j - 1;
                    const int gp = jp % RG, up = (jp / RG) & 3, hp = jp / (4 * RG);
                    if (jp % (4 * RG) == 0 && hp + 1 < 16) {      // the next head's weights
#pragma unroll
                        for (int g = 0; g < RG; ++g)
                            wn[g] = *reinterpret_cast<const v4f*>(wrow + (hp + 1) * kQ16Q + 16 * g);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[gp][4 * up + i] = fmaf(wv[gp][i], relu(dcur[i]), acc[gp][4 * up + i]);
                    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (jp % (4 * RG) == 4 * RG - 1) {
#pragma unroll
                        for (int g = 0; g < RG; ++g) wv[g] = wn[g];
                    }
                    dcur = dnext;
                }
                const bool fast = k0 + 63 < c1 && k0 + 63 <= wmin;   // uniform: every key of every row
                hbase = static_cast<uint32_t>(k0 + 4 * col) * 4u;
                hall = fast && vec_rows;
#pragma unroll
                for (int g = 0; g < RG; ++g) {
                    if (fast) {
                        hmask[g] = 0xFFFFu;                  // for rows not 16-byte aligned
#pragma unroll
                        for (int u = 0; u < 4; ++u)
#pragma unroll
                            for (int i = 0; i < 4; ++i) held[g][4 * u + i] = acc[g][4 * u + i] * sk[u];
                    } else {
                        hmask[g] = 0u;
#pragma unroll
                        for (int u = 0; u < 4; ++u)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int sidx = k0 + 4 * col + u;
                                const bool vis = sidx <= pos[g][i];
                                held[g][4 * u + i] = vis ? acc[g][4 * u + i] * sk[u] : -__builtin_inff();
                                hmask[g] |= (sidx < c1 && (vis || write_future)) ? 1u << (4 * u + i) : 0u;
                            }
                    }
                }
            } else {                                         // no row of the wave sees the tile
                hbase = static_cast<uint32_t>(k0 + 4 * col) * 4u;
                hall = false;
#pragma unroll
                for (int g = 0; g < RG; ++g) {
                    hmask[g] = 0u;
#pragma unroll
                    for (int u = 0; u < 4; ++u)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            held[g][4 * u + i] = -__builtin_inff();
                            hmask[g] |= (write_future && k0 + 4 * col + u < c1) ? 1u << (4 * u + i) : 0u;
                        }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            stage(cur ^ 1);
            __syncthreads();
            cur ^= 1;
        };
        score_tile(c0, std::true_type{});                    // c0 < cvis here
        for (int k0 = c0 + 64; k0 < cvis; k0 += 64) score_tile(k0, std::false_type{});
        flush();
        if (write_future) store_inf(cvis);                   // keys of this segment no query of the block sees
    };

    TiledWork w;
    if (!tiled_work_start<kQ16Q, kQ16Pro>(lane, nrows, base, n_k, all_keys, piece, total, w)) return;
    if (w.piece > 0) {
        run_segment(w.qb, 64 * w.t0, min(64 * min(w.t0 + w.piece, w.tj), n_k));
        return;
    }
    run_segment(w.qb, 64 * w.t0, min(64 * (w.t0 + w.ta), n_k));
    if (w.tb > 0) {
        __syncthreads();                                      // the second segment restages both LDS buffers
        run_segment(w.qb + 1, 0, min(64 * w.tb, n_k));
    }
}

// -inf for keys [e, n_k) of every row of a launch, e the end of the row's
// block's last key tile (the scorer writes the rest of the row).
__global__ void k_fill_future(float* scores, int row_off, int nrows, int kTQ, long long base, int n_k, int all_keys) {
    const int t = blockIdx.x;
    if (t >= nrows) return;
    const int tiles = tiled_block_tiles(t / kTQ, nrows, kTQ, base, n_k, all_keys != 0);
    const int e = min(64 * tiles, n_k);
    float* out = scores + static_cast<size_t>(row_off + t) * n_k;
    for (int s = e + static_cast<int>(threadIdx.x); s < n_k; s += blockDim.x) out[s] = -__builtin_inff();
}

bool index_tiled_path(const IndexArgs& a) {
    return (a.dtype == E4M3 || a.dtype == BF16) && a.H <= 16 && a.n_q >= 16;
}

// Launch of a tiled prefill kernel (query blocks of kTQ rows, `threads` per
// workgroup) over the rows of `a`; `fn` is k_index_tiled<DT> or
// k_index_fp8_q16, which take the same arguments.
typedef void (*TiledKernel)(IndexArgs, int, int, int, long long, int);

// `pro`: the kernel's prologue units per block (tiled_work_start's PRO)
static hipError_t launch_tiled(TiledKernel fn, int kTQ, int threads, int pro, int& per_cu_cache, const IndexArgs& a,
                               bool write_future, hipStream_t st) {
    // workgroups the chip holds at once
    if (per_cu_cache == 0) {
        int nb = 0;
        per_cu_cache = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(fn), threads,
                                                                    0) == hipSuccess && nb > 0 ? nb : 1;
    }
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const long long slots = static_cast<long long>(per_cu_cache) * (cus > 0 ? cus : 1);
    // one launch per sequence the rows touch, so a query block never spans two
    int r = a.row0;
    const int r_end = a.row0 + a.rows;
    while (r < r_end) {
        const int seq_end = (r / a.n_q + 1) * a.n_q;
        const int n = min(r_end, seq_end) - r;
        const long long base = static_cast<long long>(a.n_k) - a.n_q + r % a.n_q;
        const bool all_keys = a.q_pos != nullptr;
        const int nqb = (n + kTQ - 1) / kTQ;
        // (runs are cut over tiles plus `pro` prologue units per block with tiles)
        long long total = 0;
        for (int j = 0; j < nqb; ++j) {
            const int tj = tiled_block_tiles(j, n, kTQ, base, a.n_k, all_keys);
            total += tj > 0 ? tj + pro : 0;
        }
        if (total > 0) {
            // Few blocks (a fused row block): equal runs, one per resident
            // workgroup, when no block with keys is shorter than a run (a run
            // then crosses at most one block boundary).  Otherwise pieces of
            // kTiledPiece tiles over several rounds, longest blocks first.
            long long wgs = (total + kTiledMinRun - 1) / kTiledMinRun;
            if (wgs > slots) wgs = slots;
            const long long run = (total + wgs - 1) / wgs;
            int shortest = INT_MAX;
            for (int j = 0; j < nqb; ++j) {
                const int tj = tiled_block_tiles(j, n, kTQ, base, a.n_k, all_keys);
                if (tj > 0 && tj + pro < shortest) shortest = tj + pro;
            }
            long long piece = 0;
            if (nqb * 2 > slots || run > shortest) {
                piece = kTiledPiece;
                wgs = 0;
                for (int j = 0; j < nqb; ++j) wgs += (tiled_block_tiles(j, n, kTQ, base, a.n_k, all_keys) + piece - 1) / piece;
            }
            hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(wgs)), dim3(threads), 0, st, a, r, n,
                               static_cast<int>(piece), total, write_future ? 1 : 0);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        if (write_future && !all_keys) {
            hipLaunchKernelGGL(k_fill_future, dim3(n), dim3(256), 0, st, a.scores, r - a.row0, n, kTQ, base, a.n_k, 0);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        r += n;
    }
    return hipSuccess;
}

#ifndef DSA_TILED_FP8_Q16
#define DSA_TILED_FP8_Q16 1
#endif
hipError_t launch_index_tiled(const IndexArgs& a, bool write_future, hipStream_t st) {
    static int occ_q16 = 0, occ_f8 = 0, occ_bf = 0;
    if (a.dtype == E4M3) {
        if (DSA_TILED_FP8_Q16)
            return launch_tiled(k_index_fp8_q16, kQ16Q, kQ16W * 64, kQ16Pro, occ_q16, a, write_future, st);
        constexpr int tw = TiledShape<E4M3>::TW;
        return launch_tiled(k_index_tiled<E4M3>, TiledShape<E4M3>::QPW * tw, tw * 64, 0, occ_f8, a, write_future, st);
    }
    constexpr int tw = TiledShape<BF16>::TW;
    return launch_tiled(k_index_tiled<BF16>, TiledShape<BF16>::QPW * tw, tw * 64, 0, occ_bf, a, write_future, st);
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
template <int DT>
static hipError_t launch_generic_dt(const IndexArgs& a, hipStream_t st) {
    dim3 grid((a.n_k + 255) / 256, a.rows);
    if (a.H <= 4)
        hipLaunchKernelGGL((k_index_generic<DT, 4>), grid, dim3(256), 0, st, a.iq, a.iq_scale, a.ik,
                           a.ik_scale, a.iw, a.q_pos, a.row0, a.n_q, a.n_k, a.H, a.scores);
    else if (a.H <= 16)
        hipLaunchKernelGGL((k_index_generic<DT, 16>), grid, dim3(256), 0, st, a.iq, a.iq_scale, a.ik,
                           a.ik_scale, a.iw, a.q_pos, a.row0, a.n_q, a.n_k, a.H, a.scores);
    else
        hipLaunchKernelGGL((k_index_generic<DT, 64>), grid, dim3(256), 0, st, a.iq, a.iq_scale, a.ik,
                           a.ik_scale, a.iw, a.q_pos, a.row0, a.n_q, a.n_k, a.H, a.scores);
    return hipGetLastError();
}

bool index_fp8_path(const IndexArgs& a) {
    return a.dtype == E4M3 && a.H <= 16;
}

bool index_fills_hist(const IndexArgs& a) { return index_fp8_path(a) && !index_tiled_path(a); }

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t st) {
    if (index_tiled_path(a)) return launch_index_tiled(a, !a.visible_only, st);
    if (index_fp8_path(a)) {
        const int kpb = DSA_IDX_KPB;
        dim3 grid((a.n_k + kpb - 1) / kpb, a.rows);
        hipLaunchKernelGGL((k_index_fp8_mfma<DSA_IDX_U, false>), grid,
                           dim3(DSA_IDX_WAVES * 64), 0, st, a, kpb);
        return hipGetLastError();
    }
    switch (a.dtype) {
        case F32: return launch_generic_dt<F32>(a, st);
        case BF16: return launch_generic_dt<BF16>(a, st);
        default: return launch_generic_dt<E4M3>(a, st);
    }
}

hipError_t launch_index_candidates(const IndexArgs& a, hipStream_t st) {
    const int kpb = DSA_IDX_KPB;
    dim3 grid((a.n_k + kpb - 1) / kpb, a.rows);
    hipLaunchKernelGGL((k_index_fp8_mfma<DSA_IDX_U, true>), grid,
                       dim3(DSA_IDX_WAVES * 64), 0, st, a, kpb);
    return hipGetLastError();
}

}  // namespace dsa
