// indexer.hip -- lightning-indexer score kernels.
//
// I[t,s] = sum_h w[t,h] * ReLU(q_I[t,h] . k_I[s]) for s <= pos(t), -inf after.
// The indexer uses few heads, index_head_dim 128, ReLU in place of softmax and
// FP8 arithmetic ("DeepSeek-V3.2-Exp 稀疏注意力机制(DSA)技术深度解析",
// sheratonhq.com, section 1).  With E4M3 inputs the per-token scales are
// positive, so they factor out of the ReLU: I = sq[t]*sk[s]*sum_h w*ReLU(c_q.c_k)
// where c are the decoded codes; the code products are exact in fp32.
#include "dsa_kernels.h"
#include "fp8_index.h"

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
// Launch shape (measured on decode_128k: register prefetch of the next step,
// other chunk sizes, wave counts and interleaved chunks were all slower or
// equal).
#ifndef DSA_IDX_U
#define DSA_IDX_U 4          // blocks of 16 keys each wave loads per step
#endif
#ifndef DSA_IDX_KPB
#define DSA_IDX_KPB 4096     // keys per workgroup
#endif
#ifndef DSA_IDX_WAVES
#define DSA_IDX_WAVES 4      // waves per workgroup
#endif
#ifndef DSA_IDX_OCC
#define DSA_IDX_OCC 8        // waves per SIMD the register budget must allow
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
    auto load_batch = [&](int base, v8i* bv, float* sk) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            bv[u] = load_split32(kb + static_cast<size_t>(min(base + u * 16 + col, lim)) * 128, kg);
#pragma unroll
        for (int g = 0; g < U / 4; ++g) sk[g] = ksb[min(base + g * 64 + lane, lim)];
    };
    auto score_batch = [&](int base, const v8i* bv, const float* sk) {
#pragma unroll
        for (int g = 0; g < U / 4; ++g) {
            const float part = fp8_score4(q, bv + 4 * g, sk[g]);
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

    for (int base = s_begin + wave * 16 * U; base < s_end; base += step) {
        v8i bv[U];
        float sk[U / 4];
        load_batch(base, bv, sk);
        score_batch(base, bv, sk);
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
// Each workgroup takes kTQ consecutive query rows of one sequence (kQPW per
// wave) and one chunk of kIdxChunk keys; the chunk's keys are staged 64 at a
// time in LDS and shared by all kTQ queries, so every key row is fetched once
// per kTQ queries, and each key operand read from LDS feeds kQPW MFMAs.  The
// next tile is fetched into registers while the current one is scored.  Per
// (query, 16 keys) the scores come from one v_mfma_scale_f32_16x16x128_f8f6f4
// (FP8) or four v_mfma_f32_16x16x32_bf16 (bf16) with the heads as M; each lane
// folds its four heads with ReLU and the head weights, and one reduce-scatter
// over the four 16-key blocks of a tile finishes the head sums, leaving lane l
// with the score of key l of the tile (one coalesced 256-byte store per query
// and tile).  Keys past a query's last visible key are written as -inf only
// when `write_future` (the unfused entry point).
// ---------------------------------------------------------------------------
#ifndef DSA_TILED_CHUNK
#define DSA_TILED_CHUNK 4096
#endif
constexpr int kIdxChunk = DSA_TILED_CHUNK;   // keys per workgroup
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

template <int DT>
__global__ __launch_bounds__(TiledShape<DT>::TW * 64) void k_index_tiled(IndexArgs x, int t_first, int nrows,
                                                                        int write_future) {
    constexpr int kQPW = TiledShape<DT>::QPW, kTW = TiledShape<DT>::TW, kTQ = kQPW * kTW;
    constexpr int KROW = DT == E4M3 ? 128 : 256;           // bytes per key row
    constexpr int KSTR = KROW + 16;                         // padded LDS stride (conflict-free 16 B reads)
    constexpr int NC = DT == E4M3 ? 1 : 4;                  // MFMAs per 16 keys
    constexpr int LPT = kTileKeys * KROW / 16 / (kTW * 64); // 16-byte loads per thread per tile
    static_assert(LPT * kTW * 64 * 16 == kTileKeys * KROW, "a tile must split evenly over the threads");
    __shared__ __align__(16) uint8_t k_s[kTileKeys * KSTR];
    __shared__ float ks_s[kTileKeys];
    __shared__ int last_s[kTW];

    const int nqb = (nrows + kTQ - 1) / kTQ;
    const int qb = nqb - 1 - static_cast<int>(blockIdx.y);  // longest query blocks first
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, kg = lane >> 4;
    const int n_k = x.n_k, H = x.H;

    // this wave's query rows (absolute row index t_first + qb*kTQ + kQPW*wave + q)
    int rows[kQPW], pos[kQPW];
    float w[kQPW][4], sq[kQPW];
    v8i a8[DT == E4M3 ? kQPW : 1];
    v8bf a16[DT == E4M3 ? 1 : kQPW][4];
    unsigned livem = 0;                                      // bit q: row q exists
    int mp = -1;
#pragma unroll
    for (int q = 0; q < kQPW; ++q) {
        const int lr = qb * kTQ + wave * kQPW + q;          // row within the launch
        const bool live = lr < nrows;
        livem |= live ? 1u << q : 0u;
        rows[q] = t_first + (live ? lr : 0);
        pos[q] = live ? row_pos(x.q_pos, rows[q], x.n_q, n_k) : -1;  // may be negative for a live row
        mp = max(mp, pos[q]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = 4 * kg + i;
            w[q][i] = (live && h < H) ? x.iw[static_cast<size_t>(rows[q]) * H + h] : 0.0f;
        }
        if constexpr (DT == E4M3) {
            sq[q] = live ? x.iq_scale[rows[q]] : 0.0f;
            a8[q] = (live && col < H)
                ? load_split32(static_cast<const uint8_t*>(x.iq) + (static_cast<size_t>(rows[q]) * H + col) * 128, kg)
                : v8i{0, 0, 0, 0, 0, 0, 0, 0};
        } else {
            sq[q] = 1.0f;
            const uint16_t* qrow = static_cast<const uint16_t*>(x.iq) + (static_cast<size_t>(rows[q]) * H + col) * 128 + kg * 32;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                a16[q][c] = (live && col < H) ? *reinterpret_cast<const v8bf*>(qrow + c * 8) : v8bf{};
        }
    }
    mp = max(mp, __shfl_xor(mp, 16));
    mp = max(mp, __shfl_xor(mp, 32));
    if (lane == 0) last_s[wave] = mp;
    __syncthreads();
    int last = last_s[0];
#pragma unroll
    for (int i = 1; i < kTW; ++i) last = max(last, last_s[i]);
    const int b = t_first / x.n_q;                           // every row of the launch is in sequence b
    const int c0 = blockIdx.x * kIdxChunk;
    const int c1 = min(c0 + kIdxChunk, n_k);
    const int cvis = min(c1, last + 1);                      // keys some query of the block sees
    const uint8_t* kb = static_cast<const uint8_t*>(x.ik) + static_cast<size_t>(b) * n_k * KROW;
    const float* ksb = DT == E4M3 ? x.ik_scale + static_cast<size_t>(b) * n_k : nullptr;

    v4i pre[LPT];
    float pre_s = 0.0f;
    auto fetch = [&](int k0) {
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int i = threadIdx.x + u * kTW * 64;
            const int kr = i / (KROW / 16), off = (i % (KROW / 16)) * 16;
            const int key = k0 + kr;
            pre[u] = key < n_k ? *reinterpret_cast<const v4i*>(kb + static_cast<size_t>(key) * KROW + off)
                               : v4i{0, 0, 0, 0};
        }
        if constexpr (DT == E4M3) {
            const int key = k0 + threadIdx.x;
            pre_s = (threadIdx.x < kTileKeys && key < n_k) ? ksb[key] : 0.0f;
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            const int i = threadIdx.x + u * kTW * 64;
            const int kr = i / (KROW / 16), off = (i % (KROW / 16)) * 16;
            *reinterpret_cast<v4i*>(k_s + kr * KSTR + off) = pre[u];
        }
        if (DT == E4M3 && threadIdx.x < kTileKeys) ks_s[threadIdx.x] = pre_s;
    };

    if (c0 < cvis) {
        fetch(c0);
        stage();
    }
    // every prologue load (queries, weights, positions) has landed: otherwise
    // the loop's first MFMA waits on all outstanding memory operations,
    // including the previous tile's score stores, in every iteration
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int k0 = c0; k0 < cvis; k0 += kTileKeys) {
        const bool more = k0 + kTileKeys < cvis;
        if (more) fetch(k0 + kTileKeys);                     // in flight while this tile is scored
#pragma unroll
        for (int sub = 0; sub < kTileKeys / 64; ++sub) {
        // key k0 + 64*sub + g16*16 + col sits in LDS row 64*sub + g16*16 + col;
        // lane l scores key k0 + 64*sub + l
        v8i b8[4];
        v8bf b16[4][4];
#pragma unroll
        for (int g16 = 0; g16 < 4; ++g16) {
            const uint8_t* kr = k_s + (sub * 64 + g16 * 16 + col) * KSTR;
            if constexpr (DT == E4M3) {
                b8[g16] = load_split32(kr, kg);
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) b16[g16][c] = *reinterpret_cast<const v8bf*>(kr + kg * 64 + c * 16);
            }
        }
        const int s = k0 + sub * 64 + lane;
        const float sk = DT == E4M3 ? ks_s[sub * 64 + lane] : 1.0f;
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
            if (s < c1 && (livem >> q & 1u)) {
                float* out = x.scores + static_cast<size_t>(rows[q] - x.row0) * n_k;
                if (s <= pos[q]) out[s] = DT == E4M3 ? part * (sq[q] * sk) : part;
                else if (write_future) out[s] = -__builtin_inff();
            }
        }
        }
        if (more) {
            __syncthreads();                                 // every wave is done with this tile
            stage();
        }
        __syncthreads();
    }
    if (write_future) {
        // keys of this chunk no query of the block sees
        for (int q = 0; q < kQPW; ++q) {
            if (!(livem >> q & 1u)) continue;
            float* out = x.scores + static_cast<size_t>(rows[q] - x.row0) * n_k;
            for (int s = max(c0, cvis) + lane; s < c1; s += 64) out[s] = -__builtin_inff();
        }
    }
}

bool index_tiled_path(const IndexArgs& a) {
    return (a.dtype == E4M3 || a.dtype == BF16) && a.H <= 16 && a.n_q >= 16;
}

template <int DT>
static hipError_t launch_index_tiled_dt(const IndexArgs& a, bool write_future, hipStream_t st) {
    constexpr int kTW = TiledShape<DT>::TW, kTQ = TiledShape<DT>::QPW * kTW;
    // one launch per sequence the rows touch, so a query block never spans two
    int r = a.row0;
    const int r_end = a.row0 + a.rows;
    while (r < r_end) {
        const int seq_end = (r / a.n_q + 1) * a.n_q;
        const int n = min(r_end, seq_end) - r;
        const dim3 grid((a.n_k + kIdxChunk - 1) / kIdxChunk, (n + kTQ - 1) / kTQ);
        hipLaunchKernelGGL(k_index_tiled<DT>, grid, dim3(kTW * 64), 0, st, a, r, n, write_future ? 1 : 0);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        r += n;
    }
    return hipSuccess;
}

hipError_t launch_index_tiled(const IndexArgs& a, bool write_future, hipStream_t st) {
    return a.dtype == E4M3 ? launch_index_tiled_dt<E4M3>(a, write_future, st)
                           : launch_index_tiled_dt<BF16>(a, write_future, st);
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
