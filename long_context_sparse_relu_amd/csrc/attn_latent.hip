// attn_latent.hip -- attention over the selected rows of a shared latent KV
// cache (one 576-wide row per token, the value being its first 512 entries),
// bf16, many query heads per row: the 1M-token decode shape.
//
// The main attention runs over the k kept rows only ("DeepSeek-V3.2-Exp
// 稀疏注意力机制(DSA)技术深度解析", sheratonhq.com, section 1); at 1M tokens the
// pages keep k = 256..512 ("DeepSeek-V4 百万 token 上下文的工程实现",
// blog.hotdry.top, section "从 O(N²) 到 O(N・k)").
//
// Every query head reads the same selected rows, so one workgroup serves up
// to 128 heads of a (query row, slice of the index list): 8 waves of 16 heads.
// Per tile of 16 selected rows:
//   the tile (16 x 1152 B) is gathered once into LDS by all 512 threads (the
//     next tile is in flight in registers while the current one is used);
//   S^T[key][head] = K Q^T with 18 v_mfma_f32_16x16x32_bf16 per wave: A = the
//     tile rows from LDS (lane l: key l%16, dims 32c + 8(l/16)..+7), B = Q^T in
//     registers; lane l ends with keys 4(l/16)+v of head l%16;
//   online softmax per lane in fp32, base 2;
//   O^T[dim][head] += V^T P^T with 32 v_mfma_f32_16x16x16bf16_1k: the V^T
//     operand is read from the same tile with ds_read_b64_tr_b16 (lane (g, c)
//     addresses row 4g + c/4 at dims 16t + 4(c%4)), P^T is the softmax output
//     in place.
// With several slices per row the (max, sum, O) records are merged by
// k_attn_merge.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kLatDqk = 576, kLatDv = 512;
constexpr int kLatWaves = 8;                      // 16 heads each: 128 heads per workgroup
constexpr int kLatKeys = 16;                      // selected rows per tile
constexpr int kLatStr = kLatDqk + 8;              // LDS row stride (bf16): 1168 B
constexpr int kLatChunks = kLatKeys * kLatDqk / 8;   // 16-byte pieces per tile: 1152
constexpr int kLatThreads = kLatWaves * 64;
constexpr int kLatPer = (kLatChunks + kLatThreads - 1) / kLatThreads;   // 3
}

__global__ __launch_bounds__(kLatThreads) void k_attn_latent(AttnArgs a, int nsplit, int hgroups, int slice_len,
                                                             float* part) {
    __shared__ __align__(16) uint16_t tile[2][kLatKeys * kLatStr];          // 37376 B
    extern __shared__ int32_t idx_s[];                                     // [slice_len]

    const int unit = blockIdx.x;                   // (row, head group, slice)
    const int split = unit % nsplit;
    const int hg = (unit / nsplit) % hgroups;
    const int row = unit / (nsplit * hgroups);
    const int G = a.Hq;                            // one latent row serves every head (Hkv = 1)
    const int b = row / a.n_q;
    const int pos = row_pos(a.q_pos, row, a.n_q, a.n_k);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;
    const int kg = lane >> 4;
    const int head0 = hg * 128 + wave * 16;
    const bool active = head0 < G;                 // wave-uniform
    const float zscale = a.scale * kLog2e;

    const int jb = split * slice_len;
    const int nj = max(0, min(slice_len, a.kk - jb));
    const int32_t* idx_row = a.idx + static_cast<size_t>(row) * a.kk + jb;
    for (int j = threadIdx.x; j < nj; j += kLatThreads) idx_s[j] = idx_row[j];

    // Q^T operand of chunk c: head head0 + col, dims 32c + 8kg .. +7 (zero for heads >= G)
    const uint16_t* qp = static_cast<const uint16_t*>(a.q);
    const int hq = min(head0 + col, G - 1);
    v8bf qb[kLatDqk / 32];
#pragma unroll
    for (int c = 0; c < kLatDqk / 32; ++c) {
        const v8bf x = *reinterpret_cast<const v8bf*>(qp + (static_cast<size_t>(row) * G + hq) * kLatDqk + 32 * c +
                                                      8 * kg);
        qb[c] = (head0 + col < G) ? x : v8bf{};
    }
    __syncthreads();                               // idx_s is ready

    const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + static_cast<size_t>(b) * a.n_k * kLatDqk;
    const int ntiles = (nj + kLatKeys - 1) / kLatKeys;

    // loader: piece i of a tile = key i / 72, bytes 16 (i % 72); an invalid
    // entry (past the slice, < 0 or > pos) reads row 0 and is stored as zeros
    v4i pf[kLatPer];
    uint32_t pvalid = 0;
    auto fetch = [&](int t) {
#pragma unroll
        for (int u = 0; u < kLatPer; ++u) {
            const int i = min(static_cast<int>(threadIdx.x) + u * kLatThreads, kLatChunks - 1);
            const int key = i / (kLatDqk / 8), piece = i % (kLatDqk / 8);
            const int j = t * kLatKeys + key;
            const int s = idx_s[min(j, nj - 1)];
            const bool ok = j < nj && s >= 0 && s <= pos;
            pvalid = ok ? (pvalid | (1u << u)) : (pvalid & ~(1u << u));
            pf[u] = *reinterpret_cast<const v4i*>(kbase + static_cast<size_t>(ok ? s : 0) * kLatDqk + 8 * piece);
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int u = 0; u < kLatPer; ++u) {
            const int i = static_cast<int>(threadIdx.x) + u * kLatThreads;
            if (i < kLatChunks) {
                const int key = i / (kLatDqk / 8), piece = i % (kLatDqk / 8);
                *reinterpret_cast<v4i*>(&tile[buf][key * kLatStr + 8 * piece]) =
                    ((pvalid >> u) & 1u) ? pf[u] : v4i{0, 0, 0, 0};
            }
        }
    };

    float m_run = -__builtin_inff();
    float l_part = 0.0f;
    v4f o[kLatDv / 16];
#pragma unroll
    for (int t = 0; t < kLatDv / 16; ++t) o[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    if (ntiles > 0) {
        fetch(0);
        stage(0);
    }
    __syncthreads();
    int buf = 0;
    for (int t = 0; t < ntiles; ++t) {
        if (t + 1 < ntiles) fetch(t + 1);          // in flight during the multiply (uniform branch)
        const uint16_t* ks = tile[buf];
        if (active) {
            // the validity of keys 4kg..4kg+3 of this tile, for this lane's scores
            bool kv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int j = t * kLatKeys + 4 * kg + v;
                const int s = idx_s[min(j, nj - 1)];
                kv[v] = j < nj && s >= 0 && s <= pos;
            }
            v4f sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int c = 0; c < kLatDqk / 32; ++c) {
                const v8bf kr = *reinterpret_cast<const v8bf*>(ks + col * kLatStr + 32 * c + 8 * kg);
                sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr, qb[c], sacc, 0, 0, 0);
            }
            float sv[4];
            float bm = -__builtin_inff();
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                sv[v] = kv[v] ? sacc[v] * zscale : -__builtin_inff();
                bm = fmaxf(bm, sv[v]);
            }
            bm = wave_max_xor_16_32(bm);
            const float m_new = fmaxf(m_run, bm);
            float corr = 1.0f;
            float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (m_new != -__builtin_inff()) {
                corr = exp2f(m_run - m_new);
#pragma unroll
                for (int v = 0; v < 4; ++v) p[v] = exp2f(sv[v] - m_new);
            }
            l_part = l_part * corr + (p[0] + p[1] + p[2] + p[3]);
            m_run = m_new;
            v4bf pb;
#pragma unroll
            for (int v = 0; v < 4; ++v) pb[v] = static_cast<__bf16>(p[v]);
            const uint16_t* trp = ks + (4 * kg + (col >> 2)) * kLatStr + 4 * (col & 3);
#pragma unroll
            for (int d = 0; d < kLatDv / 16; ++d) {
                const v4bf va = lds_read_tr16(trp + 16 * d);
                o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[d] * corr, 0, 0, 0);
            }
        }
        if (t + 1 < ntiles) stage(buf ^ 1);        // the other buffer was last read before the previous barrier
        __syncthreads();
        buf ^= 1;
    }

    if (!active) return;
    const float l_tot = wave_sum_xor_16_32(l_part);
    if (head0 + col >= G) return;
    const int h = head0 + col;
    const size_t rh = static_cast<size_t>(row) * G + h;
    // o[d][i] = O^T[dim 16d + 4kg + i][head col]
    if (nsplit == 1) {
        uint16_t* outp = static_cast<uint16_t*>(a.out) + rh * kLatDv;
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
        for (int d = 0; d < kLatDv / 16; ++d)
#pragma unroll
            for (int i = 0; i < 4; ++i) outp[16 * d + 4 * kg + i] = f32_to_bf16_bits(o[d][i] * inv);
        if (kg == 0 && a.lse) a.lse[rh] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * kLn2 : -__builtin_inff();
        return;
    }
    float* rec = part + (rh * nsplit + split) * (kLatDv + 2);
    if (kg == 0) { rec[0] = m_run; rec[1] = l_tot; }
#pragma unroll
    for (int d = 0; d < kLatDv / 16; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) rec[2 + 16 * d + 4 * kg + i] = o[d][i];
}

bool attn_latent_eligible(const AttnArgs& a) {
    return a.dtype == BF16 && a.kv_dtype == BF16 && a.latent && a.Hkv == 1 && a.dqk == kLatDqk && a.dv == kLatDv;
}

#ifndef DSA_LATENT_TILES_PER_SLICE
#define DSA_LATENT_TILES_PER_SLICE 4
#endif
// Slices of the index list per (row, head group): about 4 tiles each (2, 8 and
// 16 measured slower on 8 rows x 512 selected rows; up to 17 tiles per slice
// measured the same on 8704), at most 32 (64 measured slower: the records
// to merge double), and none when the rows alone fill the chip.
int attn_latent_splits(const AttnArgs& a) {
    const int hgroups = (a.Hq + 127) / 128;
    const int64_t units = static_cast<int64_t>(a.rows) * hgroups;
    if (units >= 256) return 1;
    int s = (a.kk + kLatKeys * DSA_LATENT_TILES_PER_SLICE - 1) / (kLatKeys * DSA_LATENT_TILES_PER_SLICE);
    if (s > 32) s = 32;
    return s < 1 ? 1 : s;
}

size_t attn_latent_workspace_bytes(const AttnArgs& a) {
    const int s = attn_latent_splits(a);
    return s > 1 ? static_cast<size_t>(a.rows) * a.Hq * s * (kLatDv + 2) * sizeof(float) : 0;
}

hipError_t launch_attn_latent(const AttnArgs& a, float* part, hipStream_t st) {
    const int s = attn_latent_splits(a);
    const int hgroups = (a.Hq + 127) / 128;
    const int slice = ((a.kk + s - 1) / s + kLatKeys - 1) / kLatKeys * kLatKeys;
    const size_t idx_lds = static_cast<size_t>(slice) * sizeof(int32_t);   // <= 64 KiB
    if (idx_lds + sizeof(uint16_t) * 2 * kLatKeys * kLatStr > 64 * 1024) {
        hipError_t e = allow_dyn_lds(reinterpret_cast<const void*>(k_attn_latent), idx_lds);
        if (e != hipSuccess) return e;
    }
    const dim3 grid(static_cast<unsigned>(a.rows) * hgroups * s);
    hipLaunchKernelGGL(k_attn_latent, grid, dim3(kLatThreads), idx_lds, st, a, s, hgroups, slice, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || s == 1) return e;
    return launch_attn_merge(a, s, part, st);
}

}  // namespace dsa
