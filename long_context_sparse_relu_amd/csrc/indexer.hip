// indexer.hip -- lightning-indexer score kernels.
//
// I[t,s] = sum_h w[t,h] * ReLU(q_I[t,h] . k_I[s]) for s <= pos(t), -inf after.
// The indexer uses few heads, index_head_dim 128, ReLU in place of softmax and
// FP8 arithmetic ("DeepSeek-V3.2-Exp 稀疏注意力机制(DSA)技术深度解析",
// sheratonhq.com, section 1).  With E4M3 inputs the per-token scales are
// positive, so they factor out of the ReLU: I = sq[t]*sk[s]*sum_h w*ReLU(c_q.c_k)
// where c are the decoded codes; the code products are exact in fp32.
#include "dsa_device.h"
#include "dsa_kernels.h"

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
// FP8 streaming path (decode and any row count): up to 16 heads, d = 128.
// One v_mfma_scale_f32_16x16x128_f8f6f4 multiplies the query row's 16 heads
// (rows of A) by 16 keys (columns of B) over the full 128-wide dot product.
// Lane l feeds A row l%16 and B column l%16 with 32 code bytes: bytes
// [16g, 16g+16) and [64+16g, 64+16g+16) of the row, g = l/16.  A and B use the
// same byte->k assignment, so the contraction is exact whatever order the
// unit sums in, and each 16-byte load instruction of a wave covers 64
// contiguous bytes of every key row it touches.  The 16x16 result lands as
// acc[i] = dot(head 4g+i, key l%16): ReLU, head weight, then two cross-lane
// adds finish the head reduction.  Keys stream from HBM once; each wave keeps
// U blocks of 16 keys in flight.  When `hist` is given, the workgroup also
// counts the top 11 bits of each visible score's order key in LDS and adds its
// non-empty bins to the row's histogram, which saves the top-k a pass.
// ---------------------------------------------------------------------------
typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v8i load_split32(const uint8_t* row, int g) {
    v4i lo = *reinterpret_cast<const v4i*>(row + 16 * g);
    v4i hi = *reinterpret_cast<const v4i*>(row + 64 + 16 * g);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int U>
__global__ __launch_bounds__(256) void k_index_fp8_mfma(
    const uint8_t* __restrict__ iq, const float* __restrict__ iq_scale,
    const uint8_t* __restrict__ ik, const float* __restrict__ ik_scale,
    const float* __restrict__ iw, const int32_t* __restrict__ q_pos,
    int row0, int n_q, int n_k, int H, int keys_per_block, float* __restrict__ scores,
    uint32_t* __restrict__ hist)
{
    __shared__ uint32_t lh[kTopkBins];
    const int row = row0 + blockIdx.y;
    const int b = row / n_q;
    const int pos = row_pos(q_pos, row, n_q, n_k);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;       // A row (head) and B column (key in block)
    const int kg = lane >> 4;        // which byte slices of the 128-byte rows

    if (hist) {
        for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x) lh[i] = 0u;
    }
    v8i a = {0, 0, 0, 0, 0, 0, 0, 0};
    if (col < H) a = load_split32(iq + (static_cast<size_t>(row) * H + col) * 128, kg);
    float w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int h = 4 * kg + i;
        w[i] = h < H ? iw[static_cast<size_t>(row) * H + h] : 0.0f;
    }
    const float sq = iq_scale[row];
    const uint8_t* kb = ik + static_cast<size_t>(b) * n_k * 128;
    const float* ksb = ik_scale + static_cast<size_t>(b) * n_k;
    float* out = scores + static_cast<size_t>(blockIdx.y) * n_k;
    if (hist) __syncthreads();

    const int s_begin = blockIdx.x * keys_per_block;
    const int s_end = min(s_begin + keys_per_block, n_k);
    const int nwaves = blockDim.x >> 6;
    for (int base = s_begin + wave * 16 * U; base < s_end; base += nwaves * 16 * U) {
        v8i bv[U];
        float sk[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            int s = base + u * 16 + col;
            bool live = s < s_end && s <= pos;
            bv[u] = live ? load_split32(kb + static_cast<size_t>(s) * 128, kg)
                         : v8i{0, 0, 0, 0, 0, 0, 0, 0};
            sk[u] = live ? ksb[s] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bv[u], acc, 0, 0, 0, 127, 0, 127);
            float part = w[0] * fmaxf(acc[0], 0.0f);
            part = fmaf(w[1], fmaxf(acc[1], 0.0f), part);
            part = fmaf(w[2], fmaxf(acc[2], 0.0f), part);
            part = fmaf(w[3], fmaxf(acc[3], 0.0f), part);
            part = wave_sum_xor_16_32(part);
            int s = base + u * 16 + col;
            if (kg == 0 && s < s_end) {
                float score = s <= pos ? part * (sq * sk[u]) : -__builtin_inff();
                out[s] = score;
                if (hist && s <= pos) atomicAdd(&lh[order_key(score) >> 21], 1u);
            }
        }
    }
    if (hist) {
        __syncthreads();
        uint32_t* gh = hist + static_cast<size_t>(blockIdx.y) * kTopkBins;
        for (int i = threadIdx.x; i < kTopkBins; i += blockDim.x)
            if (lh[i]) atomicAdd(&gh[i], lh[i]);
    }
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

bool index_fills_hist(const IndexArgs& a) {
    return a.dtype == E4M3 && a.H <= 16;
}

hipError_t launch_index_scores(const IndexArgs& a, hipStream_t st) {
    if (a.dtype == E4M3 && a.H <= 16) {
        constexpr int U = 4;
        const int kpb = 4096;
        dim3 grid((a.n_k + kpb - 1) / kpb, a.rows);
        hipLaunchKernelGGL((k_index_fp8_mfma<U>), grid, dim3(256), 0, st,
                           static_cast<const uint8_t*>(a.iq), a.iq_scale,
                           static_cast<const uint8_t*>(a.ik), a.ik_scale, a.iw, a.q_pos,
                           a.row0, a.n_q, a.n_k, a.H, kpb, a.scores, a.hist);
        return hipGetLastError();
    }
    switch (a.dtype) {
        case F32: return launch_generic_dt<F32>(a, st);
        case BF16: return launch_generic_dt<BF16>(a, st);
        default: return launch_generic_dt<E4M3>(a, st);
    }
}

}  // namespace dsa
