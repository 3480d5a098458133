// attn_wide.hip -- bf16 sparse attention on MFMA for any head grouping and
// wide rows, including the shared latent row (key = the whole row, value = its
// first d_v entries).
//
// The main attention runs over the k kept rows only, O(n*k) instead of O(n^2)
// ("DeepSeek-V3.2-Exp 稀疏注意力机制(DSA)技术深度解析", sheratonhq.com,
// section 1); at 1M tokens the pages recommend k = 256..512 ("DeepSeek-V4 百万
// token 上下文的工程实现", blog.hotdry.top, section "从 O(N²) 到 O(N・k)").
//
// One wave per (query row, group of <= 16 query heads of one kv head, slice of
// the index list):
//   S^T[key][head] = K Q^T with d_qk/32 v_mfma_f32_16x16x32_bf16 per 16 keys:
//     lane l holds key l%16 (A) and head l%16 (B) over the same contiguous
//     d_qk/4 dims at (l/16)*d_qk/4, so A and B agree on the k order;
//   the online softmax is per lane (head l%16) in fp32, base 2;
//   O^T[dim][head] += V^T P^T with d_v/16 v_mfma_f32_16x16x16_bf16: the 16
//     value rows are staged in LDS (for latent rows straight from the key
//     registers) and read transposed, P^T is the softmax output in place.
// With several slices per row, each wave leaves (max, sum, O) in the
// workspace and a merge kernel combines them; one slice writes out directly.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
}

template <int NC, int NT>   // d_qk = 32*NC, d_v = 16*NT
__global__ __launch_bounds__(64) void k_attn_bf16_split(AttnArgs a, int nsplit, int hgroups, float* part) {
    constexpr int DQK = 32 * NC, DV = 16 * NT;
    constexpr int PER_LANE = DQK / 4;          // contiguous dims each lane holds of a row
    constexpr int VSTR = DV + 8;               // staged value row stride (bf16)
    __shared__ __align__(16) uint16_t v_s[16 * VSTR];

    const int split = blockIdx.x;
    const int g = blockIdx.y / hgroups;        // kv head
    const int hg = blockIdx.y % hgroups;       // group of 16 query heads within it
    const int row = blockIdx.z;
    const int G = a.Hq / a.Hkv;
    const int head0 = g * G + hg * 16;
    const int nh = min(16, G - hg * 16);
    const int b = row / a.n_q;
    const int pos = row_pos(a.q_pos, row, a.n_q, a.n_k);
    const int lane = threadIdx.x;
    const int col = lane & 15;
    const int kg = lane >> 4;
    const float zscale = a.scale * kLog2e;

    const uint16_t* qp = static_cast<const uint16_t*>(a.q);
    const uint16_t* kp = static_cast<const uint16_t*>(a.k);
    const uint16_t* vp = static_cast<const uint16_t*>(a.v);
    v8bf qb[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (col < nh)
            qb[c] = *reinterpret_cast<const v8bf*>(qp + (static_cast<size_t>(row) * a.Hq + head0 + col) * DQK +
                                                   kg * PER_LANE + c * 8);
        else
            qb[c] = v8bf{};
    }

    const int per = ((a.kk + nsplit * 16 - 1) / (nsplit * 16)) * 16;
    const int j_begin = split * per;
    const int j_end = min(j_begin + per, a.kk);
    const int32_t* idx_row = a.idx + static_cast<size_t>(row) * a.kk;
    const size_t k_row = static_cast<size_t>(a.Hkv) * DQK;
    const size_t v_row = static_cast<size_t>(a.Hkv) * DV;
    const uint16_t* kbase = kp + static_cast<size_t>(b) * a.n_k * k_row + g * DQK + kg * PER_LANE;

    float m_run = -__builtin_inff();
    float l_part = 0.0f;
    v4f o[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) o[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    int s_next = -1;
    if (j_begin < j_end) {
        int j = j_begin + col;
        s_next = j < j_end ? idx_row[j] : -1;
    }
    for (int j0 = j_begin; j0 < j_end; j0 += 16) {
        const int s = s_next;
        if (j0 + 16 < j_end) {                 // next block's positions, one round trip ahead
            int j = j0 + 16 + col;
            s_next = j < j_end ? idx_row[j] : -1;
        }
        const bool valid = s >= 0 && s <= pos;
        v8bf kr[NC];
        if (valid) {
            const v8bf* ks = reinterpret_cast<const v8bf*>(kbase + static_cast<size_t>(s) * k_row);
#pragma unroll
            for (int c = 0; c < NC; ++c) kr[c] = ks[c];
        } else {
#pragma unroll
            for (int c = 0; c < NC; ++c) kr[c] = v8bf{};
        }
        v4f sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < NC; ++c) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[c], qb[c], sacc, 0, 0, 0);

        // stage the value rows: lane (key col, dims of group kg)
        if (a.latent) {
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int d = kg * PER_LANE + c * 8;
                if (d < DV) *reinterpret_cast<v8bf*>(v_s + col * VSTR + d) = kr[c];
            }
        } else {
            constexpr int VPL = DV / 4;        // value dims per lane
            const v8bf* vs = reinterpret_cast<const v8bf*>(vp + (static_cast<size_t>(b) * a.n_k + (valid ? s : 0)) * v_row +
                                                          g * DV + kg * VPL);
#pragma unroll
            for (int c = 0; c < VPL / 8; ++c)
                *reinterpret_cast<v8bf*>(v_s + col * VSTR + kg * VPL + c * 8) = valid ? vs[c] : v8bf{};
        }

        const uint64_t vm = __ballot(valid);
        float sv[4];
        float bm = -__builtin_inff();
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int slot = 4 * kg + v;
            sv[v] = ((vm >> slot) & 1ull) ? sacc[v] * zscale : -__builtin_inff();
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
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        v4bf pb;
#pragma unroll
        for (int v = 0; v < 4; ++v) pb[v] = static_cast<__bf16>(p[v]);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            o[t] *= corr;
            v4bf va;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                va[v] = *reinterpret_cast<const __bf16*>(v_s + (4 * kg + v) * VSTR + 16 * t + col);
            o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[t], 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    const float l_tot = wave_sum_xor_16_32(l_part);
    if (col >= nh) return;
    const int h = head0 + col;
    if (nsplit == 1) {
        uint16_t* outp = static_cast<uint16_t*>(a.out) + (static_cast<size_t>(row) * a.Hq + h) * DV;
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) outp[16 * t + 4 * kg + v] = f32_to_bf16_bits(o[t][v] * inv);
        if (kg == 0 && a.lse)
            a.lse[static_cast<size_t>(row) * a.Hq + h] =
                l_tot > 0.0f ? (m_run + log2f(l_tot)) * kLn2 : -__builtin_inff();
        return;
    }
    // partial record of this slice: m, l, then O (unnormalised, relative to m)
    float* rec = part + ((static_cast<size_t>(row) * a.Hq + h) * nsplit + split) * (DV + 2);
    if (kg == 0) { rec[0] = m_run; rec[1] = l_tot; }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) rec[2 + 16 * t + 4 * kg + v] = o[t][v];
}

// Combine the slices of each (row, head): out = sum_s O_s 2^(m_s - M) / L.
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a, int nsplit, const float* part) {
    const int rh = blockIdx.x;                 // row * Hq + head
    const int dv = a.dv;
    const float* rec0 = part + static_cast<size_t>(rh) * nsplit * (dv + 2);
    float M = -__builtin_inff();
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, rec0[static_cast<size_t>(s) * (dv + 2)]);
    float L = 0.0f;
    if (M != -__builtin_inff())
        for (int s = 0; s < nsplit; ++s) {
            const float* r = rec0 + static_cast<size_t>(s) * (dv + 2);
            if (r[0] != -__builtin_inff()) L += r[1] * exp2f(r[0] - M);
        }
    uint16_t* outp = static_cast<uint16_t*>(a.out) + static_cast<size_t>(rh) * dv;
    for (int d = threadIdx.x; d < dv; d += blockDim.x) {
        float O = 0.0f;
        if (M != -__builtin_inff())
            for (int s = 0; s < nsplit; ++s) {
                const float* r = rec0 + static_cast<size_t>(s) * (dv + 2);
                if (r[0] != -__builtin_inff()) O += r[2 + d] * exp2f(r[0] - M);
            }
        outp[d] = f32_to_bf16_bits(L > 0.0f ? O / L : 0.0f);
    }
    if (threadIdx.x == 0 && a.lse) a.lse[rh] = L > 0.0f ? (M + log2f(L)) * kLn2 : -__builtin_inff();
}

hipError_t launch_attn_merge(const AttnArgs& a, int nsplit, const float* part, hipStream_t st) {
    hipLaunchKernelGGL(k_attn_merge, dim3(a.rows * a.Hq), dim3(256), 0, st, a, nsplit, part);
    return hipGetLastError();
}

// Shapes with an instantiated kernel.
static bool wide_shape(int dqk, int dv) {
    return (dqk == 576 && dv == 512) || (dqk == 128 && dv == 128) || (dqk == 64 && dv == 64);
}

bool attn_wide_eligible(const AttnArgs& a) {
    return a.dtype == BF16 && a.kv_dtype == BF16 && wide_shape(a.dqk, a.dv) && (!a.latent || a.Hkv == 1);
}

// Slices per row: enough waves to cover the chip, at least two blocks each.
int attn_wide_splits(const AttnArgs& a) {
    const int G = a.Hq / a.Hkv;
    const int64_t waves = static_cast<int64_t>(a.rows) * a.Hkv * ((G + 15) / 16);
    int s = static_cast<int>((2048 + waves - 1) / waves);
    const int max_s = (a.kk + 31) / 32;
    if (s > max_s) s = max_s;
    return s < 1 ? 1 : s;
}

size_t attn_wide_workspace_bytes(const AttnArgs& a) {
    const int s = attn_wide_splits(a);
    if (s <= 1) return 0;
    return static_cast<size_t>(a.rows) * a.Hq * s * (a.dv + 2) * sizeof(float);
}

hipError_t launch_attn_wide(const AttnArgs& a, float* part, hipStream_t st) {
    const int G = a.Hq / a.Hkv;
    const int hgroups = (G + 15) / 16;
    const int s = attn_wide_splits(a);
    const dim3 grid(s, a.Hkv * hgroups, a.rows);
    if (a.dqk == 576)
        hipLaunchKernelGGL((k_attn_bf16_split<18, 32>), grid, dim3(64), 0, st, a, s, hgroups, part);
    else if (a.dqk == 128)
        hipLaunchKernelGGL((k_attn_bf16_split<4, 8>), grid, dim3(64), 0, st, a, s, hgroups, part);
    else
        hipLaunchKernelGGL((k_attn_bf16_split<2, 4>), grid, dim3(64), 0, st, a, s, hgroups, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || s == 1) return e;
    hipLaunchKernelGGL(k_attn_merge, dim3(a.rows * a.Hq), dim3(256), 0, st, a, s, part);
    return hipGetLastError();
}

}  // namespace dsa
