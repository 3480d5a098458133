// attn.hip -- main attention over the selected KV rows only.
//
// The main attention runs over the k kept rows instead of the whole history,
// so it costs O(n*k) instead of O(n^2) ("DeepSeek-V3.2-Exp 稀疏注意力机制(DSA)
// 技术深度解析", sheratonhq.com, section 1).
// Per query row t and head h (kv head g = h / (Hq/Hkv)):
//   z_j = scale * q[t,h].k[s_j,g],  out = sum_j softmax(z)_j v[s_j,g],
//   lse = log sum_j exp(z_j)
// over the valid entries s_j of idx[t] (0 <= s_j <= pos(t)); softmax is
// accumulated online in fp32 (running max, rescaled sum), in base 2.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Generic path: fp32 or bf16, any head grouping, d_qk <= 576, d_v <= 512,
// latent rows.  One workgroup per (query row, kv head, chunk of <= 16 query
// heads); selected rows are staged 16 at a time in LDS as fp32.
// ---------------------------------------------------------------------------
constexpr int kGenHC = 16;   // query heads per workgroup
constexpr int kGenTK = 16;   // selected rows per tile
constexpr int kGenThreads = 256;
constexpr int kGenMaxOut = 32;  // (kGenHC * 512) / kGenThreads

template <int DT>
__global__ __launch_bounds__(kGenThreads) void k_attn_generic(AttnArgs a) {
    extern __shared__ __align__(16) float sm[];
    float* q_s = sm;                                   // [HC][dqk]
    float* k_s = q_s + kGenHC * a.dqk;                 // [TK][dqk]
    float* v_s = k_s + kGenTK * a.dqk;                 // [TK][dv]
    __shared__ float p_s[kGenHC][kGenTK];
    __shared__ float m_s[kGenHC], l_s[kGenHC], corr_s[kGenHC];
    __shared__ int sidx[kGenTK];

    const int G = a.Hq / a.Hkv;
    const int hc0 = blockIdx.x * kGenHC;
    const int nh = min(kGenHC, G - hc0);
    const int g = blockIdx.y;
    const int row = blockIdx.z;
    const int b = row / a.n_q;
    const int pos = row_pos(a.q_pos, row, a.n_q, a.n_k);
    const int tid = threadIdx.x;
    const int dqk = a.dqk, dv = a.dv;
    const size_t kv_row_stride = static_cast<size_t>(a.Hkv) * dqk;    // k row (all kv heads)
    const size_t v_row_stride = static_cast<size_t>(a.Hkv) * dv;

    for (int i = tid; i < kGenHC * dqk; i += blockDim.x) {
        int h = i / dqk, d = i % dqk;
        q_s[i] = h < nh ? load_as_f32<DT>(a.q, (static_cast<size_t>(row) * a.Hq + g * G + hc0 + h) * dqk + d) : 0.0f;
    }
    if (tid < kGenHC) { m_s[tid] = -__builtin_inff(); l_s[tid] = 0.0f; }
    float o[kGenMaxOut];
#pragma unroll
    for (int i = 0; i < kGenMaxOut; ++i) o[i] = 0.0f;
    __syncthreads();

    for (int j0 = 0; j0 < a.kk; j0 += kGenTK) {
        if (tid < kGenTK) {
            int j = j0 + tid;
            int s = j < a.kk ? a.idx[static_cast<size_t>(row) * a.kk + j] : -1;
            sidx[tid] = (s >= 0 && s <= pos) ? s : -1;
        }
        __syncthreads();
        for (int i = tid; i < kGenTK * dqk; i += blockDim.x) {
            int j = i / dqk, d = i % dqk;
            int s = sidx[j];
            k_s[i] = s >= 0 ? load_as_f32<DT>(a.k, (static_cast<size_t>(b) * a.n_k + s) * kv_row_stride + g * dqk + d) : 0.0f;
        }
        for (int i = tid; i < kGenTK * dv; i += blockDim.x) {
            int j = i / dv, d = i % dv;
            int s = sidx[j];
            float val = 0.0f;
            if (s >= 0) {
                val = a.latent ? load_as_f32<DT>(a.k, (static_cast<size_t>(b) * a.n_k + s) * kv_row_stride + d)
                               : load_as_f32<DT>(a.v, (static_cast<size_t>(b) * a.n_k + s) * v_row_stride + g * dv + d);
            }
            v_s[i] = val;
        }
        __syncthreads();
        {   // one (head, row) score per thread: HC * TK == 256
            int h = tid / kGenTK, j = tid % kGenTK;
            float z = -__builtin_inff();
            if (h < nh && sidx[j] >= 0) {
                float dot = 0.0f;
                for (int d = 0; d < dqk; ++d) dot = fmaf(q_s[h * dqk + d], k_s[j * dqk + d], dot);
                z = dot * a.scale * kLog2e;
            }
            p_s[h][j] = z;
        }
        __syncthreads();
        if (tid < kGenHC) {
            int h = tid;
            float mt = -__builtin_inff();
            for (int j = 0; j < kGenTK; ++j) mt = fmaxf(mt, p_s[h][j]);
            float m_old = m_s[h];
            float m_new = fmaxf(m_old, mt);
            float corr = 1.0f, sum = 0.0f;
            if (m_new != -__builtin_inff()) {
                corr = exp2f(m_old - m_new);
                for (int j = 0; j < kGenTK; ++j) {
                    float p = exp2f(p_s[h][j] - m_new);
                    p_s[h][j] = p;
                    sum += p;
                }
            } else {
                for (int j = 0; j < kGenTK; ++j) p_s[h][j] = 0.0f;
            }
            m_s[h] = m_new;
            l_s[h] = l_s[h] * corr + sum;
            corr_s[h] = corr;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kGenMaxOut; ++i) {
            int e = tid + i * kGenThreads;
            if (e < kGenHC * dv) {
                int h = e / dv, d = e % dv;
                float acc = o[i] * corr_s[h];
                for (int j = 0; j < kGenTK; ++j) acc = fmaf(p_s[h][j], v_s[j * dv + d], acc);
                o[i] = acc;
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < kGenMaxOut; ++i) {
        int e = tid + i * kGenThreads;
        if (e < kGenHC * dv) {
            int h = e / dv, d = e % dv;
            if (h < nh) {
                float l = l_s[h];
                float val = l > 0.0f ? o[i] / l : 0.0f;
                size_t oi = (static_cast<size_t>(row) * a.Hq + g * G + hc0 + h) * dv + d;
                if constexpr (DT == F32) static_cast<float*>(a.out)[oi] = val;
                else static_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_bits(val);
                if (d == 0 && a.lse)
                    a.lse[static_cast<size_t>(row) * a.Hq + g * G + hc0 + h] =
                        l > 0.0f ? (m_s[h] + log2f(l)) * kLn2 : -__builtin_inff();
            }
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 fast path: d_qk = d_v = 128, up to 16 query heads per kv head (GQA and
// MHA).  One workgroup per (query row, kv head), 8 waves; the row's index
// list is staged in LDS first, then wave w owns a contiguous 1/8 of it, 16
// entries per block:
//   S^T[key][head] = K Q^T  with 4 x v_mfma_f32_16x16x32_bf16: A = the 16
//     gathered key rows (lane l: key l%16, its 64 contiguous bytes at
//     64*(l/16)), B = Q^T held in registers for the whole loop;
//   the result leaves each lane with 4 keys of one head (head l%16), so the
//     online-softmax rescale is per lane and P^T is already the B operand of
//   O^T[dim][head] += V^T P^T with 8 x v_mfma_f32_16x16x16_bf16, where the
//     V^T operand is read out of a per-wave LDS copy of the 16 value rows.
// Each wave keeps DEPTH further blocks of key/value rows in flight in a
// register ring while it multiplies the current one.  The waves' (max, sum,
// O) are merged through LDS at the end.
// ---------------------------------------------------------------------------
#ifndef DSA_ATTN_DEPTH
#define DSA_ATTN_DEPTH 1
#endif
#ifndef DSA_ATTN_WAVES
#define DSA_ATTN_WAVES 8
#endif
constexpr int kGqaWaves = DSA_ATTN_WAVES;
constexpr int kGqaVStride = 136;   // bf16 elements per staged value row (128 + pad)

template <int DEPTH>
__global__ __launch_bounds__(kGqaWaves * 64) void k_attn_bf16_d128(AttnArgs a, int slice_len, float* part) {
    __shared__ __align__(16) unsigned char smem[kGqaWaves * 16 * 128 * 4];   // 64 KiB
    __shared__ float m_w[kGqaWaves][16], l_w[kGqaWaves][16];
    extern __shared__ int32_t idx_s[];                                        // [kk]
    uint16_t* v_all = reinterpret_cast<uint16_t*>(smem);                    // during the loop
    float* o_all = reinterpret_cast<float*>(smem);                           // after the loop
    constexpr int SLOTS = DEPTH + 1;

    const int G = a.Hq / a.Hkv;
    const int g = blockIdx.x;
    const int row = blockIdx.y;
    const int nsplit = gridDim.z;
    const int sl = blockIdx.z;                     // this workgroup's slice of the index list
    const int jb = sl * slice_len;
    const int nj = max(0, min(slice_len, a.kk - jb));
    const int b = row / a.n_q;
    const int pos = row_pos(a.q_pos, row, a.n_q, a.n_k);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;
    const int kg = lane >> 4;
    const float zscale = a.scale * kLog2e;
    uint16_t* v_s = v_all + wave * 16 * kGqaVStride;

    const int32_t* idx_row = a.idx + static_cast<size_t>(row) * a.kk + jb;
    for (int j = threadIdx.x; j < nj; j += blockDim.x) idx_s[j] = idx_row[j];

    const uint16_t* qp = static_cast<const uint16_t*>(a.q);
    const uint16_t* kp = static_cast<const uint16_t*>(a.k);
    const uint16_t* vp = static_cast<const uint16_t*>(a.v);
    v8bf qb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        if (col < G)
            qb[c] = *reinterpret_cast<const v8bf*>(qp + (static_cast<size_t>(row) * a.Hq + g * G + col) * 128 + kg * 32 + c * 8);
        else
            qb[c] = v8bf{};
    }

    const int per = ((nj + kGqaWaves * 16 - 1) / (kGqaWaves * 16)) * 16;
    const int j_begin = wave * per;
    const int j_end = min(j_begin + per, nj);
    const int nblk = j_end > j_begin ? (j_end - j_begin + 15) / 16 : 0;
    const size_t row_elems = static_cast<size_t>(a.Hkv) * 128;
    const uint16_t* kbase = kp + static_cast<size_t>(b) * a.n_k * row_elems + g * 128 + kg * 32;
    const uint16_t* vbase = vp + static_cast<size_t>(b) * a.n_k * row_elems + g * 128 + kg * 32;

    float m_run = -__builtin_inff();
    float l_part = 0.0f;
    v4f o[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    __syncthreads();                               // idx_s is ready

    v8bf kr[SLOTS][4], vr[SLOTS][4];
    bool valid[SLOTS];
    auto load_block = [&](int blk, v8bf* kd, v8bf* vd, bool& ok) {
        int j = j_begin + blk * 16 + col;
        int s = j < j_end ? idx_s[j] : -1;
        ok = s >= 0 && s <= pos;
        if (ok) {
            const v8bf* ks = reinterpret_cast<const v8bf*>(kbase + static_cast<size_t>(s) * row_elems);
            const v8bf* vs = reinterpret_cast<const v8bf*>(vbase + static_cast<size_t>(s) * row_elems);
#pragma unroll
            for (int c = 0; c < 4; ++c) { kd[c] = ks[c]; vd[c] = vs[c]; }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) { kd[c] = v8bf{}; vd[c] = v8bf{}; }
        }
    };
    auto attend_block = [&](const v8bf* kc, const v8bf* vc, bool ok) {
        v4f sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < 4; ++c) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc[c], qb[c], sacc, 0, 0, 0);
        const uint64_t vm = __ballot(ok);
        float sv[4];
        float bm = -__builtin_inff();
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            int slot = 4 * kg + v;
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
#pragma unroll
        for (int t = 0; t < 8; ++t) o[t] *= corr;

        // stage the 16 value rows of this wave, then read them transposed
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *reinterpret_cast<v8bf*>(v_s + col * kGqaVStride + kg * 32 + c * 8) = vc[c];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        v4bf pb;
#pragma unroll
        for (int v = 0; v < 4; ++v) pb[v] = static_cast<__bf16>(p[v]);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            v4bf va;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                va[v] = *reinterpret_cast<const __bf16*>(v_s + (4 * kg + v) * kGqaVStride + 16 * t + col);
            o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[t], 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        if (d < nblk) load_block(d, kr[d], vr[d], valid[d]);
    for (int i0 = 0; i0 < nblk; i0 += SLOTS) {
#pragma unroll
        for (int r = 0; r < SLOTS; ++r) {
            const int blk = i0 + r;
            if (blk < nblk) {
                const int ahead = blk + DEPTH;
                if (ahead < nblk) load_block(ahead, kr[(r + DEPTH) % SLOTS], vr[(r + DEPTH) % SLOTS],
                                             valid[(r + DEPTH) % SLOTS]);
                attend_block(kr[r], vr[r], valid[r]);
            }
        }
    }

    const float l_tot = wave_sum_xor_16_32(l_part);
    __syncthreads();                                   // every wave is done with v_all
    float* o_s = o_all + wave * 16 * 128;              // [head][dim]
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) o_s[col * 128 + 16 * t + 4 * kg + v] = o[t][v];
    if (kg == 0) { m_w[wave][col] = m_run; l_w[wave][col] = l_tot; }
    __syncthreads();

    uint16_t* outp = static_cast<uint16_t*>(a.out);
    for (int e = threadIdx.x; e < G * 128; e += blockDim.x) {
        int h = e >> 7, d = e & 127;
        float M = -__builtin_inff();
        for (int w = 0; w < kGqaWaves; ++w) M = fmaxf(M, m_w[w][h]);
        float L = 0.0f, O = 0.0f;
        if (M != -__builtin_inff()) {
            for (int w = 0; w < kGqaWaves; ++w) {
                float mw = m_w[w][h];
                if (mw == -__builtin_inff()) continue;
                float f = exp2f(mw - M);
                L += l_w[w][h] * f;
                O += o_all[(w * 16 + h) * 128 + d] * f;
            }
        }
        const size_t rh = static_cast<size_t>(row) * a.Hq + g * G + h;
        if (nsplit > 1) {
            // this slice's (max, sum, unnormalised O) record for k_attn_merge
            float* rec = part + (rh * nsplit + sl) * (128 + 2);
            rec[2 + d] = O;
            if (d == 0) { rec[0] = M; rec[1] = L; }
            continue;
        }
        float val = L > 0.0f ? O / L : 0.0f;
        outp[rh * 128 + d] = f32_to_bf16_bits(val);
        if (d == 0 && a.lse) a.lse[rh] = L > 0.0f ? (M + log2f(L)) * kLn2 : -__builtin_inff();
    }
}

static bool gqa_d128_eligible(const AttnArgs& a) {
    return a.dtype == BF16 && !a.latent && a.dqk == 128 && a.dv == 128 && a.Hq / a.Hkv <= 16;
}

#ifndef DSA_ATTN_TARGET_WGS
#define DSA_ATTN_TARGET_WGS 256
#endif
// Slices of each row's index list.  A workgroup's gather rate is bounded by
// its compute unit, so with fewer (row, kv head) pairs than compute units the
// list is split (at least 256 entries per slice) to reach them all, and the
// slices' (max, sum, O) records are merged afterwards.  With one workgroup
// per compute unit already, splitting measured slower.
static int gqa_splits(const AttnArgs& a) {
    const int64_t wgs = static_cast<int64_t>(a.rows) * a.Hkv;
    int s = static_cast<int>((DSA_ATTN_TARGET_WGS + wgs - 1) / wgs);
    const int max_s = a.kk / 256;
    if (s > max_s) s = max_s;
    return s < 1 ? 1 : s;
}
static int gqa_slice_len(const AttnArgs& a, int s) { return ((a.kk + s - 1) / s + 15) / 16 * 16; }

size_t attn_workspace_bytes(const AttnArgs& a) {
    if (attn_masked_eligible(a)) return attn_masked_workspace_bytes(a);
    if (gqa_d128_eligible(a)) {
        const int s = gqa_splits(a);
        return s > 1 ? static_cast<size_t>(a.rows) * a.Hq * s * (128 + 2) * sizeof(float) : 0;
    }
    if (!attn_wide_eligible(a)) return 0;
    return attn_wide_workspace_bytes(a);
}

hipError_t launch_sparse_attn(const AttnArgs& a, void* ws, hipStream_t st) {
    const int G = a.Hq / a.Hkv;
    if (attn_masked_eligible(a)) return launch_attn_masked(a, static_cast<uint32_t*>(ws), st);
    if (gqa_d128_eligible(a)) {
        const int s = gqa_splits(a);
        const int len = gqa_slice_len(a, s);
        float* part = static_cast<float*>(ws);
        const size_t idx_lds = static_cast<size_t>(len) * sizeof(int32_t);   // <= 8192 entries: 32 KiB
        hipLaunchKernelGGL((k_attn_bf16_d128<DSA_ATTN_DEPTH>), dim3(a.Hkv, a.rows, s), dim3(kGqaWaves * 64),
                           idx_lds, st, a, len, part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || s == 1) return e;
        return launch_attn_merge(a, s, part, st);
    }
    if (attn_wide_eligible(a)) return launch_attn_wide(a, static_cast<float*>(ws), st);
    const size_t smem = (static_cast<size_t>(kGenHC) * a.dqk + static_cast<size_t>(kGenTK) * a.dqk +
                         static_cast<size_t>(kGenTK) * a.dv) * sizeof(float);
    if (smem > 64 * 1024) {   // the latent shape stages ~104 KiB of rows
        hipError_t e = a.dtype == F32
            ? hipFuncSetAttribute(reinterpret_cast<const void*>(k_attn_generic<F32>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem))
            : hipFuncSetAttribute(reinterpret_cast<const void*>(k_attn_generic<BF16>),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
        if (e != hipSuccess) return e;
    }
    dim3 grid((G + kGenHC - 1) / kGenHC, a.Hkv, a.rows);
    if (a.dtype == F32)
        hipLaunchKernelGGL(k_attn_generic<F32>, grid, dim3(kGenThreads), smem, st, a);
    else
        hipLaunchKernelGGL(k_attn_generic<BF16>, grid, dim3(kGenThreads), smem, st, a);
    return hipGetLastError();
}

}  // namespace dsa
