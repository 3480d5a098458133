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
// Generic path: fp32 or bf16 (KV also E4M3 with per-row scales), any head
// grouping, d_qk <= 576, d_v <= 512, latent rows.  One workgroup per (query
// row, kv head, chunk of <= 16 query heads); selected rows are staged 16 at a
// time in LDS as fp32, decoded (code * row scale) on the way in.
// ---------------------------------------------------------------------------
constexpr int kGenHC = 16;   // query heads per workgroup
constexpr int kGenTK = 16;   // selected rows per tile
constexpr int kGenThreads = 256;
constexpr int kGenMaxOut = 32;  // (kGenHC * 512) / kGenThreads

template <int DT, int KDT>
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
    // elements per token of k and v (all kv heads); an E4M3 cache's token
    // records hold the codes first, then the scales, and may be padded
    const size_t kv_row_stride = KDT == E4M3 ? static_cast<size_t>(a.k_rec) : static_cast<size_t>(a.Hkv) * dqk;
    const size_t v_row_stride = KDT == E4M3 ? static_cast<size_t>(a.v_rec) : static_cast<size_t>(a.Hkv) * dv;
    auto rec_scale = [&](const void* base, size_t r, size_t stride, int dim, int head) {
        return *reinterpret_cast<const float*>(static_cast<const unsigned char*>(base) + r * stride +
                                               static_cast<size_t>(a.Hkv) * dim + 4 * head);
    };

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
            float val = 0.0f;
            if (s >= 0) {
                const size_t r = static_cast<size_t>(b) * a.n_k + s;
                val = load_as_f32<KDT>(a.k, r * kv_row_stride + g * dqk + d);
                if constexpr (KDT == E4M3) val *= rec_scale(a.k, r, kv_row_stride, dqk, g);
            }
            k_s[i] = val;
        }
        for (int i = tid; i < kGenTK * dv; i += blockDim.x) {
            int j = i / dv, d = i % dv;
            int s = sidx[j];
            float val = 0.0f;
            if (s >= 0) {
                const size_t r = static_cast<size_t>(b) * a.n_k + s;
                if (a.latent) {
                    val = load_as_f32<KDT>(a.k, r * kv_row_stride + d);
                    if constexpr (KDT == E4M3) val *= rec_scale(a.k, r, kv_row_stride, dqk, 0);
                } else {
                    val = load_as_f32<KDT>(a.v, r * v_row_stride + g * dv + d);
                    if constexpr (KDT == E4M3) val *= rec_scale(a.v, r, v_row_stride, dv, g);
                }
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
//     gathered key rows (lane l: key l%16; load c brings bytes
//     64c + 16(l/16)..+16 of a bf16 row, so the 4 lanes of a key read one
//     contiguous 64-byte run), B = Q^T held in registers for the whole loop;
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
// (an E4M3 block carries half the bytes of a bf16 one)
#ifndef DSA_ATTN_DEPTH8
#define DSA_ATTN_DEPTH8 DSA_ATTN_DEPTH
#endif
#ifndef DSA_ATTN_WAVES
#define DSA_ATTN_WAVES 8
#endif
constexpr int kGqaWaves = DSA_ATTN_WAVES;
constexpr int kGqaVStride = 136;   // bf16 elements per staged value row (128 + pad)

// Ring slot of one 16-key block: a lane's 32 dims of its key's k and v row,
// as bf16 or, from an E4M3 cache, as the 32 code bytes plus the row scales.
template <bool KV8> struct GqaBlock;
template <> struct GqaBlock<false> { v8bf k[4], v[4]; bool ok; };
template <> struct GqaBlock<true> { v4i k[2], v[2]; float ks, vs; bool ok; };

// 32 E4M3 codes -> 32 bf16 (exact: every E4M3 value is a bf16 value).  Byte i
// of the input becomes element i of the output.
__device__ __forceinline__ void e4m3x32_to_bf16(const v4i* w, v8bf* out) {
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint32_t w0 = static_cast<uint32_t>(w[c >> 1][(c & 1) * 2]);
        const uint32_t w1 = static_cast<uint32_t>(w[c >> 1][(c & 1) * 2 + 1]);
        const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
        const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
        const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
        const v2bf e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
        out[c] = v8bf{a[0], a[1], b[0], b[1], d[0], d[1], e[0], e[1]};
    }
}

// KV8: the cache holds E4M3 codes with one fp32 scale per (token, kv head)
// row.  The codes are widened to bf16 exactly; the key scale multiplies the
// scores (z = scale * ks * q.code) and the value scale multiplies the softmax
// weights before their bf16 rounding (p * vs * code), so the running sum stays
// the plain softmax denominator.
template <int DEPTH, bool KV8>
__global__ __launch_bounds__(kGqaWaves * 64) void k_attn_bf16_d128(AttnArgs a, int row0, int nrows, int nsplit, int slice_len,
                                                                           float* part) {
    __shared__ __align__(16) unsigned char smem[kGqaWaves * 16 * 128 * 4];   // 64 KiB
    __shared__ float m_w[kGqaWaves][16], l_w[kGqaWaves][16];
    __shared__ __align__(16) float sc_w[kGqaWaves][2][16];                   // KV8: block's k / v scales
    extern __shared__ int32_t idx_s[];                                        // [kk]
    uint16_t* v_all = reinterpret_cast<uint16_t*>(smem);                    // during the loop
    float* o_all = reinterpret_cast<float*>(smem);                           // after the loop
    constexpr int SLOTS = DEPTH + 1;

    const int G = a.Hq / a.Hkv;
    // One workgroup per (kv head, row, slice).  Consecutive workgroup ids go to
    // the 8 XCDs in turn; when the (row, slice) units divide by 8, the ids are
    // mapped so that the kv heads of one unit land on the same XCD, back to
    // back: they gather the same tokens, and the scales of an E4M3 cache's
    // token record (one 16-byte group after the codes of its 4 kv heads) are
    // then read into that XCD's L2 once instead of once per kv head.
    int g, unit;
    {
        const int id = blockIdx.x;
        const int units = nrows * nsplit;
        if ((units & 7) == 0) {
            const int k = id >> 3;
            g = k % a.Hkv;
            unit = (k / a.Hkv) * 8 + (id & 7);
        } else {
            g = id % a.Hkv;
            unit = id / a.Hkv;
        }
    }
    const int row = row0 + unit / nsplit;          // rows [row0, row0 + nrows) in this launch
    const int sl = unit % nsplit;                  // this workgroup's slice of the index list
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

    // Dims of product c held by lane (col, kg): from a bf16 cache 32c + 8kg..+8,
    // so that the 4 lanes of a key read one contiguous 64-byte run per load
    // (16 keys x 64 B per load instruction); from an E4M3 cache 32kg + 8c..+8
    // (a lane widens its own 32 contiguous code bytes).  Q takes the same order.
    const uint16_t* qp = static_cast<const uint16_t*>(a.q);
    v8bf qb[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int dim0 = KV8 ? kg * 32 + c * 8 : c * 32 + kg * 8;
        if (col < G)
            qb[c] = *reinterpret_cast<const v8bf*>(qp + (static_cast<size_t>(row) * a.Hq + g * G + col) * 128 + dim0);
        else
            qb[c] = v8bf{};
    }

    const int per = ((nj + kGqaWaves * 16 - 1) / (kGqaWaves * 16)) * 16;
    const int j_begin = wave * per;
    const int j_end = min(j_begin + per, nj);
    const int nblk = j_end > j_begin ? (j_end - j_begin + 15) / 16 : 0;
    // this lane's 32 dims of kv head g within each 128-dim row: E4M3 bytes
    // [32kg, 32kg + 32); bf16 elements 8kg..8kg+8 of each 32-dim group (the
    // loads add 64 bytes per group)
    // (an E4M3 cache: token records of codes then scales; kv head g's scale
    // sits 4g bytes past the Hkv * 128 code bytes)
    constexpr int ESZ = KV8 ? 1 : 2;
    const size_t k_bytes = KV8 ? static_cast<size_t>(a.k_rec) : static_cast<size_t>(a.Hkv) * 128 * ESZ;
    const size_t v_bytes = KV8 ? static_cast<size_t>(a.v_rec) : k_bytes;
    const size_t lane_off = g * 128 * ESZ + (KV8 ? kg * 32 : kg * 16);
    const unsigned char* kbase = static_cast<const unsigned char*>(a.k) + static_cast<size_t>(b) * a.n_k * k_bytes;
    const unsigned char* vbase = static_cast<const unsigned char*>(a.v) + static_cast<size_t>(b) * a.n_k * v_bytes;
    const size_t sc_off = static_cast<size_t>(a.Hkv) * 128 + 4 * g;

    float m_run = -__builtin_inff();
    float l_part = 0.0f;
    v4f o[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // each wave stages its own entries [j_begin, j_end) of the index list,
    // all loads of a round before any store, so no workgroup barrier is needed
    for (int j0 = j_begin; j0 < j_end; j0 += 256) {
        int e[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) e[u] = idx_row[min(j0 + lane + 64 * u, j_end - 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (j0 + lane + 64 * u < j_end) idx_s[j0 + lane + 64 * u] = e[u];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    GqaBlock<KV8> ring[SLOTS];
    // Every lane loads, whatever its entry: an invalid one (past the list, < 0
    // or > pos) reads token 0 of the sequence instead, and attend_block drops
    // it (zeroed operands, masked score).  With no branch around the loads the
    // compiler's wait counts stay exact, so a block's wait does not also wait
    // for the blocks loaded after it.
    auto load_block = [&](int blk, GqaBlock<KV8>& d) {
        const int j = j_begin + blk * 16 + col;
        const int s = idx_s[min(j, j_end - 1)];
        d.ok = j < j_end && s >= 0 && s <= pos;
        const size_t sr = d.ok ? static_cast<size_t>(s) : 0;
        // the loads go out in one fixed order wherever a block is loaded, so
        // that the wait counts agree on every path into the loop
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (KV8) {
            const unsigned char* kr = kbase + sr * k_bytes;
            const unsigned char* vr = vbase + sr * v_bytes;
            const v4i* ks = reinterpret_cast<const v4i*>(kr + lane_off);
            const v4i* vs = reinterpret_cast<const v4i*>(vr + lane_off);
            d.k[0] = ks[0]; d.k[1] = ks[1]; d.v[0] = vs[0]; d.v[1] = vs[1];
            d.ks = *reinterpret_cast<const float*>(kr + sc_off);
            d.vs = *reinterpret_cast<const float*>(vr + sc_off);
        } else {
            const unsigned char* ks = kbase + sr * k_bytes + lane_off;
            const unsigned char* vs = vbase + sr * v_bytes + lane_off;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                d.k[c] = *reinterpret_cast<const v8bf*>(ks + 64 * c);
                d.v[c] = *reinterpret_cast<const v8bf*>(vs + 64 * c);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    auto stage_values = [&](const v8bf* vc) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *reinterpret_cast<v8bf*>(v_s + col * kGqaVStride + (KV8 ? kg * 32 + c * 8 : c * 32 + kg * 8)) = vc[c];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };
    auto attend_block = [&](GqaBlock<KV8>& blkd) {
        v8bf kc[4];
        float ksc[4], vsc[4];
        // an invalid entry's operands are zeroed, so that whatever token 0
        // holds cannot reach the sums
        if constexpr (KV8) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                blkd.k[c] = blkd.ok ? blkd.k[c] : v4i{0, 0, 0, 0};
                blkd.v[c] = blkd.ok ? blkd.v[c] : v4i{0, 0, 0, 0};
            }
            blkd.ks = blkd.ok ? blkd.ks : 0.0f;
            blkd.vs = blkd.ok ? blkd.vs : 0.0f;
            v8bf vc[4];
            e4m3x32_to_bf16(blkd.v, vc);
            // key c's scales go to slot c; lane (kg, col) reads keys 4kg..4kg+3
            sc_w[wave][0][col] = blkd.ks;
            sc_w[wave][1][col] = blkd.vs;
            stage_values(vc);
            e4m3x32_to_bf16(blkd.k, kc);
            const v4f k4 = *reinterpret_cast<const v4f*>(&sc_w[wave][0][4 * kg]);
            const v4f v4 = *reinterpret_cast<const v4f*>(&sc_w[wave][1][4 * kg]);
#pragma unroll
            for (int v = 0; v < 4; ++v) { ksc[v] = zscale * k4[v]; vsc[v] = v4[v]; }
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                blkd.k[c] = blkd.ok ? blkd.k[c] : v8bf{};
                blkd.v[c] = blkd.ok ? blkd.v[c] : v8bf{};
                kc[c] = blkd.k[c];
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) { ksc[v] = zscale; vsc[v] = 1.0f; }
        }
        v4f sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < 4; ++c) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc[c], qb[c], sacc, 0, 0, 0);
        const uint64_t vm = __ballot(blkd.ok);
        float sv[4];
        float bm = -__builtin_inff();
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            int slot = 4 * kg + v;
            sv[v] = ((vm >> slot) & 1ull) ? sacc[v] * ksc[v] : -__builtin_inff();
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

        // the 16 value rows of this wave, read transposed
        if constexpr (!KV8) stage_values(blkd.v);
        v4bf pb;
#pragma unroll
        for (int v = 0; v < 4; ++v) pb[v] = static_cast<__bf16>(KV8 ? p[v] * vsc[v] : p[v]);
        // va = V[4kg + v][16t + col], v < 4: lane (kg, col) addresses row
        // 4kg + col/4 at dims 16t + 4(col%4)..+3 and the transposing read
        // hands every lane its own dim of the group's four rows
        const uint16_t* trp = v_s + (4 * kg + (col >> 2)) * kGqaVStride + 4 * (col & 3);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const v4bf va = lds_read_tr16(trp + 16 * t);
            o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb, o[t], 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    if (nblk > 0) {
        // whole turns of the ring: blocks past nblk have no valid entry and
        // change nothing
        const int nblk_pad = (nblk + SLOTS - 1) / SLOTS * SLOTS;
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) load_block(d, ring[d]);
        for (int i0 = 0; i0 < nblk_pad; i0 += SLOTS) {
#pragma unroll
            for (int r = 0; r < SLOTS; ++r) {
                load_block(i0 + r + DEPTH, ring[(r + DEPTH) % SLOTS]);
                // keep the block's use (and its wait) after the loads ahead
                __builtin_amdgcn_sched_barrier(0);
                attend_block(ring[r]);
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
    if (attn_latent_eligible(a)) return attn_latent_workspace_bytes(a);
    if (!attn_wide_eligible(a)) return 0;
    return attn_wide_workspace_bytes(a);
}

hipError_t launch_sparse_attn(const AttnArgs& a, void* ws, hipStream_t st) {
    const int G = a.Hq / a.Hkv;
    if (attn_masked_eligible(a)) return launch_attn_masked(a, ws, st);
    if (gqa_d128_eligible(a)) {
        const int s = gqa_splits(a);
        const int len = gqa_slice_len(a, s);
        float* part = static_cast<float*>(ws);
        const size_t idx_lds = static_cast<size_t>(len) * sizeof(int32_t);   // <= 8192 entries: 32 KiB
        // a 1-D grid, in launches of at most 2^22 workgroups (2^31 work-items)
        const int64_t per_row = static_cast<int64_t>(a.Hkv) * s;
        int chunk = static_cast<int>(((int64_t{1} << 22) / per_row) & ~int64_t{7});
        if (chunk < 8) chunk = 8;
        hipError_t e = hipSuccess;
        for (int r0 = 0; r0 < a.rows && e == hipSuccess; r0 += chunk) {
            const int nr = a.rows - r0 < chunk ? a.rows - r0 : chunk;
            const dim3 grid(static_cast<unsigned>(per_row * nr));
            if (a.kv_dtype == E4M3)
                hipLaunchKernelGGL((k_attn_bf16_d128<DSA_ATTN_DEPTH8, true>), grid, dim3(kGqaWaves * 64), idx_lds,
                                   st, a, r0, nr, s, len, part);
            else
                hipLaunchKernelGGL((k_attn_bf16_d128<DSA_ATTN_DEPTH, false>), grid, dim3(kGqaWaves * 64), idx_lds,
                                   st, a, r0, nr, s, len, part);
            e = hipGetLastError();
        }
        if (e != hipSuccess || s == 1) return e;
        return launch_attn_merge(a, s, part, st);
    }
    if (attn_latent_eligible(a)) return launch_attn_latent(a, static_cast<float*>(ws), st);
    if (attn_wide_eligible(a)) return launch_attn_wide(a, static_cast<float*>(ws), st);
    const size_t smem = (static_cast<size_t>(kGenHC) * a.dqk + static_cast<size_t>(kGenTK) * a.dqk +
                         static_cast<size_t>(kGenTK) * a.dv) * sizeof(float);
    const void* fn = a.dtype == F32        ? reinterpret_cast<const void*>(k_attn_generic<F32, F32>)
                     : a.kv_dtype == E4M3  ? reinterpret_cast<const void*>(k_attn_generic<BF16, E4M3>)
                                           : reinterpret_cast<const void*>(k_attn_generic<BF16, BF16>);
    {   // (the latent shape stages ~104 KiB of rows)
        hipError_t e = allow_dyn_lds(fn, smem);
        if (e != hipSuccess) return e;
    }
    dim3 grid((G + kGenHC - 1) / kGenHC, a.Hkv, a.rows);
    if (a.dtype == F32)
        hipLaunchKernelGGL((k_attn_generic<F32, F32>), grid, dim3(kGenThreads), smem, st, a);
    else if (a.kv_dtype == E4M3)
        hipLaunchKernelGGL((k_attn_generic<BF16, E4M3>), grid, dim3(kGenThreads), smem, st, a);
    else
        hipLaunchKernelGGL((k_attn_generic<BF16, BF16>), grid, dim3(kGenThreads), smem, st, a);
    return hipGetLastError();
}

}  // namespace dsa
