// attn_masked.hip -- sparse attention for prefill as masked dense MFMA tiles.
//
// Short sequences run DSA through a masked MHA mode ("DeepSeek-V3.2-Exp
// 稀疏注意力机制(DSA)技术深度解析", sheratonhq.com, section 1).  The result is the
// same attention over each query's selected keys: a softmax over the keys a
// mask admits equals the softmax over the kept subset.  In prefill, the
// selections of neighbouring queries overlap so much that reading every key
// tile once per block of 64 queries moves far fewer bytes than gathering k
// rows per query (a row kept by 1/64 of the queries of a block is already
// cheaper as a tile), so prefill rows take this path:
//   bitmap  one workgroup per query row turns its index list into a bit row
//           over the keys (bit s set <=> s kept);
//   attend  one workgroup per (block of 64 queries, query head), 4 waves of
//           16 queries each, walks the key tiles of 64 up to the block's
//           last visible key.  Per tile: S^T = K Q^T on
//           v_mfma_f32_16x16x32_bf16 (K from LDS, Q^T in registers), the
//           query's bits mask S, online softmax per lane (query l%16) in fp32,
//           then O^T += V^T P^T, also on v_mfma_f32_16x16x32_bf16, with V^T
//           read from the row-major V tile by transposing LDS reads.  Tiles
//           where none of a wave's queries keep a key are skipped by that
//           wave.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kQB = 64;            // queries per workgroup
constexpr int kKB = 64;            // keys per tile
constexpr int kStr = 136;          // LDS row stride (bf16) of the K and V tiles
constexpr int kMaskedMaxKeys = 1 << 18;
}

// Words (uint32) per bit row: keys rounded up to 64.
static inline int bitmap_words(int n_k) { return ((n_k + 63) / 64) * 2; }

__global__ __launch_bounds__(256) void k_sel_bitmap(AttnArgs a, uint32_t* bm, int words) {
    extern __shared__ uint32_t lb[];
    const int row = blockIdx.x;
    const int pos = row_pos(a.q_pos, row, a.n_q, a.n_k);
    for (int i = threadIdx.x; i < words; i += blockDim.x) lb[i] = 0u;
    __syncthreads();
    const int32_t* ir = a.idx + static_cast<size_t>(row) * a.kk;
    for (int j = threadIdx.x; j < a.kk; j += blockDim.x) {
        const int s = ir[j];
        if (s >= 0 && s <= pos) atomicOr(&lb[s >> 5], 1u << (s & 31));
    }
    __syncthreads();
    uint32_t* out = bm + static_cast<size_t>(row) * words;
    for (int i = threadIdx.x; i < words; i += blockDim.x) out[i] = lb[i];
}

// P.V runs on v_mfma_f32_16x16x32_bf16 over 32 keys.  Lane l supplies the
// eight keys {32m + 4(l/16) + i, 32m + 16 + 4(l/16) + i : i < 4} -- the four
// S^T values it already holds from each of the two 16-key tiles -- and the V^T
// operand takes the same eight keys from the row-major V tile with two
// ds_read_b64_tr_b16: within each 16-lane group, lane i of that instruction
// receives element i%4 of the 8-byte chunks addressed by lanes i/4, 4+i/4,
// 8+i/4 and 12+i/4, so lane j addresses key (j/4) of the quadruple and dims
// 4(j%4)..4(j%4)+3 of the 16-dim slice.  The next tile's rows are fetched into
// registers while the current one is multiplied.
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short lds_s4_t;
typedef __attribute__((address_space(3))) lds_s4_t* lds_s4_ptr;
typedef __attribute__((address_space(3))) uint16_t* lds_u16_ptr;

__device__ __forceinline__ v4bf lds_read_tr16(const uint16_t* p) {
    lds_s4_ptr lp = (lds_s4_ptr)((lds_u16_ptr)(const_cast<uint16_t*>(p)));
    lds_s4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp);
    v4bf r;
    __builtin_memcpy(&r, &v, sizeof r);
    return r;
}

__global__ __launch_bounds__(256) void k_attn_masked_d128(AttnArgs a, const uint32_t* bm, int words) {
    __shared__ __align__(16) uint16_t k_s[kKB * kStr];
    __shared__ __align__(16) uint16_t v_s[kKB * kStr];
    __shared__ int last_s[4];

    const int nqb = (a.n_q + kQB - 1) / kQB;
    const int qb = nqb - 1 - blockIdx.x;        // longest blocks first
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int G = a.Hq / a.Hkv;
    const int g = h / G;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, kg = lane >> 4;
    const float zscale = a.scale * kLog2e;

    const int t = qb * kQB + wave * 16 + col;   // this lane's query (S^T column)
    const bool live_q = t < a.n_q;
    const int row = b * a.n_q + (live_q ? t : 0);
    const int pos = live_q ? row_pos(a.q_pos, row, a.n_q, a.n_k) : -1;

    // the block's last visible key bounds the tile walk
    int mp = pos;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) mp = max(mp, __shfl_xor(mp, o));
    if (lane == 0) last_s[wave] = mp;

    const uint16_t* qp = static_cast<const uint16_t*>(a.q);
    v8bf qb4[4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
        qb4[c] = live_q ? *reinterpret_cast<const v8bf*>(qp + (static_cast<size_t>(row) * a.Hq + h) * 128 + kg * 32 + c * 8)
                        : v8bf{};
    __syncthreads();
    const int last = max(max(last_s[0], last_s[1]), max(last_s[2], last_s[3]));
    const int ntiles = last < 0 ? 0 : last / kKB + 1;

    const uint16_t* kp = static_cast<const uint16_t*>(a.k);
    const uint16_t* vp = static_cast<const uint16_t*>(a.v);
    const size_t rstride = static_cast<size_t>(a.Hkv) * 128;
    const uint16_t* kbase = kp + static_cast<size_t>(b) * a.n_k * rstride + g * 128;
    const uint16_t* vbase = vp + static_cast<size_t>(b) * a.n_k * rstride + g * 128;
    const uint32_t* brow = bm + static_cast<size_t>(row) * words;

    float m_run = -__builtin_inff();
    float l_part = 0.0f;
    v4f o[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // loader: 256 threads x 4 rows x 16 B of K and of V per tile
    const int lrow = threadIdx.x >> 4;          // 0..15, plus 16 per step
    const int lcol = (threadIdx.x & 15) * 8;    // bf16 offset within the 128-wide row
    v8bf pk[4], pv[4];
    uint32_t pw0 = 0u, pw1 = 0u;
    auto fetch = [&](int tile) {
        const int key0 = tile * kKB;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = key0 + lrow + 16 * r;
            if (key < a.n_k) {
                pk[r] = *reinterpret_cast<const v8bf*>(kbase + static_cast<size_t>(key) * rstride + lcol);
                pv[r] = *reinterpret_cast<const v8bf*>(vbase + static_cast<size_t>(key) * rstride + lcol);
            } else {
                pk[r] = v8bf{};
                pv[r] = v8bf{};
            }
        }
        pw0 = live_q ? brow[2 * tile] : 0u;
        pw1 = live_q ? brow[2 * tile + 1] : 0u;
    };
    auto stage = [&]() {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int kr = lrow + 16 * r;
            *reinterpret_cast<v8bf*>(&k_s[kr * kStr + lcol]) = pk[r];
            *reinterpret_cast<v8bf*>(&v_s[kr * kStr + lcol]) = pv[r];
        }
    };
    // this lane's address pattern for the transposing V reads (see above)
    const int tr_key = (col >> 2);              // key within a quadruple
    const int tr_dim = 4 * (col & 3);           // dims within a 16-dim slice

    if (ntiles > 0) {
        fetch(0);
        stage();
    }
    uint32_t w0 = pw0, w1 = pw1;
    __syncthreads();
    for (int tile = 0; tile < ntiles; ++tile) {
        if (tile + 1 < ntiles) fetch(tile + 1);  // in flight during the multiply
        const bool any = __ballot((w0 | w1) != 0u) != 0ull;
        if (any) {                               // uniform per wave
            v4f acc[4];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt) {
                acc[kt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const v8bf ka = *reinterpret_cast<const v8bf*>(k_s + (kt * 16 + col) * kStr + kg * 32 + c * 8);
                    acc[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb4[c], acc[kt], 0, 0, 0);
                }
            }
            // acc[kt][i] = S^T[key kt*16 + 4*kg + i][query col]
            float z[4][4];
            float bmax = -__builtin_inff();
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int off = kt * 16 + 4 * kg + i;
                    const uint32_t bit = off < 32 ? (w0 >> off) & 1u : (w1 >> (off - 32)) & 1u;
                    z[kt][i] = bit ? acc[kt][i] * zscale : -__builtin_inff();
                    bmax = fmaxf(bmax, z[kt][i]);
                }
            bmax = wave_max_xor_16_32(bmax);
            const float m_new = fmaxf(m_run, bmax);
            float corr = 1.0f, psum = 0.0f;
            v8bf pb[2];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = m_new != -__builtin_inff() ? exp2f(z[kt][i] - m_new) : 0.0f;
                    psum += p;
                    pb[kt >> 1][(kt & 1) * 4 + i] = static_cast<__bf16>(p);
                }
            if (m_new != -__builtin_inff()) corr = exp2f(m_run - m_new);
            l_part = l_part * corr + psum;
            m_run = m_new;
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                o[d] *= corr;
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const uint16_t* v0 = v_s + (32 * m + 4 * kg + tr_key) * kStr + 16 * d + tr_dim;
                    const v4bf lo = lds_read_tr16(v0);
                    const v4bf hi = lds_read_tr16(v0 + 16 * kStr);
                    const v8bf va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[m], o[d], 0, 0, 0);
                }
            }
        }
        if (tile + 1 < ntiles) {
            __syncthreads();                     // every wave is done with this tile
            stage();
            w0 = pw0;
            w1 = pw1;
        }
        __syncthreads();
    }

    const float l_tot = wave_sum_xor_16_32(l_part);
    if (!live_q) return;
    // o[d][i] = O^T[dim 16d + 4kg + i][query col]
    uint16_t* outp = static_cast<uint16_t*>(a.out) + (static_cast<size_t>(row) * a.Hq + h) * 128;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) outp[16 * d + 4 * kg + i] = f32_to_bf16_bits(o[d][i] * inv);
    if (kg == 0 && a.lse)
        a.lse[static_cast<size_t>(row) * a.Hq + h] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * kLn2 : -__builtin_inff();
}

bool attn_masked_eligible(const AttnArgs& a) {
    if (!(a.dtype == BF16 && !a.latent && a.dqk == 128 && a.dv == 128)) return false;
    if (a.n_q < kQB || a.n_k > kMaskedMaxKeys) return false;
    // a key tile is shared by the block's 64 queries: worth it once a row keeps
    // more than 1/64 of what it sees (the average prefix of this problem)
    const double avg_vis = static_cast<double>(a.n_k) - 0.5 * a.n_q;
    return static_cast<double>(a.kk) * kQB >= avg_vis;
}

size_t attn_masked_workspace_bytes(const AttnArgs& a) {
    return static_cast<size_t>(a.rows) * bitmap_words(a.n_k) * sizeof(uint32_t);
}

hipError_t launch_attn_masked(const AttnArgs& a, uint32_t* bm, hipStream_t st) {
    const int words = bitmap_words(a.n_k);
    const size_t lds = static_cast<size_t>(words) * sizeof(uint32_t);   // <= 32 KiB
    hipLaunchKernelGGL(k_sel_bitmap, dim3(a.rows), dim3(256), lds, st, a, bm, words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int B = a.rows / a.n_q;
    const dim3 grid((a.n_q + kQB - 1) / kQB, a.Hq, B);
    hipLaunchKernelGGL(k_attn_masked_d128, grid, dim3(256), 0, st, a, static_cast<const uint32_t*>(bm), words);
    return hipGetLastError();
}

}  // namespace dsa
