// attn_masked.hip -- sparse attention for prefill as masked dense MFMA tiles.
//
// Short sequences run DSA through a masked MHA mode ("DeepSeek-V3.2-Exp
// 稀疏注意力机制(DSA)技术深度解析", sheratonhq.com, section 1).  The result is the
// same attention over each query's selected keys: a softmax over the keys a
// mask admits equals the softmax over the kept subset.  In prefill, the
// selections of neighbouring queries overlap so much that reading every key
// tile once per block of 256 queries moves far fewer bytes than gathering k
// rows per query (a row kept by 1/256 of the queries of a block is already
// cheaper as a tile), so prefill rows take this path:
//   bitmap  one workgroup per query row turns its index list into a bit row
//           over the keys (bit s set <=> s kept);
//   attend  one workgroup per (block of 256 queries, query head), 8 waves of
//           32 queries each, walks the key tiles of 64 up to the block's
//           last visible key.  Per tile and wave: S^T = K Q^T on
//           v_mfma_f32_32x32x16_bf16 (K from LDS, Q^T in registers), the
//           query's bits mask S, online softmax per lane (query l%32, half
//           of the tile's keys; the other half sits in lane l^32) in fp32,
//           then O^T += V^T P^T, also on v_mfma_f32_32x32x16_bf16, with V^T
//           read from the row-major V tile by transposing LDS reads.  A wave
//           skips a tile none of its queries keeps a key of.
// When every row keeps all its visible keys (top_k >= pos(t) + 1, or the
// dense causal attention entry) the mask is causal only: no bit rows are built
// or read, and the same kernel is plain causal flash attention.
#include "dsa_device.h"
#include "dsa_kernels.h"

namespace dsa {

namespace {
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kMW = 8;                 // waves per workgroup
constexpr int kQB = 32 * kMW;          // queries per workgroup (32 per wave)
constexpr int kLoadRows = 16 / kMW;    // 16-byte pieces of a 64-key K (and V) tile per thread
constexpr int kLoadStride = 4 * kMW;   // key rows between them
constexpr int kKB = 64;            // keys per tile
// LDS row strides (bf16), one bank pattern per access: the K tile is read a
// row per lane (16-byte reads; 68 words per row spread 16 rows over all 64
// banks), the V tile by the transposing reads (4 keys x 32 dims per 32 lanes;
// 80 words per row puts the 4 keys 16 banks apart)
constexpr int kStr = 136;          // K tile
constexpr int kStrV = 160;         // V tile
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

// Operand layouts of v_mfma_f32_32x32x16_bf16 (A 32x16, B 16x32, D 32x32):
// lane l holds A[l%32][8(l/32)+j] and B[8(l/32)+j][l%32] for j < 8, and
// D[8(r/4) + 4(l/32) + r%4][l%32] in result register r < 16.
//
// S^T (keys x queries) leaves lane l with query l%32 and, of each 32-key
// half of the tile, keys 8(r/4) + 4(l/32) + r%4.  In P.V the 16 keys of a
// chunk are taken in the order kappa = 8h + j <-> key 4h + j (j < 4) and
// 8 + 4h + (j - 4) (j >= 4), h = l/32, so the eight P values a lane already
// holds for a chunk are its B operand as they are.  The V^T operand (rows =
// 32 dims, columns = the same 16 kappa) comes from the row-major V tile with
// two ds_read_b64_tr_b16: within each 16-lane group, lane i of that
// instruction receives element i%4 of the 8-byte chunks addressed by lanes
// i/4, 4+i/4, 8+i/4 and 12+i/4, so lane a of the group addresses key
// (a/4) of the four and dims 4(a%4)..4(a%4)+3 of the group's 16 dims, and
// every lane ends with its own dim over the four keys.  The next tile's rows
// are fetched into registers while the current one is multiplied.
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// A pointer that is the same in every lane, held as such (buffer resources
// must be uniform, and the compiler cannot always prove it).
__device__ __forceinline__ void* uniform_ptr(const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// The 32 bits of keys key0..key0+31 that a causal mask admits for a query
// whose last visible key is pos.
__device__ __forceinline__ uint32_t causal_word(int pos, int key0) {
    const int n = pos - key0 + 1;
    return n <= 0 ? 0u : (n >= 32 ? 0xFFFFFFFFu : ((1u << n) - 1u));
}

// DENSE: every query keeps all its visible keys; the mask is causal and no
// bit rows are read (bm may be null).
// With ks > 1 the key tiles of each block are split into ks ranges of tps
// tiles (blockIdx.z = b * ks + range) and each workgroup leaves its (max,
// sum, unnormalised O) record per (row, head) in part for k_attn_merge.
template <bool DENSE>
__global__ __launch_bounds__(64 * kMW) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_masked_d128(
    AttnArgs a, const uint32_t* bm, int words, int ks, int tps, float* part) {
    // two buffers: the next tile is staged into one while the other is read
    // (one barrier per tile)
    __shared__ __align__(16) uint16_t k_all[2 * kKB * kStr];
    __shared__ __align__(16) uint16_t v_all[2 * kKB * kStrV];
    __shared__ int last_s[kMW];

    // A stream = (sequence, key range, head): its query blocks read the same
    // key tiles.  Consecutive workgroup ids go to the 8 XCDs in turn; when the
    // streams divide by 8, stream sg and all its query blocks are given to
    // XCD sg % 8, back to back, so the blocks in flight on an XCD walk the
    // same tiles through its L2 (longest block first within a stream).
    const int nqb = (a.n_q + kQB - 1) / kQB;
    const int streams = (a.rows / a.n_q) * ks * a.Hq;
    int sg, j;
    {
        const int id = blockIdx.x;
        if ((streams & 7) == 0) {
            const int k8 = id >> 3;
            sg = (k8 / nqb) * 8 + (id & 7);
            j = k8 % nqb;
        } else {
            sg = id / nqb;
            j = id % nqb;
        }
    }
    const int qb = nqb - 1 - j;
    const int h = sg % a.Hq;
    const int split = (sg / a.Hq) % ks;
    const int b = sg / (a.Hq * ks);
    const int G = a.Hq / a.Hkv;
    const int g = h / G;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int qc = lane & 31;                   // this lane's query (S^T column)
    const int hh = lane >> 5;                   // which half of each 32-key block it holds
    const float zscale = a.scale * kLog2e;

    const int t = qb * kQB + wave * 32 + qc;
    const bool live_q = t < a.n_q;
    const int row = b * a.n_q + (live_q ? t : 0);
    const int pos = live_q ? row_pos(a.q_pos, row, a.n_q, a.n_k) : -1;

    // the block's last visible key bounds the tile walk
    int mp = pos;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) mp = max(mp, __shfl_xor(mp, o));
    if (lane == 0) last_s[wave] = mp;

    // Q^T operand of every 16-dim chunk: query qc, dims 16c + 8hh .. +7
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + (static_cast<size_t>(row) * a.Hq + h) * 128 + 8 * hh;
    v8bf qv[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const v8bf x = *reinterpret_cast<const v8bf*>(qp + 16 * c);
        qv[c] = live_q ? x : v8bf{};
    }
    __syncthreads();
    // (uniform; read from LDS, so named uniform for the tile offsets below)
    int last_all = last_s[0];
#pragma unroll
    for (int w = 1; w < kMW; ++w) last_all = max(last_all, last_s[w]);
    const int last = __builtin_amdgcn_readfirstlane(last_all);
    // this workgroup's key tiles [t0, t1) of the block's walk
    const int ntiles = last < 0 ? 0 : last / kKB + 1;
    // (held in scalar registers, so the tile loop, its buffer index and the
    // tile offsets below are scalar work)
    const int t0 = __builtin_amdgcn_readfirstlane(split * tps);
    const int t1 = __builtin_amdgcn_readfirstlane(min(ntiles, t0 + tps));

    const uint16_t* kp = static_cast<const uint16_t*>(a.k);
    const uint16_t* vp = static_cast<const uint16_t*>(a.v);
    const size_t rstride = static_cast<size_t>(a.Hkv) * 128;
    const uint16_t* kbase = kp + static_cast<size_t>(b) * a.n_k * rstride + g * 128;
    const uint16_t* vbase = vp + static_cast<size_t>(b) * a.n_k * rstride + g * 128;
    const uint32_t* brow = DENSE ? nullptr : bm + static_cast<size_t>(row) * words;

    // loader: 256 threads x 4 rows x 16 B of K and of V per tile, as buffer
    // loads with a fixed per-thread offset within the tile.  Each tile gets
    // its own resources, based at the tile's first row and ending at the
    // sequence's last row (the range check covers the per-thread offset only,
    // not a scalar offset), so rows past n_k read as zeros whatever memory
    // follows the tensor.  One sequence's K or V spans n_k * Hkv * 256 bytes,
    // below 2^31: masked_kv_fits is part of every way into these kernels.
    const int lrow = threadIdx.x >> 4;          // 0..4*kMW-1, plus kLoadStride per step
    const int lcol = (threadIdx.x & 15) * 8;    // bf16 offset within the 128-wide row
    const int row_bytes = static_cast<int>(rstride) * 2;
    const int kv_bytes = __builtin_amdgcn_readfirstlane((a.n_k - 1) * row_bytes + 256);
    const unsigned char* kbytes = static_cast<const unsigned char*>(uniform_ptr(kbase));
    const unsigned char* vbytes = static_cast<const unsigned char*>(uniform_ptr(vbase));
    int voff[kLoadRows];
#pragma unroll
    for (int r = 0; r < kLoadRows; ++r) voff[r] = (lrow + kLoadStride * r) * row_bytes + lcol * 2;
    v8bf pk[kLoadRows], pv[kLoadRows];
    uint32_t pw0 = 0u, pw1 = 0u;
    auto fetch = [&](int tile) {
        // tile * 64 <= n_k - 1, so the tile's offset is below kv_bytes
        const int toff = __builtin_amdgcn_readfirstlane(tile * kKB * row_bytes);
        const int rem = __builtin_amdgcn_readfirstlane(kv_bytes - toff);
        const __amdgpu_buffer_rsrc_t kr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(kbytes + toff), 0, rem, kBufferWord3);
        const __amdgpu_buffer_rsrc_t vr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(vbytes + toff), 0, rem, kBufferWord3);
#pragma unroll
        for (int r = 0; r < kLoadRows; ++r) {
            const v4i xk = __builtin_amdgcn_raw_buffer_load_b128(kr, voff[r], 0, 0);
            const v4i xv = __builtin_amdgcn_raw_buffer_load_b128(vr, voff[r], 0, 0);
            __builtin_memcpy(&pk[r], &xk, sizeof xk);
            __builtin_memcpy(&pv[r], &xv, sizeof xv);
        }
        const int pkey0 = tile * kKB;
        uint32_t x0, x1;
        if constexpr (DENSE) {
            x0 = causal_word(pos, pkey0);
            x1 = causal_word(pos, pkey0 + 32);
        } else {
            x0 = brow[2 * tile];
            x1 = brow[2 * tile + 1];
        }
        pw0 = live_q ? x0 : 0u;
        pw1 = live_q ? x1 : 0u;
    };
    auto stage = [&](int buf) {
        uint16_t* ks = k_all + buf * kKB * kStr;
        uint16_t* vs = v_all + buf * kKB * kStrV;
#pragma unroll
        for (int r = 0; r < kLoadRows; ++r) {
            const int kr = lrow + kLoadStride * r;
            *reinterpret_cast<v8bf*>(&ks[kr * kStr + lcol]) = pk[r];
            *reinterpret_cast<v8bf*>(&vs[kr * kStrV + lcol]) = pv[r];
        }
    };
    // this lane's addresses for the transposing V reads: group dims 16*(lane/16 % 2),
    // key (a/4) of the quadruple, dims 4(a%4)..+3
    const int ga = lane & 15;
    const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (ga & 3);
    const int tr_key = 4 * hh + (ga >> 2);

    float m_ref = -__builtin_inff();            // reference max of the raw scores
    float l_part = 0.0f;
    v16f o[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) o[d] = v16f{};

    if (t1 > t0) {
        fetch(t0);
        stage(0);
    }
    uint32_t w0 = pw0, w1 = pw1;
    __builtin_amdgcn_s_waitcnt(0);              // prologue loads landed (see the indexer's tile loop)
    __syncthreads();
    int buf = 0;
    for (int tile = t0; tile < t1; ++tile) {
        fetch(tile + 1 < t1 ? tile + 1 : tile);   // in flight during the multiply
        const uint16_t* k_s = k_all + buf * kKB * kStr;
        const uint16_t* v_s = v_all + buf * kKB * kStrV;
        const bool any = __ballot((w0 | w1) != 0u) != 0ull;
        if (any) {                               // uniform per wave
            v16f sa = v16f{}, sb = v16f{};       // S^T of keys 0..31 and 32..63
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const v8bf ka = *reinterpret_cast<const v8bf*>(k_s + qc * kStr + 16 * c + 8 * hh);
                const v8bf kb = *reinterpret_cast<const v8bf*>(k_s + (32 + qc) * kStr + 16 * c + 8 * hh);
                sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qv[c], sa, 0, 0, 0);
                sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qv[c], sb, 0, 0, 0);
            }
            // The softmax below runs at raised wave priority and P.V at the
            // normal one, so where one SIMD's two waves (of different
            // workgroups) reach these parts at once, the VALU work issues
            // first while the other wave's MFMAs keep the matrix core busy.
            __builtin_amdgcn_s_setprio(1);
            // the query's bits: key 8(r/4) + 4hh + r%4 of each half; a
            // sign-extended one-bit field selects the score or -inf
            const int ma = static_cast<int>(w0 >> (4 * hh)), mb = static_cast<int>(w1 >> (4 * hh));
            const uint32_t ninf = __float_as_uint(-__builtin_inff());
            float bmax = -__builtin_inff();
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int bit = 8 * (r >> 2) + (r & 3);
                const uint32_t ka = static_cast<uint32_t>(__builtin_amdgcn_sbfe(ma, bit, 1));
                const uint32_t kb = static_cast<uint32_t>(__builtin_amdgcn_sbfe(mb, bit, 1));
                sa[r] = __uint_as_float((__float_as_uint(sa[r]) & ka) | (ninf & ~ka));
                sb[r] = __uint_as_float((__float_as_uint(sb[r]) & kb) | (ninf & ~kb));
                bmax = fmaxf(fmaxf(bmax, sa[r]), sb[r]);   // one v_max3_f32
            }
            bmax = pair32_max(bmax);
            // Everything below runs on every lane (the MFMAs and transposing
            // reads take their operands from all of them).  The exponents use
            // a reference max m_ref that moves only when a query's max rises
            // more than 2^8 above it (any reference gives the same softmax;
            // p <= 256 stays exact enough in bf16 and far from overflow), so O
            // is rarely rescaled; a query with no kept key yet gets p = 0.
            const float m_new = fmaxf(m_ref, bmax);
            const bool move = m_new != -__builtin_inff() && (m_ref == -__builtin_inff() ||
                                                             (m_new - m_ref) * zscale > 8.0f);
            float corr = 1.0f;
            if (__ballot(move) != 0ull) {         // uniform per wave
                const float m_to = move ? m_new : m_ref;
                corr = m_ref == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f((m_ref - m_to) * zscale);
                m_ref = m_to;
                l_part *= corr;
#pragma unroll
                for (int d = 0; d < 4; ++d) o[d] *= corr;
            }
            const float mz = m_ref == -__builtin_inff() ? 0.0f : m_ref * zscale;
            {
                float psum = 0.0f;
                v8bf pb[4];
                const v2bf kOnes2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float pa0 = __builtin_amdgcn_exp2f(fmaf(sa[r], zscale, -mz));
                    const float pa1 = __builtin_amdgcn_exp2f(fmaf(sa[r + 1], zscale, -mz));
                    const float pc0 = __builtin_amdgcn_exp2f(fmaf(sb[r], zscale, -mz));
                    const float pc1 = __builtin_amdgcn_exp2f(fmaf(sb[r + 1], zscale, -mz));
                    // pairs convert with one v_cvt_pk_bf16_f32 (round to nearest even)
                    const v2bf qa = __builtin_convertvector((v2f){pa0, pa1}, v2bf);
                    const v2bf qc = __builtin_convertvector((v2f){pc0, pc1}, v2bf);
                    // the denominator sums the same bf16 weights P.V multiplies,
                    // two per v_dot2c_f32_bf16
                    psum = __builtin_amdgcn_fdot2_f32_bf16(qa, kOnes2, psum, false);
                    psum = __builtin_amdgcn_fdot2_f32_bf16(qc, kOnes2, psum, false);
                    pb[r >> 3][r & 7] = qa[0];               // keys 0..31: chunks 0, 1
                    pb[r >> 3][(r & 7) + 1] = qa[1];
                    pb[2 + (r >> 3)][r & 7] = qc[0];         // keys 32..63: chunks 2, 3
                    pb[2 + (r >> 3)][(r & 7) + 1] = qc[1];
                }
                l_part += psum;
                __builtin_amdgcn_s_setprio(0);
#pragma unroll
                for (int c16 = 0; c16 < 4; ++c16) {
                    const uint16_t* vr = v_s + (16 * c16 + tr_key) * kStrV + tr_dim;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const v4bf lo = lds_read_tr16(vr + 32 * d);
                        const v4bf hi = lds_read_tr16(vr + 8 * kStrV + 32 * d);
                        const v8bf va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[c16], o[d], 0, 0, 0);
                    }
                }
            }
        }
        // the other buffer was last read before the previous barrier
        if (tile + 1 < t1) {
            stage(buf ^ 1);
            w0 = pw0;
            w1 = pw1;
            buf ^= 1;
        }
        __syncthreads();
    }

    const float l_tot = pair32_sum(l_part);
    if (!live_q) return;
    // o[d][r] = O^T[dim 32d + 8(r/4) + 4hh + r%4][query qc]
    if (ks > 1) {
        float* rec = part + ((static_cast<size_t>(row) * a.Hq + h) * ks + split) * (128 + 2);
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                float4 v;
                v.x = o[d][4 * q4]; v.y = o[d][4 * q4 + 1]; v.z = o[d][4 * q4 + 2]; v.w = o[d][4 * q4 + 3];
                // dims 32d + 8 q4 + 4hh .. +3; the record's O starts 2 floats in
                float* dst = rec + 2 + 32 * d + 8 * q4 + 4 * hh;
                dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
            }
        if (hh == 0) {
            rec[0] = m_ref == -__builtin_inff() ? -__builtin_inff() : m_ref * zscale;
            rec[1] = l_tot;
        }
        return;
    }
    uint16_t* outp = static_cast<uint16_t*>(a.out) + (static_cast<size_t>(row) * a.Hq + h) * 128 + 4 * hh;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            uint16_t v4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v4[i] = f32_to_bf16_bits(o[d][4 * q4 + i] * inv);
            uint2 pk2;
            pk2.x = static_cast<uint32_t>(v4[0]) | (static_cast<uint32_t>(v4[1]) << 16);
            pk2.y = static_cast<uint32_t>(v4[2]) | (static_cast<uint32_t>(v4[3]) << 16);
            *reinterpret_cast<uint2*>(outp + 32 * d + 8 * q4) = pk2;
        }
    if (hh == 0 && a.lse)
        a.lse[static_cast<size_t>(row) * a.Hq + h] = l_tot > 0.0f ? (m_ref * zscale + log2f(l_tot)) * kLn2 : -__builtin_inff();
}

// Costs that choose between the two forms in ATTN_AUTO, from rates measured
// on MI355X (bf16, d = 128, cold caches): gathering rows of K and V (512 B
// per kept (row, kv head, key)) runs at about 5.5 TB/s; the masked walk reads
// every key tile up to a query block's last visible key once per query head
// (about 4.5 TB/s) and does the dense tile math at about 800 TFLOP/s,
// whichever is longer.  With few query rows per sequence the walk's reads
// dominate and gathering wins; with GQA one gathered row serves all the
// heads of its group, which the per-head walk does not share.
static double gather_cost_us(const AttnArgs& a) {
    const double kept = static_cast<double>(a.rows) * (a.all_visible ? 0.5 * a.n_k : a.kk);
    return kept * a.Hkv * 512.0 / 5.5e6;
}
static double masked_cost_us(const AttnArgs& a) {
    // The rates were fitted with the walk counted per 128 queries; the kernel
    // now walks per 256 (faster on long prefills), but counting per 256 halves
    // the modelled bytes of a short chunk and picks the walk where gathering
    // measured faster (GQA chunks of 256-1024 queries over 32K keys), so the
    // count stays per 128.
    constexpr int kCostQB = 128;
    const int B = a.rows / a.n_q;
    const int nqb = (a.n_q + kCostQB - 1) / kCostQB;
    // key rows walked per query block: up to its last query's position
    // (q_pos unknown on the host: n_k - n_q + t, the usual layout)
    double walked = 0.0;
    for (int qb = 0; qb < nqb; ++qb) {
        const int t_last = (qb + 1) * kCostQB < a.n_q ? (qb + 1) * kCostQB - 1 : a.n_q - 1;
        walked += static_cast<double>(a.n_k - a.n_q + t_last + 1);
    }
    const double bytes = static_cast<double>(B) * a.Hq * walked * 512.0;
    const double flops = 4.0 * 128.0 * a.Hq * static_cast<double>(B) * kCostQB * walked;
    const double t_bytes = bytes / 4.5e6, t_flops = flops / 8.0e8;
    return t_bytes > t_flops ? t_bytes : t_flops;
}

bool attn_masked_eligible(const AttnArgs& a) {
    if (!(a.dtype == BF16 && a.kv_dtype == BF16 && !a.latent && a.dqk == 128 && a.dv == 128)) return false;
    if (!masked_kv_fits(a.n_k, a.Hkv)) return false;
    if (a.mode == ATTN_GATHER) return false;
    if (a.all_visible)                                       // causal mask, no bit rows
        return a.mode == ATTN_MASKED || masked_cost_us(a) < gather_cost_us(a);
    if (a.n_k > kMaskedMaxKeys) return false;
    if (a.mode == ATTN_MASKED) return true;
    return masked_cost_us(a) < gather_cost_us(a);
}

#ifndef DSA_MASKED_TARGET_WGS
#define DSA_MASKED_TARGET_WGS 512
#endif
// Key-tile ranges per query block: with few (query block, head) pairs the
// walk over the keys is split so that about two workgroups run per compute
// unit, each range at least 8 tiles long.
static int masked_splits(const AttnArgs& a) {
    const int64_t wgs = static_cast<int64_t>((a.n_q + kQB - 1) / kQB) * a.Hq * (a.rows / a.n_q);
    const int tiles = (a.n_k + kKB - 1) / kKB;
    int s = static_cast<int>((DSA_MASKED_TARGET_WGS + wgs - 1) / wgs);
    const int max_s = tiles / 8 > 64 ? 64 : tiles / 8;
    if (s > max_s) s = max_s;
    return s < 1 ? 1 : s;
}

static size_t bitmap_bytes(const AttnArgs& a) {
    return a.all_visible ? 0 : (static_cast<size_t>(a.rows) * bitmap_words(a.n_k) * sizeof(uint32_t) + 255) & ~size_t(255);
}

size_t attn_masked_workspace_bytes(const AttnArgs& a) {
    // the bit rows (none when every row keeps all its visible keys), then the
    // split records
    const int s = masked_splits(a);
    const size_t recs = s > 1 ? static_cast<size_t>(a.rows) * a.Hq * s * (128 + 2) * sizeof(float) : 0;
    return bitmap_bytes(a) + recs;
}

hipError_t launch_attn_masked(const AttnArgs& a, void* ws, hipStream_t st) {
    const int B = a.rows / a.n_q;
    const int s = masked_splits(a);
    const int tiles = (a.n_k + kKB - 1) / kKB;
    const int tps = (tiles + s - 1) / s;
    uint32_t* bm = static_cast<uint32_t*>(ws);
    float* part = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) + bitmap_bytes(a));
    const dim3 grid(static_cast<unsigned>((a.n_q + kQB - 1) / kQB) * a.Hq * B * s);
    hipError_t e;
    if (a.all_visible) {
        hipLaunchKernelGGL(k_attn_masked_d128<true>, grid, dim3(64 * kMW), 0, st, a,
                           static_cast<const uint32_t*>(nullptr), 0, s, tps, part);
    } else {
        const int words = bitmap_words(a.n_k);
        const size_t lds = static_cast<size_t>(words) * sizeof(uint32_t);   // <= 32 KiB
        hipLaunchKernelGGL(k_sel_bitmap, dim3(a.rows), dim3(256), lds, st, a, bm, words);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(k_attn_masked_d128<false>, grid, dim3(64 * kMW), 0, st, a,
                           static_cast<const uint32_t*>(bm), words, s, tps, part);
    }
    if ((e = hipGetLastError()) != hipSuccess || s == 1) return e;
    return launch_attn_merge(a, s, part, st);
}

}  // namespace dsa
