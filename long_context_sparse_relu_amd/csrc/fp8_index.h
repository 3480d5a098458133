// fp8_index.h -- the FP8 lightning-indexer score of 16 keys at a time, shared
// by the streaming indexer, the top-k threshold sampler and the top-k
// recompute path, so that all of them produce bit-identical scores.
//
// One v_mfma_scale_f32_16x16x128_f8f6f4 multiplies a query row's heads (rows
// of A, up to 16) by 16 keys (columns of B) over the full 128-wide dot
// product.  Lane l feeds A row l%16 and B column l%16 with 32 code bytes:
// bytes [16g, 16g+16) and [64+16g, 64+16g+16) of the row, g = l/16.  A and B
// use the same byte->k assignment, so the contraction is exact whatever order
// the unit sums in, and each 16-byte load of a wave covers 64 contiguous bytes
// of every key row it touches.  The 16x16 result lands as
// acc[i] = dot(head 4g+i, key l%16); ReLU and the head weights fold each
// lane's four heads, one reduce-scatter over four blocks finishes the head
// sums (lane l ends with key l%16 of block l/16), and the positive per-token
// scales multiply last.
#pragma once

#include "dsa_device.h"

namespace dsa {

__device__ __forceinline__ v8i load_split32(const uint8_t* row, int g) {
    v4i lo = *reinterpret_cast<const v4i*>(row + 16 * g);
    v4i hi = *reinterpret_cast<const v4i*>(row + 64 + 16 * g);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Whole-line loads of 64 key rows (8 KiB) in the order the memory system
// streams best: instruction j brings keys base + 8j .. base + 8j + 7 whole,
// lane l holding bytes [16(l%8), +16) of key base + 8j + l/8, marked
// non-temporal (the keys are read once).  Key indices are clamped to lim.
// (Loads that cover only half of each 128-byte line, as load_split32's do,
// stream slower and lose more from the non-temporal hint.)
__device__ __forceinline__ void load_keys64_lines(const uint8_t* kb, int base, int lim, int lane, v4i* r) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int key = min(base + 8 * j + (lane >> 3), lim);
        r[j] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(kb + static_cast<size_t>(key) * 128) + (lane & 7));
    }
}

// The MFMA operand of keys base + 16u .. base + 16u + 15 out of those lines,
// exactly as load_split32 lays it out (lane (c, g) = (l%16, l/16) holds bytes
// [16g, +16) and [64 + 16g, +16) of key c): each dword is fetched from the
// lane that loaded it with ds_bpermute, from the line of keys 0-7 or 8-15 of
// the block.
__device__ __forceinline__ v8i keys_block_operand(const v4i* r, int u, int lane) {
    const int c = lane & 15, g = lane >> 4;
    const int a0 = (8 * (c & 7) + g) * 4, a1 = a0 + 16;     // byte addresses of the source lanes
    const bool upper = c >= 8;
    v8i out;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int x0 = __builtin_amdgcn_ds_bpermute(a0, r[2 * u][d]);
        const int y0 = __builtin_amdgcn_ds_bpermute(a0, r[2 * u + 1][d]);
        const int x1 = __builtin_amdgcn_ds_bpermute(a1, r[2 * u][d]);
        const int y1 = __builtin_amdgcn_ds_bpermute(a1, r[2 * u + 1][d]);
        out[d] = upper ? y0 : x0;
        out[4 + d] = upper ? y1 : x1;
    }
    return out;
}

// A query row's operands as one lane holds them.
struct Fp8Query {
    v8i a;        // head (lane % 16) code bytes, zero for heads >= H
    float w[4];   // weights of heads 4*(lane/16) + i
    float sq;     // the row's scale
};

// Every load is issued unconditionally (heads past H read head H-1 and are
// zeroed afterwards), so no branch separates the loads and one wait covers
// them together with whatever the caller loads next to them.
__device__ __forceinline__ Fp8Query load_fp8_query(const uint8_t* iq, const float* iq_scale, const float* iw,
                                                   int row, int H, int lane) {
    Fp8Query q;
    const int col = lane & 15, kg = lane >> 4;
    const v8i a = load_split32(iq + (static_cast<size_t>(row) * H + (col < H ? col : H - 1)) * 128, kg);
    float w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * kg + i;
        w[i] = iw[static_cast<size_t>(row) * H + (h < H ? h : H - 1)];
    }
    q.sq = iq_scale[row];
    q.a = col < H ? a : v8i{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) q.w[i] = 4 * kg + i < H ? w[i] : 0.0f;
    return q;
}

// This lane's operand bytes of key s (zeros when !live).
__device__ __forceinline__ v8i load_fp8_key(const uint8_t* kb, int s, bool live, int lane) {
    return live ? load_split32(kb + static_cast<size_t>(s) * 128, lane >> 4) : v8i{0, 0, 0, 0, 0, 0, 0, 0};
}

// Scores of four blocks of 16 keys.  bv[u] holds this lane's operand of key
// (lane % 16) of block u; the result in lane l is the score of key (l % 16) of
// block l / 16, and sk must be that key's scale.  Every lane of the wave must
// call it (the MFMAs and lane exchanges are wave-wide).
__device__ __forceinline__ float fp8_score4(const Fp8Query& q, const v8i* bv, float sk) {
    float p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(q.a, bv[u], acc, 0, 0, 0, 127, 0, 127);
        float part = q.w[0] * relu(acc[0]);
        part = fmaf(q.w[1], relu(acc[1]), part);
        part = fmaf(q.w[2], relu(acc[2]), part);
        p[u] = fmaf(q.w[3], relu(acc[3]), part);
    }
    return reduce_scatter4(p[0], p[1], p[2], p[3]) * (q.sq * sk);
}

}  // namespace dsa
