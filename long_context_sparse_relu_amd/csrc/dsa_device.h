// dsa_device.h -- device-side helpers shared by the libdsa kernels (gfx950).
//
// Storage formats: fp32, bfloat16 (upper half of a binary32 word) and OCP FP8
// E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
// infinity, S.1111.111 = NaN; largest finite value 448).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));

enum DType { F32 = 0, BF16 = 1, E4M3 = 2 };

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t rounding = 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>((u + rounding) >> 16);
}

// E4M3 code -> fp32 by rebuilding the binary32 fields.
__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
    uint32_t sign = static_cast<uint32_t>(c & 0x80) << 24;
    uint32_t e = (c >> 3) & 0xF;
    uint32_t m = c & 0x7;
    if (e == 0xF && m == 0x7) return __uint_as_float(0x7FC00000u);
    if (e == 0) {  // subnormal: m/8 * 2^-6 = m * 2^-9
        float mag = static_cast<float>(m) * 0.001953125f;
        return sign ? -mag : mag;
    }
    return __uint_as_float(sign | ((e + 120u) << 23) | (m << 20));
}

template <int DT>
__device__ __forceinline__ float load_as_f32(const void* base, size_t i) {
    if constexpr (DT == F32) return static_cast<const float*>(base)[i];
    else if constexpr (DT == BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
    else return e4m3_to_f32(static_cast<const uint8_t*>(base)[i]);
}

// Order-preserving map of fp32 onto uint32: a > b as floats <=> key(a) > key(b)
// as unsigned integers.  -0.0 is folded onto +0.0 first so equal numbers get
// equal keys.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// (order key << 32 | ~position): larger means higher score, then lower position.
__device__ __forceinline__ uint64_t composite64(uint32_t key, int s) {
    return (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(~static_cast<uint32_t>(s));
}

// Word 3 of a raw buffer resource (32-bit data format).  With stride 0 an
// access whose per-lane offset (plus the instruction's immediate offset) is at
// or past num_records bytes is out of range: a store there is dropped and a
// load returns zero.  The scalar offset operand is not part of that check.
constexpr int kBufferWord3 = 0x00020000;

// ReLU as the signed-integer max of the bit pattern with 0: a negative float
// (or -0.0) has the sign bit set and becomes +0.0, a positive one is kept.
// One VALU op, where fmaxf on an MFMA result also pays a NaN-quieting max.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

__device__ __forceinline__ int row_pos(const int32_t* q_pos, int row, int n_q, int n_k) {
    int t = row % n_q;
    int p = q_pos ? q_pos[row] : (n_k - n_q + t);
    return p < n_k - 1 ? p : n_k - 1;  // may be negative: nothing visible
}

// ds_read_b64_tr_b16: each lane addresses an 8-byte chunk (4 bf16) of LDS;
// within each 16-lane group, lane i receives element i%4 of the chunks
// addressed by lanes i/4, 4+i/4, 8+i/4 and 12+i/4 of the group, in that order.
// With lane a of a group addressing row a/4 of four rows at column 4(a%4),
// every lane ends with its own column of the four rows.
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

// Exchanges between the four 16-lane rows of a wave, on the VALU: with both
// operands equal, v_permlane16_swap leaves row r's lanes holding rows 2(r/2)
// and 2(r/2)+1 in its two results, and v_permlane32_swap does the same for
// the two halves, so one op plus one add combines lanes l and l^16 (l^32).
// The combined values are the same in every lane of a group and do not
// depend on the order of the two operands (IEEE add and max commute).
__device__ __forceinline__ float pair16_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair16_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Column sums of four 16x16 MFMA partials at once.  p[j] holds, in lane l,
// one partial of column l%16 of block j (the four 16-lane rows hold different
// partials of the same column).  v_permlane32_swap(X, Y) swaps X's upper half
// with Y's lower half, so the sum of its two results holds X's half-sums in
// the lower half and Y's in the upper; v_permlane16_swap(X, Y) swaps X's odd
// rows with Y's even rows, so the sum holds X's row-pair sums in the even rows
// and Y's in the odd ones.  Applied to (p0,p2), (p1,p3) and then to the two
// sums, lane 16j + c ends with the full sum over the four rows of column c of
// block j: one value per lane and 64 distinct columns in lane order.
__device__ __forceinline__ float reduce_scatter4(float p0, float p1, float p2, float p3) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p2), false, false);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(p1), __float_as_uint(p3), false, false);
    const float s02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const float s13 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
    auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Sum (max) over the lanes l, l^16, l^32, l^48: the four lanes holding the
// same column of a 16x16 MFMA result.
__device__ __forceinline__ float wave_sum_xor_16_32(float x) { return pair32_sum(pair16_sum(x)); }
__device__ __forceinline__ float wave_max_xor_16_32(float x) { return pair32_max(pair16_max(x)); }

}  // namespace dsa
