// Device helpers shared by the decode and prefill kernels (gfx950).
#pragma once

#include "plx_internal.h"

namespace plx {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    __bf16 h = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// quad_perm [0,0,2,2]: every lane receives the even lane of its pair.
__device__ __forceinline__ float dpp_pair_even(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xA0, 0xf, 0xf, false));
}

// Reductions over the four lanes n, n+16, n+32, n+48 (the four 16-lane rows
// of a wave), with gfx950's v_permlane32_swap / v_permlane16_swap: swapping a
// value with itself leaves each lane holding its own and its partner's value
// (partner = lane ^ 32, then lane ^ 16), all in VALU, no LDS round trip.
__device__ __forceinline__ float xor_max_rowgroups(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor_sum_rowgroups(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over each group of LPR consecutive lanes (LPR = 8, 16 or 32), every lane
// of the group receiving it: DPP exchanges within rows of 16 lanes (partners
// lane ^ 1, lane ^ 2, then the mirrored half-row and row, which hold the same
// partial sums as lane ^ 4 and lane ^ 8), then gfx950's permlane16 swap for
// the partner row. All VALU; the pairing is that of an xor butterfly.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(LPR == 8 || LPR == 16 || LPR == 32, "group of 8, 16 or 32 lanes");
    x += dpp_f32<0xb1>(x);   // quad_perm [1, 0, 3, 2]
    x += dpp_f32<0x4e>(x);   // quad_perm [2, 3, 0, 1]
    x += dpp_f32<0x141>(x);  // row_half_mirror
    if constexpr (LPR >= 16) x += dpp_f32<0x140>(x);  // row_mirror
    if constexpr (LPR >= 32) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    return x;
}

__device__ __forceinline__ bf16x8 load16(const uint16_t *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

// How far (log2 units) a tile's max may exceed the running reference max
// before the accumulators are rescaled.
constexpr float kRescaleSlack = 8.0f;

// Probe pivot re-basing. The matrix-core kernels accumulate B = sum e (s - pi) v
// from bf16 operands e (s - pi), and A = sum e v from bf16 e; the output
// (A (1 - (sbar - pi)) + B) / l then carries the rounding of each key's e
// multiplied by |sbar - pi| and that of e (s - pi) by |s - pi|. The pivot
// starts at 0 and follows the running weighted mean of s: after a tile's
// weights are formed (before they are rounded), a lane whose partial sums have
// |S| > kPivotDrift * l (S = sum e (s - pi), l = sum e over its keys, s in
// probe-scale units) triggers a re-base of its row onto the row's running mean
// d = S_row / l_row:  pi += d,  S -= d l,  B -= d A,  and the tile's
// e (s - pi) -= d e. Exact in real arithmetic. If the row's mean is off by
// more than the threshold, at least one lane's partial mean is, so no needed
// re-base is missed. Inputs whose probe scores stay within the threshold of 0
// (as with keys and probes of unit total variance) never re-base.
constexpr float kPivotDrift = 1.0f;

// Word 3 of a raw buffer resource for gfx9-family (CDNA) untyped loads.
constexpr int kBufferFlags = 0x00020000;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load at byte `voffset` of a buffer; past the buffer's range it
// returns zeros. The KV stream is read once, so it is fetched non-temporal.
// The loads are marked volatile (bit 31 of the policy operand, a compiler
// flag) so that they are issued where they are written: otherwise the
// compiler sinks a prefetch down to its first use and the pipelining is lost.
constexpr int kStreamPolicy = 2 | (int)(1u << 31);  // nt, volatile
__device__ __forceinline__ bf16x8 buffer_load16(__amdgpu_buffer_rsrc_t rs, int voffset) {
    u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rs, voffset, 0, kStreamPolicy);
    return __builtin_bit_cast(bf16x8, w);
}
// Same, cached normally (data that other workgroups read again).
constexpr int kReusePolicy = (int)(1u << 31);  // volatile only
__device__ __forceinline__ u32x4 buffer_load16_cached(__amdgpu_buffer_rsrc_t rs, int voffset) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, voffset, 0, kReusePolicy);
}

// Prefill tensors are dense [B, H, L, D] (cu == nullptr) or packed [T, H, D]
// with sequence b at tokens cu[b] .. cu[b+1] - 1. Row i of head h of sequence
// b starts at element row0_elem(...) + i * row_stride(...); the row
// statistics (lse, sbar) are dense [B, H, L] or packed [T, H].
struct PrefillSeq {
    int tok0;  // first token of the sequence (packed), 0 (dense)
    int len;
    bool packed;
};
__device__ __forceinline__ PrefillSeq prefill_seq(const int32_t *cu, int b, int L) {
    PrefillSeq s;
    s.packed = cu != nullptr;
    s.tok0 = s.packed ? cu[b] : 0;
    s.len = s.packed ? cu[b + 1] - s.tok0 : L;
    return s;
}
__device__ __forceinline__ int64_t row0_elem(const PrefillSeq &s, int b, int h, int H, int L, int D) {
    return s.packed ? ((int64_t)s.tok0 * H + h) * D : ((int64_t)b * H + h) * L * D;
}
__device__ __forceinline__ int row_stride(const PrefillSeq &s, int H, int D) { return s.packed ? H * D : D; }
__device__ __forceinline__ int64_t stat0(const PrefillSeq &s, int b, int h, int H, int L) {
    return s.packed ? (int64_t)s.tok0 * H + h : ((int64_t)b * H + h) * L;
}
__device__ __forceinline__ int stat_stride(const PrefillSeq &s, int H) { return s.packed ? H : 1; }

// Block-sparse tile scan: the first tile u >= t (u < n) with vis(u), or n.
// Every lane of the wave evaluates vis for one of 64 consecutive tiles at a
// time; the wave keeps their ballot in (bits, base) between calls (start
// with base = -64), so a sweep over n tiles reads each mask byte once.
// Wave-uniform result.
template <typename Vis>
__device__ __forceinline__ int next_visible(int t, int n, uint64_t &bits, int &base, const Vis &vis) {
    while (t < n) {
        if (t < base || t >= base + 64) {
            base = t;
            const int u = t + (int)(threadIdx.x & 63);
            bits = __builtin_amdgcn_ballot_w64(u < n && vis(u));
        }
        const uint64_t rest = bits >> (t - base);
        if (rest) return t + (int)__builtin_ctzll(rest);
        t = base + 64;
    }
    return n;
}

// Dynamic work queue of a persistent launch (packed batches, whose grid would
// otherwise hold a workgroup for every (sequence, tile) slot up to the longest
// sequence). Workgroup w draws from the share of XCD x = w % 8 (consecutive
// workgroup ids are dispatched to consecutive XCDs): items x, x + 8, x + 16,
// ... in order, through counter x, so that the items of one (sequence, KV
// head) group stay on one XCD and its L2. Returns -1 when the share is
// exhausted. Two workgroup barriers; called by every thread.
__device__ __forceinline__ int next_item(int *counters, int n_items) {
    __shared__ int slot;
    const int x = blockIdx.x & 7;
    if (threadIdx.x == 0) slot = atomicAdd(&counters[x], 1);
    __syncthreads();
    const long item = (long)slot * 8 + x;
    __syncthreads();
    return item < n_items ? (int)item : -1;
}

}  // namespace plx
