// Parallax decode kernels for gfx950 (MI355X).
//
// What is computed (PyPI README of parallax-kernel, "Decoding (CuTeDSL)";
// neuraltrendhub summary "What the paper found"): for each sequence b and
// query head h, with every cached key visible,
//   o = sum_j w_j v_j + sum_j w_j (s_j - sbar) v_j,
//   w = softmax(qk_scale q.k_j), s_j = rk_scale r.k_j, sbar = sum_j w_j s_j.
// The summary's "hardware-aware streaming kernel that reuses the same KV
// tiles as FlashAttention" is the design point kept here: each K tile is
// read from HBM once and feeds both score sets (q.k and r.k), each V tile
// once and feeds both readouts (sum e v and sum e s v).
//
// Streaming state per (query head, split), with a fixed pivot pi = the
// probe score of the sequence's first key (exact in real arithmetic, it
// keeps the fp32/bf16 sums small when all s share an offset):
//   m (log2 units), l = sum e, S = sum e (s - pi), A = sum e v,
//   B = sum e (s - pi) v,  and  o = (A + B - (S / l) A) / l.
// Two states merge as (m, l, S, A, B) -> max m and 2^(m_i - M)-weighted sums.
//
// Kernels:
//   decode_mfma_bf16_d128<G, PLX>  bf16, head_dim 128, G query heads per KV
//       head (1, 2, 4, 8). One wave per (KV head, split, sequence). Both
//       contractions on v_mfma_f32_16x16x32_bf16, no LDS at all:
//         scores   S^T[key, vec] = K_tile . [q_0, r_0, q_1, r_1, ...]^T
//         readout  O^T[dim, row] = V_tile^T . [p_0, p_0 s'_0, p_1, ...]^T
//       The key order inside each 16-key block is chosen so that the score
//       MFMA's output lands in exactly the lanes and register order the
//       readout MFMA wants for its B operand (see the lane map below), and
//       V's natural [key][dim] layout becomes the readout's A operand by an
//       8x8 16-bit transpose inside each lane's registers. K and V stream
//       with 128-bit loads, double-buffered in registers.
//   decode_generic<T, D, PLX>  fp32 or bf16, head_dim 64/128, any group size.
//       One wave per (query head, split, sequence), fp32 VALU.
//   decode_reduce<TO, D, PLX>  merges split records into o.
#include "plx_internal.h"

namespace plx {

namespace {

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

// row_shr:1 inside each 16-lane row: lane i receives lane i-1 (lane 0 of a row keeps 0).
__device__ __forceinline__ float dpp_row_shr1(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, false));
}
// row_shl:1 inside each 16-lane row: lane i receives lane i+1.
__device__ __forceinline__ float dpp_row_shl1(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x101, 0xf, 0xf, false));
}

__device__ __forceinline__ float xor_max_rowgroups(float x) {  // over lanes n, n+16, n+32, n+48
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}
__device__ __forceinline__ float xor_sum_rowgroups(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

__device__ __forceinline__ bf16x8 load16(const uint16_t *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

struct SeqRange {
    int64_t tok0;  // first token of the sequence in the K/V arrays
    int len;
};

__device__ __forceinline__ SeqRange seq_range(const DecodeArgs &a, int b) {
    SeqRange s;
    if (a.cu) {
        int c0 = a.cu[b], c1 = a.cu[b + 1];
        s.tok0 = c0;
        s.len = c1 - c0;
    } else {
        s.tok0 = (int64_t)b * a.kv_len;
        s.len = a.kv_len;
    }
    return s;
}

// -------------------------------------------------------------------------
// MFMA decode, bf16, head_dim 128.
//
// Lane map (lane = 16 * g + n, g = 0..3, n = 0..15):
//   n : column of both MFMAs -- vector / P-row n. With NR = 2 rows per
//       head (Parallax): n = 2h is head h's softmax row (q_h, then p_h),
//       n = 2h + 1 its probe row (r_h, then p_h (s_h - pi)). With NR = 1
//       (softmax baseline) n = h. Columns n >= NR*G are dead.
//   g : k-group. For the score MFMA it selects dims 8(g + 4u) .. +8 of
//       k-step u; for the readout MFMA it selects keys g + 4t, t = 0..7,
//       of the 32-key tile.
// Score MFMA for 16-key block kb: A row m <- key 16kb + (m >> 2) + 4(m & 3),
// so output row 4g + i is key 16kb + g + 4i = key g + 4t with t = 4kb + i:
// lane (g, n) receives vector n's scores for exactly the keys g + 4t that it
// supplies to the readout MFMA as element t of its B operand.
// Readout MFMA e (e = 0..7): A row m <- dim 8m + e, so output row 4g + i is
// dim 32g + 8i + e: lane (g, n) accumulates P-row n over dims 32g .. 32g+31.
// -------------------------------------------------------------------------
template <int G, bool PLX>
__global__ __launch_bounds__(64) void decode_mfma_bf16_d128(DecodeArgs a) {
    constexpr int D = 128;
    constexpr int NR = PLX ? 2 : 1;
    constexpr int NV = NR * G;
    static_assert(NV <= 16, "at most 16 live columns");
    const int lane = threadIdx.x;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int hkv = blockIdx.x;
    const int split = blockIdx.y;
    const int b = blockIdx.z;

    const SeqRange sr = seq_range(a, b);
    const int start = split * a.chunk;
    const bool live = n < NV;
    const int h = live ? n / NR : 0;  // head within the group
    const int kind = live ? n % NR : 0;
    const int hq = hkv * G + h;

    const uint16_t *qh = reinterpret_cast<const uint16_t *>(a.q);
    const uint16_t *rh = reinterpret_cast<const uint16_t *>(a.r);
    const uint16_t *kh = reinterpret_cast<const uint16_t *>(a.k);
    const uint16_t *vh = reinterpret_cast<const uint16_t *>(a.v);

    if (sr.len <= 0 || start >= sr.len) {
        // Nothing to stream: a fused call writes the zero output of an empty
        // sequence, otherwise the record is marked empty for the merge.
        if (live && kind == 0) {
            if (a.fused) {
                uint16_t *o = reinterpret_cast<uint16_t *>(a.o) + ((int64_t)b * a.Hq + hq) * D + 32 * g;
                uint4 z = {0u, 0u, 0u, 0u};
                for (int c = 0; c < 4; ++c) reinterpret_cast<uint4 *>(o)[c] = z;
            } else if (g == 0) {
                float *rec = a.ws + (((int64_t)b * a.Hq + hq) * a.splits + split) * partial_floats(D);
                reinterpret_cast<float4 *>(rec + 2 * D)[0] = float4{-INFINITY, 0.f, 0.f, 0.f};
            }
        }
        return;
    }
    const int end = min(start + a.chunk, sr.len);

    // B operand of the score MFMA: vector n, dims 8(g + 4u) .. +8.
    bf16x8 qr[4];
    {
        const uint16_t *src = (kind == 0 ? qh : rh) + ((int64_t)b * a.Hq + hq) * D;
        for (int u = 0; u < 4; ++u) {
            if (live) {
                qr[u] = load16(src + 8 * (g + 4 * u));
            } else {
                for (int e = 0; e < 8; ++e) qr[u][e] = (__bf16)0.0f;
            }
        }
    }

    const int64_t tok_stride = (int64_t)a.Hkv * D;  // elements between consecutive tokens
    const uint16_t *kseq = kh + sr.tok0 * tok_stride + (int64_t)hkv * D;
    const uint16_t *vseq = vh + sr.tok0 * tok_stride + (int64_t)hkv * D;

    // Pivot pi = rk_scale * r_h . k_0 on the probe lanes (same for every split).
    float piv = 0.0f;
    if (PLX) {
        float part = 0.0f;
        for (int u = 0; u < 4; ++u) {
            bf16x8 k0 = load16(kseq + 8 * (g + 4 * u));
            for (int e = 0; e < 8; ++e) part += (float)qr[u][e] * (float)k0[e];
        }
        part = xor_sum_rowgroups(part);
        piv = part * a.rk_scale;
    }

    // Key permutation inside a 16-key block for the score MFMA's A operand.
    const int kperm = (n >> 2) + 4 * (n & 3);

    float m_run = -INFINITY;  // running max of the column's head (log2 units)
    float lsum = 0.0f;        // per-lane partial: sum p (n even) or sum p s' (n odd)
    floatx4 acc[8];
    for (int e = 0; e < 8; ++e) acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};

    bf16x8 kA[8], vA[8], kB[8], vB[8];

    auto load_tile = [&](int t0, bf16x8 *kt, bf16x8 *vt) {
        const int last = end - 1;
        for (int kb = 0; kb < 2; ++kb) {
            int key = min(t0 + 16 * kb + kperm, last);
            const uint16_t *p = kseq + (int64_t)key * tok_stride + 8 * g;
            for (int u = 0; u < 4; ++u) kt[4 * kb + u] = load16(p + 32 * u);
        }
        for (int t = 0; t < 8; ++t) {
            int key = min(t0 + g + 4 * t, last);
            vt[t] = load16(vseq + (int64_t)key * tok_stride + 8 * n);
        }
    };

    auto compute_tile = [&](int t0, const bf16x8 *kt, const bf16x8 *vt) {
        // ---- both score sets from one K tile
        floatx4 sc0 = {0.f, 0.f, 0.f, 0.f}, sc1 = {0.f, 0.f, 0.f, 0.f};
        for (int u = 0; u < 4; ++u) {
            sc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt[u], qr[u], sc0, 0, 0, 0);
            sc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt[4 + u], qr[u], sc1, 0, 0, 0);
        }
        float raw[8];
        for (int i = 0; i < 4; ++i) {
            raw[i] = sc0[i];
            raw[4 + i] = sc1[i];
        }
        // logits of the column's head: own value on softmax rows, the left
        // neighbour's (row 2h) on probe rows
        float z[8];
        const int nvalid = end - t0;  // keys g + 4t valid iff g + 4t < nvalid
        float tmax = -INFINITY;
        for (int t = 0; t < 8; ++t) {
            float zr = raw[t];
            if (PLX) {
                float left = dpp_row_shr1(zr);
                zr = kind ? left : zr;
            }
            z[t] = (g + 4 * t < nvalid) ? zr * a.zscale : -INFINITY;
            tmax = fmaxf(tmax, z[t]);
        }
        tmax = xor_max_rowgroups(tmax);
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float pv[8];
        float tsum = 0.0f;
        for (int t = 0; t < 8; ++t) {
            float p = __builtin_amdgcn_exp2f(z[t] - m_new);
            if (PLX && kind) p *= raw[t] * a.rk_scale - piv;
            p = live ? p : 0.0f;
            pv[t] = p;
            tsum += p;
        }
        lsum = lsum * alpha + tsum;
        bf16x8 pf;
        for (int t = 0; t < 8; ++t) pf[t] = (__bf16)pv[t];

        // ---- V^T operand: 8x8 16-bit transpose in registers.
        // vt[t] holds dims 8n..8n+7 of key g + 4t; vT[e] holds keys t = 0..7 of dim 8n + e.
        uint32_t tw[8][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 x = __builtin_bit_cast(uint4, vt[2 * j]);
            const uint4 y = __builtin_bit_cast(uint4, vt[2 * j + 1]);
            const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
            const uint32_t ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
            for (int d2 = 0; d2 < 4; ++d2) {
                tw[2 * d2][j] = (xs[d2] & 0xffffu) | (ys[d2] << 16);          // dim 2*d2
                tw[2 * d2 + 1][j] = (xs[d2] >> 16) | (ys[d2] & 0xffff0000u);  // dim 2*d2+1
            }
        }
        bf16x8 vT[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            vT[e] = __builtin_bit_cast(bf16x8, uint4{tw[e][0], tw[e][1], tw[e][2], tw[e][3]});
        // ---- rescale and accumulate both readouts from one V tile
        for (int e = 0; e < 8; ++e) {
            acc[e] *= alpha;
            acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vT[e], pf, acc[e], 0, 0, 0);
        }
    };

    int t0 = start;
    load_tile(t0, kA, vA);
    while (true) {
        if (t0 + 32 < end) load_tile(t0 + 32, kB, vB);
        compute_tile(t0, kA, vA);
        t0 += 32;
        if (t0 >= end) break;
        if (t0 + 32 < end) load_tile(t0 + 32, kA, vA);
        compute_tile(t0, kB, vB);
        t0 += 32;
        if (t0 >= end) break;
    }

    lsum = xor_sum_rowgroups(lsum);

    if (!a.fused) {
        if (!live) return;
        float *rec = a.ws + (((int64_t)b * a.Hq + hq) * a.splits + split) * partial_floats(D);
        float *dst = rec + kind * D + 32 * g;
        for (int i = 0; i < 4; ++i) {
            float4 lo = {acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
            float4 hi = {acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
            reinterpret_cast<float4 *>(dst + 8 * i)[0] = lo;
            reinterpret_cast<float4 *>(dst + 8 * i)[1] = hi;
        }
        if (g == 0) {
            if (kind == 0) {
                rec[2 * D + 0] = m_run;
                rec[2 * D + 1] = lsum;
                if (!PLX) {
                    rec[2 * D + 2] = 0.f;
                    rec[2 * D + 3] = 0.f;
                }
            } else {
                rec[2 * D + 2] = lsum;
                rec[2 * D + 3] = piv;
            }
        }
        return;
    }

    // One split: finalise here. Probe rows hand B and S to the softmax row on their left.
    float bsum[32];
    float s_tot = 0.0f;
    if (PLX) {
        for (int e = 0; e < 8; ++e)
            for (int i = 0; i < 4; ++i) bsum[8 * i + e] = dpp_row_shl1(acc[e][i]);
        s_tot = dpp_row_shl1(lsum);
    }
    if (!live || kind != 0) return;
    const float inv_l = 1.0f / lsum;
    const float cA = PLX ? (1.0f - s_tot * inv_l) : 1.0f;
    uint16_t *o = reinterpret_cast<uint16_t *>(a.o) + ((int64_t)b * a.Hq + hq) * D + 32 * g;
    for (int i = 0; i < 4; ++i) {
        float ov[8];
        for (int e = 0; e < 8; ++e) {
            float A = acc[e][i];
            ov[e] = PLX ? (A * cA + bsum[8 * i + e]) * inv_l : A * inv_l;
        }
        uint4 w = {pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3]), pack_bf16x2(ov[4], ov[5]),
                   pack_bf16x2(ov[6], ov[7])};
        reinterpret_cast<uint4 *>(o + 8 * i)[0] = w;
    }
}

// -------------------------------------------------------------------------
// Generic decode: fp32 or bf16 storage, head_dim 64 or 128, any group size.
// One wave per (query head, split, sequence). Lane = LPR * kgrp + c: the c-th
// 16-byte chunk of key kgrp + KPI*step. Each key group keeps its own
// streaming state; the groups merge through shuffles at the end.
// -------------------------------------------------------------------------
template <typename T>
struct Elem;
template <>
struct Elem<float> {
    static constexpr int per16 = 4;
    __device__ static void load(const float *p, float *out) {
        float4 x = *reinterpret_cast<const float4 *>(p);
        out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    }
    __device__ static void store(float *p, const float *in) {
        float4 x = {in[0], in[1], in[2], in[3]};
        *reinterpret_cast<float4 *>(p) = x;
    }
};
template <>
struct Elem<uint16_t> {
    static constexpr int per16 = 8;
    __device__ static void load(const uint16_t *p, float *out) {
        uint4 x = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = bf16_lo(w[i]);
            out[2 * i + 1] = bf16_hi(w[i]);
        }
    }
    __device__ static void store(uint16_t *p, const float *in) {
        uint4 x = {pack_bf16x2(in[0], in[1]), pack_bf16x2(in[2], in[3]), pack_bf16x2(in[4], in[5]),
                   pack_bf16x2(in[6], in[7])};
        *reinterpret_cast<uint4 *>(p) = x;
    }
};

template <int EPL>
struct State {
    float m, l, S;
    float A[EPL], B[EPL];
};

template <int EPL>
__device__ __forceinline__ void merge_state(State<EPL> &x, const State<EPL> &y) {
    const float M = fmaxf(x.m, y.m);
    if (M == -INFINITY) return;  // both empty
    const float ax = __builtin_amdgcn_exp2f(x.m - M);
    const float ay = __builtin_amdgcn_exp2f(y.m - M);
    x.m = M;
    x.l = x.l * ax + y.l * ay;
    x.S = x.S * ax + y.S * ay;
    for (int e = 0; e < EPL; ++e) {
        x.A[e] = x.A[e] * ax + y.A[e] * ay;
        x.B[e] = x.B[e] * ax + y.B[e] * ay;
    }
}

template <typename T, int D, bool PLX>
__global__ __launch_bounds__(64) void decode_generic(DecodeArgs a) {
    constexpr int EPL = Elem<T>::per16;
    constexpr int LPR = D / EPL;
    constexpr int KPI = 64 / LPR;
    static_assert(LPR * KPI == 64, "lanes must tile the wave");
    const int lane = threadIdx.x;
    const int kgrp = lane / LPR;
    const int c = lane % LPR;
    const int hq = blockIdx.x;
    const int split = blockIdx.y;
    const int b = blockIdx.z;
    const int G = a.Hq / a.Hkv;
    const int hkv = hq / G;

    const SeqRange sr = seq_range(a, b);
    const int start = split * a.chunk;
    T *o = reinterpret_cast<T *>(a.o) + ((int64_t)b * a.Hq + hq) * D;
    if (sr.len <= 0 || start >= sr.len) {
        if (a.fused) {
            if (kgrp == 0) {
                float zero[EPL] = {};
                Elem<T>::store(o + c * EPL, zero);
            }
        } else if (lane == 0) {
            float *rec = a.ws + (((int64_t)b * a.Hq + hq) * a.splits + split) * partial_floats(D);
            reinterpret_cast<float4 *>(rec + 2 * D)[0] = float4{-INFINITY, 0.f, 0.f, 0.f};
        }
        return;
    }
    const int end = min(start + a.chunk, sr.len);

    const T *qp = reinterpret_cast<const T *>(a.q) + ((int64_t)b * a.Hq + hq) * D + c * EPL;
    const int64_t tok_stride = (int64_t)a.Hkv * D;
    const T *kseq = reinterpret_cast<const T *>(a.k) + sr.tok0 * tok_stride + (int64_t)hkv * D + c * EPL;
    const T *vseq = reinterpret_cast<const T *>(a.v) + sr.tok0 * tok_stride + (int64_t)hkv * D + c * EPL;

    float qv[EPL], rv[EPL];
    Elem<T>::load(qp, qv);
    for (int e = 0; e < EPL; ++e) qv[e] *= a.zscale;
    float piv = 0.0f;
    if (PLX) {
        const T *rp = reinterpret_cast<const T *>(a.r) + ((int64_t)b * a.Hq + hq) * D + c * EPL;
        Elem<T>::load(rp, rv);
        for (int e = 0; e < EPL; ++e) rv[e] *= a.rk_scale;
        float k0[EPL];
        Elem<T>::load(kseq, k0);
        float part = 0.0f;
        for (int e = 0; e < EPL; ++e) part += rv[e] * k0[e];
        for (int off = 1; off < LPR; off <<= 1) part += __shfl_xor(part, off, LPR);
        piv = part;
    }

    State<EPL> st;
    st.m = -INFINITY;
    st.l = 0.f;
    st.S = 0.f;
    for (int e = 0; e < EPL; ++e) {
        st.A[e] = 0.f;
        st.B[e] = 0.f;
    }

    for (int j0 = start; j0 < end; j0 += KPI) {
        const int j = j0 + kgrp;
        const bool valid = j < end;
        const int jj = valid ? j : end - 1;
        float kv[EPL], vv[EPL];
        Elem<T>::load(kseq + (int64_t)jj * tok_stride, kv);
        Elem<T>::load(vseq + (int64_t)jj * tok_stride, vv);
        float zp = 0.f, sp = 0.f;
        for (int e = 0; e < EPL; ++e) {
            zp += qv[e] * kv[e];
            if (PLX) sp += rv[e] * kv[e];
        }
        for (int off = 1; off < LPR; off <<= 1) {
            zp += __shfl_xor(zp, off, LPR);
            if (PLX) sp += __shfl_xor(sp, off, LPR);
        }
        if (valid) {
            const float m_new = fmaxf(st.m, zp);
            const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
            const float p = __builtin_amdgcn_exp2f(zp - m_new);
            const float sd = sp - piv;
            st.m = m_new;
            st.l = st.l * alpha + p;
            if (PLX) st.S = st.S * alpha + p * sd;
            for (int e = 0; e < EPL; ++e) {
                st.A[e] = st.A[e] * alpha + p * vv[e];
                if (PLX) st.B[e] = st.B[e] * alpha + (p * sd) * vv[e];
            }
        }
    }
    // merge the key groups (lanes with the same chunk c)
    for (int off = LPR; off < 64; off <<= 1) {
        State<EPL> y;
        y.m = __shfl_xor(st.m, off);
        y.l = __shfl_xor(st.l, off);
        y.S = __shfl_xor(st.S, off);
        for (int e = 0; e < EPL; ++e) {
            y.A[e] = __shfl_xor(st.A[e], off);
            y.B[e] = __shfl_xor(st.B[e], off);
        }
        merge_state(st, y);
    }
    if (kgrp != 0) return;
    if (!a.fused) {
        float *rec = a.ws + (((int64_t)b * a.Hq + hq) * a.splits + split) * partial_floats(D);
        for (int e = 0; e < EPL; ++e) {
            rec[c * EPL + e] = st.A[e];
            rec[D + c * EPL + e] = st.B[e];
        }
        if (c == 0)
            reinterpret_cast<float4 *>(rec + 2 * D)[0] = float4{st.m, st.l, st.S, piv};
        return;
    }
    const float inv_l = 1.0f / st.l;
    const float cA = PLX ? (1.0f - st.S * inv_l) : 1.0f;
    float ov[EPL];
    for (int e = 0; e < EPL; ++e) ov[e] = (PLX ? st.A[e] * cA + st.B[e] : st.A[e]) * inv_l;
    Elem<T>::store(o + c * EPL, ov);
}

// -------------------------------------------------------------------------
// Record merge: one workgroup of 256 threads per (query head, sequence).
// Wave w folds records w, w+4, ...; the four wave states meet in LDS. Empty
// records (m = -inf) are skipped; none at all gives o = 0. Records may carry
// different pivots: each is re-based onto the pivot of record 0 with
//   S' = S + (pi_i - pi_0) l,   B' = B + (pi_i - pi_0) A
// (exact algebra; zero change when the pivots agree, as they do when all
// records come from one call).
// -------------------------------------------------------------------------
template <typename TO, int D, bool PLX>
__global__ __launch_bounds__(256) void decode_reduce(DecodeArgs a) {
    constexpr int DPL = D / 64;  // dims per lane
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int hq = blockIdx.x;
    const int b = blockIdx.y;
    const int ns = a.splits;
    const float *base = a.ws + ((int64_t)b * a.Hq + hq) * ns * partial_floats(D);
    const float piv0 = PLX ? base[2 * D + 3] : 0.f;

    float m = -INFINITY, l = 0.f, S = 0.f, A[DPL], Bv[DPL];
    for (int d = 0; d < DPL; ++d) {
        A[d] = 0.f;
        Bv[d] = 0.f;
    }
    for (int i = w; i < ns; i += 4) {
        const float *rec = base + (int64_t)i * partial_floats(D);
        const float4 tail = reinterpret_cast<const float4 *>(rec + 2 * D)[0];
        const float mi = tail.x;
        if (mi == -INFINITY) continue;
        const float li = tail.y;
        const float dp = PLX ? tail.w - piv0 : 0.f;
        const float Si = PLX ? tail.z + dp * li : 0.f;
        float Ai[DPL], Bi[DPL];
        for (int d = 0; d < DPL; ++d) {
            Ai[d] = rec[lane * DPL + d];
            Bi[d] = PLX ? rec[D + lane * DPL + d] + dp * Ai[d] : 0.f;
        }
        const float M = fmaxf(m, mi);
        const float ax = __builtin_amdgcn_exp2f(m - M);
        const float ay = __builtin_amdgcn_exp2f(mi - M);
        m = M;
        l = l * ax + li * ay;
        S = S * ax + Si * ay;
        for (int d = 0; d < DPL; ++d) {
            A[d] = A[d] * ax + Ai[d] * ay;
            Bv[d] = Bv[d] * ax + Bi[d] * ay;
        }
    }
    __shared__ float sm[4][2 * D + 4];
    for (int d = 0; d < DPL; ++d) {
        sm[w][lane * DPL + d] = A[d];
        sm[w][D + lane * DPL + d] = Bv[d];
    }
    if (lane == 0) {
        sm[w][2 * D] = m;
        sm[w][2 * D + 1] = l;
        sm[w][2 * D + 2] = S;
    }
    __syncthreads();
    if (w != 0) return;
    m = -INFINITY;
    l = 0.f;
    S = 0.f;
    for (int d = 0; d < DPL; ++d) {
        A[d] = 0.f;
        Bv[d] = 0.f;
    }
    for (int x = 0; x < 4; ++x) {
        const float mi = sm[x][2 * D];
        if (mi == -INFINITY) continue;  // this wave folded no record
        const float M = fmaxf(m, mi);
        const float ax = __builtin_amdgcn_exp2f(m - M);
        const float ay = __builtin_amdgcn_exp2f(mi - M);
        m = M;
        l = l * ax + sm[x][2 * D + 1] * ay;
        S = S * ax + sm[x][2 * D + 2] * ay;
        for (int d = 0; d < DPL; ++d) {
            A[d] = A[d] * ax + sm[x][lane * DPL + d] * ay;
            Bv[d] = Bv[d] * ax + sm[x][D + lane * DPL + d] * ay;
        }
    }
    TO *o = reinterpret_cast<TO *>(a.o) + ((int64_t)b * a.Hq + hq) * D + lane * DPL;
    for (int d = 0; d < DPL; ++d) {
        float val = 0.f;
        if (m != -INFINITY) {
            const float inv_l = 1.0f / l;
            val = PLX ? (A[d] * (1.0f - S * inv_l) + Bv[d]) * inv_l : A[d] * inv_l;
        }
        if constexpr (sizeof(TO) == 4)
            o[d] = val;
        else
            o[d] = f32_to_bf16(val);
    }
}

template <bool PLX>
hipError_t launch_mfma(const DecodeArgs &a, hipStream_t stream) {
    dim3 grid(a.Hkv, a.splits, a.B);
    const int G = a.Hq / a.Hkv;
    switch (G) {
        case 1: hipLaunchKernelGGL((decode_mfma_bf16_d128<1, PLX>), grid, dim3(64), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((decode_mfma_bf16_d128<2, PLX>), grid, dim3(64), 0, stream, a); break;
        case 4: hipLaunchKernelGGL((decode_mfma_bf16_d128<4, PLX>), grid, dim3(64), 0, stream, a); break;
        case 8: hipLaunchKernelGGL((decode_mfma_bf16_d128<8, PLX>), grid, dim3(64), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, bool PLX>
hipError_t launch_generic(const DecodeArgs &a, hipStream_t stream) {
    dim3 grid(a.Hq, a.splits, a.B);
    if (a.D == 64)
        hipLaunchKernelGGL((decode_generic<T, 64, PLX>), grid, dim3(64), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_generic<T, 128, PLX>), grid, dim3(64), 0, stream, a);
    return hipGetLastError();
}

template <typename TO, bool PLX>
hipError_t launch_reduce(const DecodeArgs &a, hipStream_t stream) {
    dim3 grid(a.Hq, a.B);
    if (a.D == 64)
        hipLaunchKernelGGL((decode_reduce<TO, 64, PLX>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_reduce<TO, 128, PLX>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_split(const DecodeArgs &a, DecodePath path, int dtype, bool parallax,
                               hipStream_t stream) {
    if (path == DecodePath::Mfma)
        return parallax ? launch_mfma<true>(a, stream) : launch_mfma<false>(a, stream);
    if (dtype == 1)
        return parallax ? launch_generic<uint16_t, true>(a, stream)
                        : launch_generic<uint16_t, false>(a, stream);
    return parallax ? launch_generic<float, true>(a, stream) : launch_generic<float, false>(a, stream);
}

hipError_t launch_decode_merge(const DecodeArgs &a, int dtype, bool parallax, hipStream_t stream) {
    if (dtype == 1)
        return parallax ? launch_reduce<uint16_t, true>(a, stream) : launch_reduce<uint16_t, false>(a, stream);
    return parallax ? launch_reduce<float, true>(a, stream) : launch_reduce<float, false>(a, stream);
}

}  // namespace plx
