// Parallax causal prefill backward (training) kernels for gfx950.
//
// The pages train through parallax_func with autograd (PyPI README of
// parallax-kernel, "Training (Triton)"; its "Helion" section holds the output
// and the four gradients to one tolerance) and print no gradient formula.
// Differentiating the forward of one row (visible keys j <= i)
//   w = softmax(z), z_j = qk_scale q.k_j, s_j = rk_scale r.k_j,
//   sbar = sum_j w_j s_j, o = sum_j w_j c_j v_j with c_j = 1 + s_j - sbar,
// for an upstream gradient g = dLoss/do gives, with u_j = g.v_j,
// ubar = sum_j w_j u_j and delta = o.g (both per row):
//   dv_j += w_j c_j g
//   ds_j  = w_j (u_j - ubar)                          (adjoint of s_j)
//   dz_j  = w_j (c_j u_j - ubar (s_j - sbar) - delta)  (adjoint of z_j)
//   dq    = qk_scale sum_j dz_j k_j,   dr = rk_scale sum_j ds_j k_j
//   dk_j += qk_scale dz_j q + rk_scale ds_j r
// w_j is recomputed from the forward's lse: w_j = exp(z_j - lse).
//
// Two kernels, no atomics (results are bit-identical from call to call):
//  - row pass, one query row per output row: a first sweep over the row's
//    keys gives ubar (skipped when the forward stored vbar: ubar = g.vbar),
//    a second accumulates dq and dr together with fp32 sums that correct
//    delta and ubar (sweeping again when the correction is large); it stores
//    the row's {lse log2 e, sbar, delta, ubar} for the key pass.
//  - key pass, one key per output row: sweeps every query row that sees the
//    key, over all query heads of its KV head, and accumulates dk and dv.
#include "plx_internal.h"
#include "plx_device.h"

namespace plx {

namespace {

template <typename T>
struct Frag;
template <>
struct Frag<float> {
    static constexpr int n = 4;
    __device__ static void load(const float *p, float *out) {
        float4 x = *reinterpret_cast<const float4 *>(p);
        out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    }
    __device__ static void store(float *p, const float *in) {
        *reinterpret_cast<float4 *>(p) = float4{in[0], in[1], in[2], in[3]};
    }
};
template <>
struct Frag<uint16_t> {
    static constexpr int n = 8;
    __device__ static void load(const uint16_t *p, float *out) {
        uint4 x = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = bf16_lo(w[i]);
            out[2 * i + 1] = bf16_hi(w[i]);
        }
    }
    __device__ static void store(uint16_t *p, const float *in) {
        *reinterpret_cast<uint4 *>(p) = uint4{pack_bf16x2(in[0], in[1]), pack_bf16x2(in[2], in[3]),
                                              pack_bf16x2(in[4], in[5]), pack_bf16x2(in[6], in[7])};
    }
};

// First row-statistics slot of (sequence, query head): the workspace holds
// one RowStat per query row, [B, Hq, L] dense and [Hq, T] packed, so that
// the rows of one head are contiguous in both layouts.
__device__ __forceinline__ int64_t rowstat0(const PrefillSeq &s, int b, int h, int Hq, int L, int T) {
    return s.packed ? (int64_t)h * T + s.tok0 : ((int64_t)b * Hq + h) * L;
}

// Sum over the LPR lanes that share one row of a wave.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    return group_sum<LPR>(x);
}
// Sum over the 64 / LPR rows of a wave (lanes c, c + LPR, ...).
template <int LPR>
__device__ __forceinline__ float across_rows(float x) {
    for (int off = LPR; off < 64; off <<= 1) x += __shfl_xor(x, off);
    return x;
}

// -------------------------------------------------------------------------
// Generic kernels (any dtype, head_dim 64 or 128): one wave per output row;
// each group of LPR lanes holds one key (row pass) or one query row (key
// pass), 16 bytes of it per lane.
// -------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void bwd_rows_generic(BackwardArgs a) {
    constexpr int EPL = Frag<T>::n;
    constexpr int LPR = D / EPL;
    constexpr int KPI = 64 / LPR;
    const int lane = threadIdx.x;
    const int kgrp = lane / LPR;
    const int c = lane % LPR;
    const int i = blockIdx.x;
    const int hq = blockIdx.y;
    const int b = blockIdx.z;
    const int hkv = hq / (a.Hq / a.Hkv);
    const PrefillSeq sq = prefill_seq(a.cu, b, a.L);
    if (i >= sq.len) return;  // past this sequence's end (packed batches)
    const int ks = row_stride(sq, a.Hkv, D);
    const int64_t row = row0_elem(sq, b, hq, a.Hq, a.L, D) + (int64_t)i * row_stride(sq, a.Hq, D);
    const int64_t srow = stat0(sq, b, hq, a.Hq, a.L) + (int64_t)i * stat_stride(sq, a.Hq);
    const int64_t kvoff = row0_elem(sq, b, hkv, a.Hkv, a.L, D) + c * EPL;
    const T *kb = reinterpret_cast<const T *>(a.k) + kvoff;
    const T *vb = reinterpret_cast<const T *>(a.v) + kvoff;

    float qv[EPL], rv[EPL], gv[EPL];
    Frag<T>::load(reinterpret_cast<const T *>(a.q) + row + c * EPL, qv);
    Frag<T>::load(reinterpret_cast<const T *>(a.r) + row + c * EPL, rv);
    Frag<T>::load(reinterpret_cast<const T *>(a.go) + row + c * EPL, gv);
    const float lse2 = a.lse[srow] * kLog2e;
    const float sb = a.sbar[srow];
    const int end = i + 1;
    const int first = max(0, i - a.window + 1);  // sliding window: keys first .. i
    // block-sparse: key j is visible iff its block is the row's own or the mask shows it
    const int nb = (a.L + kMaskBlock - 1) >> kMaskShift;
    const int qb = i >> kMaskShift;
    const uint8_t *mrow =
        a.block_mask ? a.block_mask + (((int64_t)b * a.Hkv + hkv) * nb + qb) * nb : nullptr;
    auto visible = [&](int j) {
        return j < end && (!mrow || (j >> kMaskShift) == qb || mrow[j >> kMaskShift] != 0);
    };

    // sweep 1: ubar = sum_j w_j u_j and delta = sum_j w_j c_j u_j (= g . o), in
    // fp32 from the recomputed weights rather than from the forward's outputs
    // o and vbar: dz is a difference of terms up to |c_j| times larger than
    // itself, and this keeps delta and ubar consistent with the weights the
    // gradients are formed from (sum_j dz_j = sum_j ds_j = 0).
    // Both sweeps take the key rows a batch of U steps at a time, loaded while
    // the batch before is used (step t: keys first + KPI t .. + KPI - 1).
    constexpr int U = EPL == 4 ? 8 : 4;
    const int nit = (end - first + KPI - 1) / KPI;
    auto sweep = [&](auto &&body) __attribute__((always_inline)) {
        auto load_step = [&](int t, float *kv, float *vv) __attribute__((always_inline)) {
            const int jj = min(first + t * KPI + kgrp, end - 1);  // past the end: a valid row, unused
            Frag<T>::load(kb + (int64_t)jj * ks, kv);
            Frag<T>::load(vb + (int64_t)jj * ks, vv);
        };
        float kcur[U][EPL], vcur[U][EPL];
#pragma unroll
        for (int u = 0; u < U; ++u) load_step(u, kcur[u], vcur[u]);
        for (int t0 = 0; t0 < nit; t0 += U) {
            float knext[U][EPL], vnext[U][EPL];
#pragma unroll
            for (int u = 0; u < U; ++u) load_step(t0 + U + u, knext[u], vnext[u]);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (t0 + u < nit) body(first + (t0 + u) * KPI + kgrp, kcur[u], vcur[u]);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    kcur[u][e] = knext[u][e];
                    vcur[u][e] = vnext[u][e];
                }
        }
    };
    float ub = 0.f, delta = 0.f;
    sweep([&](int j, const float *kv, const float *vv) __attribute__((always_inline)) {
        float zp = 0.f, sp = 0.f, up = 0.f;
        for (int e = 0; e < EPL; ++e) {
            zp += qv[e] * kv[e];
            sp += rv[e] * kv[e];
            up += gv[e] * vv[e];
        }
        zp = row_sum<LPR>(zp);
        sp = row_sum<LPR>(sp);
        up = row_sum<LPR>(up);
        if (visible(j)) {
            const float w = __builtin_amdgcn_exp2f(fmaf(zp, a.zscale, -lse2));
            const float sc = fmaf(sp, a.rk_scale, -sb);
            ub = fmaf(w, up, ub);
            delta = fmaf(w, fmaf(sc, up, up), delta);
        }
    });
    ub = across_rows<LPR>(ub);
    delta = across_rows<LPR>(delta);

    // sweep 2: dq, dr
    float dqa[EPL], dra[EPL];
    for (int e = 0; e < EPL; ++e) dqa[e] = dra[e] = 0.f;
    sweep([&](int j, const float *kv, const float *vv) __attribute__((always_inline)) {
        float zp = 0.f, sp = 0.f, up = 0.f;
        for (int e = 0; e < EPL; ++e) {
            zp += qv[e] * kv[e];
            sp += rv[e] * kv[e];
            up += gv[e] * vv[e];
        }
        zp = row_sum<LPR>(zp);
        sp = row_sum<LPR>(sp);
        up = row_sum<LPR>(up);
        const float w = visible(j) ? __builtin_amdgcn_exp2f(fmaf(zp, a.zscale, -lse2)) : 0.f;
        const float sc = fmaf(sp, a.rk_scale, -sb);  // s_j - sbar
        const float ds = w * (up - ub);
        const float dz = w * (fmaf(sc, up, up) - fmaf(ub, sc, delta));
        for (int e = 0; e < EPL; ++e) {
            dqa[e] = fmaf(dz, kv[e], dqa[e]);
            dra[e] = fmaf(ds, kv[e], dra[e]);
        }
    });
    for (int e = 0; e < EPL; ++e) {
        dqa[e] = across_rows<LPR>(dqa[e]) * a.qk_scale;
        dra[e] = across_rows<LPR>(dra[e]) * a.rk_scale;
    }
    if (kgrp == 0) {
        Frag<T>::store(reinterpret_cast<T *>(a.dq) + row + c * EPL, dqa);
        Frag<T>::store(reinterpret_cast<T *>(a.dr) + row + c * EPL, dra);
        if (c == 0) a.rowstat[rowstat0(sq, b, hq, a.Hq, a.L, a.total) + i] = RowStat{lse2, sb, delta, ub};
    }
}

template <typename T, int D>
__global__ __launch_bounds__(64) void bwd_keys_generic(BackwardArgs a) {
    constexpr int EPL = Frag<T>::n;
    constexpr int LPR = D / EPL;
    constexpr int RPI = 64 / LPR;
    const int lane = threadIdx.x;
    const int rgrp = lane / LPR;
    const int c = lane % LPR;
    const int j = blockIdx.x;
    const int hkv = blockIdx.y;
    const int b = blockIdx.z;
    const int G = a.Hq / a.Hkv;
    const PrefillSeq sq = prefill_seq(a.cu, b, a.L);
    if (j >= sq.len) return;  // past this sequence's end (packed batches)
    const int qs = row_stride(sq, a.Hq, D);
    const int64_t kvrow = row0_elem(sq, b, hkv, a.Hkv, a.L, D) + (int64_t)j * row_stride(sq, a.Hkv, D);
    float kv[EPL], vv[EPL], dka[EPL], dva[EPL];
    Frag<T>::load(reinterpret_cast<const T *>(a.k) + kvrow + c * EPL, kv);
    Frag<T>::load(reinterpret_cast<const T *>(a.v) + kvrow + c * EPL, vv);
    for (int e = 0; e < EPL; ++e) dka[e] = dva[e] = 0.f;
    constexpr int UK = EPL == 4 ? 4 : 2;
    // block-sparse: row i sees key j iff j's block is i's own or the mask shows it
    const int nb = (a.L + kMaskBlock - 1) >> kMaskShift;
    const int kb = j >> kMaskShift;
    const uint8_t *mcol =
        a.block_mask ? a.block_mask + ((int64_t)b * a.Hkv + hkv) * nb * nb + kb : nullptr;
    for (int hs = 0; hs < G; ++hs) {
        const int hq = hkv * G + hs;
        const int64_t rbase = row0_elem(sq, b, hq, a.Hq, a.L, D);
        const int64_t sbase = rowstat0(sq, b, hq, a.Hq, a.L, a.total);
        const int rend = min(sq.len, j + a.window);  // rows that see key j
        // rows j + RPI t .. + RPI - 1 at step t, a batch of UK steps loaded while
        // the batch before is used
        const int nit = (rend - j + RPI - 1) / RPI;
        auto load_step = [&](int t, float *qv, float *rv, float *gv, RowStat &st) __attribute__((always_inline)) {
            const int ii = min(j + t * RPI + rgrp, rend - 1);  // past the end: a valid row, unused
            const int64_t row = rbase + (int64_t)ii * qs;
            Frag<T>::load(reinterpret_cast<const T *>(a.q) + row + c * EPL, qv);
            Frag<T>::load(reinterpret_cast<const T *>(a.r) + row + c * EPL, rv);
            Frag<T>::load(reinterpret_cast<const T *>(a.go) + row + c * EPL, gv);
            st = a.rowstat[sbase + ii];
        };
        auto body = [&](int i, const float *qv, const float *rv, const float *gv, const RowStat &st) __attribute__((always_inline)) {
            float zp = 0.f, sp = 0.f, up = 0.f;
            for (int e = 0; e < EPL; ++e) {
                zp += qv[e] * kv[e];
                sp += rv[e] * kv[e];
                up += gv[e] * vv[e];
            }
            zp = row_sum<LPR>(zp);
            sp = row_sum<LPR>(sp);
            up = row_sum<LPR>(up);
            const bool vis = i < rend && (!mcol || (i >> kMaskShift) == kb ||
                                          mcol[(int64_t)(i >> kMaskShift) * nb] != 0);
            const float w = vis ? __builtin_amdgcn_exp2f(fmaf(zp, a.zscale, -st.lse2)) : 0.f;
            const float sc = fmaf(sp, a.rk_scale, -st.sbar);
            const float pv = w * (1.0f + sc);
            const float ds = w * (up - st.ubar) * a.rk_scale;
            const float dz = w * (fmaf(sc, up, up) - fmaf(st.ubar, sc, st.delta)) * a.qk_scale;
            for (int e = 0; e < EPL; ++e) {
                dva[e] = fmaf(pv, gv[e], dva[e]);
                dka[e] = fmaf(dz, qv[e], fmaf(ds, rv[e], dka[e]));
            }
        };
        float qc[UK][EPL], rc[UK][EPL], gc[UK][EPL];
        RowStat sc_[UK];
#pragma unroll
        for (int u = 0; u < UK; ++u) load_step(u, qc[u], rc[u], gc[u], sc_[u]);
        for (int t0 = 0; t0 < nit; t0 += UK) {
            float qn[UK][EPL], rn[UK][EPL], gn[UK][EPL];
            RowStat sn[UK];
#pragma unroll
            for (int u = 0; u < UK; ++u) load_step(t0 + UK + u, qn[u], rn[u], gn[u], sn[u]);
#pragma unroll
            for (int u = 0; u < UK; ++u)
                if (t0 + u < nit) body(j + (t0 + u) * RPI + rgrp, qc[u], rc[u], gc[u], sc_[u]);
#pragma unroll
            for (int u = 0; u < UK; ++u) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) {
                    qc[u][e] = qn[u][e];
                    rc[u][e] = rn[u][e];
                    gc[u][e] = gn[u][e];
                }
                sc_[u] = sn[u];
            }
        }
    }
    for (int e = 0; e < EPL; ++e) {
        dka[e] = across_rows<LPR>(dka[e]);
        dva[e] = across_rows<LPR>(dva[e]);
    }
    if (rgrp == 0) {
        Frag<T>::store(reinterpret_cast<T *>(a.dk) + kvrow + c * EPL, dka);
        Frag<T>::store(reinterpret_cast<T *>(a.dv) + kvrow + c * EPL, dva);
    }
}

// -------------------------------------------------------------------------
// MFMA kernels, bf16, head_dim 128 (v_mfma_f32_16x16x32_bf16, fp32
// accumulation). Operand layout of that instruction: lane l = 16 g + n holds
// row n of A and column n of B, each with k = 8 g .. 8 g + 7 of the 32-wide
// k step; the result lane holds column n, rows 4 g .. 4 g + 3.
//
// Tiles in LDS are row-major 256-byte rows (one key or one query row of 128
// bf16) with 16-byte chunk c of row x stored at slot c ^ swz(x & 15),
// swz(x) = 2 ((x >> 2) & 3) + 9 (x & 1), filled by the buffer unit directly
// (buffer_load ... lds). For the row orders used below (permuted rows for
// the plain reads, rows g + 4 t for the transposed ones), the plain 16-byte
// reads of a row chunk (served eight lanes at a time: eight distinct
// slot & 7) and the transposing 64-bit reads (ds_read_b64_tr_b16, served 32
// lanes at a time over all 64 banks: 16 distinct slots) are both free of
// bank conflicts.
//
// Permuted score rows: the score MFMA's A row m is loaded from tile row
// (m >> 2) + 4 (m & 3) (+16 for the second 16-row block), so the result lane
// (g, n) holds, as element t = 0..7 of the two blocks, tile rows g + 4 t:
// exactly the k elements it supplies as the B operand of the next
// contraction, whose A operand is read transposed at the same rows.
// -------------------------------------------------------------------------
constexpr int kBwdWaves = 8;
// Row pass: the corrections of delta and ubar found by the sweep are applied
// by a second sweep when together they exceed kDeltaRedo times the sum of the
// row's |dz'| + |ds'| (the operands they perturb), plus kDeltaFloor times the
// row's |delta| + |ubar| (below that the sums are fp32 round-off).
constexpr float kDeltaRedo = 1.0f / 1024.0f;
constexpr float kDeltaFloor = 1.0f / 16384.0f;
constexpr int kBwdKeysPerTile = 128;  // row pass: keys per LDS tile
constexpr int kBwdRowsPerTile = 64;   // key pass: query rows per LDS tile

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int tile_swz(int x) { return 2 * ((x >> 2) & 3) + 9 * (x & 1); }

// 16-byte chunk `chunk` of tile row x.
__device__ __forceinline__ bf16x8 lds_chunk(const uint16_t *t, int x, int chunk) {
    return *reinterpret_cast<const bf16x8 *>(&t[x * 128 + ((chunk ^ tile_swz(x)) * 8)]);
}

// Transposed operand of block `blk` (columns 16 blk .. 16 blk + 15 of the
// tile) over tile rows x0 + g + 4 t, t = 0..7: lane (g, n) receives column
// 16 blk + n of those eight rows. Within each 16-lane row of the wave, lane
// j points at four columns 16 blk + 4 (j & 3) of row x0 + g + 4 ((j >> 2) + 4 h).
__device__ __forceinline__ bf16x8 lds_transposed(const uint16_t *t, int x0, int blk, int g, int n) {
    const int q4 = n >> 2, dq = n & 3;
    const int col = 16 * blk + 4 * dq;
    v4i16 part[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int x = x0 + g + 4 * (q4 + 4 * h);
        const int addr = x * 128 + (((col >> 3) ^ tile_swz(x)) * 8) + (col & 7);
        part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16 *)(t + addr));
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Copy NROWS rows (a multiple of 4 * NW; `stride` elements apart in memory)
// starting at row `row0` of the buffer behind `rs` into LDS tile `t`, shared
// by NW waves. Rows past the buffer's range read as zeros.
template <int NROWS, int NW>
__device__ __forceinline__ void dma_rows(__amdgpu_buffer_rsrc_t rs, int row0, int stride, uint16_t *t, int wave,
                                         int lane) {
    constexpr int PER_WAVE = NROWS / (4 * NW);
    static_assert(PER_WAVE * 4 * NW == NROWS, "rows must split evenly over the waves");
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
        const int xloc = 4 * (wave * PER_WAVE + j);
        const int x = xloc + (lane >> 4);
        const int chunk = (lane & 15) ^ tile_swz(x);
        const int off = ((row0 + x) * stride + chunk * 8) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(t + xloc * 128), 16, off, 0, 0, 0);
    }
}

// ---- row pass: dq, dr and the row statistics --------------------------
//
// Workgroup: eight waves over one (sequence, KV head, group of HPW query
// heads, q-tile); each wave owns 16 query rows of one head, as in the
// forward kernel. K/V tiles of 128 keys are double buffered in LDS and swept
// twice: first for ubar, then for dq and dr. Per 32-key sub-tile a wave runs
//   sweep 1: Z^T = K Q^T, U^T = V G^T                        (16 MFMAs)
//   sweep 2: Z^T, S^T = K R^T, U^T, then dQ^T += K^T dZ^T,
//            dR^T += K^T dS^T with K^T read transposed       (40 MFMAs)
// LEAN: the LDS reads take per-lane offsets XOR-ed per k step and column
// block (a dozen address registers instead of 64), which removes the
// persistent form's register spills (packed batches: 47 spilled VGPRs, row
// pass 1220 -> 1082 us); the one-item form, which does not spill, measured
// 0.8% slower with it and keeps the plain addresses. Same LDS addresses.
template <int HPW, bool MASK, bool LEAN>
__device__ __forceinline__ void bwd_rows_item(const BackwardArgs &a, const int item) {
    constexpr int D = 128;
    constexpr int NW = kBwdWaves;
    constexpr int WPH = NW / HPW;
    constexpr int RPH = 16 * WPH;
    constexpr int TK = kBwdKeysPerTile;
    constexpr int NSUB = TK / 32;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int g = lane >> 4;

    const int G = a.Hq / a.Hkv;
    const int hgroups = G / HPW;
    const int NG = a.B * a.Hkv * hgroups;
    const int QT = (a.L + RPH - 1) / RPH;
    const int grp = item % NG;
    const int qt = QT - 1 - item / NG;
    const int b = grp / (a.Hkv * hgroups);
    const int hkv = (grp / hgroups) % a.Hkv;
    const int hsub = grp % hgroups;
    const int hq = hkv * G + hsub * HPW + wave / WPH;
    const int q0 = qt * RPH + (wave % WPH) * 16;
    const PrefillSeq sq = prefill_seq(a.cu, b, a.L);
    const int L = sq.len;
    if (qt * RPH >= L) return;  // work item past this sequence's end (packed batches)
    const int kend = min(L, (qt + 1) * RPH);
    const int ntiles = (kend + TK - 1) / TK;
    const int W = a.window;                          // query i sees keys i - W + 1 .. i
    const int tile0 = max(0, qt * RPH - W + 1) / TK;  // first tile any row of the item sees

    const int64_t kvbase = row0_elem(sq, b, hkv, a.Hkv, a.L, D);
    const int ks = row_stride(sq, a.Hkv, D);
    const uint32_t kvbytes = (uint32_t)(((int64_t)(L - 1) * ks + D) * 2);  // this sequence only
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(reinterpret_cast<const uint16_t *>(a.k) + kvbase), 0, kvbytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(reinterpret_cast<const uint16_t *>(a.v) + kvbase), 0, kvbytes, kBufferFlags);

    __shared__ __attribute__((aligned(16))) uint16_t lds_k0[TK * D], lds_v0[TK * D];
    __shared__ __attribute__((aligned(16))) uint16_t lds_k1[TK * D], lds_v1[TK * D];
    auto dma_tile = [&](int tile, uint16_t *lk, uint16_t *lv) __attribute__((always_inline)) {
        dma_rows<TK, NW>(krs, tile * TK, ks, lk, wave, lane);
        dma_rows<TK, NW>(vrs, tile * TK, ks, lv, wave, lane);
    };
    // block-sparse: the key tiles (= key blocks) this item's query block sees
    static_assert(TK == kMaskBlock && kMaskBlock % RPH == 0, "a tile is one mask block");
    const int qb = (qt * RPH) >> kMaskShift;
    const int nb = (a.L + kMaskBlock - 1) >> kMaskShift;
    const uint8_t *mrow = MASK ? a.block_mask + (((int64_t)b * a.Hkv + hkv) * nb + qb) * nb : nullptr;
    uint64_t vbits = 0;
    int vbase = -64;
    auto next_tile = [&](int t) {
        if constexpr (!MASK) return t;
        return next_visible(t, ntiles, vbits, vbase, [&](int u) { return u == qb || mrow[u] != 0; });
    };
    const int first_tile = next_tile(tile0);  // the diagonal tile is always visible
    dma_tile(first_tile, lds_k0, lds_v0);     // the first sweep's first tile

    // per-wave B operands (query row n, k step u -> chunk g + 4u) and row scalars
    const int64_t qbase = row0_elem(sq, b, hq, a.Hq, a.L, D);
    const int qs = row_stride(sq, a.Hq, D);
    const int64_t sbase = stat0(sq, b, hq, a.Hq, a.L);
    const int ss = stat_stride(sq, a.Hq);
    const int row = q0 + n;
    const int rowc = min(row, L - 1);
    bf16x8 qop[4], rop[4], gop[4];
    float delta, ubar_fwd;
    {
        const int64_t ro = qbase + (int64_t)rowc * qs;
        const uint16_t *qp = reinterpret_cast<const uint16_t *>(a.q) + ro;
        const uint16_t *rp = reinterpret_cast<const uint16_t *>(a.r) + ro;
        const uint16_t *gp = reinterpret_cast<const uint16_t *>(a.go) + ro;
        const uint16_t *op = reinterpret_cast<const uint16_t *>(a.o) + ro;
        const uint16_t *vp = reinterpret_cast<const uint16_t *>(a.vbar ? a.vbar : a.o) + ro;
        float part = 0.f, vpart = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            qop[u] = load16(qp + 8 * (g + 4 * u));
            rop[u] = load16(rp + 8 * (g + 4 * u));
            gop[u] = load16(gp + 8 * (g + 4 * u));
            const bf16x8 ov = load16(op + 8 * (g + 4 * u));
            const bf16x8 vv = load16(vp + 8 * (g + 4 * u));
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                part += (float)ov[e] * (float)gop[u][e];
                vpart += (float)vv[e] * (float)gop[u][e];
            }
        }
        delta = xor_sum_rowgroups(part);
        ubar_fwd = xor_sum_rowgroups(vpart);  // g . vbar, used when the forward stored vbar
    }
    const float lse2 = a.lse[sbase + (int64_t)rowc * ss] * kLog2e;
    const float sb = a.sbar[sbase + (int64_t)rowc * ss];
    const int kperm = (n >> 2) + 4 * (n & 3);
    const int q_last = q0 + 15;

    struct Frags {
        bf16x8 x[2][4];
    };
    // Per-lane byte offsets of the LDS reads for LEAN: the swizzle of tile rows
    // kl + 16 kb + kperm is that of kperm, and g + 4u = g ^ 4u with the XOR
    // confined to bits 4..7, so row-major fragment u sits at cofs ^ 64u; the
    // transposed fragment of column block e at tofs ^ 32e (the swizzle of rows
    // kl + 16 h + g + 4 (n >> 2) is that of g + 4 (n >> 2)). Row offsets are
    // immediates of the reads.
    const uint32_t cofs = 256u * kperm + 16u * (uint32_t)(g ^ tile_swz(kperm));
    const uint32_t tofs = 256u * (g + 4 * (n >> 2)) + 8u * (n & 1) +
                          16u * (uint32_t)(((n & 3) >> 1) ^ tile_swz(g + 4 * (n >> 2)));
    // A operand rows of a 32-key sub-tile at tile row kl: block kb, k step u
    auto load_rows = [&](const uint16_t *t, int kl) __attribute__((always_inline)) {
        Frags f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if constexpr (LEAN)
                    f.x[kb][u] = *reinterpret_cast<const bf16x8 *>(reinterpret_cast<const char *>(t) +
                                                                   256 * (kl + 16 * kb) + (cofs ^ (64u * u)));
                else
                    f.x[kb][u] = lds_chunk(t, kl + 16 * kb + kperm, g + 4 * u);
            }
        return f;
    };
    // K^T operand of column block e over tile rows kl .. kl + 31
    auto rows_t = [&](const uint16_t *t, int kl, int e) __attribute__((always_inline)) {
        if constexpr (!LEAN) return lds_transposed(t, kl, e, g, n);
        v4i16 part[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4i16 *)(reinterpret_cast<const char *>(t) + 256 * kl + 4096 * h +
                                                             (tofs ^ (32u * e))));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // c = rows . bop over the 128 dims, the accumulators starting from init
    auto contract = [&](const Frags &f, const bf16x8 *bop, floatx4 &c0, floatx4 &c1,
                        floatx4 init = floatx4{0.f, 0.f, 0.f, 0.f}) __attribute__((always_inline)) {
        c0 = c1 = init;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.x[0][u], bop[u], c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.x[1][u], bop[u], c1, 0, 0, 0);
        }
    };
    // the sweep over this wave's key tiles; body(lk, lv, kl, key0, diag)
    auto sweep = [&](auto &&body) __attribute__((always_inline)) {
        auto step = [&](int tile, int nxt, uint16_t *lk, uint16_t *lv, uint16_t *nk, uint16_t *nv) __attribute__((always_inline)) {
            if (nxt < ntiles) dma_tile(nxt, nk, nv);
            const int t0 = tile * TK;
            // tiles outside the wave's visible band are skipped; the mask is
            // needed unless every key of the tile is visible to all 16 rows
            if (t0 <= q_last && t0 + TK - 1 > q0 - W) {
                const bool diag = !(t0 + TK - 1 <= q0 && t0 > q_last - W);
#pragma unroll
                for (int j = 0; j < NSUB; ++j) {
                    const int k0 = t0 + 32 * j;
                    // on a masked tile, sub-tiles with none of the wave's keys are skipped
                    if (diag && (k0 > q_last || k0 + 31 <= q0 - W)) continue;
                    body(lk, lv, 32 * j, k0, diag);
                }
            }
            __syncthreads();
        };
        __syncthreads();
        if constexpr (!MASK) {
            for (int tile = tile0; tile < ntiles; tile += 2) {
                step(tile, tile + 1, lds_k0, lds_v0, lds_k1, lds_v1);
                if (tile + 1 < ntiles) step(tile + 1, tile + 2, lds_k1, lds_v1, lds_k0, lds_v0);
            }
        } else {
            int tile = first_tile;
            while (true) {
                int nxt = next_tile(tile + 1);
                step(tile, nxt, lds_k0, lds_v0, lds_k1, lds_v1);
                if (nxt >= ntiles) break;
                tile = nxt;
                nxt = next_tile(tile + 1);
                step(tile, nxt, lds_k1, lds_v1, lds_k0, lds_v0);
                if (nxt >= ntiles) break;
                tile = nxt;
            }
        }
    };

    // ---- sweep 1: ubar = sum_j w_j g.v_j (skipped when the forward stored vbar)
    float ub_part = 0.f;
    if (!a.vbar)
    sweep([&](const uint16_t *lk, const uint16_t *lv, int kl, int key0, bool diag) __attribute__((always_inline)) {
        floatx4 z0, z1, u0, u1;
        contract(load_rows(lk, kl), qop, z0, z1);
        contract(load_rows(lv, kl), gop, u0, u1);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float z = t < 4 ? z0[t] : z1[t - 4];
            const float u = t < 4 ? u0[t] : u1[t - 4];
            float w = __builtin_amdgcn_exp2f(fmaf(z, a.zscale, -lse2));
            const int key = key0 + g + 4 * t;
            if (diag && (key > row || key <= row - W)) w = 0.f;
            ub_part = fmaf(w, u, ub_part);
        }
    });
    float ubar = a.vbar ? ubar_fwd : xor_sum_rowgroups(ub_part);

    // ---- sweep 2: dq, dr
    // delta = g . o (and ubar = g . vbar) come from the forward's bf16 outputs,
    // which carry its rounding; dz is a difference of terms up to |1 + s - sbar|
    // times larger than itself, so that rounding can dominate dz. The sweep
    // therefore also sums its fp32 dz' and ds': with the recomputed weights
    // (sum_j w_j = 1, sum_j w_j (s_j - sbar) = 0)
    //   sum_j dz'_j = delta_true - delta,   sum_j ds'_j = ubar_true - ubar
    // exactly, so both are corrected after the sweep (and the key pass reads
    // the corrected values). Where a correction exceeds kDeltaRedo of the sum
    // of the |dz'| (|ds'|) it touches, which is about the bf16 rounding of
    // those operands, the work item sweeps again with the corrected values.
    // (The |dz'| and |ds'| are summed together: one register fewer.)
    floatx4 accQ[8], accR[8];
    __shared__ int redo_flag;
    for (int pass = 0;; ++pass) {
    // sweep 2 takes u - delta straight from the matrix cores (the accumulators
    // start from -delta); u - ubar is then that plus delta - ubar
    const floatx4 neg_delta = {-delta, -delta, -delta, -delta};
    const float delta_ubar = delta - ubar;
#pragma unroll
    for (int e = 0; e < 8; ++e) accQ[e] = accR[e] = floatx4{0.f, 0.f, 0.f, 0.f};
    // sweep 1 or the first pass consumed the first copy
    if (pass > 0 || !a.vbar) dma_tile(first_tile, lds_k0, lds_v0);
    if (threadIdx.x == 0) redo_flag = 0;  // ordered by the sweep's first barrier
    float sz = 0.f, ss = 0.f, am = 0.f;  // sums of dz', ds', |dz'| + |ds'|
    sweep([&](const uint16_t *lk, const uint16_t *lv, int kl, int key0, bool diag) __attribute__((always_inline)) {
        floatx4 z0, z1, s0, s1, u0, u1;
        {
            const Frags kf = load_rows(lk, kl);
            __builtin_amdgcn_s_setprio(1);
            contract(kf, qop, z0, z1);
            contract(kf, rop, s0, s1);
            __builtin_amdgcn_s_setprio(0);
        }
        contract(load_rows(lv, kl), gop, u0, u1, neg_delta);
        bf16x8 pz, ps;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float z = t < 4 ? z0[t] : z1[t - 4];
            const float s = t < 4 ? s0[t] : s1[t - 4];
            const float ud = t < 4 ? u0[t] : u1[t - 4];  // u - delta
            float w = __builtin_amdgcn_exp2f(fmaf(z, a.zscale, -lse2));
            const int key = key0 + g + 4 * t;
            if (diag && (key > row || key <= row - W)) w = 0.f;
            const float sc = fmaf(s, a.rk_scale, -sb);
            const float uu = ud + delta_ubar;            // u - ubar
            const float dz = w * fmaf(sc, uu, ud);       // w (u - delta + (s - sbar)(u - ubar))
            const float ds = w * uu;
            sz += dz;
            ss += ds;
            am += fabsf(dz) + fabsf(ds);
            pz[t] = (__bf16)dz;
            ps[t] = (__bf16)ds;
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bf16x8 kt = rows_t(lk, kl, e);
            accQ[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, pz, accQ[e], 0, 0, 0);
            accR[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, ps, accR[e], 0, 0, 0);
        }
        __builtin_amdgcn_s_setprio(0);
    });
    const float ed = xor_sum_rowgroups(sz), eu = xor_sum_rowgroups(ss);
    delta += ed;
    ubar += eu;
    if (pass > 0) break;
    const float mag = xor_sum_rowgroups(am);
    const bool redo = row < L && fabsf(ed) + fabsf(eu) > kDeltaRedo * mag + kDeltaFloor * (fabsf(delta) + fabsf(ubar));
    if (__builtin_amdgcn_ballot_w64(redo) != 0 && lane == 0) redo_flag = 1;
    __syncthreads();
    if (!redo_flag) break;
    }

    if (row < L) {
        // block e, accumulator element i holds dim 16 e + 4 g + i
        uint16_t *dq = reinterpret_cast<uint16_t *>(a.dq) + qbase + (int64_t)row * qs + 4 * g;
        uint16_t *dr = reinterpret_cast<uint16_t *>(a.dr) + qbase + (int64_t)row * qs + 4 * g;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const floatx4 x = accQ[e] * a.qk_scale;
            const floatx4 y = accR[e] * a.rk_scale;
            *reinterpret_cast<uint2 *>(dq + 16 * e) = uint2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
            *reinterpret_cast<uint2 *>(dr + 16 * e) = uint2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        }
        if (g == 0) a.rowstat[rowstat0(sq, b, hq, a.Hq, a.L, a.total) + row] = RowStat{lse2, sb, delta, ubar};
    }
}

// ---- key pass: dk, dv ---------------------------------------------------
//
// Workgroup: four waves over one (sequence, KV head, block of 128 keys);
// wave w owns keys 32 w .. 32 w + 31 of the block (two 16-key column
// blocks), whose K and V stay in registers as B operands. The query rows
// that see the block (rows >= its first key) of every query head of the KV
// head stream through LDS in tiles of 64 rows of Q, R and dLoss/do plus
// their row statistics, double buffered. Per 32-row sub-tile a wave runs
//   Z = Q K^T, S = R K^T, U = G V^T                      (48 MFMAs)
//   dV^T += G^T P1, dK^T += Q^T dZ + R^T dS               (48 MFMAs)
// with P1 = w c, dZ = qk_scale dz, dS = rk_scale ds in bf16 and the
// transposed A operands read with ds_read_b64_tr_b16. Every A fragment read
// from LDS feeds both column blocks, which halves the LDS traffic per MFMA
// against 16-key waves; one wave per SIMD holds the 32-key accumulators.
// Blocks run first key block first (the longest), with the (sequence, KV
// head) index fastest so that all blocks of one head share an XCD and its L2.
constexpr int kKeyWaves = 4;
constexpr int kKeyBlocksPerWave = 2;  // 16-key column blocks per wave

template <bool MASK>
__device__ __forceinline__ void bwd_keys_item(const BackwardArgs &a, const int item) {
    constexpr int D = 128;
    constexpr int NW = kKeyWaves;
    constexpr int KBW = kKeyBlocksPerWave;
    constexpr int TR = kBwdRowsPerTile;
    constexpr int KB = 16 * KBW * NW;  // keys per workgroup
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int g = lane >> 4;

    const int G = a.Hq / a.Hkv;
    const int NG = a.B * a.Hkv;
    const int grp = item % NG;
    const int kblk = item / NG;
    const int b = grp / a.Hkv;
    const int hkv = grp % a.Hkv;
    const int k0 = kblk * KB;
    const PrefillSeq sq = prefill_seq(a.cu, b, a.L);
    const int L = sq.len;
    if (k0 >= L) return;  // key block past this sequence's end (packed batches)
    const int kw = k0 + 16 * KBW * wave;  // this wave's first key
    const int W = a.window;
    const int rend = min(L, k0 + KB - 1 + W);  // rows k0 .. rend - 1 see some key of the block
    const int nrt = (rend - k0 + TR - 1) / TR;   // row tiles per query head
    const int ntiles = G * nrt;
    // block-sparse: row tile t (of head t / nrt) lies in query block
    // (k0 + (t % nrt) TR) / 128, which sees this key block if it is the
    // block itself or the mask shows it
    static_assert(KB == kMaskBlock && kMaskBlock % TR == 0, "a key block is one mask block");
    const int kblock = k0 >> kMaskShift;
    const int nb = (a.L + kMaskBlock - 1) >> kMaskShift;
    const uint8_t *mcol = MASK ? a.block_mask + ((int64_t)b * a.Hkv + hkv) * nb * nb + kblock : nullptr;
    uint64_t vbits = 0;
    int vbase = -64;
    auto next_tile = [&](int t) {
        if constexpr (!MASK) return t;
        return next_visible(t, ntiles, vbits, vbase, [&](int u) {
            const int qbk = (k0 + (u % nrt) * TR) >> kMaskShift;
            return qbk == kblock || mcol[(int64_t)qbk * nb] != 0;
        });
    };

    const int64_t kvbase = row0_elem(sq, b, hkv, a.Hkv, a.L, D);
    const int ks = row_stride(sq, a.Hkv, D);
    bf16x8 kop[KBW][4], vop[KBW][4];
#pragma unroll
    for (int c = 0; c < KBW; ++c) {
        const int kc = min(kw + 16 * c + n, L - 1);
        const uint16_t *kp = reinterpret_cast<const uint16_t *>(a.k) + kvbase + (int64_t)kc * ks;
        const uint16_t *vp = reinterpret_cast<const uint16_t *>(a.v) + kvbase + (int64_t)kc * ks;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            kop[c][u] = load16(kp + 8 * (g + 4 * u));
            vop[c][u] = load16(vp + 8 * (g + 4 * u));
        }
    }

    __shared__ __attribute__((aligned(16))) uint16_t lq0[TR * D], lr0[TR * D], lg0[TR * D];
    __shared__ __attribute__((aligned(16))) uint16_t lq1[TR * D], lr1[TR * D], lg1[TR * D];
    __shared__ __attribute__((aligned(16))) RowStat ls0[TR], ls1[TR];
    const int qs = row_stride(sq, a.Hq, D);
    const uint32_t hbytes = (uint32_t)(((int64_t)(L - 1) * qs + D) * 2);  // one head of this sequence
    auto dma_tile = [&](int tile, uint16_t *tq, uint16_t *tr, uint16_t *tg, RowStat *ts) __attribute__((always_inline)) {
        const int hq = hkv * G + tile / nrt;
        const int r0 = k0 + (tile % nrt) * TR;
        const int64_t qbase = row0_elem(sq, b, hq, a.Hq, a.L, D);
        const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(reinterpret_cast<const uint16_t *>(a.q) + qbase), 0, hbytes, kBufferFlags);
        const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(reinterpret_cast<const uint16_t *>(a.r) + qbase), 0, hbytes, kBufferFlags);
        const __amdgpu_buffer_rsrc_t grs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(reinterpret_cast<const uint16_t *>(a.go) + qbase), 0, hbytes, kBufferFlags);
        dma_rows<TR, NW>(qrs, r0, qs, tq, wave, lane);
        dma_rows<TR, NW>(rrs, r0, qs, tr, wave, lane);
        dma_rows<TR, NW>(grs, r0, qs, tg, wave, lane);
        if (wave == 0) {  // 64 rows x 16 bytes: one copy by one wave
            const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(a.rowstat + rowstat0(sq, b, hq, a.Hq, a.L, a.total)), 0,
                (uint32_t)((int64_t)L * sizeof(RowStat)), kBufferFlags);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (lds_void *)ts, 16, (r0 + lane) * 16, 0, 0, 0);
        }
    };
    int tile = next_tile(0);  // the diagonal block's rows always see the block
    dma_tile(tile, lq0, lr0, lg0, ls0);

    floatx4 accK[KBW][8], accV[KBW][8];
#pragma unroll
    for (int c = 0; c < KBW; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) accK[c][e] = accV[c][e] = floatx4{0.f, 0.f, 0.f, 0.f};
    const int rperm = (n >> 2) + 4 * (n & 3);
    const float rk_over_qk = a.rk_scale / a.qk_scale;  // qk_scale > 0 (checked by the API)

    // one 32-row sub-tile at tile row xl (global row rs)
    auto sub_tile = [&](const uint16_t *tq, const uint16_t *tr, const uint16_t *tg, const RowStat *ts,
                        int xl, int rs, bool mask) __attribute__((always_inline)) {
        floatx4 z[KBW][2], s[KBW][2], uu[KBW][2];
#pragma unroll
        for (int c = 0; c < KBW; ++c)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) z[c][tb] = s[c][tb] = uu[c][tb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            const int x = xl + 16 * tb + rperm;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bf16x8 fq = lds_chunk(tq, x, g + 4 * u);
                const bf16x8 fr = lds_chunk(tr, x, g + 4 * u);
                const bf16x8 fg = lds_chunk(tg, x, g + 4 * u);
#pragma unroll
                for (int c = 0; c < KBW; ++c) {
                    z[c][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fq, kop[c][u], z[c][tb], 0, 0, 0);
                    s[c][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr, kop[c][u], s[c][tb], 0, 0, 0);
                    uu[c][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fg, vop[c][u], uu[c][tb], 0, 0, 0);
                }
            }
        }
        bf16x8 p1[KBW], pz[KBW], ps[KBW];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const RowStat st = ts[xl + g + 4 * t];
            const int rw = rs + g + 4 * t;
#pragma unroll
            for (int c = 0; c < KBW; ++c) {
                const float zz = z[c][t >> 2][t & 3], ss = s[c][t >> 2][t & 3], u = uu[c][t >> 2][t & 3];
                float w = __builtin_amdgcn_exp2f(fmaf(zz, a.zscale, -st.lse2));
                const int key = kw + 16 * c + n;
                if (mask && (rw < key || rw >= key + W || rw >= L)) w = 0.f;
                const float sc = fmaf(ss, a.rk_scale, -st.sbar);
                p1[c][t] = (__bf16)fmaf(w, sc, w);  // w (1 + sc)
                // dk = qk_scale (sum dz q + (rk_scale / qk_scale) sum ds r): qk_scale is
                // applied once to the accumulator, not to every element
                pz[c][t] = (__bf16)(w * (fmaf(sc, u, u) - fmaf(st.ubar, sc, st.delta)));
                ps[c][t] = (__bf16)(w * (u - st.ubar) * rk_over_qk);
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bf16x8 gt = lds_transposed(tg, xl, e, g, n);
            const bf16x8 qt = lds_transposed(tq, xl, e, g, n);
            const bf16x8 rt = lds_transposed(tr, xl, e, g, n);
#pragma unroll
            for (int c = 0; c < KBW; ++c) {
                accV[c][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(gt, p1[c], accV[c][e], 0, 0, 0);
                accK[c][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qt, pz[c], accK[c][e], 0, 0, 0);
                accK[c][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rt, ps[c], accK[c][e], 0, 0, 0);
            }
        }
    };
    auto step = [&](int tile, int nxt, uint16_t *tq, uint16_t *tr, uint16_t *tg, RowStat *ts,
                    uint16_t *nq, uint16_t *nr, uint16_t *ng, RowStat *ns) __attribute__((always_inline)) {
        if (nxt < ntiles) dma_tile(nxt, nq, nr, ng, ns);
        const int r0 = k0 + (tile % nrt) * TR;
#pragma unroll
        for (int j = 0; j < TR / 32; ++j) {
            const int rs = r0 + 32 * j;
            // wave-uniform: sub-tiles that see none of the wave's keys are skipped
            if (rs + 31 >= kw && rs < kw + 16 * KBW - 1 + W) {
                const bool mask = rs < kw + 16 * KBW - 1 || rs + 31 >= kw + W || rs + 31 >= L;
                if (mask)
                    sub_tile(tq, tr, tg, ts, 32 * j, rs, true);
                else
                    sub_tile(tq, tr, tg, ts, 32 * j, rs, false);
            }
        }
        __syncthreads();
    };
    __syncthreads();
    if constexpr (!MASK) {
        for (; tile < ntiles; tile += 2) {
            step(tile, tile + 1, lq0, lr0, lg0, ls0, lq1, lr1, lg1, ls1);
            if (tile + 1 < ntiles) step(tile + 1, tile + 2, lq1, lr1, lg1, ls1, lq0, lr0, lg0, ls0);
        }
    } else {
        while (true) {
            int nxt = next_tile(tile + 1);
            step(tile, nxt, lq0, lr0, lg0, ls0, lq1, lr1, lg1, ls1);
            if (nxt >= ntiles) break;
            tile = nxt;
            nxt = next_tile(tile + 1);
            step(tile, nxt, lq1, lr1, lg1, ls1, lq0, lr0, lg0, ls0);
            if (nxt >= ntiles) break;
            tile = nxt;
        }
    }

#pragma unroll
    for (int c = 0; c < KBW; ++c) {
        const int key = kw + 16 * c + n;
        if (key < L) {
            // block e, accumulator element i holds dim 16 e + 4 g + i of the key
            uint16_t *dk = reinterpret_cast<uint16_t *>(a.dk) + kvbase + (int64_t)key * ks + 4 * g;
            uint16_t *dv = reinterpret_cast<uint16_t *>(a.dv) + kvbase + (int64_t)key * ks + 4 * g;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                *reinterpret_cast<uint2 *>(dk + 16 * e) =
                    uint2{pack_bf16x2(accK[c][e][0] * a.qk_scale, accK[c][e][1] * a.qk_scale),
                          pack_bf16x2(accK[c][e][2] * a.qk_scale, accK[c][e][3] * a.qk_scale)};
                *reinterpret_cast<uint2 *>(dv + 16 * e) =
                    uint2{pack_bf16x2(accV[c][e][0], accV[c][e][1]), pack_bf16x2(accV[c][e][2], accV[c][e][3])};
            }
        }
    }
}

// PERSIST = false: one work item per workgroup (dense batches); true: a
// persistent grid drawing items from per-XCD queues (packed batches; the
// row pass uses counters 0..7, the key pass 8..15).
template <int HPW, bool PERSIST, bool MASK>
__global__ __launch_bounds__(64 * kBwdWaves) void bwd_rows_mfma_bf16_d128(BackwardArgs a) {
    if (!PERSIST) {
        bwd_rows_item<HPW, MASK, false>(a, blockIdx.x);
        return;
    }
    constexpr int RPH = 16 * kBwdWaves / HPW;
    const int n_items = a.B * a.Hkv * (a.Hq / a.Hkv / HPW) * ((a.L + RPH - 1) / RPH);
    for (int item = next_item(a.sched, n_items); item >= 0; item = next_item(a.sched, n_items))
        bwd_rows_item<HPW, MASK, true>(a, item);
}

template <bool PERSIST, bool MASK>
__global__ __launch_bounds__(64 * kKeyWaves) void bwd_keys_mfma_bf16_d128(BackwardArgs a) {
    if (!PERSIST) {
        bwd_keys_item<MASK>(a, blockIdx.x);
        return;
    }
    constexpr int KB = 16 * kKeyBlocksPerWave * kKeyWaves;
    const int n_items = a.B * a.Hkv * ((a.L + KB - 1) / KB);
    for (int item = next_item(a.sched + 8, n_items); item >= 0; item = next_item(a.sched + 8, n_items))
        bwd_keys_item<MASK>(a, item);
}

template <typename T, int D>
hipError_t launch_generic(const BackwardArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL((bwd_rows_generic<T, D>), dim3(a.L, a.Hq, a.B), dim3(64), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((bwd_keys_generic<T, D>), dim3(a.L, a.Hkv, a.B), dim3(64), 0, stream, a);
    return hipGetLastError();
}



// The row pass, then the key pass, on matrix cores (MASK: a block mask is given).
template <bool MASK>
hipError_t launch_mfma_passes(const BackwardArgs &a, int hpw, long row_items, long key_items,
                              hipStream_t stream) {
    // persistent workers, a multiple of 8 so that every XCD share is drained
    auto workers = [&](long items) { return (unsigned)(((items < a.workers ? items : a.workers) + 7) / 8 * 8); };
    hipError_t err;
    if (a.sched) {
        err = launch_zero_counters(a.sched, 16, stream);
        if (err != hipSuccess) return err;
        if (hpw == 2)
            hipLaunchKernelGGL((bwd_rows_mfma_bf16_d128<2, true, MASK>), dim3(workers(row_items)),
                               dim3(64 * kBwdWaves), 0, stream, a);
        else
            hipLaunchKernelGGL((bwd_rows_mfma_bf16_d128<1, true, MASK>), dim3(workers(row_items)),
                               dim3(64 * kBwdWaves), 0, stream, a);
    } else if (hpw == 2) {
        hipLaunchKernelGGL((bwd_rows_mfma_bf16_d128<2, false, MASK>), dim3((unsigned)row_items),
                           dim3(64 * kBwdWaves), 0, stream, a);
    } else {
        hipLaunchKernelGGL((bwd_rows_mfma_bf16_d128<1, false, MASK>), dim3((unsigned)row_items),
                           dim3(64 * kBwdWaves), 0, stream, a);
    }
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (a.sched)
        hipLaunchKernelGGL((bwd_keys_mfma_bf16_d128<true, MASK>), dim3(workers(key_items)),
                           dim3(64 * kKeyWaves), 0, stream, a);
    else
        hipLaunchKernelGGL((bwd_keys_mfma_bf16_d128<false, MASK>), dim3((unsigned)key_items),
                           dim3(64 * kKeyWaves), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_backward(const BackwardArgs &a, int dtype, hipStream_t stream) {
    const int G = a.Hq / a.Hkv;
    if (dtype == 1 && a.D == 128) {
        // as the forward: two query heads per row-pass item for even group sizes
        const int hpw = (G % 2 == 0) ? 2 : 1;
        const int rph = 16 * kBwdWaves / hpw;
        const long row_items = (long)a.B * a.Hkv * (G / hpw) * ((a.L + rph - 1) / rph);
        constexpr int kb = 16 * kKeyBlocksPerWave * kKeyWaves;
        const long key_items = (long)a.B * a.Hkv * ((a.L + kb - 1) / kb);
        if (row_items <= 0x7fffffffL && key_items <= 0x7fffffffL)
            return a.block_mask ? launch_mfma_passes<true>(a, hpw, row_items, key_items, stream)
                                : launch_mfma_passes<false>(a, hpw, row_items, key_items, stream);
    }
    if (dtype == 1)
        return a.D == 64 ? launch_generic<uint16_t, 64>(a, stream) : launch_generic<uint16_t, 128>(a, stream);
    return a.D == 64 ? launch_generic<float, 64>(a, stream) : launch_generic<float, 128>(a, stream);
}

}  // namespace plx
