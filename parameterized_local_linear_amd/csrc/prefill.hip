// Parallax causal prefill (training forward) kernels for gfx950.
//
// What is computed (PyPI README of parallax-kernel, "Training (Triton)":
// parallax_func(q, r, k, v) on (B, H, L, D) tensors, causal): for query
// row i of head h, the visible keys are 0 .. i of KV head h / (Hq / Hkv) and
//   o_i = sum_j w_ij v_j + sum_j w_ij (s_ij - sbar_i) v_j,
//   w_i = softmax(qk_scale q_i.k_j), s_ij = rk_scale r_i.k_j.
// Optional row statistics for a backward pass: lse_i = ln sum_j exp(z_ij)
// and sbar_i.
//
// prefill_mfma_bf16_d128<HPW, MASK>: bf16, head_dim 128, all four contractions
// (Q K^T, R K^T, P V, (P o S) V) on v_mfma_f32_16x16x32_bf16 with fp32
// accumulation. Described at the kernel.
// prefill_generic<T, D>: any dtype / head_dim; one wave per query row,
// the streaming state of the decode kernels (pivot = probe score of key 0),
// with the key rows of a batch of steps in flight at once.
#include "plx_internal.h"
#include "plx_device.h"


namespace plx {

namespace {

template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
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
struct Vec16<uint16_t> {
    static constexpr int n = 8;
    __device__ static void load(const uint16_t *p, float *out) {
        uint4 x = *reinterpret_cast<const uint4 *>(p);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    __device__ static void store(uint16_t *p, const float *in) {
        *reinterpret_cast<uint4 *>(p) = uint4{pack_bf16x2(in[0], in[1]), pack_bf16x2(in[2], in[3]),
                                              pack_bf16x2(in[4], in[5]), pack_bf16x2(in[6], in[7])};
    }
};

template <typename T, int D>
__global__ __launch_bounds__(64) void prefill_generic(PrefillArgs a) {
    constexpr int EPL = Vec16<T>::n;
    constexpr int LPR = D / EPL;
    constexpr int KPI = 64 / LPR;
    static_assert(LPR * KPI == 64, "lanes must tile the wave");
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
    const T *kb = reinterpret_cast<const T *>(a.k) + row0_elem(sq, b, hkv, a.Hkv, a.L, D) + c * EPL;
    const T *vb = reinterpret_cast<const T *>(a.v) + row0_elem(sq, b, hkv, a.Hkv, a.L, D) + c * EPL;

    float qv[EPL], rv[EPL];
    Vec16<T>::load(reinterpret_cast<const T *>(a.q) + row + c * EPL, qv);
    Vec16<T>::load(reinterpret_cast<const T *>(a.r) + row + c * EPL, rv);
    for (int e = 0; e < EPL; ++e) {
        qv[e] *= a.zscale;
        rv[e] *= a.rk_scale;
    }
    const int first = max(0, i - a.window + 1);  // sliding window: keys first .. i
    float piv;
    {
        float k0[EPL];
        Vec16<T>::load(kb + (int64_t)first * ks, k0);
        float part = 0.f;
        for (int e = 0; e < EPL; ++e) part += rv[e] * k0[e];
        for (int off = 1; off < LPR; off <<= 1) part += __shfl_xor(part, off, LPR);
        piv = part;
    }
    float m = -INFINITY, l = 0.f, S = 0.f, A[EPL], Bv[EPL];
    for (int e = 0; e < EPL; ++e) {
        A[e] = 0.f;
        Bv[e] = 0.f;
    }
    const int end = i + 1;
    // block-sparse: this row's query block's mask row (its own block is always visible)
    const int nb = (a.L + kMaskBlock - 1) >> kMaskShift;
    const uint8_t *mrow = a.block_mask
        ? a.block_mask + (((int64_t)b * a.Hkv + hkv) * nb + (i >> kMaskShift)) * nb : nullptr;
    // Step t covers keys first + KPI t .. + KPI - 1 (key group kgrp takes one).
    // The key rows of a batch of U steps are loaded while the batch before is
    // folded in; a batch's dot products reduce with DPP lane exchanges, and
    // its max rescales the state once.
    constexpr int U = EPL == 4 ? 8 : 4;
    const int nit = (end - first + KPI - 1) / KPI;
    auto load_step = [&](int t, float *kv, float *vv) __attribute__((always_inline)) {
        const int jj = min(first + t * KPI + kgrp, end - 1);  // past the end: a valid row, unused
        Vec16<T>::load(kb + (int64_t)jj * ks, kv);
        Vec16<T>::load(vb + (int64_t)jj * ks, vv);
    };
    auto fold_batch = [&](int t0, float (*kv)[EPL], float (*vv)[EPL]) __attribute__((always_inline)) {
        float zs[U], ss[U];
        bool val[U];
        float mb = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = first + (t0 + u) * KPI + kgrp;
            bool valid = t0 + u < nit && j < end;
            if (mrow && valid && (j >> kMaskShift) != (i >> kMaskShift)) valid = mrow[j >> kMaskShift] != 0;
            float zp = 0.f, sp = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                zp += qv[e] * kv[u][e];
                sp += rv[e] * kv[u][e];
            }
            zs[u] = group_sum<LPR>(zp);
            ss[u] = group_sum<LPR>(sp);
            val[u] = valid;
            if (valid) mb = fmaxf(mb, zs[u]);
        }
        if (mb == -INFINITY) return;  // nothing visible in this batch for this key group
        const float m_new = fmaxf(m, mb);
        const float alpha = __builtin_amdgcn_exp2f(m - m_new);
        m = m_new;
        l *= alpha;
        S *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            A[e] *= alpha;
            Bv[e] *= alpha;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!val[u]) continue;
            const float p = __builtin_amdgcn_exp2f(zs[u] - m_new);
            const float sd = ss[u] - piv;
            l += p;
            S += p * sd;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                A[e] += p * vv[u][e];
                Bv[e] += (p * sd) * vv[u][e];
            }
        }
    };
    float kcur[U][EPL], vcur[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) load_step(u, kcur[u], vcur[u]);
    for (int t0 = 0; t0 < nit; t0 += U) {
        float knext[U][EPL], vnext[U][EPL];
#pragma unroll
        for (int u = 0; u < U; ++u) load_step(t0 + U + u, knext[u], vnext[u]);
        fold_batch(t0, kcur, vcur);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                kcur[u][e] = knext[u][e];
                vcur[u][e] = vnext[u][e];
            }
    }
    for (int off = LPR; off < 64; off <<= 1) {
        const float mo = __shfl_xor(m, off);
        const float lo = __shfl_xor(l, off);
        const float So = __shfl_xor(S, off);
        const float M = fmaxf(m, mo);
        const float ax = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - M);
        const float ay = (mo == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mo - M);
        for (int e = 0; e < EPL; ++e) {
            const float Ao = __shfl_xor(A[e], off);
            const float Bo = __shfl_xor(Bv[e], off);
            A[e] = A[e] * ax + Ao * ay;
            Bv[e] = Bv[e] * ax + Bo * ay;
        }
        m = M;
        l = l * ax + lo * ay;
        S = S * ax + So * ay;
    }
    if (kgrp != 0) return;
    const float inv_l = 1.0f / l;
    const float cA = 1.0f - S * inv_l;
    float ov[EPL];
    for (int e = 0; e < EPL; ++e) ov[e] = (A[e] * cA + Bv[e]) * inv_l;
    Vec16<T>::store(reinterpret_cast<T *>(a.o) + row + c * EPL, ov);
    if (a.vbar) {
        for (int e = 0; e < EPL; ++e) ov[e] = A[e] * inv_l;
        Vec16<T>::store(reinterpret_cast<T *>(a.vbar) + row + c * EPL, ov);
    }
    if (c == 0) {
        if (a.lse) a.lse[srow] = m * 0.6931471805599453f + logf(l);
        if (a.sbar) a.sbar[srow] = S * inv_l + piv;
    }
}

// -------------------------------------------------------------------------
// MFMA prefill, bf16, head_dim 128.
//
// Workgroup: eight waves over one (sequence, KV head, group of HPW query
// heads, q-tile of 128 / HPW rows per head); each wave owns 16 query rows of
// one head. Every query head of the workgroup reads the same KV head, so one
// K/V tile in LDS feeds all eight waves.
//
// K/V tiles of kPrefillKeys keys are copied by the buffer unit straight into
// LDS (buffer_load ... lds), double buffered in two separate LDS arrays: the
// next tile's copy is issued before the current tile is consumed and only
// waited for at the end of the tile. LDS rows are 256 bytes, with 16-byte
// chunk c of key k stored at chunk slot c ^ swz(k & 15),
// swz(x) = 2 ((x >> 2) & 3) + 9 (x & 1). Both operand reads are then free of
// LDS bank conflicts (checked with the bank-conflict counter): the 128-bit K
// reads, served eight lanes at a time, see eight distinct values of
// slot & 7, and the transposing 64-bit V reads, served 32 lanes at a time
// over all 64 banks, see 16 distinct slots, each with both 8-byte halves.
//
// Per 32-key sub-tile the wave computes, as in the decode kernel but with
// query columns instead of head/probe columns:
//   scores  Z^T[key, q] = K . Q^T,  S^T[key, q] = K . R^T   (16 MFMAs)
//   readout A^T[d, q] += V^T . P^T, B^T[d, q] += V^T . (P o S')^T (16 MFMAs)
// with the score MFMA's key order permuted so that lane (g, n) receives the
// scores of query n for exactly the keys g + 4t it feeds the readout MFMA
// (P never leaves registers), and the V^T operand read from the row-major
// LDS tile with gfx950's transposing LDS read (ds_read_b64_tr_b16).
// S' is carried unscaled: the probe MFMAs accumulate onto -pivot, so they
// return r.k - pivot and the vector unit only multiplies by P; the probe
// scale multiplies B, S and the pivot once per row at the end. On tiles whose
// keys all rows see, the sub-tiles are software-pipelined (the score MFMAs of
// the next sub-tile come before the softmax of the current one); the
// vector work per sub-tile (exp, rescale test, the row sums and the bf16
// packing) costs about as many issue cycles as the products themselves.
//
// Causality: keys j <= i, and with a sliding window W also j > i - W. Tiles
// entirely outside a wave's visible band are skipped, tiles crossing either
// edge of the band are masked (and their 32-key sub-tiles holding none of the
// wave's keys skipped). A block-sparse mask removes whole tiles (a tile is one
// 128-key block, a work item's rows lie in one 128-row block): the loop walks
// the visible tiles only, so hidden ones are neither copied nor computed. Work items run heaviest-first
// (last q-tile first), and the group index varies fastest so that all
// q-tiles of one (sequence, KV head) land on one XCD when the number of
// groups is a multiple of 8 (its L2 then holds that head's K/V).
// -------------------------------------------------------------------------
constexpr int kPrefillKeys = 128;  // keys per LDS tile
constexpr int kPrefillWaves = 8;
constexpr int kDenseWorkersPerCU = 4;  // persistent workgroups per CU for dense batches

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));

// One work item; returns before any barrier when the item lies past its
// sequence's end.
template <int HPW, bool MASK>
__device__ __forceinline__ void prefill_item(const PrefillArgs &a, const int item) {
    constexpr int D = 128;
    constexpr int NW = kPrefillWaves;
    constexpr int WPH = NW / HPW;       // waves per head
    constexpr int RPH = 16 * WPH;       // rows per head per work item
    constexpr int TK = kPrefillKeys;
    constexpr int NSUB = TK / 32;       // sub-tiles per tile
    constexpr int DMA = TK / (4 * NW);  // 1 KB copies (4 keys) of K, and of V, per wave per tile
    static_assert(NW % HPW == 0 && DMA >= 1, "bad workgroup shape");
    static_assert(TK == kMaskBlock && kMaskBlock % RPH == 0, "a tile is one mask block");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int g = lane >> 4;

    // ---- work item: heaviest q-tile first, group fastest
    const int G = a.Hq / a.Hkv;
    const int hgroups = G / HPW;                    // head groups per KV head
    const int NG = a.B * a.Hkv * hgroups;           // groups
    const int QT = (a.L + RPH - 1) / RPH;           // q-tiles per group
    const int grp = item % NG;
    const int qt = QT - 1 - item / NG;
    const int b = grp / (a.Hkv * hgroups);
    const int hkv = (grp / hgroups) % a.Hkv;
    const int hsub = grp % hgroups;
    const int hq = hkv * G + hsub * HPW + wave / WPH;
    const int q0 = qt * RPH + (wave % WPH) * 16;    // this wave's first row
    const PrefillSeq sq = prefill_seq(a.cu, b, a.L);
    const int L = sq.len;
    if (qt * RPH >= L) return;  // work item past this sequence's end (packed batches)
    const int kend = min(L, (qt + 1) * RPH);        // keys the workgroup needs
    const int ntiles = (kend + TK - 1) / TK;
    const int W = a.window;                          // query i sees keys i - W + 1 .. i
    const int tile0 = max(0, qt * RPH - W + 1) / TK;  // first tile any row of the item sees

    const uint16_t *qh = reinterpret_cast<const uint16_t *>(a.q);
    const uint16_t *rh = reinterpret_cast<const uint16_t *>(a.r);
    const int64_t kvbase = row0_elem(sq, b, hkv, a.Hkv, a.L, D);
    const int ks = row_stride(sq, a.Hkv, D);                  // elements between keys
    const uint32_t kvbytes = (uint32_t)(((int64_t)(L - 1) * ks + D) * 2);  // this sequence only
    const int64_t qbase = row0_elem(sq, b, hq, a.Hq, a.L, D);
    const int qs = row_stride(sq, a.Hq, D);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(reinterpret_cast<const uint16_t *>(a.k) + kvbase), 0, kvbytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(reinterpret_cast<const uint16_t *>(a.v) + kvbase), 0, kvbytes, kBufferFlags);

    // ---- LDS: two K/V tiles in separate arrays (so that the compiler waits
    // for a tile's copy only where that tile is read)
    __shared__ __attribute__((aligned(16))) uint16_t lds_k0[TK * D], lds_v0[TK * D];
    __shared__ __attribute__((aligned(16))) uint16_t lds_k1[TK * D], lds_v1[TK * D];
    auto swz = [](int key) { return 2 * ((key >> 2) & 3) + 9 * (key & 1); };
    // copy j of this wave: keys 4 (wave * DMA + j) + lane / 16; lane writes LDS
    // slot lane % 16 of its key, i.e. fetches chunk (lane % 16) ^ swz(key)
    auto dma_tile = [&](int tile, uint16_t *lk, uint16_t *lv) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < DMA; ++j) {
            const int kloc = 4 * (wave * DMA + j);
            const int key = kloc + (lane >> 4);
            const int chunk = (lane & 15) ^ swz(key);
            const int off = ((tile * TK + key) * ks + chunk * 8) * 2;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void *)(lk + kloc * D), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void *)(lv + kloc * D), 16, off, 0, 0, 0);
        }
    };
    // block-sparse: the tiles (key blocks) this item's query block sees
    const int qb = (qt * RPH) >> kMaskShift;
    const int nb = (a.L + kMaskBlock - 1) >> kMaskShift;
    const uint8_t *mrow = MASK ? a.block_mask + (((int64_t)b * a.Hkv + hkv) * nb + qb) * nb : nullptr;
    uint64_t vbits = 0;
    int vbase = -64;
    auto next_tile = [&](int t) {
        if constexpr (!MASK) return t;
        return next_visible(t, ntiles, vbits, vbase, [&](int u) { return u == qb || mrow[u] != 0; });
    };
    int tile = next_tile(tile0);  // the diagonal tile is always visible
    dma_tile(tile, lds_k0, lds_v0);

    // ---- per-wave query operands (k-step u)
    bf16x8 qop[4], rop[4];
    {
        const int row = min(q0 + n, L - 1);
        const uint16_t *qp = qh + qbase + (int64_t)row * qs;
        const uint16_t *rp = rh + qbase + (int64_t)row * qs;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            qop[u] = load16(qp + 8 * (g + 4 * u));
            rop[u] = load16(rp + 8 * (g + 4 * u));
        }
    }

    // The row's probe pivot, in units of the raw product r . k (the probe
    // scale multiplies it, S and B once, in the epilogue). It starts at 0 and
    // follows the row's running weighted mean of r . k (kPivotDrift; the
    // threshold is taken in probe-scale units). The probe products start from
    // -pivot, so the matrix cores return the centred r . k - pivot directly.
    float piv = 0.f;
    floatx4 pivq = {0.f, 0.f, 0.f, 0.f};
    const float drift_raw = a.rk_scale != 0.f ? kPivotDrift / fabsf(a.rk_scale) : INFINITY;
    // Reference max (log2 units). Finite from the start: with a sliding window
    // a row can meet a sub-tile in which none of its keys is visible before
    // it has seen any key, and exp2(-inf - m) must then be 0, not NaN.
    float m_run = -1e30f, lsA = 0.f, lsS = 0.f;
    floatx4 accA[8], accB[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        accA[e] = floatx4{0.f, 0.f, 0.f, 0.f};
        accB[e] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    const int kperm = (n >> 2) + 4 * (n & 3);
    const int row = q0 + n;
    const int q_last = q0 + 15;

    struct Scores {
        floatx4 z0, z1, s0, s1;
    };
    struct Probs {
        bf16x8 pa, ps;
    };
    struct KOp {
        bf16x8 k[2][4];
    };
    struct VOp {
        bf16x8 v[8];
    };
    // K operand of the 32-key sub-tile at local key kl: block kb, k-step u ->
    // key kl + 16kb + kperm, chunk g + 4u
    auto load_k = [&](const uint16_t *lk, int kl) __attribute__((always_inline)) {
        KOp op;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int key = kl + 16 * kb + kperm;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                op.k[kb][u] = *reinterpret_cast<const bf16x8 *>(&lk[key * D + (((g + 4 * u) ^ swz(key)) * 8)]);
        }
        return op;
    };
    // V^T operand of readout block b (dims 16b .. 16b + 15), from LDS with the
    // transposing 64-bit read: within each 16-lane row, lane j points at
    // 4 dims of one key and lane i receives dim 16b + i of four keys. Lane
    // (g, n) gets keys g + 4t (t = 0..7, two reads), the keys it feeds as
    // element t of P in the score layout.
    auto load_vT = [&](const uint16_t *lv, int kl) __attribute__((always_inline)) {
        VOp op;
        const int q4 = n >> 2, dq = n & 3;  // this lane points at key g + 4 (q4 + 4h), dims 4 dq ..
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const int dim = 16 * b + 4 * dq;
            v4i16 part[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int key = kl + g + 4 * (q4 + 4 * h);
                const int addr = key * D + (((dim >> 3) ^ swz(key)) * 8) + (dim & 7);
                part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16 *)(lv + addr));
            }
            op.v[b] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
        return op;
    };
    auto scores = [&](const KOp &op) __attribute__((always_inline)) {
        Scores sc;
        sc.z0 = sc.z1 = floatx4{0.f, 0.f, 0.f, 0.f};
        sc.s0 = sc.s1 = pivq;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            sc.z0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.k[0][u], qop[u], sc.z0, 0, 0, 0);
            sc.z1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.k[1][u], qop[u], sc.z1, 0, 0, 0);
            sc.s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.k[0][u], rop[u], sc.s0, 0, 0, 0);
            sc.s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.k[1][u], rop[u], sc.s1, 0, 0, 0);
        }
        return sc;
    };
    auto pv = [&](const Probs &p, const VOp &vo) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            accA[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vo.v[e], p.pa, accA[e], 0, 0, 0);
            accB[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vo.v[e], p.ps, accB[e], 0, 0, 0);
        }
    };
    // Softmax update of the sub-tile at key k0, in two halves. The first masks
    // the logits of keys a row cannot see (diag) and rescales the accumulators
    // when the reference max is raised. Lazy rescale: the lane-local max decides
    // whether any logit of the column exceeds the reference by more than the
    // slack; only then is the column max taken across the four rows.
    auto rescale = [&](Scores &sc, int k0, bool diag) __attribute__((always_inline)) {
        float rmax = -INFINITY;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            float z = t < 4 ? sc.z0[t] : sc.z1[t - 4];
            const int key = k0 + g + 4 * t;
            if (diag && (key > row || key <= row - W)) {
                z = -INFINITY;
                if (t < 4) sc.z0[t] = z; else sc.z1[t - 4] = z;
            }
            rmax = fmaxf(rmax, z);
        }
        const bool raise = rmax * a.zscale > m_run + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
            const float tmax = xor_max_rowgroups(rmax) * a.zscale;
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            lsA *= alpha;
            lsS *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                accA[e] *= alpha;
                accB[e] *= alpha;
            }
        }
    };
    // The second half returns the bf16 operands P and P o S', S' taken in units
    // of the raw probe product (the scale is applied once, at the end). When a
    // lane's partial sums show the pivot has drifted from the row's running
    // mean, the row is re-based before the operands are rounded; `nx` holds
    // scores already taken against the old pivot (the next sub-tile's, when
    // the sub-tiles are software-pipelined) and is shifted with it.
    auto probs = [&](const Scores &sc, Scores &nx) __attribute__((always_inline)) {
        const float neg_m = -m_run;
        Probs pr;
        float suma = 0.f, sums = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float z = t < 4 ? sc.z0[t] : sc.z1[t - 4];
            const float s = t < 4 ? sc.s0[t] : sc.s1[t - 4];
            const float p = __builtin_amdgcn_exp2f(fmaf(z, a.zscale, neg_m));
            const float q = p * s;
            suma += p;
            sums += q;
            pr.pa[t] = (__bf16)p;
            pr.ps[t] = (__bf16)q;
        }
        lsA += suma;
        lsS += sums;
        if (__builtin_amdgcn_ballot_w64(fabsf(lsS) > drift_raw * lsA) != 0) {
            // rare: re-base the row and form this sub-tile's P o S' again
            const float lrow = xor_sum_rowgroups(lsA);
            const float srow = xor_sum_rowgroups(lsS);
            const float d = lrow > 0.f ? srow / lrow : 0.f;
            piv += d;
            pivq = floatx4{-piv, -piv, -piv, -piv};
            lsS = fmaf(-d, lsA, lsS);
#pragma unroll
            for (int e = 0; e < 8; ++e) accB[e] -= d * accA[e];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float z = t < 4 ? sc.z0[t] : sc.z1[t - 4];
                const float s = t < 4 ? sc.s0[t] : sc.s1[t - 4];
                const float p = __builtin_amdgcn_exp2f(fmaf(z, a.zscale, neg_m));
                pr.ps[t] = (__bf16)(p * (s - d));
            }
            nx.s0 -= d;
            nx.s1 -= d;
        }
        return pr;
    };
    // one tile: its sub-tiles in order
    // (on a masked tile, sub-tiles that hold none of the wave's keys are skipped)
    auto tile_body = [&](const uint16_t *lk, const uint16_t *lv, int tile, bool diag) __attribute__((always_inline)) {
        const int t0 = tile * TK;
#pragma unroll
        for (int j = 0; j < NSUB; ++j) {
            const int k0 = t0 + 32 * j;
            if (diag && (k0 > q_last || k0 + 31 <= q0 - W)) continue;  // wave-uniform
            Scores sc = scores(load_k(lk, 32 * j));
            rescale(sc, k0, diag);
            Scores none{};
            pv(probs(sc, none), load_vT(lv, 32 * j));
        }
    };
    // The same on a tile whose keys every row sees, software-pipelined: the
    // score products of sub-tile j + 1 come before the probabilities of j in
    // program order, and the compiler's scheduler interleaves the two. (Forcing
    // one MFMA between every two, three or four vector instructions with
    // sched_group_barrier measured 1-2% slower.)
    auto tile_body_full = [&](const uint16_t *lk, const uint16_t *lv, int tile) __attribute__((always_inline)) {
        const int t0 = tile * TK;
        Scores cur = scores(load_k(lk, 0));
#pragma unroll
        for (int j = 0; j < NSUB; ++j) {
            rescale(cur, t0 + 32 * j, false);
            Scores nxt{};
            if (j + 1 < NSUB) nxt = scores(load_k(lk, 32 * (j + 1)));
            const Probs p = probs(cur, nxt);
            pv(p, load_vT(lv, 32 * j));
            cur = nxt;
        }
    };
    auto tile_step = [&](int tile, int nxt, uint16_t *lk, uint16_t *lv, uint16_t *nk, uint16_t *nv) __attribute__((always_inline)) {
        if (nxt < ntiles) dma_tile(nxt, nk, nv);
        const int t0 = tile * TK;
        // wave-uniform: tiles above the wave's rows or left of all their windows are skipped;
        // a tile needs the mask unless every key is visible to all 16 rows
        if (t0 <= q_last && t0 + TK - 1 > q0 - W) {
            if (t0 + TK - 1 <= q0 && t0 > q_last - W)
                tile_body_full(lk, lv, tile);
            else
                tile_body(lk, lv, tile, true);
        }
        __syncthreads();  // waits for the next tile's copy, releases this buffer
    };

    __syncthreads();
    if constexpr (!MASK) {
        for (; tile < ntiles; tile += 2) {
            tile_step(tile, tile + 1, lds_k0, lds_v0, lds_k1, lds_v1);
            if (tile + 1 < ntiles) tile_step(tile + 1, tile + 2, lds_k1, lds_v1, lds_k0, lds_v0);
        }
    } else {
        while (true) {
            int nxt = next_tile(tile + 1);
            tile_step(tile, nxt, lds_k0, lds_v0, lds_k1, lds_v1);
            if (nxt >= ntiles) break;
            tile = nxt;
            nxt = next_tile(tile + 1);
            tile_step(tile, nxt, lds_k1, lds_v1, lds_k0, lds_v0);
            if (nxt >= ntiles) break;
            tile = nxt;
        }
    }

    // ---- epilogue: o = (A + B - (S / l) A) / l per row
    const float l = xor_sum_rowgroups(lsA);
    const float S = xor_sum_rowgroups(lsS) * a.rk_scale;
    if (row < L) {
        const float inv_l = 1.0f / l;
        const float cA = 1.0f - S * inv_l;
        const int64_t ro = stat0(sq, b, hq, a.Hq, a.L) + (int64_t)row * stat_stride(sq, a.Hq);
        // readout block b, accumulator element i holds dim 16b + 4g + i
        uint16_t *o = reinterpret_cast<uint16_t *>(a.o) + qbase + (int64_t)row * qs + 4 * g;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            float ov[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = (accA[b][i] * cA + accB[b][i] * a.rk_scale) * inv_l;
            *reinterpret_cast<uint2 *>(o + 16 * b) = uint2{pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3])};
        }
        if (a.vbar) {  // the softmax readout A / l, for a backward pass
            uint16_t *vb = reinterpret_cast<uint16_t *>(a.vbar) + qbase + (int64_t)row * qs + 4 * g;
#pragma unroll
            for (int b = 0; b < 8; ++b)
                *reinterpret_cast<uint2 *>(vb + 16 * b) = uint2{pack_bf16x2(accA[b][0] * inv_l, accA[b][1] * inv_l),
                                                                pack_bf16x2(accA[b][2] * inv_l, accA[b][3] * inv_l)};
        }
        if (g == 0) {
            if (a.lse) a.lse[ro] = fmaf(m_run, 0.6931471805599453f, logf(l));  // one rounding, whatever the contraction
            if (a.sbar) a.sbar[ro] = fmaf(piv, a.rk_scale, S * inv_l);
        }
    }
}

// Persistent grid. A packed batch (a.sched != nullptr) draws items from the
// per-XCD queues; a dense batch takes items w, w + grid, w + 2 grid, ... in
// order: heaviest first, and with a grid that is a multiple of 8, every item
// of a (sequence, KV head) group on the group's XCD. Either way each item is
// computed whole by one workgroup.
template <int HPW, bool MASK>
__global__ __launch_bounds__(64 * kPrefillWaves) void prefill_mfma_bf16_d128(PrefillArgs a) {
    const int n_items = a.B * a.Hkv * (a.Hq / a.Hkv / HPW) * ((a.L + 16 * kPrefillWaves / HPW - 1) /
                                                            (16 * kPrefillWaves / HPW));
    if (!a.sched) {
        for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
            prefill_item<HPW, MASK>(a, item);
            __syncthreads();  // the next item's first copy overwrites this one's LDS
        }
        return;
    }
    for (int item = next_item(a.sched, n_items); item >= 0; item = next_item(a.sched, n_items))
        prefill_item<HPW, MASK>(a, item);
}

__global__ void zero_counters(int *c, int n) {
    if ((int)threadIdx.x < n) c[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_zero_counters(int *c, int n, hipStream_t stream) {
    hipLaunchKernelGGL(zero_counters, dim3(1), dim3(64), 0, stream, c, n);
    return hipGetLastError();
}

bool prefill_supported(int D, int dtype) { return (D == 64 || D == 128) && (dtype == 0 || dtype == 1); }

hipError_t launch_prefill(const PrefillArgs &a, int dtype, hipStream_t stream) {
    const int G = a.Hq / a.Hkv;
    if (dtype == 1 && a.D == 128) {
        // two query heads per work item when the group size allows it (they
        // share every K/V tile), else one (any group size)
        const int hpw = (G % 2 == 0) ? 2 : 1;
        const int rph = 16 * kPrefillWaves / hpw;
        const long items = (long)a.B * a.Hkv * (G / hpw) * ((a.L + rph - 1) / rph);
        if (items <= 0x7fffffffL) {
            // persistent workers, a multiple of 8 so that every XCD share is drained:
            // one per CU draining the queues of a packed batch, kDenseWorkersPerCU per
            // CU striding over a dense batch's items (fewer launches of a workgroup
            // than items, and a shorter tail; measured 2% faster than one per item)
            const long cap = (long)a.workers * (a.sched ? 1 : kDenseWorkersPerCU);
            const long wgs = ((items < cap ? items : cap) + 7) / 8 * 8;
            if (a.sched) {
                hipError_t err = launch_zero_counters(a.sched, 8, stream);
                if (err != hipSuccess) return err;
            }
            dim3 grid((unsigned)wgs), block(64 * kPrefillWaves);
            if (a.block_mask) {
                if (hpw == 2)
                    hipLaunchKernelGGL((prefill_mfma_bf16_d128<2, true>), grid, block, 0, stream, a);
                else
                    hipLaunchKernelGGL((prefill_mfma_bf16_d128<1, true>), grid, block, 0, stream, a);
            } else if (hpw == 2) {
                hipLaunchKernelGGL((prefill_mfma_bf16_d128<2, false>), grid, block, 0, stream, a);
            } else {
                hipLaunchKernelGGL((prefill_mfma_bf16_d128<1, false>), grid, block, 0, stream, a);
            }
            return hipGetLastError();
        }
    }
    dim3 grid(a.L, a.Hq, a.B);
    if (dtype == 1) {
        if (a.D == 64)
            hipLaunchKernelGGL((prefill_generic<uint16_t, 64>), grid, dim3(64), 0, stream, a);
        else
            hipLaunchKernelGGL((prefill_generic<uint16_t, 128>), grid, dim3(64), 0, stream, a);
    } else {
        if (a.D == 64)
            hipLaunchKernelGGL((prefill_generic<float, 64>), grid, dim3(64), 0, stream, a);
        else
            hipLaunchKernelGGL((prefill_generic<float, 128>), grid, dim3(64), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace plx
