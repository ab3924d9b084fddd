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
// prefill_mfma_bf16_d128<HPW>: bf16, head_dim 128, all four contractions
// (Q K^T, R K^T, P V, (P o S) V) on v_mfma_f32_16x16x32_bf16 with fp32
// accumulation. Described at the kernel.
// prefill_generic<T, D>: any dtype / head_dim; one wave per query row,
// the streaming state of the decode kernels (pivot = probe score of key 0).
#include "plx_internal.h"
#include "plx_device.h"

#include <stdio.h>
#include <stdlib.h>

#include <type_traits>

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
    const int64_t row = ((int64_t)b * a.Hq + hq) * a.L + i;
    const T *kb = reinterpret_cast<const T *>(a.k) + ((int64_t)b * a.Hkv + hkv) * a.L * D + c * EPL;
    const T *vb = reinterpret_cast<const T *>(a.v) + ((int64_t)b * a.Hkv + hkv) * a.L * D + c * EPL;

    float qv[EPL], rv[EPL];
    Vec16<T>::load(reinterpret_cast<const T *>(a.q) + row * D + c * EPL, qv);
    Vec16<T>::load(reinterpret_cast<const T *>(a.r) + row * D + c * EPL, rv);
    for (int e = 0; e < EPL; ++e) {
        qv[e] *= a.zscale;
        rv[e] *= a.rk_scale;
    }
    float piv;
    {
        float k0[EPL];
        Vec16<T>::load(kb, k0);
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
    for (int j0 = 0; j0 < end; j0 += KPI) {
        const int j = j0 + kgrp;
        const bool valid = j < end;
        const int jj = valid ? j : end - 1;
        float kv[EPL], vv[EPL];
        Vec16<T>::load(kb + (int64_t)jj * D, kv);
        Vec16<T>::load(vb + (int64_t)jj * D, vv);
        float zp = 0.f, sp = 0.f;
        for (int e = 0; e < EPL; ++e) {
            zp += qv[e] * kv[e];
            sp += rv[e] * kv[e];
        }
        for (int off = 1; off < LPR; off <<= 1) {
            zp += __shfl_xor(zp, off, LPR);
            sp += __shfl_xor(sp, off, LPR);
        }
        if (valid) {
            const float m_new = fmaxf(m, zp);
            const float alpha = __builtin_amdgcn_exp2f(m - m_new);
            const float p = __builtin_amdgcn_exp2f(zp - m_new);
            const float sd = sp - piv;
            m = m_new;
            l = l * alpha + p;
            S = S * alpha + p * sd;
            for (int e = 0; e < EPL; ++e) {
                A[e] = A[e] * alpha + p * vv[e];
                Bv[e] = Bv[e] * alpha + (p * sd) * vv[e];
            }
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
    Vec16<T>::store(reinterpret_cast<T *>(a.o) + row * D + c * EPL, ov);
    if (c == 0) {
        if (a.lse) a.lse[row] = m * 0.6931471805599453f + logf(l);
        if (a.sbar) a.sbar[row] = S * inv_l + piv;
    }
}

// -------------------------------------------------------------------------
// MFMA prefill, bf16, head_dim 128.
//
// Workgroup: NW waves over one (sequence, KV head, group of HPW query heads,
// q-tile of 16 * QB * NW / HPW rows per head); each wave owns QB blocks of
// 16 query rows of one head. Every query head of the workgroup reads the
// same KV head, so one K/V tile in LDS feeds all the waves.
//
// K/V tiles of 64 keys are copied global -> registers -> LDS, double
// buffered: the next tile's global loads are issued before the current tile
// is consumed. LDS rows are 256 bytes, with 16-byte chunk c of key k stored
// at chunk slot c ^ (k & 15), which keeps every operand read below free of
// bank conflicts.
//
// Per 32-key sub-tile and 16-query block the wave computes, as in the decode
// kernel but with query columns instead of head/probe columns:
//   scores  Z^T[key, q] = K . Q^T,  S^T[key, q] = K . R^T   (16 MFMAs)
//   readout A^T[d, q] += V^T . P^T, B^T[d, q] += V^T . (P o S')^T (16 MFMAs)
// with the score MFMA's key order permuted so that lane (g, n) receives the
// scores of query n for exactly the keys g + 4t it feeds the readout MFMA
// (P never leaves registers), and V^T built by an in-register 8x8 transpose
// of rows read from LDS. The K and V operands are read once per sub-tile and
// shared by the wave's query blocks and by both score/readout pairs.
//
// Causality: keys j <= i. Sub-tiles entirely above a wave's rows are
// skipped, sub-tiles crossing the diagonal are masked. Work items run
// heaviest-first (last q-tile first), and the group index varies fastest so
// that all q-tiles of one (sequence, KV head) land on one XCD when the
// number of groups is a multiple of 8 (its L2 then holds that head's K/V).
// -------------------------------------------------------------------------
constexpr int kPrefillKeys = 64;  // keys per LDS tile

template <int HPW, int QB, int NW>
__global__ __launch_bounds__(64 * NW) void prefill_mfma_bf16_d128(PrefillArgs a) {
    constexpr int D = 128;
    constexpr int WPH = NW / HPW;       // waves per head
    constexpr int RW = 16 * QB;         // rows per wave
    constexpr int RPH = RW * WPH;       // rows per head per work item
    constexpr int TK = kPrefillKeys;
    constexpr int NT = 64 * NW;         // threads
    constexpr int LOADS = TK * 16 / NT; // 16-byte chunks of K (and of V) per thread per tile
    static_assert(NW % HPW == 0 && LOADS >= 1, "bad workgroup shape");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int g = lane >> 4;

    // ---- work item: heaviest q-tile first, group fastest
    const int G = a.Hq / a.Hkv;
    const int hgroups = G / HPW;                    // head groups per KV head
    const int NG = a.B * a.Hkv * hgroups;           // groups
    const int QT = (a.L + RPH - 1) / RPH;           // q-tiles per group
    const int item = blockIdx.x;
    const int grp = item % NG;
    const int qt = QT - 1 - item / NG;
    const int b = grp / (a.Hkv * hgroups);
    const int hkv = (grp / hgroups) % a.Hkv;
    const int hsub = grp % hgroups;
    const int hq = hkv * G + hsub * HPW + wave / WPH;
    const int q0 = qt * RPH + (wave % WPH) * RW;    // this wave's first row
    const int kend = min(a.L, (qt + 1) * RPH);      // keys the workgroup needs
    const int ntiles = (kend + TK - 1) / TK;

    const uint16_t *qh = reinterpret_cast<const uint16_t *>(a.q);
    const uint16_t *rh = reinterpret_cast<const uint16_t *>(a.r);
    const int64_t kvbase = ((int64_t)b * a.Hkv + hkv) * a.L * D;
    const uint32_t kvbytes = (uint32_t)((int64_t)a.L * D * 2);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(reinterpret_cast<const uint16_t *>(a.k) + kvbase), 0, kvbytes, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(reinterpret_cast<const uint16_t *>(a.v) + kvbase), 0, kvbytes, kBufferFlags);

    // ---- LDS: two K/V tiles
    __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][TK * D];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][TK * D];
    // loader: thread handles chunk tc of keys tk + (NT / 16) * j
    const int tk = threadIdx.x >> 4, tc = threadIdx.x & 15;
    u32x4 stage_k[LOADS], stage_v[LOADS];
    auto global_tile = [&](int tile) {
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int key = tile * TK + tk + (NT / 16) * j;
            const int off = (key * D + tc * 8) * 2;
            stage_k[j] = buffer_load16_cached(krs, off);
            stage_v[j] = buffer_load16_cached(vrs, off);
        }
    };
    auto lds_store = [&](int buf) {
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int key = tk + (NT / 16) * j;
            const int slot = key * D + ((tc ^ (key & 15)) * 8);
            *reinterpret_cast<u32x4 *>(&lds_k[buf][slot]) = stage_k[j];
            *reinterpret_cast<u32x4 *>(&lds_v[buf][slot]) = stage_v[j];
        }
    };
    global_tile(0);

    // ---- per-wave query operands: block qb, k-step u
    bf16x8 qop[QB][4], rop[QB][4];
    float piv[QB];
    {
        const int64_t rowbase = ((int64_t)b * a.Hq + hq) * a.L;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int row = min(q0 + 16 * qb + n, a.L - 1);
            const uint16_t *qp = qh + (rowbase + row) * D;
            const uint16_t *rp = rh + (rowbase + row) * D;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                qop[qb][u] = load16(qp + 8 * (g + 4 * u));
                rop[qb][u] = load16(rp + 8 * (g + 4 * u));
            }
        }
        // pivot: probe score of key 0 for each query row
        const uint16_t *k0 = reinterpret_cast<const uint16_t *>(a.k) + kvbase;
        float part[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) part[qb] = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bf16x8 kk = load16(k0 + 8 * (g + 4 * u));
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int e = 0; e < 8; ++e) part[qb] += (float)rop[qb][u][e] * (float)kk[e];
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) piv[qb] = xor_sum_rowgroups(part[qb]) * a.rk_scale;
    }

    float m_run[QB], lsA[QB], lsS[QB];
    floatx4 accA[QB][8], accB[QB][8];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = -INFINITY;
        lsA[qb] = 0.f;
        lsS[qb] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            accA[qb][e] = floatx4{0.f, 0.f, 0.f, 0.f};
            accB[qb][e] = floatx4{0.f, 0.f, 0.f, 0.f};
        }
    }

    const int kperm = (n >> 2) + 4 * (n & 3);
    const int q_last = q0 + RW - 1;

    // One 32-key sub-tile at key k0 from LDS buffer `buf` (local key offset kl).
    auto subtile = [&](int buf, int kl, int k0, bool diag) {
        // K operand: block kb, k-step u -> key kl + 16kb + kperm, chunk g + 4u
        bf16x8 kop[2][4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int key = kl + 16 * kb + kperm;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int slot = key * D + (((g + 4 * u) ^ (key & 15)) * 8);
                kop[kb][u] = *reinterpret_cast<const bf16x8 *>(&lds_k[buf][slot]);
            }
        }
        // V^T operand: rows key kl + g + 4t, chunk n, transposed in registers
        bf16x8 vT[8];
        {
            bf16x8 vrow[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int key = kl + g + 4 * t;
                const int slot = key * D + ((n ^ (key & 15)) * 8);
                vrow[t] = *reinterpret_cast<const bf16x8 *>(&lds_v[buf][slot]);
            }
#pragma unroll
            for (int d2 = 0; d2 < 4; ++d2) {
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t x = __builtin_bit_cast(uint4, vrow[2 * j])[d2];
                    const uint32_t y = __builtin_bit_cast(uint4, vrow[2 * j + 1])[d2];
                    lo[j] = __builtin_amdgcn_perm(y, x, 0x05040100u);
                    hi[j] = __builtin_amdgcn_perm(y, x, 0x07060302u);
                }
                vT[2 * d2] = __builtin_bit_cast(bf16x8, uint4{lo[0], lo[1], lo[2], lo[3]});
                vT[2 * d2 + 1] = __builtin_bit_cast(bf16x8, uint4{hi[0], hi[1], hi[2], hi[3]});
            }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            floatx4 z0 = {0.f, 0.f, 0.f, 0.f}, z1 = z0, s0 = z0, s1 = z0;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                z0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[0][u], qop[qb][u], z0, 0, 0, 0);
                z1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[1][u], qop[qb][u], z1, 0, 0, 0);
                s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[0][u], rop[qb][u], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[1][u], rop[qb][u], s1, 0, 0, 0);
            }
            float zr[8], sr[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                zr[i] = z0[i];
                zr[4 + i] = z1[i];
                sr[i] = s0[i];
                sr[4 + i] = s1[i];
            }
            const int row = q0 + 16 * qb + n;
            float rmax = -INFINITY;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                if (diag && k0 + g + 4 * t > row) zr[t] = -INFINITY;
                rmax = fmaxf(rmax, zr[t]);
            }
            const float tmax = xor_max_rowgroups(rmax) * a.zscale;
            const bool raise = tmax > m_run[qb] + kRescaleSlack;
            if (__builtin_amdgcn_ballot_w64(raise) != 0) {
                const float m_new = fmaxf(m_run[qb], tmax);
                const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
                m_run[qb] = m_new;
                lsA[qb] *= alpha;
                lsS[qb] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    accA[qb][e] *= alpha;
                    accB[qb][e] *= alpha;
                }
            }
            const float neg_m = -m_run[qb];
            bf16x8 pa, ps;
            float suma = 0.f, sums = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float p = __builtin_amdgcn_exp2f(fmaf(zr[t], a.zscale, neg_m));
                const float q = p * fmaf(sr[t], a.rk_scale, -piv[qb]);
                suma += p;
                sums += q;
                pa[t] = (__bf16)p;
                ps[t] = (__bf16)q;
            }
            lsA[qb] += suma;
            lsS[qb] += sums;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                accA[qb][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vT[e], pa, accA[qb][e], 0, 0, 0);
                accB[qb][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vT[e], ps, accB[qb][e], 0, 0, 0);
            }
        }
    };

    // One 64-key tile from LDS buffer BUF (compile-time, so every LDS
    // address is a per-lane constant plus an immediate offset).
    auto tile_step = [&](auto bufc, int tile) {
        constexpr int BUF = decltype(bufc)::value;
        if (tile + 1 < ntiles) global_tile(tile + 1);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int k0 = tile * TK + 32 * half;
            if (k0 <= q_last) {  // wave-uniform: sub-tiles above the wave's rows are skipped
                if (k0 + 31 <= q0)
                    subtile(BUF, 32 * half, k0, false);
                else
                    subtile(BUF, 32 * half, k0, true);
            }
        }
        if (tile + 1 < ntiles) lds_store(BUF ^ 1);
        __syncthreads();
    };

    lds_store(0);
    __syncthreads();
    for (int tile = 0; tile < ntiles; tile += 2) {
        tile_step(std::integral_constant<int, 0>{}, tile);
        if (tile + 1 < ntiles) tile_step(std::integral_constant<int, 1>{}, tile + 1);
    }

    // ---- epilogue: o = (A + B - (S / l) A) / l per row
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = xor_sum_rowgroups(lsA[qb]);
        const float S = xor_sum_rowgroups(lsS[qb]);
        const int row = q0 + 16 * qb + n;
        if (row >= a.L) continue;
        const float inv_l = 1.0f / l;
        const float cA = 1.0f - S * inv_l;
        const int64_t ro = ((int64_t)b * a.Hq + hq) * a.L + row;
        uint16_t *o = reinterpret_cast<uint16_t *>(a.o) + ro * D + 32 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float ov[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) ov[e] = (accA[qb][e][i] * cA + accB[qb][e][i]) * inv_l;
            *reinterpret_cast<uint4 *>(o + 8 * i) =
                uint4{pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3]), pack_bf16x2(ov[4], ov[5]),
                      pack_bf16x2(ov[6], ov[7])};
        }
        if (g == 0) {
            if (a.lse) a.lse[ro] = m_run[qb] * 0.6931471805599453f + logf(l);
            if (a.sbar) a.sbar[ro] = S * inv_l + piv[qb];
        }
    }
}

}  // namespace

bool prefill_supported(int D, int dtype) { return (D == 64 || D == 128) && (dtype == 0 || dtype == 1); }

// Workgroup shape of the MFMA prefill: QB query blocks of 16 rows per wave,
// NW waves; selectable for measurement through PARALLAX_PREFILL_SHAPE
// ("QB,NW"), default below.
static int prefill_shape_qb = 0, prefill_shape_nw = 0;

hipError_t launch_prefill(const PrefillArgs &a, int dtype, hipStream_t stream) {
    const int G = a.Hq / a.Hkv;
    if (prefill_shape_qb == 0) {
        prefill_shape_qb = 1;
        prefill_shape_nw = 8;
        if (const char *env = getenv("PARALLAX_PREFILL_SHAPE")) {
            int qb = 0, nw = 0;
            if (sscanf(env, "%d,%d", &qb, &nw) == 2 && ((qb == 2 && nw == 4) || (qb == 1 && nw == 8))) {
                prefill_shape_qb = qb;
                prefill_shape_nw = nw;
            }
        }
    }
    if (dtype == 1 && a.D == 128 && (G % 2 == 0 || G == 1)) {
        const int hpw = (G % 2 == 0) ? 2 : 1;
        const int rph = 16 * prefill_shape_qb * prefill_shape_nw / hpw;
        const long items = (long)a.B * a.Hkv * (G / hpw) * ((a.L + rph - 1) / rph);
        if (items <= 0x7fffffffL) {
            dim3 grid((unsigned)items);
            const bool wide = prefill_shape_qb == 2;
            if (hpw == 2) {
                if (wide)
                    hipLaunchKernelGGL((prefill_mfma_bf16_d128<2, 2, 4>), grid, dim3(256), 0, stream, a);
                else
                    hipLaunchKernelGGL((prefill_mfma_bf16_d128<2, 1, 8>), grid, dim3(512), 0, stream, a);
            } else {
                if (wide)
                    hipLaunchKernelGGL((prefill_mfma_bf16_d128<1, 2, 4>), grid, dim3(256), 0, stream, a);
                else
                    hipLaunchKernelGGL((prefill_mfma_bf16_d128<1, 1, 8>), grid, dim3(512), 0, stream, a);
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
