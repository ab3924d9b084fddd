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
// prefill_generic<T, D>: any dtype / head_dim; one wave per query row,
// the streaming state of the decode kernels (pivot = probe score of key 0).
#include "plx_internal.h"

namespace plx {

namespace {

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

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

}  // namespace

bool prefill_supported(int D, int dtype) { return (D == 64 || D == 128) && (dtype == 0 || dtype == 1); }

hipError_t launch_prefill(const PrefillArgs &a, int dtype, hipStream_t stream) {
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
