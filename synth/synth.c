/*
 * Seeded synthetic inputs for the Parallax attention tests and benchmark.
 *
 * This module holds no attention arithmetic: it only draws numbers. It is the
 * one piece of code that both the CPU oracle side and the GPU side of the
 * tests consume, so that both see bit-identical inputs.
 *
 * Generator (counter-based, so any slice can be regenerated on its own):
 *   stream key  K(seed, tid) = mix64(seed + G * (tid + 1))
 *   pair word   U(p)         = mix64(K + G * (p + 1))        -- SplitMix64 output p
 *   uniforms    u1 = (hi32(U) + 0.5) / 2^32,  u2 = (lo32(U) + 0.5) / 2^32
 *   normals     x[2p]   = sqrt(-2 ln u1) * cos(2 pi u2)       -- Box & Muller (1958)
 *               x[2p+1] = sqrt(-2 ln u1) * sin(2 pi u2)
 * where G = 0x9E3779B97F4A7C15 and mix64 is Stafford's "Mix13" finaliser
 * used by SplitMix64 (Steele, Lea, Flood 2014). Each normal is scaled in
 * double and rounded once, to nearest-even, to fp32 or bf16.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z)
{
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t tid)
{
    return mix64(seed + GOLDEN * (tid + 1ULL));
}

uint64_t synth_word(uint64_t seed, uint64_t tid, uint64_t p)
{
    return mix64(stream_key(seed, tid) + GOLDEN * (p + 1ULL));
}

static inline void pair_normals(uint64_t key, uint64_t p, double *n0, double *n1)
{
    uint64_t u = mix64(key + GOLDEN * (p + 1ULL));
    double u1 = ((double)(u >> 32) + 0.5) * (1.0 / 4294967296.0);
    double u2 = ((double)(u & 0xffffffffULL) + 0.5) * (1.0 / 4294967296.0);
    double rad = sqrt(-2.0 * log(u1));
    double th = 6.283185307179586476925286766559 * u2;
    *n0 = rad * cos(th);
    *n1 = rad * sin(th);
}

/* Round a double once, to nearest-even, to bfloat16 bits. */
uint16_t synth_bf16_from_double(double x)
{
    uint64_t bits;
    memcpy(&bits, &x, 8);
    uint16_t sign = (uint16_t)((bits >> 48) & 0x8000u);
    double a = fabs(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7fc0u);
    if (a < 0x1p-126) {
        /* bf16 subnormal range: quantum 2^-133; scaling by 2^133 is exact */
        double m = nearbyint(a * 0x1p133); /* default mode: nearest-even */
        return (uint16_t)(sign | (uint16_t)m); /* m == 128 is the smallest normal */
    }
    uint64_t ab = bits & 0x7fffffffffffffffULL;
    int e = (int)(ab >> 52) - 1023;          /* unbiased exponent */
    uint64_t man = ab & ((1ULL << 52) - 1);
    uint64_t keep = man >> 45;               /* 7 stored mantissa bits */
    uint64_t rem = man & ((1ULL << 45) - 1);
    uint64_t half = 1ULL << 44;
    uint32_t out = ((uint32_t)(e + 127) << 7) | (uint32_t)keep;
    if (rem > half || (rem == half && (keep & 1u)))
        out += 1; /* a carry into the exponent is the correct result */
    if (out >= 0x7f80u)
        out = 0x7f80u; /* overflow to infinity */
    return (uint16_t)(sign | out);
}

/*
 * Fill out[0..count) with elements first .. first+count-1 of the stream
 * (seed, tid), each N(0,1) * scale, rounded to fp32 (dtype 0) or bf16 (1).
 */
void synth_normal(uint64_t seed, uint64_t tid, uint64_t first, uint64_t count,
                  double scale, int dtype, void *out)
{
    uint64_t key = stream_key(seed, tid);
    if (count == 0)
        return;
    uint64_t p0 = first >> 1;
    uint64_t p1 = (first + count - 1) >> 1;
    int64_t np = (int64_t)(p1 - p0 + 1);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < np; ++t) {
        uint64_t p = p0 + (uint64_t)t;
        double n[2];
        pair_normals(key, p, &n[0], &n[1]);
        for (int h = 0; h < 2; ++h) {
            uint64_t idx = 2 * p + (uint64_t)h;
            if (idx < first || idx >= first + count)
                continue;
            uint64_t o = idx - first;
            double val = n[h] * scale;
            if (dtype == 0)
                ((float *)out)[o] = (float)val;
            else
                ((uint16_t *)out)[o] = synth_bf16_from_double(val);
        }
    }
}

/* Integer draws lo + (word mod (hi - lo + 1)), element i of stream (seed, tid). */
void synth_uniform_int(uint64_t seed, uint64_t tid, uint64_t count, int64_t lo, int64_t hi,
                       int64_t *out)
{
    uint64_t key = stream_key(seed, tid);
    uint64_t span = (uint64_t)(hi - lo) + 1ULL;
    for (uint64_t i = 0; i < count; ++i)
        out[i] = lo + (int64_t)(mix64(key + GOLDEN * (i + 1ULL)) % span);
}
