// C ABI of the Parallax library: argument checks, the decode split plan,
// and the launches. See include/parallax.h for the contract of every entry
// point. Argument checks are host-only and run before any launch.
#include "../../include/parallax.h"
#include "plx_internal.h"

#include <math.h>

#include <mutex>

namespace plx {

namespace {

int g_cu_count[64];  // per-device compute-unit count, filled on first use

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (g_cu_count[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        g_cu_count[dev] = n;
    }
    return g_cu_count[dev];
}

}  // namespace

// Decode plan. The MFMA path (bf16, head_dim 128, any group size; groups of
// more than 8 query heads in chunks of 8) runs one four-wave workgroup per
// (KV head, chunk, split, sequence) over a multiple of
// 128 keys; the generic path one wave per (query head, split, sequence) over
// a multiple of 32 keys. Without a forced count, the sequence is cut into
// enough splits for about kTargetWavesPerCU resident waves per compute unit,
// with at least kMinKeysPerWave keys per wave; one split fuses the final
// normalisation into the streaming kernel and needs no workspace.
constexpr int kTargetWavesPerCU = 4;
constexpr int kMinKeysPerWave = 32;  // one tile: short sequences split for latency
// On the MFMA path a sequence of at most this many visible keys (four tiles
// per wave) runs as one fused split: a second, dependent merge launch costs
// more than the parallelism buys (B = 1, 8 KV heads: 256 keys 5.2 us fused
// against 7.7 us split, 512 keys 6.4 against 8.0; from 1024 keys the split
// plan is faster, 7.8 against 8.6).
constexpr int kFusedMaxKeys = 512;
// Most keys one split (or stream-K range) may hold: its keys, plus the keys
// its streaming loop reads ahead (up to two 128-key strides and one 32-key
// tile past its end), must span less than 2^31 bytes, since the kernels
// address them with 32-bit offsets.
// A range is also at most kMaxRangeKeys keys, whose block-sparse visibility a
// workgroup stages in LDS.
static long long max_split_keys(int Hkv, int D, int dtype) {
    const long long tok_bytes = (long long)Hkv * D * (dtype == PLX_BF16 ? 2 : 4);
    const long long by_offsets = (0x7fffffffLL - 1024) / tok_bytes - 320;
    return by_offsets < kMaxRangeKeys ? by_offsets : kMaxRangeKeys;
}

DecodePlan plan_decode(int B, int Hq, int Hkv, int D, int kv_len, int window, int dtype,
                       int num_splits) {
    DecodePlan p;
    if (window > 0 && window < kv_len) kv_len = window;  // keys a query can see at most
    const int G = Hq / Hkv;
    // matrix cores for bf16 at D = 128: 2G MFMA columns <= 16, so larger groups run in
    // chunks of 8 query heads, one workgroup per (KV head, chunk)
    const bool mfma = dtype == PLX_BF16 && D == 128;
    p.path = mfma ? DecodePath::Mfma : DecodePath::Generic;
    const int waves = mfma ? 4 : 1;      // waves per workgroup
    const int quantum = 32 * waves;      // keys per split are a multiple of this
    const long units = (long)B * (mfma ? (long)Hkv * ((G + 7) / 8) : Hq);
    const int max_splits = (kv_len + quantum - 1) / quantum;
    int splits = num_splits;
    if (splits <= 0) {
        const long target = (long)kTargetWavesPerCU * device_cu_count() / waves;
        long s = (target + units - 1) / units;
        const long by_len = (kv_len + (long)kMinKeysPerWave * waves - 1) / ((long)kMinKeysPerWave * waves);
        if (s > by_len) s = by_len;
        if (s < 1 || (mfma && kv_len <= kFusedMaxKeys)) s = 1;
        splits = (int)s;
    }
    if (splits > max_splits) splits = max_splits;
    const long long max_keys = max_split_keys(Hkv, D, dtype);
    const long long min_splits = (kv_len + max_keys - 1) / max_keys;
    if (splits < min_splits) splits = (int)min_splits;
    if (splits > 65535) splits = 65535;  // grid.y limit
    if (splits < 1) splits = 1;
    int chunk = (kv_len + splits - 1) / splits;
    chunk = (chunk + quantum - 1) / quantum * quantum;
    splits = (kv_len + chunk - 1) / chunk;
    p.splits = splits;
    p.chunk = chunk;
    p.ws_bytes = splits > 1 ? (size_t)B * Hq * splits * partial_floats(D) * sizeof(float) : 0;
    return p;
}

}  // namespace plx

using plx::DecodePlan;

// Longest prefill sequence: the kernels address one head's [L, D] tensor
// with 32-bit byte offsets.
constexpr int kMaxPrefillLen = 1 << 22;

static int check_decode_sizes(int B, int Hq, int Hkv, int D, int kv_len, int window, int dtype) {
    if (B < 1 || Hq < 1 || Hkv < 1 || kv_len < 1 || window < 0) return PLX_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return PLX_ERR_INVALID_ARG;
    if (B > 65535 || Hq > 65535) return PLX_ERR_UNSUPPORTED;
    if (dtype != PLX_F32 && dtype != PLX_BF16) return PLX_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return PLX_ERR_UNSUPPORTED;
    return PLX_OK;
}

static inline plx_status as_status(int s) { return static_cast<plx_status>(s); }

extern "C" {

int parallax_abi_version(void) { return PARALLAX_ABI_VERSION; }

const char *parallax_status_string(int status) {
    switch (status) {
        case PLX_OK: return "ok";
        case PLX_ERR_INVALID_ARG: return "invalid argument";
        case PLX_ERR_UNSUPPORTED: return "unsupported configuration";
        case PLX_ERR_WORKSPACE: return "workspace missing or too small";
        case PLX_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

// Packed caches with an automatic plan and no window run the stream-K kernel:
// each KV head's tokens in equal ranges, one workgroup per range and four
// workgroups per CU in all (measured side by side on the 64-sequence
// mixed-length batch: 1 per CU 214-216 us, 2 per CU 205-209 us, 3 per CU
// 212 us, 4 per CU 203-206 us, 6 per CU 209 us, 8 per CU 215 us). Returns
// the range count per KV head, or 0 where it does not apply (the
// per-sequence split plan then runs).
static int streamk_parts(const DecodePlan &p, int B, int Hq, int Hkv, int D, int kv_len, int dtype,
                         int window, int num_splits) {
    if (p.path != plx::DecodePath::Mfma || window != 0 || num_splits != 0 || Hq / Hkv > 8) return 0;
    int parts = 4 * plx::device_cu_count() / Hkv;
    parts = parts < 1 ? 1 : (parts > 65535 ? 65535 : parts);
    // the cache holds at most B * kv_len tokens; a range must fit 32-bit offsets
    const long long range = ((long long)B * kv_len + parts - 1) / parts;
    return range <= plx::max_split_keys(Hkv, D, dtype) ? parts : 0;
}
static size_t streamk_bytes(int B, int Hq, int D, int parts) {
    return (size_t)Hq * ((size_t)parts + B - 1) * plx::partial_floats(D) * sizeof(float);
}

size_t parallax_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int kv_len, int window,
                                       plx_dtype dtype, int num_splits) {
    if (check_decode_sizes(B, Hq, Hkv, D, kv_len, window, dtype) != PLX_OK) return 0;
    const DecodePlan p = plx::plan_decode(B, Hq, Hkv, D, kv_len, window, dtype, num_splits);
    // the same size must also cover a packed cache's stream-K plan
    const int parts = streamk_parts(p, B, Hq, Hkv, D, kv_len, dtype, window, num_splits);
    const size_t sk = parts ? streamk_bytes(B, Hq, D, parts) : 0;
    return p.ws_bytes > sk ? p.ws_bytes : sk;
}

int parallax_decode_num_splits(int B, int Hq, int Hkv, int D, int kv_len, int window, plx_dtype dtype,
                               int num_splits) {
    if (check_decode_sizes(B, Hq, Hkv, D, kv_len, window, dtype) != PLX_OK) return 0;
    return plx::plan_decode(B, Hq, Hkv, D, kv_len, window, dtype, num_splits).splits;
}

static int fill_decode_args(plx::DecodeArgs &a, const void *q, const void *r, const void *k,
                            const void *v, void *o, const int32_t *cu, int B, int Hq, int Hkv, int D,
                            int kv_len, int window, const uint8_t *block_mask, float qk_scale,
                            float rk_scale, int dtype, int num_splits, bool parallax,
                            DecodePlan &p) {
    int st = check_decode_sizes(B, Hq, Hkv, D, kv_len, window, dtype);
    if (st != PLX_OK) return st;
    if (!q || !k || !v || !o || (parallax && !r)) return PLX_ERR_INVALID_ARG;
    if (num_splits < 0) return PLX_ERR_INVALID_ARG;
    // masked logits are -inf before scaling, so the scale must be positive
    if (!isfinite(qk_scale) || !(qk_scale > 0.f) || !isfinite(rk_scale)) return PLX_ERR_INVALID_ARG;
    p = plx::plan_decode(B, Hq, Hkv, D, kv_len, window, dtype, num_splits);
    a.q = q;
    a.r = r;
    a.k = k;
    a.v = v;
    a.o = o;
    a.cu = cu;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.D = D;
    a.kv_len = kv_len;
    a.window = window;
    a.block_mask = block_mask;
    a.mask_cols = (kv_len + plx::kMaskBlock - 1) / plx::kMaskBlock;
    a.zscale = qk_scale * plx::kLog2e;
    a.rk_scale = rk_scale;
    a.splits = p.splits;
    a.chunk = p.chunk;
    a.sk_parts = 0;
    a.ws = nullptr;
    a.fused = p.splits == 1;
    return PLX_OK;
}

static int decode_common(const void *q, const void *r, const void *k, const void *v, void *o,
                         const int32_t *cu, int B, int Hq, int Hkv, int D, int kv_len, int window,
                         const uint8_t *block_mask, float qk_scale, float rk_scale, int dtype,
                         int num_splits, void *ws, size_t ws_bytes, void *stream, bool parallax) {
    plx::DecodeArgs a;
    DecodePlan p;
    int st = fill_decode_args(a, q, r, k, v, o, cu, B, Hq, Hkv, D, kv_len, window, block_mask,
                              qk_scale, rk_scale, dtype, num_splits, parallax, p);
    if (st != PLX_OK) return st;
    if (cu) {
        a.sk_parts = streamk_parts(p, B, Hq, Hkv, D, kv_len, dtype, window, num_splits);
        if (a.sk_parts) {
            a.fused = false;
            p.ws_bytes = streamk_bytes(B, Hq, D, a.sk_parts);
        }
    }
    if (p.ws_bytes > 0 && (!ws || ws_bytes < p.ws_bytes)) return PLX_ERR_WORKSPACE;
    a.ws = reinterpret_cast<float *>(ws);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t err = plx::launch_decode_split(a, p.path, dtype, parallax, s);
    if (err == hipSuccess && !a.fused) err = plx::launch_decode_merge(a, dtype, parallax, s);
    return err == hipSuccess ? PLX_OK : PLX_ERR_HIP;
}

plx_status parallax_decode(const void *q, const void *r, const void *k, const void *v, void *o,
                    const int32_t *cu_seqlens_k, int B, int Hq, int Hkv, int D, int kv_len,
                    int window, const uint8_t *block_mask, float qk_scale, float rk_scale,
                    plx_dtype dtype, int num_splits, void *workspace, size_t workspace_bytes,
                    void *stream) {
    return as_status(decode_common(q, r, k, v, o, cu_seqlens_k, B, Hq, Hkv, D, kv_len, window, block_mask,
                         qk_scale, rk_scale, dtype, num_splits, workspace, workspace_bytes, stream,
                         true));
}

plx_status softmax_decode(const void *q, const void *k, const void *v, void *o, const int32_t *cu_seqlens_k,
                   int B, int Hq, int Hkv, int D, int kv_len, int window,
                   const uint8_t *block_mask, float qk_scale, plx_dtype dtype, int num_splits,
                   void *workspace, size_t workspace_bytes, void *stream) {
    return as_status(decode_common(q, nullptr, k, v, o, cu_seqlens_k, B, Hq, Hkv, D, kv_len, window,
                         block_mask, qk_scale, 1.0f, dtype, num_splits, workspace, workspace_bytes,
                         stream, false));
}

}  // extern "C"

// ---- decode with the library's own device workspace ---------------------
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops): the split records of parallax_decode_noalloc live in
// this file-scope device array. Each device that runs the call holds its own
// copy until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that
// address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[PLX_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// The current device's copy of `scratch` (looked up on its first use).
int current_scratch(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PLX_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return PLX_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PLX_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PLX_OK;
}
}  // namespace

extern "C" {

plx_status parallax_decode_noalloc(const void *q, const void *r, const void *k, const void *v, void *o,
                            const int32_t *cu_seqlens_k, int B, int Hq, int Hkv, int D,
                            int kv_len, int window, const uint8_t *block_mask, float qk_scale,
                            float rk_scale, plx_dtype dtype, int num_splits, void *stream) {
    // host-only checks first: invalid arguments, and a plan whose records
    // exceed the static workspace, are refused before anything touches the device
    plx::DecodeArgs a;
    DecodePlan p;
    int st = fill_decode_args(a, q, r, k, v, o, cu_seqlens_k, B, Hq, Hkv, D, kv_len, window,
                              block_mask, qk_scale, rk_scale, dtype, num_splits, true, p);
    if (st != PLX_OK) return as_status(st);
    // the records of the plan this call runs: the per-sequence splits, or a packed
    // cache's stream-K ranges (parallax_decode_workspace_bytes bounds both)
    size_t need = p.ws_bytes;
    if (cu_seqlens_k) {
        const int parts = streamk_parts(p, B, Hq, Hkv, D, kv_len, dtype, window, num_splits);
        if (parts) need = streamk_bytes(B, Hq, D, parts);
    }
    if (need > PLX_NOALLOC_SCRATCH_BYTES) return as_status(PLX_ERR_WORKSPACE);
    void *ws = nullptr;
    st = current_scratch(&ws);
    if (st != PLX_OK) return as_status(st);
    // no kernel of the decode path needs its workspace cleared: every record
    // the merge reads is written by the streaming kernel of the same call
    return as_status(decode_common(q, r, k, v, o, cu_seqlens_k, B, Hq, Hkv, D, kv_len, window, block_mask,
                         qk_scale, rk_scale, dtype, num_splits, ws, PLX_NOALLOC_SCRATCH_BYTES,
                         stream, true));
}

size_t parallax_decode_record_bytes(int B, int Hq, int D, int num_records) {
    if (B < 1 || Hq < 1 || num_records < 1 || (D != 64 && D != 128)) return 0;
    return (size_t)B * Hq * num_records * plx::partial_floats(D) * sizeof(float);
}

plx_status parallax_decode_partial(const void *q, const void *r, const void *k, const void *v,
                            const int32_t *cu_seqlens_k, int B, int Hq, int Hkv, int D, int kv_len,
                            int window, const uint8_t *block_mask, float qk_scale, float rk_scale,
                            plx_dtype dtype, int num_splits, void *records, size_t records_bytes,
                            void *stream) {
    plx::DecodeArgs a;
    DecodePlan p;
    const bool parallax = r != nullptr;
    // o is not written in this mode; any non-null value passes the checks
    int st = fill_decode_args(a, q, r, k, v, records, cu_seqlens_k, B, Hq, Hkv, D, kv_len, window,
                              block_mask, qk_scale, rk_scale, dtype, num_splits, parallax, p);
    if (st != PLX_OK) return as_status(st);
    if (!records || records_bytes < parallax_decode_record_bytes(B, Hq, D, p.splits))
        return as_status(PLX_ERR_WORKSPACE);
    a.o = nullptr;
    a.ws = reinterpret_cast<float *>(records);
    a.fused = false;
    hipError_t err = plx::launch_decode_split(a, p.path, dtype, parallax, reinterpret_cast<hipStream_t>(stream));
    return as_status(err == hipSuccess ? PLX_OK : PLX_ERR_HIP);
}

plx_status parallax_decode_merge(const void *records, void *o, int B, int Hq, int D, int num_records, plx_dtype dtype,
                          int with_probe, void *stream) {
    if (B < 1 || Hq < 1 || num_records < 1 || !records || !o) return as_status(PLX_ERR_INVALID_ARG);
    if (B > 65535 || Hq > 65535) return as_status(PLX_ERR_UNSUPPORTED);
    if (D != 64 && D != 128) return as_status(PLX_ERR_UNSUPPORTED);
    if (dtype != PLX_F32 && dtype != PLX_BF16) return as_status(PLX_ERR_UNSUPPORTED);
    plx::DecodeArgs a = {};
    a.o = o;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hq;
    a.D = D;
    a.splits = num_records;
    a.ws = const_cast<float *>(reinterpret_cast<const float *>(records));
    hipError_t err = plx::launch_decode_merge(a, dtype, with_probe != 0, reinterpret_cast<hipStream_t>(stream));
    return as_status(err == hipSuccess ? PLX_OK : PLX_ERR_HIP);
}

}  // extern "C"

// Checks shared by the prefill entry points (dense when cu == nullptr,
// packed with `total` tokens otherwise); fills the sizes of `a`.
// Packed batches run persistent workgroups fed from per-XCD queues: the
// workspace starts with their counters (16 ints used, 256 bytes reserved).
constexpr size_t kQueueBytes = 256;

template <typename Args>
static int check_prefill(Args &a, const int32_t *cu, int B, int Hq, int Hkv, int L, int total, int D,
                         int window, const uint8_t *block_mask, float qk_scale, float rk_scale,
                         int dtype) {
    if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || D < 1 || window < 0) return PLX_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return PLX_ERR_INVALID_ARG;
    if (cu && total < 0) return PLX_ERR_INVALID_ARG;
    // masked logits are -inf before scaling, so the scale must be positive
    if (!isfinite(qk_scale) || !(qk_scale > 0.f) || !isfinite(rk_scale)) return PLX_ERR_INVALID_ARG;
    if (dtype != PLX_F32 && dtype != PLX_BF16) return PLX_ERR_UNSUPPORTED;
    if (!plx::prefill_supported(D, dtype)) return PLX_ERR_UNSUPPORTED;
    if (B > 65535 || Hq > 65535 || L > kMaxPrefillLen) return PLX_ERR_UNSUPPORTED;
    // one head of one sequence is addressed with 32-bit byte offsets
    const long long row_bytes = (long long)(cu ? (Hq > Hkv ? Hq : Hkv) : 1) * D * (dtype == PLX_BF16 ? 2 : 4);
    if ((long long)L * row_bytes >= 0x7fffffffLL) return PLX_ERR_UNSUPPORTED;
    a.cu = cu;
    a.sched = nullptr;
    a.workers = plx::device_cu_count();  // one workgroup per CU fits the LDS of each kernel
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.L = L;
    a.D = D;
    a.window = (window > 0 && window < L) ? window : L;
    a.block_mask = block_mask;
    a.zscale = qk_scale * plx::kLog2e;
    a.rk_scale = rk_scale;
    return PLX_OK;
}

static int prefill_common(const void *q, const void *r, const void *k, const void *v, void *o, float *lse,
                          float *sbar, void *vbar, const int32_t *cu, int B, int Hq, int Hkv, int L, int total, int D,
                          int window, const uint8_t *block_mask, float qk_scale, float rk_scale,
                          int dtype, void *ws, size_t ws_bytes, void *stream) {
    if (!q || !r || !k || !v || !o) return PLX_ERR_INVALID_ARG;
    plx::PrefillArgs a;
    int st = check_prefill(a, cu, B, Hq, Hkv, L, total, D, window, block_mask, qk_scale, rk_scale,
                           dtype);
    if (st != PLX_OK) return st;
    if (cu && (!ws || ws_bytes < kQueueBytes)) return PLX_ERR_WORKSPACE;
    if (cu && total == 0) return PLX_OK;  // every sequence empty
    if (cu) a.sched = reinterpret_cast<int *>(ws);
    a.q = q;
    a.r = r;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.sbar = sbar;
    a.vbar = vbar;
    hipError_t err = plx::launch_prefill(a, dtype, reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? PLX_OK : PLX_ERR_HIP;
}

static int backward_common(const void *q, const void *r, const void *k, const void *v, const void *o,
                           const void *d_o, const float *lse, const float *sbar, const void *vbar,
                           const int32_t *cu,
                           void *dq, void *dr, void *dk, void *dv, int B, int Hq, int Hkv, int L,
                           int total, int D, int window, const uint8_t *block_mask, float qk_scale,
                           float rk_scale, int dtype, void *workspace, size_t workspace_bytes,
                           void *stream) {
    if (!q || !r || !k || !v || !o || !d_o || !lse || !sbar || !dq || !dr || !dk || !dv)
        return PLX_ERR_INVALID_ARG;
    plx::BackwardArgs a;
    int st = check_prefill(a, cu, B, Hq, Hkv, L, total, D, window, block_mask, qk_scale, rk_scale,
                           dtype);
    if (st != PLX_OK) return st;
    if (cu && total == 0) return PLX_OK;  // every sequence empty
    const size_t need = cu ? kQueueBytes + (size_t)Hq * total * sizeof(plx::RowStat)
                           : (size_t)B * Hq * L * sizeof(plx::RowStat);
    if (!workspace || workspace_bytes < need) return PLX_ERR_WORKSPACE;
    if (cu) {
        a.sched = reinterpret_cast<int *>(workspace);
        workspace = reinterpret_cast<char *>(workspace) + kQueueBytes;
    }
    a.q = q;
    a.r = r;
    a.k = k;
    a.v = v;
    a.o = o;
    a.go = d_o;
    a.lse = lse;
    a.sbar = sbar;
    a.vbar = vbar;
    a.dq = dq;
    a.dr = dr;
    a.dk = dk;
    a.dv = dv;
    a.rowstat = reinterpret_cast<plx::RowStat *>(workspace);
    a.total = cu ? total : 0;
    a.qk_scale = qk_scale;
    hipError_t err = plx::launch_prefill_backward(a, dtype, reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? PLX_OK : PLX_ERR_HIP;
}

extern "C" {

plx_status parallax_prefill(const void *q, const void *r, const void *k, const void *v, void *o, float *lse,
                     float *sbar, void *vbar, int B, int Hq, int Hkv, int L, int D, int window,
                     const uint8_t *block_mask, float qk_scale, float rk_scale, plx_dtype dtype,
                     void *stream) {
    return as_status(prefill_common(q, r, k, v, o, lse, sbar, vbar, nullptr, B, Hq, Hkv, L, 0, D, window,
                          block_mask, qk_scale, rk_scale, dtype, nullptr, 0, stream));
}

size_t parallax_prefill_varlen_workspace_bytes(int Hq, int total_tokens, int backward) {
    if (Hq < 1 || total_tokens < 0) return 0;
    return kQueueBytes + (backward ? (size_t)Hq * total_tokens * sizeof(plx::RowStat) : 0);
}

plx_status parallax_prefill_varlen(const void *q, const void *r, const void *k, const void *v, void *o,
                            float *lse, float *sbar, void *vbar, const int32_t *cu_seqlens, int B, int Hq, int Hkv,
                            int max_len, int total_tokens, int D, int window,
                            const uint8_t *block_mask, float qk_scale, float rk_scale, plx_dtype dtype,
                            void *workspace, size_t workspace_bytes, void *stream) {
    if (!cu_seqlens) return as_status(PLX_ERR_INVALID_ARG);
    return as_status(prefill_common(q, r, k, v, o, lse, sbar, vbar, cu_seqlens, B, Hq, Hkv, max_len, total_tokens, D,
                          window, block_mask, qk_scale, rk_scale, dtype, workspace, workspace_bytes,
                          stream));
}

size_t parallax_prefill_backward_workspace_bytes(int B, int Hq, int L) {
    if (B < 1 || Hq < 1 || L < 1) return 0;
    return (size_t)B * Hq * L * sizeof(plx::RowStat);
}

plx_status parallax_prefill_backward(const void *q, const void *r, const void *k, const void *v, const void *o,
                              const void *d_o, const float *lse, const float *sbar, const void *vbar,
                              void *dq, void *dr,
                              void *dk, void *dv, int B, int Hq, int Hkv, int L, int D, int window,
                              const uint8_t *block_mask, float qk_scale, float rk_scale, plx_dtype dtype,
                              void *workspace, size_t workspace_bytes, void *stream) {
    return as_status(backward_common(q, r, k, v, o, d_o, lse, sbar, vbar, nullptr, dq, dr, dk, dv, B, Hq, Hkv, L, 0, D,
                           window, block_mask, qk_scale, rk_scale, dtype, workspace,
                           workspace_bytes, stream));
}

plx_status parallax_prefill_varlen_backward(const void *q, const void *r, const void *k, const void *v,
                                     const void *o, const void *d_o, const float *lse, const float *sbar,
                                     const void *vbar, const int32_t *cu_seqlens, void *dq, void *dr, void *dk, void *dv,
                                     int B, int Hq, int Hkv, int max_len, int total_tokens, int D,
                                     int window, const uint8_t *block_mask, float qk_scale,
                                     float rk_scale, plx_dtype dtype, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    if (!cu_seqlens) return as_status(PLX_ERR_INVALID_ARG);
    return as_status(backward_common(q, r, k, v, o, d_o, lse, sbar, vbar, cu_seqlens, dq, dr, dk, dv, B, Hq, Hkv, max_len,
                           total_tokens, D, window, block_mask, qk_scale, rk_scale, dtype,
                           workspace, workspace_bytes, stream));
}

}  // extern "C"
