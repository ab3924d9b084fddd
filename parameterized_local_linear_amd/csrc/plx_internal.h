// Internal declarations shared by the HIP translation units of the Parallax
// library (kernels, launchers, the C ABI). Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace plx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

// Block-sparse masks: positions are cut into blocks of kMaskBlock from the
// start of each sequence; one byte per (sequence, KV head, [query block,]
// key block), nonzero = visible. A query always sees its own block.
constexpr int kMaskBlock = 128;
constexpr int kMaskShift = 7;
// Keys one decode workgroup streams in one range at most (its blocks'
// visibility is staged in LDS).
constexpr int kMaxRangeBlocks = 4096;
constexpr int kMaxRangeKeys = (kMaxRangeBlocks - 2) * kMaskBlock;

// One decode split's streaming state ("record"), stored in the workspace as
// A[D], B[D], m, l, S, pi (2D + 4 floats) for every (b, hq, split).
//   m  : maximum of the logits over the split's keys, in log2 units
//        (z_j * log2 e); -inf marks an empty record
//   l  : sum_j e_j                         e_j = 2^(z_j log2e - m)
//   S  : sum_j e_j (s_j - pi)
//   A  : sum_j e_j v_j
//   B  : sum_j e_j (s_j - pi) v_j
//   pi : the pivot the record's probe scores are taken against
__host__ __device__ constexpr int partial_floats(int D) { return 2 * D + 4; }

struct DecodeArgs {
    const void *q, *r, *k, *v;
    void *o;
    const int32_t *cu;  // device [B+1] or nullptr (dense cache)
    int B, Hq, Hkv, D, kv_len;
    int window;         // > 0: a sequence's last `window` keys only; 0: all
    float zscale;       // qk_scale * log2(e)
    float rk_scale;
    int splits;         // >= 1
    int chunk;          // keys per split, multiple of 32
    int sk_parts;       // 0, or the stream-K plan's ranges per KV head (packed batches)
    float *ws;          // records [B][Hq][splits] ([Hq][sk_parts + B - 1] stream-K), unless fused
    bool fused;         // one split and no records: write o directly
    const uint8_t *block_mask;  // nullptr, or [B, Hkv, mask_cols] key-block visibility
    int mask_cols;      // ceil(kv_len / kMaskBlock)
};

enum class DecodePath { Mfma, Generic };

// Host-side decode plan shared by the workspace query and the launch.
struct DecodePlan {
    DecodePath path;
    int splits;
    int chunk;
    size_t ws_bytes;
};

DecodePlan plan_decode(int B, int Hq, int Hkv, int D, int kv_len, int window, int dtype,
                       int num_splits);

// Streaming kernel (records, or o when a.fused).
hipError_t launch_decode_split(const DecodeArgs &a, DecodePath path, int dtype, bool parallax,
                               hipStream_t stream);
// Merge of a.splits records per (b, hq) into o (a.q/k/v/r/cu unused).
hipError_t launch_decode_merge(const DecodeArgs &a, int dtype, bool parallax, hipStream_t stream);

struct PrefillArgs {
    const void *q, *r, *k, *v;
    void *o;
    float *lse, *sbar;
    void *vbar;         // nullptr, or the softmax readout sum_j w_j v_j (layout and dtype of o)
    const int32_t *cu;  // nullptr: dense [B, H, L, D]; else packed [T, H, D], cu [B + 1]
    int *sched;         // nullptr: persistent workgroups stride over the work items (dense
                        // batches); else 8 zeroed queue counters they draw items from
    int workers;        // compute units of the device (sizes the persistent grid)
    int B, Hq, Hkv, L, D;  // L: the (maximum) sequence length
    int window;         // query i sees keys i - window + 1 .. i (window = L: causal only)
    const uint8_t *block_mask;  // nullptr, or [B, Hkv, nb, nb], nb = ceil(L / kMaskBlock)
    float zscale;       // qk_scale * log2(e)
    float rk_scale;
};

hipError_t launch_prefill(const PrefillArgs &a, int dtype, hipStream_t stream);
bool prefill_supported(int D, int dtype);

// Per-row statistics the backward's key pass reads, written by its row pass:
// {lse * log2 e, sbar, delta = o . dLoss/do, ubar = sum_j w_j dLoss/do . v_j}.
struct RowStat {
    float lse2, sbar, delta, ubar;
};

struct BackwardArgs {
    const void *q, *r, *k, *v, *o, *go;  // go: dLoss/do, layout of o
    const float *lse, *sbar;             // the forward's row statistics
    const void *vbar;                    // nullptr, or the forward's softmax readout (then
                                         // ubar = dLoss/do . vbar needs no sweep of the keys)
    void *dq, *dr, *dk, *dv;
    RowStat *rowstat;                    // workspace: [B, Hq, L] dense, [Hq, T] packed
    const int32_t *cu;                   // as in PrefillArgs
    int total;                           // T, the packed token count
    int *sched;                          // nullptr, or 16 zeroed queue counters (rows 0..7, keys 8..15)
    int workers;                         // workgroups of a persistent launch
    int B, Hq, Hkv, L, D;
    int window;                          // as in PrefillArgs, 1 .. L
    const uint8_t *block_mask;           // as in PrefillArgs
    float zscale;                        // qk_scale * log2(e)
    float qk_scale, rk_scale;
};

hipError_t launch_prefill_backward(const BackwardArgs &a, int dtype, hipStream_t stream);

// Zero n (<= 64) int counters on the stream (a kernel, so that it can be
// captured in a graph).
hipError_t launch_zero_counters(int *c, int n, hipStream_t stream);

}  // namespace plx
