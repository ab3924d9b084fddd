// Parallax decode kernels for gfx950 (MI355X).
//
// What is computed (PyPI README of parallax-kernel, "Decoding (CuTeDSL)";
// neuraltrendhub summary "What the paper found"): for each sequence b and
// query head h, with every cached key visible,
//   o = sum_j w_j v_j + sum_j w_j (s_j - sbar) v_j,
//   w = softmax(qk_scale q.k_j), s_j = rk_scale r.k_j, sbar = sum_j w_j s_j.
// The summary describes a streaming decode kernel that keeps FlashAttention's
// KV tiling; that is the design point kept here: each K tile is read from
// HBM once and feeds both score sets (q.k and r.k), each V tile once and
// feeds both readouts (sum e v and sum e s v).
//
// Streaming state per (query head, split), with a pivot pi that follows the
// running weighted mean of the probe scores (re-based exactly whenever it
// drifts, see kPivotDrift):
//   m (log2 units), l = sum e, S = sum e (s - pi), A = sum e v,
//   B = sum e (s - pi) v,  and  o = (A + B - (S / l) A) / l.
// Two states merge as (m, l, S, A, B) -> max m and 2^(m_i - M)-weighted sums,
// after re-basing them onto one pivot (S += (pi_i - pi) l, B += (pi_i - pi) A).
//
// Kernels:
//   decode_mfma_bf16_d128<G, PLX>  bf16, head_dim 128, G query heads per KV
//       head (1 to 8; larger groups in chunks of 8). One workgroup of four
//       waves per (KV head, split, sequence), or per (KV head, chunk, split,
//       sequence). Both contractions on v_mfma_f32_16x16x32_bf16:
//         scores   S^T[key, vec] = K_tile . [q_0, r_0, q_1, r_1, ...]^T
//         readout  O^T[dim, row] = V_tile^T . [p_0, p_0 s'_0, p_1, ...]^T
//       The key order inside each 16-key block is chosen so that the score
//       MFMA's output lands in exactly the lanes and register order the
//       readout MFMA wants for its B operand (see the lane map below), and
//       V's natural [key][dim] layout becomes the readout's A operand by an
//       8x8 16-bit transpose inside each lane's registers. K tiles are
//       copied into LDS by the buffer unit (whole 256-byte rows) and read
//       back in the score MFMA's layout; V streams with 128-bit non-temporal
//       buffer loads straight into registers. The four waves' states meet in
//       LDS only once, at the end of the split.
//   decode_mfma_streamk<G, PLX>  the same streaming for a packed batch: each
//       KV head's tokens, all sequences back to back, cut into equal ranges,
//       one workgroup per range and one record per sequence piece.
//   decode_generic<T, D, PLX>  fp32 or bf16, head_dim 64/128, any group size.
//       One wave per (query head, split, sequence), fp32 VALU.
//   decode_reduce<TO, D, PLX>  merges split records into o.
#include "plx_internal.h"
#include "plx_device.h"

namespace plx {

namespace {

// Waves per workgroup of the MFMA decode kernel; a split's keys are a
// multiple of 32 * kDecodeWaves.
constexpr int kDecodeWaves = 4;
// K tiles are staged through LDS by the buffer unit (each copy reads whole
// 256-byte key rows) and read back in the score MFMA's layout. Loading that
// layout straight from memory reads 64 bytes of each of 16 keys per
// instruction, half of every cache line it touches, which a read-only probe
// of this access pattern measured 10% slower than whole rows.
constexpr bool kDecodeKInLds = true;

typedef __attribute__((address_space(3))) void lds_void;

// 16-byte chunk slot of chunk c of key k in an LDS K tile: c ^ kswz(k); the
// 128-bit operand reads (16 permuted keys, eight lanes served at a time) see
// eight distinct values of slot & 7.
__device__ __forceinline__ int kswz(int key) { return 2 * ((key >> 2) & 3) + 9 * (key & 1); }

struct SeqRange {
    int64_t tok0;  // first token of the visible range in the K/V arrays
    int len;       // keys in the visible range
    int pos0;      // sequence position of the range's first key (window start)
    int last_blk;  // block-sparse: block of the sequence's last key (always visible)
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
    s.pos0 = 0;
    s.last_blk = (s.len - 1) >> kMaskShift;
    if (a.window > 0 && s.len > a.window) {  // sliding window: the last `window` keys
        s.pos0 = s.len - a.window;
        s.tok0 += s.pos0;
        s.len = a.window;
    }
    return s;
}

// Block-sparse visibility of a sequence's key block (uniform), nullptr: all.
__device__ __forceinline__ const uint8_t *mask_row(const DecodeArgs &a, int b, int hkv) {
    return a.block_mask ? a.block_mask + ((int64_t)b * a.Hkv + hkv) * a.mask_cols : nullptr;
}

// -------------------------------------------------------------------------
// MFMA decode, bf16, head_dim 128.
//
// Workgroup = kDecodeWaves waves on one (KV head, split, sequence); wave w
// streams tiles w, w + kDecodeWaves, ... of the split's 32-key tiles, so the
// workgroup reads neighbouring tiles together, and the wave states merge in
// LDS into one record (or, with a single split, straight into o).
//
// Lane map inside a wave (lane = 16 * g + n, g = 0..3, n = 0..15):
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
// Keys start .. end - 1 (range-relative, non-empty) of sequence b, whose
// range starts at token seq_tok0 and sequence position pos0, for KV head
// hkv: writes the G heads' records at record index rbase + h * rstride, or o
// when `fused`. With `more` (the workgroup streams another range after this
// one) the record path ends with a workgroup barrier, so that the next range
// may reuse the LDS; the fused path runs once per workgroup.
//
// MASK (a block mask is given): the waves walk the visible 128-key blocks of
// the range only -- wave w takes keys 32w .. 32w + 31 of each -- so every
// load in flight is a visible tile. With nvsplit > 0 the range is the whole
// window (start = 0) and this workgroup takes the vsplit-th of nvsplit equal
// shares of its visible blocks, which balances the splits whatever the mask.
// Keys outside start .. end - 1 of a block that straddles the range's edge
// are masked per key.
template <int G, bool PLX, bool MASK>
__device__ __forceinline__ void decode_range(const DecodeArgs &a, const int hkv, const int b,
                                             const int64_t seq_tok0, const int start, const int end,
                                             const int pos0, const int last_blk,
                                             const int vsplit, const int nvsplit,
                                             const int64_t rbase, const int64_t rstride,
                                             const bool fused, const int hq0, const int ngl,
                                             const bool more) {
    constexpr int D = 128;
    constexpr int NR = PLX ? 2 : 1;
    constexpr int NV = NR * G;
    constexpr int W = kDecodeWaves;
    static_assert(NV <= 16, "at most 16 live columns");
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int nv = NR * ngl;  // live columns (NV unless a chunk of a larger group ends early)
    const bool live = n < nv;
    const int h = live ? n / NR : 0;  // head within the group
    const int kind = live ? n % NR : 0;
    const int hq = hq0 + h;
    const int64_t row0 = (int64_t)b * a.Hq + hq0;  // first query row of the group

    const uint16_t *qh = reinterpret_cast<const uint16_t *>(a.q);
    const uint16_t *rh = reinterpret_cast<const uint16_t *>(a.r);
    const uint16_t *kh = reinterpret_cast<const uint16_t *>(a.k);
    const uint16_t *vh = reinterpret_cast<const uint16_t *>(a.v);

    // K/V of this split through buffer resources whose range ends at the
    // split's last key: tail lanes past `end` read zeros (their logits are
    // masked below), all addressing is 32-bit offsets from a scalar base.
    const int64_t tok_stride = (int64_t)a.Hkv * D;  // elements between consecutive tokens
    const int ts_bytes = (int)(tok_stride * 2);
    const int64_t split0 = (seq_tok0 + start) * tok_stride + (int64_t)hkv * D;
    const uint32_t span = (uint32_t)(((int64_t)(end - start - 1) * tok_stride + D) * 2);
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(kh + split0), 0, span, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(vh + split0), 0, span, kBufferFlags);
    // Key permutation inside a 16-key block for the score MFMA's A operand.
    const int kperm = (n >> 2) + 4 * (n & 3);
    const int koff0 = kperm * ts_bytes + 16 * g;         // block 0, k-step u at +64u bytes
    const int koff1 = (16 + kperm) * ts_bytes + 16 * g;  // block 1
    const int voff = g * ts_bytes + 16 * n;              // key g + 4t at + 4t keys

    // Block-sparse: the visibility of the blocks this range touches, staged in
    // LDS by all threads at once (the block holding the sequence's last key is
    // always visible); each wave then walks the visible ones with a 64-block
    // ballot window. A tile past the walk's end reads past the buffer range.
    __shared__ uint8_t svis[MASK ? kMaxRangeBlocks : 1];
    __shared__ int svis_total;
    const int blk0 = (pos0 + start) >> kMaskShift;
    const int nblk = MASK ? ((pos0 + end - 1) >> kMaskShift) - blk0 + 1 : 0;
    int walk_first = 0, walk_count = 0;  // ordinal share of the visible blocks (MASK)
    uint64_t wbits = 0;
    int wbase = -64;
    if constexpr (MASK) {
        const uint8_t *mrow = mask_row(a, b, hkv);
        if (threadIdx.x == 0) svis_total = 0;
        __syncthreads();
        int mine = 0;
        for (int i = threadIdx.x; i < nblk; i += 64 * W) {
            const bool v = blk0 + i == last_blk || mrow[blk0 + i] != 0;
            svis[i] = v ? 1 : 0;
            mine += v ? 1 : 0;
        }
        if (nvsplit > 0 && mine > 0) atomicAdd(&svis_total, mine);
        __syncthreads();
        if (nvsplit > 0) {
            const int per = (svis_total + nvsplit - 1) / nvsplit;
            walk_first = vsplit * per;
            walk_count = max(0, min(svis_total - walk_first, per));
        } else {
            walk_count = nblk;  // every visible block of the range
        }
    }
    // next visible block index (relative to blk0) at or after i, or nblk
    auto next_block = [&](int i) {
        return next_visible(i, nblk, wbits, wbase, [&](int u) { return svis[u] != 0; });
    };
    const int oob = (end - start + kMaskBlock) * ts_bytes;  // a tile offset past the buffer range
    auto tile_offset = [&](int t) {
        if constexpr (!MASK) return (t - start) * ts_bytes;  // past `end`: outside the range too
        return t < end ? (t - start) * ts_bytes : oob;
    };

    // The whole offset goes in the VGPR operand: the range check of a raw
    // buffer access covers the VGPR and immediate offsets, not soffset.
    auto load_k = [&](int t0, bf16x8 *kt) {
        const int tb = tile_offset(t0);  // wave-uniform
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            kt[u] = buffer_load16(krs, tb + koff0 + 64 * u);
            kt[4 + u] = buffer_load16(krs, tb + koff1 + 64 * u);
        }
    };
    auto load_v = [&](int t0, bf16x8 *vt) {
        const int vo = tile_offset(t0) + voff;
#pragma unroll
        for (int t = 0; t < 8; ++t) vt[t] = buffer_load16(vrs, vo + 4 * t * ts_bytes);
    };
    // LDS K tiles: two slots per wave, in separate arrays so that waiting for
    // one slot's copy never waits for the other's. Copy j moves keys 4j ..
    // 4j + 3 of the wave's tile (a 256-byte row per 16 lanes); lane l writes
    // slot l % 16 of its key, i.e. fetches chunk (l % 16) ^ kswz(key).
    __shared__ __attribute__((aligned(16))) uint16_t sk0[kDecodeKInLds ? W * 32 * D : 8];
    __shared__ __attribute__((aligned(16))) uint16_t sk1[kDecodeKInLds ? W * 32 * D : 8];
    auto dma_k = [&](int t0, uint16_t *slot) __attribute__((always_inline)) {
        uint16_t *base = slot + wave * 32 * D;
        const int tb = tile_offset(t0);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int key = 4 * j + (lane >> 4);
            const int chunk = (lane & 15) ^ kswz(key);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void *)(base + 4 * j * D), 16,
                                                     tb + key * ts_bytes + 16 * chunk, 0, 0, 2);
        }
    };
    // the score operand from the wave's slot: the same keys and dims as the
    // direct load (block kb, k-step u -> key 16 kb + kperm, chunk g + 4u)
    auto lds_k = [&](const uint16_t *slot, bf16x8 *kt) __attribute__((always_inline)) {
        const uint16_t *lk = slot + wave * 32 * D;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int key = 16 * kb + kperm;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                kt[4 * kb + u] = *reinterpret_cast<const bf16x8 *>(&lk[key * D + (((g + 4 * u) ^ kswz(key)) * 8)]);
        }
    };

    // B operand of the score MFMA (vector n, dims 8(g + 4u) .. +8): loaded
    // before the K/V tiles, so that waiting for it (loads complete in order)
    // leaves the tiles in flight. Dead columns load head 0's row and are
    // zeroed afterwards.
    bf16x8 qr[4];
    {
        const uint16_t *src = (kind == 0 ? qh : rh) + ((int64_t)b * a.Hq + hq) * D;
#pragma unroll
        for (int u = 0; u < 4; ++u) qr[u] = load16(src + 8 * (g + 4 * u));
    }
    __builtin_amdgcn_sched_barrier(0);

    // Two tile buffers per wave: while one tile is consumed the next is in
    // flight. Loads are never predicated: a tile past `end` lies outside the
    // buffer range and reads zeros without touching memory, so every step
    // issues the same loads and waits for exactly the tile it consumes. A
    // tile's K registers take the next loads as soon as its scores are
    // issued, its V registers after its readout.
    constexpr int kStride = 32 * W;  // keys between a wave's consecutive tiles
    bf16x8 kA[8], vA[8], kB[8], vB[8];
    int t0 = start + 32 * wave;
    // MASK: the walk's first two tiles (end: none). The walk starts at the
    // walk_first-th visible block.
    int tw[2] = {end, end};
    int wblk = -1;
    if constexpr (MASK) {
        // the walk_first-th visible block: skip whole 64-block windows by their
        // popcount, then clear the remaining lower set bits of the window
        int i = 0, skip_n = walk_first;
        while (skip_n > 0 && i < nblk) {
            const int u = i + lane;
            uint64_t m = __builtin_amdgcn_ballot_w64(u < nblk && svis[u] != 0);
            const int c = __builtin_popcountll(m);
            if (c <= skip_n) {
                skip_n -= c;
                i += 64;
            } else {
                for (; skip_n > 0; --skip_n) m &= m - 1;
                i += __builtin_ctzll(m);
            }
        }
        for (int k = 0; k < 2 && k < walk_count; ++k) {
            wblk = next_block(k == 0 ? i : wblk + 1);
            tw[k] = ((blk0 + wblk) << kMaskShift) + 32 * wave - pos0;
        }
    }
    if constexpr (MASK) {
        if constexpr (kDecodeKInLds) dma_k(tw[0], sk0); else load_k(tw[0], kA);
        load_v(tw[0], vA);
        if constexpr (kDecodeKInLds) dma_k(tw[1], sk1); else load_k(tw[1], kB);
        load_v(tw[1], vB);
    } else {
        if constexpr (kDecodeKInLds) dma_k(t0, sk0); else load_k(t0, kA);
        load_v(t0, vA);
        if constexpr (kDecodeKInLds) dma_k(t0 + kStride, sk1); else load_k(t0 + kStride, kB);
        load_v(t0 + kStride, vB);
    }

    if (!live) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            for (int e = 0; e < 8; ++e) qr[u][e] = (__bf16)0.0f;
    }
    // Probe pivot of the column (probe lanes; probe-scale units): starts at 0
    // and follows the running weighted mean of the column's probe scores.
    float piv = 0.0f;

    // Running reference max of the column's head, in log2 units. It is only
    // raised when a tile's max exceeds it by more than kRescaleSlack (or on
    // the first tile), so the accumulators are rarely rescaled; terms are
    // then at most 2^kRescaleSlack, far from fp32 or bf16 overflow.
    // (MASK: finite, because a wave's quarter of a block that straddles the
    // range's edge can lie wholly outside the range, and exp2(-inf - m_run)
    // must then be 0; a wave that saw no key is marked -inf again below.)
    float m_run = MASK ? -1e30f : -INFINITY;
    float lsum = 0.0f;  // per-lane partial: sum p (n even) or sum p s' (n odd)
    floatx4 acc[8];
    for (int e = 0; e < 8; ++e) acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};
    // per-lane factor turning p into the column's P-row: 1 on softmax rows,
    // (rk_scale * raw - pi) on probe rows -- one FMA, no select
    const float fa = (PLX && kind) ? a.rk_scale : 0.f;
    float fc = (PLX && kind) ? -piv : 1.f;

    // Consume the tile at t0 (range-relative), then issue this buffer's loads
    // for the tile at tn. masked: some keys of the tile lie outside start ..
    // end - 1 (the range's tail, or the edge of a straddling block).
    auto step = [&](bool masked, bf16x8 *kt, bf16x8 *vt, uint16_t *slot, int t0, int tn) {
        // ---- both score sets from one K tile
        bf16x8 kl[8];
        if constexpr (kDecodeKInLds) {
            lds_k(slot, kl);
            kt = kl;
        }
        floatx4 sc0 = {0.f, 0.f, 0.f, 0.f}, sc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            sc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt[u], qr[u], sc0, 0, 0, 0);
            sc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt[4 + u], qr[u], sc1, 0, 0, 0);
        }
        // this buffer's next K tile, as soon as the scores hold its operands.
        // The copy overwrites the slot the score operand was just read from:
        // it must not be issued before those LDS reads have returned, which
        // the MFMAs' use of them guarantees (the compiler would otherwise
        // hoist the copy above the wait for the reads).
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kDecodeKInLds) dma_k(tn, slot); else load_k(tn, kt);
        float raw[8], zr[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            raw[i] = sc0[i];
            raw[4 + i] = sc1[i];
        }
        // the column's head logit (unscaled): own value on softmax rows, the
        // left neighbour's on probe rows (quad_perm [0,0,2,2])
        const int nvalid = end - t0;  // key g + 4t is valid iff g + 4t < nvalid
        float rmax = -INFINITY;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            zr[t] = PLX ? dpp_pair_even(raw[t]) : raw[t];
            if (masked && (g + 4 * t >= nvalid || (MASK && t0 + g + 4 * t < start)))
                zr[t] = -INFINITY;
            rmax = fmaxf(rmax, zr[t]);
        }
        // lazy rescale, decided for the whole wave from the lane-local max;
        // the column max across the four rows is only taken when it is raised
        const bool raise = rmax * a.zscale > m_run + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
            const float tmax = xor_max_rowgroups(rmax) * a.zscale;
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            lsum *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] *= alpha;
        }
        const float neg_m = -m_run;
        float tsum = 0.0f;
        float pe[8], pv[8];  // the weight e, and the column's P-row value
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            pe[t] = __builtin_amdgcn_exp2f(fmaf(zr[t], a.zscale, neg_m));
            pv[t] = pe[t] * fmaf(raw[t], fa, fc);
            tsum += pv[t];
        }
        lsum += tsum;
        if constexpr (PLX) {
            // pivot drift: a probe lane compares its partial S with the partial
            // l of its head's softmax lane (same keys); a re-base moves the
            // column's pivot to its running mean, before this tile's P o S'
            // is rounded
            const float lnb = dpp_pair_even(lsum);
            const bool drift = kind != 0 && fabsf(lsum) > kPivotDrift * lnb;
            if (__builtin_amdgcn_ballot_w64(drift) != 0) {
                const float col = xor_sum_rowgroups(lsum);  // l (softmax lanes), S (probe lanes)
                const float lcol = dpp_pair_even(col);
                const float d = (kind != 0 && lcol > 0.f) ? col / lcol : 0.f;
                piv += d;
                fc -= d;
                lsum = fmaf(-d, lnb, lsum);
#pragma unroll
                for (int t = 0; t < 8; ++t) pv[t] = fmaf(-d, pe[t], pv[t]);
#pragma unroll
                for (int e = 0; e < 8; ++e)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[e][i] = fmaf(-d, dpp_pair_even(acc[e][i]), acc[e][i]);
            }
        }
        bf16x8 pf;
#pragma unroll
        for (int t = 0; t < 8; ++t) pf[t] = (__bf16)pv[t];

        // ---- V^T operand: 8x8 16-bit transpose in registers.
        // vt[t] holds dims 8n..8n+7 of key g + 4t; vT[e] holds keys t = 0..7 of dim 8n + e.
        bf16x8 vT[8];
#pragma unroll
        for (int d2 = 0; d2 < 4; ++d2) {
            uint32_t lo[4], hi[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t x = __builtin_bit_cast(uint4, vt[2 * j])[d2];
                const uint32_t y = __builtin_bit_cast(uint4, vt[2 * j + 1])[d2];
                lo[j] = __builtin_amdgcn_perm(y, x, 0x05040100u);  // dim 2*d2   of keys 2j, 2j+1
                hi[j] = __builtin_amdgcn_perm(y, x, 0x07060302u);  // dim 2*d2+1 of keys 2j, 2j+1
            }
            vT[2 * d2] = __builtin_bit_cast(bf16x8, uint4{lo[0], lo[1], lo[2], lo[3]});
            vT[2 * d2 + 1] = __builtin_bit_cast(bf16x8, uint4{hi[0], hi[1], hi[2], hi[3]});
        }
        // ---- both readouts from one V tile
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vT[e], pf, acc[e], 0, 0, 0);
        load_v(tn, vt);  // and its next V tile
    };

    if constexpr (!MASK) {
        while (true) {
            if (t0 >= end) break;
            if (t0 + 32 <= end) step(false, kA, vA, sk0, t0, t0 + 2 * kStride);
            else step(true, kA, vA, sk0, t0, t0 + 2 * kStride);
            t0 += kStride;
            if (t0 >= end) break;
            if (t0 + 32 <= end) step(false, kB, vB, sk1, t0, t0 + 2 * kStride);
            else step(true, kB, vB, sk1, t0, t0 + 2 * kStride);
            t0 += kStride;
        }
    } else {
        // tiles cur (buffer A), nx1 (buffer B), nx2 as range-relative t0;
        // `end` marks a finished walk
        int cur = tw[0], nx1 = tw[1], done = 2;
        while (true) {
            if (cur >= end) break;
            int nx2 = end;
            if (done < walk_count) {
                wblk = next_block(wblk + 1);
                nx2 = ((blk0 + wblk) << kMaskShift) + 32 * wave - pos0;
                ++done;
            }
            step(cur < start || cur + 32 > end, kA, vA, sk0, cur, nx2);
            cur = nx1;
            nx1 = nx2;
            if (cur >= end) break;
            nx2 = end;
            if (done < walk_count) {
                wblk = next_block(wblk + 1);
                nx2 = ((blk0 + wblk) << kMaskShift) + 32 * wave - pos0;
                ++done;
            }
            step(cur < start || cur + 32 > end, kB, vB, sk1, cur, nx2);
            cur = nx1;
            nx1 = nx2;
        }
    }
    // the wave's read-ahead copies land in its LDS slots before the workgroup
    // moves on or ends (the slots are the wave's own; the barrier after the
    // state writes below then holds every wave until all copies have landed)
    if constexpr (kDecodeKInLds) __builtin_amdgcn_s_waitcnt(0);

    if (MASK && m_run < -1e29f) m_run = -INFINITY;  // no visible key in this wave
    lsum = xor_sum_rowgroups(lsum);

    // ---- merge the waves' states in LDS
    __shared__ __attribute__((aligned(16))) float sm_acc[W][NV][D];
    __shared__ float sm_m[W][NV], sm_l[W][NV], sm_piv[W][NV];
    if (live) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) sm_acc[wave][n][32 * g + 8 * i + e] = acc[e][i];
        if (g == 0) {
            sm_m[wave][n] = m_run;
            sm_l[wave][n] = lsum;
            sm_piv[wave][n] = piv;
        }
    }
    __syncthreads();
    // The waves' probe terms are re-based onto wave 0's pivot:
    //   B_w + (pi_w - pi_0) A_w,  S_w + (pi_w - pi_0) l_w.
    // Each thread below issues all its LDS reads before it uses any of them:
    // the weight of a wave that saw no key is selected to 0, not branched
    // around, so the merge is one round of LDS reads after the barrier.
    // Weights of the waves' states for a column whose wave maxima are mw.
    auto wave_weights = [](const float (&mw)[W], float (&c)[W]) __attribute__((always_inline)) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, mw[w]);
#pragma unroll
        for (int w = 0; w < W; ++w) c[w] = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
        return M;
    };

    if (!fused) {
        // thread: dims d, d + 1 of record column cn (a wave covers one column);
        // the column's first thread also writes its scalars
        for (int idx = threadIdx.x; idx < nv * (D / 2); idx += 64 * W) {
            const int cn = idx / (D / 2), d = 2 * (idx % (D / 2));
            const bool probe = PLX && cn % NR != 0;
            const int cb = probe ? cn - 1 : cn;  // the probe column's softmax neighbour
            float mw[W], c[W], dp[W], lw[W], lb[W];
            float2 x[W], y[W];
#pragma unroll
            for (int w = 0; w < W; ++w) {
                mw[w] = sm_m[w][cn];
                x[w] = *reinterpret_cast<const float2 *>(&sm_acc[w][cn][d]);
                y[w] = *reinterpret_cast<const float2 *>(&sm_acc[w][cb][d]);
                dp[w] = sm_piv[w][cn] - sm_piv[0][cn];
                lw[w] = sm_l[w][cn];
                lb[w] = sm_l[w][cb];
            }
            const float M = wave_weights(mw, c);
            float2 val = {0.f, 0.f};
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const float e = probe ? dp[w] : 0.f;
                val.x = fmaf(c[w], fmaf(e, y[w].x, x[w].x), val.x);
                val.y = fmaf(c[w], fmaf(e, y[w].y, x[w].y), val.y);
                sum = fmaf(c[w], fmaf(e, lb[w], lw[w]), sum);
            }
            float *rec = a.ws + (rbase + (cn / NR) * rstride) * partial_floats(D);
            *reinterpret_cast<float2 *>(rec + (cn % NR) * D + d) = val;
            if (d == 0) {
                if (!probe)
                    *reinterpret_cast<float2 *>(rec + 2 * D) = float2{M, sum};
                if (!PLX)
                    *reinterpret_cast<float2 *>(rec + 2 * D + 2) = float2{0.f, 0.f};
                else if (probe)
                    *reinterpret_cast<float2 *>(rec + 2 * D + 2) = float2{sum, sm_piv[0][cn]};
            }
        }
        if (more) __syncthreads();  // the workgroup's next range reuses the LDS
        return;
    }

    // One split: finalise here, o = (A + B - (S / l) A) / l per (head, dim).
    for (int idx = threadIdx.x; idx < ngl * D; idx += 64 * W) {
        const int hh = idx / D, d = idx % D;
        const int ca = NR * hh;
        const int cp = PLX ? ca + 1 : ca;  // the head's probe column
        float mw[W], c[W], xa[W], xb[W], la[W], lp[W], dp[W];
#pragma unroll
        for (int w = 0; w < W; ++w) {
            mw[w] = sm_m[w][ca];
            xa[w] = sm_acc[w][ca][d];
            la[w] = sm_l[w][ca];
            xb[w] = sm_acc[w][cp][d];
            lp[w] = sm_l[w][cp];
            dp[w] = sm_piv[w][cp] - sm_piv[0][cp];
        }
        wave_weights(mw, c);
        float A = 0.f, Bv = 0.f, l = 0.f, S = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            A = fmaf(c[w], xa[w], A);
            l = fmaf(c[w], la[w], l);
            if (PLX) {
                Bv = fmaf(c[w], fmaf(dp[w], xa[w], xb[w]), Bv);
                S = fmaf(c[w], fmaf(dp[w], la[w], lp[w]), S);
            }
        }
        const float inv_l = 1.0f / l;
        const float val = PLX ? (A * (1.0f - S * inv_l) + Bv) * inv_l : A * inv_l;
        reinterpret_cast<uint16_t *>(a.o)[(row0 + hh) * D + d] = f32_to_bf16(val);
    }
}

// One workgroup per (KV head, split, sequence): the split's keys of its
// sequence. An empty split writes an empty record (or, fused, o = 0).
// For G <= 2 the launch bound asks for two waves per SIMD: the kernel then
// fits 224 VGPRs without spills and keeps the V tiles in VGPRs rather than
// AGPRs (no copies before the transpose), and two workgroups share a CU when
// the grid has more than one per CU (measured: kernel 24.7 -> 24.4 us at
// B = 1 with 32 splits, 2.60 -> 2.58 ms per step at B = 2048).
// CHUNK: more than G query heads per KV head (G = 8 then), taken G at a time:
// workgroup x = (KV head, chunk) streams the KV head's keys for heads
// 8 chunk .. 8 chunk + 7 of its group (fewer in a last, partial chunk).
template <int G, bool PLX, bool MASK, bool CHUNK = false>
__global__ __launch_bounds__(64 * kDecodeWaves, G <= 2 ? 2 : 1)
void decode_mfma_bf16_d128(DecodeArgs a) {
    constexpr int D = 128;
    const int gq = a.Hq / a.Hkv;                          // query heads per KV head
    const int nch = CHUNK ? (gq + G - 1) / G : 1;
    const int hkv = CHUNK ? blockIdx.x / nch : blockIdx.x;
    const int hq0 = CHUNK ? hkv * gq + G * (blockIdx.x % nch) : hkv * G;  // first query head
    const int ngl = CHUNK ? min(G, gq - G * (int)(blockIdx.x % nch)) : G;  // its heads
    const int split = blockIdx.y;
    const int b = blockIdx.z;
    const SeqRange sr = seq_range(a, b);
    const int start = split * a.chunk;
    const int64_t row0 = (int64_t)b * a.Hq + hq0;  // first query row of the workgroup
    // Block mask: the splits share the window's visible blocks equally when its
    // blocks fit the LDS staging and its bytes 32-bit offsets; otherwise each
    // split walks the visible blocks of its own key range.
    bool whole = false;
    if constexpr (MASK) {
        const int nblk = ((sr.pos0 + sr.len - 1) >> kMaskShift) - (sr.pos0 >> kMaskShift) + 1;
        const int64_t tok_bytes = (int64_t)a.Hkv * D * 2;
        whole = sr.len > 0 && nblk <= kMaxRangeBlocks &&
                ((int64_t)sr.len + 2 * kMaskBlock + 64) * tok_bytes + 1024 < 0x7fffffffLL;
    }
    if (sr.len <= 0 || (!whole && start >= sr.len)) {
        // Nothing to stream: a fused call writes the zero output of an empty
        // sequence, otherwise the records are marked empty for the merge.
        if (a.fused) {
            uint16_t *o = reinterpret_cast<uint16_t *>(a.o) + row0 * D;
            for (int i = threadIdx.x; i < ngl * D; i += 64 * kDecodeWaves) o[i] = 0;
        } else if (threadIdx.x < ngl) {
            float *rec = a.ws + ((row0 + threadIdx.x) * a.splits + split) * partial_floats(D);
            reinterpret_cast<float4 *>(rec + 2 * D)[0] = float4{-INFINITY, 0.f, 0.f, 0.f};
        }
        return;
    }
    if (whole)
        decode_range<G, PLX, MASK>(a, hkv, b, sr.tok0, 0, sr.len, sr.pos0, sr.last_blk, split,
                                   a.splits, row0 * a.splits + split, a.splits, a.fused, hq0, ngl,
                                   false);
    else
        decode_range<G, PLX, MASK>(a, hkv, b, sr.tok0, start, min(start + a.chunk, sr.len),
                                   sr.pos0, sr.last_blk, 0, 0, row0 * a.splits + split, a.splits,
                                   a.fused, hq0, ngl, false);
}

// Packed batches (stream-K): the tokens of one KV head, all sequences back to
// back, are cut into a.sk_parts equal ranges, one workgroup each, so every
// workgroup streams the same number of keys whatever the length mix. A range
// that crosses sequence boundaries yields one record per sequence piece;
// piece (range w, sequence b) goes to record slot w + b of its query head
// (unique: when range w + k overlaps sequence b - k, sequence b starts after
// range w ends), [Hq][sk_parts + B - 1] records in all.
template <int G, bool PLX, bool MASK>
__global__ __launch_bounds__(64 * kDecodeWaves)
void decode_mfma_streamk(DecodeArgs a) {
    const int part = blockIdx.x;
    const int hkv = blockIdx.y;
    const int T = a.cu[a.B];
    const int R = (T + a.sk_parts - 1) / a.sk_parts;
    const int t_lo = part * R;
    const int t_hi = min(T, t_lo + R);
    if (t_lo >= t_hi) return;
    // first sequence holding token t_lo: the last b with cu[b] <= t_lo
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.cu[mid] <= t_lo) lo = mid; else hi = mid - 1;
    }
    const int64_t ns = a.sk_parts + a.B - 1;
    for (int b = lo; b < a.B; ++b) {
        const int s0 = a.cu[b], s1 = a.cu[b + 1];
        if (s0 >= t_hi) break;
        const int p0 = max(t_lo, s0), p1 = min(t_hi, s1);
        if (p0 >= p1) continue;  // empty sequence, or one that ends before the range
        decode_range<G, PLX, MASK>(a, hkv, b, s0, p0 - s0, p1 - s0, 0, (s1 - s0 - 1) >> kMaskShift,
                                   0, 0, (int64_t)hkv * G * ns + part + b, ns, false, hkv * G, G,
                                   true);
    }
}

// -------------------------------------------------------------------------
// Generic decode: fp32 or bf16 storage, head_dim 64 or 128, any group size.
// One wave per (query head, split, sequence). Lane = LPR * kgrp + c: the c-th
// 16-byte chunk of key kgrp + KPI*step. Each key group keeps its own
// streaming state; the groups merge through shuffles at the end. The key
// rows of a batch of steps are loaded while the batch before is folded in,
// a batch's dot products reduce through DPP lane exchanges, and its max
// rescales the state once (measured: B = 1, 2 heads, D = 64, fp32, 256 keys
// 8.6 -> 6.4 us per step; B = 4, 8 heads, 2048 keys 18.2 -> 10.0 us).
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

    const uint8_t *mrow = mask_row(a, b, hkv);
    // Iteration it covers keys start + KPI it .. + KPI - 1 (key group kgrp takes
    // one). Loads run a batch of U iterations ahead of their use: each batch's
    // K and V rows are all in flight while the batch before is folded in.
    constexpr int U = EPL == 4 ? 8 : 4;
    const int nit = (end - start + KPI - 1) / KPI;
    auto load_it = [&](int it, float *kv, float *vv) __attribute__((always_inline)) {
        const int jj = min(start + it * KPI + kgrp, end - 1);  // past the end: a valid row, unused
        Elem<T>::load(kseq + (int64_t)jj * tok_stride, kv);
        Elem<T>::load(vseq + (int64_t)jj * tok_stride, vv);
    };
    // Fold one batch: the U iterations' scores first (independent reductions),
    // then one rescale to the batch's max, then the weighted sums.
    auto fold_batch = [&](int it0, float (*kv)[EPL], float (*vv)[EPL]) __attribute__((always_inline)) {
        float zs[U], ss[U];
        bool val[U];
        float mb = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = start + (it0 + u) * KPI + kgrp;
            bool valid = it0 + u < nit && j < end;
            if (mrow && valid) {  // block-sparse: hidden blocks other than the last key's
                const int blk = (sr.pos0 + j) >> kMaskShift;
                valid = blk == sr.last_blk || mrow[blk] != 0;
            }
            float zp = 0.f, sp = 0.f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                zp += qv[e] * kv[u][e];
                if (PLX) sp += rv[e] * kv[u][e];
            }
            zs[u] = group_sum<LPR>(zp);
            ss[u] = PLX ? group_sum<LPR>(sp) : 0.f;
            val[u] = valid;
            if (valid) mb = fmaxf(mb, zs[u]);
        }
        if (mb == -INFINITY) return;  // nothing visible in this batch for this key group
        const float m_new = fmaxf(st.m, mb);
        const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
        st.m = m_new;
        st.l *= alpha;
        if (PLX) st.S *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            st.A[e] *= alpha;
            if (PLX) st.B[e] *= alpha;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!val[u]) continue;
            const float p = __builtin_amdgcn_exp2f(zs[u] - m_new);
            const float sd = ss[u] - piv;
            st.l += p;
            if (PLX) st.S += p * sd;
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                st.A[e] += p * vv[u][e];
                if (PLX) st.B[e] += (p * sd) * vv[u][e];
            }
        }
    };
    float kb[U][EPL], vb[U][EPL];
#pragma unroll
    for (int u = 0; u < U; ++u) load_it(u, kb[u], vb[u]);
    for (int it0 = 0; it0 < nit; it0 += U) {
        float kn[U][EPL], vn[U][EPL];
#pragma unroll
        for (int u = 0; u < U; ++u) load_it(it0 + U + u, kn[u], vn[u]);
        fold_batch(it0, kb, vb);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < EPL; ++e) {
                kb[u][e] = kn[u][e];
                vb[u][e] = vn[u][e];
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
// Record merge. One wave per (query head, sequence, slice of kMergeDims
// dims): the merge is latency-bound (a few hundred kilobytes written by the
// previous kernel), so it is spread over as many compute units as there are
// slices and every record load is issued before any is used. Lane
// (group rg, dim dd) folds records rg, rg + RG, rg + 2 RG, ... of the slice's
// dim dd with the online rescaling; the RG groups then combine through
// cross-lane exchanges. No LDS, no barrier.
// Empty records (m = -inf) are skipped (their A, B are never written); a row
// with no record gets o = 0. Records may carry different pivots: each is
// re-based onto the first record's pivot pi_0 with
//   S' = S + (pi_i - pi_0) l,   B' = B + (pi_i - pi_0) A
// (exact algebra).
// -------------------------------------------------------------------------
constexpr int kMergeDims = 16;     // dims per wave
constexpr int kMergeBatch = 8;     // records per lane whose loads are in flight together

struct MergeState {
    float m, l, S, A, B;
};

__device__ __forceinline__ void merge_into(MergeState &x, float mi, float li, float Si, float Ai, float Bi) {
    const float M = fmaxf(x.m, mi);
    if (M == -INFINITY) return;
    const float ax = __builtin_amdgcn_exp2f(x.m - M);
    const float ay = __builtin_amdgcn_exp2f(mi - M);
    x.m = M;
    x.l = x.l * ax + li * ay;
    x.S = x.S * ax + Si * ay;
    x.A = x.A * ax + Ai * ay;
    x.B = x.B * ax + Bi * ay;
}

template <typename TO, int D, bool PLX>
__global__ __launch_bounds__(64) void decode_reduce(DecodeArgs a) {
    constexpr int DW = kMergeDims;
    constexpr int RG = 64 / DW;  // record groups per wave
    const int lane = threadIdx.x;
    const int rg = lane / DW;
    const int d = blockIdx.z * DW + lane % DW;
    const int hq = blockIdx.x;
    const int b = blockIdx.y;
    // this (sequence, head)'s records: a.splits of them, or, for a stream-K
    // plan, the slots b + w of the ranges w that overlap the sequence
    int ns = a.splits;
    int64_t first = ((int64_t)b * a.Hq + hq) * ns;
    if (a.sk_parts) {
        const int T = a.cu[a.B];
        const int R = (T + a.sk_parts - 1) / a.sk_parts;
        const int s0 = a.cu[b], s1 = a.cu[b + 1];
        const int w_lo = s1 > s0 ? s0 / R : 0;
        ns = s1 > s0 ? (s1 - 1) / R - w_lo + 1 : 0;
        first = (int64_t)hq * (a.sk_parts + a.B - 1) + b + w_lo;
    }
    const float *base = a.ws + first * partial_floats(D);
    const float piv0 = PLX && ns > 0 ? base[2 * D + 3] : 0.f;

    MergeState st = {-INFINITY, 0.f, 0.f, 0.f, 0.f};
    for (int i0 = rg; i0 < ns; i0 += RG * kMergeBatch) {
        float4 tail[kMergeBatch];
        float Ai[kMergeBatch], Bi[kMergeBatch];
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            const int i = min(i0 + RG * j, ns - 1);
            const float *rec = base + (int64_t)i * partial_floats(D);
            tail[j] = reinterpret_cast<const float4 *>(rec + 2 * D)[0];
            Ai[j] = rec[d];
            Bi[j] = PLX ? rec[D + d] : 0.f;
        }
        // The batch's max first, then every record's weight at once: no
        // dependent chain of rescales through the records. A record past the
        // end or empty (its A, B never written) gets weight 0 and zeroed terms.
        bool ok[kMergeBatch];
        float M = st.m;
#pragma unroll
        for (int j = 0; j < kMergeBatch; ++j) {
            ok[j] = i0 + RG * j < ns && tail[j].x != -INFINITY;
            M = fmaxf(M, ok[j] ? tail[j].x : -INFINITY);
        }
        if (M != -INFINITY) {
            const float a0 = __builtin_amdgcn_exp2f(st.m - M);  // 0 while the state is empty
            st.l *= a0;
            st.S *= a0;
            st.A *= a0;
            st.B *= a0;
#pragma unroll
            for (int j = 0; j < kMergeBatch; ++j) {
                const float c = ok[j] ? __builtin_amdgcn_exp2f(tail[j].x - M) : 0.f;
                const float lj = ok[j] ? tail[j].y : 0.f;
                const float aj = ok[j] ? Ai[j] : 0.f;
                st.l = fmaf(c, lj, st.l);
                st.A = fmaf(c, aj, st.A);
                if (PLX) {
                    const float dp = tail[j].w - piv0;
                    const float sj = ok[j] ? fmaf(dp, lj, tail[j].z) : 0.f;
                    const float bj = ok[j] ? fmaf(dp, aj, Bi[j]) : 0.f;
                    st.S = fmaf(c, sj, st.S);
                    st.B = fmaf(c, bj, st.B);
                }
            }
            st.m = M;
        }
    }
    // combine the record groups (lanes dd, dd + DW, dd + 2 DW, ...)
#pragma unroll
    for (int off = DW; off < 64; off <<= 1)
        merge_into(st, __shfl_xor(st.m, off), __shfl_xor(st.l, off), __shfl_xor(st.S, off),
                   __shfl_xor(st.A, off), __shfl_xor(st.B, off));
    if (rg != 0) return;
    float val = 0.f;
    if (st.m != -INFINITY) {
        const float inv_l = 1.0f / st.l;
        val = PLX ? (st.A * (1.0f - st.S * inv_l) + st.B) * inv_l : st.A * inv_l;
    }
    TO *o = reinterpret_cast<TO *>(a.o) + ((int64_t)b * a.Hq + hq) * D + d;
    if constexpr (sizeof(TO) == 4)
        *o = val;
    else
        *o = f32_to_bf16(val);
}

template <bool PLX, bool MASK>
hipError_t launch_mfma(const DecodeArgs &a, hipStream_t stream) {
    dim3 block(64 * kDecodeWaves);
    const int G = a.Hq / a.Hkv;
    if (a.sk_parts) {
        dim3 grid(a.sk_parts, a.Hkv);
        switch (G) {
            case 1: hipLaunchKernelGGL((decode_mfma_streamk<1, PLX, MASK>), grid, block, 0, stream, a); break;
            case 2: hipLaunchKernelGGL((decode_mfma_streamk<2, PLX, MASK>), grid, block, 0, stream, a); break;
            case 3: hipLaunchKernelGGL((decode_mfma_streamk<3, PLX, MASK>), grid, block, 0, stream, a); break;
            case 4: hipLaunchKernelGGL((decode_mfma_streamk<4, PLX, MASK>), grid, block, 0, stream, a); break;
            case 5: hipLaunchKernelGGL((decode_mfma_streamk<5, PLX, MASK>), grid, block, 0, stream, a); break;
            case 6: hipLaunchKernelGGL((decode_mfma_streamk<6, PLX, MASK>), grid, block, 0, stream, a); break;
            case 7: hipLaunchKernelGGL((decode_mfma_streamk<7, PLX, MASK>), grid, block, 0, stream, a); break;
            case 8: hipLaunchKernelGGL((decode_mfma_streamk<8, PLX, MASK>), grid, block, 0, stream, a); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (G > 8) {  // groups of more than 8 query heads: chunks of 8
        dim3 grid(a.Hkv * ((G + 7) / 8), a.splits, a.B);
        hipLaunchKernelGGL((decode_mfma_bf16_d128<8, PLX, MASK, true>), grid, block, 0, stream, a);
        return hipGetLastError();
    }
    dim3 grid(a.Hkv, a.splits, a.B);
    switch (G) {
        case 1: hipLaunchKernelGGL((decode_mfma_bf16_d128<1, PLX, MASK>), grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((decode_mfma_bf16_d128<2, PLX, MASK>), grid, block, 0, stream, a); break;
        case 3: hipLaunchKernelGGL((decode_mfma_bf16_d128<3, PLX, MASK>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((decode_mfma_bf16_d128<4, PLX, MASK>), grid, block, 0, stream, a); break;
        case 5: hipLaunchKernelGGL((decode_mfma_bf16_d128<5, PLX, MASK>), grid, block, 0, stream, a); break;
        case 6: hipLaunchKernelGGL((decode_mfma_bf16_d128<6, PLX, MASK>), grid, block, 0, stream, a); break;
        case 7: hipLaunchKernelGGL((decode_mfma_bf16_d128<7, PLX, MASK>), grid, block, 0, stream, a); break;
        case 8: hipLaunchKernelGGL((decode_mfma_bf16_d128<8, PLX, MASK>), grid, block, 0, stream, a); break;
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
    dim3 grid(a.Hq, a.B, a.D / kMergeDims);
    if (a.D == 64)
        hipLaunchKernelGGL((decode_reduce<TO, 64, PLX>), grid, dim3(64), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_reduce<TO, 128, PLX>), grid, dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_split(const DecodeArgs &a, DecodePath path, int dtype, bool parallax,
                               hipStream_t stream) {
    if (path == DecodePath::Mfma) {
        if (a.block_mask)
            return parallax ? launch_mfma<true, true>(a, stream) : launch_mfma<false, true>(a, stream);
        return parallax ? launch_mfma<true, false>(a, stream) : launch_mfma<false, false>(a, stream);
    }
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
