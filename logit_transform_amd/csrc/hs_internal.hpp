// hs_internal.hpp -- kernel argument blocks and launchers shared by hs_api.hip and
// hs_kernels.hip. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hs_device.hpp"

namespace hs {

// Rows split over more than this many blocks are not generated; the workspace reserves this
// many (max, sum) pairs per row.
constexpr int kMaxChunks = 64;
// Polls (with a short sleep between them) a block makes, by default, for the other chunks'
// partials before it works them out itself.
constexpr int kExchangeSpins = 1 << 14;

// Per-row curve settings, laid out as hs_hlg_row of the public header (32 bytes).
struct RowCurve {
    float m, w, beta_t, beta_h;
    int32_t pivot;
    float pivot_offset;
    int32_t enabled;
    int32_t reserved;
};
static_assert(sizeof(RowCurve) == 32, "RowCurve layout");

// Chunk sizes (slots per lane) that have a work-queue sampling kernel: 12 and 16, where a
// pre-pass's second read of the chunks costs the most. (With 19 slots the loop around the
// item no longer fits the register budget of four waves per SIMD.)
constexpr bool queue_nv(int nv) { return nv == 12 || nv == 16; }

struct SampleArgs {
    const void *data;          // logits, row-major [B, ld]
    int64_t ld;                // row stride (elements)
    int64_t V;                 // vocabulary
    int64_t nvec;              // 16-byte vectors per row = ceil(V / epv)
    int64_t cv;                // vectors per chunk
    int32_t nchunk;            // blocks per row
    int32_t nkg;               // blocks sharing a row's draws
    int32_t kpg;               // draws per such block
    int32_t K;                 // draws per row
    int32_t aligned;           // rows are 16-byte aligned
    int32_t no_screen;         // evaluate every element exactly
    const float *T;
    const float *mu;
    const uint64_t *seed;
    const uint64_t *offset;
    int32_t *out;
    float *best_out;
    Curve curve;
    // workspace (split rows only)
    uint32_t *counters;        // [B * nkg]: blocks done per (row, draw group)
    uint64_t *keys;            // [B * K]
    float4 *partials;          // [B * part_stride]: per chunk (max, sum, u, -) in nats
    int64_t part_stride;
    float pivot_offset;        // c of the top anchor
    const RowCurve *row_curves;   // [B] per-row curve settings (pivot mode 3), else null
    const float *tau;             // [B] top-k / top-p thresholds (curve off), else null
    // split rows with the curve on: exchange the chunks' partials inside the sampling kernel
    // instead of a pre-pass (one draw group per row, a row's blocks running together: every
    // block resident at once, or the work-queue grid)
    int32_t exchange;
    int32_t spins;                // polls before a block works a missing partial out itself
    uint32_t *xslots;             // [B * part_stride * 4]: chunk partials of the exchange,
                                  // each word stored inverted (zero: not yet published)
    const uint32_t *done;         // [B] rows the threshold kernel has drawn (filters), else null
    const float *shift;           // [B] the curve's shift c per row (mass-median pivot), else null
    int32_t layout;               // word layout of the random stream: LAY_PLAIN / LAY_SCREENED
    // a resident grid taking work items from a counter (workspace): [0] next item, [1] blocks
    // done; null: one item per block
    uint32_t *queue;
    int32_t items;                // work items: B * nkg * nchunk
};

struct RowOpArgs {
    const void *data;
    int64_t ld, V;
    int32_t aligned;
    const float *mu;
    float *lse;
    float *out;
    int64_t ldo;
    Curve curve;
    float pivot_offset;   // c of the top anchor
    float *mu_out;        // the pivot of every row (op 2)
    // pivot 4 (the mass median): the shift c of row b at shift[b * shift_stride], read before
    // the kernel writes any output (it may lie in the output)
    const float *shift;
    int64_t shift_stride;
};

// Top-k / top-p threshold of every row (curve off): tau[b] = -inf keeps every token, NaN marks
// an invalid temperature or p.
struct FilterArgs {
    const void *data;
    int64_t ld, V;
    int32_t aligned;
    const float *T;
    const int32_t *top_k;   // [B] or null (0: no top-k)
    const float *top_p;     // [B] or null (1: no top-p)
    float *tau;             // [B]
    // the mass median of every row instead (T = 1, top-p 0.5, no top-k; T, top_k and top_p
    // unused): tau is the logit where the mass from the top first reaches one half
    int32_t median;
    int64_t tau_stride;     // tau of row b at tau[b * tau_stride]; 0 means 1
    // median mode with per-row settings: only rows whose record is an enabled median pivot
    const RowCurve *row_curves;
    // Drawing rows that keep few tokens in the threshold kernel (16-bit logits); done null:
    // thresholds only. done[b] = 1 marks a row drawn there (out / best_out written), 0 a row
    // left to the sampler.
    uint32_t *done;         // [B]
    int32_t *out;           // [B * K]
    float *best_out;        // [B * K] or null
    const uint64_t *seed;
    const uint64_t *offset;
    int32_t K;
    int32_t layout;         // word layout of the random stream of the draws
};
// The largest kept set, draw count and (kept tokens x draws) the threshold kernel draws itself.
constexpr int kSparseKept = 2048;
constexpr int kSparsePairs = 65536;
hipError_t launch_filter_tau(int dt, const FilterArgs &a, int grid, hipStream_t s);

// piv: the curve's pivot, 0 given per row, 1 top-anchored, 2 entropy-anchored, 3 set per row
// (a.row_curves), 4 the shift read per row (a.shift: the mass median)
// occ: when not null, the kernel's resident blocks per CU are written there instead of a launch
// the word layout comes from a.layout (LAY_PLAIN or LAY_SCREENED)
hipError_t launch_sample(int dt, bool hlg, int piv, const SampleArgs &a, int nv, int bs,
                         int grid, hipStream_t s, int *occ = nullptr);
// per family of pivots and word layout (each instantiated in a translation unit of its own)
template <int LAY>
hipError_t launch_sample_given(int dt, bool hlg, const SampleArgs &a, int nv, int bs, int grid,
                               hipStream_t s, int *occ);
template <int LAY>
hipError_t launch_sample_pivot(int dt, int piv, const SampleArgs &a, int nv, int bs, int grid,
                               hipStream_t s, int *occ);
template <int LAY>
hipError_t launch_sample_rows(int dt, const SampleArgs &a, int nv, int bs, int grid,
                              hipStream_t s, int *occ);
hipError_t launch_lse_partial(int dt, int piv, const SampleArgs &a, int bs, int grid,
                              hipStream_t s);
hipError_t launch_lse_partial_pivot(int dt, int piv, const SampleArgs &a, int bs, int grid,
                                    hipStream_t s);
hipError_t launch_lse_partial_rows(int dt, const SampleArgs &a, int bs, int grid,
                                   hipStream_t s);
// op: 0 log-sum-exp, 1 transform, 2 pivot
hipError_t launch_row_lse(int dt, int op, int piv, const RowOpArgs &a, int grid, hipStream_t s);
hipError_t launch_philox(const uint32_t *ctr, const uint32_t *key, uint32_t *out, int64_t n,
                         hipStream_t s);
hipError_t launch_stream_words(const uint64_t *seed, const uint64_t *offset, int64_t B,
                               int64_t V, int32_t k, int32_t layout, uint32_t *out,
                               hipStream_t s);
hipError_t launch_gumbel(const uint32_t *w, float *g, int64_t n, hipStream_t s);
hipError_t launch_fill_zero(void *p, int64_t nwords, hipStream_t s);

}  // namespace hs
