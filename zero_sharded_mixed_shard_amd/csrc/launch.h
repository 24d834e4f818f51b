// Internal interface between the C-ABI layer (api.cpp) and the gfx950
// kernels (shard_kernels.hip).  Not installed; callers use zero_shard.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "zero_shard.h"

namespace zs {

// Per-call scalars of the Adam step, all formed on the host.
//
// Three of the step's four FP32 divisions divide by per-call constants: the
// loss scale S and the bias corrections bc1, bc2.  The kernels form those
// quotients without a division, bit for bit the same:
//  - S a power of two whose reciprocal is a normal FP32 number: g * (1/S) is
//    the same real number as g / S, rounded once (inv_scale).
//  - any other divisor d: (float)((double)a * RN64(1/d)), with a true
//    division wherever that result is below 2^-125 in magnitude and a != 0
//    (rcp_scale, rcp_bc1, rcp_bc2; the argument is beside the kernels).
struct AdamScalars {
    float loss_scale;  // S: gradients are divided by it
    float inv_scale;   // 1/S (exact) when scale_pow2, else unused
    int scale_pow2;    // S = 2^k with -126 <= k <= 126
    float lr;
    float beta1;
    float beta2;
    float omb1;        // 1 - beta1 (FP32 subtraction)
    float omb2;        // 1 - beta2 (FP32 subtraction)
    float eps;
    float bc1;         // 1 - beta1^t, FP64 then rounded to FP32
    float bc2;         // 1 - beta2^t, FP64 then rounded to FP32
    float decay;       // 1 - lr * weight_decay (two FP32 operations)
    double rcp_scale;  // RN64(1 / S)
    double rcp_bc1;    // RN64(1 / bc1)
    double rcp_bc2;    // RN64(1 / bc2)
};

// S = 2^k with a normal FP32 reciprocal: biased exponent 1..253, no
// significand bits.
inline bool scale_is_pow2(float S) {
    uint32_t b;
    __builtin_memcpy(&b, &S, 4);
    const uint32_t e = (b >> 23) & 0xffu;
    return (b & 0x807fffffu) == 0 && e >= 1 && e <= 253;
}

// Largest grid of the streaming kernels, in 256-thread blocks: one tile per
// block measured fastest, and 2^23 blocks keep the grid below 2^32 threads.
// Larger shards loop over tiles.
constexpr uint64_t kMaxBlocks = 1ull << 23;

// The grid cap in force for the calling thread: kMaxBlocks, or the lower cap
// that thread set with zero_tuning_set_grid_cap (tests use it to run the tile
// loops at small sizes).
uint64_t max_blocks();

// What the launchers need to know of the current device, and the calling
// thread's overrides of the launch shape.
struct DeviceProps {
    int cus;              // compute units
    int lds_per_cu;       // LDS bytes of one compute unit
    int lds_per_block;    // largest LDS allocation of one workgroup
    int occupancy;        // resident blocks per CU of the streaming kernels: 0 = each
                          // kernel's own rule, 1-7 this cap, 8 no cap
    uint64_t piece;       // most elements per launch of the step and the accumulates:
                          // 0 = each kernel's own rule
};

// Dynamic LDS to reserve, unused by the kernel, so that at most per_cu blocks
// of 256 threads are resident on a CU (0: no reservation; 8 or more is the
// kernels' own limit).  One more block than per_cu would not fit.
inline size_t cap_lds_bytes(int per_cu, const DeviceProps &dev) {
    if (per_cu <= 0 || per_cu >= 8 || dev.lds_per_cu <= 0) return 0;
    const size_t bytes = static_cast<size_t>(dev.lds_per_cu) / (per_cu + 1) + 256;
    return bytes <= static_cast<size_t>(dev.lds_per_block) ? bytes : 0;
}

// The calling thread's override of resident blocks per CU, if any, else the
// kernel's own rule.
inline int per_cu_or(int rule, const DeviceProps &dev) {
    return dev.occupancy != 0 ? dev.occupancy : rule;
}

// Consecutive ranges of at most piece_tiles whole tiles of a shard, each
// enqueued by launch(offset, count, head, n_tiles) over the views advanced by
// offset elements: the first range keeps the shard's head, the last one its
// ragged rest, and every later range starts head + a multiple of the tile in,
// so it keeps the shard's alignment.  piece_tiles == 0, or a shard of at most
// piece_tiles tiles: one launch over everything.  Stops at the first error.
template <typename F>
hipError_t by_pieces(uint64_t count, uint32_t head, uint64_t n_tiles, uint64_t tile,
                     uint64_t piece_tiles, F &&launch) {
    if (piece_tiles == 0 || n_tiles <= piece_tiles) return launch(0, count, head, n_tiles);
    for (uint64_t t0 = 0; t0 < n_tiles; t0 += piece_tiles) {
        const uint64_t nt = n_tiles - t0 < piece_tiles ? n_tiles - t0 : piece_tiles;
        const uint64_t off = t0 == 0 ? 0 : head + t0 * tile;
        const uint32_t h = t0 == 0 ? head : 0;
        const uint64_t cnt = t0 + nt == n_tiles ? count - off : h + nt * tile;
        const hipError_t e = launch(off, cnt, h, nt);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Whole tiles per launch of a shard of n_tiles tiles: the thread's override
// as it stands, else the kernel's rule (elements per piece; 0: one launch),
// which splits only a shard that holds at least two whole pieces.
inline uint64_t piece_tiles(uint64_t rule, uint64_t tile, uint64_t n_tiles,
                            const DeviceProps &dev) {
    if (dev.piece != 0) return dev.piece < tile ? 1 : dev.piece / tile;
    const uint64_t per = rule / tile;
    return per != 0 && n_tiles >= 2 * per ? per : 0;
}

// Enqueue the Adam step over `count` elements of five shard views.  The
// caller has validated every argument; count > 0.  flag (nullable): skip if
// set.  ctl (nullable): skip unless ctl->apply, and take S, bc1, bc2 from it.
hipError_t launch_adam_step(int dtype, uint16_t *w16, const uint16_t *g16, float *master, float *m,
                            float *v, uint64_t count, const AdamScalars &s, const int32_t *flag,
                            const zero_device_ctl *ctl, const DeviceProps &dev,
                            hipStream_t stream);

// Enqueue the unscale + overflow check of `count` gradients (count may be 0:
// then only the outputs are cleared).  partials holds ZERO_SUMSQ_PARTIALS
// doubles when sumsq is non-null.  loss_scale_dev (nullable) replaces
// loss_scale with a value read on the device.
hipError_t launch_overflow_check(int dtype, const uint16_t *g16, uint64_t count, float loss_scale,
                                 const float *loss_scale_dev, int32_t *flag, float *sumsq,
                                 double *partials, const DeviceProps &dev, hipStream_t stream);

// launch_overflow_check with the partial sums in the library's fixed device
// array (ZERO_SUMSQ_PARTIALS doubles per device, shared by every such call on
// the device) instead of caller memory; no allocation.  The sum-of-squares
// grid never exceeds the array (scratch_partials_capacity() partials).
hipError_t launch_overflow_check_noalloc(int dtype, const uint16_t *g16, uint64_t count,
                                         float loss_scale, int32_t *flag, float *sumsq,
                                         const DeviceProps &dev, hipStream_t stream);
int scratch_partials_capacity();
// Partial sums the sum-of-squares check of `count` gradients at `g` writes
// (dtype 0/1: 16-bit, 2: FP32).
uint64_t sumsq_partials_needed(int dtype, const void *g, uint64_t count);

// The step with FP32 gradients (dtype: the working weights' format); flag and
// ctl as for launch_adam_step.
hipError_t launch_adam_step_g32(int dtype, uint16_t *w16, const float *g32, float *master,
                                float *m, float *v, uint64_t count, const AdamScalars &s,
                                const int32_t *flag, const zero_device_ctl *ctl,
                                const DeviceProps &dev, hipStream_t stream);

// acc = float(g16) (first) or acc + float(g16), in FP32; count > 0.
hipError_t launch_grad_accumulate(int dtype, float *acc, const uint16_t *g16, uint64_t count,
                                  bool first, const DeviceProps &dev, hipStream_t stream);

// The same accumulate, raising *flag (cleared first, also when count == 0)
// iff some written acc[i] / S is not finite -- the check over FP32 gradients
// of the result, fused into the pass that writes it.  loss_scale_dev
// (nullable) replaces loss_scale with a value read on the device.
hipError_t launch_grad_accumulate_check(int dtype, float *acc, const uint16_t *g16,
                                        uint64_t count, bool first, float loss_scale,
                                        const float *loss_scale_dev, int32_t *flag,
                                        const DeviceProps &dev, hipStream_t stream);

// The check over FP32 gradients (count may be 0: only the outputs are cleared);
// loss_scale_dev as for launch_overflow_check.
hipError_t launch_overflow_check_g32(const float *g32, uint64_t count, float loss_scale,
                                     const float *loss_scale_dev, int32_t *flag, float *sumsq,
                                     double *partials, const DeviceProps &dev,
                                     hipStream_t stream);

// Views of up to ZERO_MAX_LOCAL_RANKS replicas or shards, passed by value.
constexpr uint32_t kMaxLocalRanks = 64;  // == ZERO_MAX_LOCAL_RANKS
struct ReplicaSet {
    const void *p[kMaxLocalRanks];        // replica k advanced to the rank's first element
};
struct GatherSet {
    const void *p[kMaxLocalRanks];        // shard k (shard-local)
    uint64_t count[kMaxLocalRanks];       // real elements of shard k
    uint32_t head[kMaxLocalRanks];        // filled by the launcher
    uint32_t vec[kMaxLocalRanks];         // filled by the launcher
};

// The overflow check fused into the reduce: with flag set, *flag is cleared
// first (also when count == 0) and raised iff some written out[i] / S is not
// finite.  flag == nullptr: the plain reduce.
struct ReduceCheck {
    float loss_scale;             // S, unless loss_scale_dev is set
    const float *loss_scale_dev;  // S read on the device, or null
    int32_t *flag;                // the flag, or null
};

// out[i] = FP32 sum over k < n of in.p[k][i], rounded to out_fmt (0 FP16,
// 1 BF16, 2 FP32), i < count; count > 0 unless chk.flag is set.
hipError_t launch_reduce_shard(void *out, int out_fmt, const ReplicaSet &in, int in_fmt,
                               uint32_t n, uint64_t count, const ReduceCheck &chk,
                               const DeviceProps &dev, hipStream_t stream);

// Enqueue a one-lane kernel that sets *flag = 0 (a kernel rather than a memset,
// so that a captured graph replays it correctly).
hipError_t launch_clear_flag(int32_t *flag, hipStream_t stream);

// full[k*shard + i] = set.p[k][i] for i < set.count[k], k < n.
hipError_t launch_gather_shards(void *full, int elem_bytes, GatherSet &set, uint32_t n,
                                uint64_t shard, uint64_t max_count, const DeviceProps &dev,
                                hipStream_t stream);

// Enqueue the one-lane skip-or-apply decision on a device control block.
hipError_t launch_scaler_decide(zero_device_ctl *ctl, const float *bias, uint64_t t_first,
                                uint32_t len, hipStream_t stream);

}  // namespace zs
