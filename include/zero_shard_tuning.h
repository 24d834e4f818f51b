/*
 * zero_shard_tuning.h -- test and tuning overrides of the launch shapes used
 * by libzero_shard.so.  Not part of the product interface of zero_shard.h:
 * no result depends on them (every output is bitwise the same under every
 * setting), only how the work is spread over the GPU.
 *
 * Each setting belongs to the calling host thread and applies to the calls
 * that thread makes afterwards; other threads keep their own (initially the
 * defaults).  Tests use them to run the kernels' tile loops at small sizes
 * and to compare occupancy settings; measurement scripts use them to sweep
 * launch shapes.
 */
#ifndef ZERO_SHARD_TUNING_H_
#define ZERO_SHARD_TUNING_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * zero_set_grid_cap -- cap the grid of every streaming kernel this thread
 * launches at `blocks` workgroups of 256 threads (0, or a value above the
 * default, restores the default of 2^23).  A shard with more tiles than the
 * grid has blocks is walked by each block in turn, as shards of more than
 * 2^23 tiles always are.  The sum-of-squares form of the check keeps its own
 * size-only grid, so its partial sums do not change.  Returns ZERO_OK (0).
 */
int zero_set_grid_cap(uint32_t blocks);

/*
 * zero_set_occupancy -- resident blocks per compute unit of the streaming
 * kernels this thread launches afterwards: the step (both gradient formats,
 * host or device control), the accumulates, the flag-only overflow check and
 * the exchange stand-ins (reduce and gather).  0 (the default) leaves each
 * kernel its own rule; 1 to 7 caps every launch
 * at that many; 8 or more removes the cap.  The cap is an LDS reservation the
 * kernels do not use, so results are bitwise the same under every setting.
 * Returns ZERO_OK.
 */
int zero_set_occupancy(uint32_t blocks_per_cu);

/*
 * zero_set_launch_piece -- most elements per launch of the step (both
 * gradient formats, host or device control), of the accumulates and of the
 * flag-only overflow check that this thread enqueues afterwards.  A longer shard goes out as consecutive launches
 * over whole tiles, back to back on the same stream; elementwise work, so
 * results are bitwise the same under every setting.  0 (the default) restores
 * each kernel's own rule (the step and the accumulate with the fused check
 * of a later micro-batch: launches of 2^27 elements once a shard holds two of
 * them; the other accumulates and the check: one launch).  A value below one tile
 * means one tile; UINT64_MAX means one launch whatever the size.  Returns
 * ZERO_OK.
 */
int zero_set_launch_piece(uint64_t elements);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_SHARD_TUNING_H_ */
