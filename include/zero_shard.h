/*
 * zero_shard.h -- C ABI of the ZeRO-partitioned mixed-precision Adam step
 * that one data-parallel rank runs on its 1/N shard of a flat parameter
 * buffer, on an MI355X (gfx950).
 *
 * Model state per parameter is 2 + 2 + 12 bytes: 16-bit working weights
 * (w16), 16-bit gradients (g16), and FP32 master weights, first moment and
 * second moment (master, m, v) -- "Training models too big for one GPU:
 * ZeRO & FSDP", "The memory bill: 16 bytes per parameter".  Rank r owns
 * chunk r of the flat buffer, all chunks the same size, and updates only
 * that chunk ("Training models too big for one GPU", "ZeRO stages 1, 2 and
 * 3"; "ZeRO memory math" (tm_zero_math), "Stage 1 - P_os").
 *
 * Conventions shared by every entry point
 *   - Return 0 on success, a negative ZERO_E* code on error; no C++
 *     exception ever crosses this boundary.  zero_strerror() explains a code.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     keeps a pointer past the call.
 *   - Device pointers are SHARD VIEWS: element 0 is the first element of
 *     rank r's range, i.e. either base + r*S into a full flat buffer (the
 *     replicated arrays of ZeRO-1/2) or a shard-local allocation (ZeRO-3).
 *     Exactly elements [0, count) of each view are read or written, where
 *     count is the layout's count for (psi, n, rank).  The padding of a short
 *     last shard and anything past count are never touched.
 *   - The views of one call may not overlap one another, nor the flag,
 *     sum-of-squares, partial-sum or control-block memory of the call (the
 *     kernels stream them as independent arrays); overlaps are rejected with
 *     ZERO_EINVAL.  Read-only views may repeat (the same replica passed twice
 *     to zero_reduce_shard); zero_reduce_shard's output may be exactly rank
 *     r's chunk of one replica in the same format (an in-place
 *     reduce-scatter), and a shard
 *     passed to zero_gather_shards may sit exactly at its place in the full
 *     buffer (an in-place all-gather).
 *   - Any element-aligned pointer is accepted (4 bytes for FP32 arrays, 2
 *     for 16-bit ones).  The kernels do a head of h < 64 elements one at a
 *     time, h bringing the FP32 master view (and, where one head does both,
 *     the 16-bit views) to a 128-byte line, and stream
 *     the rest in vectors when at element h every FP32 view is 16-byte and
 *     every 16-bit view 8-byte aligned.  That holds whenever all views sit at
 *     the same element offset into 16-byte-aligned buffers.  Otherwise a
 *     slower element-wise kernel gives the same results.
 *   - All device work is enqueued on `stream` (a hipStream_t; 0 = the null
 *     stream) of the current HIP device, and the call returns without
 *     synchronising.  A call may enqueue several kernel launches: the step
 *     of a shard of 2^28 elements or more, for one, goes out as consecutive
 *     launches of 2^27 elements (a HIP graph captured from it holds one node
 *     per launch).  Argument errors are found before anything is enqueued;
 *     if a launch itself fails (ZERO_EHIP), launches before it in the same
 *     call may already be enqueued, and the arrays they write are then in
 *     an unspecified state.  Calls are thread-safe and stateless: the only
 *     mutable state the library keeps between calls is a per-device cache of
 *     device properties (compute units, LDS sizes), written once with the
 *     values the runtime reports.  (zero_shard_tuning.h declares test and tuning
 *     overrides of launch shapes; they are per thread and change no result.)
 */
#ifndef ZERO_SHARD_H_
#define ZERO_SHARD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Format of the 16-bit gradients and working weights (one for both).
 * ZERO_F32 is accepted only by the functions that say so. */
typedef enum { ZERO_F16 = 0, ZERO_BF16 = 1, ZERO_F32 = 2 } zero_dtype;

#define ZERO_OK 0
#define ZERO_EINVAL (-1) /* an argument is out of its documented domain */
#define ZERO_EDTYPE (-2) /* dt is not a zero_dtype value */
#define ZERO_EHIP (-3)   /* the HIP runtime reported an error (see zero_strerror) */
#define ZERO_EIO (-5)    /* a checkpoint file could not be opened, written or read */
#define ZERO_ECORRUPT (-6) /* a checkpoint file failed its header, size or hash check */

/* Largest flat buffer accepted: keeps every byte count below 2^64. */
#define ZERO_MAX_PSI (1ull << 56)

/* Doubles the caller provides in `d_partials` when asking for a sum of squares. */
#define ZERO_SUMSQ_PARTIALS 4096

/* Shard layout of one rank (all counts in elements unless named bytes_*). */
typedef struct {
    uint64_t psi;          /* parameters in the flat buffer */
    uint64_t shard;        /* S = ceil(psi / n): every chunk's size, padding included */
    uint64_t offset;       /* rank * S: flat index of the chunk's first element */
    uint64_t count;        /* real elements in the chunk: clamp(psi - offset, 0, S) */
    uint64_t pad;          /* S - count: padding at the tail of the flat buffer */
    uint64_t padded_total; /* n * S */
    uint32_t n;            /* data-parallel ranks */
    uint32_t rank;
    /* Model-state bytes held by one rank ("ZeRO stages 1, 2 and 3" on the
     * first page; "The three stages of ZeRO" on "Stop Replicating What You
     * Can Shard"; "Stage 3: divide everything by N" on "ZeRO Stage 3 Math").
     * Sharded terms hold S elements; replicated terms hold the padded flat
     * buffer of n*S elements.  They equal 16psi, 4psi + 12psi/n,
     * 2psi + 14psi/n and 16psi/n exactly when n divides psi. */
    uint64_t bytes_dp;     /* plain data parallel: 16 * psi */
    uint64_t bytes_z1;     /* optimizer states sharded: 4 * n*S + 12 * S */
    uint64_t bytes_z2;     /* gradients sharded too:    2 * n*S + 14 * S */
    uint64_t bytes_z3;     /* weights sharded too:      16 * S */
} zero_layout;

/*
 * zero_shard_layout -- where rank `rank` of `n` sits in a flat buffer of
 * `psi` parameters, and what each ZeRO stage costs it in bytes.
 * Chunk i of an equally chunked buffer belongs to rank i ("Training models
 * too big for one GPU", "Data parallelism and the all-reduce"; "ZeRO memory
 * math", "Stage 1 - P_os").  When n does not divide psi the chunk size is
 * ceil(psi/n) and the padding sits at the tail; trailing ranks may own
 * fewer, or zero, real elements.
 *   Host only: no device access, no allocation.
 *   Errors: ZERO_EINVAL if out is NULL, psi == 0, psi > ZERO_MAX_PSI,
 *   n == 0 or rank >= n (out is then left untouched).
 */
int zero_shard_layout(uint64_t psi, uint32_t n, uint32_t rank, zero_layout *out);

/*
 * zero_overflow_check -- unscale this rank's gradients by the loss scale and
 * report whether any is +-inf or NaN, so that the step can be skipped
 * ("Training models too big for one GPU", "Mixed-precision training": the
 * gradients are divided by S before the update; frameworks pick S
 * dynamically and skip a step on overflow).
 *   g16          device, shard view of `count` 16-bit gradients of format dt.
 *   loss_scale   S > 0 and finite; each gradient is tested as float(g)/S.
 *   d_found_inf  device int32, written with 0 or 1 (1 iff some unscaled
 *                gradient in [0, count) is not finite).  Required.
 *   d_sumsq      device float or NULL.  If given, receives the sum over the
 *                shard of the unscaled gradients' squares, accumulated in
 *                FP64 in a fixed order (so repeatable bit for bit) and
 *                rounded to FP32: the local term of a gradient norm.
 *   d_partials   device buffer of ZERO_SUMSQ_PARTIALS doubles, scratch for
 *                d_sumsq (the per-block partial sums of the two-pass sum: the
 *                library allocates nothing, so they live in caller memory);
 *                required iff d_sumsq is given, otherwise ignored.
 *   An empty rank (count == 0) still writes 0 to d_found_inf (and d_sumsq).
 *   Errors: ZERO_EDTYPE for a bad dt; ZERO_EINVAL for bad layout arguments,
 *   a NULL d_found_inf, a NULL g16 with count > 0, a NULL d_partials with a
 *   d_sumsq, a misaligned pointer, or S not positive and finite;
 *   ZERO_EHIP if a launch fails.
 */
int zero_overflow_check(const void *g16, zero_dtype dt, uint64_t psi, uint32_t n, uint32_t rank,
                        float loss_scale, int32_t *d_found_inf, float *d_sumsq,
                        double *d_partials, void *stream);

/*
 * zero_overflow_check_noalloc -- zero_overflow_check for callers that cannot
 * allocate device memory or pass a workspace: code being captured into a HIP
 * graph, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, outputs and errors, without d_partials: the partial sums of the
 * sum of squares live in a fixed array of ZERO_SUMSQ_PARTIALS doubles (32 KiB)
 * that the library holds on each device it runs on until the process ends.
 * The call allocates nothing.  Every call on a device shares that device's
 * array, so calls that overlap in time on one device (different streams, or
 * threads racing on one stream) corrupt each other's sums; calls enqueued one
 * after another on a stream are safe (each writes the partials it reads).
 * Without d_sumsq the array is not used.
 *   Errors: as zero_overflow_check, and ZERO_EINVAL if the sum of squares
 *   would need more partial sums than the array holds (never for a shard the
 *   layout accepts: that grid has at most 1792 blocks).
 */
int zero_overflow_check_noalloc(const void *g16, zero_dtype dt, uint64_t psi, uint32_t n,
                                uint32_t rank, float loss_scale, int32_t *d_found_inf,
                                float *d_sumsq, void *stream);

/*
 * zero_adam_step -- one Adam (weight_decay == 0) or AdamW step over this
 * rank's shard, elementwise, each operation one FP32 rounding to nearest
 * even, no contraction:
 *     g  = float(g16) / loss_scale
 *     p  = master * (1 - lr*weight_decay)            decoupled weight decay
 *     m  = beta1*m + (1 - beta1)*g
 *     v  = beta2*v + (1 - beta2)*(g*g)
 *     m^ = m / (1 - beta1^step),   v^ = v / (1 - beta2^step)
 *     p  = p - (lr * m^) / (sqrt(v^) + eps)         eps outside the root
 *     master = p;  w16 = p rounded to nearest-even in format dt
 * ("Training models too big for one GPU", "Adam, and why it's expensive":
 * the moment, bias-correction and update equations; "Mixed-precision
 * training": the FP32 master copy is updated and rounded to 16 bits for the
 * next forward pass.)  1 - beta^step is formed on the host in FP64 and
 * rounded once to FP32; 1 - beta, and 1 - lr*weight_decay, are FP32
 * operations.  Reads 2 + 4 + 4 + 4 and writes 4 + 4 + 4 + 2 bytes per
 * element: 28 bytes.
 *   w16, g16     device, shard views of 16-bit working weights (written) and
 *                gradients (read), both of format dt.
 *   master, m, v device, shard views of FP32 state, read and written.
 *   step         t >= 1: the number of updates applied so far, this one
 *                included (a skipped step does not count).
 *   d_found_inf  device int32 or NULL.  If given and non-zero when the
 *                kernel runs, nothing is written: the step is skipped on the
 *                device without a host round trip.
 *   An empty rank (count == 0) returns ZERO_OK without touching the device.
 *   Errors: ZERO_EDTYPE for a bad dt; ZERO_EINVAL for bad layout arguments,
 *   step == 0, loss_scale not positive and finite, beta1 or beta2 outside
 *   [0, 1), eps negative or not finite, lr or weight_decay not finite, a
 *   NULL or misaligned array pointer with count > 0 (nothing enqueued);
 *   ZERO_EHIP if a launch fails (see the note on launches above).
 */
int zero_adam_step(void *w16, const void *g16, float *master, float *m, float *v, zero_dtype dt,
                   uint64_t psi, uint32_t n, uint32_t rank, float lr, float beta1, float beta2,
                   float eps, float weight_decay, uint64_t step, float loss_scale,
                   const int32_t *d_found_inf, void *stream);

/* Dynamic loss scale and applied-update counter of one training run; the
 * caller owns it (host memory) and passes it to every decision. */
typedef struct {
    float loss_scale;         /* S in force for the next check and step: > 0, finite */
    uint32_t growth_interval; /* clean steps in a row before S doubles; 0 = never */
    uint64_t step;            /* updates applied so far (t of the last applied update) */
    uint64_t clean_steps;     /* clean steps since the last overflow or doubling */
} zero_scaler;

/*
 * zero_scaler_update -- the skip-or-apply decision between the overflow
 * check and the step ("Training models too big for one GPU",
 * "Mixed-precision training": S is picked dynamically and a step with an
 * overflow is skipped).
 *   found_inf != 0: *apply = 0; S halves; step and the update are skipped;
 *                   clean_steps = 0.
 *   found_inf == 0: *apply = 1; step += 1 (the update about to run is number
 *                   `step`); clean_steps += 1, and when it reaches a non-zero
 *                   growth_interval S doubles (unless 2S would overflow) and
 *                   clean_steps = 0.
 * The update, when applied, must unscale with the S in force BEFORE this
 * call: the gradients were produced with it.  In data parallelism found_inf
 * is the OR of every rank's flag.
 *   Host only.  Errors: ZERO_EINVAL if s or apply is NULL or s->loss_scale is
 *   not positive and finite (s is then left untouched).
 */
int zero_scaler_update(zero_scaler *s, int32_t found_inf, int32_t *apply);

/* ---------------------------------------------------------------------------
 * FP32 gradients.  Accumulating many 16-bit micro-batch gradients in a 16-bit
 * buffer loses the small contributions, so the accumulator is FP32 and the
 * reduction and the step read FP32 gradients ("How far does splitting the
 * batch get you?", "What does gradient accumulation actually buy?").
 * ------------------------------------------------------------------------- */

/*
 * zero_grad_accumulate -- acc[i] = float(g16[i]) when `first` is non-zero,
 * acc[i] + float(g16[i]) (one FP32 addition) otherwise, for i in [0, count):
 * one micro-batch into the FP32 accumulator of this rank's shard.  10 bytes
 * of traffic per element (6 for the first micro-batch).
 *   acc  device, FP32 shard view (4-byte aligned), read unless first, written.
 *   g16  device, 16-bit shard view of format dt.
 *   Errors: ZERO_EDTYPE; ZERO_EINVAL for bad layout arguments or a NULL or
 *   misaligned pointer with count > 0; ZERO_EHIP.  count == 0: no-op.
 */
int zero_grad_accumulate(float *acc, const void *g16, zero_dtype dt, uint64_t psi, uint32_t n,
                         uint32_t rank, int32_t first, void *stream);

/*
 * zero_grad_accumulate_check -- zero_grad_accumulate for the last
 * micro-batch of a step, with the overflow check over the FP32 gradients it
 * writes fused in: *d_found_inf becomes 1 iff some written acc[i] / S is
 * not finite (the flag zero_overflow_check_g32 would give on the result, no
 * sum of squares), without reading the accumulator again.
 *   loss_scale   S > 0 and finite.
 *   d_found_inf  device int32, cleared on `stream` first (also for an empty
 *                rank), may not overlap acc or g16.
 *   Other arguments and errors as for zero_grad_accumulate; ZERO_EINVAL also
 *   for a NULL or misaligned d_found_inf or a bad S.
 */
int zero_grad_accumulate_check(float *acc, const void *g16, zero_dtype dt, uint64_t psi,
                               uint32_t n, uint32_t rank, int32_t first, float loss_scale,
                               int32_t *d_found_inf, void *stream);

/*
 * zero_overflow_check_g32 -- zero_overflow_check over FP32 gradients
 * (4 bytes per element); same outputs, scratch and errors.
 */
int zero_overflow_check_g32(const float *g32, uint64_t psi, uint32_t n, uint32_t rank,
                            float loss_scale, int32_t *d_found_inf, float *d_sumsq,
                            double *d_partials, void *stream);

/*
 * zero_adam_step_g32 -- zero_adam_step with FP32 gradients: g = g32 / S, the
 * rest identical; dt is the working weights' format.  30 bytes per element.
 */
int zero_adam_step_g32(void *w16, const float *g32, float *master, float *m, float *v,
                       zero_dtype dt, uint64_t psi, uint32_t n, uint32_t rank, float lr,
                       float beta1, float beta2, float eps, float weight_decay, uint64_t step,
                       float loss_scale, const int32_t *d_found_inf, void *stream);

/* ---------------------------------------------------------------------------
 * The exchanges on either side of the step, on one GPU.  A reduce-scatter
 * leaves rank i with the SUM over ranks of chunk i of the gradients; an
 * all-gather copies every rank's finished chunk to all ("Training models too
 * big for one GPU", "Data parallelism and the all-reduce").  These stand-ins
 * take the n replicas or shards as views on one device, so the sharded path
 * can be exercised end to end without a second GPU.
 * ------------------------------------------------------------------------- */

#define ZERO_MAX_LOCAL_RANKS 64 /* most replicas / shards one call takes */

/*
 * zero_reduce_shard -- rank `rank`'s chunk of the element-wise sum of n
 * replica buffers: out[i] = sum over k = 0..n-1 of replica_k[offset + i],
 * i < count, accumulated in FP32 in rank order and rounded once to out_dt.
 *   replicas  HOST array of n device pointers; replica k is a full flat buffer
 *             of at least psi elements of format in_dt (FP16, BF16 or FP32).
 *   out       device, shard view of count elements of format out_dt.
 *   Reads n x (2 or 4) bytes and writes 2 or 4 bytes per element.
 *   Errors: ZERO_EDTYPE for a format outside FP16/BF16/FP32; ZERO_EINVAL for
 *   bad layout arguments, n > ZERO_MAX_LOCAL_RANKS, a NULL or misaligned
 *   pointer with count > 0; ZERO_EHIP.  count == 0: no-op.
 */
int zero_reduce_shard(void *out, zero_dtype out_dt, const void *const *replicas,
                      zero_dtype in_dt, uint64_t psi, uint32_t n, uint32_t rank, void *stream);

/*
 * zero_reduce_shard_check -- zero_reduce_shard with the unscale + overflow
 * check of its result fused in ("Training models too big for one GPU: ZeRO &
 * FSDP", "Data parallelism and the all-reduce": each rank's chunk is the sum
 * over ranks; "Mixed-precision training": the gradients are divided by S and
 * the step is skipped if any is inf or NaN).  The reduced chunk is the one
 * zero_reduce_shard writes, bit for bit, and *d_found_inf becomes 1 iff some
 * written out[i] / loss_scale is not finite, else 0: the flag that
 * zero_overflow_check (16-bit out_dt) or zero_overflow_check_g32 (FP32) would
 * give on out, without reading it again.  For a ZeRO-2/3 rank whose
 * gradients arrive by a reduce-scatter.
 *   loss_scale   S > 0, finite.
 *   d_found_inf  device int32, written (cleared first, also for an empty
 *                rank); it may not overlap out or a replica's chunk.
 *   Errors: those of zero_reduce_shard, and ZERO_EINVAL for a bad loss_scale
 *   or a NULL, misaligned or overlapping d_found_inf.
 */
int zero_reduce_shard_check(void *out, zero_dtype out_dt, const void *const *replicas,
                            zero_dtype in_dt, uint64_t psi, uint32_t n, uint32_t rank,
                            float loss_scale, int32_t *d_found_inf, void *stream);

/*
 * zero_gather_shards -- full[k*S + i] = shard_k[i] for every rank k < n and
 * i < count(k): the flat buffer from its n shards.  Elements of full at
 * psi and beyond (the padding) are not written.
 *   full    device, flat buffer of at least psi elements of format dt.
 *   shards  HOST array of n device pointers (NULL allowed for empty ranks).
 *   Errors: ZERO_EDTYPE; ZERO_EINVAL for bad layout arguments,
 *   n > ZERO_MAX_LOCAL_RANKS, a NULL or misaligned pointer; ZERO_EHIP.
 */
int zero_gather_shards(void *full, const void *const *shards, zero_dtype dt, uint64_t psi,
                       uint32_t n, void *stream);

/* Communication of one step per rank (see zero_comm_volume). */
typedef struct {
    uint32_t collectives; /* 2 (reduce-scatter + all-gather) or 3 at stage 3 */
    uint32_t ring_hops;   /* sequential hops of those collectives on a ring: collectives*(n-1) */
    uint64_t elements;    /* collectives * psi: 2 psi at stages 0-2, 3 psi at stage 3 */
    uint64_t wire_bytes;  /* elements * elem_bytes */
    uint64_t ring_bytes;  /* bytes a rank sends on a ring: collectives * (n-1) * S * elem_bytes */
} zero_comm;

/*
 * zero_comm_volume -- what one data-parallel step moves per rank at ZeRO
 * stage 0 (plain data parallelism) to 3: 2 psi elements at stages 0-2, 3 psi
 * at stage 3 ("How far does splitting the batch get you?", "What does each
 * stage cost on the wire?"; "Stop Replicating What You Can Shard", FSDP
 * communication), and what a ring sends for it: (d-1)/d of each message in
 * d-1 hops ("Why does the all-reduce not get more expensive with more
 * ranks?").  Host only.  Errors: ZERO_EINVAL for bad layout arguments,
 * stage > 3, elem_bytes outside 1..8 or a NULL out.
 */
int zero_comm_volume(uint64_t psi, uint32_t n, uint32_t stage, uint32_t elem_bytes,
                     zero_comm *out);

/*
 * zero_peak_memory -- ZeRO-3 peak bytes per rank: the persistent 16 psi / N
 * shard (padded: 16 S) plus units_resident gathered units of unit_params
 * 16-bit weights plus activation_bytes ("ZeRO Stage 3 Math", "Peak transient
 * memory").  Host only.  Errors: ZERO_EINVAL for bad layout arguments,
 * unit_params > psi, overflow or a NULL out_bytes.
 */
int zero_peak_memory(uint64_t psi, uint32_t n, uint64_t unit_params, uint32_t units_resident,
                     uint64_t activation_bytes, uint64_t *out_bytes);

/* ---------------------------------------------------------------------------
 * Device-resident control: the same check -> decision -> step sequence with
 * the loss scale, the step counter and the flag kept in device memory, so a
 * training loop can enqueue step after step without reading anything back.
 * ------------------------------------------------------------------------- */

/* Control block in device memory.  The caller allocates sizeof(zero_device_ctl)
 * bytes (4-byte aligned) and initialises `scaler` by copying a host struct in;
 * the other fields are outputs. */
typedef struct {
    zero_scaler scaler;    /* as for zero_scaler_update: S in force, counters */
    int32_t found_inf;     /* flag of the last zero_overflow_check_dev (0/1) */
    int32_t apply;         /* 1 if the last zero_scaler_update_dev applied the update */
    float loss_scale_used; /* S that the applied update unscales with */
    float bc1;             /* 1 - beta1^t of the applied update */
    float bc2;             /* 1 - beta2^t of the applied update */
    int32_t status;        /* 0; ZERO_ERANGE if the bias table missed t (update skipped) */
    double rcp_loss_scale; /* 1 / loss_scale_used, FP64 correctly rounded */
    double rcp_bc1;        /* 1 / bc1, FP64 correctly rounded */
    double rcp_bc2;        /* 1 / bc2, FP64 correctly rounded */
} zero_device_ctl;

#define ZERO_ERANGE (-4) /* written to zero_device_ctl.status: t outside the bias table */

/*
 * zero_bias_corrections -- host helper: bc1[k] = 1 - beta1^(t_first + k) and
 * bc2[k] = 1 - beta2^(t_first + k) for k < len, each formed in FP64 and
 * rounded once to FP32, exactly as zero_adam_step forms them ("Training
 * models too big for one GPU", "Adam, and why it's expensive": bias-corrected
 * moments).  The device path reads them from a table because the host's libm
 * fixes their last bit.
 *   out  host, 2*len floats: bc1[0..len) then bc2[0..len).
 *   Errors: ZERO_EINVAL if out is NULL, len == 0, t_first == 0, or a beta
 *   is outside [0, 1).
 */
int zero_bias_corrections(float beta1, float beta2, uint64_t t_first, uint32_t len, float *out);

/*
 * zero_overflow_check_dev -- zero_overflow_check with S read from
 * d_ctl->scaler.loss_scale on the device; writes d_ctl->found_inf.  In data
 * parallelism, OR (MAX all-reduce) every rank's found_inf before the decision.
 *   Errors: as zero_overflow_check (d_ctl replaces loss_scale and d_found_inf;
 *   S is not checked on the host, a non-positive S on the device reads as
 *   overflow).
 */
int zero_overflow_check_dev(const void *g16, zero_dtype dt, uint64_t psi, uint32_t n,
                            uint32_t rank, zero_device_ctl *d_ctl, void *stream);

/*
 * zero_scaler_update_dev -- zero_scaler_update on the device (one thread):
 * reads found_inf, updates scaler, sets apply, and for an applied update
 * records loss_scale_used (S before the decision) and bc1, bc2 for the new
 * step t from the table (entries for t_first .. t_first + len - 1, as
 * zero_bias_corrections writes them), with their FP64 reciprocals (the step
 * forms its quotients by those three from them, with the same result as the
 * FP32 division).  If t falls outside the table the
 * update is skipped, status = ZERO_ERANGE and scaler is left as it was.
 *   d_bias  device, 2*len floats.
 *   Errors: ZERO_EINVAL for a NULL or misaligned pointer, len == 0 or
 *   t_first == 0; ZERO_EHIP if the launch fails.
 */
int zero_scaler_update_dev(zero_device_ctl *d_ctl, const float *d_bias, uint64_t t_first,
                           uint32_t len, void *stream);

/*
 * zero_adam_step_dev -- zero_adam_step with loss_scale, 1 - beta1^t and
 * 1 - beta2^t read from d_ctl on the device; writes nothing unless
 * d_ctl->apply is set.  The other arguments are as for zero_adam_step.
 */
int zero_adam_step_dev(void *w16, const void *g16, float *master, float *m, float *v,
                       zero_dtype dt, uint64_t psi, uint32_t n, uint32_t rank, float lr,
                       float beta1, float beta2, float eps, float weight_decay,
                       const zero_device_ctl *d_ctl, void *stream);

/*
 * zero_overflow_check_g32_dev, zero_adam_step_g32_dev -- the device-resident
 * sequence over FP32 gradients (an FP32 micro-batch accumulator; "How far
 * does splitting the batch get you?", "What does gradient accumulation
 * actually buy?"): zero_overflow_check_g32 with S read from
 * d_ctl->scaler.loss_scale and the flag written to d_ctl->found_inf (no sum
 * of squares), and zero_adam_step_g32 with S and the bias corrections read
 * from d_ctl, writing nothing unless d_ctl->apply is set.  The decision
 * between them is zero_scaler_update_dev.  Arguments, alignment, overlap
 * rules and errors are as for the host-controlled forms and
 * zero_overflow_check_dev / zero_adam_step_dev.
 */
int zero_overflow_check_g32_dev(const float *g32, uint64_t psi, uint32_t n, uint32_t rank,
                                zero_device_ctl *d_ctl, void *stream);
int zero_adam_step_g32_dev(void *w16, const float *g32, float *master, float *m, float *v,
                           zero_dtype dt, uint64_t psi, uint32_t n, uint32_t rank, float lr,
                           float beta1, float beta2, float eps, float weight_decay,
                           const zero_device_ctl *d_ctl, void *stream);

/*
 * zero_grad_accumulate_check_dev -- zero_grad_accumulate_check with S read from
 * d_ctl->scaler.loss_scale and the flag written to d_ctl->found_inf, for the
 * device-resident sequence (zero_scaler_update_dev and zero_adam_step_g32_dev
 * follow).  d_ctl may not overlap acc or g16.
 */
int zero_grad_accumulate_check_dev(float *acc, const void *g16, zero_dtype dt, uint64_t psi,
                                   uint32_t n, uint32_t rank, int32_t first,
                                   zero_device_ctl *d_ctl, void *stream);

/*
 * zero_reduce_shard_check_dev -- zero_reduce_shard_check with S read from
 * d_ctl->scaler.loss_scale and the flag written to d_ctl->found_inf, for the
 * device-resident sequence (zero_scaler_update_dev and zero_adam_step_dev
 * follow).  d_ctl may not overlap out or a replica's chunk.
 */
int zero_reduce_shard_check_dev(void *out, zero_dtype out_dt, const void *const *replicas,
                                zero_dtype in_dt, uint64_t psi, uint32_t n, uint32_t rank,
                                zero_device_ctl *d_ctl, void *stream);

/* ---------------------------------------------------------------------------
 * Sharded checkpoints: each rank writes its own slice of the model states to
 * its own file, in parallel with the others ("Stop Replicating What You Can
 * Shard", "Two memory levers you compose with sharding"); a run resumes on
 * the same or another number of ranks.  Host pointers and host files only
 * (copy device buffers to host memory first).
 * ------------------------------------------------------------------------- */

/* What a shard file records besides the four arrays. */
typedef struct {
    uint64_t psi;       /* flat buffer size */
    uint32_t n, rank;   /* the layout the shard belongs to */
    uint64_t offset;    /* rank * S (filled by the reader; ignored by the writer) */
    uint64_t count;     /* real elements (filled by the reader; ignored by the writer) */
    zero_dtype dtype;   /* working weights' format: ZERO_F16 or ZERO_BF16 */
    zero_scaler scaler; /* loss scale, growth interval, applied steps, clean steps */
} zero_ckpt_info;

/*
 * zero_ckpt_write -- write rank info->rank's slice: a 128-byte header, then
 * count 16-bit working weights and count FP32 master, m and v values (count
 * from the layout), little-endian.  Header (byte offset: field): 0 magic
 * "ZSHARD01", 8 version (u32, 2), 12 dtype (u32), 16 psi (u64), 24 n (u32),
 * 28 rank (u32), 32 offset (u64), 40 count (u64), 48 step (u64), 56
 * clean_steps (u64), 64 loss_scale (f32), 68 growth_interval (u32), 72
 * payload bytes (u64), 80 payload hash (u64), then zeros.  The hash reads
 * the payload as 8-byte little-endian words (the last zero-padded), folds
 * word i into lane i mod 4 by FNV-1a (h = (h ^ w) * 0x100000001b3, each lane
 * starting at 0xcbf29ce484222325), then folds the four lanes, lane 0 first,
 * into one more FNV-1a state from the same start.
 * The file is written as path + ".tmp", flushed to the device and renamed
 * over path, so a reader finds either the previous file or the complete new
 * one; the directory is then flushed too where the file system allows it.
 * On failure the temporary file is removed.  Two writers of the same path at
 * once share that temporary name and race: give each rank its own path.
 *   w16, master, m, v  HOST arrays of count elements.
 *   Errors: ZERO_EINVAL (bad layout, NULL pointers), ZERO_EDTYPE, ZERO_EIO.
 */
int zero_ckpt_write(const char *path, const zero_ckpt_info *info, const void *w16,
                    const float *master, const float *m, const float *v);

/* zero_ckpt_read_info -- header of a shard file, checked against its layout
 * and the file size.  Errors: ZERO_EINVAL, ZERO_EIO, ZERO_ECORRUPT. */
int zero_ckpt_read_info(const char *path, zero_ckpt_info *info);

/* zero_ckpt_verify -- recompute the payload hash.  ZERO_OK, or ZERO_ECORRUPT /
 * ZERO_EIO. */
int zero_ckpt_verify(const char *path);

/*
 * zero_ckpt_read -- elements [first, first + count) of a shard file's arrays
 * into HOST arrays (w16: 2-byte elements; master, m, v: FP32).  It checks the
 * header and the file size but not the payload hash, so that a range can be
 * read without reading the whole file: call zero_ckpt_verify first to detect
 * changed payload bytes (zero_ckpt_read_resharded does).  Errors: ZERO_EINVAL
 * for a range outside the shard or NULL pointers with count > 0; ZERO_EIO;
 * ZERO_ECORRUPT for a bad header or size.
 */
int zero_ckpt_read(const char *path, uint64_t first, uint64_t count, void *w16, float *master,
                   float *m, float *v);

/* One piece of a new rank's range: count elements starting at src_first of
 * old rank src_rank's shard go to dst_first of the new shard. */
typedef struct {
    uint32_t src_rank;
    uint64_t src_first;
    uint64_t dst_first;
    uint64_t count;
} zero_ckpt_piece;

/*
 * zero_reshard_plan -- the pieces of the n_old shards that rank rank_new of a
 * layout with n_new ranks reads, in flat order.  The concatenation of the
 * shards is the flat buffer, so a new layout's range is read from the old
 * shards that overlap it.  pieces may be NULL to count them only.
 *   Errors: ZERO_EINVAL for bad layouts or a NULL n_pieces; ZERO_ERANGE if
 *   more than max_pieces pieces are needed.
 */
int zero_reshard_plan(uint64_t psi, uint32_t n_old, uint32_t n_new, uint32_t rank_new,
                      zero_ckpt_piece *pieces, uint32_t max_pieces, uint32_t *n_pieces);

/*
 * zero_ckpt_read_resharded -- rank rank_new's slice of a layout with n_new
 * ranks, read from the n_old shard files of the same flat buffer (paths_old[k]
 * is old rank k's file), into HOST arrays of the new rank's count elements.
 * Every one of the n_old headers is checked against psi, n_old and its rank,
 * and all must share one format and one scaler state (loss scale, growth
 * interval, step, clean steps): a save interrupted between ranks leaves files
 * of two steps, which are refused.  The payload hash of every file the new
 * rank reads (those zero_reshard_plan names) is verified before its pieces
 * are copied, so such files are read twice.
 *   Errors: ZERO_EINVAL (NULL paths or arrays, bad layouts), ZERO_EIO,
 *   ZERO_ECORRUPT (a bad header, a mismatch between files, a bad hash).
 */
int zero_ckpt_read_resharded(const char *const *paths_old, uint32_t n_old, uint64_t psi,
                             uint32_t n_new, uint32_t rank_new, void *w16, float *master,
                             float *m, float *v);

/*
 * zero_strerror -- text for a return code.  For ZERO_EHIP it names the HIP
 * error of the most recent failing call made by this thread.  The pointer
 * stays valid until this thread's next call into the library.
 */
const char *zero_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_SHARD_H_ */
