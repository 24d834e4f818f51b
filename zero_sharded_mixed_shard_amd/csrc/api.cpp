// C-ABI entry points: argument checks, host-side scalars, kernel dispatch.
//
// Every check runs before anything is enqueued, so an error leaves the
// device untouched.  No C++ exception crosses the boundary.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>

#include "launch.h"
#include "zero_shard.h"
#include "zero_shard_tuning.h"

namespace {

thread_local char g_err[256];

int fail_hip(hipError_t e, const char *what) {
    std::snprintf(g_err, sizeof g_err, "HIP error in %s: %s (%d)", what, hipGetErrorString(e),
                  static_cast<int>(e));
    return ZERO_EHIP;
}

constexpr int kMaxDevices = 64;
// Per-device cache of the properties the launchers use; a zero compute-unit
// count marks an entry not yet filled.  Each field is written once with the
// same value by whichever thread gets there first, the CU count last.
std::atomic<int> g_cus[kMaxDevices];
std::atomic<int> g_lds_cu[kMaxDevices];
std::atomic<int> g_lds_block[kMaxDevices];

// Test and tuning overrides (zero_shard_tuning.h), kept per thread so that one
// caller's setting never changes another thread's launches: the grid cap and
// the resident blocks per CU of the streaming kernels and the elements per
// launch (0: each kernel's rule).
thread_local uint64_t t_grid_cap = zs::kMaxBlocks;
thread_local int t_occupancy = 0;
thread_local uint64_t t_piece = 0;

int device_props(zs::DeviceProps *out) {
    out->occupancy = t_occupancy;
    out->piece = t_piece;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, "hipGetDevice");
    const bool cacheable = dev >= 0 && dev < kMaxDevices;
    if (cacheable) {
        const int cus = g_cus[dev].load(std::memory_order_acquire);
        if (cus > 0) {
            out->cus = cus;
            out->lds_per_cu = g_lds_cu[dev].load(std::memory_order_relaxed);
            out->lds_per_block = g_lds_block[dev].load(std::memory_order_relaxed);
            return ZERO_OK;
        }
    }
    int n = 0, lds_cu = 0, lds_block = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&lds_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return fail_hip(e, "hipDeviceGetAttribute");
    if (n <= 0) n = 1;
    if (cacheable) {
        g_lds_cu[dev].store(lds_cu, std::memory_order_relaxed);
        g_lds_block[dev].store(lds_block, std::memory_order_relaxed);
        g_cus[dev].store(n, std::memory_order_release);
    }
    out->cus = n;
    out->lds_per_cu = lds_cu;
    out->lds_per_block = lds_block;
    return ZERO_OK;
}

bool aligned(const void *p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// Byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void *a, uint64_t na, const void *b, uint64_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

// No two of the n views (pointer, bytes) overlap: the kernels stream them as
// independent arrays.
bool disjoint(const void *const *p, const uint64_t *bytes, int n) {
    for (int i = 0; i < n; ++i)
        for (int j = i + 1; j < n; ++j)
            if (overlap(p[i], bytes[i], p[j], bytes[j])) return false;
    return true;
}

// The check's outputs (flag, sum, partial sums) may not overlap the gradients
// it reads, nor one another.
bool check_outputs_ok(const void *g, uint64_t g_bytes, const void *flag, uint64_t flag_bytes,
                      const float *sumsq, const double *partials) {
    const void *p[4] = {g, flag, sumsq, partials};
    const uint64_t b[4] = {g_bytes, flag_bytes, sumsq != nullptr ? 4u : 0u,
                           partials != nullptr ? 8ull * ZERO_SUMSQ_PARTIALS : 0u};
    return disjoint(p, b, 4);
}

bool finite(float x) { return std::isfinite(x); }

bool beta_ok(float b) { return b >= 0.0f && b < 1.0f; }

// 1 - beta^t formed in FP64 and rounded once to FP32 (bias correction).
float bias_correction(float beta, uint64_t t) {
    return static_cast<float>(1.0 - std::pow(static_cast<double>(beta), static_cast<double>(t)));
}

// The scalars that depend on the loss scale and the step number: S, its exact
// inverse when it is a power of two, the bias corrections, and the FP64
// reciprocals the kernels form their quotients with.
void call_scalars(zs::AdamScalars *s, float loss_scale, uint64_t step) {
    s->loss_scale = loss_scale;
    s->scale_pow2 = zs::scale_is_pow2(loss_scale) ? 1 : 0;
    s->inv_scale = 1.0f / loss_scale;  // exact when scale_pow2
    s->rcp_scale = 1.0 / static_cast<double>(loss_scale);
    s->bc1 = bias_correction(s->beta1, step);
    s->bc2 = bias_correction(s->beta2, step);
    s->rcp_bc1 = 1.0 / static_cast<double>(s->bc1);
    s->rcp_bc2 = 1.0 / static_cast<double>(s->bc2);
}

// Checks of a 16-bit gradient view and its layout, shared by the checks and the
// accumulates; returns the layout's count.
int check_args(const void *g16, zero_dtype dt, uint64_t psi, uint32_t n, uint32_t rank,
               uint64_t *count) {
    if (dt != ZERO_F16 && dt != ZERO_BF16) return ZERO_EDTYPE;
    zero_layout lay;
    if (zero_shard_layout(psi, n, rank, &lay) != ZERO_OK) return ZERO_EINVAL;
    if (lay.count > 0 && (g16 == nullptr || !aligned(g16, 2))) return ZERO_EINVAL;
    *count = lay.count;
    return ZERO_OK;
}

// Checks shared by every form of the step, and the scalars that depend on
// neither the step number nor the loss scale.  g is the gradient view and
// g_align its element size (2 for 16-bit, 4 for FP32 gradients).
int step_args(void *w16, const void *g, uintptr_t g_align, float *master, float *m, float *v,
              zero_dtype dt, uint64_t psi, uint32_t n, uint32_t rank, float lr, float beta1,
              float beta2, float eps, float weight_decay, const void *ctl, uint64_t ctl_bytes,
              uint64_t *count, zs::AdamScalars *s) {
    if (dt != ZERO_F16 && dt != ZERO_BF16) return ZERO_EDTYPE;
    zero_layout lay;
    if (zero_shard_layout(psi, n, rank, &lay) != ZERO_OK) return ZERO_EINVAL;
    if (!beta_ok(beta1) || !beta_ok(beta2)) return ZERO_EINVAL;
    if (!(eps >= 0.0f) || !finite(eps) || !finite(lr) || !finite(weight_decay)) return ZERO_EINVAL;
    *count = lay.count;
    if (lay.count > 0) {
        if (w16 == nullptr || g == nullptr || master == nullptr || m == nullptr || v == nullptr)
            return ZERO_EINVAL;
        if (!aligned(w16, 2) || !aligned(g, g_align) || !aligned(master, 4) || !aligned(m, 4) ||
            !aligned(v, 4))
            return ZERO_EINVAL;
        // the five views, and the flag or control block every block reads
        const void *views[6] = {w16, g, master, m, v, ctl};
        const uint64_t c = lay.count;
        const uint64_t bytes[6] = {2 * c, g_align * c, 4 * c, 4 * c, 4 * c,
                                   ctl != nullptr ? ctl_bytes : 0};
        if (!disjoint(views, bytes, 6)) return ZERO_EINVAL;
    }
    s->lr = lr;
    s->beta1 = beta1;
    s->beta2 = beta2;
    s->omb1 = 1.0f - beta1;
    s->omb2 = 1.0f - beta2;
    s->eps = eps;
    const float lw = lr * weight_decay;
    s->decay = 1.0f - lw;
    call_scalars(s, 1.0f, 1);  // placeholders: the host forms or the control block gives them
    return ZERO_OK;
}

}  // namespace

uint64_t zs::max_blocks() { return t_grid_cap; }

extern "C" int zero_set_grid_cap(uint32_t blocks) {
    t_grid_cap = blocks == 0 || blocks > zs::kMaxBlocks ? zs::kMaxBlocks : blocks;
    return ZERO_OK;
}

extern "C" int zero_set_occupancy(uint32_t blocks_per_cu) {
    t_occupancy = blocks_per_cu >= 8 ? 8 : static_cast<int>(blocks_per_cu);
    return ZERO_OK;
}

extern "C" int zero_set_launch_piece(uint64_t elements) {
    t_piece = elements;
    return ZERO_OK;
}

extern "C" int zero_overflow_check(const void *g16, zero_dtype dt, uint64_t psi, uint32_t n,
                                   uint32_t rank, float loss_scale, int32_t *d_found_inf,
                                   float *d_sumsq, double *d_partials, void *stream) {
    uint64_t count = 0;
    int rc = check_args(g16, dt, psi, n, rank, &count);
    if (rc != ZERO_OK) return rc;
    if (!(loss_scale > 0.0f) || !finite(loss_scale)) return ZERO_EINVAL;
    if (d_found_inf == nullptr || !aligned(d_found_inf, 4)) return ZERO_EINVAL;
    if (d_sumsq != nullptr &&
        (!aligned(d_sumsq, 4) || d_partials == nullptr || !aligned(d_partials, 8)))
        return ZERO_EINVAL;
    if (!check_outputs_ok(g16, 2 * count, d_found_inf, 4, d_sumsq,
                          d_sumsq != nullptr ? d_partials : nullptr))
        return ZERO_EINVAL;
    zs::DeviceProps dev;
    rc = device_props(&dev);
    if (rc != ZERO_OK) return rc;
    const hipError_t e = zs::launch_overflow_check(
        static_cast<int>(dt), static_cast<const uint16_t *>(g16), count, loss_scale, nullptr,
        d_found_inf, d_sumsq, d_partials, dev, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZERO_OK : fail_hip(e, "zero_overflow_check launch");
}

extern "C" int zero_overflow_check_noalloc(const void *g16, zero_dtype dt, uint64_t psi,
                                           uint32_t n, uint32_t rank, float loss_scale,
                                           int32_t *d_found_inf, float *d_sumsq, void *stream) {
    uint64_t count = 0;
    int rc = check_args(g16, dt, psi, n, rank, &count);
    if (rc != ZERO_OK) return rc;
    if (!(loss_scale > 0.0f) || !finite(loss_scale)) return ZERO_EINVAL;
    if (d_found_inf == nullptr || !aligned(d_found_inf, 4)) return ZERO_EINVAL;
    if (d_sumsq != nullptr && !aligned(d_sumsq, 4)) return ZERO_EINVAL;
    if (!check_outputs_ok(g16, 2 * count, d_found_inf, 4, d_sumsq, nullptr)) return ZERO_EINVAL;
    if (d_sumsq != nullptr && zs::sumsq_partials_needed(static_cast<int>(dt), g16, count) >
                                  static_cast<uint64_t>(zs::scratch_partials_capacity()))
        return ZERO_EINVAL;
    zs::DeviceProps dev;
    rc = device_props(&dev);
    if (rc != ZERO_OK) return rc;
    const hipError_t e = zs::launch_overflow_check_noalloc(
        static_cast<int>(dt), static_cast<const uint16_t *>(g16), count, loss_scale, d_found_inf,
        d_sumsq, dev, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZERO_OK : fail_hip(e, "zero_overflow_check_noalloc launch");
}

extern "C" int zero_adam_step(void *w16, const void *g16, float *master, float *m, float *v,
                              zero_dtype dt, uint64_t psi, uint32_t n, uint32_t rank, float lr,
                              float beta1, float beta2, float eps, float weight_decay,
                              uint64_t step, float loss_scale, const int32_t *d_found_inf,
                              void *stream) {
    uint64_t count = 0;
    zs::AdamScalars s;
    const int rc = step_args(w16, g16, 2, master, m, v, dt, psi, n, rank, lr, beta1, beta2, eps,
                             weight_decay, d_found_inf, 4, &count, &s);
    if (rc != ZERO_OK) return rc;
    if (step == 0) return ZERO_EINVAL;
    if (!(loss_scale > 0.0f) || !finite(loss_scale)) return ZERO_EINVAL;
    if (d_found_inf != nullptr && !aligned(d_found_inf, 4)) return ZERO_EINVAL;
    if (count == 0) return ZERO_OK;
    call_scalars(&s, loss_scale, step);
    zs::DeviceProps dev;
    const int prc = device_props(&dev);
    if (prc != ZERO_OK) return prc;
    const hipError_t e = zs::launch_adam_step(
        static_cast<int>(dt), static_cast<uint16_t *>(w16), static_cast<const uint16_t *>(g16),
        master, m, v, count, s, d_found_inf, nullptr, dev, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZERO_OK : fail_hip(e, "zero_adam_step launch");
}

extern "C" int zero_grad_accumulate(float *acc, const void *g16, zero_dtype dt, uint64_t psi,
                                    uint32_t n, uint32_t rank, int32_t first, void *stream) {
    uint64_t count = 0;
    const int rc = check_args(g16, dt, psi, n, rank, &count);
    if (rc != ZERO_OK) return rc;
    if (count == 0) return ZERO_OK;
    if (acc == nullptr || !aligned(acc, 4)) return ZERO_EINVAL;
    if (overlap(acc, 4 * count, g16, 2 * count)) return ZERO_EINVAL;
    zs::DeviceProps dev;
    const int prc = device_props(&dev);
    if (prc != ZERO_OK) return prc;
    const hipError_t e =
        zs::launch_grad_accumulate(static_cast<int>(dt), acc, static_cast<const uint16_t *>(g16),
                                   count, first != 0, dev, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZERO_OK : fail_hip(e, "zero_grad_accumulate launch");
}

// Shared by both forms of the fused accumulate-and-check: arguments of the
// accumulate, and the flag (or control block) apart from both views.
int accumulate_check_args(float *acc, const void *g16, zero_dtype dt, uint64_t psi, uint32_t n,
                          uint32_t rank, const void *flag, uint64_t flag_bytes, uint64_t *count) {
    const int rc = check_args(g16, dt, psi, n, rank, count);
    if (rc != ZERO_OK) return rc;
    if (*count > 0 && (acc == nullptr || !aligned(acc, 4))) return ZERO_EINVAL;
    if (overlap(acc, 4 * *count, g16, 2 * *count)) return ZERO_EINVAL;
    if (flag == nullptr || !aligned(flag, 4)) return ZERO_EINVAL;
    if (overlap(flag, flag_bytes, acc, 4 * *count) || overlap(flag, flag_bytes, g16, 2 * *count))
        return ZERO_EINVAL;
    return ZERO_OK;
}

extern "C" int zero_grad_accumulate_check(float *acc, const void *g16, zero_dtype dt,
                                          uint64_t psi, uint32_t n, uint32_t rank, int32_t first,
                                          float loss_scale, int32_t *d_found_inf, void *stream) {
    uint64_t count = 0;
    int rc = accumulate_check_args(acc, g16, dt, psi, n, rank, d_found_inf, 4, &count);
    if (rc != ZERO_OK) return rc;
    if (!(loss_scale > 0.0f) || !finite(loss_scale)) return ZERO_EINVAL;
    zs::DeviceProps dev;
    rc = device_props(&dev);
    if (rc != ZERO_OK) return rc;
    const hipError_t e = zs::launch_grad_accumulate_check(
        static_cast<int>(dt), acc, static_cast<const uint16_t *>(g16), count, first != 0,
        loss_scale, nullptr, d_found_inf, dev, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZERO_OK : fail_hip(e, "zero_grad_accumulate_check launch");
}

extern "C" int zero_grad_accumulate_check_dev(float *acc, const void *g16, zero_dtype dt,
                                              uint64_t psi, uint32_t n, uint32_t rank,
                                              int32_t first, zero_device_ctl *d_ctl,
                                              void *stream) {
    uint64_t count = 0;
    if (d_ctl != nullptr && !aligned(d_ctl, alignof(zero_device_ctl))) return ZERO_EINVAL;
    int rc = accumulate_check_args(acc, g16, dt, psi, n, rank, d_ctl, sizeof(zero_device_ctl),
                                   &count);
    if (rc != ZERO_OK) return rc;
    zs::DeviceProps dev;
    rc = device_props(&dev);
    if (rc != ZERO_OK) return rc;
    const hipError_t e = zs::launch_grad_accumulate_check(
        static_cast<int>(dt), acc, static_cast<const uint16_t *>(g16), count, first != 0, 1.0f,
        &d_ctl->scaler.loss_scale, &d_ctl->found_inf, dev, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZERO_OK : fail_hip(e, "zero_grad_accumulate_check_dev launch");
}

extern "C" int zero_overflow_check_g32(const float *g32, uint64_t psi, uint32_t n, uint32_t rank,
                                       float loss_scale, int32_t *d_found_inf, float *d_sumsq,
                                       double *d_partials, void *stream) {
    zero_layout lay;
    if (zero_shard_layout(psi, n, rank, &lay) != ZERO_OK) return ZERO_EINVAL;
    if (lay.count > 0 && (g32 == nullptr || !aligned(g32, 4))) return ZERO_EINVAL;
    if (!(loss_scale > 0.0f) || !finite(loss_scale)) return ZERO_EINVAL;
    if (d_found_inf == nullptr || !aligned(d_found_inf, 4)) return ZERO_EINVAL;
    if (d_sumsq != nullptr &&
        (!aligned(d_sumsq, 4) || d_partials == nullptr || !aligned(d_partials, 8)))
        return ZERO_EINVAL;
    if (!check_outputs_ok(g32, 4 * lay.count, d_found_inf, 4, d_sumsq,
                          d_sumsq != nullptr ? d_partials : nullptr))
        return ZERO_EINVAL;
    zs::DeviceProps dev;
    const int rc = device_props(&dev);
    if (rc != ZERO_OK) return rc;
    const hipError_t e =
        zs::launch_overflow_check_g32(g32, lay.count, loss_scale, nullptr, d_found_inf, d_sumsq,
                                      d_partials, dev, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZERO_OK : fail_hip(e, "zero_overflow_check_g32 launch");
}

extern "C" int zero_adam_step_g32(void *w16, const float *g32, float *master, float *m, float *v,
                                  zero_dtype dt, uint64_t psi, uint32_t n, uint32_t rank,
                                  float lr, float beta1, float beta2, float eps,
                                  float weight_decay, uint64_t step, float loss_scale,
                                  const int32_t *d_found_inf, void *stream) {
    uint64_t count = 0;
    zs::AdamScalars s;
    const int rc = step_args(w16, g32, 4, master, m, v, dt, psi, n, rank, lr, beta1, beta2, eps,
                             weight_decay, d_found_inf, 4, &count, &s);
    if (rc != ZERO_OK) return rc;
    if (step == 0) return ZERO_EINVAL;
    if (!(loss_scale > 0.0f) || !finite(loss_scale)) return ZERO_EINVAL;
    if (d_found_inf != nullptr && !aligned(d_found_inf, 4)) return ZERO_EINVAL;
    if (count == 0) return ZERO_OK;
    call_scalars(&s, loss_scale, step);
    zs::DeviceProps dev;
    const int prc = device_props(&dev);
    if (prc != ZERO_OK) return prc;
    const hipError_t e = zs::launch_adam_step_g32(static_cast<int>(dt),
                                                  static_cast<uint16_t *>(w16), g32, master, m, v,
                                                  count, s, d_found_inf, nullptr, dev,
                                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZERO_OK : fail_hip(e, "zero_adam_step_g32 launch");
}

namespace {

// Checks shared by the reduce and the reduce with the fused check: formats,
// layout, pointers, and that the output overlaps no replica's chunk unless it
// is exactly one of them in the same format (in place: each element is
// written after every replica's element was read).  Fills the replica views
// advanced to the rank's first element, the count and the byte spans of the
// views (for the flag's overlap test).
int reduce_args(void *out, zero_dtype out_dt, const void *const *replicas, zero_dtype in_dt,
                uint64_t psi, uint32_t n, uint32_t rank, zs::ReplicaSet *set, uint64_t *count,
                uint64_t *out_bytes, uint64_t *in_bytes) {
    const auto fmt_ok = [](zero_dtype d) { return d == ZERO_F16 || d == ZERO_BF16 || d == ZERO_F32; };
    if (!fmt_ok(out_dt) || !fmt_ok(in_dt)) return ZERO_EDTYPE;
    zero_layout lay;
    if (zero_shard_layout(psi, n, rank, &lay) != ZERO_OK) return ZERO_EINVAL;
    if (n > zs::kMaxLocalRanks) return ZERO_EINVAL;
    *count = lay.count;
    const uintptr_t in_b = in_dt == ZERO_F32 ? 4 : 2, out_b = out_dt == ZERO_F32 ? 4 : 2;
    *out_bytes = out_b * lay.count;
    *in_bytes = in_b * lay.count;
    if (lay.count == 0) return ZERO_OK;
    if (out == nullptr || !aligned(out, out_b) || replicas == nullptr) return ZERO_EINVAL;
    for (uint32_t k = 0; k < n; ++k) {
        if (replicas[k] == nullptr || !aligned(replicas[k], in_b)) return ZERO_EINVAL;
        set->p[k] = static_cast<const char *>(replicas[k]) + lay.offset * in_b;
        // replicas may repeat one another (read-only)
        const bool in_place = out == set->p[k] && out_b == in_b;
        if (!in_place && overlap(out, *out_bytes, set->p[k], *in_bytes)) return ZERO_EINVAL;
    }
    return ZERO_OK;
}

// The flag of the fused check may share no byte with the output or a replica's chunk.
bool flag_clear_of(const int32_t *flag, uint64_t flag_bytes, const void *out, uint64_t out_bytes,
                   const zs::ReplicaSet &set, uint32_t n, uint64_t in_bytes, uint64_t count) {
    if (count == 0) return true;
    if (overlap(flag, flag_bytes, out, out_bytes)) return false;
    for (uint32_t k = 0; k < n; ++k)
        if (overlap(flag, flag_bytes, set.p[k], in_bytes)) return false;
    return true;
}

int reduce_launch(void *out, zero_dtype out_dt, const zs::ReplicaSet &set, zero_dtype in_dt,
                  uint32_t n, uint64_t count, const zs::ReduceCheck &chk, void *stream,
                  const char *what) {
    zs::DeviceProps dev;
    const int prc = device_props(&dev);
    if (prc != ZERO_OK) return prc;
    const hipError_t e = zs::launch_reduce_shard(out, static_cast<int>(out_dt), set,
                                                 static_cast<int>(in_dt), n, count, chk, dev,
                                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZERO_OK : fail_hip(e, what);
}

}  // namespace

extern "C" int zero_reduce_shard(void *out, zero_dtype out_dt, const void *const *replicas,
                                 zero_dtype in_dt, uint64_t psi, uint32_t n, uint32_t rank,
                                 void *stream) {
    zs::ReplicaSet set;
    uint64_t count = 0, out_bytes = 0, in_bytes = 0;
    const int rc = reduce_args(out, out_dt, replicas, in_dt, psi, n, rank, &set, &count,
                               &out_bytes, &in_bytes);
    if (rc != ZERO_OK || count == 0) return rc;
    return reduce_launch(out, out_dt, set, in_dt, n, count, zs::ReduceCheck{1.0f, nullptr, nullptr},
                         stream, "zero_reduce_shard launch");
}

extern "C" int zero_reduce_shard_check(void *out, zero_dtype out_dt, const void *const *replicas,
                                       zero_dtype in_dt, uint64_t psi, uint32_t n, uint32_t rank,
                                       float loss_scale, int32_t *d_found_inf, void *stream) {
    zs::ReplicaSet set;
    uint64_t count = 0, out_bytes = 0, in_bytes = 0;
    const int rc = reduce_args(out, out_dt, replicas, in_dt, psi, n, rank, &set, &count,
                               &out_bytes, &in_bytes);
    if (rc != ZERO_OK) return rc;
    if (!(loss_scale > 0.0f) || !finite(loss_scale)) return ZERO_EINVAL;
    if (d_found_inf == nullptr || !aligned(d_found_inf, 4)) return ZERO_EINVAL;
    if (!flag_clear_of(d_found_inf, 4, out, out_bytes, set, n, in_bytes, count))
        return ZERO_EINVAL;
    return reduce_launch(out, out_dt, set, in_dt, n, count,
                         zs::ReduceCheck{loss_scale, nullptr, d_found_inf}, stream,
                         "zero_reduce_shard_check launch");
}

extern "C" int zero_reduce_shard_check_dev(void *out, zero_dtype out_dt,
                                           const void *const *replicas, zero_dtype in_dt,
                                           uint64_t psi, uint32_t n, uint32_t rank,
                                           zero_device_ctl *d_ctl, void *stream) {
    zs::ReplicaSet set;
    uint64_t count = 0, out_bytes = 0, in_bytes = 0;
    const int rc = reduce_args(out, out_dt, replicas, in_dt, psi, n, rank, &set, &count,
                               &out_bytes, &in_bytes);
    if (rc != ZERO_OK) return rc;
    if (d_ctl == nullptr || !aligned(d_ctl, alignof(zero_device_ctl))) return ZERO_EINVAL;
    if (!flag_clear_of(reinterpret_cast<const int32_t *>(d_ctl), sizeof(zero_device_ctl), out,
                       out_bytes, set, n, in_bytes, count))
        return ZERO_EINVAL;
    return reduce_launch(out, out_dt, set, in_dt, n, count,
                         zs::ReduceCheck{1.0f, &d_ctl->scaler.loss_scale, &d_ctl->found_inf},
                         stream, "zero_reduce_shard_check_dev launch");
}

extern "C" int zero_gather_shards(void *full, const void *const *shards, zero_dtype dt,
                                  uint64_t psi, uint32_t n, void *stream) {
    if (dt != ZERO_F16 && dt != ZERO_BF16 && dt != ZERO_F32) return ZERO_EDTYPE;
    zero_layout lay;
    if (zero_shard_layout(psi, n, 0, &lay) != ZERO_OK) return ZERO_EINVAL;
    if (n > zs::kMaxLocalRanks) return ZERO_EINVAL;
    const uintptr_t eb = dt == ZERO_F32 ? 4 : 2;
    if (full == nullptr || !aligned(full, eb) || shards == nullptr) return ZERO_EINVAL;
    zs::GatherSet set;
    uint64_t max_count = 0;
    for (uint32_t k = 0; k < n; ++k) {
        zero_layout lk;
        zero_shard_layout(psi, n, k, &lk);
        if (lk.count > 0 && (shards[k] == nullptr || !aligned(shards[k], eb))) return ZERO_EINVAL;
        // a shard may sit exactly at its place in the full buffer (an in-place
        // all-gather: the copy is then the identity), but may not overlap it otherwise
        const char *dst = static_cast<const char *>(full) + lk.offset * eb;
        if (shards[k] != dst && overlap(full, psi * eb, shards[k], lk.count * eb))
            return ZERO_EINVAL;
        set.p[k] = shards[k];
        set.count[k] = lk.count;
        set.head[k] = 0;
        set.vec[k] = 0;
        if (lk.count > max_count) max_count = lk.count;
    }
    zs::DeviceProps dev;
    const int prc = device_props(&dev);
    if (prc != ZERO_OK) return prc;
    const hipError_t e = zs::launch_gather_shards(full, static_cast<int>(eb), set, n, lay.shard,
                                                  max_count, dev,
                                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZERO_OK : fail_hip(e, "zero_gather_shards launch");
}

extern "C" int zero_bias_corrections(float beta1, float beta2, uint64_t t_first, uint32_t len,
                                     float *out) {
    if (out == nullptr || len == 0 || t_first == 0 || !beta_ok(beta1) || !beta_ok(beta2))
        return ZERO_EINVAL;
    for (uint32_t k = 0; k < len; ++k) {
        out[k] = bias_correction(beta1, t_first + k);
        out[len + k] = bias_correction(beta2, t_first + k);
    }
    return ZERO_OK;
}

extern "C" int zero_overflow_check_dev(const void *g16, zero_dtype dt, uint64_t psi, uint32_t n,
                                       uint32_t rank, zero_device_ctl *d_ctl, void *stream) {
    uint64_t count = 0;
    int rc = check_args(g16, dt, psi, n, rank, &count);
    if (rc != ZERO_OK) return rc;
    if (d_ctl == nullptr || !aligned(d_ctl, alignof(zero_device_ctl))) return ZERO_EINVAL;
    if (!check_outputs_ok(g16, 2 * count, d_ctl, sizeof(zero_device_ctl), nullptr, nullptr))
        return ZERO_EINVAL;
    zs::DeviceProps dev;
    rc = device_props(&dev);
    if (rc != ZERO_OK) return rc;
    const hipError_t e = zs::launch_overflow_check(
        static_cast<int>(dt), static_cast<const uint16_t *>(g16), count, 1.0f,
        &d_ctl->scaler.loss_scale, &d_ctl->found_inf, nullptr, nullptr, dev,
        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZERO_OK : fail_hip(e, "zero_overflow_check_dev launch");
}

extern "C" int zero_scaler_update_dev(zero_device_ctl *d_ctl, const float *d_bias,
                                      uint64_t t_first, uint32_t len, void *stream) {
    if (d_ctl == nullptr || !aligned(d_ctl, alignof(zero_device_ctl))) return ZERO_EINVAL;
    if (d_bias == nullptr || !aligned(d_bias, 4) || len == 0 || t_first == 0) return ZERO_EINVAL;
    if (overlap(d_ctl, sizeof(zero_device_ctl), d_bias, 8ull * len)) return ZERO_EINVAL;
    const hipError_t e =
        zs::launch_scaler_decide(d_ctl, d_bias, t_first, len, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZERO_OK : fail_hip(e, "zero_scaler_update_dev launch");
}

extern "C" int zero_adam_step_dev(void *w16, const void *g16, float *master, float *m, float *v,
                                  zero_dtype dt, uint64_t psi, uint32_t n, uint32_t rank,
                                  float lr, float beta1, float beta2, float eps,
                                  float weight_decay, const zero_device_ctl *d_ctl,
                                  void *stream) {
    uint64_t count = 0;
    zs::AdamScalars s;
    const int rc = step_args(w16, g16, 2, master, m, v, dt, psi, n, rank, lr, beta1, beta2, eps,
                             weight_decay, d_ctl, sizeof(zero_device_ctl), &count, &s);
    if (rc != ZERO_OK) return rc;
    if (d_ctl == nullptr || !aligned(d_ctl, alignof(zero_device_ctl))) return ZERO_EINVAL;
    if (count == 0) return ZERO_OK;
    zs::DeviceProps dev;
    const int prc = device_props(&dev);
    if (prc != ZERO_OK) return prc;
    const hipError_t e = zs::launch_adam_step(
        static_cast<int>(dt), static_cast<uint16_t *>(w16), static_cast<const uint16_t *>(g16),
        master, m, v, count, s, nullptr, d_ctl, dev, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZERO_OK : fail_hip(e, "zero_adam_step_dev launch");
}

extern "C" int zero_overflow_check_g32_dev(const float *g32, uint64_t psi, uint32_t n,
                                           uint32_t rank, zero_device_ctl *d_ctl, void *stream) {
    zero_layout lay;
    if (zero_shard_layout(psi, n, rank, &lay) != ZERO_OK) return ZERO_EINVAL;
    if (lay.count > 0 && (g32 == nullptr || !aligned(g32, 4))) return ZERO_EINVAL;
    if (d_ctl == nullptr || !aligned(d_ctl, alignof(zero_device_ctl))) return ZERO_EINVAL;
    if (!check_outputs_ok(g32, 4 * lay.count, d_ctl, sizeof(zero_device_ctl), nullptr, nullptr))
        return ZERO_EINVAL;
    zs::DeviceProps dev;
    const int rc = device_props(&dev);
    if (rc != ZERO_OK) return rc;
    const hipError_t e = zs::launch_overflow_check_g32(
        g32, lay.count, 1.0f, &d_ctl->scaler.loss_scale, &d_ctl->found_inf, nullptr, nullptr, dev,
        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZERO_OK : fail_hip(e, "zero_overflow_check_g32_dev launch");
}

extern "C" int zero_adam_step_g32_dev(void *w16, const float *g32, float *master, float *m,
                                      float *v, zero_dtype dt, uint64_t psi, uint32_t n,
                                      uint32_t rank, float lr, float beta1, float beta2,
                                      float eps, float weight_decay, const zero_device_ctl *d_ctl,
                                      void *stream) {
    uint64_t count = 0;
    zs::AdamScalars s;
    const int rc = step_args(w16, g32, 4, master, m, v, dt, psi, n, rank, lr, beta1, beta2, eps,
                             weight_decay, d_ctl, sizeof(zero_device_ctl), &count, &s);
    if (rc != ZERO_OK) return rc;
    if (d_ctl == nullptr || !aligned(d_ctl, alignof(zero_device_ctl))) return ZERO_EINVAL;
    if (count == 0) return ZERO_OK;
    zs::DeviceProps dev;
    const int prc = device_props(&dev);
    if (prc != ZERO_OK) return prc;
    const hipError_t e = zs::launch_adam_step_g32(static_cast<int>(dt),
                                                  static_cast<uint16_t *>(w16), g32, master, m, v,
                                                  count, s, nullptr, d_ctl, dev,
                                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZERO_OK : fail_hip(e, "zero_adam_step_g32_dev launch");
}

extern "C" const char *zero_strerror(int code) {
    switch (code) {
        case ZERO_OK:
            return "ok";
        case ZERO_EINVAL:
            return "invalid argument";
        case ZERO_EDTYPE:
            return "unsupported dtype (ZERO_F16 or ZERO_BF16; the exchanges also take ZERO_F32)";
        case ZERO_EHIP:
            return g_err[0] ? g_err : "HIP runtime error";
        case ZERO_ERANGE:
            return "value out of range (step outside the bias-correction table, or too few "
                   "reshard pieces)";
        case ZERO_EIO:
            return "checkpoint file could not be opened, written or read";
        case ZERO_ECORRUPT:
            return "checkpoint file failed its header, size or hash check";
        default:
            return "unknown error code";
    }
}
