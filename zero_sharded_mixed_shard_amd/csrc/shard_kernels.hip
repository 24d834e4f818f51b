// gfx950 (MI355X) kernels of the ZeRO-sharded mixed-precision Adam step.
//
// The step is elementwise over five structure-of-arrays streams (gradients,
// FP32 master / m / v, 16-bit working weights): 28 bytes of HBM traffic per
// element with 16-bit gradients (30 with FP32 gradients) and ~54 VALU
// operations, far below the FP32 ridge point, so the kernels are built for
// bandwidth: every lane moves one 16-B FP32 vector per array and one 8-B
// 16-bit vector per group of 4 elements, a wave's accesses are contiguous
// 1 KiB (FP32) or 512 B (16-bit) runs, and each lane keeps U groups in
// flight.  No LDS is read or written: nothing is reused (launches may reserve
// LDS only to cap the resident blocks per CU).  Every access of the streaming
// kernels is non-temporal (the data is touched once), and the step launches
// one block per tile (a grid-stride loop only past 2^23 tiles): both measured
// faster on MI355X than a resident grid looping over tiles.  A shard of at
// least 2^28 elements steps (and accumulates its last micro-batch with the
// fused check) in consecutive launches of 2^27 (kStepPiece).
//
// Numerics follow the update of "Training models too big for one GPU: ZeRO &
// FSDP" ("Adam, and why it's expensive", "Mixed-precision training") with
// one binary32 rounding per operation: contraction is off for this file,
// FP32 division and square root stay correctly rounded (the HIP default),
// denormals are kept, and the 16-bit conversions round to nearest even.  The
// quotients by per-call constants are formed without a division but with the
// division's exact result (the argument is below, before adam_update).
//
// Gradient element types: uint16_t holds FP16 (DT = 0) or BF16 (DT = 1) bit
// patterns; float holds FP32 gradients (accumulated across micro-batches,
// "How far does splitting the batch get you?", gradient accumulation).  DT is
// always the working weights' format.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "launch.h"
#include "zero_shard.h"

#pragma clang fp contract(off)

// Partial sums of the sum-of-squares check for callers that cannot allocate
// (zero_overflow_check_noalloc): 4096 doubles (32 KiB), one copy per device,
// held until the process ends and shared by every such call on the device.
// Host code never passes this name to a kernel: it stands for the host-side
// shadow.  The device address comes from hipGetSymbolAddress (below).
static __device__ __align__(256) double scratch[ZERO_SUMSQ_PARTIALS];

namespace zs {
namespace {

constexpr int kThreads = 256;              // 4 wave64s
constexpr int kVec = 4;                    // elements per lane per group
constexpr int kGroup = kThreads * kVec;    // elements per block per group
constexpr uint32_t kSumsqPartials = 4096;  // == ZERO_SUMSQ_PARTIALS (room for the grid)

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Streaming accesses: every byte is read once and written once.
template <typename T>
__device__ __forceinline__ T load_nt(const T *p) {
    return __builtin_nontemporal_load(p);
}
template <typename T>
__device__ __forceinline__ void store_nt(T *p, T v) {
    __builtin_nontemporal_store(v, p);
}

// ---- 16-bit formats -------------------------------------------------------

template <int DT> __device__ __forceinline__ float widen(uint32_t h);
template <> __device__ __forceinline__ float widen<0>(uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}
template <> __device__ __forceinline__ float widen<1>(uint32_t h) {
    return __builtin_bit_cast(float, h << 16);
}

template <int DT> __device__ __forceinline__ uint32_t narrow(float f);
template <> __device__ __forceinline__ uint32_t narrow<0>(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));  // RNE
}
template <> __device__ __forceinline__ uint32_t narrow<1>(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));    // RNE
}

__device__ __forceinline__ uint32_t not_finite(float x) {
    return (__builtin_bit_cast(uint32_t, x) & 0x7f800000u) == 0x7f800000u;
}

// ---- gradient access ------------------------------------------------------

template <typename GT, int DT>
__device__ __forceinline__ float grad_at(const GT *__restrict__ g, uint64_t i) {
    if constexpr (sizeof(GT) == 2)
        return widen<DT>(g[i]);
    else
        return g[i];
}

// Four consecutive gradients from an aligned address (8 B for 16-bit, 16 B for FP32).
template <typename GT, int DT>
__device__ __forceinline__ void grad4(const GT *__restrict__ g, uint64_t e, float out[4]) {
    if constexpr (sizeof(GT) == 2) {
        const u32x2 x = load_nt(reinterpret_cast<const u32x2 *>(g + e));
        out[0] = widen<DT>(x.x & 0xffffu);
        out[1] = widen<DT>(x.x >> 16);
        out[2] = widen<DT>(x.y & 0xffffu);
        out[3] = widen<DT>(x.y >> 16);
    } else {
        const f32x4 x = load_nt(reinterpret_cast<const f32x4 *>(g + e));
        out[0] = x.x;
        out[1] = x.y;
        out[2] = x.z;
        out[3] = x.w;
    }
}

// ---- quotients by the per-call constants ------------------------------------
//
// The update divides by three numbers that are the same for every element:
// S, bc1 = 1 - beta1^t and bc2 = 1 - beta2^t.  Each quotient a / d (FP32 a,
// FP32 d > 0) is formed as q = (float)((double)a * r) with r = RN64(1/d):
//  - r is within 2^-53 of 1/d and the FP64 product rounds once more, so the
//    product is within 2^-52 (relative, plus a negligible cross term) of the
//    real quotient a/d.
//  - Write a = A*2^x and d = D*2^y with A, D odd integers below 2^24.  A
//    rounding boundary of FP32 in the normal range (a midpoint between
//    neighbours, or the overflow threshold) is M*2^z with M odd,
//    2^24 <= M < 2^25.  a/d equals no such point: that needs A = M*D >= M
//    > A.  So A*2^x - M*D*2^(y+z) is a non-zero multiple of
//    2^min(x, y+z), and for a boundary next to a/d (M*2^z within a factor
//    1 + 2^-23 of a/d) the distance |a/d - M*2^z| is at least 2^-49 * |a/d|.
//    The product therefore never lies across a boundary from a/d, and one
//    rounding to FP32 gives exactly the correctly rounded a / d --
//    wherever a/d and the product lie in the normal range.
//  - A rounded q of at least 2^-125 in magnitude puts both there; q = 0 from
//    a = 0 is exact too.  Every other element (a != 0 with |q| < 2^-125,
//    where subnormal spacing breaks the argument) is divided as written.
//    One compare per quotient finds them; a lane divides only when one of
//    its elements needs it.
//  - S = 2^k with a normal reciprocal needs nothing of this: g * 2^-k is the
//    same real number as g / S, rounded once.
// tests/method/quotient_check.c compares the rule with the FP32 division on
// the CPU, including numerators built to sit next to a boundary.

__device__ __forceinline__ float quot_rcp(float a, double rcp) {
    return static_cast<float>(static_cast<double>(a) * rcp);
}

// The product differs from a / d only if this holds.
__device__ __forceinline__ bool needs_division(float q, float a) {
    return __builtin_fabsf(q) < 0x1p-125f && a != 0.0f;
}

// How the kernels undo the loss scale: multiply by the exact 1/S (S a power
// of two), the FP64 reciprocal product, or either as the device control
// block says (S is known only on the device).
enum Unscale : int { kUnscaleMul = 0, kUnscaleRcp = 1, kUnscaleCtl = 2 };

// ---- K elements of the step -------------------------------------------------

template <int DT, int MODE, int K>
__device__ __forceinline__ void adam_update(const float (&graw)[K], float (&p)[K], float (&m)[K],
                                            float (&v)[K], uint32_t (&w)[K],
                                            const AdamScalars &s) {
    static_assert(MODE == kUnscaleMul || MODE == kUnscaleRcp, "resolved unscale mode");
    float g[K];
    if constexpr (MODE == kUnscaleMul) {
#pragma unroll
        for (int j = 0; j < K; ++j) g[j] = graw[j] * s.inv_scale;
    } else {
        bool redo = false;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            g[j] = quot_rcp(graw[j], s.rcp_scale);
            redo |= needs_division(g[j], graw[j]);
        }
        if (redo) {
#pragma unroll
            for (int j = 0; j < K; ++j)
                if (needs_division(g[j], graw[j])) g[j] = graw[j] / s.loss_scale;
        }
    }
    float mh[K], vh[K];
    bool redo = false;
#pragma unroll
    for (int j = 0; j < K; ++j) {
        m[j] = s.beta1 * m[j] + s.omb1 * g[j];
        v[j] = s.beta2 * v[j] + s.omb2 * (g[j] * g[j]);
        mh[j] = quot_rcp(m[j], s.rcp_bc1);
        vh[j] = quot_rcp(v[j], s.rcp_bc2);
        redo |= needs_division(mh[j], m[j]) | needs_division(vh[j], v[j]);
    }
    if (redo) {
#pragma unroll
        for (int j = 0; j < K; ++j) {
            if (needs_division(mh[j], m[j])) mh[j] = m[j] / s.bc1;
            if (needs_division(vh[j], v[j])) vh[j] = v[j] / s.bc2;
        }
    }
#pragma unroll
    for (int j = 0; j < K; ++j) {
        const float pd = p[j] * s.decay;
        const float denom = __builtin_sqrtf(vh[j]) + s.eps;
        p[j] = pd - s.lr * mh[j] / denom;
        w[j] = narrow<DT>(p[j]);
    }
}

template <int DT, int MODE, typename GT>
__device__ __forceinline__ void adam_one(uint16_t *__restrict__ w16, const GT *__restrict__ g,
                                         float *__restrict__ master, float *__restrict__ m,
                                         float *__restrict__ v, uint64_t i,
                                         const AdamScalars &s) {
    const float gr[1] = {grad_at<GT, DT>(g, i)};
    float p[1] = {master[i]}, mm[1] = {m[i]}, vv[1] = {v[i]};
    uint32_t w[1];
    adam_update<DT, MODE, 1>(gr, p, mm, vv, w, s);
    master[i] = p[0];
    m[i] = mm[0];
    v[i] = vv[0];
    w16[i] = static_cast<uint16_t>(w[0]);
}

// With a device control block, S, the bias corrections and their FP64
// reciprocals come from the block (the decision wrote them); returns whether
// the loss scale is a power of two with a normal reciprocal, whose exact
// inverse it then stores.
__device__ __forceinline__ bool take_device_scalars(const zero_device_ctl *__restrict__ ctl,
                                                    AdamScalars &s) {
    s.loss_scale = ctl->loss_scale_used;
    s.bc1 = ctl->bc1;
    s.bc2 = ctl->bc2;
    s.rcp_scale = ctl->rcp_loss_scale;
    s.rcp_bc1 = ctl->rcp_bc1;
    s.rcp_bc2 = ctl->rcp_bc2;
    const uint32_t b = __builtin_bit_cast(uint32_t, s.loss_scale);
    const uint32_t e = (b >> 23) & 0xffu;
    const bool pow2 = (b & 0x807fffffu) == 0 && e >= 1 && e <= 253;
    // S = 2^(e - 127), so 1/S = 2^(127 - e): biased exponent 254 - e (used only if pow2)
    s.inv_scale = __builtin_bit_cast(float, (254u - e) << 23);
    return pow2;
}

// ---- the step: aligned vector path ----------------------------------------
//
// Elements [0, head) and [head + n_tiles*U*kGroup, count) are done one at a
// time; in between, tile t covers U groups of kGroup elements and lane l of
// group u owns elements head + t*U*kGroup + u*kGroup + 4l .. +3.  The host
// guarantees that master/m/v (and FP32 gradients) + head are 16-B aligned
// and 16-bit arrays + head are 8-B aligned.

template <int DT, typename GT, int U, int MODE>
__device__ __forceinline__ void step_tiles(uint16_t *__restrict__ w16, const GT *__restrict__ g,
                                           float *__restrict__ master, float *__restrict__ m,
                                           float *__restrict__ v, uint64_t count, uint32_t head,
                                           uint64_t n_tiles, const AdamScalars &s) {
    const uint32_t tid = threadIdx.x;
    if (blockIdx.x == 0 && tid < head) adam_one<DT, MODE>(w16, g, master, m, v, tid, s);

    constexpr uint64_t kTile = static_cast<uint64_t>(U) * kGroup;
    for (uint64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
        const uint64_t base = head + t * kTile + static_cast<uint64_t>(tid) * kVec;
        f32x4 P[U], M[U], V[U];
        float G[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t e = base + static_cast<uint64_t>(u) * kGroup;
            grad4<GT, DT>(g, e, G[u]);
            P[u] = load_nt(reinterpret_cast<const f32x4 *>(master + e));
            M[u] = load_nt(reinterpret_cast<const f32x4 *>(m + e));
            V[u] = load_nt(reinterpret_cast<const f32x4 *>(v + e));
        }
        // one group at a time: its stores go out while the next group computes
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t e = base + static_cast<uint64_t>(u) * kGroup;
            float p[4] = {P[u].x, P[u].y, P[u].z, P[u].w};
            float mm[4] = {M[u].x, M[u].y, M[u].z, M[u].w};
            float vv[4] = {V[u].x, V[u].y, V[u].z, V[u].w};
            uint32_t w[4];
            adam_update<DT, MODE, 4>(G[u], p, mm, vv, w, s);
            store_nt(reinterpret_cast<f32x4 *>(master + e), f32x4{p[0], p[1], p[2], p[3]});
            store_nt(reinterpret_cast<f32x4 *>(m + e), f32x4{mm[0], mm[1], mm[2], mm[3]});
            store_nt(reinterpret_cast<f32x4 *>(v + e), f32x4{vv[0], vv[1], vv[2], vv[3]});
            store_nt(reinterpret_cast<u32x2 *>(w16 + e),
                     u32x2{w[0] | (w[1] << 16), w[2] | (w[3] << 16)});
        }
    }

    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kThreads;
    for (uint64_t i = head + n_tiles * kTile + static_cast<uint64_t>(blockIdx.x) * kThreads + tid;
         i < count; i += stride)
        adam_one<DT, MODE>(w16, g, master, m, v, i, s);
}

template <int DT, typename GT, int U, int MODE>
__global__ __launch_bounds__(kThreads) void adam_step_vec(
    uint16_t *__restrict__ w16, const GT *__restrict__ g, float *__restrict__ master,
    float *__restrict__ m, float *__restrict__ v, uint64_t count, uint32_t head,
    uint64_t n_tiles, AdamScalars s, const int32_t *__restrict__ flag,
    const zero_device_ctl *__restrict__ ctl) {
    if (flag != nullptr && *flag != 0) return;
    if constexpr (MODE == kUnscaleCtl) {
        if (ctl->apply == 0) return;
        if (take_device_scalars(ctl, s))
            step_tiles<DT, GT, U, kUnscaleMul>(w16, g, master, m, v, count, head, n_tiles, s);
        else
            step_tiles<DT, GT, U, kUnscaleRcp>(w16, g, master, m, v, count, head, n_tiles, s);
    } else {
        step_tiles<DT, GT, U, MODE>(w16, g, master, m, v, count, head, n_tiles, s);
    }
}

// ---- the step: element-wise path for views of different alignment phase --

template <int DT, typename GT, int MODE>
__device__ __forceinline__ void step_elems(uint16_t *__restrict__ w16, const GT *__restrict__ g,
                                           float *__restrict__ master, float *__restrict__ m,
                                           float *__restrict__ v, uint64_t count,
                                           const AdamScalars &s) {
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kThreads;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x; i < count;
         i += stride)
        adam_one<DT, MODE>(w16, g, master, m, v, i, s);
}

template <int DT, typename GT, int MODE>
__global__ __launch_bounds__(kThreads) void adam_step_elem(
    uint16_t *__restrict__ w16, const GT *__restrict__ g, float *__restrict__ master,
    float *__restrict__ m, float *__restrict__ v, uint64_t count, AdamScalars s,
    const int32_t *__restrict__ flag, const zero_device_ctl *__restrict__ ctl) {
    if (flag != nullptr && *flag != 0) return;
    if constexpr (MODE == kUnscaleCtl) {
        if (ctl->apply == 0) return;
        if (take_device_scalars(ctl, s))
            step_elems<DT, GT, kUnscaleMul>(w16, g, master, m, v, count, s);
        else
            step_elems<DT, GT, kUnscaleRcp>(w16, g, master, m, v, count, s);
    } else {
        step_elems<DT, GT, MODE>(w16, g, master, m, v, count, s);
    }
}

// ---- FP32 accumulation of 16-bit micro-batch gradients ----------------------
//
// acc = float(g16) on the first micro-batch, acc + float(g16) after it: one
// FP32 addition per element per micro-batch (10 B of traffic; 6 B for the
// first).  Same head / tile / tail split and alignment rule as the step.
//
// With CHECK the kernel also raises the overflow flag of the values it
// writes, as the check over FP32 gradients would on the result (some
// acc/S not finite): each lane keeps the largest magnitude bits it wrote and
// divides once at the end (correctly rounded division by S > 0 is monotone
// in |acc|), so the last micro-batch needs no separate 4-B/element check
// pass.  The flag is cleared by a kernel launched before this one.

struct AccCheck {
    float loss_scale;             // S, unless loss_scale_dev is set
    const float *loss_scale_dev;  // S read on the device, or null
    int32_t *flag;                // set to 1 by each wave that wrote a value with acc/S not finite
};

template <int DT, bool FIRST>
__device__ __forceinline__ float accumulate_one(float *__restrict__ acc,
                                                const uint16_t *__restrict__ g16, uint64_t i) {
    const float g = widen<DT>(g16[i]);
    const float r = FIRST ? g : acc[i] + g;
    acc[i] = r;
    return r;
}

__device__ __forceinline__ uint32_t magnitude_bits(float x) {
    return __builtin_bit_cast(uint32_t, x) & 0x7fffffffu;
}

// The flag from a lane's largest magnitude bits; every lane of the wave calls it.
__device__ __forceinline__ void accumulate_flag(uint32_t mx, const AccCheck &chk) {
    const float S = chk.loss_scale_dev != nullptr ? *chk.loss_scale_dev : chk.loss_scale;
    const uint32_t bad = mx >= 0x7f800000u || not_finite(__builtin_bit_cast(float, mx) / S) ||
                         !(S > 0.0f) || not_finite(S);
    if (__any(bad)) {
        if ((threadIdx.x & 63u) == 0) *chk.flag = 1;
    }
}

template <int DT, bool FIRST, int U, bool CHECK>
__global__ __launch_bounds__(kThreads) void accumulate_vec(float *__restrict__ acc,
                                                           const uint16_t *__restrict__ g16,
                                                           uint64_t count, uint32_t head,
                                                           uint64_t n_tiles, AccCheck chk) {
    const uint32_t tid = threadIdx.x;
    uint32_t mx = 0;
    auto note = [&](float r) {
        if constexpr (CHECK) {
            const uint32_t a = magnitude_bits(r);
            mx = a > mx ? a : mx;
        }
    };
    if (blockIdx.x == 0 && tid < head) note(accumulate_one<DT, FIRST>(acc, g16, tid));
    constexpr uint64_t kTile = static_cast<uint64_t>(U) * kGroup;
    for (uint64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
        const uint64_t base = head + t * kTile + static_cast<uint64_t>(tid) * kVec;
        float G[U][4];
        f32x4 A[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t e = base + static_cast<uint64_t>(u) * kGroup;
            grad4<uint16_t, DT>(g16, e, G[u]);
            if (!FIRST) A[u] = load_nt(reinterpret_cast<const f32x4 *>(acc + e));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t e = base + static_cast<uint64_t>(u) * kGroup;
            const f32x4 r = FIRST ? f32x4{G[u][0], G[u][1], G[u][2], G[u][3]}
                                  : f32x4{A[u].x + G[u][0], A[u].y + G[u][1], A[u].z + G[u][2],
                                          A[u].w + G[u][3]};
            store_nt(reinterpret_cast<f32x4 *>(acc + e), r);
            note(r.x);
            note(r.y);
            note(r.z);
            note(r.w);
        }
    }
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kThreads;
    for (uint64_t i = head + n_tiles * kTile + static_cast<uint64_t>(blockIdx.x) * kThreads + tid;
         i < count; i += stride)
        note(accumulate_one<DT, FIRST>(acc, g16, i));
    if constexpr (CHECK) accumulate_flag(mx, chk);
}

template <int DT, bool FIRST, bool CHECK>
__global__ __launch_bounds__(kThreads) void accumulate_elem(float *__restrict__ acc,
                                                            const uint16_t *__restrict__ g16,
                                                            uint64_t count, AccCheck chk) {
    uint32_t mx = 0;
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kThreads;
    for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x; i < count;
         i += stride) {
        const float r = accumulate_one<DT, FIRST>(acc, g16, i);
        if constexpr (CHECK) {
            const uint32_t a = magnitude_bits(r);
            mx = a > mx ? a : mx;
        }
    }
    if constexpr (CHECK) accumulate_flag(mx, chk);
}

// ---- unscale + overflow check ----------------------------------------------

__global__ void check_init(int32_t *__restrict__ flag, float *__restrict__ sumsq) {
    if (threadIdx.x == 0) {
        *flag = 0;
        if (sumsq != nullptr) *sumsq = 0.0f;
    }
}

// Elements per 16-B vector and the field of the magnitude bits at or above
// which a value is inf or NaN.
template <typename GT, int DT> struct GradBits;
template <> struct GradBits<uint16_t, 0> {
    static constexpr uint32_t kPerVec = 8, kExpField = 0x7c00u;
};
template <> struct GradBits<uint16_t, 1> {
    static constexpr uint32_t kPerVec = 8, kExpField = 0x7f80u;
};
template <int DT> struct GradBits<float, DT> {
    static constexpr uint32_t kPerVec = 4, kExpField = 0x7f800000u;
};

// Flag only.  Division by S > 0 correctly rounded is monotone in |g|, so
// some g/S is not finite iff some g is inf/NaN or the largest finite |g|
// divided by S overflows.  With the sign bit cleared, floating-point bit
// patterns order like their magnitudes, so each lane keeps the maximum of
// the magnitude bits (packed 16-bit maxima for 16-bit gradients) and divides
// once at the end: the pass is two integer operations per gradient and runs
// at read bandwidth.  Elements [0, head) and [head + kPerVec*n_vec, count)
// one at a time; in between, 16-B vectors in tiles of U*256: lane l of tile
// t reads vectors t*U*256 + u*256 + l, so every wave instruction covers one
// contiguous 1 KiB, and each block reads one tile (a loop only past the grid
// cap), like the step.
template <typename GT, int DT, int U>
__global__ __launch_bounds__(kThreads) void overflow_flag_kernel(
    const GT *__restrict__ g, uint64_t count, uint32_t head, uint64_t n_vec, float loss_scale,
    const float *__restrict__ loss_scale_dev, int32_t *__restrict__ flag) {
    using B = GradBits<GT, DT>;
    constexpr bool k16 = sizeof(GT) == 2;
    if (loss_scale_dev != nullptr) loss_scale = *loss_scale_dev;
    const uint32_t tid = threadIdx.x;
    u16x2 mx2 = {0, 0};
    uint32_t mx = 0;
    auto mag = [](GT x) -> uint32_t {
        if constexpr (k16)
            return x & 0x7fffu;
        else
            return __builtin_bit_cast(uint32_t, x) & 0x7fffffffu;
    };
    if (blockIdx.x == 0 && tid < head) mx = mag(g[tid]);

    auto fold = [&](const u32x4 &x) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (k16) {
                mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(u16x2, x[j] & 0x7fff7fffu));
            } else {
                const uint32_t a = x[j] & 0x7fffffffu;
                mx = a > mx ? a : mx;
            }
        }
    };
    const u32x4 *vec = reinterpret_cast<const u32x4 *>(g + head);
    constexpr uint64_t kTileVec = static_cast<uint64_t>(U) * kThreads;
    for (uint64_t t = blockIdx.x; t * kTileVec < n_vec; t += gridDim.x) {
        const uint64_t k0 = t * kTileVec + tid;
        u32x4 x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t k = k0 + static_cast<uint64_t>(u) * kThreads;
            x[u] = k < n_vec ? load_nt(vec + k) : u32x4{0u, 0u, 0u, 0u};  // 0: no magnitude
        }
#pragma unroll
        for (int u = 0; u < U; ++u) fold(x[u]);
    }
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kThreads;
    for (uint64_t i = head + n_vec * B::kPerVec + static_cast<uint64_t>(blockIdx.x) * kThreads + tid;
         i < count; i += stride) {
        const uint32_t a = mag(g[i]);
        mx = a > mx ? a : mx;
    }
    if constexpr (k16) {
        mx = mx > mx2.x ? mx : mx2.x;
        mx = mx > mx2.y ? mx : mx2.y;
    }
    float largest;
    if constexpr (k16)
        largest = widen<DT>(mx);
    else
        largest = __builtin_bit_cast(float, mx);
    const uint32_t bad = mx >= B::kExpField || not_finite(largest / loss_scale) ||
                         !(loss_scale > 0.0f) || not_finite(loss_scale);
    if (__any(bad)) {
        if ((tid & 63u) == 0) *flag = 1;
    }
}

// One DPP move of a double (both 32-bit halves with the same control); lanes
// whose source is outside the row, or whose row is masked off, read 0.
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ double dpp_move(double x) {
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(static_cast<uint32_t>(b)), kCtrl, kRowMask, 0xf, true));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
        0, static_cast<int>(static_cast<uint32_t>(b >> 32)), kCtrl, kRowMask, 0xf, true));
    return __builtin_bit_cast(double, static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
}

// Sum of a wave's 64 doubles, left in lane 63, by DPP row operations in a
// fixed order: pairs and quads (quad permutes), then rows of 16 (row shifts
// by 4 and 8), then the four rows (row broadcasts of lanes 15 and 31).
__device__ __forceinline__ double wave_sum_to_lane63(double x) {
    x += dpp_move<0xb1>(x);        // quad_perm [1,0,3,2]
    x += dpp_move<0x4e>(x);        // quad_perm [2,3,0,1]
    x += dpp_move<0x114>(x);       // row_shr:4
    x += dpp_move<0x118>(x);       // row_shr:8  (lane 15 of a row: the row's sum)
    x += dpp_move<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_move<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

// Flag and sum of squares.  Every gradient is unscaled and squared as its
// definition says, with exact shortcuts for the unscaling and the sum:
//  - S a power of two whose reciprocal is a normal number: g * (1/S) is the
//    same correctly rounded value as g / S.
//  - Any other S: q = (float)((double)g * RN64(1/S)).  The FP64 product is
//    within 2^-52 (relative) of g/S, and g/S is never within 2^-49 of a
//    point where rounding to FP32 changes: such a midpoint has a 25-bit odd
//    significand, which the product of S's odd significand (> 1) and a
//    16-bit or FP32 gradient's cannot equal, and two unequal multiples of a
//    power of two differ by at least that power.  So the one rounding to
//    FP32 gives exactly g / S -- wherever the quotient is a normal number.
//    A rounded quotient of at least 2^-125 in magnitude comes from a normal
//    one, and g = 0 gives 0 either way; every other gradient (g != 0 with
//    |q| < 2^-125) is divided as written.  One compare per gradient finds
//    the vectors that hold any quotient below 2^-125 (zeros included); only
//    those check their gradients one by one.
//  - q*q is exact in FP64 (a 24-bit significand squared), so one FP64 fma
//    equals the square followed by the addition.
//  - A lane's FP64 sum is not finite iff one of its q is (finite squares of
//    FP32 values cannot overflow an FP64 sum of fewer than 2^60 terms), so
//    the flag is read off the sums.
// Lanes accumulate in FP64 in element order, waves reduce by DPP, and block b
// writes its partial sum to partials[b].  Same element split as the flag
// kernel.
template <typename GT, int DT, int U>
__global__ __launch_bounds__(kThreads) void overflow_sumsq_kernel(
    const GT *__restrict__ g, uint64_t count, uint32_t head, uint64_t n_vec, float loss_scale,
    const float *__restrict__ loss_scale_dev, int32_t *__restrict__ flag,
    double *__restrict__ partials) {
    using B = GradBits<GT, DT>;
    if (loss_scale_dev != nullptr) loss_scale = *loss_scale_dev;
    const uint32_t tid = threadIdx.x;
    const bool scale_ok = loss_scale > 0.0f && !not_finite(loss_scale);
    const uint32_t sbits = __builtin_bit_cast(uint32_t, loss_scale);
    const uint32_t sexp = (sbits >> 23) & 0xffu;
    const bool pow2 = scale_ok && (sbits & 0x7fffffu) == 0 && sexp >= 1 && sexp <= 253;
    const float inv = 1.0f / loss_scale;                              // exact when pow2
    const double rcp = 1.0 / static_cast<double>(loss_scale);          // RN64(1/S)
    double acc = 0.0;

    auto run = [&](auto pow2_tag) {
        constexpr bool kPow2 = decltype(pow2_tag)::value;
        // K gradients: unscale all, divide those whose product may have
        // missed the quotient (never with the power-of-two multiply), then
        // add the squares in order
        auto visit_n = [&](auto k_tag, const float *gr) {
            constexpr int K = decltype(k_tag)::value;
            float q[K];
            bool tiny = false;
#pragma unroll
            for (int j = 0; j < K; ++j) {
                if constexpr (kPow2) {
                    q[j] = gr[j] * inv;
                } else {
                    q[j] = static_cast<float>(static_cast<double>(gr[j]) * rcp);
                    tiny |= __builtin_fabsf(q[j]) < 0x1p-125f;
                }
            }
            if (!kPow2 && tiny) {
#pragma unroll
                for (int j = 0; j < K; ++j)
                    if (gr[j] != 0.0f && __builtin_fabsf(q[j]) < 0x1p-125f)
                        q[j] = gr[j] / loss_scale;
            }
#pragma unroll
            for (int j = 0; j < K; ++j) {
                const double qd = static_cast<double>(q[j]);
                acc = __builtin_fma(qd, qd, acc);
            }
        };
        auto visit_vec = [&](const u32x4 &x) {
            if constexpr (sizeof(GT) == 2) {
                float gr[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    gr[2 * j] = widen<DT>(x[j] & 0xffffu);
                    gr[2 * j + 1] = widen<DT>(x[j] >> 16);
                }
                visit_n(std::integral_constant<int, 8>{}, gr);
            } else {
                // copy each lane out first: bit-casting the vector element in
                // place made the compiler reuse one element for all four
                float gr[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t bits = x[j];
                    gr[j] = __builtin_bit_cast(float, bits);
                }
                visit_n(std::integral_constant<int, 4>{}, gr);
            }
        };
        auto visit = [&](float graw) { visit_n(std::integral_constant<int, 1>{}, &graw); };
        if (blockIdx.x == 0 && tid < head) visit(grad_at<GT, DT>(g, tid));
        const u32x4 *vec = reinterpret_cast<const u32x4 *>(g + head);
        const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kThreads;
        uint64_t k = static_cast<uint64_t>(blockIdx.x) * kThreads + tid;
        for (; k + (U - 1) * stride < n_vec; k += U * stride) {
            u32x4 x[U];
#pragma unroll
            for (int u = 0; u < U; ++u) x[u] = load_nt(vec + k + u * stride);
#pragma unroll
            for (int u = 0; u < U; ++u) visit_vec(x[u]);
        }
        for (; k < n_vec; k += stride) visit_vec(load_nt(vec + k));
        for (uint64_t i = head + n_vec * B::kPerVec + static_cast<uint64_t>(blockIdx.x) * kThreads +
                          tid;
             i < count; i += stride)
            visit(grad_at<GT, DT>(g, i));
    };
    if (pow2)
        run(std::true_type{});
    else
        run(std::false_type{});

    const uint64_t abits = __builtin_bit_cast(uint64_t, acc);
    const bool bad = !scale_ok || ((abits >> 52) & 0x7ffu) == 0x7ffu;
    if (__any(bad)) {
        if ((tid & 63u) == 0) *flag = 1;
    }
    acc = wave_sum_to_lane63(acc);
    __shared__ double wave_sum[kThreads / 64];
    if ((tid & 63u) == 63u) wave_sum[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) {
        double b = 0.0;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) b += wave_sum[w];
        partials[blockIdx.x] = b;
    }
}

// Sum the per-block partials in a fixed order and round once to FP32.
__global__ __launch_bounds__(kThreads) void sumsq_finalize(const double *__restrict__ partials,
                                                           uint32_t n_parts,
                                                           float *__restrict__ sumsq) {
    __shared__ double red[kThreads];
    const uint32_t tid = threadIdx.x;
    double a = 0.0;
    for (uint32_t i = tid; i < n_parts; i += kThreads) a += partials[i];
    red[tid] = a;
    __syncthreads();
    for (uint32_t h = kThreads / 2; h > 0; h >>= 1) {
        if (tid < h) red[tid] += red[tid + h];
        __syncthreads();
    }
    if (tid == 0) *sumsq = static_cast<float>(red[0]);
}

// ---- skip-or-apply decision on the device ---------------------------------
//
// One lane applies the host policy of zero_scaler_update to the control
// block: overflow halves S; a clean step advances t, doubles S after a run of
// growth_interval clean steps (unless 2S overflows), and records the S the
// update unscales with and the bias corrections of t from the host's table,
// with the FP64 reciprocals of all three.
__global__ void scaler_decide(zero_device_ctl *__restrict__ ctl, const float *__restrict__ bias,
                              uint64_t t_first, uint32_t len) {
    if (threadIdx.x != 0) return;
    zero_scaler sc = ctl->scaler;
    const float S = sc.loss_scale;
    if (!(S > 0.0f) || not_finite(S)) {
        ctl->apply = 0;
        ctl->status = ZERO_EINVAL;
        return;
    }
    if (ctl->found_inf != 0) {
        sc.loss_scale = S * 0.5f;
        sc.clean_steps = 0;
        ctl->scaler = sc;
        ctl->apply = 0;
        ctl->status = ZERO_OK;
        return;
    }
    const uint64_t t = sc.step + 1;
    if (t < t_first || t - t_first >= len) {
        ctl->apply = 0;
        ctl->status = ZERO_ERANGE;
        return;
    }
    sc.step = t;
    sc.clean_steps += 1;
    if (sc.growth_interval != 0 && sc.clean_steps >= sc.growth_interval) {
        const float grown = S * 2.0f;
        if (!not_finite(grown)) sc.loss_scale = grown;
        sc.clean_steps = 0;
    }
    ctl->scaler = sc;
    const float bc1 = bias[t - t_first], bc2 = bias[len + (t - t_first)];
    ctl->loss_scale_used = S;
    ctl->bc1 = bc1;
    ctl->bc2 = bc2;
    // FP64 division is correctly rounded, as on the host
    ctl->rcp_loss_scale = 1.0 / static_cast<double>(S);
    ctl->rcp_bc1 = 1.0 / static_cast<double>(bc1);
    ctl->rcp_bc2 = 1.0 / static_cast<double>(bc2);
    ctl->apply = 1;
    ctl->status = ZERO_OK;
}

// ---- launch helpers --------------------------------------------------------

constexpr int kAdamU = 2;              // groups in flight per lane in the step
constexpr int kAccU = 2;               // groups in flight per lane in the accumulate
constexpr int kCheckU = 4;             // 16-B vectors in flight per lane in the check
// The flag-only check reads one tile of 4 x 256 vectors per block, 3 resident
// blocks per CU from 128 MiB of gradients (measured on MI355X, same arrays,
// TB/s against the grid-stride loop it replaced at 7 or 128 blocks per CU):
// 1e10 FP16 gradients 7.35-7.40 against 6.77-7.07, 937.5M 7.17-7.29
// against 6.62-6.86, 137.7M 6.93-6.99 against 6.57-6.66 (2 per CU: 6.1-7.0,
// 4: 6.8-7.1, uncapped: 6.8-7.3); below, uncapped (15.5M: 5.6 TB/s, the
// same as before).  The sum of squares takes at most 1792 blocks (one round
// on 256 CUs) whatever the device, so its partial sums depend on the size
// and the view's phase only.
constexpr uint64_t kCheckCapFromBytes = 128ull << 20;
constexpr int kCheckCapPerCU = 3;
constexpr uint32_t kSumsqBlocks = 1792;
static_assert(kSumsqBlocks <= kSumsqPartials, "one partial per block");
static_assert(kSumsqPartials == ZERO_SUMSQ_PARTIALS, "the caller's and the fixed partials agree");

inline uintptr_t addr(const void *p) { return reinterpret_cast<uintptr_t>(p); }

inline uint32_t align_head(uintptr_t a, uint32_t elem_bytes, uint32_t align) {
    // elements to skip until a is `align`-aligned (a is elem-aligned)
    const uintptr_t mis = a % align;
    return mis == 0 ? 0u : static_cast<uint32_t>((align - mis) / elem_bytes);
}

// Bytes of a cache line: vector parts start on one, so every wave's 1 KB (FP32)
// or 512 B (16-bit) access covers whole lines.  A view that starts mid-line
// otherwise costs about a fifth of the bandwidth (partial first and last line
// of every access).
constexpr uint32_t kLine = 128;

// Head that aligns the FP32 reference array to a cache line, and whether it
// also leaves every other view vector-aligned: FP32 arrays (a, b, FP32
// gradients) at 16 B and 16-bit arrays (16-bit gradients, h16) at 8 B.  When
// a head of up to 63 elements puts the 16-bit view on a line as well (it
// does whenever the views share one element phase), that one is taken: a
// wave's 512-B 16-bit access then covers whole lines too.  Either head is
// congruent mod 4 to the one that aligns ref to 16 B, so the test is the same
// as for a 16-B head.  b and h16 may be null.
template <typename GT>
bool common_phase(const float *ref, const float *a, const float *b, const GT *g,
                  const uint16_t *h16, uint32_t *head) {
    *head = align_head(addr(ref), 4, kLine);
    const uint16_t *v16 = h16;
    if constexpr (sizeof(GT) == 2) v16 = g;
    if (v16 != nullptr) {
        const uint32_t h2 = align_head(addr(v16), 2, kLine);
        if ((addr(ref) + 4ull * h2) % kLine == 0) *head = h2;
    }
    const bool g_ok = sizeof(GT) == 2 ? (addr(g) + 2u * *head) % 8 == 0
                                      : addr(g) % 16 == addr(ref) % 16;
    return addr(a) % 16 == addr(ref) % 16 && (b == nullptr || addr(b) % 16 == addr(ref) % 16) &&
           g_ok && (h16 == nullptr || (addr(h16) + 2u * *head) % 8 == 0);
}

// Resident step blocks per CU.  One tile per block keeps the hardware
// dispatcher feeding CUs in tile order; how many tiles are in flight at once
// is set by reserving LDS the kernel does not use (the code and the bytes
// moved are the same).  Two per CU (8 waves) is the one rule, for every size,
// format and gradient type.  Measured on MI355X with the arrays of one process
// timed under every setting in turn, three rounds, three fresh processes per
// size (median TB/s at 2 / 3 / 4 / uncapped blocks per CU):
//   FP16: 15.5M 6.11 / 5.80 / 5.79 / 5.81; 2^26 6.29 / 6.02 / 5.95 / 5.80;
//     137.7M (view phase 5) 6.00 / 5.70 / 5.69 / 5.64; 2^32 6.29 / 5.78 /
//     5.72 / 5.58; 1e10 6.18 / 5.98 / 6.02 / 5.99 (one process placed the
//     160 GB well: 6.45 / 6.54 / 6.49 / 6.47).
//   BF16: 2^28 6.27 / 5.90 / 5.81 / 5.66; 937.5M 6.26 / 5.81 / 5.74 / 5.53;
//     1.5e9 6.03 / 5.65 / 5.63 / 5.44.
//   FP32 gradients (30 B per element): 2^30 5.98 / 5.58 / 5.59 / 5.47;
//     2^32 6.44 / 6.45 / 6.46 / 6.43.
constexpr int kStepPerCU = 2;

// The accumulate (three streams, the same tiles) gains more from fewer blocks:
// 2 per CU run 2^28 elements at 6.35-6.44 TB/s against 6.07-6.17 uncapped,
// 2^30 at 6.37-6.40 against 5.84-5.91 and 2^32 at 6.33-6.39 against
// 5.78-5.85; at 15.5M the cap loses (6.07-6.33 against 6.47-6.63).  The first
// micro-batch (a 16-bit read and an FP32 write, nothing read back) wants 4:
// 6.48-6.53 TB/s against 5.97-6.10 uncapped and 4.96-4.99 at 2 per CU, from
// 2^28 to 2^32 elements.  So does the accumulate with the check fused in,
// whose blocks end with the divide: at 2^30 elements 1.704-1.730 ms at 4 per
// CU against 1.772-1.782 at 2 and 1.799-1.828 uncapped.
constexpr uint64_t kAccCapFrom = 1ull << 28;
constexpr int kAccCapPerCU = 2;
constexpr int kAccFirstCapPerCU = 4;
constexpr int kAccCheckCapPerCU = 4;

inline size_t step_lds_bytes(const DeviceProps &dev) {
    return cap_lds_bytes(per_cu_or(kStepPerCU, dev), dev);
}

inline size_t accumulate_lds_bytes(uint64_t count, bool first, bool check,
                                   const DeviceProps &dev) {
    const int rule = count < kAccCapFrom ? 8
                     : first             ? kAccFirstCapPerCU
                     : check             ? kAccCheckCapPerCU
                                         : kAccCapPerCU;
    return cap_lds_bytes(per_cu_or(rule, dev), dev);
}

inline uint32_t grid_for(uint64_t need) {
    if (need == 0) need = 1;
    const uint64_t cap = max_blocks();
    return static_cast<uint32_t>(need < cap ? need : cap);
}

// Elements per launch of the step.  A shard of two or more such pieces goes
// out as launches of at most this many elements, back to back on one stream,
// which ran faster than one launch over the whole shard at every such size
// (MI355X, the arrays of one process timed under every setting in turn,
// median TB/s):
//   1e10 FP16, three processes, one launch / 2^28 / 2^27 / 2^26 / 2^25 / 2^24:
//     6.33 / 6.44 / 6.44 / 6.41 / 6.34 / 6.18;  6.32 / 6.42 / 6.41 / 6.38 /
//     6.31 / 6.16;  6.25 / 6.36 / 6.35 / 6.31 / 6.23 / 6.08
//   two processes each, one launch against 2^27: 937.5M BF16 6.09, 6.02 ->
//     6.21, 6.15; 1.5e9 BF16 6.00, 6.00 -> 6.17, 6.18; 2^32 FP16 6.22, 6.22 ->
//     6.41, 6.41; FP32 gradients 2^30 5.85, 5.51 -> 6.09, 5.61 and 2^32
//     6.33, 6.38 -> 6.43, 6.43
// Between 2^26 and 2^28 the sizes differ by less than the spread between
// processes; below 2^26 the gaps between launches cost more than the split
// gains.  Pieces of exactly 2^27 beat equal pieces of another size (1.5e9 BF16,
// three processes: 6.28 TB/s in 2^27-element launches, 6.22 in twelve equal
// ones), and a shard of less than two pieces runs best in one launch (137.7M
// FP16, three processes: 6.09 / 6.00 / 6.01 in one, 6.07 / 5.97 / 5.98 as
// 2^27 + the rest).
//   The accumulate with the fused check (a later micro-batch) gains as well,
// two processes each, one launch against 2^27: 2^30 6.16, 6.18 -> 6.22, 6.24;
// 2^32 6.26, 6.27 -> 6.31, 6.30; 2^33 6.19, 6.05 -> 6.25, 6.13.  The plain
// accumulate does not (2^30 6.35, 6.37 -> 6.35, 6.34; 2^33 6.34, 6.34 -> 6.34,
// 6.33) and the first micro-batch loses (2^30 6.41, 6.45 -> 6.38, 6.38; 2^33
// 6.50, 6.51 -> 6.44, 6.44), so those stay one launch.
constexpr uint64_t kStepPiece = 1ull << 27;

// Elements per launch of the flag-only check: one launch.  The same plan of
// back-to-back launches (one clear of the flag first) read 1e10 FP16
// gradients at 7.40-7.42 TB/s in launches of 2^30, 7.16-7.17 of 2^28 and
// 6.93-6.94 of 2^27, against 7.50 in one launch (three processes): a check
// launch is short, so its boundaries cost more than a read stream gains.
constexpr uint64_t kCheckPiece = 0;

template <int DT, typename GT, int MODE>
hipError_t adam_launch(uint16_t *w16, const GT *g, float *master, float *m, float *v,
                       uint64_t count, const AdamScalars &s, const int32_t *flag,
                       const zero_device_ctl *ctl, const DeviceProps &dev, hipStream_t stream) {
    uint32_t head = 0;
    if (!common_phase<GT>(master, m, v, g, w16, &head)) {
        adam_step_elem<DT, GT, MODE><<<grid_for((count + kThreads - 1) / kThreads), kThreads, 0,
                                       stream>>>(w16, g, master, m, v, count, s, flag, ctl);
        return hipGetLastError();
    }
    if (head > count) head = static_cast<uint32_t>(count);
    constexpr uint64_t kTile = static_cast<uint64_t>(kAdamU) * kGroup;
    const uint64_t n_tiles = (count - head) / kTile;
    const size_t lds = step_lds_bytes(dev);
    return by_pieces(
        count, head, n_tiles, kTile, piece_tiles(kStepPiece, kTile, n_tiles, dev),
        [&](uint64_t off, uint64_t cnt, uint32_t h, uint64_t nt) {
            const uint64_t r = cnt - h - nt * kTile;
            const uint64_t need = nt > 0 ? nt : (r + kThreads - 1) / kThreads;
            adam_step_vec<DT, GT, kAdamU, MODE><<<grid_for(need), kThreads, lds, stream>>>(
                w16 + off, g + off, master + off, m + off, v + off, cnt, h, nt, s, flag, ctl);
            return hipGetLastError();
        });
}

// The unscale mode: from the control block when there is one, else by S.
template <int DT, typename GT>
hipError_t adam_dispatch(uint16_t *w16, const GT *g, float *master, float *m, float *v,
                         uint64_t count, const AdamScalars &s, const int32_t *flag,
                         const zero_device_ctl *ctl, const DeviceProps &dev,
                         hipStream_t stream) {
    if (ctl != nullptr)
        return adam_launch<DT, GT, kUnscaleCtl>(w16, g, master, m, v, count, s, flag, ctl, dev,
                                                stream);
    if (s.scale_pow2)
        return adam_launch<DT, GT, kUnscaleMul>(w16, g, master, m, v, count, s, flag, ctl, dev,
                                                stream);
    return adam_launch<DT, GT, kUnscaleRcp>(w16, g, master, m, v, count, s, flag, ctl, dev,
                                            stream);
}

template <int DT, bool FIRST, bool CHECK>
hipError_t accumulate_dispatch(float *acc, const uint16_t *g16, uint64_t count,
                               const AccCheck &chk, const DeviceProps &dev, hipStream_t stream) {
    uint32_t head = 0;
    if (!common_phase<uint16_t>(acc, acc, nullptr, g16, nullptr, &head)) {
        accumulate_elem<DT, FIRST, CHECK><<<grid_for((count + kThreads - 1) / kThreads), kThreads,
                                            0, stream>>>(acc, g16, count, chk);
        return hipGetLastError();
    }
    if (head > count) head = static_cast<uint32_t>(count);
    constexpr uint64_t kTile = static_cast<uint64_t>(kAccU) * kGroup;
    const uint64_t n_tiles = (count - head) / kTile;
    const size_t lds = accumulate_lds_bytes(count, FIRST, CHECK, dev);
    return by_pieces(
        count, head, n_tiles, kTile,
        piece_tiles(CHECK && !FIRST ? kStepPiece : 0, kTile, n_tiles, dev),
        [&](uint64_t off, uint64_t cnt, uint32_t h, uint64_t nt) {
            const uint64_t r = cnt - h - nt * kTile;
            const uint64_t need = nt > 0 ? nt : (r + kThreads - 1) / kThreads;
            accumulate_vec<DT, FIRST, kAccU, CHECK><<<grid_for(need), kThreads, lds, stream>>>(
                acc + off, g16 + off, cnt, h, nt, chk);
            return hipGetLastError();
        });
}

struct CheckGrid {
    uint32_t head;    // elements done one at a time before the first line-aligned vector
    uint64_t n_vec;   // 16-B vectors
    uint32_t blocks;  // grid size (with a sum of squares: the number of partials)
    size_t lds;       // LDS reserved per block to cap resident blocks (flag only)
};

// With a sum of squares the grid depends on the size and the pointer's phase
// only, never on the device, so the partial sums and their order are the
// same everywhere.  The flag-only grid is one block per tile.
template <typename GT, int DT>
CheckGrid check_grid(const GT *g, uint64_t count, bool sumsq, const DeviceProps &dev) {
    CheckGrid c;
    c.head = align_head(addr(g), sizeof(GT), kLine);
    if (c.head > count) c.head = static_cast<uint32_t>(count);
    c.n_vec = (count - c.head) / GradBits<GT, DT>::kPerVec;
    const uint64_t rest = count - c.head - GradBits<GT, DT>::kPerVec * c.n_vec;
    const uint64_t per_block = static_cast<uint64_t>(kThreads) * kCheckU;
    uint64_t need = c.n_vec > 0 ? (c.n_vec + per_block - 1) / per_block
                                : (rest + kThreads - 1) / kThreads;
    if (need == 0) need = 1;
    const uint64_t cap = sumsq ? kSumsqBlocks : max_blocks();  // the partials' grid stays fixed
    c.blocks = static_cast<uint32_t>(need < cap ? need : cap);
    const int rule = count * sizeof(GT) >= kCheckCapFromBytes ? kCheckCapPerCU : 8;
    c.lds = sumsq ? 0 : cap_lds_bytes(per_cu_or(rule, dev), dev);
    return c;
}

template <typename GT, int DT>
hipError_t check_dispatch(const GT *g, uint64_t count, float loss_scale,
                          const float *loss_scale_dev, int32_t *flag, float *sumsq,
                          double *partials, const DeviceProps &dev, hipStream_t stream) {
    const CheckGrid c = check_grid<GT, DT>(g, count, sumsq != nullptr, dev);
    if (sumsq == nullptr) {
        // one block per tile of kCheckU * 256 vectors; a long shard may go out as
        // consecutive launches of whole tiles (the last one with the partial
        // tile and the elements after the last vector), all raising one flag
        constexpr uint64_t kTileVec = static_cast<uint64_t>(kThreads) * kCheckU;
        constexpr uint64_t kPer = GradBits<GT, DT>::kPerVec;
        const uint64_t n_tiles = c.n_vec / kTileVec;
        return by_pieces(
            count, c.head, n_tiles, kTileVec * kPer,
            piece_tiles(kCheckPiece, kTileVec * kPer, n_tiles, dev),
            [&](uint64_t off, uint64_t cnt, uint32_t h, uint64_t) {
                const uint64_t nv = (cnt - h) / kPer;
                const uint64_t need = nv > 0 ? (nv + kTileVec - 1) / kTileVec
                                             : (cnt - h + kThreads - 1) / kThreads;
                overflow_flag_kernel<GT, DT, kCheckU><<<grid_for(need), kThreads, c.lds, stream>>>(
                    g + off, cnt, h, nv, loss_scale, loss_scale_dev, flag);
                return hipGetLastError();
            });
    }
    overflow_sumsq_kernel<GT, DT, kCheckU><<<c.blocks, kThreads, 0, stream>>>(
        g, count, c.head, c.n_vec, loss_scale, loss_scale_dev, flag, partials);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    sumsq_finalize<<<1, kThreads, 0, stream>>>(partials, c.blocks, sumsq);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_adam_step(int dtype, uint16_t *w16, const uint16_t *g16, float *master, float *m,
                            float *v, uint64_t count, const AdamScalars &s, const int32_t *flag,
                            const zero_device_ctl *ctl, const DeviceProps &dev,
                            hipStream_t stream) {
    if (dtype == 0)
        return adam_dispatch<0>(w16, g16, master, m, v, count, s, flag, ctl, dev, stream);
    return adam_dispatch<1>(w16, g16, master, m, v, count, s, flag, ctl, dev, stream);
}

hipError_t launch_adam_step_g32(int dtype, uint16_t *w16, const float *g32, float *master,
                                float *m, float *v, uint64_t count, const AdamScalars &s,
                                const int32_t *flag, const zero_device_ctl *ctl,
                                const DeviceProps &dev, hipStream_t stream) {
    if (dtype == 0)
        return adam_dispatch<0>(w16, g32, master, m, v, count, s, flag, ctl, dev, stream);
    return adam_dispatch<1>(w16, g32, master, m, v, count, s, flag, ctl, dev, stream);
}

hipError_t launch_grad_accumulate(int dtype, float *acc, const uint16_t *g16, uint64_t count,
                                  bool first, const DeviceProps &dev, hipStream_t stream) {
    const AccCheck none{1.0f, nullptr, nullptr};
    if (dtype == 0)
        return first ? accumulate_dispatch<0, true, false>(acc, g16, count, none, dev, stream)
                     : accumulate_dispatch<0, false, false>(acc, g16, count, none, dev, stream);
    return first ? accumulate_dispatch<1, true, false>(acc, g16, count, none, dev, stream)
                 : accumulate_dispatch<1, false, false>(acc, g16, count, none, dev, stream);
}

hipError_t launch_clear_flag(int32_t *flag, hipStream_t stream) {
    check_init<<<1, 64, 0, stream>>>(flag, nullptr);
    return hipGetLastError();
}

hipError_t launch_grad_accumulate_check(int dtype, float *acc, const uint16_t *g16,
                                        uint64_t count, bool first, float loss_scale,
                                        const float *loss_scale_dev, int32_t *flag,
                                        const DeviceProps &dev, hipStream_t stream) {
    check_init<<<1, 64, 0, stream>>>(flag, nullptr);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess || count == 0) return err;
    const AccCheck chk{loss_scale, loss_scale_dev, flag};
    if (dtype == 0)
        return first ? accumulate_dispatch<0, true, true>(acc, g16, count, chk, dev, stream)
                     : accumulate_dispatch<0, false, true>(acc, g16, count, chk, dev, stream);
    return first ? accumulate_dispatch<1, true, true>(acc, g16, count, chk, dev, stream)
                 : accumulate_dispatch<1, false, true>(acc, g16, count, chk, dev, stream);
}

hipError_t launch_overflow_check(int dtype, const uint16_t *g16, uint64_t count, float loss_scale,
                                 const float *loss_scale_dev, int32_t *flag, float *sumsq,
                                 double *partials, const DeviceProps &dev, hipStream_t stream) {
    check_init<<<1, 64, 0, stream>>>(flag, sumsq);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess || count == 0) return err;
    if (dtype == 0)
        return check_dispatch<uint16_t, 0>(g16, count, loss_scale, loss_scale_dev, flag, sumsq,
                                           partials, dev, stream);
    return check_dispatch<uint16_t, 1>(g16, count, loss_scale, loss_scale_dev, flag, sumsq,
                                       partials, dev, stream);
}

hipError_t launch_overflow_check_g32(const float *g32, uint64_t count, float loss_scale,
                                     const float *loss_scale_dev, int32_t *flag, float *sumsq,
                                     double *partials, const DeviceProps &dev,
                                     hipStream_t stream) {
    check_init<<<1, 64, 0, stream>>>(flag, sumsq);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess || count == 0) return err;
    return check_dispatch<float, 0>(g32, count, loss_scale, loss_scale_dev, flag, sumsq,
                                    partials, dev, stream);
}

hipError_t launch_scaler_decide(zero_device_ctl *ctl, const float *bias, uint64_t t_first,
                                uint32_t len, hipStream_t stream) {
    scaler_decide<<<1, 64, 0, stream>>>(ctl, bias, t_first, len);
    return hipGetLastError();
}

namespace {

// Device address of `scratch` on each device, looked up once per device with
// that device current (each device holds its own copy at its own address).
constexpr int kScratchDevices = 64;
std::atomic<double *> g_scratch[kScratchDevices];

hipError_t scratch_on_current_device(double **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    double *p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void *addr = nullptr;
        e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (addr == nullptr) return hipErrorInvalidSymbol;
        p = static_cast<double *>(addr);
        g_scratch[dev].store(p, std::memory_order_release);  // same value from any thread
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

int scratch_partials_capacity() { return ZERO_SUMSQ_PARTIALS; }

uint64_t sumsq_partials_needed(int dtype, const void *g, uint64_t count) {
    const DeviceProps none{1, 0, 0, 0};  // the sum-of-squares grid ignores the device
    if (dtype == 2)
        return check_grid<float, 0>(static_cast<const float *>(g), count, true, none).blocks;
    return check_grid<uint16_t, 0>(static_cast<const uint16_t *>(g), count, true, none).blocks;
}

hipError_t launch_overflow_check_noalloc(int dtype, const uint16_t *g16, uint64_t count,
                                         float loss_scale, int32_t *flag, float *sumsq,
                                         const DeviceProps &dev, hipStream_t stream) {
    double *partials = nullptr;
    if (sumsq != nullptr) {
        const hipError_t e = scratch_on_current_device(&partials);
        if (e != hipSuccess) return e;
    }
    return launch_overflow_check(dtype, g16, count, loss_scale, nullptr, flag, sumsq, partials,
                                 dev, stream);
}

}  // namespace zs
