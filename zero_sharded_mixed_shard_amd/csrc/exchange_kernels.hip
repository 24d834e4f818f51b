// gfx950 kernels that stand in, on one GPU, for the collectives around the
// sharded step: the reduce-scatter that hands rank r the sum of chunk r over
// all ranks, and the all-gather that puts every rank's chunk back into the
// full flat buffer ("Training models too big for one GPU: ZeRO & FSDP",
// "Data parallelism and the all-reduce").  Both are streams over HBM: the
// reduction reads n inputs and writes one output per element, the gather
// copies.  When every view shares one 16-B alignment phase, each lane moves
// 16 B of every input per access (8 elements of 16-bit data, 4 of FP32) with
// non-temporal loads and stores, one 256-lane tile per block; the few
// elements before the first cache-line boundary and after the last whole
// vector are done one at a time.  Views of different phases take an element
// loop.
//
// The sum of an element is taken in FP32 over ranks 0..n-1 in order and
// rounded once to the output format, so the result does not depend on the
// launch shape.  Format codes: 0 FP16, 1 BF16, 2 FP32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

#pragma clang fp contract(off)

namespace zs {
namespace {

constexpr int kThreads = 256;
constexpr uint32_t kVecBytes = 16;  // bytes of each input a lane moves per access

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int F> struct Fmt;  // element type of a format
template <> struct Fmt<0> { using T = uint16_t; };
template <> struct Fmt<1> { using T = uint16_t; };
template <> struct Fmt<2> { using T = float; };

template <int F> constexpr uint32_t kBytes = F == 2 ? 4 : 2;
template <int F> constexpr int kPerVec = static_cast<int>(kVecBytes / kBytes<F>);

template <int F>
__device__ __forceinline__ float to_f32(typename Fmt<F>::T x) {
    if constexpr (F == 0)
        return static_cast<float>(__builtin_bit_cast(_Float16, x));
    else if constexpr (F == 1)
        return __builtin_bit_cast(float, static_cast<uint32_t>(x) << 16);
    else
        return x;
}

template <int F>
__device__ __forceinline__ typename Fmt<F>::T from_f32(float f) {
    if constexpr (F == 0)
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));  // RNE
    else if constexpr (F == 1)
        return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));    // RNE
    else
        return f;
}

// One 16-B vector (kPerVec<F> consecutive elements) from a 16-B aligned address,
// as raw bits; widen() turns it into FP32 values.
template <int F>
__device__ __forceinline__ u32x4 load_raw(const typename Fmt<F>::T *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

template <int F>
__device__ __forceinline__ void widen(const u32x4 &x, float out[kPerVec<F>]) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    if constexpr (F == 2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = __builtin_bit_cast(float, w[j]);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            out[2 * j] = to_f32<F>(static_cast<uint16_t>(w[j] & 0xffffu));
            out[2 * j + 1] = to_f32<F>(static_cast<uint16_t>(w[j] >> 16));
        }
    }
}

// K values stored in format F at an address aligned to min(16, K * bytes of F).
template <int F, int K>
__device__ __forceinline__ void store_vec(typename Fmt<F>::T *p, const float v[K]) {
    if constexpr (F == 2) {
#pragma unroll
        for (int h = 0; h < K / 4; ++h)
            __builtin_nontemporal_store(f32x4{v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]},
                                        reinterpret_cast<f32x4 *>(p + 4 * h));
    } else {
        uint32_t w[K / 2];
#pragma unroll
        for (int j = 0; j < K / 2; ++j)
            w[j] = static_cast<uint32_t>(from_f32<F>(v[2 * j])) |
                   (static_cast<uint32_t>(from_f32<F>(v[2 * j + 1])) << 16);
        if constexpr (K == 8)
            __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]},
                                        reinterpret_cast<u32x4 *>(p));
        else
            __builtin_nontemporal_store(u32x2{w[0], w[1]}, reinterpret_cast<u32x2 *>(p));
    }
}

// Magnitude bits of the value a format stores for the FP32 sum s: the value
// after rounding to the output format, as FP32 bits with the sign cleared.
// Non-negative FP32 bit patterns order like the values, so the largest
// magnitude a lane wrote is an integer maximum.
template <int OUT>
__device__ __forceinline__ uint32_t stored_magnitude(float s) {
    return __builtin_bit_cast(uint32_t, to_f32<OUT>(from_f32<OUT>(s))) & 0x7fffffffu;
}

// The flag of the check over the written values, from a lane's largest
// magnitude: some out[i] / S is not finite iff the largest finite |out[i]|
// divided by S overflows or some out[i] is inf or NaN (a correctly rounded
// division by S > 0 is monotone in |out[i]|).  Every lane of the wave calls it.
__device__ __forceinline__ void raise_check_flag(uint32_t mx, const ReduceCheck &chk) {
    const float S = chk.loss_scale_dev != nullptr ? *chk.loss_scale_dev : chk.loss_scale;
    const uint32_t e = 0x7f800000u;
    const uint32_t q = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, mx) / S);
    const bool bad = mx >= e || (q & e) == e || !(S > 0.0f) ||
                     (__builtin_bit_cast(uint32_t, S) & e) == e;
    if (__any(bad)) {
        if ((threadIdx.x & 63u) == 0) *chk.flag = 1;
    }
}

// out[i] = sum over k < n of in_k[i] for i in [0, count), where in_k already
// points at rank r's first element of replica k.  With n_vec > 0: vector q
// covers elements head + q*K .. +K-1 (K = kPerVec<IN>), one 256-vector tile
// per block, and block 0 does [0, head) and [head + n_vec*K, count) one at a
// time.  With n_vec == 0 the whole grid walks every element.
// out is not restrict-qualified: it may be one of the replicas' chunks (in
// place); every lane reads all replicas at its elements before it writes them.
// With CHECK the kernel also raises chk.flag (cleared by a kernel launched
// before it) iff some written out[i] / S is not finite: the overflow check of
// the result, with no second pass over it.
template <int IN, int OUT, bool CHECK>
__global__ __launch_bounds__(kThreads) void reduce_shard_kernel(
    typename Fmt<OUT>::T *out, ReplicaSet in, uint32_t n, uint64_t count,
    uint32_t head, uint64_t n_vec, ReduceCheck chk) {
    using TI = typename Fmt<IN>::T;
    constexpr int K = kPerVec<IN>;
    uint32_t mx = 0;   // largest magnitude written (CHECK)
    auto note = [&](float s) {
        if constexpr (CHECK) {
            const uint32_t a = stored_magnitude<OUT>(s);
            mx = a > mx ? a : mx;
        }
    };
    auto one = [&](uint64_t i) {
        float s = 0.0f;
        for (uint32_t k = 0; k < n; ++k) s = s + to_f32<IN>(static_cast<const TI *>(in.p[k])[i]);
        out[i] = from_f32<OUT>(s);
        note(s);
    };
    if (n_vec == 0) {
        const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kThreads;
        for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x; i < count;
             i += stride)
            one(i);
    } else {
        const uint64_t n_tiles = (n_vec + kThreads - 1) / kThreads;
        for (uint64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
            const uint64_t q = t * kThreads + threadIdx.x;
            if (q < n_vec) {
                const uint64_t e = head + q * K;
                float s[K];
#pragma unroll
                for (int j = 0; j < K; ++j) s[j] = 0.0f;
                // one replica at a time, in rank order: keeping several replicas' loads
                // in flight per lane (4 or 8, with or without an occupancy cap) measured
                // no better over sizes on MI355X -- nine streams at once are what limit it
                for (uint32_t k = 0; k < n; ++k) {
                    float x[K];
                    widen<IN>(load_raw<IN>(static_cast<const TI *>(in.p[k]) + e), x);
#pragma unroll
                    for (int j = 0; j < K; ++j) s[j] = s[j] + x[j];
                }
                store_vec<OUT, K>(out + e, s);
#pragma unroll
                for (int j = 0; j < K; ++j) note(s[j]);
            }
        }
        if (blockIdx.x == 0) {
            if (threadIdx.x < head) one(threadIdx.x);
            const uint64_t tail = head + n_vec * K + threadIdx.x;
            if (tail < count) one(tail);
        }
    }
    if constexpr (CHECK) raise_check_flag(mx, chk);
}

// full[k*S + i] = shard_k[i] for i < count_k; blockIdx.y = k.  A shard whose
// source and destination share a 16-B phase is copied 16 B per lane after its
// head (one 256-vector tile per block, block 0 doing head and tail); otherwise
// one element at a time over the whole grid.
// Not restrict-qualified: a shard may already sit at its place in full (an
// in-place all-gather), when each copy rewrites the value it read.
template <typename T>
__global__ __launch_bounds__(kThreads) void gather_kernel(T *full, GatherSet set, uint64_t shard) {
    constexpr uint32_t K = kVecBytes / sizeof(T);
    const uint32_t k = blockIdx.y;
    const T *src = static_cast<const T *>(set.p[k]);
    T *dst = full + static_cast<uint64_t>(k) * shard;
    const uint64_t count = set.count[k];
    const uint32_t head = set.head[k];
    if (!set.vec[k]) {
        const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kThreads;
        for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x; i < count;
             i += stride)
            dst[i] = src[i];
        return;
    }
    const uint64_t n_vec = (count - head) / K;
    const uint64_t n_tiles = (n_vec + kThreads - 1) / kThreads;
    for (uint64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
        const uint64_t q = t * kThreads + threadIdx.x;
        if (q < n_vec) {
            const uint64_t e = head + q * K;
            __builtin_nontemporal_store(
                __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + e)),
                reinterpret_cast<u32x4 *>(dst + e));
        }
    }
    if (blockIdx.x == 0) {
        if (threadIdx.x < head) dst[threadIdx.x] = src[threadIdx.x];
        const uint64_t tail = head + n_vec * K + threadIdx.x;
        if (tail < count) dst[tail] = src[tail];
    }
}

inline uintptr_t addr(const void *p) { return reinterpret_cast<uintptr_t>(p); }

inline uint32_t blocks_for(uint64_t work) {
    uint64_t b = (work + kThreads - 1) / kThreads;
    if (b == 0) b = 1;
    const uint64_t cap = max_blocks();
    return static_cast<uint32_t>(b < cap ? b : cap);
}

// Elements before the first cache-line (128-B) boundary of an element-aligned
// view.  Vector parts start there, so each wave's accesses cover whole lines;
// it is also 16-B aligned.
constexpr uint32_t kLine = 128;
inline uint32_t head_to_line(const void *p, uint32_t elem_bytes) {
    return static_cast<uint32_t>(((kLine - addr(p) % kLine) % kLine) / elem_bytes);
}

// Resident blocks per CU of the exchange kernels: no cap by default.
constexpr int kReducePerCU = 8;
constexpr int kGatherPerCU = 8;

template <int IN, int OUT>
hipError_t reduce_dispatch(void *out, const ReplicaSet &in, uint32_t n, uint64_t count,
                           const ReduceCheck &chk, const DeviceProps &dev, hipStream_t stream) {
    constexpr uint32_t in_b = kBytes<IN>, out_b = kBytes<OUT>;
    constexpr uint32_t K = kPerVec<IN>;
    constexpr uint32_t out_align = K * out_b < kVecBytes ? K * out_b : kVecBytes;
    // the head that puts replica 0 on a line; vectors if every view is then
    // aligned for its accesses
    uint32_t head = head_to_line(in.p[0], in_b);
    bool vec = head <= count && (addr(out) + static_cast<uint64_t>(head) * out_b) % out_align == 0;
    for (uint32_t k = 0; k < n && vec; ++k)
        if ((addr(in.p[k]) + static_cast<uint64_t>(head) * in_b) % kVecBytes != 0) vec = false;
    const uint64_t n_vec = vec ? (count - head) / K : 0;
    if (n_vec == 0) head = 0;  // every element one at a time
    const uint32_t blocks = blocks_for(n_vec > 0 ? n_vec : count);
    const size_t lds = cap_lds_bytes(per_cu_or(kReducePerCU, dev), dev);
    auto *o = static_cast<typename Fmt<OUT>::T *>(out);
    if (chk.flag != nullptr)
        reduce_shard_kernel<IN, OUT, true><<<blocks, kThreads, lds, stream>>>(o, in, n, count,
                                                                             head, n_vec, chk);
    else
        reduce_shard_kernel<IN, OUT, false><<<blocks, kThreads, lds, stream>>>(o, in, n, count,
                                                                              head, n_vec, chk);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce_shard(void *out, int out_fmt, const ReplicaSet &in, int in_fmt,
                               uint32_t n, uint64_t count, const ReduceCheck &chk,
                               const DeviceProps &dev, hipStream_t stream) {
    if (chk.flag != nullptr) {
        const hipError_t e = launch_clear_flag(chk.flag, stream);
        if (e != hipSuccess || count == 0) return e;
    }
#define ZS_REDUCE(I, O) \
    if (in_fmt == I && out_fmt == O) \
        return reduce_dispatch<I, O>(out, in, n, count, chk, dev, stream);
    ZS_REDUCE(0, 0) ZS_REDUCE(0, 1) ZS_REDUCE(0, 2)
    ZS_REDUCE(1, 0) ZS_REDUCE(1, 1) ZS_REDUCE(1, 2)
    ZS_REDUCE(2, 0) ZS_REDUCE(2, 1) ZS_REDUCE(2, 2)
#undef ZS_REDUCE
    return hipErrorInvalidValue;
}

hipError_t launch_gather_shards(void *full, int elem_bytes, GatherSet &set, uint32_t n,
                                uint64_t shard, uint64_t max_count, const DeviceProps &dev,
                                hipStream_t stream) {
    const uint32_t eb = static_cast<uint32_t>(elem_bytes);
    for (uint32_t k = 0; k < n; ++k) {
        const uintptr_t s = addr(set.p[k]);
        const uintptr_t d = addr(full) + static_cast<uint64_t>(k) * shard * eb;
        // the head that puts the destination on a line (the source shares its 16-B phase)
        const uint32_t head =
            static_cast<uint32_t>(((kLine - d % kLine) % kLine) / eb);
        set.vec[k] = (s % kVecBytes == d % kVecBytes) && head <= set.count[k];
        set.head[k] = set.vec[k] ? head : 0;
    }
    const uint64_t per_vec = kVecBytes / eb;
    const dim3 grid(blocks_for((max_count + per_vec - 1) / per_vec), n);
    const size_t lds = cap_lds_bytes(per_cu_or(kGatherPerCU, dev), dev);
    if (elem_bytes == 4)
        gather_kernel<float><<<grid, kThreads, lds, stream>>>(static_cast<float *>(full), set,
                                                              shard);
    else
        gather_kernel<uint16_t><<<grid, kThreads, lds, stream>>>(static_cast<uint16_t *>(full), set,
                                                                 shard);
    return hipGetLastError();
}

}  // namespace zs
