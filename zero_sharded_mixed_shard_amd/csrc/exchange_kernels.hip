// gfx950 kernels that stand in, on one GPU, for the collectives around the
// sharded step: the reduce-scatter that hands rank r the sum of chunk r over
// all ranks, and the all-gather that puts every rank's chunk back into the
// full flat buffer ("Training models too big for one GPU: ZeRO & FSDP",
// "Data parallelism and the all-reduce").  Both are streams over HBM: the
// reduction reads n inputs and writes one output per element, the gather
// copies; lanes move 4 consecutive elements (8 B of 16-bit or 16 B of FP32
// data per array) with non-temporal accesses when every view shares one
// alignment phase, one element otherwise.
//
// The sum of an element is taken in FP32 over ranks 0..n-1 in order and
// rounded once to the output format, so the result does not depend on the
// launch shape.  Format codes: 0 FP16, 1 BF16, 2 FP32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch.h"

#pragma clang fp contract(off)

namespace zs {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int F> struct Fmt;  // element type of a format
template <> struct Fmt<0> { using T = uint16_t; };
template <> struct Fmt<1> { using T = uint16_t; };
template <> struct Fmt<2> { using T = float; };

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

// Four consecutive elements from a 8-B (16-bit) or 16-B (FP32) aligned address.
template <int F>
__device__ __forceinline__ void load4(const typename Fmt<F>::T *p, float out[4]) {
    if constexpr (F == 2) {
        const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
        out[0] = x.x;
        out[1] = x.y;
        out[2] = x.z;
        out[3] = x.w;
    } else {
        const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
        out[0] = to_f32<F>(static_cast<uint16_t>(x.x & 0xffffu));
        out[1] = to_f32<F>(static_cast<uint16_t>(x.x >> 16));
        out[2] = to_f32<F>(static_cast<uint16_t>(x.y & 0xffffu));
        out[3] = to_f32<F>(static_cast<uint16_t>(x.y >> 16));
    }
}

template <int F>
__device__ __forceinline__ void store4(typename Fmt<F>::T *p, const float v[4]) {
    if constexpr (F == 2) {
        __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4 *>(p));
    } else {
        const uint32_t a = from_f32<F>(v[0]), b = from_f32<F>(v[1]);
        const uint32_t c = from_f32<F>(v[2]), d = from_f32<F>(v[3]);
        __builtin_nontemporal_store(u32x2{a | (b << 16), c | (d << 16)},
                                    reinterpret_cast<u32x2 *>(p));
    }
}

// out[i] = sum over k < n of in_k[i] for i in [0, count), where in_k already
// points at rank r's first element of replica k.  Elements [0, head) and
// [head + 4*n_groups, count) one at a time; in between, 4 per lane.
template <int IN, int OUT>
__global__ __launch_bounds__(kThreads) void reduce_shard_kernel(
    typename Fmt<OUT>::T *__restrict__ out, ReplicaSet in, uint32_t n, uint64_t count,
    uint32_t head, uint64_t n_groups) {
    using TI = typename Fmt<IN>::T;
    const uint64_t tid = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kThreads;
    auto one = [&](uint64_t i) {
        float s = 0.0f;
        for (uint32_t k = 0; k < n; ++k) s = s + to_f32<IN>(static_cast<const TI *>(in.p[k])[i]);
        out[i] = from_f32<OUT>(s);
    };
    if (tid < head) one(tid);
    for (uint64_t q = tid; q < n_groups; q += stride) {
        const uint64_t e = head + q * kVec;
        float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (uint32_t k = 0; k < n; ++k) {
            float x[4];
            load4<IN>(static_cast<const TI *>(in.p[k]) + e, x);
#pragma unroll
            for (int j = 0; j < 4; ++j) s[j] = s[j] + x[j];
        }
        store4<OUT>(out + e, s);
    }
    for (uint64_t i = head + n_groups * kVec + tid; i < count; i += stride) one(i);
}

// full[k*S + i] = shard_k[i] for i < count_k; blockIdx.y = k.  A shard whose
// source and destination share an alignment phase is copied 4 elements per
// lane after its head; otherwise one at a time.
template <typename T>
__global__ __launch_bounds__(kThreads) void gather_kernel(T *__restrict__ full, GatherSet set,
                                                          uint64_t shard) {
    const uint32_t k = blockIdx.y;
    const T *__restrict__ src = static_cast<const T *>(set.p[k]);
    T *__restrict__ dst = full + static_cast<uint64_t>(k) * shard;
    const uint64_t count = set.count[k];
    const uint32_t head = set.head[k];
    const uint64_t tid = static_cast<uint64_t>(blockIdx.x) * kThreads + threadIdx.x;
    const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kThreads;
    if (!set.vec[k]) {
        for (uint64_t i = tid; i < count; i += stride) dst[i] = src[i];
        return;
    }
    if (tid < head) dst[tid] = src[tid];
    const uint64_t n_groups = (count - head) / kVec;
    using V = typename std::conditional<sizeof(T) == 4, f32x4, u32x2>::type;
    for (uint64_t q = tid; q < n_groups; q += stride) {
        const uint64_t e = head + q * kVec;
        __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const V *>(src + e)),
                                    reinterpret_cast<V *>(dst + e));
    }
    for (uint64_t i = head + n_groups * kVec + tid; i < count; i += stride) dst[i] = src[i];
}

inline uintptr_t addr(const void *p) { return reinterpret_cast<uintptr_t>(p); }

inline uint32_t blocks_for(uint64_t work) {
    uint64_t b = (work + kThreads - 1) / kThreads;
    if (b == 0) b = 1;
    return static_cast<uint32_t>(b < kMaxBlocks ? b : kMaxBlocks);
}

template <int IN, int OUT>
hipError_t reduce_dispatch(void *out, const ReplicaSet &in, uint32_t n, uint64_t count,
                           hipStream_t stream) {
    constexpr uint32_t in_b = IN == 2 ? 4 : 2, out_b = OUT == 2 ? 4 : 2;
    // head that aligns the output to 4 elements; vector path if it aligns every input too
    const uint32_t out_align = 4 * out_b;
    uint32_t head = static_cast<uint32_t>(((out_align - addr(out) % out_align) % out_align) / out_b);
    bool vec = true;
    for (uint32_t k = 0; k < n; ++k)
        if ((addr(in.p[k]) + static_cast<uint64_t>(head) * in_b) % (4 * in_b) != 0) vec = false;
    uint64_t n_groups = 0;
    if (!vec) {
        head = 0;  // every element one at a time, by the grid-stride tail loop
    } else {
        if (head > count) head = static_cast<uint32_t>(count);  // head < 4 <= block size
        n_groups = (count - head) / kVec;
    }
    const uint64_t work = n_groups > 0 ? n_groups : count;
    reduce_shard_kernel<IN, OUT><<<blocks_for(work), kThreads, 0, stream>>>(
        static_cast<typename Fmt<OUT>::T *>(out), in, n, count, head, n_groups);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce_shard(void *out, int out_fmt, const ReplicaSet &in, int in_fmt,
                               uint32_t n, uint64_t count, hipStream_t stream) {
#define ZS_REDUCE(I, O) \
    if (in_fmt == I && out_fmt == O) return reduce_dispatch<I, O>(out, in, n, count, stream);
    ZS_REDUCE(0, 0) ZS_REDUCE(0, 1) ZS_REDUCE(0, 2)
    ZS_REDUCE(1, 0) ZS_REDUCE(1, 1) ZS_REDUCE(1, 2)
    ZS_REDUCE(2, 0) ZS_REDUCE(2, 1) ZS_REDUCE(2, 2)
#undef ZS_REDUCE
    return hipErrorInvalidValue;
}

hipError_t launch_gather_shards(void *full, int elem_bytes, GatherSet &set, uint32_t n,
                                uint64_t shard, uint64_t max_count, hipStream_t stream) {
    const uint32_t vec_bytes = 4 * static_cast<uint32_t>(elem_bytes);
    for (uint32_t k = 0; k < n; ++k) {
        const uintptr_t s = addr(set.p[k]);
        const uintptr_t d = addr(full) + static_cast<uint64_t>(k) * shard * elem_bytes;
        const uint32_t head =
            static_cast<uint32_t>(((vec_bytes - s % vec_bytes) % vec_bytes) / elem_bytes);
        set.vec[k] = (s % vec_bytes == d % vec_bytes) && head <= set.count[k];
        set.head[k] = set.vec[k] ? head : 0;
    }
    const dim3 grid(blocks_for((max_count + kVec - 1) / kVec), n);
    if (elem_bytes == 4)
        gather_kernel<float><<<grid, kThreads, 0, stream>>>(static_cast<float *>(full), set, shard);
    else
        gather_kernel<uint16_t><<<grid, kThreads, 0, stream>>>(static_cast<uint16_t *>(full), set,
                                                               shard);
    return hipGetLastError();
}

}  // namespace zs
