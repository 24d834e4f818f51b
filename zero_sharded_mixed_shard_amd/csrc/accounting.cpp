// Communication and peak-memory accounting of one data-parallel step:
// host-only 64-bit integer arithmetic, no device access.
//
// Per rank per step, plain data parallelism and ZeRO stages 1 and 2 move 2 psi
// elements (a reduce-scatter and an all-gather of psi each) and stage 3 moves
// 3 psi (the weights are gathered again for the backward pass) ("How far does
// splitting the batch get you?", "What does each stage cost on the wire?";
// "Stop Replicating What You Can Shard", FSDP communication).  A ring
// collective over an M-byte message sends (d-1)/d of it per rank, in d-1
// sequential hops ("Why does the all-reduce not get more expensive with more
// ranks?").  Stage-3 peak memory is the persistent 16 psi / N shard plus the
// 16-bit weights of the units gathered at once plus activations ("ZeRO Stage 3
// Math", "Peak transient memory").
#include "zero_shard.h"

extern "C" int zero_comm_volume(uint64_t psi, uint32_t n, uint32_t stage, uint32_t elem_bytes,
                                zero_comm *out) {
    zero_layout lay;
    if (out == nullptr || stage > 3 || elem_bytes == 0 || elem_bytes > 8) return ZERO_EINVAL;
    if (zero_shard_layout(psi, n, 0, &lay) != ZERO_OK) return ZERO_EINVAL;
    const uint32_t collectives = stage == 3 ? 3 : 2;
    zero_comm c;
    c.collectives = collectives;
    c.ring_hops = collectives * (n - 1);
    c.elements = collectives * psi;
    c.wire_bytes = c.elements * elem_bytes;
    c.ring_bytes = static_cast<uint64_t>(collectives) * (n - 1) * lay.shard * elem_bytes;
    *out = c;
    return ZERO_OK;
}

extern "C" int zero_peak_memory(uint64_t psi, uint32_t n, uint64_t unit_params,
                                uint32_t units_resident, uint64_t activation_bytes,
                                uint64_t *out_bytes) {
    zero_layout lay;
    if (out_bytes == nullptr) return ZERO_EINVAL;
    if (zero_shard_layout(psi, n, 0, &lay) != ZERO_OK) return ZERO_EINVAL;
    if (unit_params > psi) return ZERO_EINVAL;
    uint64_t gathered = 0, total = 0;
    if (__builtin_mul_overflow(unit_params, 2ull * units_resident, &gathered) ||
        __builtin_add_overflow(lay.bytes_z3, gathered, &total) ||
        __builtin_add_overflow(total, activation_bytes, &total))
        return ZERO_EINVAL;
    *out_bytes = total;
    return ZERO_OK;
}
