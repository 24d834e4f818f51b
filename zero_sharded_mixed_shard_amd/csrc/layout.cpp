// Shard layout of one data-parallel rank: host-only 64-bit integer arithmetic.
//
// Rank i owns chunk i of the flat buffer and the chunks are equal
// ("Training models too big for one GPU: ZeRO & FSDP", "Data parallelism and
// the all-reduce"; "ZeRO memory math" (tm_zero_math), "Stage 1 - P_os").
// With S = ceil(psi/n) the padding needed when n does not divide psi sits at
// the tail of the buffer.  Per-rank bytes follow the stage formulas ("ZeRO
// stages 1, 2 and 3"; "Stop Replicating What You Can Shard", "The three
// stages of ZeRO"): sharded terms hold S elements, replicated ones the padded
// buffer of n*S elements.
#include "zero_shard.h"

extern "C" int zero_shard_layout(uint64_t psi, uint32_t n, uint32_t rank, zero_layout *out) {
    if (out == nullptr || psi == 0 || psi > ZERO_MAX_PSI || n == 0 || rank >= n)
        return ZERO_EINVAL;
    const uint64_t shard = psi / n + (psi % n != 0 ? 1 : 0);
    const uint64_t offset = static_cast<uint64_t>(rank) * shard;
    const uint64_t left = offset < psi ? psi - offset : 0;
    const uint64_t count = left < shard ? left : shard;
    const uint64_t padded = static_cast<uint64_t>(n) * shard;

    zero_layout l;
    l.psi = psi;
    l.shard = shard;
    l.offset = offset;
    l.count = count;
    l.pad = shard - count;
    l.padded_total = padded;
    l.n = n;
    l.rank = rank;
    l.bytes_dp = (2 + 2 + 12) * psi;               // weights + grads + (master, m, v)
    l.bytes_z1 = (2 + 2) * padded + 12 * shard;    // optimizer states split
    l.bytes_z2 = 2 * padded + (2 + 12) * shard;    // + gradients split
    l.bytes_z3 = (2 + 2 + 12) * shard;             // + weights split
    *out = l;
    return ZERO_OK;
}
