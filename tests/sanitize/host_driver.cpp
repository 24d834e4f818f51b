// Calls the library's host-only entry points (layout, loss-scale decision,
// communication and memory accounting, sharded checkpoints) on heap buffers
// of exactly the sizes they may touch, for a build of their sources with
// AddressSanitizer and UndefinedBehaviorSanitizer.  argv[1]: a scratch
// directory.  Prints "ok" when every call returned what its declaration in
// zero_shard.h promises; the sanitizers abort on any memory or arithmetic
// error.
#include <unistd.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "zero_shard.h"

static int bad = 0;
#define EXPECT(c)                                                     \
    do {                                                              \
        if (!(c)) {                                                   \
            std::fprintf(stderr, "line %d: %s\n", __LINE__, #c);      \
            ++bad;                                                    \
        }                                                             \
    } while (0)

static void layouts() {
    zero_layout lay;
    for (uint64_t psi = 1; psi <= 300; ++psi)
        for (uint32_t n = 1; n <= 40; ++n) {
            uint64_t total = 0;
            for (uint32_t r = 0; r < n; ++r) {
                EXPECT(zero_shard_layout(psi, n, r, &lay) == ZERO_OK);
                total += lay.count;
            }
            EXPECT(total == psi);
        }
    EXPECT(zero_shard_layout(0, 8, 0, &lay) == ZERO_EINVAL);
    EXPECT(zero_shard_layout(10, 8, 8, &lay) == ZERO_EINVAL);
    EXPECT(zero_shard_layout(10, 8, 0, nullptr) == ZERO_EINVAL);
    EXPECT(zero_shard_layout(ZERO_MAX_PSI + 1, 8, 0, &lay) == ZERO_EINVAL);
    EXPECT(zero_shard_layout(ZERO_MAX_PSI, 1u << 31, (1u << 31) - 1, &lay) == ZERO_OK);
}

static void scaler() {
    zero_scaler s{65536.0f, 3, 0, 0};
    int32_t apply = -1;
    uint32_t r = 12345;
    for (int i = 0; i < 2000; ++i) {
        r = r * 1103515245u + 12345u;
        EXPECT(zero_scaler_update(&s, (r >> 28) == 0, &apply) == ZERO_OK);
    }
    zero_scaler big{3.0e38f, 1, 0, 0};
    EXPECT(zero_scaler_update(&big, 0, &apply) == ZERO_OK && big.loss_scale == 3.0e38f);
    zero_scaler zero{0.0f, 1, 0, 0};
    EXPECT(zero_scaler_update(&zero, 0, &apply) == ZERO_EINVAL);
    EXPECT(zero_scaler_update(nullptr, 0, &apply) == ZERO_EINVAL);
    EXPECT(zero_scaler_update(&s, 0, nullptr) == ZERO_EINVAL);
}

static void accounting() {
    zero_comm c;
    for (uint32_t stage = 0; stage <= 3; ++stage)
        for (uint32_t n = 1; n <= 64; n *= 2)
            EXPECT(zero_comm_volume(8810000003ull, n, stage, 2, &c) == ZERO_OK);
    EXPECT(zero_comm_volume(100, 8, 4, 2, &c) == ZERO_EINVAL);
    EXPECT(zero_comm_volume(100, 8, 0, 9, &c) == ZERO_EINVAL);
    EXPECT(zero_comm_volume(100, 8, 0, 2, nullptr) == ZERO_EINVAL);
    uint64_t bytes = 0;
    EXPECT(zero_peak_memory(7500000000ull, 64, 100000000, 2, 1u << 30, &bytes) == ZERO_OK);
    EXPECT(zero_peak_memory(100, 8, 101, 1, 0, &bytes) == ZERO_EINVAL);
    EXPECT(zero_peak_memory(ZERO_MAX_PSI, 1, ZERO_MAX_PSI, 0xffffffffu, ~0ull, &bytes) ==
           ZERO_EINVAL);
    EXPECT(zero_peak_memory(100, 8, 10, 1, 0, nullptr) == ZERO_EINVAL);
}

struct Slice {
    std::vector<uint16_t> w16;
    std::vector<float> master, m, v;
    explicit Slice(uint64_t n) : w16(n), master(n), m(n), v(n) {}
};

static void checkpoints(const std::string &dir) {
    const uint64_t psi = 1003;
    const uint32_t n_old = 3, n_new = 5;
    std::vector<std::string> paths;
    std::vector<float> flat(psi);
    for (uint64_t i = 0; i < psi; ++i) flat[i] = static_cast<float>(i) * 0.5f;
    for (uint32_t r = 0; r < n_old; ++r) {
        zero_layout lay;
        EXPECT(zero_shard_layout(psi, n_old, r, &lay) == ZERO_OK);
        Slice s(lay.count);
        for (uint64_t i = 0; i < lay.count; ++i) {
            s.w16[i] = static_cast<uint16_t>(lay.offset + i);
            s.master[i] = flat[lay.offset + i];
            s.m[i] = -s.master[i];
            s.v[i] = 2.0f * s.master[i];
        }
        zero_ckpt_info info{};
        info.psi = psi;
        info.n = n_old;
        info.rank = r;
        info.dtype = ZERO_BF16;
        info.scaler = zero_scaler{1024.0f, 2000, 7, 3};
        paths.push_back(dir + "/rank" + std::to_string(r) + ".zs");
        EXPECT(zero_ckpt_write(paths.back().c_str(), &info, s.w16.data(), s.master.data(),
                               s.m.data(), s.v.data()) == ZERO_OK);
        zero_ckpt_info back{};
        EXPECT(zero_ckpt_read_info(paths.back().c_str(), &back) == ZERO_OK &&
               back.count == lay.count && back.offset == lay.offset);
        EXPECT(zero_ckpt_verify(paths.back().c_str()) == ZERO_OK);
        Slice t(lay.count);
        EXPECT(zero_ckpt_read(paths.back().c_str(), 0, lay.count, t.w16.data(), t.master.data(),
                              t.m.data(), t.v.data()) == ZERO_OK);
        EXPECT(t.master == s.master && t.w16 == s.w16);
        EXPECT(zero_ckpt_read(paths.back().c_str(), 1, lay.count, t.w16.data(), t.master.data(),
                              t.m.data(), t.v.data()) == ZERO_EINVAL);
    }
    std::vector<const char *> cpaths;
    for (auto &p : paths) cpaths.push_back(p.c_str());
    for (uint32_t r = 0; r < n_new; ++r) {
        zero_layout lay;
        EXPECT(zero_shard_layout(psi, n_new, r, &lay) == ZERO_OK);
        uint32_t np = 0;
        EXPECT(zero_reshard_plan(psi, n_old, n_new, r, nullptr, 0, &np) == ZERO_OK);
        std::vector<zero_ckpt_piece> plan(np);
        EXPECT(zero_reshard_plan(psi, n_old, n_new, r, plan.data(), np, &np) == ZERO_OK);
        if (np > 0) {
            EXPECT(zero_reshard_plan(psi, n_old, n_new, r, plan.data(), np - 1, &np) ==
                   ZERO_ERANGE);
        }
        Slice s(lay.count);
        EXPECT(zero_ckpt_read_resharded(cpaths.data(), n_old, psi, n_new, r, s.w16.data(),
                                        s.master.data(), s.m.data(), s.v.data()) == ZERO_OK);
        for (uint64_t i = 0; i < lay.count; ++i) EXPECT(s.master[i] == flat[lay.offset + i]);
    }
    // a flipped payload byte fails the hash; a truncated file fails its size check
    {
        std::FILE *f = std::fopen(paths[1].c_str(), "r+b");
        EXPECT(f != nullptr);
        if (f != nullptr) {
            std::fseek(f, 200, SEEK_SET);
            const int c = std::fgetc(f);
            std::fseek(f, 200, SEEK_SET);
            std::fputc(c ^ 0x40, f);
            std::fclose(f);
        }
        EXPECT(zero_ckpt_verify(paths[1].c_str()) == ZERO_ECORRUPT);
    }
    EXPECT(truncate(paths[2].c_str(), 300) == 0);
    zero_ckpt_info info{};
    EXPECT(zero_ckpt_read_info(paths[2].c_str(), &info) == ZERO_ECORRUPT);
    EXPECT(zero_ckpt_verify((dir + "/missing.zs").c_str()) == ZERO_EIO);
    EXPECT(zero_ckpt_write((dir + "/nodir/x.zs").c_str(), &info, nullptr, nullptr, nullptr,
                           nullptr) != ZERO_OK);
}

int main(int argc, char **argv) {
    if (argc < 2) {
        std::fprintf(stderr, "usage: host_driver <scratch directory>\n");
        return 2;
    }
    layouts();
    scaler();
    accounting();
    checkpoints(argv[1]);
    if (bad != 0) {
        std::fprintf(stderr, "%d unexpected results\n", bad);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
