// The launch plan of the streaming kernels (by_pieces, piece_tiles in
// launch.h), run on the host: for seeded random shards it records the
// launches a shard is cut into and checks that they tile [0, count) exactly,
// one after another; that the first launch keeps the shard's head and only
// the last one holds the ragged rest; that every later launch starts a whole
// number of tiles after the head (so the views keep the shard's alignment);
// that no launch exceeds the piece; and that piece_tiles follows its rule: an
// override as it stands, else pieces only for a shard of two or more.
// Prints "ok" on success.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "launch.h"

namespace {

struct Launch {
    uint64_t off, cnt, nt;
    uint32_t head;
};

uint64_t g_state = 0x9e3779b97f4a7c15ull;
uint64_t next() {  // splitmix64
    uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

int fail(const char *what, uint64_t count, uint32_t head, uint64_t piece) {
    std::printf("FAIL %s: count %llu head %u piece %llu\n", what,
                static_cast<unsigned long long>(count), head,
                static_cast<unsigned long long>(piece));
    return 1;
}

int check(uint64_t count, uint32_t head, uint64_t tile, uint64_t piece) {
    const uint64_t n_tiles = (count - head) / tile;
    std::vector<Launch> ls;
    const hipError_t e = zs::by_pieces(count, head, n_tiles, tile, piece,
                                       [&](uint64_t off, uint64_t cnt, uint32_t h, uint64_t nt) {
                                           ls.push_back({off, cnt, nt, h});
                                           return hipSuccess;
                                       });
    if (e != hipSuccess || ls.empty()) return fail("no launches", count, head, piece);
    const bool split = piece != 0 && n_tiles > piece;
    if (!split && ls.size() != 1) return fail("split without need", count, head, piece);
    if (split && ls.size() != (n_tiles + piece - 1) / piece)
        return fail("launch count", count, head, piece);
    uint64_t next_off = 0, tiles = 0;
    for (size_t i = 0; i < ls.size(); ++i) {
        const Launch &l = ls[i];
        const bool last = i + 1 == ls.size();
        if (l.off != next_off) return fail("gap or overlap", count, head, piece);
        if (l.head != (i == 0 ? head : 0)) return fail("head", count, head, piece);
        if (i > 0 && (l.off - head) % tile != 0) return fail("alignment", count, head, piece);
        if (split && l.nt > piece) return fail("piece exceeded", count, head, piece);
        if (split && !last && l.nt != piece) return fail("short middle piece", count, head, piece);
        const uint64_t rest = l.cnt - l.head - l.nt * tile;
        if (l.cnt < l.head + l.nt * tile) return fail("count below tiles", count, head, piece);
        if (!last && rest != 0) return fail("rest before the end", count, head, piece);
        if (last && rest >= tile) return fail("whole tile left in the rest", count, head, piece);
        next_off = l.off + l.cnt;
        tiles += l.nt;
    }
    if (next_off != count || tiles != n_tiles) return fail("coverage", count, head, piece);
    return 0;
}

int check_rule() {
    zs::DeviceProps dev{256, 163840, 65536, 0, 0};
    const uint64_t tile = 2048, rule = 1ull << 27, per = rule / tile;
    // the kernel's rule: one launch below two pieces, pieces from two on
    if (zs::piece_tiles(rule, tile, 2 * per - 1, dev) != 0) return 1;
    if (zs::piece_tiles(rule, tile, 2 * per, dev) != per) return 2;
    if (zs::piece_tiles(rule, tile, 4882812, dev) != per) return 3;
    if (zs::piece_tiles(0, tile, 4882812, dev) != 0) return 4;
    // an override as it stands, whatever the size
    dev.piece = 1;
    if (zs::piece_tiles(rule, tile, 5, dev) != 1) return 5;
    dev.piece = 3 * tile + 5;
    if (zs::piece_tiles(0, tile, 5, dev) != 3) return 6;
    dev.piece = ~0ull;
    if (zs::piece_tiles(rule, tile, 4882812, dev) != (~0ull) / tile) return 7;
    return 0;
}

}  // namespace

int main() {
    if (const int r = check_rule()) {
        std::printf("FAIL piece_tiles rule %d\n", r);
        return 1;
    }
    int cases = 0;
    // fixed edges: empty tile range, exact multiples, one tile more or less
    const uint64_t tile = 2048;
    const uint64_t counts[] = {0, 1, 63, 2047, 2048, 2049, 7 * 2048, 7 * 2048 + 63,
                               10000000000ull, (1ull << 28) + 12345};
    const uint64_t pieces[] = {0, 1, 2, 3, 7, 65536, 1ull << 40};
    for (uint64_t c : counts)
        for (uint32_t h : {0u, 5u, 63u})
            for (uint64_t p : pieces) {
                if (h > c) continue;
                if (p != 0 && (c - h) / tile / p > 100000) continue;
                if (check(c, h, tile, p)) return 1;
                ++cases;
            }
    // seeded random shards: sizes over 40 bits, heads below 64 elements
    for (int i = 0; i < 20000; ++i) {
        const uint64_t count = next() >> (24 + next() % 40);
        const uint32_t head = static_cast<uint32_t>(next() % (count < 63 ? count + 1 : 64));
        const uint64_t n_tiles = (count - head) / tile;
        uint64_t piece = next() % 4 == 0 ? 0 : 1 + next() % (n_tiles + 2);
        if (piece != 0 && n_tiles / piece > 20000) piece = n_tiles / 20000 + 1;
        if (check(count, head, tile, piece)) return 1;
        ++cases;
    }
    // the launch callback's error stops the plan at once
    int calls = 0;
    const hipError_t e = zs::by_pieces(100 * tile, 0, 100, tile, 10,
                                       [&](uint64_t, uint64_t, uint32_t, uint64_t) {
                                           return ++calls == 3 ? hipErrorInvalidValue : hipSuccess;
                                       });
    if (e != hipErrorInvalidValue || calls != 3) {
        std::printf("FAIL error not propagated\n");
        return 1;
    }
    std::printf("%d launch plans checked\nok\n", cases);
    return 0;
}
