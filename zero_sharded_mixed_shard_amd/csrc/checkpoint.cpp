// Sharded checkpoints: each rank writes its own slice of the model states to
// its own file ("Stop Replicating What You Can Shard: ZeRO and FSDP", "Two
// memory levers you compose with sharding"), and a run can resume on a
// different number of ranks by reading, for each new rank, the pieces of the
// old shards that its range covers.  Host memory and host files only.
//
// File layout (little-endian):
//   header  (zero_ckpt_header below, 128 bytes)
//   w16     count x 2 bytes
//   master  count x 4 bytes
//   m       count x 4 bytes
//   v       count x 4 bytes
// The header carries a 64-bit hash of the payload: the payload is read as
// 8-byte little-endian words (the last one zero-padded), word i is folded into
// lane i mod 4 by FNV-1a (h ^= w; h *= prime), and the four lane values are
// then folded, lane 0 first, into one more FNV-1a state.  Four lanes give four
// independent multiply chains, so hashing keeps up with the file system.
#include <fcntl.h>
#include <unistd.h>

#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "zero_shard.h"

namespace {

constexpr char kMagic[8] = {'Z', 'S', 'H', 'A', 'R', 'D', '0', '1'};
constexpr uint32_t kVersion = 2;  // 2: four-lane payload hash

struct zero_ckpt_header {
    char magic[8];
    uint32_t version;
    uint32_t dtype;
    uint64_t psi;
    uint32_t n;
    uint32_t rank;
    uint64_t offset;
    uint64_t count;
    uint64_t step;
    uint64_t clean_steps;
    float loss_scale;
    uint32_t growth_interval;
    uint64_t payload_bytes;
    uint64_t payload_hash;
    uint8_t reserved[128 - 88];
};
static_assert(sizeof(zero_ckpt_header) == 128, "header size");

constexpr uint64_t kFnvOffset = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

// The payload hash: FNV-1a in four interleaved lanes over 8-byte words;
// `tail` carries a partial word between calls.
struct Hasher {
    uint64_t h[4] = {kFnvOffset, kFnvOffset, kFnvOffset, kFnvOffset};
    uint64_t words = 0;
    uint8_t tail[8];
    size_t tail_len = 0;

    static void fold(uint64_t &x, uint64_t w) {
        x ^= w;
        x *= kFnvPrime;
    }
    void word(uint64_t w) {
        fold(h[words & 3], w);
        ++words;
    }
    void add(const void *data, uint64_t bytes) {
        const uint8_t *p = static_cast<const uint8_t *>(data);
        while (bytes > 0 && tail_len > 0) {
            tail[tail_len++] = *p++;
            --bytes;
            if (tail_len == 8) {
                uint64_t w;
                std::memcpy(&w, tail, 8);
                word(w);
                tail_len = 0;
            }
        }
        while (bytes >= 8 && (words & 3) != 0) {
            uint64_t w;
            std::memcpy(&w, p, 8);
            word(w);
            p += 8;
            bytes -= 8;
        }
        while (bytes >= 32) {  // lane 0 next: four words, one per lane
            uint64_t w[4];
            std::memcpy(w, p, 32);
            fold(h[0], w[0]);
            fold(h[1], w[1]);
            fold(h[2], w[2]);
            fold(h[3], w[3]);
            words += 4;
            p += 32;
            bytes -= 32;
        }
        while (bytes >= 8) {
            uint64_t w;
            std::memcpy(&w, p, 8);
            word(w);
            p += 8;
            bytes -= 8;
        }
        while (bytes > 0) {
            tail[tail_len++] = *p++;
            --bytes;
        }
    }
    uint64_t finish() {
        if (tail_len > 0) {
            uint64_t w = 0;
            std::memcpy(&w, tail, tail_len);
            word(w);
            tail_len = 0;
        }
        uint64_t r = kFnvOffset;
        for (int j = 0; j < 4; ++j) fold(r, h[j]);
        return r;
    }
};

bool write_all(FILE *f, const void *p, uint64_t bytes) {
    const char *c = static_cast<const char *>(p);
    while (bytes > 0) {
        const size_t chunk = bytes > (1ull << 30) ? (1ull << 30) : static_cast<size_t>(bytes);
        if (std::fwrite(c, 1, chunk, f) != chunk) return false;
        c += chunk;
        bytes -= chunk;
    }
    return true;
}

bool read_all(FILE *f, void *p, uint64_t bytes) {
    char *c = static_cast<char *>(p);
    while (bytes > 0) {
        const size_t chunk = bytes > (1ull << 30) ? (1ull << 30) : static_cast<size_t>(bytes);
        if (std::fread(c, 1, chunk, f) != chunk) return false;
        c += chunk;
        bytes -= chunk;
    }
    return true;
}

uint64_t payload_bytes(uint64_t count) { return count * (2 + 4 + 4 + 4); }

// Read and check the header and the file size.
int read_header(FILE *f, zero_ckpt_header *h) {
    if (std::fread(h, sizeof *h, 1, f) != 1) return ZERO_ECORRUPT;
    if (std::memcmp(h->magic, kMagic, 8) != 0 || h->version != kVersion) return ZERO_ECORRUPT;
    if (h->dtype != ZERO_F16 && h->dtype != ZERO_BF16) return ZERO_ECORRUPT;
    zero_layout lay;
    if (zero_shard_layout(h->psi, h->n, h->rank, &lay) != ZERO_OK) return ZERO_ECORRUPT;
    if (lay.offset != h->offset || lay.count != h->count) return ZERO_ECORRUPT;
    if (h->payload_bytes != payload_bytes(h->count)) return ZERO_ECORRUPT;
    if (fseeko(f, 0, SEEK_END) != 0) return ZERO_EIO;
    const off_t size = ftello(f);
    if (size < 0) return ZERO_EIO;
    if (static_cast<uint64_t>(size) != sizeof *h + h->payload_bytes) return ZERO_ECORRUPT;
    return ZERO_OK;
}

void to_info(const zero_ckpt_header &h, zero_ckpt_info *info) {
    info->psi = h.psi;
    info->n = h.n;
    info->rank = h.rank;
    info->offset = h.offset;
    info->count = h.count;
    info->dtype = static_cast<zero_dtype>(h.dtype);
    info->scaler.loss_scale = h.loss_scale;
    info->scaler.growth_interval = h.growth_interval;
    info->scaler.step = h.step;
    info->scaler.clean_steps = h.clean_steps;
}

// Flush the directory entry of `path` after a rename, so that the new name
// survives a crash too; best effort (some file systems cannot sync a
// directory, and the file's own data is already on the device).
void sync_parent_dir(const char *path) {
    const std::string p(path);
    const size_t slash = p.find_last_of('/');
    const std::string dir = slash == std::string::npos ? "." : slash == 0 ? "/" : p.substr(0, slash);
    const int fd = open(dir.c_str(), O_RDONLY | O_DIRECTORY);
    if (fd < 0) return;
    (void)fsync(fd);
    close(fd);
}

}  // namespace

extern "C" int zero_ckpt_write(const char *path, const zero_ckpt_info *info, const void *w16,
                               const float *master, const float *m, const float *v) {
    if (path == nullptr || info == nullptr) return ZERO_EINVAL;
    if (info->dtype != ZERO_F16 && info->dtype != ZERO_BF16) return ZERO_EDTYPE;
    zero_layout lay;
    if (zero_shard_layout(info->psi, info->n, info->rank, &lay) != ZERO_OK) return ZERO_EINVAL;
    if (lay.count > 0 && (w16 == nullptr || master == nullptr || m == nullptr || v == nullptr))
        return ZERO_EINVAL;

    zero_ckpt_header h;
    std::memset(&h, 0, sizeof h);
    std::memcpy(h.magic, kMagic, 8);
    h.version = kVersion;
    h.dtype = static_cast<uint32_t>(info->dtype);
    h.psi = info->psi;
    h.n = info->n;
    h.rank = info->rank;
    h.offset = lay.offset;
    h.count = lay.count;
    h.step = info->scaler.step;
    h.clean_steps = info->scaler.clean_steps;
    h.loss_scale = info->scaler.loss_scale;
    h.growth_interval = info->scaler.growth_interval;
    h.payload_bytes = payload_bytes(lay.count);
    Hasher hs;
    hs.add(w16, lay.count * 2);
    hs.add(master, lay.count * 4);
    hs.add(m, lay.count * 4);
    hs.add(v, lay.count * 4);
    h.payload_hash = hs.finish();

    // Written beside the target, flushed to the device, then renamed over it:
    // a reader sees either the previous file or the whole new one.
    const std::string tmp = std::string(path) + ".tmp";
    FILE *f = std::fopen(tmp.c_str(), "wb");
    if (f == nullptr) return ZERO_EIO;
    bool ok = write_all(f, &h, sizeof h) && write_all(f, w16, lay.count * 2) &&
              write_all(f, master, lay.count * 4) && write_all(f, m, lay.count * 4) &&
              write_all(f, v, lay.count * 4);
    ok = ok && std::fflush(f) == 0 && fsync(fileno(f)) == 0;
    ok = (std::fclose(f) == 0) && ok;
    if (ok && std::rename(tmp.c_str(), path) != 0) ok = false;
    if (!ok) {
        std::remove(tmp.c_str());
        return ZERO_EIO;
    }
    sync_parent_dir(path);
    return ZERO_OK;
}

extern "C" int zero_ckpt_read_info(const char *path, zero_ckpt_info *info) {
    if (path == nullptr || info == nullptr) return ZERO_EINVAL;
    FILE *f = std::fopen(path, "rb");
    if (f == nullptr) return ZERO_EIO;
    zero_ckpt_header h{};
    const int rc = read_header(f, &h);
    std::fclose(f);
    if (rc != ZERO_OK) return rc;
    to_info(h, info);
    return ZERO_OK;
}

extern "C" int zero_ckpt_verify(const char *path) {
    if (path == nullptr) return ZERO_EINVAL;
    FILE *f = std::fopen(path, "rb");
    if (f == nullptr) return ZERO_EIO;
    zero_ckpt_header h{};
    int rc = read_header(f, &h);
    if (rc == ZERO_OK && fseeko(f, sizeof h, SEEK_SET) != 0) rc = ZERO_EIO;
    Hasher hs;
    std::vector<char> buf(1 << 20);
    uint64_t left = rc == ZERO_OK ? h.payload_bytes : 0;
    while (rc == ZERO_OK && left > 0) {
        const size_t chunk = left > buf.size() ? buf.size() : static_cast<size_t>(left);
        if (std::fread(buf.data(), 1, chunk, f) != chunk) {
            rc = ZERO_EIO;
            break;
        }
        hs.add(buf.data(), chunk);
        left -= chunk;
    }
    std::fclose(f);
    if (rc != ZERO_OK) return rc;
    return hs.finish() == h.payload_hash ? ZERO_OK : ZERO_ECORRUPT;
}

extern "C" int zero_ckpt_read(const char *path, uint64_t first, uint64_t count, void *w16,
                              float *master, float *m, float *v) {
    if (path == nullptr) return ZERO_EINVAL;
    if (count > 0 && (w16 == nullptr || master == nullptr || m == nullptr || v == nullptr))
        return ZERO_EINVAL;
    FILE *f = std::fopen(path, "rb");
    if (f == nullptr) return ZERO_EIO;
    zero_ckpt_header h{};
    int rc = read_header(f, &h);
    if (rc == ZERO_OK && (first > h.count || count > h.count - first)) rc = ZERO_EINVAL;
    const uint64_t base = sizeof h;
    struct Part {
        void *dst;
        uint64_t offset;
        uint64_t elem;
    } parts[4] = {{w16, base, 2},
                  {master, base + 2 * h.count, 4},
                  {m, base + 6 * h.count, 4},
                  {v, base + 10 * h.count, 4}};
    for (int i = 0; rc == ZERO_OK && count > 0 && i < 4; ++i) {
        if (fseeko(f, static_cast<off_t>(parts[i].offset + first * parts[i].elem), SEEK_SET) != 0 ||
            !read_all(f, parts[i].dst, count * parts[i].elem))
            rc = ZERO_EIO;
    }
    std::fclose(f);
    return rc;
}

extern "C" int zero_reshard_plan(uint64_t psi, uint32_t n_old, uint32_t n_new, uint32_t rank_new,
                                 zero_ckpt_piece *pieces, uint32_t max_pieces,
                                 uint32_t *n_pieces) {
    if (n_pieces == nullptr) return ZERO_EINVAL;
    zero_layout old0, dst;
    if (zero_shard_layout(psi, n_old, 0, &old0) != ZERO_OK ||
        zero_shard_layout(psi, n_new, rank_new, &dst) != ZERO_OK)
        return ZERO_EINVAL;
    uint32_t np = 0;
    const uint64_t a = dst.offset, b = dst.offset + dst.count;  // new rank's flat range
    for (uint64_t j = a; j < b;) {
        const uint64_t k = j / old0.shard;               // old rank owning flat index j
        const uint64_t k_end = (k + 1) * old0.shard;     // end of its chunk
        const uint64_t end = k_end < b ? k_end : b;
        if (pieces != nullptr) {
            if (np >= max_pieces) return ZERO_ERANGE;
            pieces[np].src_rank = static_cast<uint32_t>(k);
            pieces[np].src_first = j - k * old0.shard;
            pieces[np].dst_first = j - a;
            pieces[np].count = end - j;
        }
        ++np;
        j = end;
    }
    *n_pieces = np;
    return ZERO_OK;
}

extern "C" int zero_ckpt_read_resharded(const char *const *paths_old, uint32_t n_old,
                                        uint64_t psi, uint32_t n_new, uint32_t rank_new,
                                        void *w16, float *master, float *m, float *v) {
    if (paths_old == nullptr) return ZERO_EINVAL;
    uint32_t np = 0;
    int rc = zero_reshard_plan(psi, n_old, n_new, rank_new, nullptr, 0, &np);
    if (rc != ZERO_OK) return rc;
    zero_layout dst;
    zero_shard_layout(psi, n_new, rank_new, &dst);
    if (dst.count > 0 && (w16 == nullptr || master == nullptr || m == nullptr || v == nullptr))
        return ZERO_EINVAL;
    std::vector<zero_ckpt_piece> plan(np);
    rc = zero_reshard_plan(psi, n_old, n_new, rank_new, plan.data(), np, &np);
    if (rc != ZERO_OK) return rc;
    // Every old file's header must name this layout and share one format and one
    // scaler state: each rank renames its own file into place, so a save that
    // failed part-way leaves files of two steps side by side, and new ranks that
    // read disjoint subsets of them would otherwise resume from different steps.
    zero_ckpt_info first{};
    for (uint32_t k = 0; k < n_old; ++k) {
        if (paths_old[k] == nullptr) return ZERO_EINVAL;
        zero_ckpt_info info;
        rc = zero_ckpt_read_info(paths_old[k], &info);
        if (rc != ZERO_OK) return rc;
        if (info.psi != psi || info.n != n_old || info.rank != k) return ZERO_ECORRUPT;
        if (k == 0) {
            first = info;
            continue;
        }
        const zero_scaler &a = first.scaler, &b = info.scaler;
        if (info.dtype != first.dtype || a.step != b.step || a.clean_steps != b.clean_steps ||
            a.growth_interval != b.growth_interval ||
            std::memcmp(&a.loss_scale, &b.loss_scale, sizeof(float)) != 0)
            return ZERO_ECORRUPT;
    }
    // the payload of every file this rank reads must match its hash
    std::vector<char> verified(n_old, 0);
    for (const zero_ckpt_piece &pc : plan) {
        if (verified[pc.src_rank]) continue;
        rc = zero_ckpt_verify(paths_old[pc.src_rank]);
        if (rc != ZERO_OK) return rc;
        verified[pc.src_rank] = 1;
    }
    for (const zero_ckpt_piece &pc : plan) {
        rc = zero_ckpt_read(paths_old[pc.src_rank], pc.src_first, pc.count,
                            static_cast<uint16_t *>(w16) + pc.dst_first, master + pc.dst_first,
                            m + pc.dst_first, v + pc.dst_first);
        if (rc != ZERO_OK) return rc;
    }
    return ZERO_OK;
}
