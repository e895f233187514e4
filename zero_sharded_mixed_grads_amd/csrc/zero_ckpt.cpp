// Sharded checkpoints of one rank's optimizer state ("ZeRO" AI-library
// tutorial page, section "Checkpoint 与恢复": each rank writes only the state
// it owns; resuming may need a different number of GPUs).
//
// File layout (little-endian): a 64-byte zero_ckpt_header, then the rank's
// fp32 master, momentum and variance, n = end - begin elements each, then,
// when the header's flags bit 0 is set, the 32-byte loss-scale state.  Save
// writes to "<path>.tmp", flushes it to storage and renames it over <path>,
// so a crash never leaves a half-written file under the final name.  Load
// takes the shard files of a saved run with any number of ranks, checks that
// they describe one run (same psi and step, ranges tiling [0, psi)), and
// copies the intersection of each file with the loading rank's range.  A save
// that fails removes its temporary file; a completed one also flushes the
// directory entry, so the rename itself survives a crash.
#include <hip/hip_runtime_api.h>

#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cerrno>
#include <cstring>
#include <string>
#include <vector>

#include "zero_internal.h"

using zero::fail;

namespace {

constexpr char kMagic[8] = {'Z', 'E', 'R', 'O', 'C', 'K', 'P', 'T'};
constexpr uint32_t kVersion = 1;
constexpr uint64_t kChunk = 64ull << 20;  // bytes staged through host memory at a time
constexpr uint64_t kFlagLossScale = 1;    // a zero_loss_scale_t follows the arrays

static_assert(sizeof(zero_loss_scale_t) == 32, "loss-scale record is 32 bytes");

uint64_t file_bytes(const zero_ckpt_header &h)
{
    return sizeof h + 12 * (h.end - h.begin) +
           ((h.flags & kFlagLossScale) ? sizeof(zero_loss_scale_t) : 0);
}

static_assert(sizeof(zero_ckpt_header) == 64, "checkpoint header is 64 bytes");

struct Fd {
    int fd = -1;
    ~Fd() { if (fd >= 0) close(fd); }
};

// Removes the temporary file of a save unless the save completed.
struct TmpFile {
    std::string path;
    bool keep = false;
    ~TmpFile() { if (!keep) unlink(path.c_str()); }
};

// Flushes the directory entry of `path` (its parent directory) to storage, so
// that a completed rename survives a crash.
bool sync_parent_dir(const char *path)
{
    std::string dir(path);
    const size_t slash = dir.find_last_of('/');
    dir = slash == std::string::npos ? "." : (slash == 0 ? "/" : dir.substr(0, slash));
    Fd d;
    d.fd = open(dir.c_str(), O_RDONLY | O_DIRECTORY);
    return d.fd >= 0 && fsync(d.fd) == 0;
}

bool write_all(int fd, const void *buf, size_t len)
{
    const char *p = (const char *)buf;
    while (len) {
        const ssize_t k = write(fd, p, len);
        if (k < 0 && errno == EINTR)
            continue;
        if (k <= 0)
            return false;
        p += k;
        len -= (size_t)k;
    }
    return true;
}

bool read_at(int fd, void *buf, size_t len, uint64_t off)
{
    char *p = (char *)buf;
    while (len) {
        const ssize_t k = pread(fd, p, len, (off_t)off);
        if (k < 0 && errno == EINTR)
            continue;
        if (k <= 0)
            return false;
        p += k;
        off += (uint64_t)k;
        len -= (size_t)k;
    }
    return true;
}

zero_status hip_check(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(ZERO_EDEVICE, "%s: %s", what, hipGetErrorString(e));
    return ZERO_OK;
}

// Two pinned host slots of `slot` bytes with one event each, so that the copy
// of one chunk between device and host overlaps the file I/O of the other.
// The destructor drains the stream before freeing the slots: no copy queued
// into or out of them outlives the call, also on an error path.
struct Staging {
    hipStream_t stream;
    size_t slot = 0;
    char *buf = nullptr;
    hipEvent_t ev[2] = {nullptr, nullptr};
    explicit Staging(hipStream_t s) : stream(s) {}
    ~Staging()
    {
        (void)hipStreamSynchronize(stream);
        for (hipEvent_t e : ev)
            if (e)
                (void)hipEventDestroy(e);
        if (buf)
            (void)hipHostFree(buf);
    }
    zero_status init(size_t bytes, const char *what)
    {
        slot = bytes;
        zero_status st = hip_check(hipHostMalloc((void **)&buf, 2 * bytes, hipHostMallocDefault),
                                   what);
        for (int i = 0; i < 2 && st == ZERO_OK; ++i)
            st = hip_check(hipEventCreateWithFlags(&ev[i], hipEventDisableTiming), what);
        return st;
    }
    char *at(uint64_t k) const { return buf + (k % 2) * slot; }
};

// One staged piece of an array: `len` bytes at byte offset `off`.
struct Piece {
    int array;
    uint64_t off;
    size_t len;
};

}  // namespace

extern "C" zero_status zero_ckpt_save(const char *path, uint64_t psi, uint32_t nd, uint32_t rank,
                                      const float *master, const float *exp_avg,
                                      const float *exp_avg_sq, const zero_adam_state_t *d_state,
                                      const zero_loss_scale_t *d_scale, void *stream)
{
    if (!path || !d_state)
        return fail(ZERO_EINVAL, "zero_ckpt_save: NULL path or d_state");
    uint64_t begin, end;
    zero_status st = zero_partition(psi, nd, rank, &begin, &end);
    if (st != ZERO_OK)
        return st;
    const uint64_t n = end - begin;
    if (n > 0 && (!master || !exp_avg || !exp_avg_sq))
        return fail(ZERO_EINVAL, "zero_ckpt_save: NULL state array with n > 0");
    hipStream_t s = (hipStream_t)stream;
    zero_adam_state_t state;
    zero_loss_scale_t scale{};
    if ((st = hip_check(hipMemcpyAsync(&state, d_state, sizeof state, hipMemcpyDeviceToHost, s),
                        "zero_ckpt_save: reading the step state")) != ZERO_OK ||
        (d_scale &&
         (st = hip_check(hipMemcpyAsync(&scale, d_scale, sizeof scale, hipMemcpyDeviceToHost, s),
                         "zero_ckpt_save: reading the loss-scale state")) != ZERO_OK) ||
        (st = hip_check(hipStreamSynchronize(s), "zero_ckpt_save: stream")) != ZERO_OK)
        return st;

    zero_ckpt_header h{};
    std::memcpy(h.magic, kMagic, sizeof kMagic);
    h.version = kVersion;
    h.nd = nd;
    h.rank = rank;
    h.psi = psi;
    h.begin = begin;
    h.end = end;
    h.step = state.step;
    h.flags = d_scale ? kFlagLossScale : 0;

    const std::string tmp = std::string(path) + ".tmp";
    Fd f;
    f.fd = open(tmp.c_str(), O_WRONLY | O_CREAT | O_TRUNC, 0644);
    if (f.fd < 0)
        return fail(ZERO_EIO, "zero_ckpt_save: cannot create %s: %s", tmp.c_str(), strerror(errno));
    TmpFile guard{tmp};
    if (!write_all(f.fd, &h, sizeof h))
        return fail(ZERO_EIO, "zero_ckpt_save: writing %s: %s", tmp.c_str(), strerror(errno));
    // the arrays in chunks through two pinned slots: the copy of chunk k + 1 to
    // the host runs while chunk k is written to the file
    const float *arrays[3] = {master, exp_avg, exp_avg_sq};
    std::vector<Piece> pieces;
    for (int a = 0; a < 3; ++a)
        for (uint64_t off = 0; off < 4 * n; off += kChunk)
            pieces.push_back({a, off, (size_t)std::min<uint64_t>(kChunk, 4 * n - off)});
    Staging stg(s);
    if (!pieces.empty() &&
        (st = stg.init((size_t)std::min<uint64_t>(kChunk, 4 * n), "zero_ckpt_save: staging")) !=
            ZERO_OK)
        return st;
    auto fetch = [&](uint64_t k) -> zero_status {
        const Piece &q = pieces[k];
        zero_status r = hip_check(hipMemcpyAsync(stg.at(k), (const char *)arrays[q.array] + q.off,
                                                 q.len, hipMemcpyDeviceToHost, s),
                                  "zero_ckpt_save: copy to host");
        return r != ZERO_OK ? r : hip_check(hipEventRecord(stg.ev[k % 2], s), "zero_ckpt_save");
    };
    if (!pieces.empty() && (st = fetch(0)) != ZERO_OK)
        return st;
    for (uint64_t k = 0; k < pieces.size(); ++k) {
        if (k + 1 < pieces.size() && (st = fetch(k + 1)) != ZERO_OK)
            return st;
        if ((st = hip_check(hipEventSynchronize(stg.ev[k % 2]), "zero_ckpt_save: copy to host")) !=
            ZERO_OK)
            return st;
        if (!write_all(f.fd, stg.at(k), pieces[k].len))
            return fail(ZERO_EIO, "zero_ckpt_save: writing %s: %s", tmp.c_str(), strerror(errno));
    }
    if (d_scale && !write_all(f.fd, &scale, sizeof scale))
        return fail(ZERO_EIO, "zero_ckpt_save: writing %s: %s", tmp.c_str(), strerror(errno));
    if (fsync(f.fd) != 0)
        return fail(ZERO_EIO, "zero_ckpt_save: fsync %s: %s", tmp.c_str(), strerror(errno));
    const int fd = f.fd;
    f.fd = -1;
    if (close(fd) != 0)
        return fail(ZERO_EIO, "zero_ckpt_save: closing %s: %s", tmp.c_str(), strerror(errno));
    if (rename(tmp.c_str(), path) != 0)
        return fail(ZERO_EIO, "zero_ckpt_save: rename to %s: %s", path, strerror(errno));
    guard.keep = true;
    if (!sync_parent_dir(path))
        return fail(ZERO_EIO, "zero_ckpt_save: syncing the directory of %s: %s", path,
                    strerror(errno));
    return ZERO_OK;
}

extern "C" zero_status zero_ckpt_read_header(const char *path, zero_ckpt_header *out)
{
    if (!path || !out)
        return fail(ZERO_EINVAL, "zero_ckpt_read_header: NULL argument");
    Fd f;
    f.fd = open(path, O_RDONLY);
    if (f.fd < 0)
        return fail(ZERO_EIO, "zero_ckpt_read_header: cannot open %s: %s", path, strerror(errno));
    zero_ckpt_header h;
    if (!read_at(f.fd, &h, sizeof h, 0))
        return fail(ZERO_EIO, "zero_ckpt_read_header: %s is shorter than a header", path);
    if (std::memcmp(h.magic, kMagic, sizeof kMagic) != 0 || h.version != kVersion)
        return fail(ZERO_EINVAL, "zero_ckpt_read_header: %s is not a version-%u shard", path,
                    kVersion);
    if (h.flags & ~kFlagLossScale)
        return fail(ZERO_EINVAL, "zero_ckpt_read_header: %s has unknown flags %llx", path,
                    (unsigned long long)h.flags);
    uint64_t b, e;
    if (zero_partition(h.psi, h.nd, h.rank, &b, &e) != ZERO_OK || b != h.begin || e != h.end)
        return fail(ZERO_EINVAL, "zero_ckpt_read_header: %s: range [%llu, %llu) is not rank %u of %u",
                    path, (unsigned long long)h.begin, (unsigned long long)h.end, h.rank, h.nd);
    struct stat sb;
    if (fstat(f.fd, &sb) != 0 || (uint64_t)sb.st_size != file_bytes(h))
        return fail(ZERO_EIO, "zero_ckpt_read_header: %s has the wrong size", path);
    *out = h;
    return ZERO_OK;
}

extern "C" zero_status zero_ckpt_load(const char *const *paths, uint32_t n_paths, uint64_t psi,
                                      uint32_t nd, uint32_t rank, float *master, float *exp_avg,
                                      float *exp_avg_sq, zero_adam_state_t *d_state,
                                      zero_loss_scale_t *d_scale, void *stream)
{
    if (!paths || n_paths == 0 || !d_state)
        return fail(ZERO_EINVAL, "zero_ckpt_load: no shard files or NULL d_state");
    uint64_t begin, end;
    zero_status st = zero_partition(psi, nd, rank, &begin, &end);
    if (st != ZERO_OK)
        return st;
    const uint64_t n = end - begin;
    if (n > 0 && (!master || !exp_avg || !exp_avg_sq))
        return fail(ZERO_EINVAL, "zero_ckpt_load: NULL state array with n > 0");

    // the files must be the complete set of shards of one saved run
    std::vector<zero_ckpt_header> hs(n_paths);
    for (uint32_t i = 0; i < n_paths; ++i) {
        if (!paths[i])
            return fail(ZERO_EINVAL, "zero_ckpt_load: NULL path %u", i);
        if ((st = zero_ckpt_read_header(paths[i], &hs[i])) != ZERO_OK)
            return st;
        if (hs[i].psi != psi)
            return fail(ZERO_EINVAL, "zero_ckpt_load: %s holds psi %llu, not %llu", paths[i],
                        (unsigned long long)hs[i].psi, (unsigned long long)psi);
        if (hs[i].step != hs[0].step || hs[i].nd != hs[0].nd)
            return fail(ZERO_EINVAL, "zero_ckpt_load: %s is from another save (step or rank count)",
                        paths[i]);
    }
    std::vector<uint32_t> order(n_paths);
    for (uint32_t i = 0; i < n_paths; ++i)
        order[i] = i;
    std::sort(order.begin(), order.end(),
              [&](uint32_t a, uint32_t b) { return hs[a].begin < hs[b].begin; });
    uint64_t covered = 0;
    for (uint32_t i : order) {
        if (hs[i].begin != covered)
            return fail(ZERO_EINVAL, "zero_ckpt_load: the shard files do not tile [0, %llu): "
                        "gap or overlap at %llu", (unsigned long long)psi,
                        (unsigned long long)covered);
        covered = hs[i].end;
    }
    if (covered != psi || n_paths != hs[0].nd)
        return fail(ZERO_EINVAL, "zero_ckpt_load: %u shard files do not cover all %u ranks",
                    n_paths, hs[0].nd);

    // the loss-scale record, when asked for: present and identical in every file
    zero_loss_scale_t scale{};
    if (d_scale) {
        for (uint32_t i = 0; i < n_paths; ++i) {
            if (!(hs[i].flags & kFlagLossScale))
                return fail(ZERO_EINVAL, "zero_ckpt_load: %s holds no loss-scale state",
                            paths[i]);
            Fd f;
            f.fd = open(paths[i], O_RDONLY);
            zero_loss_scale_t r;
            if (f.fd < 0 ||
                !read_at(f.fd, &r, sizeof r, file_bytes(hs[i]) - sizeof r))
                return fail(ZERO_EIO, "zero_ckpt_load: reading the loss-scale state of %s",
                            paths[i]);
            if (i == 0)
                scale = r;
            else if (std::memcmp(&r, &scale, sizeof r) != 0)
                return fail(ZERO_EINVAL, "zero_ckpt_load: %s has a different loss-scale state",
                            paths[i]);
        }
    }

    hipStream_t s = (hipStream_t)stream;
    if ((st = hip_check(hipStreamSynchronize(s), "zero_ckpt_load: stream")) != ZERO_OK)
        return st;
    // chunks through two pinned slots: chunk k is read from its file while the
    // copy of chunk k - 1 to the device runs; a slot is refilled only after its
    // previous copy has finished
    Staging stg(s);
    if (n > 0 && (st = stg.init((size_t)std::min<uint64_t>(kChunk, 4 * n),
                                "zero_ckpt_load: staging")) != ZERO_OK)
        return st;
    float *dsts[3] = {master, exp_avg, exp_avg_sq};
    uint64_t k = 0;  // chunks staged so far
    for (uint32_t i : order) {
        const uint64_t lo = std::max(begin, hs[i].begin), hi = std::min(end, hs[i].end);
        if (lo >= hi)
            continue;
        Fd f;
        f.fd = open(paths[i], O_RDONLY);
        if (f.fd < 0)
            return fail(ZERO_EIO, "zero_ckpt_load: cannot open %s: %s", paths[i], strerror(errno));
        const uint64_t file_n = hs[i].end - hs[i].begin;
        for (int a = 0; a < 3; ++a) {
            const uint64_t src0 = sizeof(zero_ckpt_header) + 4 * (a * file_n + (lo - hs[i].begin));
            char *dst0 = (char *)dsts[a] + 4 * (lo - begin);
            for (uint64_t off = 0; off < 4 * (hi - lo); off += stg.slot, ++k) {
                const size_t len = (size_t)std::min<uint64_t>(stg.slot, 4 * (hi - lo) - off);
                if (k >= 2 && (st = hip_check(hipEventSynchronize(stg.ev[k % 2]),
                                              "zero_ckpt_load: copy to device")) != ZERO_OK)
                    return st;
                if (!read_at(f.fd, stg.at(k), len, src0 + off))
                    return fail(ZERO_EIO, "zero_ckpt_load: reading %s", paths[i]);
                if ((st = hip_check(hipMemcpyAsync(dst0 + off, stg.at(k), len,
                                                   hipMemcpyHostToDevice, s),
                                    "zero_ckpt_load: copy to device")) != ZERO_OK ||
                    (st = hip_check(hipEventRecord(stg.ev[k % 2], s), "zero_ckpt_load")) != ZERO_OK)
                    return st;
            }
        }
    }
    // step counter restored; the per-step scalars are recomputed by the next step
    zero_adam_state_t state{};
    state.step = hs[0].step;
    if ((st = hip_check(hipMemcpyAsync(d_state, &state, sizeof state, hipMemcpyHostToDevice, s),
                        "zero_ckpt_load: writing the step state")) != ZERO_OK)
        return st;
    if (d_scale &&
        (st = hip_check(hipMemcpyAsync(d_scale, &scale, sizeof scale, hipMemcpyHostToDevice, s),
                        "zero_ckpt_load: writing the loss-scale state")) != ZERO_OK)
        return st;
    return hip_check(hipStreamSynchronize(s), "zero_ckpt_load: stream");
}
