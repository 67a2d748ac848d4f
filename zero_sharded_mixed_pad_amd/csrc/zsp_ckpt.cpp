// zsp_ckpt.cpp -- sharded checkpoint, resume and reshard ("ZeRO Stages:
// Sharding Optimizer State, Gradients, and Parameters", "Where the shards live
// and what happens on failure": each rank writes its own shard set with
// enough metadata to rebuild the partitioning; loading at a different rank
// count reshuffles the shards; the safe point is between steps).
//
// File format, one file per rank, "rank-<r>-of-<nd>.zsp" in the checkpoint
// directory, all fields little-endian:
//   char[8]  magic "ZSPCKPT1"
//   int64    n_d, rank, T, S, step
//   int64    numel[T]
//   float    master[S], m[S], v[S]
//   uint16   work[S]
//   uint64   FNV-1a hash of every byte above
// Files are written to a temporary name and renamed, so a crash mid-write
// never leaves a truncated file under the final name.
#include <dirent.h>

#include <cerrno>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "zsp_ckpt.hpp"
#include "zsp.h"

namespace zsp {
namespace {

const char kMagic[8] = {'Z', 'S', 'P', 'C', 'K', 'P', 'T', '1'};

struct Fnv {
    uint64_t h = 1469598103934665603ull;
    void add(const void* p, size_t n) {
        const unsigned char* b = static_cast<const unsigned char*>(p);
        for (size_t i = 0; i < n; ++i) {
            h ^= b[i];
            h *= 1099511628211ull;
        }
    }
};

std::string rank_path(const char* dir, int64_t r, int64_t nd) {
    char name[96];
    std::snprintf(name, sizeof(name), "/rank-%lld-of-%lld.zsp", (long long)r, (long long)nd);
    return std::string(dir) + name;
}

struct Writer {
    FILE* f = nullptr;
    Fnv fnv;
    bool ok = true;
    void put(const void* p, size_t n) {
        if (!ok || n == 0) return;
        fnv.add(p, n);
        ok = std::fwrite(p, 1, n, f) == n;
    }
};

struct Reader {
    FILE* f = nullptr;
    Fnv fnv;
    bool ok = true;
    void get(void* p, size_t n) {
        if (!ok || n == 0) return;
        ok = std::fread(p, 1, n, f) == n;
        if (ok) fnv.add(p, n);
    }
};

}  // namespace

// Write rank r's shard set (host arrays of S elements) to its file.
CkptStatus ckpt_write_rank(const char* dir, int32_t nd, int32_t rank,
                           const std::vector<int64_t>& numel, int64_t S, int64_t step,
                           const float* master, const float* m, const float* v,
                           const uint16_t* work, std::string* err) {
    const std::string path = rank_path(dir, rank, nd);
    const std::string tmp = path + ".tmp";
    Writer w;
    w.f = std::fopen(tmp.c_str(), "wb");
    if (!w.f) {
        *err = "cannot create " + tmp + ": " + std::strerror(errno);
        return CkptStatus::Io;
    }
    const int64_t hdr[5] = {nd, rank, static_cast<int64_t>(numel.size()), S, step};
    w.put(kMagic, sizeof(kMagic));
    w.put(hdr, sizeof(hdr));
    w.put(numel.data(), numel.size() * sizeof(int64_t));
    w.put(master, size_t(S) * sizeof(float));
    w.put(m, size_t(S) * sizeof(float));
    w.put(v, size_t(S) * sizeof(float));
    w.put(work, size_t(S) * sizeof(uint16_t));
    const uint64_t h = w.fnv.h;
    if (w.ok) w.ok = std::fwrite(&h, 1, sizeof(h), w.f) == sizeof(h);
    if (std::fclose(w.f) != 0) w.ok = false;
    if (!w.ok || std::rename(tmp.c_str(), path.c_str()) != 0) {
        std::remove(tmp.c_str());
        *err = "cannot write " + path;
        return CkptStatus::Io;
    }
    return CkptStatus::Ok;
}

// Read the file of rank r of an nd-rank checkpoint; checks magic, header and
// hash, and returns the header's numel list, S and step.
CkptStatus ckpt_read_rank(const char* dir, int32_t nd, int32_t rank, std::vector<int64_t>* numel,
                          int64_t* S, int64_t* step, std::vector<float>* master,
                          std::vector<float>* m, std::vector<float>* v,
                          std::vector<uint16_t>* work, std::string* err) {
    const std::string path = rank_path(dir, rank, nd);
    Reader r;
    r.f = std::fopen(path.c_str(), "rb");
    if (!r.f) {
        *err = "cannot open " + path + ": " + std::strerror(errno);
        return CkptStatus::Missing;
    }
    char magic[8];
    int64_t hdr[5];
    r.get(magic, sizeof(magic));
    r.get(hdr, sizeof(hdr));
    if (!r.ok || std::memcmp(magic, kMagic, 8) != 0 || hdr[0] != nd || hdr[1] != rank ||
        hdr[2] < 1 || hdr[2] > (int64_t(1) << 31) || hdr[3] < 0 || hdr[3] > (int64_t(1) << 40)) {
        std::fclose(r.f);
        *err = path + ": not a shard file of rank " + std::to_string(rank) + " of " +
               std::to_string(nd);
        return CkptStatus::Corrupt;
    }
    numel->resize(size_t(hdr[2]));
    r.get(numel->data(), numel->size() * sizeof(int64_t));
    *S = hdr[3];
    *step = hdr[4];
    master->resize(size_t(*S));
    m->resize(size_t(*S));
    v->resize(size_t(*S));
    work->resize(size_t(*S));
    r.get(master->data(), size_t(*S) * sizeof(float));
    r.get(m->data(), size_t(*S) * sizeof(float));
    r.get(v->data(), size_t(*S) * sizeof(float));
    r.get(work->data(), size_t(*S) * sizeof(uint16_t));
    const uint64_t want = r.fnv.h;
    uint64_t got = 0;
    const bool tail_ok = r.ok && std::fread(&got, 1, sizeof(got), r.f) == sizeof(got);
    char extra;
    const bool at_end = std::fread(&extra, 1, 1, r.f) == 0;
    std::fclose(r.f);
    if (!tail_ok || got != want || !at_end) {
        *err = path + ": truncated or corrupt (hash mismatch)";
        return CkptStatus::Corrupt;
    }
    return CkptStatus::Ok;
}

// Number of ranks of the checkpoint in `dir`, from the names of the shard
// files present ("rank-<r>-of-<nd>.zsp"; a one-rank save leaves only its own
// file). 0: none found; -1: files of several rank counts.
int32_t ckpt_find_nd(const char* dir) {
    DIR* d = opendir(dir);
    if (!d) return 0;
    int32_t found = 0;
    while (const dirent* e = readdir(d)) {
        long long r = -1, nd = -1;
        char tail[8] = {0};
        if (std::sscanf(e->d_name, "rank-%lld-of-%lld.%7s", &r, &nd, tail) != 3) continue;
        if (std::strcmp(tail, "zsp") != 0 || nd < 1 || nd > ZSP_MAX_RANKS || r < 0 || r >= nd)
            continue;
        if (found == 0) found = int32_t(nd);
        else if (found != nd) found = -1;
    }
    closedir(d);
    return found;
}

}  // namespace zsp
