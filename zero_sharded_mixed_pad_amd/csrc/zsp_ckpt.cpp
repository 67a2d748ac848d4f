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
//   uint64   XXH64 (seed 0) of every byte above
// Files are written to a temporary name and renamed, so a process that dies
// mid-write never leaves a short file under the final name. The data is not
// forced to disk before the rename; a file cut short by a system crash fails
// the length and checksum checks of every read.
#include <dirent.h>
#include <fcntl.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
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

// XXH64 (Yann Collet's xxHash, 64-bit variant, as its specification
// defines it), fed incrementally: four accumulators over 32-byte stripes,
// then the stripes' merge, the length, the tail and the final avalanche.
// Four independent multiply chains hash at several GB/s, so the checksum
// does not limit a fast file system. Assumes a little-endian host.
class Xxh64 {
  public:
    void add(const void* data, size_t n) {
        const unsigned char* p = static_cast<const unsigned char*>(data);
        total_ += n;
        if (nbuf_ > 0) {
            const size_t k = std::min(n, sizeof(buf_) - nbuf_);
            std::memcpy(buf_ + nbuf_, p, k);
            nbuf_ += k;
            p += k;
            n -= k;
            if (nbuf_ < sizeof(buf_)) return;
            stripes(buf_, 1);
            nbuf_ = 0;
        }
        const size_t whole = n / 32;
        stripes(p, whole);
        p += whole * 32;
        n -= whole * 32;
        std::memcpy(buf_, p, n);
        nbuf_ = n;
    }
    uint64_t digest() const {
        uint64_t h;
        if (total_ >= 32) {
            h = rotl(a_[0], 1) + rotl(a_[1], 7) + rotl(a_[2], 12) + rotl(a_[3], 18);
            for (uint64_t a : a_) h = (h ^ mix(0, a)) * kP1 + kP4;
        } else {
            h = kP5;  // seed 0
        }
        h += total_;
        const unsigned char* p = buf_;
        size_t n = nbuf_;
        for (; n >= 8; n -= 8, p += 8) h = rotl(h ^ mix(0, load64(p)), 27) * kP1 + kP4;
        if (n >= 4) {
            uint32_t w;
            std::memcpy(&w, p, 4);
            h = rotl(h ^ (uint64_t(w) * kP1), 23) * kP2 + kP3;
            p += 4;
            n -= 4;
        }
        for (; n > 0; --n, ++p) h = rotl(h ^ (uint64_t(*p) * kP5), 11) * kP1;
        h ^= h >> 33;
        h *= kP2;
        h ^= h >> 29;
        h *= kP3;
        h ^= h >> 32;
        return h;
    }

  private:
    static constexpr uint64_t kP1 = 0x9E3779B185EBCA87ull, kP2 = 0xC2B2AE3D27D4EB4Full,
                              kP3 = 0x165667B19E3779F9ull, kP4 = 0x85EBCA77C2B2AE63ull,
                              kP5 = 0x27D4EB2F165667C5ull;
    static uint64_t rotl(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }
    static uint64_t mix(uint64_t acc, uint64_t in) { return rotl(acc + in * kP2, 31) * kP1; }
    static uint64_t load64(const unsigned char* p) {
        uint64_t x;
        std::memcpy(&x, p, 8);
        return x;
    }
    void stripes(const unsigned char* p, size_t count) {
        uint64_t a0 = a_[0], a1 = a_[1], a2 = a_[2], a3 = a_[3];
        for (size_t i = 0; i < count; ++i, p += 32) {
            a0 = mix(a0, load64(p));
            a1 = mix(a1, load64(p + 8));
            a2 = mix(a2, load64(p + 16));
            a3 = mix(a3, load64(p + 24));
        }
        a_[0] = a0, a_[1] = a1, a_[2] = a2, a_[3] = a3;
    }

    uint64_t a_[4] = {kP1 + kP2, kP2, 0, 0 - kP1};  // seed 0
    uint64_t total_ = 0;
    unsigned char buf_[32];
    size_t nbuf_ = 0;
};

std::string rank_path(const char* dir, int64_t r, int64_t nd) {
    char name[96];
    std::snprintf(name, sizeof(name), "/rank-%lld-of-%lld.zsp", (long long)r, (long long)nd);
    return std::string(dir) + name;
}

struct Writer {
    FILE* f = nullptr;
    Xxh64 hash;
    bool ok = true;
    void put(const void* p, size_t n) {
        if (!ok || n == 0) return;
        hash.add(p, n);
        ok = std::fwrite(p, 1, n, f) == n;
    }
};

}  // namespace

HostPayload::HostPayload(const float* master, const float* m, const float* v,
                         const uint16_t* work, int64_t S) {
    seg_[0] = reinterpret_cast<const char*>(master);
    seg_[1] = reinterpret_cast<const char*>(m);
    seg_[2] = reinterpret_cast<const char*>(v);
    seg_[3] = reinterpret_cast<const char*>(work);
    for (int i = 0; i < 4; ++i) len_[i] = size_t(S) * (i < 3 ? 4 : 2);
}

bool HostPayload::next(const void** data, size_t* n, std::string*) {
    while (cur_ < 4 && len_[cur_] == 0) ++cur_;
    if (cur_ == 4) {
        *n = 0;
        return true;
    }
    *data = seg_[cur_];
    *n = len_[cur_];
    ++cur_;
    return true;
}

CkptStatus ckpt_write_rank(const char* dir, int32_t nd, int32_t rank,
                           const std::vector<int64_t>& numel, int64_t S, int64_t step,
                           PayloadSource& src, std::string* err) {
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
    int64_t total = 0;
    std::string why;
    bool src_ok = true;
    while (w.ok) {
        const void* data = nullptr;
        size_t n = 0;
        if (!src.next(&data, &n, &why)) {
            src_ok = false;
            break;
        }
        if (n == 0) break;
        w.put(data, n);
        total += int64_t(n);
    }
    if (src_ok && total != ckpt_payload_bytes(S)) {
        src_ok = false;
        why = "payload of " + std::to_string(total) + " bytes, expected " +
              std::to_string(ckpt_payload_bytes(S));
    }
    const uint64_t h = w.hash.digest();
    if (w.ok && src_ok) w.ok = std::fwrite(&h, 1, sizeof(h), w.f) == sizeof(h);
    if (std::fclose(w.f) != 0) w.ok = false;
    if (!src_ok || !w.ok || std::rename(tmp.c_str(), path.c_str()) != 0) {
        std::remove(tmp.c_str());
        *err = !src_ok ? "writing " + path + ": " + why : "cannot write " + path;
        return CkptStatus::Io;
    }
    return CkptStatus::Ok;
}

MappedRank::~MappedRank() {
    if (base_) munmap(base_, len_);
}

CkptStatus MappedRank::open(const char* dir, int32_t nd, int32_t rank,
                            std::vector<int64_t>* numel, int64_t* S, int64_t* step,
                            std::string* err) {
    const std::string path = rank_path(dir, rank, nd);
    const int fd = ::open(path.c_str(), O_RDONLY);
    if (fd < 0) {
        *err = "cannot open " + path + ": " + std::strerror(errno);
        return CkptStatus::Missing;
    }
    struct stat sb;
    if (fstat(fd, &sb) != 0) {
        *err = "cannot stat " + path + ": " + std::strerror(errno);
        close(fd);
        return CkptStatus::Io;
    }
    int64_t hdr[5];
    const size_t head0 = sizeof(kMagic) + sizeof(hdr);
    if (sb.st_size < int64_t(head0 + sizeof(uint64_t))) {
        close(fd);
        *err = path + ": truncated (" + std::to_string(sb.st_size) + " bytes)";
        return CkptStatus::Corrupt;
    }
    const size_t size = size_t(sb.st_size);
    void* p = mmap(nullptr, size, PROT_READ, MAP_PRIVATE, fd, 0);
    close(fd);
    if (p == MAP_FAILED) {
        *err = "cannot map " + path + ": " + std::strerror(errno);
        return CkptStatus::Io;
    }
    base_ = p;  // unmapped by the destructor, also after a failed check below
    len_ = size;
    const char* b = static_cast<const char*>(p);
    std::memcpy(hdr, b + sizeof(kMagic), sizeof(hdr));
    if (std::memcmp(b, kMagic, sizeof(kMagic)) != 0 || hdr[0] != nd || hdr[1] != rank ||
        hdr[2] < 1 || hdr[2] > (int64_t(1) << 31) || hdr[3] < 0 || hdr[3] > (int64_t(1) << 40)) {
        *err = path + ": not a shard file of rank " + std::to_string(rank) + " of " +
               std::to_string(nd);
        return CkptStatus::Corrupt;
    }
    // The header fixes the file's length (the bounds above keep this sum far
    // from overflow); only then is anything sized from it.
    const int64_t want = int64_t(head0) + 8 * hdr[2] + ckpt_payload_bytes(hdr[3]) +
                         int64_t(sizeof(uint64_t));
    if (int64_t(size) != want) {
        *err = path + ": truncated or corrupt (" + std::to_string(size) +
               " bytes, its header needs " + std::to_string(want) + ")";
        return CkptStatus::Corrupt;
    }
    Xxh64 hash;
    hash.add(b, size - sizeof(uint64_t));
    uint64_t stored = 0;
    std::memcpy(&stored, b + size - sizeof(uint64_t), sizeof(stored));
    if (hash.digest() != stored) {
        *err = path + ": corrupt (hash mismatch)";
        return CkptStatus::Corrupt;
    }
    numel->resize(size_t(hdr[2]));
    std::memcpy(numel->data(), b + head0, numel->size() * sizeof(int64_t));
    *S = hdr[3];
    *step = hdr[4];
    payload_ = b + head0 + numel->size() * sizeof(int64_t);
    S_ = hdr[3];
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
