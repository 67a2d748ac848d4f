// zsp_ckpt.hpp -- per-rank shard files of a sharded checkpoint (format in
// zsp_ckpt.cpp): writing one rank's file from a payload passed chunk by
// chunk (so callers can stage it while the file side runs), and mapping a
// file, checking it whole on the mapping and reading its payload in place.
// Host only; no HIP here.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

namespace zsp {

enum class CkptStatus { Ok, Io, Missing, Corrupt };

// The payload of a rank file: master[S], m[S], v[S] (fp32), work[S] (bf16
// bits), back to back.
inline int64_t ckpt_payload_bytes(int64_t S) { return 14 * S; }

// Where ckpt_write_rank takes the payload from.
struct PayloadSource {
    virtual ~PayloadSource() = default;
    // The next chunk; *n == 0 after the last. false: failed (*err says why).
    virtual bool next(const void** data, size_t* n, std::string* err) = 0;
};

// Four host arrays of S elements as a payload source.
class HostPayload : public PayloadSource {
  public:
    HostPayload(const float* master, const float* m, const float* v, const uint16_t* work,
                int64_t S);
    bool next(const void** data, size_t* n, std::string* err) override;

  private:
    const char* seg_[4];
    size_t len_[4];
    int cur_ = 0;
};

// Write rank `rank`'s file of an nd-rank checkpoint: header, the payload
// from `src` (exactly ckpt_payload_bytes(S) bytes), checksum. Written under
// a temporary name, then renamed.
CkptStatus ckpt_write_rank(const char* dir, int32_t nd, int32_t rank,
                           const std::vector<int64_t>& numel, int64_t S, int64_t step,
                           PayloadSource& src, std::string* err);

// Rank `rank`'s file mapped read-only and checked whole on that one mapping:
// magic, header, length and the checksum over the mapped bytes. The payload
// read afterwards is the one the checksum covered (a file renamed into
// place meanwhile, e.g. by another save, does not replace the mapped one).
// open() returns the header's numel list, S and step.
class MappedRank {
  public:
    MappedRank() = default;
    MappedRank(const MappedRank&) = delete;
    MappedRank& operator=(const MappedRank&) = delete;
    ~MappedRank();
    CkptStatus open(const char* dir, int32_t nd, int32_t rank, std::vector<int64_t>* numel,
                    int64_t* S, int64_t* step, std::string* err);
    // master, m, v (fp32) and work (bf16 bits) of the payload
    const float* master() const { return reinterpret_cast<const float*>(payload_); }
    const float* m() const { return master() + S_; }
    const float* v() const { return master() + 2 * S_; }
    const uint16_t* work() const { return reinterpret_cast<const uint16_t*>(master() + 3 * S_); }

  private:
    void* base_ = nullptr;
    size_t len_ = 0;
    const char* payload_ = nullptr;
    int64_t S_ = 0;
};

// Number of ranks of the checkpoint in `dir` from the file names present.
// 0: none; -1: files of several rank counts.
int32_t ckpt_find_nd(const char* dir);

}  // namespace zsp
