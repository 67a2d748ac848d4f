// zsp_ckpt.hpp -- per-rank shard files of a sharded checkpoint (format in
// zsp_ckpt.cpp): writing, verifying and reading one rank's file, with the
// payload passed chunk by chunk so that callers can stage it (device copies,
// pinned buffers) while the file side runs. Host only; no HIP here.
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

// Where ckpt_stream_rank puts the payload.
struct PayloadSink {
    virtual ~PayloadSink() = default;
    // Called once the header is read and checked, before any payload.
    virtual bool begin(int64_t S, std::string* err) = 0;
    // A buffer for the next payload bytes, at most *cap of them (> 0).
    virtual bool buffer(void** data, size_t* cap, std::string* err) = 0;
    // The buffer last handed out now holds its next n payload bytes.
    virtual bool commit(size_t n, std::string* err) = 0;
};

// Four host arrays of S elements as a payload source, or as a sink that
// fills them (vectors are resized to S first). As a sink it accepts only a
// file whose S is the one given here.
class HostPayload : public PayloadSource, public PayloadSink {
  public:
    HostPayload(const float* master, const float* m, const float* v, const uint16_t* work,
                int64_t S);
    HostPayload(std::vector<float>* master, std::vector<float>* m, std::vector<float>* v,
                std::vector<uint16_t>* work, int64_t S);
    bool next(const void** data, size_t* n, std::string* err) override;
    bool begin(int64_t S, std::string* err) override;
    bool buffer(void** data, size_t* cap, std::string* err) override;
    bool commit(size_t n, std::string* err) override;

  private:
    void set_segments(int64_t S);
    std::vector<float>*vm_ = nullptr, *vmm_ = nullptr, *vv_ = nullptr;
    std::vector<uint16_t>* vw_ = nullptr;
    int64_t S_ = 0;
    char* seg_[4] = {nullptr, nullptr, nullptr, nullptr};
    size_t len_[4] = {0, 0, 0, 0};
    int cur_ = 0;
    size_t off_ = 0;
};

// Write rank `rank`'s file of an nd-rank checkpoint: header, the payload
// from `src` (exactly ckpt_payload_bytes(S) bytes), checksum. Written under
// a temporary name, then renamed.
CkptStatus ckpt_write_rank(const char* dir, int32_t nd, int32_t rank,
                           const std::vector<int64_t>& numel, int64_t S, int64_t step,
                           PayloadSource& src, std::string* err);

// Read rank `rank`'s file into `sink`, checking magic, header, length,
// checksum and that nothing follows it; returns the header's numel list, S
// and step. On failure the sink may have received part of the payload.
CkptStatus ckpt_stream_rank(const char* dir, int32_t nd, int32_t rank,
                            std::vector<int64_t>* numel, int64_t* S, int64_t* step,
                            PayloadSink& sink, std::string* err);

// The same checks with the payload discarded (read through `scratch`).
CkptStatus ckpt_verify_rank(const char* dir, int32_t nd, int32_t rank,
                            std::vector<int64_t>* numel, int64_t* S, int64_t* step,
                            void* scratch, size_t scratch_bytes, std::string* err);

// Number of ranks of the checkpoint in `dir` from the file names present.
// 0: none; -1: files of several rank counts.
int32_t ckpt_find_nd(const char* dir);

}  // namespace zsp
