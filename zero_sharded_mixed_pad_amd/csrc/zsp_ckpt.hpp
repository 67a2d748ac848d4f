// zsp_ckpt.hpp -- per-rank shard files of a sharded checkpoint (format in
// zsp_ckpt.cpp), used by the checkpoint entry points in zsp_capi.cpp.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace zsp {

enum class CkptStatus { Ok, Io, Missing, Corrupt };

CkptStatus ckpt_write_rank(const char* dir, int32_t nd, int32_t rank,
                           const std::vector<int64_t>& numel, int64_t S, int64_t step,
                           const float* master, const float* m, const float* v,
                           const uint16_t* work, std::string* err);
CkptStatus ckpt_read_rank(const char* dir, int32_t nd, int32_t rank, std::vector<int64_t>* numel,
                          int64_t* S, int64_t* step, std::vector<float>* master,
                          std::vector<float>* m, std::vector<float>* v,
                          std::vector<uint16_t>* work, std::string* err);
int32_t ckpt_find_nd(const char* dir);

}  // namespace zsp
