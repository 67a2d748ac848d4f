// zsp_plan.hpp -- the plan behind the opaque zsp_plan handle: layout
// tables on the host, the bound state pointers, the device copies of the
// piece tables, and the checkpoint staging the plan keeps between calls.
#pragma once

#include <cstdint>
#include <vector>

#include "zsp.h"
#include "zsp_internal.hpp"

namespace zsp {
struct CkptStaging;                    // pinned chunks, streams, events (zsp_ckpt_dev.cpp)
void staging_free(CkptStaging* st);    // NULL is a no-op
struct ListStaging;                    // staging slots of long list gathers (zsp_gather_list.cpp)
ListStaging* list_staging_new();       // NULL when out of host memory
void list_staging_free(ListStaging* ls);  // NULL is a no-op
}  // namespace zsp

struct zsp_plan {
    int32_t T = 0;
    int32_t nd = 0;
    std::vector<int64_t> numel, pad, shard_len, full_off, shard_off, flat_off;
    std::vector<int64_t> piece_off;  // gather pieces (rank runs) before parameter t
    std::vector<int64_t> slot_off;   // parameters with shard_len > 0 before parameter t
    int64_t S = 0;
    int64_t total_padded = 0;
    int64_t total_numel = 0;

    bool bound = false;
    int32_t bind_rank = ZSP_ALL_RANKS;
    int device = -1;
    float* master = nullptr;
    float* m = nullptr;
    float* v = nullptr;
    uint16_t* work = nullptr;
    float* acc = nullptr;

    void* dev_blob = nullptr;  // one device allocation holding every table
    zsp::ShardTable shard;
    zsp::GatherTable gather;
    std::vector<int64_t> span_k;  // first flat index of each span (host copy)
    const zsp::ParamInfo* params = nullptr;  // per parameter (all-rank bindings)
    zsp::ListStaging* lists = nullptr;       // made at an all-rank bind

    zsp::CkptStaging* staging = nullptr;  // made by the first checkpoint save / load
};

