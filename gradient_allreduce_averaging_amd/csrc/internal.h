// Internal definitions shared by the host planner (plan.cpp) and the HIP
// launch code (reduce.hip, copy.hip, params.hip).  Not part of the ABI.
#pragma once

#include <cstdint>
#include <atomic>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>
#include <vector>

#include "ddp.h"

// Device-side copy of a plan's bucket table, for one device and one tile size.
struct ddp_dev_tables {
    int64_t *bucket_base = nullptr;   // [n_buckets + 1] flat start of each bucket, then total
    int32_t *tile_bucket = nullptr;   // bucket holding the first element of every
                                      // 2^kTileTableShift-th tile
    int64_t n_tiles = 0;
};

struct ddp_plan {
    ddp_dtype_t dtype = DDP_F32;
    int32_t n_params = 0;
    int64_t total = 0;                        // elements in the flat layout
    std::vector<int64_t> numel;               // registration order
    std::vector<int32_t> slot_param;          // parameter at each flat slot
    std::vector<int32_t> param_bucket;        // bucket of each parameter
    std::vector<int64_t> param_offset;        // element offset inside its bucket
    std::vector<int64_t> bucket_base;         // [n_buckets + 1], last entry = total
    std::vector<int32_t> bucket_first_slot;   // [n_buckets + 1], last entry = n_params

    int32_t n_buckets() const { return (int32_t)bucket_base.size() - 1; }

    std::atomic<int> occupancy{DDP_OCCUPANCY_DEFAULT};   // of the launches over this plan
    std::mutex mu;                            // guards dev and ring_desc
    std::map<std::pair<int, int64_t>, ddp_dev_tables> dev;   // (device, tile elements)
    // (device, tile elements, ranks): device array of one ring-segment word per tile
    std::map<std::tuple<int, int64_t, int>, uint32_t *> ring_desc;
};

// One flatten/unflatten copy unit: `count` elements between a parameter's
// gradient and the flat buffer.  Units are sorted by flat position, so the
// units of bucket b are the range [bucket_first_unit[b], bucket_first_unit[b+1]).
struct ddp_copy_unit {
    uint64_t param_addr;   // device address of the parameter's gradient
    int64_t param_elem;    // first element of this unit inside the parameter
    int64_t flat_elem;     // first flat element of this unit
    int32_t count;         // elements, 1..kCopyUnitElems
    int32_t more;          // bits 0-7: elements of the same parameter after this unit, at
                           // most 16; bits 8 + 2e, 9 + 2e: the parameter's first / last
                           // 16-byte chunk in its own storage is shared with another
                           // parameter, for elements of 2 << e bytes (unflatten)
};

// A 16-byte chunk of parameter storage that holds bytes of two or more bound
// parameters (views carved out of one buffer), as unflatten writes it for
// one bucket: piece[k] is the flat byte offset of the chunk's bytes
// [2k, 2k + 2), or -1 where they belong to no parameter of that bucket.
struct ddp_unflatten_edge {
    uint64_t chunk;
    int64_t piece[8];
};

struct ddp_binding {
    const ddp_plan *plan = nullptr;
    int device = -1;
    ddp_copy_unit *units = nullptr;           // device array: the units, then tensor_first
    int64_t n_units = 0;
    int64_t *tensor_first = nullptr;          // device: each parameter's first unit and flat
                                              // element (pairs of int64), in flat order
    std::vector<int64_t> bucket_first_unit;   // [n_buckets + 1]
    std::vector<int64_t> bucket_first_tensor; // [n_buckets + 1] into tensor_first
    std::vector<uint8_t> bucket_edge_mask;    // [n_buckets] bit f % 8 for every flat element f
                                              // at which one of its parameters starts or it ends
    uint8_t edge_mask = 0;                    // the union over all buckets
    ddp_unflatten_edge *uedges[2] = {nullptr, nullptr};   // device, per element size 2 << e,
                                              // grouped by bucket (in the units' allocation)
    std::vector<int64_t> bucket_first_uedge[2];   // [n_buckets + 1] into uedges[e]
    std::vector<uint64_t> param_addr;         // [n_params] the bound gradient pointers
};

// A synchronisation over per-parameter tensors (params.hip): an 8-byte record
// per tile of each parameter (its parameter and ring chunks), then an entry
// per parameter with every rank's address and those of the tensors it writes.
struct ddp_param_sync {
    int device = -1;
    int n_ranks = 0;
    int order = 0;
    int in = 0, out = 0;                      // ddp_dtype_t of inputs and outputs
    bool sgd = false;                         // built by ddp_param_sgd_create
    bool momentum = false;                    // sgd: with a momentum buffer
    std::atomic<int> occupancy{DDP_OCCUPANCY_DEFAULT};   // of its launches
    char *table = nullptr;                    // device array: tile records, then parameter entries
    int64_t n_tiles = 0;
    int64_t rstride = 0;                      // tile records per XCD stripe
    int64_t pstride = 0;                      // bytes per parameter entry
    int64_t params_offset = 0;                // byte offset of the parameter entries
    std::vector<int64_t> bucket_tile;         // [n_buckets + 1] first entry of each bucket
};

// Frees every device table of a plan (defined next to the kernels).
void ddp_internal_free_plan_tables(ddp_plan *plan);
