// Host-side bucket planning for libddp (no GPU work).
//
// Pages: [DDP] "DDP" (sgdbs.github.io, AI_Infra/1.DataParallel), sections 3.2
// and 4.2 -- parameters are taken in reverse registration order (gradients of
// the last layers are ready first in backward) and packed into buckets of
// about bucket_cap_mb, each bucket one flat tensor; [TR24] "(24) NCCL通信与分布式
// 数据并行", section 八 -- the two-bucket split DEEP_COMM / FIRST_COMM over the
// gradient regions, whose memory order is that of [TR16] "(16) DTensor：一张图纸，
// 多卡共享的分布式张量抽象", section 四 (regions in enum order, tensors placed
// one after another without gaps).
#include <climits>
#include <cstring>
#include <new>

#include "internal.h"

namespace {

int elem_bytes(ddp_dtype_t dt) { return dt == DDP_BF16 ? 2 : 4; }
bool dtype_ok(int dt) { return dt == DDP_F32 || dt == DDP_BF16; }

// Fills the derived tables of `p` from its buckets, given as lists of
// parameter indices in slot order.  Fails with OVERFLOW if the flat layout
// (in elements or in bytes) leaves int64.
ddp_status_t finish(ddp_plan *p, const std::vector<std::vector<int32_t>> &buckets)
{
    const int32_t n = p->n_params;
    p->slot_param.clear();
    p->slot_param.reserve(n);
    p->param_bucket.assign(n, -1);
    p->param_offset.assign(n, 0);
    p->bucket_base.clear();
    p->bucket_first_slot.clear();
    int64_t cursor = 0;
    const int64_t max_elems = INT64_MAX / 4;
    for (size_t b = 0; b < buckets.size(); ++b) {
        p->bucket_base.push_back(cursor);
        p->bucket_first_slot.push_back((int32_t)p->slot_param.size());
        int64_t within = 0;
        for (int32_t prm : buckets[b]) {
            p->param_bucket[prm] = (int32_t)b;
            p->param_offset[prm] = within;
            p->slot_param.push_back(prm);
            if (p->numel[prm] > max_elems - cursor) return DDP_ERR_OVERFLOW;
            within += p->numel[prm];
            cursor += p->numel[prm];
        }
    }
    p->bucket_base.push_back(cursor);
    p->bucket_first_slot.push_back((int32_t)p->slot_param.size());
    p->total = cursor;
    return DDP_OK;
}

ddp_status_t new_plan(const int64_t *numel, int32_t n_params, ddp_dtype_t dtype,
                      ddp_plan **out)
{
    ddp_plan *p = new (std::nothrow) ddp_plan();
    if (!p) return DDP_ERR_NOMEM;
    p->dtype = dtype;
    p->n_params = n_params;
    try {
        p->numel.assign(numel, numel + n_params);
    } catch (...) {
        delete p;
        return DDP_ERR_NOMEM;
    }
    *out = p;
    return DDP_OK;
}

ddp_status_t check_common(const int64_t *numel, int32_t n_params, int dtype, void *out)
{
    if (!numel || !out || n_params < 1 || !dtype_ok(dtype)) return DDP_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n_params; ++i)
        if (numel[i] < 0) return DDP_ERR_INVALID_ARG;
    return DDP_OK;
}

}  // namespace

extern "C" {

ddp_status_t ddp_plan_buckets(const int64_t *numel, int32_t n_params,
                              int64_t bucket_cap_bytes, ddp_dtype_t dtype,
                              ddp_plan_t **out)
{
    ddp_status_t st = check_common(numel, n_params, (int)dtype, out);
    if (st != DDP_OK) return st;
    if (bucket_cap_bytes <= 0) return DDP_ERR_INVALID_ARG;
    const int64_t eb = elem_bytes(dtype);
    for (int32_t i = 0; i < n_params; ++i)
        if (numel[i] > INT64_MAX / eb) return DDP_ERR_OVERFLOW;

    ddp_plan *p = nullptr;
    if ((st = new_plan(numel, n_params, dtype, &p)) != DDP_OK) return st;
    try {
        // Walk from the last-registered parameter to the first.  `fill` is
        // the byte count of the open (never empty) bucket, saturated at
        // cap + 1 once a lone oversize parameter sits in it.  A parameter
        // that does not fit in what is left starts the next bucket.
        std::vector<std::vector<int32_t>> buckets;
        int64_t fill = 0;
        for (int32_t prm = n_params - 1; prm >= 0; --prm) {
            const int64_t bytes = numel[prm] * eb;
            if (buckets.empty() || bytes > bucket_cap_bytes - fill) {
                buckets.emplace_back();
                fill = 0;
            }
            buckets.back().push_back(prm);
            fill = (bytes > bucket_cap_bytes - fill) ? bucket_cap_bytes + 1 : fill + bytes;
        }
        st = finish(p, buckets);
    } catch (...) {
        st = DDP_ERR_NOMEM;
    }
    if (st != DDP_OK) {
        delete p;
        return st;
    }
    *out = p;
    return DDP_OK;
}

ddp_status_t ddp_plan_two_bucket(const int64_t *numel, const uint8_t *region,
                                 int32_t n_params, ddp_dtype_t dtype, ddp_plan_t **out)
{
    ddp_status_t st = check_common(numel, n_params, (int)dtype, out);
    if (st != DDP_OK) return st;
    if (!region) return DDP_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n_params; ++i)
        if (region[i] > DDP_REGION_DEEP) return DDP_ERR_INVALID_ARG;

    ddp_plan *p = nullptr;
    if ((st = new_plan(numel, n_params, dtype, &p)) != DDP_OK) return st;
    try {
        // DEEP_COMM first: it is the bucket whose all-reduce starts while the
        // first layer's backward still runs.  FIRST_COMM then covers the
        // regions BN_BIAS .. FIRST as one span in region order.
        std::vector<std::vector<int32_t>> by_region(DDP_REGION_DEEP + 1);
        for (int32_t i = 0; i < n_params; ++i) by_region[region[i]].push_back(i);
        std::vector<std::vector<int32_t>> buckets;
        if (!by_region[DDP_REGION_DEEP].empty()) buckets.push_back(by_region[DDP_REGION_DEEP]);
        std::vector<int32_t> first_comm;
        for (int r = DDP_REGION_BN_BIAS; r <= DDP_REGION_FIRST; ++r)
            first_comm.insert(first_comm.end(), by_region[r].begin(), by_region[r].end());
        if (!first_comm.empty()) buckets.push_back(first_comm);
        st = finish(p, buckets);
    } catch (...) {
        st = DDP_ERR_NOMEM;
    }
    if (st != DDP_OK) {
        delete p;
        return st;
    }
    *out = p;
    return DDP_OK;
}

void ddp_plan_free(ddp_plan_t *plan)
{
    if (!plan) return;
    ddp_internal_free_plan_tables(plan);
    delete plan;
}

int32_t ddp_plan_num_buckets(const ddp_plan_t *plan) { return plan ? plan->n_buckets() : -1; }

int64_t ddp_plan_total(const ddp_plan_t *plan) { return plan ? plan->total : -1; }

ddp_status_t ddp_plan_bucket(const ddp_plan_t *plan, int32_t b, int64_t *len,
                             int64_t *base, int32_t *first_slot, int32_t *n_slots)
{
    if (!plan || b < 0 || b >= plan->n_buckets()) return DDP_ERR_INVALID_ARG;
    if (len) *len = plan->bucket_base[b + 1] - plan->bucket_base[b];
    if (base) *base = plan->bucket_base[b];
    if (first_slot) *first_slot = plan->bucket_first_slot[b];
    if (n_slots) *n_slots = plan->bucket_first_slot[b + 1] - plan->bucket_first_slot[b];
    return DDP_OK;
}

ddp_status_t ddp_plan_slot_param(const ddp_plan_t *plan, int32_t slot, int32_t *param)
{
    if (!plan || !param || slot < 0 || slot >= plan->n_params) return DDP_ERR_INVALID_ARG;
    *param = plan->slot_param[slot];
    return DDP_OK;
}

ddp_status_t ddp_plan_param(const ddp_plan_t *plan, int32_t p, int32_t *bucket,
                            int64_t *offset)
{
    if (!plan || p < 0 || p >= plan->n_params) return DDP_ERR_INVALID_ARG;
    if (bucket) *bucket = plan->param_bucket[p];
    if (offset) *offset = plan->param_offset[p];
    return DDP_OK;
}

ddp_status_t ddp_plan_set_occupancy(ddp_plan_t *plan, ddp_occupancy_t policy)
{
    if (!plan || (policy != DDP_OCCUPANCY_TUNED && policy != DDP_OCCUPANCY_SHARED &&
                  policy != DDP_OCCUPANCY_DEFAULT))
        return DDP_ERR_INVALID_ARG;
    plan->occupancy.store(policy, std::memory_order_relaxed);
    return DDP_OK;
}

ddp_occupancy_t ddp_plan_get_occupancy(const ddp_plan_t *plan)
{
    return plan ? static_cast<ddp_occupancy_t>(plan->occupancy.load(std::memory_order_relaxed))
                : DDP_OCCUPANCY_DEFAULT;
}

const char *ddp_status_string(ddp_status_t status)
{
    switch (status) {
    case DDP_OK: return "ok";
    case DDP_ERR_INVALID_ARG: return "invalid argument";
    case DDP_ERR_UNSUPPORTED: return "unsupported dtype pair or rank count";
    case DDP_ERR_OVERFLOW: return "size overflows the int64 layout";
    case DDP_ERR_ALIAS: return "output partially overlaps an input";
    case DDP_ERR_HIP: return "HIP runtime error";
    case DDP_ERR_NOMEM: return "out of memory";
    case DDP_ERR_CAPACITY: return "exceeds the static buffer of the no-allocation entry point";
    }
    return "unknown status";
}

int32_t ddp_abi_version(void) { return DDP_ABI_VERSION; }

}  // extern "C"
