// checkpoint.cpp - owner-shard checkpoint resharding: byte copies between one
// owner's flat buffers and whole per-tensor buffers.  Host only (no HIP).
//
// "MatrixFSDP: Communication-Free Matrix Optimizers Under ZeRO-3 Parameter
// Sharding" (arXiv 2607.05895), Abstract: owner-shard checkpoint resharding.
// The owner's layout is its plan's: parameters at the table's offsets,
// fp32 state at the offsets mfsdp_plan_create assigned (Muon momentum,
// AdamW first and second moments).
#include <cstring>
#include <string>

#include "plan_internal.h"

using namespace mfsdp;

namespace {

int elem_bytes(int32_t dtype) { return dtype == kBF16 ? 2 : 4; }

// Walk the plan's entries; for each part that applies and whose array is
// given, call copy(flat offset, bytes, per-tensor pointer slot, is_state).
template <typename F>
mfsdp_status walk(mfsdp_plan_t plan, uint64_t param_bytes, uint64_t state_bytes, bool want_params, bool want_s1,
                  bool want_s2, F&& copy) {
    if (!plan) return fail(MFSDP_ERR_INVALID_ARGUMENT, "null plan");
    if (want_params && param_bytes < plan->max_param_end)
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "param buffer smaller than the table's extent");
    if ((want_s1 || want_s2) && state_bytes < plan->state_bytes)
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "state buffer smaller than the plan's state");
    const int64_t n = int64_t(plan->entries.size());
    for (int64_t i = 0; i < n; ++i) {
        const mfsdp_entry& e = plan->entries[size_t(i)];
        const mfsdp_entry_info& inf = plan->info[size_t(i)];
        const uint64_t numel = uint64_t(e.rows) * uint64_t(e.cols);
        if (numel == 0) continue;
        if (want_params) {
            const mfsdp_status st = copy(i, 0, e.offset, numel * uint64_t(elem_bytes(e.dtype)));
            if (st != MFSDP_OK) return st;
        }
        if (want_s1) {
            const uint64_t s1_bytes =
                inf.role == MFSDP_ROLE_MUON && plan->hp.momentum_dtype == MFSDP_BF16 ? 2 : 4;
            const mfsdp_status st = copy(i, 1, inf.state_offset, numel * s1_bytes);
            if (st != MFSDP_OK) return st;
        }
        if (want_s2 && inf.role == MFSDP_ROLE_ADAMW) {
            const mfsdp_status st = copy(i, 2, inf.state_offset2, numel * 4);
            if (st != MFSDP_OK) return st;
        }
    }
    return MFSDP_OK;
}

}  // namespace

extern "C" mfsdp_status mfsdp_owner_gather(mfsdp_plan_t plan, const void* params, uint64_t param_bytes,
                                           const void* state, uint64_t state_bytes, void* const* tensors,
                                           void* const* state1, void* const* state2) {
    clear_error();
    if ((tensors && !params) || ((state1 || state2) && !state))
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "null owner buffer");
    void* const* arrays[3] = {tensors, state1, state2};
    return walk(plan, param_bytes, state_bytes, tensors != nullptr, state1 != nullptr, state2 != nullptr,
                [&](int64_t i, int part, uint64_t off, uint64_t bytes) -> mfsdp_status {
                    void* dst = arrays[part][i];
                    if (!dst)
                        return fail(MFSDP_ERR_INVALID_ARGUMENT,
                                    "entry " + std::to_string(i) + ": null per-tensor buffer");
                    const uint8_t* src = static_cast<const uint8_t*>(part == 0 ? params : state) + off;
                    std::memcpy(dst, src, bytes);
                    return MFSDP_OK;
                });
}

extern "C" mfsdp_status mfsdp_owner_scatter(mfsdp_plan_t plan, const void* const* tensors, const void* const* state1,
                                            const void* const* state2, void* params, uint64_t param_bytes,
                                            void* state, uint64_t state_bytes) {
    clear_error();
    if ((tensors && !params) || ((state1 || state2) && !state))
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "null owner buffer");
    const void* const* arrays[3] = {tensors, state1, state2};
    return walk(plan, param_bytes, state_bytes, tensors != nullptr, state1 != nullptr, state2 != nullptr,
                [&](int64_t i, int part, uint64_t off, uint64_t bytes) -> mfsdp_status {
                    const void* src = arrays[part][i];
                    if (!src)
                        return fail(MFSDP_ERR_INVALID_ARGUMENT,
                                    "entry " + std::to_string(i) + ": null per-tensor buffer");
                    uint8_t* dst = static_cast<uint8_t*>(part == 0 ? params : state) + off;
                    std::memcpy(dst, src, bytes);
                    return MFSDP_OK;
                });
}
