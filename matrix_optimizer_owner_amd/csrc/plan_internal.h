// plan_internal.h - the host-side plan object shared by plan.cpp (lowering,
// no HIP calls) and step.hip (launch sequence).
#pragma once
#include <string>
#include <vector>

#include "layout.h"
#include "mfsdp.h"

struct mfsdp_plan_s {
    std::vector<mfsdp_entry> entries;
    std::vector<mfsdp_entry_info> info;
    mfsdp_hparams hp;
    mfsdp::WorkspaceMap map;
    std::vector<uint8_t> desc_blob;   // copied to the start of the workspace
    std::vector<mfsdp_region> regions;  // every state and workspace region, in layout order
    uint64_t state_bytes = 0;
    uint64_t ns_out_elems = 0;
    uint64_t max_param_end = 0;       // highest byte any entry touches
    uint64_t id = 0;                  // unique per plan in the process (never 0)
};

namespace mfsdp {
// Thread-local error text; returns `status` for convenient `return fail(...)`.
mfsdp_status fail(mfsdp_status status, const std::string& msg);
void clear_error();
}  // namespace mfsdp
