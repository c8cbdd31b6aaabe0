// step.hip - mfsdp_owner_step: enqueue one owner step on the caller's stream.
//
// Order on the stream: descriptor upload (unless resident), AdamW tail,
// momentum/cast/norm partials, norm finalize, ns_steps x (Gram, polynomial,
// update), the last update carrying the parameter write.  Nothing here
// synchronises; the owner step of MatrixFSDP (arXiv 2607.05895, Abstract)
// has no collective inside it, so the whole step is local to this stream.
#include <cmath>
#include <mutex>
#include <string>

#include "kernels.h"
#include "plan_internal.h"

using namespace mfsdp;

namespace {

mfsdp_status hip_fail(hipError_t e, const char* what) {
    return fail(MFSDP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

namespace {

// Checks of the step arguments other than the workspace.
mfsdp_status check_args(mfsdp_plan_t plan, const mfsdp_step_args* args) {
    const WorkspaceMap& map = plan->map;
    if (!args->params || !args->grads) return fail(MFSDP_ERR_INVALID_ARGUMENT, "params or grads is NULL");
    if (!args->state && plan->state_bytes > 0) return fail(MFSDP_ERR_INVALID_ARGUMENT, "state is NULL");
    if (reinterpret_cast<uintptr_t>(args->params) % 16 != 0 || reinterpret_cast<uintptr_t>(args->grads) % 16 != 0 ||
        (args->state && reinterpret_cast<uintptr_t>(args->state) % kAlign != 0))
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "params/grads must be 16-byte aligned and state 256-byte aligned");
    if (map.n_tail > 0 && args->step < 1)
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "step must be >= 1 (AdamW bias correction is 1-based)");
    if (args->ns_out && reinterpret_cast<uintptr_t>(args->ns_out) % 16 != 0)
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "ns_out must be 16-byte aligned");
    const uint32_t n_events = uint32_t(3 + 3 * plan->hp.ns_steps);
    if (args->events && args->n_events < n_events)
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "events array needs " + std::to_string(n_events) + " entries");
    return MFSDP_OK;
}

// The launch sequence of one step over workspace `ws` (checked by the caller).
mfsdp_status enqueue_step(mfsdp_plan_t plan, const mfsdp_step_args* args, uint8_t* ws, bool upload) {
    const WorkspaceMap& map = plan->map;
    hipStream_t stream = static_cast<hipStream_t>(args->stream);
    StepBuffers b;
    b.params = static_cast<uint8_t*>(args->params);
    b.grads = static_cast<const uint8_t*>(args->grads);
    b.state = static_cast<uint8_t*>(args->state);
    b.ws = ws;
    b.ns_out = args->ns_out;

    hipError_t e;
    auto mark = [&](uint32_t k) -> hipError_t {
        return args->events ? hipEventRecord(static_cast<hipEvent_t>(args->events[k]), stream) : hipSuccess;
    };
    if (upload && !plan->desc_blob.empty()) {
        e = hipMemcpyAsync(b.ws, plan->desc_blob.data(), plan->desc_blob.size(), hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) return hip_fail(e, "descriptor upload");
    }
    if ((e = mark(0)) != hipSuccess) return hip_fail(e, "event record");
    if (map.n_tail > 0) {
        e = launch_adamw(map, plan->hp, args->step, b, stream);
        if (e != hipSuccess) return hip_fail(e, "AdamW launch");
    }
    if ((e = mark(1)) != hipSuccess) return hip_fail(e, "event record");
    const int prec = plan->hp.ns_precision;
    if (map.n_mat > 0) {
        e = launch_momentum(prec, map, plan->hp, b, stream);
        if (e != hipSuccess) return hip_fail(e, "momentum launch");
        if (plan->hp.ns_steps == 0) {
            e = launch_final_from_x(prec, map, plan->hp, b, stream);
            if (e != hipSuccess) return hip_fail(e, "update launch");
        }
    }
    if ((e = mark(2)) != hipSuccess) return hip_fail(e, "event record");
    for (int it = 1; it <= plan->hp.ns_steps; ++it) {
        for (int ph = 0; ph < 3; ++ph) {
            if (map.n_mat > 0) {
                e = launch_ns_phase(prec, map, plan->hp, it, ph, b, stream);
                if (e != hipSuccess) return hip_fail(e, "Newton-Schulz launch");
            }
            if ((e = mark(uint32_t(3 * it + ph))) != hipSuccess) return hip_fail(e, "event record");
        }
    }
    return MFSDP_OK;
}

// ---- the library's own workspace, for mfsdp_owner_step_static ----
//
// One file-scope device array: every GPU the library runs on holds its own
// copy, at its own address, until the process ends.  In host code the
// name `scratch` is only a stand-in for the symbol (passing it to a kernel
// would hand the kernel a host address), so its device address is looked
// up once per device, with that device current, and only that address is
// used afterwards.  The step writes every workspace byte it reads before
// reading it, so nothing here needs clearing between calls.
constexpr uint64_t kStaticWorkspaceBytes = MFSDP_STATIC_WORKSPACE_BYTES;
__device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices] = {};           // device address of `scratch` per device
uint64_t g_static_last_plan[kMaxDevices] = {};  // plan whose descriptors the array holds (0: none)

}  // namespace

extern "C" mfsdp_status mfsdp_owner_step(mfsdp_plan_t plan, const mfsdp_step_args* args) {
    clear_error();
    if (!plan || !args) return fail(MFSDP_ERR_INVALID_ARGUMENT, "NULL plan or args");
    const WorkspaceMap& map = plan->map;
    if (map.n_mat == 0 && map.n_tail == 0) return MFSDP_OK;  // nothing but empty shards
    if (mfsdp_status st = check_args(plan, args); st != MFSDP_OK) return st;
    if (!args->workspace) return fail(MFSDP_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(args->workspace) % kAlign != 0)
        return fail(MFSDP_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    if (args->workspace_bytes < map.total_bytes)
        return fail(MFSDP_ERR_WORKSPACE_TOO_SMALL,
                    "workspace has " + std::to_string(args->workspace_bytes) + " bytes, plan needs " +
                        std::to_string(map.total_bytes));
    return enqueue_step(plan, args, static_cast<uint8_t*>(args->workspace),
                        !(args->flags & MFSDP_STEP_DESCRIPTORS_RESIDENT));
}

extern "C" mfsdp_status mfsdp_owner_step_static(mfsdp_plan_t plan, const mfsdp_step_args* args) {
    clear_error();
    if (!plan || !args) return fail(MFSDP_ERR_INVALID_ARGUMENT, "NULL plan or args");
    const WorkspaceMap& map = plan->map;
    if (map.n_mat == 0 && map.n_tail == 0) return MFSDP_OK;
    if (mfsdp_status st = check_args(plan, args); st != MFSDP_OK) return st;
    if (args->workspace || args->workspace_bytes)
        return fail(MFSDP_ERR_INVALID_ARGUMENT,
                    "mfsdp_owner_step_static uses the library's own workspace: pass workspace = NULL, "
                    "workspace_bytes = 0");
    if (map.total_bytes > kStaticWorkspaceBytes)
        return fail(MFSDP_ERR_WORKSPACE_TOO_SMALL,
                    "plan needs " + std::to_string(map.total_bytes) + " workspace bytes; the static workspace holds " +
                        std::to_string(kStaticWorkspaceBytes) + " (use mfsdp_owner_step with a caller workspace)");
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(MFSDP_ERR_UNSUPPORTED, "device index above the static table");
    uint8_t* ws = nullptr;
    bool upload = true;
    {
        std::lock_guard<std::mutex> lock(g_static_mu);
        if (!g_static_ptr[dev]) {
            void* ptr = nullptr;
            e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !ptr) return hip_fail(e, "hipGetSymbolAddress of the static workspace");
            g_static_ptr[dev] = ptr;
        }
        ws = static_cast<uint8_t*>(g_static_ptr[dev]);
        // descriptors are skipped only if this plan's are known to be there
        upload = !((args->flags & MFSDP_STEP_DESCRIPTORS_RESIDENT) && g_static_last_plan[dev] == plan->id);
        g_static_last_plan[dev] = plan->id;
    }
    return enqueue_step(plan, args, ws, upload);
}
