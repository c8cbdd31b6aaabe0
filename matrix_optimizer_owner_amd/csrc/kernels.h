// kernels.h - host-side launchers of the gfx950 kernels (one grouped launch
// per phase over every matrix of the plan).
#pragma once
#include <hip/hip_runtime.h>

#include "layout.h"
#include "mfsdp.h"

namespace mfsdp {

struct StepBuffers {
    uint8_t* params;
    const uint8_t* grads;
    uint8_t* state;
    uint8_t* ws;
    float* ns_out;
};

// Momentum / Nesterov / cast / orient, with Frobenius partial sums, then the
// per-matrix normalisation factor s = 1/(||U||_F + eps).
hipError_t launch_momentum(int ns_precision, const WorkspaceMap& map, const mfsdp_hparams& hp,
                           const StepBuffers& b, hipStream_t stream);

// O = s * X0 and the parameter update, for ns_steps == 0.
hipError_t launch_final_from_x(int ns_precision, const WorkspaceMap& map, const mfsdp_hparams& hp,
                               const StepBuffers& b, hipStream_t stream);

// AdamW over every tail tensor (step is 1-based).
hipError_t launch_adamw(const WorkspaceMap& map, const mfsdp_hparams& hp, int64_t step,
                        const StepBuffers& b, hipStream_t stream);

// One phase of Newton-Schulz iteration `iter` (1-based) over every matrix:
// phase 0 Gram, 1 polynomial, 2 update (the last iteration's update applies
// the parameter update).
hipError_t launch_ns_phase(int ns_precision, const WorkspaceMap& map, const mfsdp_hparams& hp, int iter,
                           int phase, const StepBuffers& b, hipStream_t stream);

}  // namespace mfsdp
