/* Prints the size and field offsets of every struct in mfsdp.h as seen by a
 * C compiler, one "name value" per line; the test compares them with the
 * Python binding's ctypes declarations. */
#include <stddef.h>
#include <stdio.h>

#include "mfsdp.h"

#define SZ(t) printf("sizeof:%s %zu\n", #t, sizeof(t))
#define OF(t, f) printf("offsetof:%s.%s %zu\n", #t, #f, offsetof(t, f))

int main(void) {
    SZ(mfsdp_entry);
    OF(mfsdp_entry, offset); OF(mfsdp_entry, rows); OF(mfsdp_entry, cols); OF(mfsdp_entry, dtype); OF(mfsdp_entry, role);
    SZ(mfsdp_hparams);
    OF(mfsdp_hparams, lr); OF(mfsdp_hparams, weight_decay); OF(mfsdp_hparams, momentum); OF(mfsdp_hparams, nesterov);
    OF(mfsdp_hparams, ns_steps); OF(mfsdp_hparams, ns_a); OF(mfsdp_hparams, ns_b); OF(mfsdp_hparams, ns_c);
    OF(mfsdp_hparams, ns_eps); OF(mfsdp_hparams, lr_scale_mode); OF(mfsdp_hparams, ns_precision);
    OF(mfsdp_hparams, adam_lr); OF(mfsdp_hparams, adam_beta1); OF(mfsdp_hparams, adam_beta2); OF(mfsdp_hparams, adam_eps);
    OF(mfsdp_hparams, adam_weight_decay); OF(mfsdp_hparams, momentum_dtype); OF(mfsdp_hparams, ns_tile_gram);
    OF(mfsdp_hparams, ns_tile_poly); OF(mfsdp_hparams, ns_tile_update); OF(mfsdp_hparams, guard_bytes);
    SZ(mfsdp_region);
    OF(mfsdp_region, offset); OF(mfsdp_region, bytes); OF(mfsdp_region, buffer); OF(mfsdp_region, entry);
    SZ(mfsdp_entry_info);
    OF(mfsdp_entry_info, role); OF(mfsdp_entry_info, transposed); OF(mfsdp_entry_info, m); OF(mfsdp_entry_info, n);
    OF(mfsdp_entry_info, state_offset); OF(mfsdp_entry_info, state_offset2); OF(mfsdp_entry_info, ns_out_offset);
    OF(mfsdp_entry_info, lr_scale);
    SZ(mfsdp_step_args);
    OF(mfsdp_step_args, params); OF(mfsdp_step_args, grads); OF(mfsdp_step_args, state); OF(mfsdp_step_args, workspace);
    OF(mfsdp_step_args, workspace_bytes); OF(mfsdp_step_args, step); OF(mfsdp_step_args, stream);
    OF(mfsdp_step_args, ns_out); OF(mfsdp_step_args, flags); OF(mfsdp_step_args, events); OF(mfsdp_step_args, n_events);
    SZ(mfsdp_tensor);
    OF(mfsdp_tensor, rows); OF(mfsdp_tensor, cols); OF(mfsdp_tensor, dtype); OF(mfsdp_tensor, role);
    SZ(mfsdp_partition_params);
    OF(mfsdp_partition_params, n_owners); OF(mfsdp_partition_params, ns_steps); OF(mfsdp_partition_params, ns_precision);
    OF(mfsdp_partition_params, momentum_dtype); OF(mfsdp_partition_params, mem_cap_bytes);
    OF(mfsdp_partition_params, flop_rate); OF(mfsdp_partition_params, byte_rate);
    SZ(mfsdp_tensor_place);
    OF(mfsdp_tensor_place, owner); OF(mfsdp_tensor_place, role); OF(mfsdp_tensor_place, offset);
    OF(mfsdp_tensor_place, cost); OF(mfsdp_tensor_place, mem_bytes);
    return 0;
}
