// Host-side argument checks of the device entry points (plain C++, no HIP):
// dims, row counts and flags.  The workspace layouts they size are in
// layout.h.
#pragma once
#include "layout.h"

namespace moe {

// MOE_OK, or the status a decode call (rows <= MOE_MAX_DECODE_ROWS) with
// these dims must return before launching anything.
int check_dims(const moe_dims* d, int rows);
// The same for the many-row path (MOE_MAX_DECODE_ROWS < rows <=
// MOE_MAX_PREFILL_ROWS).
int check_many_row_dims(const moe_dims* d, int rows);

}  // namespace moe
