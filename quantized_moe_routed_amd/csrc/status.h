// The calling thread's last-error message behind moe_last_error (internal to
// libmoe; defined in host.cpp).
#pragma once
#include "../../include/moe.h"

namespace moe {
// Sets the message (printf format) and returns st.
moe_status fail(moe_status st, const char* fmt, ...);
// Clears the message and returns MOE_OK.
moe_status ok();
}  // namespace moe
