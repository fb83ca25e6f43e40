// Helpers the C ABI's translation units share (host only).
#pragma once

#include "../../include/gemm.h"

namespace dtg {

// Store `msg` as the calling thread's last error (gemm_last_error) and return st.
gemm_status record_error(gemm_status st, const char* msg);

// gemm_device_query for `device`, cached per device.
gemm_status cached_device_info(int device, gemm_device_info* info);

}  // namespace dtg
