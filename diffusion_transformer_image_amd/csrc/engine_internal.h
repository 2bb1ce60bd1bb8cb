// Host-side helpers the engine shares with the weight loader (not part of
// the C ABI).
#pragma once

#include <string>

#include "../../include/zimg_dit.h"

namespace zimg {
// Record ``msg`` as the calling thread's last error and return ``code``.
int set_error(int code, const std::string& msg);
// The configuration a handle was made with; whether its weights are final.
const zimg_dit_config* handle_config(const zimg_dit* h);
bool handle_finalized(const zimg_dit* h);
}  // namespace zimg
