// Error reporting shared by the C ABI entry points of libnkv.so: the message that
// nkv_last_error() returns is kept per calling thread (defined in api.hip).
#pragma once

#include "nkv.h"

namespace nkv {
nkv_status_t set_error(nkv_status_t st, const char* msg);   // returns st
nkv_status_t clear_error();                                // returns NKV_OK
}  // namespace nkv
