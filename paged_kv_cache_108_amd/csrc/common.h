// Shared host-side helpers of libpkv: the per-thread error message and the
// status plumbing. No device code here.
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "../../include/pkv.h"

namespace pkv {

// Records a printf-style message for pkv_last_error() and returns `st`.
pkv_status fail(pkv_status st, const char* fmt, ...);
// Clears the message (called by successful entry points).
pkv_status ok();

inline bool is_pow2_block(int32_t bs) { return bs == 8 || bs == 16 || bs == 32 || bs == 64 || bs == 128; }
inline bool is_head_dim(int32_t d) { return d == 64 || d == 128; }

}  // namespace pkv
