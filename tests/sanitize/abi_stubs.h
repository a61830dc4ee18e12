// What the host-only launcher stand-ins recorded (see abi_stubs.cpp).
#pragma once
#include "attn_launch.h"

namespace stub {
enum { LAUNCH_NONE = 0, LAUNCH_FWD, LAUNCH_MASKED, LAUNCH_GENERAL, LAUNCH_ROPE_K, LAUNCH_DECODE, LAUNCH_MASKED_TUNED };
extern int calls;
extern int last;
extern attn_detail::LaunchArgs args;
extern attn_detail::DecodeArgs dargs;
extern void* k_out;
}  // namespace stub
