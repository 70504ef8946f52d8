// Host-side helpers shared by the translation units of the codec library
// (not part of the C ABI; hidden from the library's exported symbols).
#pragma once

#include "zc.h"

// A plan the codec accepts: flags 0 or ZC_PLAN_RAW_FALLBACK, exps strictly
// ascending.
__attribute__((visibility("hidden"))) bool zc_plan_is_valid(const zc_plan *p);
