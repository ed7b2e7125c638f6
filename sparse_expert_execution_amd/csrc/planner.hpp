// planner.hpp - internal interface of the LRU planner used by the cache.
#pragma once
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {
int set_error(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int planner_plan(moe_planner* p, int32_t layer, const int32_t* ids, const float* w, int32_t n,
                 int32_t q, moe_plan* plan);
int planner_rollback(moe_planner* p);
int planner_resize(moe_planner* p, int32_t n_new, int32_t* old_of_new);
void planner_forget_slot(moe_planner* p, int32_t slot);
int32_t planner_slot_key(const moe_planner* p, int32_t slot);
}  // namespace moe
