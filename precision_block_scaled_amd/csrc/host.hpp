// Host-side plumbing shared by the C-ABI entry points: thread-local error
// text, argument checks, the PBS_LOG_LEVEL dispatch log, launch checks.
#pragma once
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/pbs.h"

namespace pbs {

pbs_status set_error(pbs_status st, const char* fmt, ...);
int log_level();
void log_dispatch(const char* fmt, ...);

// Check the last launch on this thread; returns PBS_OK or PBS_ERR_HIP.
pbs_status check_launch(const char* what);

#define PBS_REQUIRE(cond, status, ...)                  \
  do {                                                  \
    if (!(cond)) return ::pbs::set_error(status, __VA_ARGS__); \
  } while (0)

static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace pbs
