// Error reporting, dispatch logging, version and storage accounting.
#include <stdlib.h>
#include <string.h>

#include "host.hpp"

namespace pbs {

static thread_local char g_err[512] = "";

pbs_status set_error(pbs_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  if (log_level() > 0) fprintf(stderr, "[pbs] error %d: %s\n", (int)st, g_err);
  return st;
}

int log_level() {
  static int level = -1;
  if (level < 0) {
    const char* s = getenv("PBS_LOG_LEVEL");
    level = s ? atoi(s) : 0;
  }
  return level;
}

void log_dispatch(const char* fmt, ...) {
  if (log_level() <= 0) return;
  va_list ap;
  va_start(ap, fmt);
  fprintf(stderr, "[pbs] ");
  vfprintf(stderr, fmt, ap);
  fprintf(stderr, "\n");
  va_end(ap);
}

pbs_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(PBS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return PBS_OK;
}

}  // namespace pbs

extern "C" {

const char* pbs_last_error(void) { return pbs::g_err; }

int pbs_version(void) { return PBS_VERSION; }

pbs_status pbs_quantized_bytes(pbs_recipe recipe, int64_t rows, int64_t cols, int weight_2d,
                               size_t* code_bytes, size_t* scale_bytes) {
  PBS_REQUIRE(code_bytes && scale_bytes, PBS_ERR_INVALID_ARG, "null output pointer");
  PBS_REQUIRE(rows >= 0 && cols >= 0, PBS_ERR_SHAPE, "negative shape");
  int64_t n = rows * cols;
  switch (recipe) {
    case PBS_RECIPE_BF16:
      *code_bytes = (size_t)n * 2; *scale_bytes = 0; break;
    case PBS_RECIPE_FP8_CURRENT:
    case PBS_RECIPE_FP8_DELAYED:
      *code_bytes = (size_t)n; *scale_bytes = 0; break;
    case PBS_RECIPE_FP8_BLOCK128:
    case PBS_RECIPE_FP8_BLOCK128_1D1D:
    case PBS_RECIPE_FP8_BLOCK128_2D2D:
      PBS_REQUIRE(cols % 128 == 0 && (!weight_2d || rows % 128 == 0), PBS_ERR_SHAPE,
                  "block128 needs dims that are multiples of 128");
      *code_bytes = (size_t)n;
      *scale_bytes = (size_t)(weight_2d ? (rows / 128) * (cols / 128) : rows * (cols / 128)) * 4;
      break;
    case PBS_RECIPE_FP8_BLOCK128_POW2:
      PBS_REQUIRE(cols % 128 == 0 && (!weight_2d || rows % 128 == 0), PBS_ERR_SHAPE,
                  "block128 needs dims that are multiples of 128");
      *code_bytes = (size_t)n;
      *scale_bytes = (size_t)(weight_2d ? (rows / 128) * (cols / 128) : rows * (cols / 128)) * 4;
      break;
    case PBS_RECIPE_MXFP8:
      PBS_REQUIRE(cols % 32 == 0, PBS_ERR_SHAPE, "MXFP8 needs cols % 32 == 0");
      *code_bytes = (size_t)n; *scale_bytes = (size_t)(rows * (cols / 32)); break;
    case PBS_RECIPE_NVFP4:
      PBS_REQUIRE(cols % 16 == 0 && (!weight_2d || rows % 16 == 0), PBS_ERR_SHAPE,
                  "NVFP4 needs dims that are multiples of 16");
      *code_bytes = (size_t)(n / 2);
      *scale_bytes = (size_t)(weight_2d ? (rows / 16) * (cols / 16) : rows * (cols / 16));
      break;
    case PBS_RECIPE_FP8_CHANNEL:
      *code_bytes = (size_t)n; *scale_bytes = (size_t)rows * 4; break;
    case PBS_RECIPE_MXFP4:
      PBS_REQUIRE(cols % 32 == 0, PBS_ERR_SHAPE, "MXFP4 needs cols % 32 == 0");
      *code_bytes = (size_t)(n / 2); *scale_bytes = (size_t)(rows * (cols / 32)); break;
    default:
      return pbs::set_error(PBS_ERR_INVALID_ARG, "unknown recipe %d", (int)recipe);
  }
  return PBS_OK;
}

}  // extern "C"
