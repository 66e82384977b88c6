/* A stand-in for the four HIP runtime calls libiq's host code makes around
 * its kernel launches, for CPU-only tests of the launchers' error paths: a
 * test build of the library is linked against it, kernels never run, and
 * launch number `fail_at` (1-based) fails as a real failed launch would
 * (hipLaunchKernel returns an error that hipGetLastError then reports). */
#include <stddef.h>

typedef struct { unsigned x, y, z; } dim3;
typedef int hipError_t;

static int launches, fail_at, last_err, events;
static dim3 cfg_grid, cfg_block;
static size_t cfg_shared;
static void *cfg_stream;

hipError_t __hipPushCallConfiguration(dim3 grid, dim3 block, size_t shared, void *stream) {
  cfg_grid = grid; cfg_block = block; cfg_shared = shared; cfg_stream = stream;
  return 0;
}

hipError_t __hipPopCallConfiguration(dim3 *grid, dim3 *block, size_t *shared, void **stream) {
  *grid = cfg_grid; *block = cfg_block; *shared = cfg_shared; *stream = cfg_stream;
  return 0;
}

hipError_t hipLaunchKernel(const void *fn, dim3 grid, dim3 block, void **args, size_t shared, void *stream) {
  (void)fn; (void)grid; (void)block; (void)args; (void)shared; (void)stream;
  ++launches;
  if (launches == fail_at) { last_err = 1; return 1; }
  return 0;
}

hipError_t hipGetLastError(void) { int e = last_err; last_err = 0; return e; }

hipError_t hipEventRecord(void *event, void *stream) { (void)event; (void)stream; ++events; return 0; }

void stub_reset(int fail) { launches = 0; events = 0; last_err = 0; fail_at = fail; }
int stub_launches(void) { return launches; }
int stub_events(void) { return events; }
