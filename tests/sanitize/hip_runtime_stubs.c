/* Host stand-ins for the HIP runtime (test infrastructure only).
 *
 * The library's sources compiled host-only (hipcc --offload-host-only) call
 * these instead of libamdhip64, so that every host-side step of an entry
 * point -- argument validation, defaults, launch-shape arithmetic -- runs
 * under AddressSanitizer and UndefinedBehaviorSanitizer on a machine with
 * no GPU.  A kernel launch is checked for a plausible shape and counted;
 * nothing runs.  The device reports 256 compute units and four resident
 * workgroups per CU for every kernel. */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef struct { uint32_t x, y, z; } dim3;
typedef struct { uint32_t x, y, z; } uint3;
typedef void *hipStream_t;

unsigned long stub_launches = 0;  /* read by the driver */
unsigned long stub_bad_launches = 0;

static void *module_handle;
static dim3 cfg_grid, cfg_block;
static size_t cfg_shmem;
static hipStream_t cfg_stream;

void **__hipRegisterFatBinary(const void *data) {
  (void)data;
  return &module_handle;
}
void __hipUnregisterFatBinary(void **modules) { (void)modules; }
void __hipRegisterFunction(void **modules, const void *host_fn, char *device_fn,
                           const char *device_name, unsigned int thread_limit, uint3 *tid,
                           uint3 *bid, dim3 *block, dim3 *grid, int *wsize) {
  (void)modules; (void)host_fn; (void)device_fn; (void)device_name; (void)thread_limit;
  (void)tid; (void)bid; (void)block; (void)grid; (void)wsize;
}
void __hipRegisterVar(void **modules, void *var, char *host_var, char *device_var, int ext,
                      size_t size, int constant, int global) {
  (void)modules; (void)var; (void)host_var; (void)device_var; (void)ext; (void)size;
  (void)constant; (void)global;
}
int __hipPushCallConfiguration(dim3 grid, dim3 block, size_t shmem, hipStream_t stream) {
  cfg_grid = grid; cfg_block = block; cfg_shmem = shmem; cfg_stream = stream;
  return 0;
}
int __hipPopCallConfiguration(dim3 *grid, dim3 *block, size_t *shmem, hipStream_t *stream) {
  *grid = cfg_grid; *block = cfg_block; *shmem = cfg_shmem; *stream = cfg_stream;
  return 0;
}
int hipLaunchKernel(const void *fn, dim3 grid, dim3 block, void **args, size_t shmem,
                    hipStream_t stream) {
  (void)fn; (void)args; (void)stream;
  const int ok = grid.x >= 1 && grid.x <= 0x7FFFFFFFu && grid.y == 1 && grid.z == 1 &&
                 block.x >= 64 && block.x <= 1024 && block.x % 64 == 0 && block.y == 1 &&
                 block.z == 1 && shmem <= 65536;
  if (!ok) {
    fprintf(stderr, "implausible launch: grid %u,%u,%u block %u,%u,%u shmem %zu\n", grid.x, grid.y,
            grid.z, block.x, block.y, block.z, shmem);
    ++stub_bad_launches;
  }
  ++stub_launches;
  return 0;
}
int hipGetDevice(int *dev) {
  *dev = 0;
  return 0;
}
int hipDeviceGetAttribute(int *value, int attr, int dev) {
  (void)attr; (void)dev;
  *value = 256;
  return 0;
}
int hipOccupancyMaxActiveBlocksPerMultiprocessor(int *n, const void *fn, int block, size_t shmem) {
  (void)fn; (void)block; (void)shmem;
  *n = 4;
  return 0;
}
int hipGetSymbolAddress(void **ptr, const void *symbol) {
  static _Alignas(256) unsigned char memory[1 << 17];
  (void)symbol;
  *ptr = memory;
  return 0;
}
int hipGetLastError(void) { return 0; }
