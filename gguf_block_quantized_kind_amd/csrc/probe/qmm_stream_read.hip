// qmm_stream_read.hip -- a plain streaming-read kernel, the practical HBM
// ceiling that the decode GEMV is measured against (built into its own
// library, libqmm_probe.so; not part of the matmul C ABI).
//
// Every byte of a buffer is read once with 16-byte loads: each lane takes
// four words per iteration at a stride of the whole grid and folds them with
// XOR, and stores its fold only when it equals `never`, a value the caller
// picks (so the loads cannot be dropped, and in practice nothing is stored;
// a store that does happen stays inside `out`).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ p, int64_t n16, uint32_t never,
                                                          uint32_t *__restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < n16; i += stride) acc ^= p[i];
  const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (r == never) out[(int64_t)blockIdx.x * 256 + threadIdx.x] = r;
}

// Reads `bytes` bytes at p (16-byte aligned, bytes a multiple of 16) with
// `grid` workgroups of 256 lanes on `stream`; out holds grid * 256 words.
// Returns 0, or -1 for bad arguments, or the HIP error of the launch.
extern "C" __attribute__((visibility("default"))) int qmm_probe_stream_read(const void *p, int64_t bytes, int grid,
                                                                            uint32_t never, uint32_t *out,
                                                                            void *stream) {
  if (!p || !out || bytes <= 0 || bytes % 16 != 0 || (uintptr_t)p % 16 != 0 || grid <= 0) return -1;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4 *)p, bytes / 16, never, out);
  return (int)hipGetLastError();
}
