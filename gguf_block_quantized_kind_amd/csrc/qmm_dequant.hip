// qmm_dequant.hip -- whole-block dequantization to f32.  One thread decodes
// one 16-element sub-block with the shared decoders, so this kernel is the
// bit-exact check of those decoders against the oracle.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

template <int KIND>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ W,
                                                      float *__restrict__ out, int64_t n_subs) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_subs) return;
  const int64_t blk = t / kSubs<KIND>;
  const int sub = (int)(t % kSubs<KIND>);
  float v[16];
  decode16<KIND>(W + blk * Geometry<KIND>::bytes, sub, v);
  float *o = out + t * 16;
#pragma unroll
  for (int i = 0; i < 16; ++i) o[i] = v[i];
}

template <int KIND>
static hipError_t run_dequant(const uint8_t *W, float *out, int64_t n_blocks, hipStream_t s) {
  const int64_t n_subs = n_blocks * kSubs<KIND>;
  const int64_t grid = (n_subs + 255) / 256;
  hipLaunchKernelGGL(dequant_kernel<KIND>, dim3((unsigned)grid), dim3(256), 0, s, W, out, n_subs);
  return hipGetLastError();
}

hipError_t launch_dequant(int kind, const uint8_t *W, float *out, int64_t n_blocks, hipStream_t s) {
  switch (kind) {
#define QMM_CASE(K) \
  case K:           \
    return run_dequant<K>(W, out, n_blocks, s);
    QMM_FOR_EACH_KIND(QMM_CASE)
#undef QMM_CASE
  }
  return hipErrorInvalidValue;
}

}  // namespace qmm
