// qmm_gemv.hip -- decode GEMV, 1 <= M <= 8 tokens.
//
// One wave (64 lanes) owns one weight row.  Lane l walks the row's 16-element
// sub-blocks l, l+64, ...; it decodes each sub-block exactly to f32 in
// registers and multiplies it with the M activation rows, accumulating in
// f32.  A wave-wide reduction ends the row.  Every weight is exact, so with a
// unit-vector x the result is the decoded weight itself.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

template <typename XT> __device__ __forceinline__ float to_f32(XT v) { return (float)v; }

template <int KIND, typename XT>
__global__ __launch_bounds__(256) void gemv_rows_kernel(const uint8_t *__restrict__ W, int64_t row_bytes,
                                                        const XT *__restrict__ X, float *__restrict__ Y,
                                                        int M, int64_t N, int K) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= N) return;  // the whole wave leaves; no barrier follows
  const uint8_t *wr = W + row * row_bytes;
  float acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = 0.f;
  const int nsub = K / 16;
  for (int s = lane; s < nsub; s += 64) {
    float w[16];
    decode16<KIND>(wr + (int64_t)(s / kSubs<KIND>) * Geometry<KIND>::bytes, s % kSubs<KIND>, w);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      if (m < M) {
        const XT *xp = X + (int64_t)m * K + 16 * s;
        float a = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a += w[i] * to_f32(xp[i]);
        acc[m] += a;
      }
    }
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = wave_sum(acc[m]);
  if (lane == 0) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
      if (m < M) Y[(int64_t)m * N + row] = acc[m];
  }
}

template <int KIND>
static hipError_t run_gemv(const uint8_t *W, const void *x, int x_f16, float *y, int M, int64_t N,
                           int64_t K, hipStream_t s) {
  const int64_t row_bytes = (K / Geometry<KIND>::elems) * Geometry<KIND>::bytes;
  const dim3 grid((unsigned)((N + 3) / 4)), block(256);
  if (x_f16)
    hipLaunchKernelGGL((gemv_rows_kernel<KIND, _Float16>), grid, block, 0, s, W, row_bytes,
                       (const _Float16 *)x, y, M, N, (int)K);
  else
    hipLaunchKernelGGL((gemv_rows_kernel<KIND, float>), grid, block, 0, s, W, row_bytes,
                       (const float *)x, y, M, N, (int)K);
  return hipGetLastError();
}

hipError_t launch_gemv(int kind, const uint8_t *W, const void *x, int x_f16, float *y, int M,
                       int64_t N, int64_t K, hipStream_t s) {
  const hipError_t e = launch_gemv_mfma(kind, W, x, x_f16, y, M, N, K, s);
  if (e != hipErrorNotSupported) return e;
  switch (kind) {
#define QMM_CASE(K_) \
  case K_:           \
    return run_gemv<K_>(W, x, x_f16, y, M, N, K, s);
    QMM_FOR_EACH_KIND(QMM_CASE)
#undef QMM_CASE
  }
  return hipErrorInvalidValue;
}

}  // namespace qmm
