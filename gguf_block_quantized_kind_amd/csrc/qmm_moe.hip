// qmm_moe.hip -- routed expert products in one grouped launch.
//
// A one-workgroup prologue groups the (token, slot) pairs by expert: it counts
// the pairs per expert, scans the counts into offsets and scatters the pair
// indices into expert order in the workspace.  The grouped kernel then runs
// one wave per (expert, weight row): the wave decodes the row exactly, as the
// decode GEMV does, and multiplies it with the activations of up to eight of
// the expert's pairs at a time, so each touched expert's weights are streamed
// from memory once per eight pairs and untouched experts cost one early exit.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

// Workspace layout (int32): counts[E], offsets[E + 1], order[M * topk].
size_t moe_workspace_bytes(int64_t E, int64_t M, int64_t topk) {
  return (size_t)(E + (E + 1) + M * topk) * sizeof(int32_t);
}

__global__ __launch_bounds__(1024) void moe_route_kernel(const int32_t *__restrict__ ids, int64_t pairs,
                                                         int E, int32_t *__restrict__ ws) {
  extern __shared__ int32_t lds[];  // counts[E] then cursor[E]
  int32_t *cnt = lds, *cur = lds + E;
  int32_t *offsets = ws + E, *order = ws + 2 * E + 1;
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int64_t p = threadIdx.x; p < pairs; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      offsets[e] = run;
      cur[e] = run;
      ws[e] = cnt[e];
      run += cnt[e];
    }
    offsets[E] = run;
  }
  __syncthreads();
  for (int64_t p = threadIdx.x; p < pairs; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E) order[atomicAdd(&cur[e], 1)] = (int32_t)p;
  }
}

template <int KIND, typename XT>
__global__ __launch_bounds__(256) void moe_rows_kernel(const uint8_t *__restrict__ W, int64_t row_bytes,
                                                       const int32_t *__restrict__ ws, int E, int topk,
                                                       const XT *__restrict__ X, int x_per_slot,
                                                       float *__restrict__ Y, int64_t N, int K) {
  const int e = blockIdx.y;
  const int32_t *offsets = ws + E, *order = ws + 2 * E + 1;
  const int begin = offsets[e], end = offsets[e + 1];
  if (begin == end) return;  // expert not routed to: the whole block leaves
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= N) return;
  const uint8_t *wr = W + ((int64_t)e * N + row) * row_bytes;
  const int nsub = K / 16;
  for (int c0 = begin; c0 < end; c0 += 8) {
    const int cn = min(8, end - c0);
    const XT *xs[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t p = order[c0 + (j < cn ? j : 0)];
      xs[j] = X + (x_per_slot ? p : p / topk) * (int64_t)K;
    }
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = 0.f;
    for (int s = lane; s < nsub; s += 64) {
      float w[16];
      decode16<KIND>(wr + (int64_t)(s / kSubs<KIND>) * Geometry<KIND>::bytes, s % kSubs<KIND>, w);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < cn) {
          const XT *xp = xs[j] + 16 * s;
          float a = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) a += w[i] * (float)xp[i];
          acc[j] += a;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = wave_sum(acc[j]);
    if (lane == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < cn) Y[(int64_t)order[c0 + j] * N + row] = acc[j];
    }
  }
}

template <int KIND>
static hipError_t run_moe(const uint8_t *W, int64_t E, int64_t topk, const void *X, int x_f16,
                          int x_per_slot, float *Y, int64_t N, int64_t K, const int32_t *ws,
                          hipStream_t s) {
  const int64_t row_bytes = (K / Geometry<KIND>::elems) * Geometry<KIND>::bytes;
  const dim3 grid((unsigned)((N + 3) / 4), (unsigned)E), block(256);
  if (x_f16)
    hipLaunchKernelGGL((moe_rows_kernel<KIND, _Float16>), grid, block, 0, s, W, row_bytes, ws, (int)E,
                       (int)topk, (const _Float16 *)X, x_per_slot, Y, N, (int)K);
  else
    hipLaunchKernelGGL((moe_rows_kernel<KIND, float>), grid, block, 0, s, W, row_bytes, ws, (int)E,
                       (int)topk, (const float *)X, x_per_slot, Y, N, (int)K);
  return hipGetLastError();
}

hipError_t launch_moe(int kind, const uint8_t *W, int64_t E, const int32_t *ids, int64_t topk,
                      const void *X, int x_f16, int x_per_slot, float *Y, int64_t M, int64_t N,
                      int64_t K, void *ws, hipStream_t s) {
  int32_t *wsi = static_cast<int32_t *>(ws);
  hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(1024), (size_t)(2 * E) * sizeof(int32_t), s, ids,
                     M * topk, (int)E, wsi);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  switch (kind) {
#define QMM_CASE(K_) \
  case K_:           \
    return run_moe<K_>(W, E, topk, X, x_f16, x_per_slot, Y, N, K, wsi, s);
    QMM_FOR_EACH_KIND(QMM_CASE)
#undef QMM_CASE
  }
  return hipErrorInvalidValue;
}

}  // namespace qmm
