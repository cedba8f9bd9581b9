// qmm_moe.hip -- routed expert products in one grouped launch.
//
// A one-workgroup prologue groups the (token, slot) pairs by expert: it counts
// the pairs per expert, scans the counts into offsets, scatters the pair
// indices into expert order in the workspace and cuts every expert's pairs
// into work items of at most `mt` pairs.
//
// Kinds with a matrix-core GEMV decoder (and K a whole number of 256-element
// k-blocks) then run the matrix-core GEMV kernel in its routed form: one
// workgroup per (work item, 16-row tile), the item's pairs as the tokens, so
// each touched expert's weights stream from memory once per item (mt = 16,
// 8 or 1 pairs, by the number of pairs per expert).  Items of one pair need
// no grouping, so that case skips the prologue and reads ids directly.  The other cases run one wave per
// (expert, weight row), decoding the row to f32 and applying it to up to
// eight of the expert's pairs at a time.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

// Workspace layout (int32): counts[E], offsets[E + 1], order[P], nwork,
// work[2 * (P + min(E, P))] with P = M * topk pairs.  Every expert with c
// pairs gives ceil(c / mt) items, so there are at most P / mt + min(E, P).
struct MoeLayout {
  int64_t E, P;
  __host__ __device__ int64_t offsets() const { return E; }
  __host__ __device__ int64_t order() const { return 2 * E + 1; }
  __host__ __device__ int64_t nwork() const { return 2 * E + 1 + P; }
  __host__ __device__ int64_t work() const { return 2 * E + 2 + P; }
  int64_t max_items() const { return P + (E < P ? E : P); }
  int64_t words() const { return work() + 2 * max_items(); }
};

size_t moe_workspace_bytes(int64_t E, int64_t M, int64_t topk) {
  return (size_t)MoeLayout{E, M * topk}.words() * sizeof(int32_t);
}

// One workgroup of 1024 threads; E <= 4096 experts, so each thread owns at
// most four consecutive experts in the scans.
__global__ __launch_bounds__(1024) void moe_route_kernel(const int32_t *__restrict__ ids, int64_t pairs,
                                                         int E, int mt, int32_t *__restrict__ ws) {
  extern __shared__ int32_t lds[];  // counts[E], cursor[E], first item[E], then 2 x 1024 scan slots
  int32_t *cnt = lds, *cur = lds + E, *wof = lds + 2 * E;
  int32_t *scan_p = lds + 3 * E, *scan_i = scan_p + 1024;
  const MoeLayout L{E, pairs};
  int32_t *offsets = ws + L.offsets(), *order = ws + L.order(), *work = ws + L.work();
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  for (int64_t p = tid; p < pairs; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // Exclusive scans of the pair counts and of the item counts: each thread
  // sums its experts; an inclusive scan runs within each wave (lane
  // shuffles), the 16 wave totals are scanned by one wave, and each thread
  // then writes its experts' offsets.
  const int per = (E + 1023) / 1024, e0 = tid * per, e1 = min(E, e0 + per);
  int sp = 0, si = 0;
  for (int e = e0; e < e1; ++e) {
    sp += cnt[e];
    si += (cnt[e] + mt - 1) / mt;
  }
  const int lane = tid & 63, wv = tid >> 6;
  int ip = sp, ii = si;  // inclusive within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int ap = __shfl_up(ip, off, 64), ai = __shfl_up(ii, off, 64);
    if (lane >= off) {
      ip += ap;
      ii += ai;
    }
  }
  if (lane == 63) {
    scan_p[wv] = ip;
    scan_i[wv] = ii;
  }
  __syncthreads();
  if (wv == 0) {  // inclusive scan of the 16 wave totals
    int tp = lane < 16 ? scan_p[lane] : 0, ti = lane < 16 ? scan_i[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int ap = __shfl_up(tp, off, 64), ai = __shfl_up(ti, off, 64);
      if (lane >= off) {
        tp += ap;
        ti += ai;
      }
    }
    if (lane < 16) {
      scan_p[64 + lane] = tp;
      scan_i[64 + lane] = ti;
    }
  }
  __syncthreads();
  const int bp = wv > 0 ? scan_p[64 + wv - 1] : 0, bi = wv > 0 ? scan_i[64 + wv - 1] : 0;
  int run = bp + ip - sp, items = bi + ii - si;  // exclusive prefix of this thread's experts
  for (int e = e0; e < e1; ++e) {
    offsets[e] = run;
    cur[e] = run;
    wof[e] = items;
    ws[e] = cnt[e];
    run += cnt[e];
    items += (cnt[e] + mt - 1) / mt;
  }
  if (tid == 1023) {
    offsets[E] = bp + ip;
    ws[L.nwork()] = bi + ii;
  }
  __syncthreads();
  for (int64_t p = tid; p < pairs; p += blockDim.x) {
    const int e = ids[p];
    if (e >= 0 && e < E) order[atomicAdd(&cur[e], 1)] = (int32_t)p;
  }
  for (int e = tid; e < E; e += blockDim.x) {
    for (int c = 0; c < cnt[e]; c += mt) {
      const int item = wof[e] + c / mt;
      work[2 * item] = e;
      work[2 * item + 1] = offsets[e] + c;
    }
  }
}

template <int KIND, typename XT>
__global__ __launch_bounds__(256) void moe_rows_kernel(const uint8_t *__restrict__ W, int64_t row_bytes,
                                                       const int32_t *__restrict__ ws, int E, int topk,
                                                       const XT *__restrict__ X, int x_per_slot,
                                                       float *__restrict__ Y, int64_t N, int K) {
  const int e = blockIdx.y;
  const int32_t *offsets = ws + E, *order = ws + 2 * E + 1;  // MoeLayout
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

int moe_item_pairs(int kind, int64_t E, int64_t M, int64_t topk, int64_t K, bool packed) {
  const MoeLayout L{E, M * topk};
  // The matrix-core kernel addresses activations with 32-bit element offsets.
  const bool mfma = packed || (moe_mfma_supported(kind, K) && L.P * K < ((int64_t)1 << 31));
  // Pairs per work item: 16 (one full matrix-core tile of tokens) when a
  // uniform routing gives experts 16 pairs on average, 8 from 4 pairs on
  // average, else 1 (an 8-pair item that carries one or two pairs costs
  // more than streaming the expert once per pair).
  return !mfma ? 1 : (L.P >= 16 * E ? 16 : (L.P >= 4 * E ? 8 : 1));
}

hipError_t launch_moe(int kind, const uint8_t *W, int64_t E, const int32_t *ids, int64_t topk,
                      const void *X, int x_f16, int x_per_slot, float *Y, int64_t M, int64_t N,
                      int64_t K, void *ws, hipStream_t s, bool packed, bool routed) {
  int32_t *wsi = static_cast<int32_t *>(ws);
  const MoeLayout L{E, M * topk};
  const bool mfma = packed || (moe_mfma_supported(kind, K) && L.P * K < ((int64_t)1 << 31));
  const int mt = moe_item_pairs(kind, E, M, topk, K, packed);
  if (mfma && mt == 1) {
    // One pair per item needs no grouping: each workgroup reads its pair's
    // expert from ids and the routing prologue is skipped.
    const MoeRoute rt{wsi, 0, 0, 0, 0, (int)topk, x_per_slot, ids, (int)E, (int)L.P};
    return launch_moe_mfma(kind, W, X, x_f16, Y, 1, N, K, rt, (int)L.P, s, packed);
  }
  if (!routed) {
    hipLaunchKernelGGL(moe_route_kernel, dim3(1), dim3(1024), (size_t)(3 * E + 2048) * sizeof(int32_t), s, ids,
                       M * topk, (int)E, mt, wsi);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (mfma) {
    const MoeRoute rt{wsi, (int)L.offsets(), (int)L.order(), (int)L.nwork(), (int)L.work(), (int)topk, x_per_slot,
                      nullptr, (int)E, (int)L.P};
    const int64_t items = (L.P + mt - 1) / mt + (E < L.P ? E : L.P);
    return launch_moe_mfma(kind, W, X, x_f16, Y, mt, N, K, rt, (int)items, s, packed);
  }
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
