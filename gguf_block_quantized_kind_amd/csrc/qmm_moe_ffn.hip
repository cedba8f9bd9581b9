// qmm_moe_ffn.hip -- routed SiLU-gated expert FFN with a weighted top-k
// combine, composed from the routed expert products.
//
// For token t and slot s with e = ids[t][s] in [0, E):
//   gate, up = rows [0, N_ff) and [N_ff, 2 N_ff) of W_gu[e] times X[t]
//   h        = silu(gate) * up                       (f32)
//   d        = W_d[e] . h                            (the slot's down output)
//   Y[t]     = sum over valid slots, in slot order, of topk_w[t][s] * d
// Four stream-ordered launches: the routed gate/up product, the SiLU-product,
// the routed down product (per-slot activations) and the combine.  The two
// routed launches group pairs by expert, so each touched expert's weights
// stream once per work item.
//
// The routed product's matrix-core path takes its activations as f16, whose
// range ends at 65504, and h can exceed that (large gate and up outputs
// multiply).  Each pair's h is therefore divided by 2^k, the smallest power
// of two (k >= 0) that brings max |h| to 2^14 or below, and the combine
// multiplies that pair's down output by 2^k again: both steps are exact.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// Workspace: routing words, then G [P][2 N_ff], H [P][N_ff], D [P][K] f32
// and the per-pair scales S [P] f32, each section 256-byte aligned.
struct FfnLayout {
  int64_t route, g, h, d, sc, total;
  FfnLayout(int64_t E, int64_t M, int64_t topk, int64_t N_ff, int64_t K) {
    auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
    const int64_t P = M * topk;
    route = 0;
    g = up((int64_t)moe_workspace_bytes(E, M, topk));
    h = g + up(P * 2 * N_ff * 4);
    d = h + up(P * N_ff * 4);
    sc = d + up(P * K * 4);
    total = sc + up(P * 4);
  }
};

// One workgroup per pair: h = silu(g) * u for its N_ff elements, four per
// thread at a time; silu(v) = v / (1 + e^-v), which tends to v for large v
// and to -0 for very negative v (e^-v = inf).  Then the pair's scale.
__global__ __launch_bounds__(256) void silu_mul_kernel(const float *__restrict__ G, float *__restrict__ H,
                                                       float *__restrict__ S, int n_ff) {
  __shared__ float red[4];
  const int64_t p = blockIdx.x;
  const float *gp = G + p * 2 * n_ff;
  float *hp = H + p * n_ff;
  float amax = 0.f;
  for (int c = 4 * (int)threadIdx.x; c < n_ff; c += 4 * 256) {
    const floatx4 g = *reinterpret_cast<const floatx4 *>(gp + c);
    const floatx4 u = *reinterpret_cast<const floatx4 *>(gp + n_ff + c);
    floatx4 h;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[j] = g[j] / (1.0f + expf(-g[j])) * u[j];
      amax = fmaxf(amax, fabsf(h[j]));
    }
    *reinterpret_cast<floatx4 *>(hp + c) = h;
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // amax = f 2^x with f in [0.5, 1): amax <= 2^x, so k = x - 14 (if positive)
  // gives amax / 2^k <= 2^14.
  const int k = amax > 0.f ? max(0, __builtin_amdgcn_frexp_expf(amax) - 14) : 0;
  if (threadIdx.x == 0) S[p] = __builtin_amdgcn_ldexpf(1.0f, k);
  if (k == 0) return;  // the whole workgroup: k is uniform
  for (int c = 4 * (int)threadIdx.x; c < n_ff; c += 4 * 256) {
    floatx4 h = *reinterpret_cast<const floatx4 *>(hp + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) h[j] = __builtin_amdgcn_ldexpf(h[j], -k);
    *reinterpret_cast<floatx4 *>(hp + c) = h;
  }
}

// Y[t][k] = sum over valid slots s (in order) of w[t][s] * D[t][s][k].
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ D, const float *__restrict__ S,
                                                      const int32_t *__restrict__ ids,
                                                      const float *__restrict__ w, float *__restrict__ Y,
                                                      int64_t M, int topk, int K, int64_t E) {
  const int q = K / 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * q) return;
  const int64_t t = i / q;
  const int c = (int)(i % q) * 4;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < topk; ++s) {
    const int32_t e = ids[t * topk + s];
    if (e < 0 || e >= E) continue;
    const float ws = w[t * topk + s] * S[t * topk + s];  // S is a power of two: exact
    const floatx4 d = *reinterpret_cast<const floatx4 *>(D + (t * topk + s) * (int64_t)K + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = fmaf(ws, d[j], acc[j]);
  }
  *reinterpret_cast<floatx4 *>(Y + t * (int64_t)K + c) = acc;
}

}  // namespace

size_t moe_ffn_workspace_bytes(int64_t E, int64_t M, int64_t topk, int64_t N_ff, int64_t K) {
  return (size_t)FfnLayout(E, M, topk, N_ff, K).total;
}

hipError_t launch_moe_ffn(int kind, const uint8_t *W_gu, const uint8_t *W_d, int64_t E, const int32_t *ids,
                          const float *topk_w, int64_t topk, const void *X, int x_f16, float *Y, int64_t M,
                          int64_t N_ff, int64_t K, void *ws, hipStream_t s, bool packed) {
  const FfnLayout L(E, M, topk, N_ff, K);
  uint8_t *base = static_cast<uint8_t *>(ws);
  float *G = reinterpret_cast<float *>(base + L.g);
  float *H = reinterpret_cast<float *>(base + L.h);
  float *D = reinterpret_cast<float *>(base + L.d);
  float *S = reinterpret_cast<float *>(base + L.sc);
  const int64_t P = M * topk;
  hipError_t e = launch_moe(kind, W_gu, E, ids, topk, X, x_f16, 0, G, M, 2 * N_ff, K, base + L.route, s, packed);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)P), dim3(256), 0, s, G, H, S, (int)N_ff);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = launch_moe(kind, W_d, E, ids, topk, H, 0, 1, D, M, K, N_ff, base + L.route, s, packed);
  if (e != hipSuccess) return e;
  const int64_t n2 = M * (K / 4);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, s, D, S, ids, topk_w, Y, M,
                     (int)topk, (int)K, E);
  return hipGetLastError();
}

}  // namespace qmm
