// qmm_gemm.hip -- prefill GEMM on the matrix cores.
//
// C[M][N] = A[M][K] . W^T.  A workgroup owns a BM x BN tile of C and walks K
// in steps of 32.  Per step it stages the A tile in LDS as f16 and decodes the
// W tile (BN rows x 32 elements, 16 elements per thread with the shared
// decoders) into LDS, each weight rounded once from its exact f32 value to
// f16.  Waves then run v_mfma_f32_16x16x32_f16 with f32 accumulation.
//
// f32 activations are split into hi = RN_f16(a) and lo = RN_f16(a - hi) and
// both halves go through the matrix cores, so the activations keep about 22
// significant bits and only the weight operand is ever rounded.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 64;    // tokens per tile
constexpr int kBN = 128;   // weight rows per tile
constexpr int kBK = 32;    // elements of K per step
constexpr int kPad = 8;    // halves of padding per LDS row
constexpr int kLd = kBK + kPad;
static_assert(kBN * kBK == 256 * 16, "each thread decodes one 16-element sub-block");
static_assert(kBM * kBK == 256 * 8, "each thread stages 8 activations");

template <int KIND, typename AT>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t *__restrict__ W, int64_t row_bytes,
                                                   const AT *__restrict__ A, float *__restrict__ C,
                                                   int64_t M, int64_t N, int K) {
  constexpr bool kSplit = sizeof(AT) == 4;
  __shared__ __attribute__((aligned(16))) _Float16 a_hi[kBM][kLd];
  __shared__ __attribute__((aligned(16))) _Float16 a_lo[kSplit ? kBM : 1][kLd];
  __shared__ __attribute__((aligned(16))) _Float16 w_s[kBN][kLd];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;
  const int wm = wave >> 1, wn = wave & 1;  // wave tile: 32 tokens x 64 rows

  // This thread's decode slot: weight row n0 + (tid >> 1), k offset 16*(tid&1).
  int64_t wrow = n0 + (tid >> 1);
  if (wrow >= N) wrow = N - 1;  // read a real row; its outputs are not stored
  const uint8_t *wp = W + wrow * row_bytes;
  // This thread's staging slot: token m0 + (tid >> 2), k offset 8*(tid&3).
  const int64_t arow = m0 + (tid >> 2);
  const bool a_live = arow < M;
  const AT *ap = A + (a_live ? arow : 0) * (int64_t)K + 8 * (tid & 3);

  floatx4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();  // the previous step's fragments have been read
    {
      const int s = (k0 >> 4) + (tid & 1);
      float w[16];
      decode16<KIND>(wp + (int64_t)(s / kSubs<KIND>) * Geometry<KIND>::bytes, s % kSubs<KIND>, w);
      _Float16 *dst = &w_s[tid >> 1][16 * (tid & 1)];
#pragma unroll
      for (int i = 0; i < 16; ++i) dst[i] = (_Float16)w[i];
    }
    {
      _Float16 *dh = &a_hi[tid >> 2][8 * (tid & 3)];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float a = a_live ? (float)ap[k0 + i] : 0.f;
        const _Float16 h = (_Float16)a;
        dh[i] = h;
        if constexpr (kSplit) a_lo[tid >> 2][8 * (tid & 3) + i] = (_Float16)(a - (float)h);
      }
    }
    __syncthreads();
    const int r = lane & 15, kq = 8 * (lane >> 4);
    half8 bf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = *reinterpret_cast<const half8 *>(&w_s[64 * wn + 16 * j + r][kq]);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const half8 af = *reinterpret_cast<const half8 *>(&a_hi[32 * wm + 16 * i + r][kq]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, bf[j], acc[i][j], 0, 0, 0);
      if constexpr (kSplit) {
        const half8 al = *reinterpret_cast<const half8 *>(&a_lo[32 * wm + 16 * i + r][kq]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bf[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  // D[i][j] of a 16x16 tile sits in lane j + 16*(i/4), register i%4.
  const int col = lane & 15, rq = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + 64 * wn + 16 * j + col;
      if (n >= N) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t m = m0 + 32 * wm + 16 * i + rq + q;
        if (m < M) C[m * N + n] = acc[i][j][q];
      }
    }
}

template <int KIND>
static hipError_t run_gemm(const uint8_t *W, const void *A, int a_f16, float *C, int64_t M, int64_t N,
                           int64_t K, hipStream_t s) {
  const int64_t row_bytes = (K / Geometry<KIND>::elems) * Geometry<KIND>::bytes;
  const dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM)), block(256);
  if (a_f16)
    hipLaunchKernelGGL((gemm_kernel<KIND, _Float16>), grid, block, 0, s, W, row_bytes,
                       (const _Float16 *)A, C, M, N, (int)K);
  else
    hipLaunchKernelGGL((gemm_kernel<KIND, float>), grid, block, 0, s, W, row_bytes,
                       (const float *)A, C, M, N, (int)K);
  return hipGetLastError();
}

hipError_t launch_gemm(int kind, const uint8_t *W, const void *A, int a_f16, float *C, int64_t M,
                       int64_t N, int64_t K, hipStream_t s) {
  switch (kind) {
#define QMM_CASE(K_) \
  case K_:           \
    return run_gemm<K_>(W, A, a_f16, C, M, N, K, s);
    QMM_FOR_EACH_KIND(QMM_CASE)
#undef QMM_CASE
  }
  return hipErrorInvalidValue;
}

}  // namespace qmm
