// qmm_gemm_ks.hip -- prefill GEMM for the super-block kinds Q2_K, Q3_K,
// Q4_K, Q5_K and IQ4_XS: wave-private tiles and a K split across the waves
// of a workgroup.
//
// C[M][N] = A[M][K] . W^T.  A workgroup of four waves owns a 64 x 64 tile of
// C (64 tokens by 64 weight rows; 32 tokens for f32 activations).  Every
// wave computes the whole tile over its own quarter of K, so the waves share
// nothing until the end.  Per step of 64 elements of K a wave
//   1. writes into its private LDS area the activation rows and the weight
//      runs the step needs (loaded into registers during the previous step;
//      16-byte pieces, contiguous lanes on consecutive bytes of a row),
//   2. issues the global loads of the next step,
//   3. reads its activation fragments and each lane's weight fields back
//      from LDS, decodes the weights in registers (qmm_gemm_ks.h) and feeds
//      v_mfma_f32_16x16x32_f16.
// The LDS area is the wave's own and LDS operations of one wave complete in
// order, so no barrier is needed.  Two workgroups share a compute unit (two
// waves per SIMD), one hiding the other's waits.  At the end the four
// partial tiles are summed through LDS in a fixed order (deterministic) and
// stored.  Rows past M or N are clamped to the last row when loading (never
// stored), so every address is inside the operands.
//
// Workgroups are numbered so that the token tiles of one weight tile run on
// one XCD (workgroup i runs on XCD i mod 8) and read that weight tile through
// one L2.
//
// Numerics: each weight is rounded once to f16 (qmm_gemm_ks.h); f16
// activations are exact; f32 activations are split into hi = RN_f16(a) and
// lo = RN_f16(a - hi) and both halves are multiplied; accumulation is f32.
#include <stdlib.h>

#include <type_traits>

#include "qmm_gemm_ks.h"
#include "qmm_internal.h"

// The kinds this GEMM serves: the super-block kinds whose decode it does
// with matrix-core-ready f16 pieces (measured faster than the LDS-tiled GEMM
// of qmm_gemm.hip for these kinds; Q6_K and the 32-element kinds are
// faster there).
#define QMM_KS_KINDS(X) X(Q2_K) X(Q3_K) X(Q4_K) X(Q5_K) X(IQ4_XS)

namespace qmm {
namespace gk {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kWgPerCu = 2;  // two workgroups per compute unit: two waves per SIMD
constexpr int kStep = 64;  // elements of K per step
constexpr int kRedChunk = 32;  // accumulator values per lane per reduction round

__device__ __forceinline__ half8 as_h8(u32x4 v) { return __builtin_bit_cast(half8, v); }

typedef float f32x4 __attribute__((ext_vector_type(4)));

// hi = RN_f16(a), lo = RN_f16(a - hi) of eight f32 values.  (The whole
// vectors are bit-cast: a bit cast of one vector element compiled to a read
// of element 0.)
__device__ __forceinline__ void split8(const u32x4 (&f)[2], half8 &hi, half8 &lo) {
  const f32x4 a0 = __builtin_bit_cast(f32x4, f[0]), a1 = __builtin_bit_cast(f32x4, f[1]);
  const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const _Float16 h = (_Float16)a[e];
    hi[e] = h;
    lo[e] = (_Float16)(a[e] - (float)h);
  }
}

// A wave's LDS area for one step:
//   activations: the wave's 16 TM rows of the step, row r at r * RB, its
//     16-byte chunks XOR-permuted by r so that the sixteen rows one fragment
//     read touches fall in different banks;
//   weights: each of the 16 TN rows' runs (qmm_gemm_ks.h) at the same byte
//     offsets as in the row, 16 * NCT bytes per row.
template <typename AT, int TM>
struct AStage {
  static constexpr int RB = kStep * (int)sizeof(AT);  // bytes per row per step
  static constexpr int CPR = RB / 16;                  // 16-byte chunks per row
  static constexpr int ROWS = 16 * TM;
  static constexpr int BYTES = ROWS * RB;
  static constexpr int NLD = BYTES / 1024;            // 16-byte loads per lane per step
};

// 16-byte pieces of run k of a kind (at most kRunMax[k] bytes), and the
// first piece slot of run k in a row's image (row_chunks(kRuns) in all).
__host__ __device__ constexpr int run_chunks(int len) { return (len + 15) / 16; }
template <int KIND>
__host__ __device__ constexpr int row_chunks(int upto) {
  int c = 0;
  for (int k = 0; k < upto; ++k) c += run_chunks(Frag<KIND>::kRunMax[k]);
  return c;
}
template <int KIND, typename AT, int TM, int TN>
struct Stage {
  static constexpr int NCT = row_chunks<KIND>(Frag<KIND>::kRuns);  // chunk slots per weight row
  static constexpr int W_LD = (16 * TN * NCT + 63) / 64;  // 16-byte loads per lane; the last may repeat rows
  static constexpr int W_BYTES = 1024 * W_LD;
  static constexpr int BYTES = AStage<AT, TM>::BYTES + W_BYTES;
};

// A lane's view of one weight row's image in a stage: run k's bytes start
// at img + 16 * (first slot of run k).
template <int KIND>
struct WRow {
  const uint8_t *img;
  template <int k, typename T> __device__ __forceinline__ T get(int off) const {
    T v;
    __builtin_memcpy(&v, img + 16 * row_chunks<KIND>(k) + off, sizeof(T));
    return v;
  }
};

template <int KIND, typename AT, int TM, int TN>
__global__ __launch_bounds__(64 * kWaves, kWgPerCu) void gemm_ks_kernel(const uint8_t *__restrict__ W, uint32_t row_bytes,
                                                                  const AT *__restrict__ A, float *__restrict__ C,
                                                                  int M, int N, int K, int tiles_m) {
  using F = Frag<KIND>;
  using AS = AStage<AT, TM>;
  using ST = Stage<KIND, AT, TM, TN>;
  constexpr bool kF32 = sizeof(AT) == 4;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  // The wave number is uniform across the wave; saying so keeps the step
  // loop scalar.
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = lane >> 4, l16 = lane & 15;

  // Tile of this workgroup: XCD x = i mod 8 receives a contiguous range of
  // tile numbers, token tiles fastest.
  const int T = gridDim.x, L = blockIdx.x;
  const int xcd = L & 7, jx = L >> 3, q8 = T >> 3, r8 = T & 7;
  const int V = xcd < r8 ? xcd * (q8 + 1) + jx : r8 * (q8 + 1) + (xcd - r8) * q8 + jx;
  const int m0 = (V % tiles_m) * 16 * TM, n0 = (V / tiles_m) * 16 * TN;

  // This wave's steps (K is a whole number of 256-element super-blocks).
  const int S = K / kStep;
  const int s_begin = (S * wave) / kWaves, s_end = (S * (wave + 1)) / kWaves;
  const int nst = s_end - s_begin;

  // Activation loads: load d of a step fills LDS chunk d * 64 + lane,
  // which holds row r = (d * 64 + lane) / CPR, logical chunk
  // (physical chunk) ^ (r mod CPR); its source offset (bytes) without k.
  uint32_t aoff[AS::NLD];
#pragma unroll
  for (int d = 0; d < AS::NLD; ++d) {
    const int pos = d * 64 + lane, r = pos / AS::CPR, c = (pos % AS::CPR) ^ (r % AS::CPR);
    aoff[d] = ((uint32_t)min(m0 + r, M - 1) * (uint32_t)K) * (uint32_t)sizeof(AT) + 16u * (uint32_t)c;
  }
  uint8_t *const my_lds = lds + wave * ST::BYTES;
  // Fragment reads: lane (row l16 of tile i, group G) takes the 16 bytes of
  // logical chunk koff / (16 / sizeof(AT)) (and the next, for f32).
  constexpr int kEPC = 16 / (int)sizeof(AT);  // elements per chunk
  int frd[2][kF32 ? 2 : 1];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int h = 0; h < (kF32 ? 2 : 1); ++h) {
      const int c = koff<F::kPat>(G, s) / kEPC + h;
      frd[s][h] = l16 * AS::RB + 16 * (c ^ (l16 % AS::CPR));
    }

  // Weight piece slots: load d's lane takes slot w = 64 d + lane of the
  // stage's image, row w / NCT, slot w % NCT (piece cc of run k).  Per
  // load: the row's byte offset, its image offset, and (k, cc).
  constexpr int NCT = ST::NCT;
  uint32_t wrow[ST::W_LD];
  int wimg[ST::W_LD], wkc[ST::W_LD];
#pragma unroll
  for (int d = 0; d < ST::W_LD; ++d) {
    const int w = 64 * d + lane, r = min(w / NCT, 16 * TN - 1), c = w % NCT;
    wrow[d] = (uint32_t)min(n0 + r, N - 1) * row_bytes;
    int k = 0, first = 0;
#pragma unroll
    for (int kk = 0; kk < F::kRuns; ++kk)
      if (c >= row_chunks<KIND>(kk)) { k = kk; first = row_chunks<KIND>(kk); }
    wkc[d] = (k << 8) | (c - first);
    wimg[d] = AS::BYTES + 16 * (NCT * r + first);
  }

  // Global loads of step st into registers: activation chunks, then the
  // weight runs' pieces (piece cc of run k at run offset min(16 cc, len - 16)).
  u32x4 areg[AS::NLD], wreg[ST::W_LD];
  int wpos[ST::W_LD];  // LDS offset each weight piece goes to
  auto load_step = [&](int st) {
    const uint8_t *abase = reinterpret_cast<const uint8_t *>(A) + (uint32_t)(st * kStep) * (uint32_t)sizeof(AT);
#pragma unroll
    for (int d = 0; d < AS::NLD; ++d) {
      areg[d] = *reinterpret_cast<const u32x4 *>(abase + aoff[d]);
    }
#pragma unroll
    for (int d = 0; d < ST::W_LD; ++d) {
      const int k = F::kRuns == 1 ? 0 : (wkc[d] >> 8), cc = wkc[d] & 255;
      const int len = F::run_len(k, st);
      const int co = min(16 * cc, len - 16);
      wpos[d] = wimg[d] + co;
      wreg[d] = ld16(W + (wrow[d] + (uint32_t)(F::run_start(k, st) + co)));
    }
  };
  // The loaded chunks into the wave's LDS stage: lane l of load d to slot
  // 64 d + l.
  auto store_step = [&]() {
#pragma unroll
    for (int d = 0; d < AS::NLD; ++d) *reinterpret_cast<u32x4 *>(my_lds + d * 1024 + lane * 16) = areg[d];
#pragma unroll
    for (int d = 0; d < ST::W_LD; ++d) __builtin_memcpy(my_lds + wpos[d], &wreg[d], 16);
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // One step: the chunks loaded one step earlier go to LDS, the next step's
  // loads are issued, and the products run out of LDS.
  auto step = [&](auto more_tag, int st) {
    constexpr bool kMore = decltype(more_tag)::value;
    store_step();
    if constexpr (kMore) load_step(st + 1);
    // The next step's loads stay ahead of this step's products.
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t *src = my_lds;
    // All LDS reads first (activation fragments, every tile's weight
    // fields), then per tile: decode, and its products, with the decode of
    // the next tile interleaved with them (scheduling groups below).
    typename F::Raw r[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      WRow<KIND> rd;
      rd.img = src + AS::BYTES + 16 * NCT * (16 * j + l16);
      F::gather(rd, st, G, r[j]);
    }
    half8 ahi[2][TM], alo[2][TM];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const uint8_t *row = src + 16 * i * AS::RB;
        if constexpr (kF32) {
          const u32x4 f[2] = {*reinterpret_cast<const u32x4 *>(row + frd[s][0]),
                        *reinterpret_cast<const u32x4 *>(row + frd[s][1])};
          split8(f, ahi[s][i], alo[s][i]);
        } else {
          const u32x4 a = *reinterpret_cast<const u32x4 *>(row + frd[s][0]);
          ahi[s][i] = as_h8(a);
        }
      }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      u32x4 b0, b1;
      F::decode(r[j], st, G, b0, b1);
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const half8 bb = as_h8(s ? b1 : b0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[s][i], bb, acc[i][j], 0, 0, 0);
          if constexpr (kF32) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[s][i], bb, acc[i][j], 0, 0, 0);
        }
    }
#ifndef QMM_GEMM_NO_SCHED
    // One matrix-core instruction, then a few vector-ALU instructions (the
    // decode of the following tile), so the SIMD issues the decode while the
    // matrix core works.
    constexpr int kM = TM * TN * 2 * (kF32 ? 2 : 1);
#pragma unroll
    for (int q = 0; q < kM; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }
#endif
  };

  if (nst > 0) {
    load_step(s_begin);
    for (int st = s_begin; st < s_end - 1; ++st) step(std::true_type{}, st);
    step(std::false_type{}, s_end - 1);
  }
  __syncthreads();

  // Sum the four waves' partial tiles through LDS, kRedChunk accumulator
  // values per lane at a time: wave w writes red[w][v][lane]; then thread
  // (wave, lane) adds the four partials of value v = c0 + wave + 4 r for its
  // own lane position and stores it.
  float *red = reinterpret_cast<float *>(lds);
  constexpr int NV = TM * TN * 4;
  const int col = l16, rq = 4 * G;
#pragma unroll
  for (int c0 = 0; c0 < NV; c0 += kRedChunk) {
    if (c0) __syncthreads();
#pragma unroll
    for (int v = c0; v < c0 + kRedChunk && v < NV; ++v)
      red[(wave * kRedChunk + (v - c0)) * 64 + lane] = acc[(v >> 2) / TN][(v >> 2) % TN][v & 3];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRedChunk / kWaves; ++r) {
      const int vl = wave + kWaves * r, v = c0 + vl;
      if (v < NV) {
        const float s = ((red[(0 * kRedChunk + vl) * 64 + lane] + red[(1 * kRedChunk + vl) * 64 + lane]) +
                         red[(2 * kRedChunk + vl) * 64 + lane]) +
                        red[(3 * kRedChunk + vl) * 64 + lane];
        const int i = (v >> 2) / TN, j = (v >> 2) % TN;
        const int m = m0 + 16 * i + rq + (v & 3), n = n0 + 16 * j + col;
        if (m < M && n < N) C[(int64_t)m * N + n] = s;
      }
    }
  }
}

constexpr size_t kRedLds = (size_t)kWaves * kRedChunk * 64 * sizeof(float);

template <int KIND, typename AT, int TM, int TN>
static hipError_t run_as(const uint8_t *W, const void *A, float *C, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  constexpr size_t ring = (size_t)kWaves * Stage<KIND, AT, TM, TN>::BYTES;
  constexpr size_t lds = ring > kRedLds ? ring : kRedLds;
  if constexpr (lds > 160 * 1024 / kWgPerCu) {
    return hipErrorInvalidConfiguration;  // a shape that does not fit is never launched
  } else {
    const int64_t row_bytes = (K / Geometry<KIND>::elems) * Geometry<KIND>::bytes;
    const int64_t tm = (M + 16 * TM - 1) / (16 * TM), tn = (N + 16 * TN - 1) / (16 * TN);
    hipLaunchKernelGGL((gemm_ks_kernel<KIND, AT, TM, TN>), dim3((unsigned)(tm * tn)), dim3(64 * kWaves), lds, s, W,
                       (uint32_t)row_bytes, (const AT *)A, C, (int)M, (int)N, (int)K, (int)tm);
    return hipGetLastError();
  }
}

// f32 activations take tiles of half as many tokens: a step of 64 f32 per
// row is twice the LDS of f16.
template <int KIND, int TM, int TN>
static hipError_t run(const uint8_t *W, const void *A, int a_f16, float *C, int64_t M, int64_t N, int64_t K,
                      hipStream_t s) {
  return a_f16 ? run_as<KIND, _Float16, TM, TN>(W, A, C, M, N, K, s)
               : run_as<KIND, float, TM / 2, TN>(W, A, C, M, N, K, s);
}

// Tile shape: 64 tokens x 128 rows (x 64 rows for the kinds with more
// chunk slots per row); for the 32-element nibble kinds 64 x 176 when 128-row tiles
// would leave the last round of workgroups on the 256 compute units mostly
// empty and 176-row tiles fit in one round.
template <int KIND>
static hipError_t run_m(const uint8_t *W, const void *A, int a_f16, float *C, int64_t M, int64_t N, int64_t K,
                        hipStream_t s, int cfg) {
  // Kinds whose step needs more chunk slots per row take 64-row tiles so
  // that two stages of four waves fit the 160 KiB of LDS.
  constexpr int TN = 4;
#ifdef QMM_TUNING
  switch (cfg) {
    case 1: return run<KIND, 4, TN>(W, A, a_f16, C, M, N, K, s);
    case 2: return run<KIND, 4, 4>(W, A, a_f16, C, M, N, K, s);
    case 3: return run<KIND, 8, 4>(W, A, a_f16, C, M, N, K, s);
    case 4: return run<KIND, 2, TN>(W, A, a_f16, C, M, N, K, s);
    default: break;
  }
#else
  (void)cfg;
#endif
  return run<KIND, 4, TN>(W, A, a_f16, C, M, N, K, s);
}

}  // namespace gk

bool gemm_ks_supported(int kind, int64_t M, int64_t N, int64_t K, int a_f16) {
  int64_t row_bytes = -1;
  switch (kind) {
#define QMM_CASE(K_) \
  case K_:           \
    row_bytes = K / Geometry<K_>::elems * Geometry<K_>::bytes; \
    break;
    QMM_KS_KINDS(QMM_CASE)
#undef QMM_CASE
  }
  // 32-bit element and byte offsets.
  return row_bytes > 0 && M * K * (a_f16 ? 2 : 4) < ((int64_t)1 << 31) && N * row_bytes < ((int64_t)1 << 31) &&
         (M + 31) / 32 * ((N + 63) / 64) < ((int64_t)1 << 31);
}

hipError_t launch_gemm_ks(int kind, const uint8_t *W, const void *A, int a_f16, float *C, int64_t M, int64_t N,
                          int64_t K, hipStream_t s) {
#ifdef QMM_TUNING
  static const int cfg = [] {
    const char *e = getenv("QMM_GEMM_KS_CFG");
    return e ? atoi(e) : 0;
  }();
#else
  constexpr int cfg = 0;
#endif
  switch (kind) {
#define QMM_CASE(K_) \
  case K_:           \
    return gk::run_m<K_>(W, A, a_f16, C, M, N, K, s, cfg);
    QMM_KS_KINDS(QMM_CASE)
#undef QMM_CASE
  }
  return hipErrorInvalidValue;
}

}  // namespace qmm
