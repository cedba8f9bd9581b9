// qmm_gemm.hip -- prefill GEMM on the matrix cores.
//
// C[M][N] = A[M][K] . W^T.  A workgroup owns a BM x BN tile of C (BM tokens,
// BN weight rows) and walks K in stages of BK elements through two LDS
// buffers.  While the waves multiply stage s out of one buffer, the global
// loads of stage s+1 (activation tile and raw weight blocks) are already in
// flight; after the multiplies each thread decodes its share of the weight
// tile to f16 (qmm_gemm_dec.h) and writes it, with the activation tile, into
// the other buffer.  One barrier per stage.
//
// Waves are arranged WM x WN over the tile; each runs
// v_mfma_f32_16x16x32_f16 over a (BM/WM) x (BN/WN) sub-tile with f32
// accumulation.  A operand = activations (16 tokens x 32 k), B operand =
// decoded weights (32 k x 16 weight rows); both fragments are 16-byte LDS
// reads of 8 consecutive k of one row.  Rows are not padded; instead the
// 16-byte chunks of row r are XOR-permuted by r, so the 16 rows one fragment
// read touches fall in 16 different chunk columns (distinct banks), and so
// do the chunks one row's writer threads store.
//
// Numerics: each weight is rounded once to f16 (relative error <= 2^-11).
// f32 activations are split into hi = RN_f16(a) and lo = RN_f16(a - hi) and
// both halves go through the matrix cores, so the activations keep about 22
// significant bits.  Decoded weights beyond the f16 range (|w| > 65504)
// become infinities; generated and real checkpoints stay far inside it.
#include <stdlib.h>

#include "qmm_gemm_dec.h"
#include "qmm_internal.h"

namespace qmm {
namespace gm {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

template <int BM, int BN, int BK, bool SPLIT>
struct Tile {
  static constexpr int LD = BK;                     // halves per LDS row
  // 16-byte chunk c of row r is stored at chunk c ^ (r & SW): the 16 rows a
  // fragment read touches then hit 16 different chunk columns.
  static constexpr int SW = (BK / 8 < 16 ? BK / 8 : 16) - 1;
  static constexpr int A_HALVES = BM * LD;
  static constexpr int W_HALVES = BN * LD;
  static constexpr int STAGE = A_HALVES * (SPLIT ? 2 : 1) + W_HALVES;
  static constexpr size_t LDS_BYTES = 2 * (size_t)STAGE * sizeof(_Float16);
};

template <int KIND, typename AT, int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(const uint8_t *__restrict__ W, int64_t row_bytes,
                                                            const AT *__restrict__ A, float *__restrict__ C,
                                                            int M, int N, int K) {
  constexpr int T = 64 * WM * WN;
  constexpr bool kSplit = sizeof(AT) == 4;
  using Tl = Tile<BM, BN, BK, kSplit>;
  constexpr int LD = Tl::LD;
  constexpr int TM = BM / WM / 16, TN = BN / WN / 16;
  constexpr int KC = BK / 32;                        // 32-element chunks per row per stage
  constexpr int NCH = BN * KC, CW = (NCH + T - 1) / T;
  constexpr int KP = BK / 8;                         // 8-element activation pieces per row
  constexpr int NP = BM * KP, CA = (NP + T - 1) / T;
  static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0 && BK % 32 == 0, "tile shape");
  using Dec = Chunk<KIND>;
  typedef typename std::conditional<kSplit, u32x4[2], u32x4>::type APiece;

  extern __shared__ __attribute__((aligned(16))) _Float16 smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;


  // Loads are unconditional (indices clamped to real data) so that no branch
  // separates them from the code that consumes them a stage later; pieces
  // outside the matrix are replaced by zeros when they are written to LDS.
  // When a stage has fewer pieces than threads, several threads load and
  // write the same piece (identical values to the same LDS address).
  auto load_stage = [&](int k0, typename Dec::Raw(&wraw)[CW], APiece(&araw)[CA]) {
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int c = (tid + i * T) % NCH;
      const int kk = min(k0 + 32 * (c % KC), K - 32);
      const int64_t row = min(n0 + c / KC, N - 1);  // rows past N: outputs not stored
      Dec::load(W + row * row_bytes, kk, wraw[i]);
    }
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int p = (tid + i * T) % NP;
      const int m = min(m0 + p / KP, M - 1), kk = min(k0 + 8 * (p % KP), K - 8);
      const AT *src = A + (int64_t)m * K + kk;
      if constexpr (kSplit) {
        araw[i][0] = *reinterpret_cast<const u32x4 *>(src);
        araw[i][1] = *reinterpret_cast<const u32x4 *>(src + 4);
      } else {
        araw[i] = *reinterpret_cast<const u32x4 *>(src);
      }
    }
  };

  auto store_stage = [&](int k0, int buf, const typename Dec::Raw(&wraw)[CW], const APiece(&araw)[CA]) {
    _Float16 *as = smem + buf * Tl::STAGE;
    _Float16 *ws = as + Tl::A_HALVES * (kSplit ? 2 : 1);
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int c = (tid + i * T) % NCH;
      // A bit mask, not a branch: a branch here would pull the loads into it.
      const uint32_t keep = 0u - (uint32_t)(k0 + 32 * (c % KC) < K);
      uint32_t o[16];
      Dec::decode(wraw[i], o);
      const int r = c / KC;
      u32x4 *dst = reinterpret_cast<u32x4 *>(ws + r * LD);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        dst[(4 * (c % KC) + q) ^ (r & Tl::SW)] =
            u32x4{o[4 * q] & keep, o[4 * q + 1] & keep, o[4 * q + 2] & keep, o[4 * q + 3] & keep};
    }
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int p = (tid + i * T) % NP;
      {
        const bool live = m0 + p / KP < M && k0 + 8 * (p % KP) < K;
        const int off = (p / KP) * LD + 8 * ((p % KP) ^ ((p / KP) & Tl::SW));
        if constexpr (kSplit) {
          const float *f = reinterpret_cast<const float *>(&araw[i][0]);
          uint32_t hi[4], lo[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float a0 = live ? f[2 * e] : 0.f, a1 = live ? f[2 * e + 1] : 0.f;
            const _Float16 h0 = (_Float16)a0, h1 = (_Float16)a1;
            hi[e] = bits(half2v{h0, h1});
            lo[e] = bits(half2v{(_Float16)(a0 - (float)h0), (_Float16)(a1 - (float)h1)});
          }
          *reinterpret_cast<u32x4 *>(as + off) = u32x4{hi[0], hi[1], hi[2], hi[3]};
          *reinterpret_cast<u32x4 *>(as + Tl::A_HALVES + off) = u32x4{lo[0], lo[1], lo[2], lo[3]};
        } else {
          const uint32_t keep = 0u - (uint32_t)live;
          *reinterpret_cast<u32x4 *>(as + off) = araw[i] & keep;
        }
      }
    }
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Fragment reads: lane l takes row l % 16 of a 16-row tile, chunk
  // 4 ks + l / 16 of the stage (8 consecutive k), swizzled.
  const int fr = lane & 15, fsw = fr & Tl::SW;
  int fc[BK / 32];
#pragma unroll
  for (int ks = 0; ks < BK / 32; ++ks) fc[ks] = 4 * ks + (lane >> 4);
  auto compute = [&](int buf) {
    const _Float16 *as = smem + buf * Tl::STAGE;
    const _Float16 *ws = as + Tl::A_HALVES * (kSplit ? 2 : 1);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      half8 af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const half8 *>(as + (wm * TM * 16 + 16 * i + fr) * LD + 8 * (fc[ks] ^ fsw));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[j] = *reinterpret_cast<const half8 *>(ws + (wn * TN * 16 + 16 * j + fr) * LD + 8 * (fc[ks] ^ fsw));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
      if constexpr (kSplit) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
          af[i] = *reinterpret_cast<const half8 *>(as + Tl::A_HALVES + (wm * TM * 16 + 16 * i + fr) * LD +
                                                   8 * (fc[ks] ^ fsw));
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  // Pipeline: while stage s is multiplied out of one LDS buffer, stage s+1
  // (loaded one step earlier, now in registers) is decoded into the other
  // buffer and stage s+2 is loaded -- every load has a whole stage of
  // multiplies to arrive.  The body runs two stages so that the two register
  // sets alternate statically; it is straight-line (stages past the end are
  // clamped re-reads stored as zero tiles), which keeps the compiler from
  // sinking loads next to their use.
  typename Dec::Raw wx[CW], wy[CW];
  APiece ax[CA], ay[CA];
  load_stage(0, wx, ax);
  store_stage(0, 0, wx, ax);
  load_stage(BK, wx, ax);
  __syncthreads();
  const int stages = (K + BK - 1) / BK;
  // Schedule of one stage: the loads go first; then each matrix-core
  // instruction is followed by a few vector-ALU instructions of the decode,
  // which the SIMD issues while the matrix core works.
  constexpr int NM = (BK / 32) * TM * TN * (kSplit ? 2 : 1);
  auto shape = [&]() {
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // four VALU
    }
  };
  for (int st = 0; st < stages; st += 2) {
    load_stage((st + 2) * BK, wy, ay);
    __builtin_amdgcn_sched_barrier(0);
    compute(0);
    store_stage((st + 1) * BK, 1, wx, ax);
    shape();
    __syncthreads();
    load_stage((st + 3) * BK, wx, ax);
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
    store_stage((st + 2) * BK, 0, wy, ay);
    shape();
    __syncthreads();
  }

  // D[i][j] of a 16x16 tile sits in lane j + 16*(i/4), register i%4.
  const int rq = 4 * (lane >> 4);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int n = n0 + wn * TN * 16 + 16 * j + fr;
      if (n >= N) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = m0 + wm * TM * 16 + 16 * i + rq + q;
        if (m < M) C[(int64_t)m * N + n] = acc[i][j][q];
      }
    }
}

// A workgroup's LDS on gfx950 holds at most 160 KiB.
constexpr size_t kMaxLds = 160 * 1024;

template <int KIND, typename AT, int BM, int BN, int BK, int WM, int WN>
static hipError_t run_as(const uint8_t *W, const void *A, float *C, int64_t M, int64_t N, int64_t K,
                         hipStream_t s) {
  constexpr size_t lds = Tile<BM, BN, BK, sizeof(AT) == 4>::LDS_BYTES;
  if constexpr (lds > kMaxLds) {
    return hipErrorInvalidConfiguration;  // a shape that does not fit is never launched
  } else {
    const int64_t row_bytes = (K / Geometry<KIND>::elems) * Geometry<KIND>::bytes;
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM)), block(64 * WM * WN);
    hipLaunchKernelGGL((gemm_kernel<KIND, AT, BM, BN, BK, WM, WN>), grid, block, lds, s, W, row_bytes,
                       (const AT *)A, C, (int)M, (int)N, (int)K);
    return hipGetLastError();
  }
}

template <int KIND, int BM, int BN, int BK, int WM, int WN>
static hipError_t run(const uint8_t *W, const void *A, int a_f16, float *C, int64_t M, int64_t N, int64_t K,
                      hipStream_t s) {
  return a_f16 ? run_as<KIND, _Float16, BM, BN, BK, WM, WN>(W, A, C, M, N, K, s)
               : run_as<KIND, float, BM, BN, BK, WM, WN>(W, A, C, M, N, K, s);
}

// Tile shapes.  Up to 64 tokens: 64 x 128 tiles.  Otherwise 128 x 64 tiles
// with 128-element stages while that grid still fits the 256 compute units
// in one round, else 128 x 128 tiles with eight waves (fewer re-reads of the
// activations, two waves per SIMD): 128-element stages for f16 A, 64-element
// stages for f32 A, whose two f16 planes would need 192 KiB of LDS with
// 128-element stages.
template <int KIND>
static hipError_t run_m(const uint8_t *W, const void *A, int a_f16, float *C, int64_t M, int64_t N, int64_t K,
                        hipStream_t s, int cfg) {
#ifdef QMM_TUNING
  switch (cfg) {
    case 1: return run<KIND, 64, 128, 64, 1, 4>(W, A, a_f16, C, M, N, K, s);
    case 2: return run<KIND, 128, 128, 64, 2, 2>(W, A, a_f16, C, M, N, K, s);
    case 3: return run<KIND, 128, 64, 64, 2, 2>(W, A, a_f16, C, M, N, K, s);
    case 4: return run<KIND, 256, 128, 64, 4, 2>(W, A, a_f16, C, M, N, K, s);
    case 5: return run<KIND, 128, 128, 32, 2, 2>(W, A, a_f16, C, M, N, K, s);
    case 6: return run<KIND, 128, 64, 128, 2, 2>(W, A, a_f16, C, M, N, K, s);
    case 7: return run<KIND, 128, 128, 128, 2, 2>(W, A, a_f16, C, M, N, K, s);
    case 8: return run<KIND, 64, 128, 128, 1, 4>(W, A, a_f16, C, M, N, K, s);
    case 9: return run<KIND, 128, 128, 128, 2, 4>(W, A, a_f16, C, M, N, K, s);
    default: break;
  }
#else
  (void)cfg;
#endif
  if (M <= 64) return run<KIND, 64, 128, 64, 1, 4>(W, A, a_f16, C, M, N, K, s);
  if (((M + 127) / 128) * ((N + 63) / 64) <= 256) return run<KIND, 128, 64, 128, 2, 2>(W, A, a_f16, C, M, N, K, s);
  if (a_f16) return run_as<KIND, _Float16, 128, 128, 128, 2, 4>(W, A, C, M, N, K, s);
  return run_as<KIND, float, 128, 128, 64, 2, 4>(W, A, C, M, N, K, s);
}

}  // namespace gm

hipError_t launch_gemm(int kind, const uint8_t *W, const void *A, int a_f16, float *C, int64_t M,
                       int64_t N, int64_t K, hipStream_t s) {
  if (gemm_ks_supported(kind, M, N, K, a_f16)) return launch_gemm_ks(kind, W, A, a_f16, C, M, N, K, s);
  return launch_gemm_lds(kind, W, A, a_f16, C, M, N, K, s);
}

hipError_t launch_gemm_lds(int kind, const uint8_t *W, const void *A, int a_f16, float *C, int64_t M,
                           int64_t N, int64_t K, hipStream_t s) {
  // Launch shapes are fixed by the rules in run_m.  A tuning build
  // (-DQMM_TUNING) can pick an alternative shape from QMM_GEMM_CFG.
#ifdef QMM_TUNING
  static const int cfg = [] {
    const char *e = getenv("QMM_GEMM_CFG");
    return e ? atoi(e) : 0;
  }();
#else
  constexpr int cfg = 0;
#endif
  switch (kind) {
#define QMM_CASE(K_) \
  case K_:           \
    return gm::run_m<K_>(W, A, a_f16, C, M, N, K, s, cfg);
    QMM_FOR_EACH_KIND(QMM_CASE)
#undef QMM_CASE
  }
  return hipErrorInvalidValue;
}

}  // namespace qmm
