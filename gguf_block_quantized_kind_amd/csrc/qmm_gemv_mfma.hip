// qmm_gemv_mfma.hip -- the matrix-core decode GEMV (see qmm_gemv_mfma.h).
//
// Work split.  A workgroup owns R tiles of 16 weight rows and S waves.  Wave
// w takes k-blocks [w*n/S, (w+1)*n/S) of every row, so the S waves cut K into
// S ranges and their partial sums meet in LDS at the end; every activation
// k-block a wave stages serves its R tiles.
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "qmm_gemv_mfma.h"
#include "qmm_internal.h"

namespace qmm {
namespace gv {

// Software pipeline.  Each wave walks its k-blocks in order with PD k-blocks
// in flight: before it decodes k-block kb it issues, for k-block kb+PD, the
// weight loads of its R tiles and its slice of the activations (each lane
// loads 4 consecutive elements of one token, 16 bytes); then it waits for kb,
// converts kb's activation slice to f16 into a wave-private LDS ring
// (fragment layout below), and decodes and multiplies kb.  Loads therefore leave in the order they are
// consumed, the activations never queue behind a full HBM stream, and only PD
// k-blocks of registers are held.
//
// Fragment layout of one k-block: fragment (s, t, G) -- 8 elements of token
// t in the pair order 0,2,1,3,4,6,5,7, 16 bytes -- at (s * MT + t) * 4 + G, so
// the MT token rows of one step are MT * 64 contiguous bytes and no two lanes
// of a read share a bank.  Lanes whose A-row is >= MT read a zero fragment.

template <int KIND, int MT>
struct XSlice {
  using Dd = Dec<KIND>;
  static constexpr int kFrag = Dd::NSTEP * MT * 4;   // fragments per k-block
  static constexpr int kHalves = 2 * kFrag;          // 4-element halves per k-block
  static constexpr int kPerLane = (kHalves + 63) / 64;
};

// Weight bytes a lane holds for one tile and k-block between issue and
// decode: the decoder's own fields, or (CHUNKED decoders) its share of the
// k-block as 16-byte chunks (Chunks in qmm_gemv_mfma.h).
template <int KIND, bool PACKED, typename Dd>
struct HeldOf {  // native rows (kinds without repacked records stop here)
  using type = typename std::conditional<Dd::CHUNKED, typename Chunks<Dd>::Held, typename Dd::Raw>::type;
};
template <int KIND, typename Dd>
struct HeldOf<KIND, true, Dd> {
  using type = typename Rec<KIND>::Packed;
};
template <int KIND, bool PACKED, typename Dd = Dec<KIND>>
using Held = typename HeldOf<KIND, PACKED, Dd>::type;

// PACKED: W is the repacked layout (the records above Rec in
// qmm_gemv_mfma.h) instead of native rows; row_bytes is then unused.
template <int KIND, typename XT, int MT, int S, int R, int PD, int OCC, bool ROUTED, bool PACKED>
__global__ __launch_bounds__(64 * S) __attribute__((amdgpu_waves_per_eu(OCC, 8))) void gemv_mfma_kernel(
    const uint8_t *__restrict__ W, int64_t row_bytes, const XT *__restrict__ X, float *__restrict__ Y, int M,
    int64_t N, int K, MoeRoute rt) {
  using Dd = Dec<KIND>;
  using XS = XSlice<KIND, MT>;
  using X4 = typename XVec<XT>::type;
  constexpr int kFrag = XS::kFrag;
  extern __shared__ u32x4 lds[];  // S rings of PD+1 k-blocks, one zero fragment, S weight stagings;
                                  // later the reduction
  using CK = Chunks<Dd>;
  // The wave index is uniform: in a scalar register the k-block loop below
  // runs on scalar branches.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = lane & 15, G = lane >> 4;
  // Routed experts: this workgroup serves one work item, up to MT pairs
  // order[c0 ..] of expert e, whose rows start at expert e's weights.
  int c0 = 0;
  const int32_t *order = nullptr;
  if constexpr (ROUTED) {
    const int item = blockIdx.x;
    int e;
    if (rt.ids != nullptr) {  // one pair per item, no grouping
      e = item < rt.pairs ? rt.ids[item] : -1;
      if (e < 0 || e >= rt.E) return;  // the whole workgroup leaves before any barrier
      c0 = item;
      M = 1;
    } else {
      if (item >= rt.ws[rt.nwork_at]) return;  // the whole workgroup leaves before any barrier
      e = rt.ws[rt.work_at + 2 * item];
      c0 = rt.ws[rt.work_at + 2 * item + 1];
      order = rt.ws + rt.order_at;
      M = min(MT, rt.ws[rt.offsets_at + e + 1] - c0);
    }
    // Expert e's rows (repacked: its records, N padded to whole tiles).
    W += (int64_t)e * (PACKED ? (N + 15) / 16 * 16 : N) * row_bytes;
  }
  // Pair of token slot t of this item.
  auto pair_of = [&](int t) { return order != nullptr ? order[c0 + t] : c0 + t; };
  const int64_t row0 = (int64_t)(ROUTED ? blockIdx.y : blockIdx.x) * (16 * R);
  const int nkb = K / Dd::KB;
  u32x4 *ring = lds + wave * (PD + 1) * kFrag;
  const u32x4 *zero = lds + S * (PD + 1) * kFrag;
  if (threadIdx.x == 0) lds[S * (PD + 1) * kFrag] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  constexpr int64_t kRec = 16 * Dd::BYTES;  // one repacked record
  const uint8_t *wr[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if constexpr (PACKED) {
      // Tiles past the last one decode the last (padded) tile; their
      // outputs are not stored.
      const int64_t tile = min(row0 / 16 + r, (N - 1) / 16);
      wr[r] = W + tile * nkb * kRec;
    } else {
      int64_t row = row0 + 16 * r + j;
      if (row >= N) row = N - 1;  // decode a real row; its outputs are not stored
      wr[r] = W + row * row_bytes;
    }
  }
  floatx4 acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = floatx4{0.f, 0.f, 0.f, 0.f};

  // This lane's activation slice: half-fragment h = lane + 64 i of a k-block
  // is elements x_off(s, G', h & 1) + [0, 4) of token t.
  int xoff[XS::kPerLane], xdst[XS::kPerLane];
  bool xlive[XS::kPerLane];
#pragma unroll
  for (int i = 0; i < XS::kPerLane; ++i) {
    const int h = lane + 64 * i, f = h >> 1;
    const int g2 = f & 3, t = (f >> 2) % MT, st = (f >> 2) / MT;
    xlive[i] = h < XS::kHalves && t < M;
    int64_t xrow = (int64_t)t * K;
    if constexpr (ROUTED) {
      const int pair = xlive[i] ? pair_of(t) : 0;
      xrow = (int64_t)(rt.x_per_slot ? pair : pair / rt.topk) * K;
    }
    xoff[i] = xlive[i] ? xrow + Dd::x_off(st, g2, h & 1) : 0;
    xdst[i] = h < XS::kHalves ? h : -1;
  }

  // Ring of NS = PD + 1 slots: while k-block kb is decoded, k-blocks
  // kb+1 .. kb+PD are in flight; the refill for kb+PD is issued before kb is
  // decoded, so the memory pipe stays busy through every compute phase.
  constexpr int NS = PD + 1;
  const int kb0 = (int)((int64_t)wave * nkb / S), kb1 = (int)((int64_t)(wave + 1) * nkb / S);
  Held<KIND, PACKED> raw[NS][R];
  X4 xv[NS][XS::kPerLane];
  // Dead lanes skip their activation loads (zeros); no k-block past the
  // wave's last is issued.  (A form that issues every load unconditionally,
  // in whole rounds of NS k-blocks so that no wait drains the later ones,
  // holds more registers here and measured 5-100% slower on this kernel's
  // shapes.)
  auto issue = [&](int kb, int slot) {
#pragma unroll
    for (int i = 0; i < XS::kPerLane; ++i) {
      X4 v = {};
      if (xlive[i]) __builtin_memcpy(&v, X + xoff[i] + (int64_t)kb * Dd::KB, sizeof(X4));
      xv[slot][i] = v;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if constexpr (PACKED) {
        Rec<KIND>::load(wr[r] + kb * kRec, lane, j, G, raw[slot][r]);
      } else if constexpr (Dd::CHUNKED) {
        CK::load(wr[r] + (int64_t)kb * Dd::BYTES, G, raw[slot][r]);
      } else {
        Dd::load(wr[r] + (int64_t)kb * Dd::BYTES, G, raw[slot][r]);
      }
    }
  };
  // This wave's LDS copy of one tile's k-block (CHUNKED decoders): row j at
  // j * RS, each chunk at its byte offset in the k-block.
  uint8_t *stage = reinterpret_cast<uint8_t *>(lds + S * (PD + 1) * kFrag + 1) + wave * 16 * CK::RS;
#pragma unroll
  for (int d = 0; d < PD; ++d)
    if (kb0 + d < kb1) issue(kb0 + d, d);

  // Decode and multiply the k-block held in ring slot d.
  auto consume = [&](int d) {
    // Its activations into LDS ring slot d (pair order per half).
    u32x4 *xk = ring + d * kFrag;
#pragma unroll
    for (int i = 0; i < XS::kPerLane; ++i) {
      if (xdst[i] < 0) continue;
      const X4 v = xv[d][i];
      const half2v p0 = {(_Float16)v[0], (_Float16)v[2]}, p1 = {(_Float16)v[1], (_Float16)v[3]};
      u32x2 *dst = reinterpret_cast<u32x2 *>(xk) + xdst[i];
      *dst = u32x2{as_u(p0), as_u(p1)};
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const u32x4 *xr = j < MT ? xk + j * 4 + G : zero;
    const int xstep = j < MT ? MT * 4 : 0;
    half8 a[Dd::NSTEP];
    floatx4 xsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < Dd::NSTEP; ++st) {
      a[st] = __builtin_bit_cast(half8, xr[st * xstep]);
      if constexpr (Dd::HAS_MIN) {
        const _Float16 v = Dd::ind(st, G, j) ? (_Float16)1.0f : (_Float16)0.0f;
        xsum = mfma16(half8{v, v, v, v, v, v, v, v}, a[st], xsum);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      typename Dd::Raw fr;  // the decoder's fields for this tile and k-block
      if constexpr (PACKED) {
        fr = Rec<KIND>::unpack(raw[d][r], G);
      } else if constexpr (Dd::CHUNKED) {
        // Stage the tile's k-block in LDS, then read the decoder's fields.
        uint8_t *row = stage + j * CK::RS;
        CK::stage(row, raw[d][r], G);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        Dd::load(row, G, fr);
      } else {
        fr = raw[d][r];
      }
      const typename Dd::Sc sc = Dd::prep(fr, G);
      if constexpr (Dd::STEP_SCALE) {
#pragma unroll
        for (int st = 0; st < Dd::NSTEP; ++st) {
          const floatx4 D = mfma16(a[st], Dd::bop(fr, sc, st, 0), floatx4{0.f, 0.f, 0.f, 0.f});
          acc[r] = Dd::post_step(acc[r], D, fr, st);
        }
      } else {
        floatx4 D[Dd::NPART];
#pragma unroll
        for (int p = 0; p < Dd::NPART; ++p) D[p] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < Dd::NSTEP; ++st)
#pragma unroll
          for (int p = 0; p < Dd::NPART; ++p) D[p] = mfma16(a[st], Dd::bop(fr, sc, st, p), D[p]);
        acc[r] = Dd::post(acc[r], D, xsum, sc);
      }
      if constexpr (Dd::CHUNKED && !PACKED) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();  // the staging is rewritten by the next tile
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // slot d is rewritten NS k-blocks later
  };
  // Whole rounds of NS k-blocks: every round issues NS refills, never under a
  // branch, so each wait leaves the PD newer k-blocks in flight.  The last
  // cnt % NS k-blocks (already issued) follow.
  for (int kb = kb0; kb < kb1; kb += NS) {
#pragma unroll
    for (int d = 0; d < NS; ++d) {
      if (kb + d >= kb1) break;
      if (kb + d + PD < kb1) issue(kb + d + PD, (d + PD) % NS);
      consume(d);
    }
  }

  if constexpr (S > 1) {
    __syncthreads();  // every wave is done with its ring
    floatx4 *red = reinterpret_cast<floatx4 *>(lds);
    if (wave > 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) red[((wave - 1) * R + r) * 64 + lane] = acc[r];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < S - 1; ++w)
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] += red[(w * R + r) * 64 + lane];
  }
  // Lane (j, G) holds D[token 4G + q][row j] of each tile.
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + 16 * r + j;
    if (row >= N) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = 4 * G + q;
      if (t < M) Y[(int64_t)(ROUTED ? pair_of(t) : t) * N + row] = acc[r][q];
    }
  }
}

template <int KIND, int MT, int S, int R, int PD, int OCC = 1, bool ROUTED = false, bool PACKED = false>
static hipError_t run(const uint8_t *W, const void *x, int x_f16, float *y, int M, int64_t N, int64_t K,
                      hipStream_t s, MoeRoute rt = MoeRoute{}, int items = 0) {
  const int64_t row_bytes = (K / Geometry<KIND>::elems) * Geometry<KIND>::bytes;
  const size_t ring = (size_t)S * (PD + 1) * XSlice<KIND, MT>::kFrag * 16 + 16 +
                      (Dec<KIND>::CHUNKED && !PACKED ? (size_t)S * 16 * Chunks<Dec<KIND>>::RS : 0);
  const size_t lds = std::max<size_t>(ring, (size_t)(S - 1) * R * 64 * sizeof(floatx4));
  const unsigned tiles = (unsigned)((N + 16 * R - 1) / (16 * R));
  const dim3 grid = ROUTED ? dim3((unsigned)items, tiles) : dim3(tiles), block(64 * S);
  if (x_f16)
    hipLaunchKernelGGL((gemv_mfma_kernel<KIND, _Float16, MT, S, R, PD, OCC, ROUTED, PACKED>), grid, block, lds, s, W,
                       row_bytes, (const _Float16 *)x, y, M, N, (int)K, rt);
  else
    hipLaunchKernelGGL((gemv_mfma_kernel<KIND, float, MT, S, R, PD, OCC, ROUTED, PACKED>), grid, block, lds, s, W,
                       row_bytes, (const float *)x, y, M, N, (int)K, rt);
  return hipGetLastError();
}

// Launch shapes, chosen by M: small M keeps many k-blocks in flight per
// wave; large M shares each staged activation k-block among R tiles.
template <int KIND>
static hipError_t run_m(const uint8_t *W, const void *x, int x_f16, float *y, int M, int64_t N, int64_t K,
                        hipStream_t s, int cfg) {
#ifdef QMM_TUNING
  switch (cfg) {
    case 1: if (M <= 1) return run<KIND, 1, 4, 1, 1>(W, x, x_f16, y, M, N, K, s); break;
    case 2: if (M <= 1) return run<KIND, 1, 2, 1, 2>(W, x, x_f16, y, M, N, K, s); break;
    case 3: if (M <= 1) return run<KIND, 1, 2, 1, 3>(W, x, x_f16, y, M, N, K, s); break;
    case 7: if (M <= 1) return run<KIND, 1, 1, 1, 3>(W, x, x_f16, y, M, N, K, s); break;

    case 8: if (M <= 1) return run<KIND, 1, 8, 1, 1>(W, x, x_f16, y, M, N, K, s); break;
    case 9: if (M <= 1) return run<KIND, 1, 8, 1, 2>(W, x, x_f16, y, M, N, K, s); break;
    case 10: if (M <= 1) return run<KIND, 1, 4, 1, 2>(W, x, x_f16, y, M, N, K, s); break;
    case 4: if (M > 4) return run<KIND, 8, 4, 1, 2>(W, x, x_f16, y, M, N, K, s); break;
    case 5: if (M > 4) return run<KIND, 8, 4, 2, 1>(W, x, x_f16, y, M, N, K, s); break;
    case 6: if (M > 4) return run<KIND, 8, 2, 2, 2>(W, x, x_f16, y, M, N, K, s); break;
    default: break;
  }
#else
  (void)cfg;
#endif
  if constexpr (Dec<KIND>::CHUNKED) {
    // Staged decoders hold one k-block ahead and split K over 4 to 16 waves
    // (more waves per tile when there are few tiles).
    if (M <= 1) {
      if (N <= 4096) return run<KIND, 1, 16, 1, 1>(W, x, x_f16, y, M, N, K, s);
      if (N < 8192) return run<KIND, 1, 8, 1, 1>(W, x, x_f16, y, M, N, K, s);
      return run<KIND, 1, 4, 1, 1>(W, x, x_f16, y, M, N, K, s);
    }
  }
  if (M <= 1) return run<KIND, 1, 2, 1, 2>(W, x, x_f16, y, M, N, K, s);
  if (M <= 2) return run<KIND, 2, 2, 1, 2>(W, x, x_f16, y, M, N, K, s);
  if (M <= 4) return run<KIND, 4, 2, 2, 2>(W, x, x_f16, y, M, N, K, s);
  return run<KIND, 8, 2, 2, 2>(W, x, x_f16, y, M, N, K, s);
}

template <int KIND, bool PACKED>
static hipError_t run_routed(const uint8_t *W, const void *x, int x_f16, float *y, int mt, int64_t N, int64_t K,
                             hipStream_t s, const MoeRoute &rt, int items) {
  if (mt == 1) {
    // Three k-blocks (an expert down matrix of 768 columns): one per wave
    // rather than one and two.
    if (K == 3 * Dec<KIND>::KB) return run<KIND, 1, 3, 1, 1, 1, true, PACKED>(W, x, x_f16, y, 1, N, K, s, rt, items);
    return run<KIND, 1, 2, 1, 2, 1, true, PACKED>(W, x, x_f16, y, 1, N, K, s, rt, items);
  }
  if (mt == 8) return run<KIND, 8, 2, 2, 2, 1, true, PACKED>(W, x, x_f16, y, 8, N, K, s, rt, items);
  // Sixteen pairs per item: the activation k-block staged by a wave serves
  // four 16-row tiles.
  return run<KIND, 16, 1, 4, 1, 1, true, PACKED>(W, x, x_f16, y, 16, N, K, s, rt, items);
}

// Launch shapes over the repacked layout (no staging), for what the kernels
// of qmm_gemv_t1.hip and qmm_gemv_xs.hip do not take (in default builds:
// Q2_K, Q3_K and Q5_K at one token).  Fewer waves per tile (two tiles per
// wave) measured 40-70% slower at one token.
template <int KIND>
static hipError_t run_packed(const uint8_t *P, const void *x, int x_f16, float *y, int M, int64_t N, int64_t K,
                             hipStream_t s, int cfg) {
#ifdef QMM_TUNING
  switch (cfg) {
    case 21: if (M <= 1) return run<KIND, 1, 4, 1, 2, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 22: if (M <= 1) return run<KIND, 1, 2, 1, 3, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 23: if (M <= 1) return run<KIND, 1, 4, 1, 1, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 24: if (M <= 1) return run<KIND, 1, 1, 1, 3, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 25: if (M <= 1) return run<KIND, 1, 2, 2, 2, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 26: if (M > 4) return run<KIND, 8, 4, 1, 2, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 27: if (M > 4) return run<KIND, 8, 2, 1, 2, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 28: if (M <= 1) return run<KIND, 1, 8, 1, 2, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 29: if (M <= 1) return run<KIND, 1, 8, 1, 1, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 30: if (M <= 1) return run<KIND, 1, 16, 1, 1, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 31: if (M <= 1) return run<KIND, 1, 4, 1, 3, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 32: if (M > 4) return run<KIND, 8, 2, 2, 1, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 33: if (M > 4) return run<KIND, 8, 4, 2, 1, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 34: if (M > 4) return run<KIND, 8, 2, 3, 1, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 35: if (M > 4) return run<KIND, 8, 1, 2, 2, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 36: if (M <= 1) return run<KIND, 1, 2, 2, 2, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 37: if (M <= 1) return run<KIND, 1, 1, 2, 2, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 38: if (M <= 1) return run<KIND, 1, 4, 2, 2, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 40: if (M <= 1) return run<KIND, 1, 4, 1, 2, 4, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 41: if (M <= 1) return run<KIND, 1, 4, 1, 1, 4, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 42: if (M <= 1) return run<KIND, 1, 2, 1, 2, 4, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 43: if (M <= 1) return run<KIND, 1, 8, 1, 1, 4, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 44: if (M <= 1) return run<KIND, 1, 2, 1, 2, 3, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 45: if (M > 4) return run<KIND, 8, 4, 2, 2, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 46: if (M > 4) return run<KIND, 8, 2, 2, 2, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 47: if (M > 4) return run<KIND, 8, 8, 2, 1, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 48: if (M > 4) return run<KIND, 8, 2, 4, 1, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 49: if (M > 4) return run<KIND, 8, 4, 4, 1, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 50: if (M > 4) return run<KIND, 8, 8, 1, 1, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 51: if (M > 4) return run<KIND, 8, 4, 1, 1, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 52: if (M > 4) return run<KIND, 8, 4, 1, 3, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 53: if (M <= 1) return run<KIND, 1, 4, 2, 1, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 54: if (M <= 1) return run<KIND, 1, 2, 1, 1, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 55: if (M <= 1) return run<KIND, 1, 2, 2, 1, 1, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 56: if (M <= 1) return run<KIND, 1, 4, 1, 3, 4, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 57: if (M > 4) return run<KIND, 8, 2, 2, 1, 2, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 58: if (M > 4) return run<KIND, 8, 2, 2, 1, 3, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 59: if (M > 4) return run<KIND, 8, 4, 2, 1, 2, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 60: if (M > 4) return run<KIND, 8, 4, 2, 1, 3, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 61: if (M > 4) return run<KIND, 8, 2, 1, 1, 3, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 62: if (M > 4) return run<KIND, 8, 4, 1, 1, 4, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 63: if (M <= 1) return run<KIND, 1, 2, 1, 2, 2, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 64: if (M <= 1) return run<KIND, 1, 4, 1, 1, 3, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 65: if (M <= 1) return run<KIND, 1, 4, 1, 2, 3, false, true>(P, x, x_f16, y, M, N, K, s); break;
    case 66: if (M <= 1) return run<KIND, 1, 8, 1, 1, 3, false, true>(P, x, x_f16, y, M, N, K, s); break;
    default: break;
  }
#else
  (void)cfg;
#endif
  if (M <= 1) return run<KIND, 1, 2, 1, 2, 1, false, true>(P, x, x_f16, y, M, N, K, s);
  if (M <= 2) return run<KIND, 2, 2, 1, 2, 1, false, true>(P, x, x_f16, y, M, N, K, s);
  if (M <= 4) return run<KIND, 4, 2, 2, 2, 1, false, true>(P, x, x_f16, y, M, N, K, s);
  // Eight tokens: one k-block in flight (the activation ring of eight
  // tokens is most of the registers; measured 3-4% faster than two).
  return run<KIND, 8, 2, 2, 1, 1, false, true>(P, x, x_f16, y, M, N, K, s);
}

}  // namespace gv

bool packed_supported(int kind) {
  switch (kind) {
    case Q4_K: case Q6_K: case IQ4_XS: case Q4_0: case Q5_0: case Q8_0: case IQ4_NL: case MXFP4:
    case Q2_K: case Q3_K: case Q5_K:
      return true;
    default:
      return false;
  }
}

hipError_t launch_gemv_packed(int kind, const uint8_t *P, const void *x, int x_f16, float *y, int M, int64_t N,
                              int64_t K, hipStream_t s) {
#ifdef QMM_TUNING
  static const int cfg = [] {
    const char *e = getenv("QMM_GEMV_CFG");
    return e ? atoi(e) : 0;
  }();
#else
  constexpr int cfg = 0;
#endif
  // Two to eight tokens: the kernel that stages activations per workgroup
  // (tuning shapes below 100 select this file's kernels instead).
  if (M > 1 && (cfg == 0 || cfg >= 100)) return launch_gemv_xs(kind, P, x, x_f16, y, M, N, K, s, cfg);
  // One token: the kernel that applies the sub-block or block scales after
  // the products (tuning shapes from 200 up).
  if (M == 1 && gemv_t1_supported(kind, true) && (cfg == 0 || cfg >= 200))
    return launch_gemv_t1(kind, P, x, x_f16, y, N, K, s, cfg);
  switch (kind) {
    case Q4_K: return gv::run_packed<Q4_K>(P, x, x_f16, y, M, N, K, s, cfg);
    case Q6_K: return gv::run_packed<Q6_K>(P, x, x_f16, y, M, N, K, s, cfg);
    case IQ4_XS: return gv::run_packed<IQ4_XS>(P, x, x_f16, y, M, N, K, s, cfg);
    case Q4_0: return gv::run_packed<Q4_0>(P, x, x_f16, y, M, N, K, s, cfg);
    case Q5_0: return gv::run_packed<Q5_0>(P, x, x_f16, y, M, N, K, s, cfg);
    case Q8_0: return gv::run_packed<Q8_0>(P, x, x_f16, y, M, N, K, s, cfg);
    case IQ4_NL: return gv::run_packed<IQ4_NL>(P, x, x_f16, y, M, N, K, s, cfg);
    case MXFP4: return gv::run_packed<MXFP4>(P, x, x_f16, y, M, N, K, s, cfg);
    case Q2_K: return gv::run_packed<Q2_K>(P, x, x_f16, y, M, N, K, s, cfg);
    case Q3_K: return gv::run_packed<Q3_K>(P, x, x_f16, y, M, N, K, s, cfg);
    case Q5_K: return gv::run_packed<Q5_K>(P, x, x_f16, y, M, N, K, s, cfg);
    default: break;
  }
  return hipErrorNotSupported;
}

bool moe_mfma_supported(int kind, int64_t K) {
  switch (kind) {
    case Q4_K: case Q6_K: case IQ4_XS: case Q4_0: case Q5_0: case Q8_0: case IQ4_NL: case MXFP4:
    case Q2_K: case Q3_K: case Q5_K:
      return K % 256 == 0;
    default:
      return false;
  }
}

hipError_t launch_moe_mfma(int kind, const uint8_t *W, const void *X, int x_f16, float *Y, int mt, int64_t N,
                           int64_t K, const MoeRoute &rt, int items, hipStream_t s, bool packed) {
  // One pair per item, a super-block kind: the single-token decoders (the
  // step-scaled kinds keep this file's kernel for routed pairs).
  if (mt == 1 && rt.ids != nullptr && items <= 65535 && gemv_t1_supported(kind, false))
    return launch_moe_t1(kind, W, X, x_f16, Y, N, K, rt, items, s, packed);
  // Grouped items: activations staged once for eight tiles (repacked
  // experts, or native rows of the super-block kinds).
  if ((mt == 8 || mt == 16) && items <= 65535 && (packed || xs_native_supported(kind)))
    return launch_moe_xs(kind, W, X, x_f16, Y, mt, N, K, rt, items, s, packed);
  if (packed) {
    switch (kind) {
      case Q4_K: return gv::run_routed<Q4_K, true>(W, X, x_f16, Y, mt, N, K, s, rt, items);
      case Q6_K: return gv::run_routed<Q6_K, true>(W, X, x_f16, Y, mt, N, K, s, rt, items);
      case IQ4_XS: return gv::run_routed<IQ4_XS, true>(W, X, x_f16, Y, mt, N, K, s, rt, items);
      case Q4_0: return gv::run_routed<Q4_0, true>(W, X, x_f16, Y, mt, N, K, s, rt, items);
      case Q5_0: return gv::run_routed<Q5_0, true>(W, X, x_f16, Y, mt, N, K, s, rt, items);
      case Q8_0: return gv::run_routed<Q8_0, true>(W, X, x_f16, Y, mt, N, K, s, rt, items);
      case IQ4_NL: return gv::run_routed<IQ4_NL, true>(W, X, x_f16, Y, mt, N, K, s, rt, items);
      case MXFP4: return gv::run_routed<MXFP4, true>(W, X, x_f16, Y, mt, N, K, s, rt, items);
      case Q2_K: return gv::run_routed<Q2_K, true>(W, X, x_f16, Y, mt, N, K, s, rt, items);
      case Q3_K: return gv::run_routed<Q3_K, true>(W, X, x_f16, Y, mt, N, K, s, rt, items);
      case Q5_K: return gv::run_routed<Q5_K, true>(W, X, x_f16, Y, mt, N, K, s, rt, items);
      default: return hipErrorNotSupported;
    }
  }
  switch (kind) {
    case Q4_K: return gv::run_routed<Q4_K, false>(W, X, x_f16, Y, mt, N, K, s, rt, items);
    case Q6_K: return gv::run_routed<Q6_K, false>(W, X, x_f16, Y, mt, N, K, s, rt, items);
    case IQ4_XS: return gv::run_routed<IQ4_XS, false>(W, X, x_f16, Y, mt, N, K, s, rt, items);
    case Q2_K: return gv::run_routed<Q2_K, false>(W, X, x_f16, Y, mt, N, K, s, rt, items);
    case Q3_K: return gv::run_routed<Q3_K, false>(W, X, x_f16, Y, mt, N, K, s, rt, items);
    case Q5_K: return gv::run_routed<Q5_K, false>(W, X, x_f16, Y, mt, N, K, s, rt, items);
    case Q4_0: return gv::run_routed<Q4_0, false>(W, X, x_f16, Y, mt, N, K, s, rt, items);
    case Q5_0: return gv::run_routed<Q5_0, false>(W, X, x_f16, Y, mt, N, K, s, rt, items);
    case Q8_0: return gv::run_routed<Q8_0, false>(W, X, x_f16, Y, mt, N, K, s, rt, items);
    case IQ4_NL: return gv::run_routed<IQ4_NL, false>(W, X, x_f16, Y, mt, N, K, s, rt, items);
    case MXFP4: return gv::run_routed<MXFP4, false>(W, X, x_f16, Y, mt, N, K, s, rt, items);
    default: break;
  }
  return hipErrorNotSupported;
}

// Returns hipErrorNotSupported when the kind has no matrix-core decoder or K
// is not a whole number of the decoder's k-blocks.
hipError_t launch_gemv_mfma(int kind, const uint8_t *W, const void *x, int x_f16, float *y, int M,
                            int64_t N, int64_t K, hipStream_t s) {
  // Activation offsets are 32-bit inside the kernel.
  if ((int64_t)M * K >= ((int64_t)1 << 31)) return hipErrorNotSupported;
  // Launch shapes are fixed by the rules in run_m.  A tuning build
  // (-DQMM_TUNING) can pick an alternative shape from QMM_GEMV_CFG.
#ifdef QMM_TUNING
  static const int cfg = [] {
    const char *e = getenv("QMM_GEMV_CFG");
    return e ? atoi(e) : 0;
  }();
#else
  constexpr int cfg = 0;
#endif
  // One token: the single-token decoders; two to eight tokens of a
  // super-block kind: the staged-activation kernel.
  if (M == 1 && K % 256 == 0 && gemv_t1_supported(kind, false) && (cfg == 0 || cfg >= 200))
    return launch_gemv_t1(kind, W, x, x_f16, y, N, K, s, cfg, false);
  if (M > 1 && xs_native_supported(kind) && (cfg == 0 || cfg >= 100))
    return launch_gemv_xs_native(kind, W, x, x_f16, y, M, N, K, s);
  switch (kind) {
    case Q4_K: return gv::run_m<Q4_K>(W, x, x_f16, y, M, N, K, s, cfg);
    case Q6_K: return gv::run_m<Q6_K>(W, x, x_f16, y, M, N, K, s, cfg);
    case IQ4_XS: return gv::run_m<IQ4_XS>(W, x, x_f16, y, M, N, K, s, cfg);
    case Q2_K: return gv::run_m<Q2_K>(W, x, x_f16, y, M, N, K, s, cfg);
    case Q3_K: return gv::run_m<Q3_K>(W, x, x_f16, y, M, N, K, s, cfg);
    case Q5_K: return gv::run_m<Q5_K>(W, x, x_f16, y, M, N, K, s, cfg);
    default: break;
  }
  // The 32-element kinds walk K in k-blocks of eight blocks.
  if (K % 256 != 0) return hipErrorNotSupported;
  switch (kind) {
    case Q4_0: return gv::run_m<Q4_0>(W, x, x_f16, y, M, N, K, s, cfg);
    case Q5_0: return gv::run_m<Q5_0>(W, x, x_f16, y, M, N, K, s, cfg);
    case Q8_0: return gv::run_m<Q8_0>(W, x, x_f16, y, M, N, K, s, cfg);
    case IQ4_NL: return gv::run_m<IQ4_NL>(W, x, x_f16, y, M, N, K, s, cfg);
    case MXFP4: return gv::run_m<MXFP4>(W, x, x_f16, y, M, N, K, s, cfg);
    default: break;
  }
  return hipErrorNotSupported;
}

}  // namespace qmm
