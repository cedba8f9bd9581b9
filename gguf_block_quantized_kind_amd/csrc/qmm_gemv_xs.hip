// qmm_gemv_xs.hip -- the decode GEMV over repacked weights for 2 to 8
// tokens, with each activation k-block staged once per workgroup.
//
// Work split.  The grid's workgroups split the tiles of 16 weight rows
// evenly, at most T each (a grid of one workgroup per compute unit when
// that is more than ceil(tiles / T), so that no unit idles).  A workgroup
// has T * S waves; wave w decodes its workgroup's tile w % T over k-part
// p = w / T, the k-blocks
// [p * n / S, (p + 1) * n / S); the S partial sums of a tile meet in LDS at
// the end.  The T waves of one k-part walk the same k-blocks in step: each
// activation k-block is loaded, rounded to f16 and written in fragment layout
// into the k-part's LDS ring once, every wave taking a 1/T share, and all T
// waves read it from there.
//
// Registers.  A wave holds its tile's weights for PD + 1 k-blocks (one
// decoded, PD in flight) and its share of one activation k-block; the
// activation fragments are read from LDS one MFMA step at a time.  That keeps
// a wave near 100 registers, so several waves share each SIMD and hide one
// another's memory waits.
//
// Order of loads.  A wave's vector loads complete in issue order, so round r
// issues the activations of round r + XD before the weights of round r + PD:
// the wait for a round's activations then covers only weights that are due
// no later than that round.  Every load is issued on every path (past the
// last k-block the last one is read again), so no wait is ever widened by a
// branch.
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "qmm_gemv_mfma.h"
#include "qmm_internal.h"

namespace qmm {
namespace gv {

// s_waitcnt with lgkmcnt(0) and the vector-memory and export counts left
// at their maximum (this wave's LDS writes have landed; its global loads may
// still be in flight).
constexpr int kWaitLds = 0xC07F;

// ROUTED: workgroup (b, item) serves work item `item` of a grouped expert
// product (up to MT pairs of one expert, as the routing prologue of
// qmm_moe.hip cut them): the expert's records, the pairs' activation rows
// (gathered through the pair order) as the tokens, outputs scattered to the
// pairs' rows.
// PACKED false: P holds native GGUF rows of row_bytes bytes (decoders that
// load their fields straight from global memory only, not the LDS-staged
// ones).
template <int KIND, typename XT, int MT, int T, int S, int PD, int XD, bool ROUTED = false, bool PACKED = true>
__global__ __launch_bounds__(64 * T * S) void gemv_xs_kernel(const uint8_t *__restrict__ P,
                                                             const XT *__restrict__ X, float *__restrict__ Y,
                                                             int M, int64_t N, int K, int per_wg, int extra,
                                                             MoeRoute rt, int64_t row_bytes) {
  using Dd = Dec<KIND>;
  using X4 = typename XVec<XT>::type;
  constexpr int kFrag = Dd::NSTEP * MT * 4;  // 16-byte fragments per k-block (layout of qmm_gemv_mfma.hip)
  constexpr int kHalves = 2 * kFrag;         // 4-element halves per k-block
  static_assert(kHalves % T == 0, "activation shares");
  constexpr int kShare = kHalves / T;        // halves per wave
  constexpr int kPerLane = (kShare + 63) / 64;
  constexpr int NS = PD + 1;                 // weight slots
  static_assert(XD == 1 || XD == 2, "activation distance");
  constexpr int U = NS % 2 == 0 ? NS : 2 * NS;  // rounds per unrolled turn: every slot index static
  constexpr int64_t kRec = 16 * Dd::BYTES;   // one repacked record
  static_assert(PACKED || !Dd::CHUNKED, "native rows: decoders with direct field loads only");
  extern __shared__ u32x4 lds[];  // S rings of 2 k-blocks of fragments, one zero fragment; later the reduction

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = lane & 15, G = lane >> 4;
  const int t = wave % T, kp = wave / T;
  int c0 = 0;
  const int32_t *order = nullptr;
  if constexpr (ROUTED) {
    const int item = blockIdx.y;
    if (item >= rt.ws[rt.nwork_at]) return;  // the whole workgroup leaves before any barrier
    const int e = rt.ws[rt.work_at + 2 * item];
    c0 = rt.ws[rt.work_at + 2 * item + 1];
    order = rt.ws + rt.order_at;
    M = min(MT, rt.ws[rt.offsets_at + e + 1] - c0);
    P += (int64_t)e * (PACKED ? ((N + 15) / 16) * (K / Dd::KB) * kRec : N * row_bytes);  // expert e's weights
  }
  // Workgroup b owns tiles [t0, t1): per_wg each, one more for the first
  // `extra` workgroups (never past the last tile).
  const int b = blockIdx.x;
  const int t0 = b * per_wg + min(b, extra);
  const int t1 = (int)min<int64_t>(t0 + per_wg + (b < extra ? 1 : 0), (N + 15) / 16);
  // A wave without a tile (t >= t1 - t0) stages its share of the activations
  // and loads the workgroup's last tile again (cache hits), but decodes and
  // stores nothing.
  const bool owner = t0 + t < t1;
  const int64_t tile = owner ? t0 + t : t1 - 1;
  const int nkb = K / Dd::KB;
  const int kb0 = (int)((int64_t)kp * nkb / S), kb1 = (int)((int64_t)(kp + 1) * nkb / S);
  const int cnt = kb1 - kb0;
  const int rounds = (nkb + S - 1) / S;  // every k-part walks the longest k-part's count
  const int kb_last = max(kb1 - 1, 0);
  u32x4 *ring = lds + kp * 2 * kFrag;
  const u32x4 *zero = lds + S * 2 * kFrag;

  // This wave's share of an activation k-block: half h = t * kShare + lane +
  // 64 i is elements x_off(s, G', h & 1) + [0, 4) of token tok.
  int xoff[kPerLane], xdst[kPerLane];
  bool xlive[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int in = lane + 64 * i;
    const int h = t * kShare + in, f = h >> 1;
    const int g2 = f & 3, tok = (f >> 2) % MT, st = (f >> 2) / MT;
    xlive[i] = in < kShare && tok < M;
    int64_t xrow = (int64_t)tok * K;
    if constexpr (ROUTED) {
      const int pair = xlive[i] ? order[c0 + tok] : 0;
      xrow = (int64_t)(rt.x_per_slot ? pair : pair / rt.topk) * K;
    }
    xoff[i] = xlive[i] ? (int)(xrow + Dd::x_off(st, g2, h & 1)) : 0;
    xdst[i] = in < kShare ? h : -1;
  }
  // This tile's records, or row j of it (rows past N decode the last row;
  // their outputs are not stored).
  const uint8_t *wt = PACKED ? P + tile * nkb * kRec : P + min<int64_t>(tile * 16 + j, N - 1) * row_bytes;
  typename std::conditional<PACKED, typename Rec<KIND>::Packed, typename Dd::Raw>::type raw[NS];
  X4 xv[XD][kPerLane];  // activation shares of the next XD k-blocks
  auto issue_w = [&](int kb, int slot) {
    kb = min(kb, kb_last);
    if constexpr (PACKED) Rec<KIND>::load(wt + kb * kRec, lane, j, G, raw[slot]);
    else Dd::load(wt + (int64_t)kb * Dd::BYTES, G, raw[slot]);
  };
  auto issue_x = [&](int kb, int slot) {
    kb = min(kb, kb_last);
#pragma unroll
    for (int i = 0; i < kPerLane; ++i)
      __builtin_memcpy(&xv[slot][i], X + xoff[i] + (int64_t)kb * Dd::KB, sizeof(X4));
  };

  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  const int xstep = j < MT ? MT * 4 : 0;
  // Round r (u = r mod U): stage k-block kb0 + r's activations, then decode
  // it from weight slot u mod NS.
  auto round = [&](int r, int u) {
    const int d = u % NS;
    u32x4 *xk = ring + (u & 1) * kFrag;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      if (!xlive[i]) continue;
      const X4 v = xv[u % XD][i];
      const half2v p0 = {(_Float16)v[0], (_Float16)v[2]}, p1 = {(_Float16)v[1], (_Float16)v[3]};
      reinterpret_cast<u32x2 *>(xk)[xdst[i]] = u32x2{as_u(p0), as_u(p1)};
    }
    issue_x(kb0 + r + XD, u % XD);
    issue_w(kb0 + r + PD, (d + PD) % NS);
    // Every wave's share of slot r & 1 has landed; slot r & 1 was last read
    // two rounds ago, before every wave passed the previous barrier.
    __builtin_amdgcn_s_waitcnt(kWaitLds);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (r >= cnt || !owner) return;  // this k-part has no k-block in this round, or the wave no tile
    typename Dd::Raw fr;
    if constexpr (PACKED) fr = Rec<KIND>::unpack(raw[d], G);
    else fr = raw[d];
    const typename Dd::Sc sc = Dd::prep(fr, G);
    const u32x4 *xr = j < MT ? xk + j * 4 + G : zero;
    floatx4 xsum = {0.f, 0.f, 0.f, 0.f};
    if constexpr (Dd::STEP_SCALE) {
#pragma unroll
      for (int st = 0; st < Dd::NSTEP; ++st) {
        const half8 a = __builtin_bit_cast(half8, xr[st * xstep]);
        const floatx4 D = mfma16(a, Dd::bop(fr, sc, st, 0), floatx4{0.f, 0.f, 0.f, 0.f});
        acc = Dd::post_step(acc, D, fr, st);
      }
    } else {
      floatx4 D[Dd::NPART];
#pragma unroll
      for (int p = 0; p < Dd::NPART; ++p) D[p] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < Dd::NSTEP; ++st) {
        const half8 a = __builtin_bit_cast(half8, xr[st * xstep]);
        if constexpr (Dd::HAS_MIN) {
          const _Float16 v = Dd::ind(st, G, j) ? (_Float16)1.0f : (_Float16)0.0f;
          xsum = mfma16(half8{v, v, v, v, v, v, v, v}, a, xsum);
        }
#pragma unroll
        for (int p = 0; p < Dd::NPART; ++p) D[p] = mfma16(a, Dd::bop(fr, sc, st, p), D[p]);
      }
      acc = Dd::post(acc, D, xsum, sc);
    }
  };

  // The loads of rounds -max(XD, PD) .. -1 in the order those rounds would
  // issue them (activations of round q + XD, then weights of round q + PD),
  // so that the first round's waits are those of every other round.
  constexpr int kLead = XD > PD ? XD : PD;
#pragma unroll
  for (int q = -kLead; q < 0; ++q) {
    if (q + XD >= 0) issue_x(kb0 + q + XD, (q + XD) % XD);
    if (q + PD >= 0) issue_w(kb0 + q + PD, (q + PD) % NS);
  }
  // With the first loads in flight: halves of absent tokens stay zero in both
  // ring slots (the first round's barrier orders these writes before any
  // read).
  if (threadIdx.x == 0) lds[S * 2 * kFrag] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < kPerLane; ++i)
    if (xdst[i] >= 0 && !xlive[i]) {
      reinterpret_cast<u32x2 *>(ring)[xdst[i]] = u32x2{0u, 0u};
      reinterpret_cast<u32x2 *>(ring + kFrag)[xdst[i]] = u32x2{0u, 0u};
    }
  const int full = rounds - rounds % U;
  for (int r = 0; r < full; r += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) round(r + u, u);
  }
#pragma unroll
  for (int u = 0; u < U - 1; ++u)
    if (u < rounds - full) round(full + u, u);

  if constexpr (S > 1) {
    __syncthreads();  // every wave is done with the rings
    floatx4 *red = reinterpret_cast<floatx4 *>(lds);
    if (kp > 0) red[((kp - 1) * T + t) * 64 + lane] = acc;
    __syncthreads();
    if (kp > 0) return;
#pragma unroll
    for (int q = 1; q < S; ++q) acc += red[((q - 1) * T + t) * 64 + lane];
  }
  if (!owner) return;
  // Lane (j, G) holds D[token 4G + q][row j].
  const int64_t row = tile * 16 + j;
  if (row >= N) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int tok = 4 * G + q;
    if (tok < M) Y[(int64_t)(ROUTED ? order[c0 + tok] : tok) * N + row] = acc[q];
  }
}

}  // namespace gv

// Compute units of the current device (looked up once per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 1;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

namespace gv {

template <int KIND, int MT, int T, int S, int PD, int XD = 2, bool PACKED = true>
static hipError_t run_xs(const uint8_t *P, const void *x, int x_f16, float *y, int M, int64_t N, int64_t K,
                         hipStream_t s, bool spread = true) {
  const int64_t row_bytes = (K / Geometry<KIND>::elems) * Geometry<KIND>::bytes;
  constexpr int kFrag = Dec<KIND>::NSTEP * MT * 4;
  const size_t lds = std::max<size_t>((size_t)S * 2 * kFrag * 16 + 16, (size_t)(S - 1) * T * 64 * 16);
  const int64_t ntiles = (N + 15) / 16;
  const int64_t wgs = std::max<int64_t>((ntiles + T - 1) / T, spread ? std::min<int64_t>(ntiles, device_cus()) : 1);
  const int per_wg = (int)(ntiles / wgs), extra = (int)(ntiles % wgs);
  const dim3 grid((unsigned)wgs), block(64 * T * S);
  if (x_f16)
    hipLaunchKernelGGL((gemv_xs_kernel<KIND, _Float16, MT, T, S, PD, XD, false, PACKED>), grid, block, lds, s, P,
                       (const _Float16 *)x, y, M, N, (int)K, per_wg, extra, MoeRoute{}, row_bytes);
  else
    hipLaunchKernelGGL((gemv_xs_kernel<KIND, float, MT, T, S, PD, XD, false, PACKED>), grid, block, lds, s, P,
                       (const float *)x, y, M, N, (int)K, per_wg, extra, MoeRoute{}, row_bytes);
  return hipGetLastError();
}

// Grouped expert products: grid (tile groups of T, work items); T tiles
// share each staged activation k-block of the item's MT pairs.
template <int KIND, int MT, int T, int S, int PD, int XD, bool PACKED = true>
static hipError_t run_xs_routed(const uint8_t *P, const void *x, int x_f16, float *y, int64_t N, int64_t K,
                                hipStream_t s, const MoeRoute &rt, int items) {
  constexpr int kFrag = Dec<KIND>::NSTEP * MT * 4;
  const int64_t row_bytes = (K / Geometry<KIND>::elems) * Geometry<KIND>::bytes;
  const size_t lds = std::max<size_t>((size_t)S * 2 * kFrag * 16 + 16, (size_t)(S - 1) * T * 64 * 16);
  const int64_t ntiles = (N + 15) / 16;
  const dim3 grid((unsigned)((ntiles + T - 1) / T), (unsigned)items), block(64 * T * S);
  if (x_f16)
    hipLaunchKernelGGL((gemv_xs_kernel<KIND, _Float16, MT, T, S, PD, XD, true, PACKED>), grid, block, lds, s, P,
                       (const _Float16 *)x, y, MT, N, (int)K, T, 0, rt, row_bytes);
  else
    hipLaunchKernelGGL((gemv_xs_kernel<KIND, float, MT, T, S, PD, XD, true, PACKED>), grid, block, lds, s, P,
                       (const float *)x, y, MT, N, (int)K, T, 0, rt, row_bytes);
  return hipGetLastError();
}

template <int KIND, bool PACKED>
static hipError_t run_xs_routed_m(const uint8_t *P, const void *x, int x_f16, float *y, int mt, int64_t N, int64_t K,
                                  hipStream_t s, const MoeRoute &rt, int items) {
#ifdef QMM_TUNING
  static const int cfg = [] {
    const char *e = getenv("QMM_MOE_XS_CFG");
    return e ? atoi(e) : 0;
  }();
  if (mt == 16) {
    switch (cfg) {
      case 1: return run_xs_routed<KIND, 16, 4, 1, 1, 1, PACKED>(P, x, x_f16, y, N, K, s, rt, items);
      case 3: return run_xs_routed<KIND, 16, 16, 1, 1, 1, PACKED>(P, x, x_f16, y, N, K, s, rt, items);
      case 6: return run_xs_routed<KIND, 16, 8, 1, 2, 1, PACKED>(P, x, x_f16, y, N, K, s, rt, items);
      default: break;
    }
  }
#endif
  // Eight tiles per workgroup, one k-block of weights in flight (measured
  // best among 4, 8 and 16 tiles, with K split in one or two parts, at the
  // 128-expert top-8 workload with 256 tokens).
  if (mt == 8) return run_xs_routed<KIND, 8, 8, 1, 1, 1, PACKED>(P, x, x_f16, y, N, K, s, rt, items);
  return run_xs_routed<KIND, 16, 8, 1, 1, 1, PACKED>(P, x, x_f16, y, N, K, s, rt, items);
}

template <int KIND>
static hipError_t run_xs_m(const uint8_t *P, const void *x, int x_f16, float *y, int M, int64_t N, int64_t K,
                           hipStream_t s, int cfg) {
#ifdef QMM_TUNING
  switch (cfg) {
    case 101: return run_xs<KIND, 8, 4, 2, 2, 1>(P, x, x_f16, y, M, N, K, s);
    case 102: return run_xs<KIND, 8, 4, 2, 2, 2>(P, x, x_f16, y, M, N, K, s);
    case 103: return run_xs<KIND, 8, 4, 2, 1, 2>(P, x, x_f16, y, M, N, K, s);
    case 104: return run_xs<KIND, 8, 4, 2, 3, 2>(P, x, x_f16, y, M, N, K, s);
    case 105: return run_xs<KIND, 8, 4, 1, 2, 2>(P, x, x_f16, y, M, N, K, s);
    case 106: return run_xs<KIND, 8, 2, 2, 2, 2>(P, x, x_f16, y, M, N, K, s);
    case 107: return run_xs<KIND, 8, 2, 2, 3, 2>(P, x, x_f16, y, M, N, K, s);
    case 108: return run_xs<KIND, 8, 4, 4, 2, 2>(P, x, x_f16, y, M, N, K, s);
    case 109: return run_xs<KIND, 8, 8, 1, 2, 2>(P, x, x_f16, y, M, N, K, s);
    case 110: return run_xs<KIND, 8, 8, 2, 2, 2>(P, x, x_f16, y, M, N, K, s);
    case 111: return run_xs<KIND, 8, 2, 4, 2, 2>(P, x, x_f16, y, M, N, K, s);
    case 112: return run_xs<KIND, 8, 4, 2, 1, 1>(P, x, x_f16, y, M, N, K, s);
    case 113: return run_xs<KIND, 8, 4, 2, 1, 1>(P, x, x_f16, y, M, N, K, s, false);
    case 114: return run_xs<KIND, 8, 4, 2, 2, 1>(P, x, x_f16, y, M, N, K, s);
    case 115: return run_xs<KIND, 8, 4, 2, 1, 2>(P, x, x_f16, y, M, N, K, s);
    case 116: return run_xs<KIND, 8, 2, 2, 1, 1>(P, x, x_f16, y, M, N, K, s);
    case 117: return run_xs<KIND, 8, 2, 4, 1, 1>(P, x, x_f16, y, M, N, K, s);
    case 118: return run_xs<KIND, 8, 4, 1, 1, 1>(P, x, x_f16, y, M, N, K, s);
    case 119: return run_xs<KIND, 8, 8, 1, 1, 1>(P, x, x_f16, y, M, N, K, s);
    case 120: return run_xs<KIND, 8, 8, 2, 1, 1>(P, x, x_f16, y, M, N, K, s);
    default: break;
  }
#else
  (void)cfg;
#endif
  if (M <= 2) return run_xs<KIND, 2, 4, 2, 1, 1>(P, x, x_f16, y, M, N, K, s);
  if (M <= 4) return run_xs<KIND, 4, 4, 2, 1, 1>(P, x, x_f16, y, M, N, K, s);
  return run_xs<KIND, 8, 4, 2, 1, 1>(P, x, x_f16, y, M, N, K, s);
}

}  // namespace gv

bool xs_native_supported(int kind) {
  return kind == Q4_K || kind == Q6_K || kind == Q5_K || kind == Q2_K || kind == Q3_K;
}

hipError_t launch_moe_xs(int kind, const uint8_t *P, const void *X, int x_f16, float *Y, int mt, int64_t N,
                         int64_t K, const MoeRoute &rt, int items, hipStream_t s, bool packed) {
  if (!packed) {
    switch (kind) {
#define QMM_CASE(K_) \
  case K_: return gv::run_xs_routed_m<K_, false>(P, X, x_f16, Y, mt, N, K, s, rt, items);
      QMM_CASE(Q4_K) QMM_CASE(Q6_K) QMM_CASE(Q2_K) QMM_CASE(Q3_K) QMM_CASE(Q5_K)
#undef QMM_CASE
      default: return hipErrorNotSupported;
    }
  }
  switch (kind) {
#define QMM_CASE(K_) \
  case K_: return gv::run_xs_routed_m<K_, true>(P, X, x_f16, Y, mt, N, K, s, rt, items);
    QMM_CASE(Q4_K) QMM_CASE(Q6_K) QMM_CASE(IQ4_XS) QMM_CASE(Q4_0) QMM_CASE(Q5_0) QMM_CASE(Q8_0) QMM_CASE(IQ4_NL)
    QMM_CASE(MXFP4) QMM_CASE(Q2_K) QMM_CASE(Q3_K) QMM_CASE(Q5_K)
#undef QMM_CASE
    default: break;
  }
  return hipErrorNotSupported;
}

// 2 to 8 tokens over native rows (the super-block kinds).
hipError_t launch_gemv_xs_native(int kind, const uint8_t *W, const void *x, int x_f16, float *y, int M, int64_t N,
                                 int64_t K, hipStream_t s) {
  switch (kind) {
#define QMM_CASE(K_)                                                                         \
  case K_:                                                                                   \
    if (M <= 2) return gv::run_xs<K_, 2, 4, 2, 1, 1, false>(W, x, x_f16, y, M, N, K, s);     \
    if (M <= 4) return gv::run_xs<K_, 4, 4, 2, 1, 1, false>(W, x, x_f16, y, M, N, K, s);     \
    return gv::run_xs<K_, 8, 4, 2, 1, 1, false>(W, x, x_f16, y, M, N, K, s);
    QMM_CASE(Q4_K) QMM_CASE(Q6_K) QMM_CASE(Q2_K) QMM_CASE(Q3_K) QMM_CASE(Q5_K)
#undef QMM_CASE
    default: break;
  }
  return hipErrorNotSupported;
}

hipError_t launch_gemv_xs(int kind, const uint8_t *P, const void *x, int x_f16, float *y, int M, int64_t N,
                          int64_t K, hipStream_t s, int cfg) {
  switch (kind) {
    case Q4_K: return gv::run_xs_m<Q4_K>(P, x, x_f16, y, M, N, K, s, cfg);
    case Q6_K: return gv::run_xs_m<Q6_K>(P, x, x_f16, y, M, N, K, s, cfg);
    case IQ4_XS: return gv::run_xs_m<IQ4_XS>(P, x, x_f16, y, M, N, K, s, cfg);
    case Q4_0: return gv::run_xs_m<Q4_0>(P, x, x_f16, y, M, N, K, s, cfg);
    case Q5_0: return gv::run_xs_m<Q5_0>(P, x, x_f16, y, M, N, K, s, cfg);
    case Q8_0: return gv::run_xs_m<Q8_0>(P, x, x_f16, y, M, N, K, s, cfg);
    case IQ4_NL: return gv::run_xs_m<IQ4_NL>(P, x, x_f16, y, M, N, K, s, cfg);
    case MXFP4: return gv::run_xs_m<MXFP4>(P, x, x_f16, y, M, N, K, s, cfg);
    case Q2_K: return gv::run_xs_m<Q2_K>(P, x, x_f16, y, M, N, K, s, cfg);
    case Q3_K: return gv::run_xs_m<Q3_K>(P, x, x_f16, y, M, N, K, s, cfg);
    case Q5_K: return gv::run_xs_m<Q5_K>(P, x, x_f16, y, M, N, K, s, cfg);
    default: break;
  }
  return hipErrorNotSupported;
}

}  // namespace qmm
