// qmm_gemv_t1.hip -- the single-token decode GEMV: the super-block kinds
// over repacked records or native GGUF rows, the step-scaled kinds over
// records, and its routed form for expert products of one pair per
// workgroup.
//
// Rows of A as sub-block selectors.  With one token, 15 of the 16 A rows of
// v_mfma_f32_16x16x32_f16 would hold zeros.  Here, at each MFMA step, lane
// group G's 8 activations go into the A row of the sub-block that group's
// weights belong to at that step (every other row of that group's columns
// is zero), so row r of D collects one sub-block's partial dot product and
// nothing else.  The sub-block scales and minimums are then applied to D in
// f32 once per k-block, instead of being folded into every B element:
//
//   Q4_K  B holds each raw 4-bit code as an f16 subnormal: the nibble masked
//         into the low mantissa bits is q * 2^-24 (a high nibble left in
//         place, 16q * 2^-24), one AND per two codes.  D rows 4G and 4G + 1
//         are sub-blocks 2G and 2G + 1 of lane group G (low and high
//         nibbles), later scaled by d * sc * 2^24 (2^20).  The sums of the
//         activations per sub-block, for the minimum term, come from the
//         same A against a B of ones.
//   Q6_K  B holds q - 32 exactly (the 6-bit code under the f16 1024 offset,
//         removed by one packed add or fma).  D row 8h + 2g + a is sub-block
//         8h + 2g + a (half h, quarter g, byte lane a of the decoder in
//         qmm_gemv_mfma.h), later scaled by d * sc.
//
// Every product is exact in f32 (an f16 activation times a small integer, or
// times a small integer times 2^-24) and the MFMA accumulates in f32, so the
// error bound of the folded decoders holds unchanged: the activations rounded
// once to f16, then f32 sums.
//
// (The decoders themselves are in qmm_gemv_t1.h.)  Work split and pipeline
// as the single-token shapes of qmm_gemv_mfma.hip: a workgroup of S waves
// owns one 16-row tile and wave w takes k-blocks
// [w * n / S, (w + 1) * n / S) with PD k-blocks in flight; every load is
// issued on every path (clamped past the wave's last k-block), so no wait is
// widened by a branch.
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "qmm_gemv_mfma.h"
#include "qmm_gemv_t1.h"
#include "qmm_internal.h"

namespace qmm {
namespace gv {

// PACKED: W holds repacked records (otherwise native GGUF rows of row_bytes
// bytes).  ROUTED: workgroup (tile, i) serves pair i of an expert product
// (one pair per workgroup): expert ids[i] (pairs with an id outside [0, E)
// are skipped), activations row x_per_slot ? i : i / topk, output row i.
template <int KIND, typename XT, int S, int PD, int OCC, bool PACKED, bool ROUTED>
__global__ __launch_bounds__(64 * S) __attribute__((amdgpu_waves_per_eu(OCC, 8))) void gemv_t1_kernel(
    const uint8_t *__restrict__ W, int64_t row_bytes, const XT *__restrict__ X, float *__restrict__ Y, int64_t N,
    int K, MoeRoute rt) {
  using Tr = T1<KIND>;
  using Dd = typename Tr::Dd;
  using Raw = typename Tr::Raw;
  using X4 = typename XVec<XT>::type;
  static_assert(PACKED || !Dd::CHUNKED, "native rows: decoders with direct field loads only");
  using Held = typename std::conditional<PACKED, typename Rec<KIND>::Packed, Raw>::type;
  constexpr int kFrag = Dd::NSTEP * 4;  // 16-byte fragments of one k-block (step s, group G at 4s + G)
  constexpr int NS = PD + 1;
  constexpr int64_t kRec = 16 * Dd::BYTES;
  // LDS per wave: kFrag zero fragments (read by lanes whose A row is empty)
  // and a ring of NS k-blocks; later the reduction.
  extern __shared__ u32x4 lds[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = lane & 15, G = lane >> 4;
  const int64_t tile = blockIdx.x;
  const int nkb = K / Dd::KB;
  if constexpr (ROUTED) {
    const int pair = blockIdx.y;
    const int e = pair < rt.pairs ? rt.ids[pair] : -1;
    if (e < 0 || e >= rt.E) return;  // the whole workgroup, before any barrier
    W += (int64_t)e * (PACKED ? (N + 15) / 16 * nkb * kRec : N * row_bytes);
    X += (int64_t)(rt.x_per_slot ? pair : pair / rt.topk) * K;
    Y += (int64_t)pair * N;
  }
  const int kb0 = (int)((int64_t)wave * nkb / S), kb1 = (int)((int64_t)(wave + 1) * nkb / S);
  const int kb_last = max(kb1 - 1, 0);
  u32x4 *zrun = lds + wave * (NS + 1) * kFrag, *ring = zrun + kFrag;

  // Lane h = lane converts elements x_off(s, G', h & 1) + [0, 4) of the
  // k-block: fragment f = h / 2 = 4s + G', half h & 1.
  const int xoff = Dd::x_off(lane >> 3, (lane >> 1) & 3, lane & 1);
  // A fragment base of selector group c in slot d: this lane's fragment run
  // if its row is that group's A row, else the zero run.
  const u32x4 *abase[NS][Tr::NSEL];
#pragma unroll
  for (int d = 0; d < NS; ++d)
#pragma unroll
    for (int c = 0; c < Tr::NSEL; ++c) abase[d][c] = (j == Tr::arow(c, G) ? ring + d * kFrag : zrun) + G;

  // Records of this tile, or row j of it (rows past N decode the last row;
  // their outputs are not stored).
  const uint8_t *wt = PACKED ? W + tile * nkb * kRec : W + min(tile * 16 + j, N - 1) * row_bytes;
  Held raw[NS];
  X4 xv[NS];
  auto issue = [&](int kb, int slot) {
    kb = min(kb, kb_last);
    __builtin_memcpy(&xv[slot], X + xoff + (int64_t)kb * Dd::KB, sizeof(X4));
    if constexpr (PACKED) Rec<KIND>::load(wt + kb * kRec, lane, j, G, raw[slot]);
    else Dd::load(wt + (int64_t)kb * Dd::BYTES, G, raw[slot]);
  };
  float acc = 0.0f;
  const half8 ones = {1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16};
  auto consume = [&](int d) {
    {
      const X4 v = xv[d];
      const half2v p0 = {(_Float16)v[0], (_Float16)v[2]}, p1 = {(_Float16)v[1], (_Float16)v[3]};
      reinterpret_cast<u32x2 *>(ring + d * kFrag)[lane] = u32x2{as_u(p0), as_u(p1)};
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    Raw fr;
    if constexpr (PACKED) fr = Rec<KIND>::unpack(raw[d], G);
    else fr = raw[d];
    const typename Tr::Sc sc = Tr::prep(fr, G);
    floatx4 D = {0.f, 0.f, 0.f, 0.f}, Xs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < Dd::NSTEP; ++st) {
      const half8 a = __builtin_bit_cast(half8, abase[d][Tr::sel_of_step(st)][4 * st]);
      if constexpr (Tr::HAS_MIN) Xs = mfma16(a, ones, Xs);
      D = mfma16(a, Tr::bop(fr, sc, st), D);
    }
    acc = Tr::post(acc, D, Xs, sc);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // slot d is rewritten NS k-blocks later
  };

#pragma unroll
  for (int d = 0; d < PD; ++d) issue(kb0 + d, d);
  // With the first loads in flight: this wave's zero run (the wave barrier
  // in the first consume orders it before any read).
  if (lane < kFrag) zrun[lane] = u32x4{0u, 0u, 0u, 0u};
  const int cnt = max(kb1 - kb0, 0), full = cnt - cnt % NS;
  for (int i = 0; i < full; i += NS) {
#pragma unroll
    for (int d = 0; d < NS; ++d) {
      issue(kb0 + i + d + PD, (d + PD) % NS);
      consume(d);
    }
  }
#pragma unroll
  for (int d = 0; d < NS - 1; ++d)
    if (d < cnt - full) consume(d);

  // Row j's sum is spread over the four lane groups, then over the S waves.
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  if constexpr (S > 1) {
    __syncthreads();  // every wave is done with its ring
    float *red = reinterpret_cast<float *>(lds);
    if (wave > 0 && lane < 16) red[(wave - 1) * 16 + lane] = acc;
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < S - 1; ++w) acc += red[w * 16 + (lane & 15)];
  }
  const int64_t row = tile * 16 + j;
  if (lane < 16 && row < N) Y[row] = acc;
}

template <int KIND, int S, int PD, int OCC = 1, bool PACKED = true, bool ROUTED = false>
static hipError_t run_t1(const uint8_t *W, const void *x, int x_f16, float *y, int64_t N, int64_t K, hipStream_t s,
                         const MoeRoute &rt = MoeRoute{}, int items = 1) {
  constexpr int kFrag = T1<KIND>::Dd::NSTEP * 4;
  const size_t lds = std::max<size_t>((size_t)S * (PD + 2) * kFrag * 16, (size_t)(S - 1) * 16 * 4);
  const int64_t row_bytes = (K / Geometry<KIND>::elems) * Geometry<KIND>::bytes;
  // Tile-major grid: workgroup i runs on XCD i mod 8, and the pairs of one
  // tile (a multiple of 8 apart when the tile count is) share its L2.
  const dim3 grid((unsigned)((N + 15) / 16), (unsigned)items), block(64 * S);
  if (x_f16)
    hipLaunchKernelGGL((gemv_t1_kernel<KIND, _Float16, S, PD, OCC, PACKED, ROUTED>), grid, block, lds, s, W,
                       row_bytes, (const _Float16 *)x, y, N, (int)K, rt);
  else
    hipLaunchKernelGGL((gemv_t1_kernel<KIND, float, S, PD, OCC, PACKED, ROUTED>), grid, block, lds, s, W, row_bytes,
                       (const float *)x, y, N, (int)K, rt);
  return hipGetLastError();
}

template <int KIND, bool PACKED>
static hipError_t run_t1_k(const uint8_t *P, const void *x, int x_f16, float *y, int64_t N, int64_t K, hipStream_t s,
                           int cfg) {
#ifdef QMM_TUNING
  switch (cfg) {
    case 201: return run_t1<KIND, 4, 1, 4, PACKED>(P, x, x_f16, y, N, K, s);
    case 202: return run_t1<KIND, 4, 1, 1, PACKED>(P, x, x_f16, y, N, K, s);
    case 203: return run_t1<KIND, 4, 2, 1, PACKED>(P, x, x_f16, y, N, K, s);
    case 204: return run_t1<KIND, 2, 1, 1, PACKED>(P, x, x_f16, y, N, K, s);
    case 205: return run_t1<KIND, 2, 2, 1, PACKED>(P, x, x_f16, y, N, K, s);
    case 206: return run_t1<KIND, 2, 3, 1, PACKED>(P, x, x_f16, y, N, K, s);
    case 207: return run_t1<KIND, 8, 1, 1, PACKED>(P, x, x_f16, y, N, K, s);
    case 208: return run_t1<KIND, 8, 2, 1, PACKED>(P, x, x_f16, y, N, K, s);
    case 209: return run_t1<KIND, 4, 3, 1, PACKED>(P, x, x_f16, y, N, K, s);
    case 210: return run_t1<KIND, 1, 3, 1, PACKED>(P, x, x_f16, y, N, K, s);
    case 211: return run_t1<KIND, 4, 2, 3, PACKED>(P, x, x_f16, y, N, K, s);
    case 212: return run_t1<KIND, 16, 1, 1, PACKED>(P, x, x_f16, y, N, K, s);
    default: break;
  }
#else
  (void)cfg;
#endif
  if constexpr (Dec<KIND>::STEP_SCALE) {
    // The step-scaled kinds (records only) decode with more VALU per byte:
    // more waves per tile, one k-block in flight each; MXFP4 at four waves
    // held to 128 registers (measured over 1 to 16 waves and 1 to 2 k-blocks
    // in flight at 4096 x 4096 and 11008 x 4096).
    if (N <= 4096) return run_t1<KIND, 16, 1, 1, true>(P, x, x_f16, y, N, K, s);
    if constexpr (KIND == MXFP4) return run_t1<KIND, 4, 1, 4, true>(P, x, x_f16, y, N, K, s);
    return run_t1<KIND, 8, 1, 1, true>(P, x, x_f16, y, N, K, s);
  } else {
    // Two waves per tile (measured best for Q4_K and Q6_K at 14336 x 4096
    // among 1 to 16 waves and 1 to 3 k-blocks in flight): one k-block in
    // flight over records, two over native rows (whose per-lane field loads
    // are slower to land; Q4_K 12.0 -> 11.0 us, Q6_K 20.2 -> 18.0 us).
    if constexpr (!PACKED) return run_t1<KIND, 2, 2, 1, false>(P, x, x_f16, y, N, K, s);
    return run_t1<KIND, 2, 1, 1, true>(P, x, x_f16, y, N, K, s);
  }
}

// Routed pairs: K of three k-blocks (an expert down matrix of 768 columns)
// takes three waves of one k-block each, else the shapes above.
template <int KIND, bool PACKED>
static hipError_t run_t1_routed(const uint8_t *W, const void *x, int x_f16, float *y, int64_t N, int64_t K,
                                hipStream_t s, const MoeRoute &rt, int items) {
  if (K == 3 * T1<KIND>::Dd::KB) return run_t1<KIND, 3, 1, 1, PACKED, true>(W, x, x_f16, y, N, K, s, rt, items);
  return run_t1<KIND, 2, PACKED ? 1 : 2, 1, PACKED, true>(W, x, x_f16, y, N, K, s, rt, items);
}

}  // namespace gv

// Over native rows only the super-block kinds: the step-scaled kinds read
// native rows through an LDS staging (the matrix-core GEMV's), with which
// this kernel measured no faster (Q4_0, IQ4_NL, IQ4_XS) or slower (MXFP4
// 15.4 -> 17.3 us at 11008 x 4096).
bool gemv_t1_supported(int kind, bool packed) {
  switch (kind) {
    case Q4_K: case Q6_K: case Q5_K: case Q2_K: case Q3_K: return true;
    case Q4_0: case Q5_0: case Q8_0: case IQ4_NL: case MXFP4: case IQ4_XS: return packed;
    default: return false;
  }
}

hipError_t launch_gemv_t1(int kind, const uint8_t *W, const void *x, int x_f16, float *y, int64_t N, int64_t K,
                          hipStream_t s, int cfg, bool packed) {
  if (!gemv_t1_supported(kind, packed)) return hipErrorNotSupported;
  switch (kind) {
    case Q4_K: return packed ? gv::run_t1_k<Q4_K, true>(W, x, x_f16, y, N, K, s, cfg)
                             : gv::run_t1_k<Q4_K, false>(W, x, x_f16, y, N, K, s, cfg);
    case Q6_K: return packed ? gv::run_t1_k<Q6_K, true>(W, x, x_f16, y, N, K, s, cfg)
                             : gv::run_t1_k<Q6_K, false>(W, x, x_f16, y, N, K, s, cfg);
    case Q5_K: return packed ? gv::run_t1_k<Q5_K, true>(W, x, x_f16, y, N, K, s, cfg)
                             : gv::run_t1_k<Q5_K, false>(W, x, x_f16, y, N, K, s, cfg);
    case Q2_K: return packed ? gv::run_t1_k<Q2_K, true>(W, x, x_f16, y, N, K, s, cfg)
                             : gv::run_t1_k<Q2_K, false>(W, x, x_f16, y, N, K, s, cfg);
    case Q3_K: return packed ? gv::run_t1_k<Q3_K, true>(W, x, x_f16, y, N, K, s, cfg)
                             : gv::run_t1_k<Q3_K, false>(W, x, x_f16, y, N, K, s, cfg);
#define QMM_CASE(K_) \
  case K_: return gv::run_t1_k<K_, true>(W, x, x_f16, y, N, K, s, cfg);
    QMM_CASE(Q4_0) QMM_CASE(Q5_0) QMM_CASE(Q8_0) QMM_CASE(IQ4_NL) QMM_CASE(MXFP4) QMM_CASE(IQ4_XS)
#undef QMM_CASE
    default: break;
  }
  return hipErrorNotSupported;
}

hipError_t launch_moe_t1(int kind, const uint8_t *W, const void *X, int x_f16, float *Y, int64_t N, int64_t K,
                         const MoeRoute &rt, int items, hipStream_t s, bool packed) {
  if (!gemv_t1_supported(kind, packed)) return hipErrorNotSupported;
  switch (kind) {
    case Q4_K: return packed ? gv::run_t1_routed<Q4_K, true>(W, X, x_f16, Y, N, K, s, rt, items)
                             : gv::run_t1_routed<Q4_K, false>(W, X, x_f16, Y, N, K, s, rt, items);
    case Q6_K: return packed ? gv::run_t1_routed<Q6_K, true>(W, X, x_f16, Y, N, K, s, rt, items)
                             : gv::run_t1_routed<Q6_K, false>(W, X, x_f16, Y, N, K, s, rt, items);
    case Q5_K: return packed ? gv::run_t1_routed<Q5_K, true>(W, X, x_f16, Y, N, K, s, rt, items)
                             : gv::run_t1_routed<Q5_K, false>(W, X, x_f16, Y, N, K, s, rt, items);
    case Q2_K: return packed ? gv::run_t1_routed<Q2_K, true>(W, X, x_f16, Y, N, K, s, rt, items)
                             : gv::run_t1_routed<Q2_K, false>(W, X, x_f16, Y, N, K, s, rt, items);
    case Q3_K: return packed ? gv::run_t1_routed<Q3_K, true>(W, X, x_f16, Y, N, K, s, rt, items)
                             : gv::run_t1_routed<Q3_K, false>(W, X, x_f16, Y, N, K, s, rt, items);
#define QMM_CASE(K_) \
  case K_: return gv::run_t1_routed<K_, true>(W, X, x_f16, Y, N, K, s, rt, items);
    QMM_CASE(Q4_0) QMM_CASE(Q5_0) QMM_CASE(Q8_0) QMM_CASE(IQ4_NL) QMM_CASE(MXFP4) QMM_CASE(IQ4_XS)
#undef QMM_CASE
    default: break;
  }
  return hipErrorNotSupported;
}

}  // namespace qmm
