// qmm_moe_ffn.hip -- routed SiLU-gated expert FFN with a weighted top-k
// combine.
//
// For token t and slot s with e = ids[t][s] in [0, E):
//   gate, up = rows [0, N_ff) and [N_ff, 2 N_ff) of W_gu[e] times X[t]
//   h        = silu(gate) * up                       (f32)
//   d        = W_d[e] . h                            (the slot's down output)
//   Y[t]     = sum over valid slots of topk_w[t][s] * d
//
// Two launches when experts see about one pair each (fewer than four pairs
// per expert on average; pairs are then not worth grouping by expert), the
// kind decodes on the matrix cores over the given layout, and N_ff and K
// are whole numbers of 256-element k-blocks:
//   1. gate/up: one workgroup per (pair, 16-row tile of h).  It decodes the
//      gate tile and the matching up tile of the pair's expert against the
//      pair's token, applies silu(gate) * up in its epilogue, and writes the
//      16 values of h and their largest magnitude (f32).
//   2. down + combine: one workgroup per (token, 16-row tile of Y).  It
//      walks the token's slots and the k-blocks of each (the pairs (slot,
//      k-block) split over its waves in a fixed order), multiplies each
//      slot's h by that slot's down tile and adds topk_w[t][s] times the
//      result, then writes Y's 16 values.  No per-slot outputs exist.
// Otherwise four stream-ordered launches: the routed gate/up product, the
// SiLU-product, the routed down product (per-slot activations) and the
// combine.  Their routed launches group pairs by expert, so each touched
// expert's weights stream once per work item, and share one routing pass.
//
// The matrix-core products take their activations as f16, whose range ends
// at 65504, and h can exceed that (large gate and up outputs multiply).
// Each pair's h is therefore divided by 2^k, the smallest power of two
// (k >= 0) that brings max |h| to 2^14 or below, and the down output of that
// pair is multiplied by 2^k again: both steps are exact.
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "qmm_device.h"
#include "qmm_gemv_mfma.h"
#include "qmm_gemv_t1.h"
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


// ---------------------------------------------------------------------------
// The two-launch path.  Both kernels are single-token matrix-core GEMVs
// (one A row carries the token, the decoders of qmm_gemv_mfma.h supply exact
// f16 B operands) whose waves walk a fixed list of units with PD units of
// loads in flight, issued on every path (clamped), as the decode GEMV does.
// ---------------------------------------------------------------------------
namespace fz {
using gv::Dec;
using gv::half8;
using gv::half2v;
using gv::u32x2;
using gv::u32x4;
using Fx4 = gv::floatx4;

// One tile's k-block as loaded: the repacked record's fields, or the
// decoder's fields of a native row.
template <int KIND, bool PACKED>
struct HeldOf {
  using type = typename Dec<KIND>::Raw;
};
template <int KIND>
struct HeldOf<KIND, true> {
  using type = typename gv::Rec<KIND>::Packed;
};
template <int KIND, bool PACKED>
using Held = typename HeldOf<KIND, PACKED>::type;

// Where a tile's k-block lives: expert base W, tile (16 rows) `tile` of an
// expert with `rows` rows, k-block kb; lane (j, G).
template <int KIND, bool PACKED>
struct Tiles {
  const uint8_t *W;
  int64_t expert_bytes, row_bytes;
  int rows, nkb;
  __device__ void load(int e, int tile, int kb, int lane, int j, int G, Held<KIND, PACKED> &h) const {
    const uint8_t *base = W + (int64_t)e * expert_bytes;
    if constexpr (PACKED) {
      constexpr int64_t kRec = 16 * Dec<KIND>::BYTES;
      gv::Rec<KIND>::load(base + ((int64_t)tile * nkb + kb) * kRec, lane, j, G, h);
    } else {
      Dec<KIND>::load(base + ((int64_t)tile * 16 + j) * row_bytes + (int64_t)kb * Dec<KIND>::BYTES, G, h);
    }
  }
  __device__ static typename Dec<KIND>::Raw raw(const Held<KIND, PACKED> &h, int G) {
    if constexpr (PACKED) return gv::Rec<KIND>::unpack(h, G);
    else return h;
  }
};

// One k-block of one token's activations (this lane's four elements) into
// the single-token fragment layout of LDS slot xk: fragment 4s + G', half
// order (0, 2), (1, 3); then the wave reads them back.
template <typename X4>
__device__ __forceinline__ void stage_x(u32x4 *xk, int lane, X4 v, float scale) {
  const half2v p0 = {(_Float16)(v[0] * scale), (_Float16)(v[2] * scale)};
  const half2v p1 = {(_Float16)(v[1] * scale), (_Float16)(v[3] * scale)};
  reinterpret_cast<u32x2 *>(xk)[lane] = u32x2{gv::as_u(p0), gv::as_u(p1)};
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Products of one k-block for tile raws r[0 .. R): D lane (j, G) q = 0 of
// lanes G = 0 is row j's partial dot product; xr is this lane's A fragment
// run (the token's fragments for lanes j = 0, zeros otherwise).
template <int KIND, int R>
__device__ __forceinline__ void kblock(const typename Dec<KIND>::Raw (&fr)[R], const u32x4 *xr, int xstep, int G,
                                       int j, Fx4 (&acc)[R], float weight) {
  using Dd = Dec<KIND>;
  half8 a[Dd::NSTEP];
  Fx4 xsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < Dd::NSTEP; ++st) {
    a[st] = __builtin_bit_cast(half8, xr[st * xstep]);
    if constexpr (Dd::HAS_MIN) {
      const _Float16 v = Dd::ind(st, G, j) ? (_Float16)1.0f : (_Float16)0.0f;
      xsum = gv::mfma16(half8{v, v, v, v, v, v, v, v}, a[st], xsum);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const typename Dd::Sc sc = Dd::prep(fr[r], G);
    Fx4 c = {0.f, 0.f, 0.f, 0.f};
    if constexpr (Dd::STEP_SCALE) {
#pragma unroll
      for (int st = 0; st < Dd::NSTEP; ++st)
        c = Dd::post_step(c, gv::mfma16(a[st], Dd::bop(fr[r], sc, st, 0), Fx4{0.f, 0.f, 0.f, 0.f}), fr[r], st);
    } else {
      Fx4 D[Dd::NPART];
#pragma unroll
      for (int p = 0; p < Dd::NPART; ++p) D[p] = Fx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < Dd::NSTEP; ++st)
#pragma unroll
        for (int p = 0; p < Dd::NPART; ++p) D[p] = gv::mfma16(a[st], Dd::bop(fr[r], sc, st, p), D[p]);
      c = Dd::post(c, D, xsum, sc);
    }
    acc[r] += weight * c;
  }
}

// The super-block kinds take the single-token decoders of qmm_gemv_t1.h: the
// A rows select sub-blocks, the B operands carry no scales, and the scales
// are applied to D once per k-block.
template <int KIND>
constexpr bool kT1 = KIND == Q4_K || KIND == Q6_K || KIND == Q5_K || KIND == Q2_K || KIND == Q3_K;
// Selector groups of those decoders (1 for the other kinds: unused).
template <int KIND, bool = kT1<KIND>>
struct Nsel {
  static constexpr int value = 1;
};
template <int KIND>
struct Nsel<KIND, true> {
  static constexpr int value = gv::T1<KIND>::NSEL;
};

// One k-block of tile raws r[0 .. R) with those decoders.  abase[c] is this
// lane's fragment run for selector group c (its own run where its row is that
// group's A row, the zero run elsewhere); acc[r] gathers this lane's share of
// row j's dot product (the four lane groups' shares add up to it).
template <int KIND, int R>
__device__ __forceinline__ void kblock_t1(const typename Dec<KIND>::Raw (&fr)[R],
                                          const u32x4 *const (&abase)[gv::T1<KIND>::NSEL], int G, float (&acc)[R],
                                          float weight) {
  using Tr = gv::T1<KIND>;
  using Dd = Dec<KIND>;
  const half8 ones = {1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16};
  Fx4 xs = {0.f, 0.f, 0.f, 0.f}, D[R];
  typename Tr::Sc sc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    D[r] = Fx4{0.f, 0.f, 0.f, 0.f};
    sc[r] = Tr::prep(fr[r], G);
  }
#pragma unroll
  for (int st = 0; st < Dd::NSTEP; ++st) {
    const half8 a = __builtin_bit_cast(half8, abase[Tr::sel_of_step(st)][4 * st]);
    if constexpr (Tr::HAS_MIN) xs = gv::mfma16(a, ones, xs);
#pragma unroll
    for (int r = 0; r < R; ++r) D[r] = gv::mfma16(a, Tr::bop(fr[r], sc[r], st), D[r]);
  }
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] += weight * Tr::post(0.f, D[r], xs, sc[r]);
}

// Launch 1.  Workgroup (t, p): pair p's gate tile t and up tile t + n_ff/16
// of expert ids[p], against token p / topk; S waves split the k-blocks.
template <int KIND, typename XT, int S, int PD, bool PACKED>
__global__ __launch_bounds__(64 * S) void gu_kernel(Tiles<KIND, PACKED> W, int E, const int32_t *__restrict__ ids,
                                                   int topk, const XT *__restrict__ X, int K, int n_ff,
                                                   float *__restrict__ H, float *__restrict__ Hmax) {
  using Dd = Dec<KIND>;
  using X4 = typename gv::XVec<XT>::type;
  constexpr int kFrag = Dd::NSTEP * 4, NS = PD + 1;
  extern __shared__ u32x4 lds[];  // zero fragment run, S rings of NS k-blocks; later the reduction
  const int p = blockIdx.y, t = blockIdx.x;
  const int e = ids[p];
  if (e < 0 || e >= E) return;  // the whole workgroup, before any barrier
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = lane & 15, G = lane >> 4;
  const int nkb = K / Dd::KB;
  const int kb0 = (int)((int64_t)wave * nkb / S), kb1 = (int)((int64_t)(wave + 1) * nkb / S);
  const int kb_last = max(kb1 - 1, 0);
  const int tiles[2] = {t, t + n_ff / 16};
  u32x4 *zrun = lds + wave * (NS + 1) * kFrag, *ring = zrun + kFrag;
  const XT *xt = X + (int64_t)(p / topk) * K + Dd::x_off(lane >> 3, (lane >> 1) & 3, lane & 1);
  Held<KIND, PACKED> raw[NS][2];
  X4 xv[NS];
  auto issue = [&](int kb, int slot) {
    kb = min(kb, kb_last);
    __builtin_memcpy(&xv[slot], xt + (int64_t)kb * Dd::KB, sizeof(X4));
#pragma unroll
    for (int r = 0; r < 2; ++r) W.load(e, tiles[r], kb, lane, j, G, raw[slot][r]);
  };
  Fx4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  float acc1[2] = {0.f, 0.f};  // the single-token decoders' per-lane shares
  const u32x4 *xbase[NS];
#pragma unroll
  for (int d = 0; d < NS; ++d) xbase[d] = (j == 0 ? ring + d * kFrag : zrun) + G;
  const int xstep = j == 0 ? 4 : 0;
  constexpr int NSEL = Nsel<KIND>::value;
  const u32x4 *abase[NS][NSEL];
  if constexpr (kT1<KIND>) {
#pragma unroll
    for (int d = 0; d < NS; ++d)
#pragma unroll
      for (int c = 0; c < NSEL; ++c) abase[d][c] = (j == gv::T1<KIND>::arow(c, G) ? ring + d * kFrag : zrun) + G;
  }
  auto consume = [&](int d) {
    stage_x(ring + d * kFrag, lane, xv[d], 1.0f);
    typename Dd::Raw fr[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) fr[r] = Tiles<KIND, PACKED>::raw(raw[d][r], G);
    if constexpr (kT1<KIND>) kblock_t1<KIND, 2>(fr, abase[d], G, acc1, 1.0f);
    else kblock<KIND, 2>(fr, xbase[d], xstep, G, j, acc, 1.0f);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // slot d is rewritten NS k-blocks later
  };
#pragma unroll
  for (int d = 0; d < PD; ++d) issue(kb0 + d, d);
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

  // Row j of the gate and up tiles in lanes 0 .. 15 (token row 0 of D, or
  // the sum of the four lane groups' shares).
  float v[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if constexpr (kT1<KIND>) {
      v[r] = acc1[r] + __shfl_xor(acc1[r], 16);
      v[r] += __shfl_xor(v[r], 32);
    } else {
      v[r] = acc[r][0];
    }
  }
  if constexpr (S > 1) {
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds);
    if (wave > 0 && lane < 16) {
      red[((wave - 1) * 2 + 0) * 16 + lane] = v[0];
      red[((wave - 1) * 2 + 1) * 16 + lane] = v[1];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < S - 1; ++w) {
      v[0] += red[(w * 2 + 0) * 16 + (lane & 15)];
      v[1] += red[(w * 2 + 1) * 16 + (lane & 15)];
    }
  }
  const float g = v[0], u = v[1];
  const float h = g / (1.0f + expf(-g)) * u;
  float m = lane < 16 ? fabsf(h) : 0.f;
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if (lane < 16) H[(int64_t)p * n_ff + 16 * t + j] = h;
  if (lane == 0) Hmax[(int64_t)p * (n_ff / 16) + t] = m;
}

// Launch 2.  Workgroup (c, t): row tile c of Y[t], the sum over slots s and
// k-blocks kb of topk_w[t][s] * 2^k_s * (down tile c of expert e_s, k-block
// kb) . (h_s / 2^k_s), h_s the pair's h; S waves split the (s, kb) units in
// order.  Slots past 64 are not supported (the caller checks topk <= 64).
template <int KIND, int S, int PD, bool PACKED>
__global__ __launch_bounds__(64 * S) void down_kernel(Tiles<KIND, PACKED> W, int E, const int32_t *__restrict__ ids,
                                                     const float *__restrict__ topk_w, int topk,
                                                     const float *__restrict__ H, const float *__restrict__ Hmax,
                                                     int n_ff, int K, float *__restrict__ Y) {
  using Dd = Dec<KIND>;
  using X4 = typename gv::XVec<float>::type;
  constexpr int kFrag = Dd::NSTEP * 4, NS = PD + 1;
  extern __shared__ u32x4 lds[];
  const int t = blockIdx.y, c = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = lane & 15, G = lane >> 4;
  const int nkb = n_ff / Dd::KB, units = topk * nkb;
  const int u0 = (int)((int64_t)wave * units / S), u1 = (int)((int64_t)(wave + 1) * units / S);
  const int u_last = max(u1 - 1, 0);
  // Lane s < topk: slot s's expert (-1 if outside [0, E)).
  int es = -1;
  if (lane < topk) {
    const int v = ids[(int64_t)t * topk + lane];
    es = (v >= 0 && v < E) ? v : -1;
  }
  u32x4 *zrun = lds + wave * (NS + 1) * kFrag, *ring = zrun + kFrag;
  const int xo = Dd::x_off(lane >> 3, (lane >> 1) & 3, lane & 1);
  Held<KIND, PACKED> raw[NS][1];
  X4 xv[NS];
  auto issue = [&](int u, int slot) {
    u = min(u, u_last);
    const int s = u / nkb, kb = u % nkb;
    const int e = max(__builtin_amdgcn_readlane(es, s), 0);  // an absent slot reads expert 0, adds nothing
    __builtin_memcpy(&xv[slot], H + ((int64_t)t * topk + s) * n_ff + (int64_t)kb * Dd::KB + xo, sizeof(X4));
    W.load(e, c, kb, lane, j, G, raw[slot][0]);
  };
#pragma unroll
  for (int d = 0; d < PD; ++d) issue(u0 + d, d);
  if (lane < kFrag) zrun[lane] = u32x4{0u, 0u, 0u, 0u};
  // Lane s < topk: the slot's power-of-two scale 2^k (max |h| / 2^k <= 2^14)
  // and its weight topk_w[t][s] * 2^k (both exact powers of two times w).
  float xs = 1.f, ws = 0.f;
  {
    const int per = n_ff / 16;
    float m = 0.f;
    // Eight lanes per slot for up to eight slots at a time.
    for (int s0 = 0; s0 < topk; s0 += 8) {
      const int s = s0 + (lane >> 3);
      float mm = 0.f;
      if (s < topk)
        for (int i = lane & 7; i < per; i += 8) mm = fmaxf(mm, Hmax[((int64_t)t * topk + s) * per + i]);
#pragma unroll
      for (int off = 4; off > 0; off >>= 1) mm = fmaxf(mm, __shfl_xor(mm, off, 64));
      // Slot s0 + q's maximum sits in lanes 8q .. 8q + 7: move it to lane s0 + q.
      const float got = __shfl(mm, 8 * (lane - s0), 64);
      if (lane >= s0 && lane < s0 + 8) m = got;
    }
    if (lane < topk && es >= 0) {
      const int k = m > 0.f ? max(0, __builtin_amdgcn_frexp_expf(m) - 14) : 0;
      xs = __builtin_amdgcn_ldexpf(1.0f, -k);
      ws = topk_w[(int64_t)t * topk + lane] * __builtin_amdgcn_ldexpf(1.0f, k);
    }
  }
  Fx4 acc[1] = {{0.f, 0.f, 0.f, 0.f}};
  float acc1[1] = {0.f};  // the single-token decoders' per-lane share
  const u32x4 *xbase[NS];
#pragma unroll
  for (int d = 0; d < NS; ++d) xbase[d] = (j == 0 ? ring + d * kFrag : zrun) + G;
  const int xstep = j == 0 ? 4 : 0;
  constexpr int NSEL = Nsel<KIND>::value;
  const u32x4 *abase[NS][NSEL];
  if constexpr (kT1<KIND>) {
#pragma unroll
    for (int d = 0; d < NS; ++d)
#pragma unroll
      for (int c = 0; c < NSEL; ++c) abase[d][c] = (j == gv::T1<KIND>::arow(c, G) ? ring + d * kFrag : zrun) + G;
  }
  auto consume = [&](int u, int d) {
    const int s = u / nkb;
    stage_x(ring + d * kFrag, lane, xv[d],
            __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, xs), s)));
    const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ws), s));
    typename Dd::Raw fr[1] = {Tiles<KIND, PACKED>::raw(raw[d][0], G)};
    if (__builtin_amdgcn_readlane(es, s) >= 0) {
      if constexpr (kT1<KIND>) kblock_t1<KIND, 1>(fr, abase[d], G, acc1, w);
      else kblock<KIND, 1>(fr, xbase[d], xstep, G, j, acc, w);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
  };
  const int cnt = max(u1 - u0, 0), full = cnt - cnt % NS;
  for (int i = 0; i < full; i += NS) {
#pragma unroll
    for (int d = 0; d < NS; ++d) {
      issue(u0 + i + d + PD, (d + PD) % NS);
      consume(u0 + i + d, d);
    }
  }
#pragma unroll
  for (int d = 0; d < NS - 1; ++d)
    if (d < cnt - full) consume(u0 + full + d, d);

  float v;
  if constexpr (kT1<KIND>) {
    v = acc1[0] + __shfl_xor(acc1[0], 16);
    v += __shfl_xor(v, 32);
  } else {
    v = acc[0][0];
  }
  if constexpr (S > 1) {
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds);
    if (wave > 0 && lane < 16) red[(wave - 1) * 16 + lane] = v;
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < S - 1; ++w) v += red[w * 16 + (lane & 15)];
  }
  if (lane < 16) Y[(int64_t)t * K + 16 * c + j] = v;
}

template <int KIND, bool PACKED, int S1, int PD1, int S2, int PD2>
hipError_t run_fused_shape(const uint8_t *W_gu, const uint8_t *W_d, int64_t E, const int32_t *ids,
                           const float *topk_w, int64_t topk, const void *X, int x_f16, float *Y, int64_t M,
                           int64_t N_ff, int64_t K, float *H, float *Hmax, hipStream_t s) {
  constexpr int kFrag = Dec<KIND>::NSTEP * 4;
  const int64_t P = M * topk;
  auto tiles = [&](const uint8_t *W, int64_t rows, int64_t cols) {
    Tiles<KIND, PACKED> t;
    t.W = W;
    t.rows = (int)rows;
    t.nkb = (int)(cols / 256);
    t.row_bytes = (cols / Geometry<KIND>::elems) * Geometry<KIND>::bytes;
    t.expert_bytes = PACKED ? packed_bytes_of(KIND, rows, cols) : rows * t.row_bytes;
    return t;
  };
  const size_t lds1 = std::max<size_t>((size_t)S1 * (PD1 + 2) * kFrag * 16, (size_t)(S1 - 1) * 2 * 16 * 4);
  // Tile-major grid: workgroup i runs on XCD i mod 8, so every pair's
  // workgroup for one tile shares that XCD's L2 (pairs of one expert read
  // its tile from there).
  const dim3 g1((unsigned)(N_ff / 16), (unsigned)P);
  if (x_f16)
    hipLaunchKernelGGL((gu_kernel<KIND, _Float16, S1, PD1, PACKED>), g1, dim3(64 * S1), lds1, s,
                       tiles(W_gu, 2 * N_ff, K), (int)E, ids, (int)topk, (const _Float16 *)X, (int)K, (int)N_ff, H,
                       Hmax);
  else
    hipLaunchKernelGGL((gu_kernel<KIND, float, S1, PD1, PACKED>), g1, dim3(64 * S1), lds1, s,
                       tiles(W_gu, 2 * N_ff, K), (int)E, ids, (int)topk, (const float *)X, (int)K, (int)N_ff, H,
                       Hmax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds2 = std::max<size_t>((size_t)S2 * (PD2 + 2) * kFrag * 16, (size_t)(S2 - 1) * 16 * 4);
  const dim3 g2((unsigned)(K / 16), (unsigned)M);  // tile-major, as above
  hipLaunchKernelGGL((down_kernel<KIND, S2, PD2, PACKED>), g2, dim3(64 * S2), lds2, s, tiles(W_d, K, N_ff), (int)E,
                     ids, topk_w, (int)topk, H, Hmax, (int)N_ff, (int)K, Y);
  return hipGetLastError();
}

template <int KIND, bool PACKED>
hipError_t run_fused(const uint8_t *W_gu, const uint8_t *W_d, int64_t E, const int32_t *ids, const float *topk_w,
                     int64_t topk, const void *X, int x_f16, float *Y, int64_t M, int64_t N_ff, int64_t K, float *H,
                     float *Hmax, hipStream_t s) {
#ifdef QMM_TUNING
  static const int cfg = [] {
    const char *e = getenv("QMM_FFN_CFG");
    return e ? atoi(e) : 0;
  }();
#define QMM_SHAPE(C, A, B, C2, D)                                                                            \
  if (cfg == C)                                                                                            \
    return run_fused_shape<KIND, PACKED, A, B, C2, D>(W_gu, W_d, E, ids, topk_w, topk, X, x_f16, Y, M, N_ff, K, H, \
                                                      Hmax, s);
  QMM_SHAPE(1, 2, 1, 4, 1)
  QMM_SHAPE(2, 8, 1, 4, 1)
  QMM_SHAPE(3, 4, 2, 4, 1)
  QMM_SHAPE(4, 4, 1, 8, 1)
  QMM_SHAPE(5, 4, 1, 2, 1)
  QMM_SHAPE(6, 4, 1, 4, 2)
  QMM_SHAPE(7, 4, 1, 12, 1)
  QMM_SHAPE(8, 2, 2, 8, 1)
  QMM_SHAPE(9, 8, 1, 8, 1)
  QMM_SHAPE(10, 4, 1, 6, 1)
#undef QMM_SHAPE
#endif
  // Waves per workgroup by grid size (measured at the 128-expert top-8
  // workload, 1 and 16 tokens): many workgroups take fewer waves each.
  const bool many_gu = M * topk * (N_ff / 16) >= 1024, many_d = M * (K / 16) >= 512;
  if (many_gu)
    return many_d ? run_fused_shape<KIND, PACKED, 2, 1, 4, 1>(W_gu, W_d, E, ids, topk_w, topk, X, x_f16, Y, M, N_ff,
                                                               K, H, Hmax, s)
                  : run_fused_shape<KIND, PACKED, 2, 1, 8, 1>(W_gu, W_d, E, ids, topk_w, topk, X, x_f16, Y, M, N_ff,
                                                               K, H, Hmax, s);
  return many_d ? run_fused_shape<KIND, PACKED, 4, 1, 4, 1>(W_gu, W_d, E, ids, topk_w, topk, X, x_f16, Y, M, N_ff, K,
                                                             H, Hmax, s)
                : run_fused_shape<KIND, PACKED, 4, 1, 8, 1>(W_gu, W_d, E, ids, topk_w, topk, X, x_f16, Y, M, N_ff, K,
                                                             H, Hmax, s);
}

}  // namespace fz

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
  // Two launches: about one pair per expert (the routed products would not
  // group), a matrix-core decoder over this layout, whole k-blocks.
  const bool fused_kind = packed ? packed_supported(kind) : xs_native_supported(kind);
  if (fused_kind && P < 4 * E && N_ff % 256 == 0 && K % 256 == 0 && topk <= 64 && M * K < ((int64_t)1 << 31) &&
      P * N_ff < ((int64_t)1 << 31)) {
    switch (kind) {
#define QMM_FUSED(K_)                                                                                             \
  case K_:                                                                                                        \
    return packed ? fz::run_fused<K_, true>(W_gu, W_d, E, ids, topk_w, topk, X, x_f16, Y, M, N_ff, K, H, G, s)  \
                  : fz::run_fused<K_, false>(W_gu, W_d, E, ids, topk_w, topk, X, x_f16, Y, M, N_ff, K, H, G, s);
      QMM_FUSED(Q4_K)
      QMM_FUSED(Q6_K)
      QMM_FUSED(Q5_K)
      QMM_FUSED(Q2_K)
      QMM_FUSED(Q3_K)
#undef QMM_FUSED
      case Q4_0: return fz::run_fused<Q4_0, true>(W_gu, W_d, E, ids, topk_w, topk, X, x_f16, Y, M, N_ff, K, H, G, s);
      case Q5_0: return fz::run_fused<Q5_0, true>(W_gu, W_d, E, ids, topk_w, topk, X, x_f16, Y, M, N_ff, K, H, G, s);
      case Q8_0: return fz::run_fused<Q8_0, true>(W_gu, W_d, E, ids, topk_w, topk, X, x_f16, Y, M, N_ff, K, H, G, s);
      case IQ4_NL:
        return fz::run_fused<IQ4_NL, true>(W_gu, W_d, E, ids, topk_w, topk, X, x_f16, Y, M, N_ff, K, H, G, s);
      case IQ4_XS:
        return fz::run_fused<IQ4_XS, true>(W_gu, W_d, E, ids, topk_w, topk, X, x_f16, Y, M, N_ff, K, H, G, s);
      case MXFP4:
        return fz::run_fused<MXFP4, true>(W_gu, W_d, E, ids, topk_w, topk, X, x_f16, Y, M, N_ff, K, H, G, s);
      default: break;
    }
  }
  hipError_t e = launch_moe(kind, W_gu, E, ids, topk, X, x_f16, 0, G, M, 2 * N_ff, K, base + L.route, s, packed);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)P), dim3(256), 0, s, G, H, S, (int)N_ff);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // The same pairs, experts and item size: the routing the gate/up product
  // left in the workspace serves the down product.
  e = launch_moe(kind, W_d, E, ids, topk, H, 0, 1, D, M, K, N_ff, base + L.route, s, packed,
                 moe_item_pairs(kind, E, M, topk, K, packed) == moe_item_pairs(kind, E, M, topk, N_ff, packed));
  if (e != hipSuccess) return e;
  const int64_t n2 = M * (K / 4);
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, s, D, S, ids, topk_w, Y, M,
                     (int)topk, (int)K, E);
  return hipGetLastError();
}

}  // namespace qmm
