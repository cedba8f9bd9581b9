// qmm_gemv_t1.h -- single-token decoders for Q4_K and Q6_K that keep
// sub-blocks apart in the rows of the matrix-core product (A row r holds the
// token's activations of the sub-block that row selects at that step, every
// other row of those columns zero) and apply the sub-block scales and
// minimums to D in f32, once per k-block.  Used by the single-token decode
// GEMV (qmm_gemv_t1.hip) and the single-token expert FFN kernels
// (qmm_moe_ffn.hip).
//
//   Q4_K  B holds each raw 4-bit code as an f16 subnormal (q * 2^-24, or
//         16q * 2^-24 for a high nibble left in place); D rows 4G, 4G + 1
//         are sub-blocks 2G, 2G + 1 of lane group G.
//   Q6_K  B holds q - 32 exactly; D row 8h + 2g + a is sub-block 8h + 2g + a.
//   Q5_K, Q2_K, Q3_K  the raw codes (with the fifth or high-mask bit) as
//         subnormals, as Q4_K; the Q3_K offset -4 enters through the
//         activation sums.
//   the 32-element kinds and IQ4_XS (one block or group per step, its own
//         scale): B is the step-scaled decoder's exact code value, A row s
//         holds step s's activations, so D row s is block s's dot product;
//         lane group G = 0, 1 holds rows 4G .. 4G + 3 and scales them.
//
// Every product is exact in f32 and the matrix cores accumulate in f32, so
// the folded decoders' error bound holds: activations rounded once to f16,
// then f32 sums.
#pragma once

#include "qmm_gemv_mfma.h"

namespace qmm {
namespace gv {

template <int KIND> struct T1;

template <> struct T1<Q4_K> {
  using Dd = DecQ4K;
  using Raw = DecQ4K::Raw;
  static constexpr bool HAS_MIN = true;
  static constexpr int NSEL = 2;  // A-row groups: steps 0-3 and 4-7
  __device__ static int sel_of_step(int s) { return s >> 2; }
  // The A row lane group G fills in selector group c: sub-block 2G + c.
  __device__ static int arow(int c, int G) { return 4 * G + c; }
  struct Sc { float f0, f1, g0, g1; };
  __device__ static Sc prep(const Raw &r, int G) {
    // Scales and mins of sub-blocks 2G, 2G + 1 (the 12-byte pack; Vulkore
    // quant_test.cpp, ref::q4k_scale_min), two 8-bit lanes at once.
    const int c = 16 * (G & 1);
    const uint32_t a = r.hdr.y >> c, b = r.hdr.z >> c, e = r.hdr.w >> c;
    uint32_t sc2, mn2;
    if (G < 2) {
      sc2 = a & 0x3F3Fu;
      mn2 = b & 0x3F3Fu;
    } else {
      sc2 = (e & 0x0F0Fu) | ((a >> 2) & 0x3030u);
      mn2 = ((e >> 4) & 0x0F0Fu) | ((b >> 2) & 0x3030u);
    }
    const float d = lo_f16(r.hdr.x), dmin = hi_f16(r.hdr.x);
    Sc s;
    s.f0 = (d * 16777216.0f) * (float)(sc2 & 0xFFu);        // codes arrive as q * 2^-24
    s.f1 = (d * 1048576.0f) * (float)((sc2 >> 8) & 0xFFu);  // and as 16q * 2^-24
    s.g0 = -dmin * (float)(mn2 & 0xFFu);
    s.g1 = -dmin * (float)((mn2 >> 8) & 0xFFu);
    return s;
  }
  __device__ static half8 bop(const Raw &r, const Sc &, int st) {
    const int w = st & 3;
    const uint32_t v0 = w < 2 ? (w == 0 ? r.q0.x : r.q0.z) : (w == 2 ? r.q1.x : r.q1.z);
    const uint32_t v1 = w < 2 ? (w == 0 ? r.q0.y : r.q0.w) : (w == 2 ? r.q1.y : r.q1.w);
    const uint32_t m = st < 4 ? 0x000F000Fu : 0x00F000F0u;
    return pack8(v0 & m, (v0 >> 8) & m, v1 & m, (v1 >> 8) & m);
  }
  // Lane (j, G) holds D rows 4G .. 4G + 3: sub-blocks 2G, 2G + 1, then zeros.
  __device__ static float post(float acc, floatx4 D, floatx4 X, const Sc &s) {
    return acc + s.f0 * D[0] + s.f1 * D[1] + s.g0 * X[0] + s.g1 * X[1];
  }
};

template <> struct T1<Q6_K> {
  using Dd = DecQ6K;
  using Raw = DecQ6K::Raw;
  static constexpr bool HAS_MIN = false;
  static constexpr int NSEL = 4;  // A-row groups: quarters g = step / 2
  __device__ static int sel_of_step(int s) { return s >> 1; }
  // Group G = 2h + a at quarter g: sub-block 8h + 2g + a.
  __device__ static int arow(int g, int G) { return 8 * (G >> 1) + 2 * g + (G & 1); }
  struct Sc { float sc[4], d; };
  __device__ static Sc prep(const Raw &r, int G) {
    // Lane (j, G) holds D rows 4G .. 4G + 3, sub-blocks 4G + q: bytes
    // 4(G & 1) + q of the eight scales this lane loaded (8 (G >> 1) ..).
    const uint32_t w = (G & 1) ? r.sc.y : r.sc.x;
    Sc s;
#pragma unroll
    for (int q = 0; q < 4; ++q) s.sc[q] = (float)(int)(int8_t)(uint8_t)((w >> (8 * q)) & 0xFFu);
    s.d = lo_f16(r.d);
    return s;
  }
  __device__ static half8 bop(const Raw &r, const Sc &, int st) {
    const int g = st >> 1, w = 2 * (st & 1);
    const u32x4 &ql = (g & 1) ? r.ql1 : r.ql0;
    const uint32_t q0 = w == 0 ? ql.x : ql.z, q1 = w == 0 ? ql.y : ql.w;
    const uint32_t h0 = w == 0 ? r.qh.x : r.qh.z, h1 = w == 0 ? r.qh.y : r.qh.w;
    // As the folded decoder: low case, nibble at bits 0-3 and the two high
    // bits moved to 4-5 (e = 1024 + q); high case, nibble left at 4-7 and
    // the high bits moved to 8-9 (e = 1024 + 16q).
    const uint32_t qm = g < 2 ? 0x000F000Fu : 0x00F000F0u;
    const uint32_t hm = g < 2 ? 0x00300030u : 0x03000300u;
    const int up = (g & 1) ? 2 : 4;
    const uint32_t e0 = and_or(h0 << up, hm, mag(q0, qm));
    const uint32_t e1 = and_or(h0 >> (8 - up), hm, mag(q0 >> 8, qm));
    const uint32_t e2 = and_or(h1 << up, hm, mag(q1, qm));
    const uint32_t e3 = and_or(h1 >> (8 - up), hm, mag(q1 >> 8, qm));
    // q - 32: e - 1056, or e / 16 - 96 (both exact).
    if (g < 2) {
      const half2v off = {-1056.0f16, -1056.0f16};
      return pack8(as_u(as_h2(e0) + off), as_u(as_h2(e1) + off), as_u(as_h2(e2) + off), as_u(as_h2(e3) + off));
    }
    const uint32_t f = 0x2C002C00u, b = 0xD600D600u;  // (1/16, 1/16), (-96, -96)
    return pack8(fold(e0, f, b), fold(e1, f, b), fold(e2, f, b), fold(e3, f, b));
  }
  __device__ static float post(float acc, floatx4 D, floatx4, const Sc &s) {
    return acc + s.d * (s.sc[0] * D[0] + s.sc[1] * D[1] + s.sc[2] * D[2] + s.sc[3] * D[3]);
  }
};

// Q5_K: as Q4_K, with the fifth bit just above the nibble (bit 4 for a low
// nibble, bit 8 for a high nibble left in place): q5 * 2^-24 or
// 16 q5 * 2^-24, still subnormal.
template <> struct T1<Q5_K> {
  using Dd = DecQ5K;
  using Raw = DecQ5K::Raw;
  static constexpr bool HAS_MIN = true;
  static constexpr int NSEL = 2;
  __device__ static int sel_of_step(int s) { return s >> 2; }
  __device__ static int arow(int c, int G) { return 4 * G + c; }
  struct Sc : T1<Q4_K>::Sc { int sh; };  // sh = 2G: this group's fifth-bit position in qh
  __device__ static Sc prep(const Raw &r, int G) {
    Sc s;
    static_cast<T1<Q4_K>::Sc &>(s) = T1<Q4_K>::prep(DecQ4K::Raw{r.hdr, r.q0, r.q1}, G);
    s.sh = 2 * G;
    return s;
  }
  __device__ static half8 bop(const Raw &r, const Sc &s, int st) {
    const int w = st & 3;
    const uint32_t v0 = w < 2 ? (w == 0 ? r.q0.x : r.q0.z) : (w == 2 ? r.q1.x : r.q1.z);
    const uint32_t v1 = w < 2 ? (w == 0 ? r.q0.y : r.q0.w) : (w == 2 ? r.q1.y : r.q1.w);
    const uint32_t g0 = w < 2 ? (w == 0 ? r.h0.x : r.h0.z) : (w == 2 ? r.h1.x : r.h1.z);
    const uint32_t g1 = w < 2 ? (w == 0 ? r.h0.y : r.h0.w) : (w == 2 ? r.h1.y : r.h1.w);
    const uint32_t a0 = g0 >> s.sh, a1 = g1 >> s.sh;
    const bool lo = st < 4;
    const uint32_t qm = lo ? 0x000F000Fu : 0x00F000F0u, hm = lo ? 0x00100010u : 0x01000100u;
    return pack8(and_or(lo ? a0 << 4 : a0 << 7, hm, v0 & qm), and_or(lo ? a0 >> 4 : a0 >> 1, hm, (v0 >> 8) & qm),
                 and_or(lo ? a1 << 4 : a1 << 7, hm, v1 & qm), and_or(lo ? a1 >> 4 : a1 >> 1, hm, (v1 >> 8) & qm));
  }
  __device__ static float post(float acc, floatx4 D, floatx4 X, const Sc &s) { return T1<Q4_K>::post(acc, D, X, s); }
};

// Q2_K: step s = 2j + b of group G = 2n + a lies in sub-block 8n + 2j + a;
// selector j, A row 4G + j.  B holds each 2-bit code left in place, at bits
// 2j of its byte: q * 4^j * 2^-24.  Scale d * sc * 2^24 / 4^j; minimum
// -dmin * m times the sub-block's activation sum.
template <> struct T1<Q2_K> {
  using Dd = DecQ2K;
  using Raw = DecQ2K::Raw;
  static constexpr bool HAS_MIN = true;
  static constexpr int NSEL = 4;
  __device__ static int sel_of_step(int s) { return s >> 1; }
  __device__ static int arow(int c, int G) { return 4 * G + c; }
  struct Sc { float f[4], g[4]; };
  __device__ static Sc prep(const Raw &r, int G) {
    const float d = lo_f16(r.dd), dmin = hi_f16(r.dd);
    Sc s;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 8 * (G >> 1) + 2 * j + (G & 1);
      const uint32_t byte = (r.sc[i >> 2] >> (8 * (i & 3))) & 0xFFu;
      s.f[j] = (d * (16777216.0f / (float)(1 << (2 * j)))) * (float)(byte & 15u);
      s.g[j] = -dmin * (float)(byte >> 4);
    }
    return s;
  }
  __device__ static half8 bop(const Raw &r, const Sc &, int st) {
    const int j = st >> 1, b = st & 1;
    const uint32_t v0 = b ? r.q.z : r.q.x, v1 = b ? r.q.w : r.q.y;
    const uint32_t m = 0x00030003u << (2 * j);
    return pack8(v0 & m, (v0 >> 8) & m, v1 & m, (v1 >> 8) & m);
  }
  __device__ static float post(float acc, floatx4 D, floatx4 X, const Sc &s) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc += s.f[q] * D[q] + s.g[q] * X[q];
    return acc;
  }
};

// Q3_K: as Q2_K, with v = q + 4 h (the high-mask bit; 0 .. 7) at bits 0-2 of
// each half: v * 2^-24.  The weight is (v - 4)(sc - 32) d, so the scale is
// d (sc - 32) 2^24 and the sub-block's activation sum enters times
// -4 d (sc - 32).
template <> struct T1<Q3_K> {
  using Dd = DecQ3K;
  using Raw = DecQ3K::Raw;
  static constexpr bool HAS_MIN = true;
  static constexpr int NSEL = 4;
  __device__ static int sel_of_step(int s) { return s >> 1; }
  __device__ static int arow(int c, int G) { return 4 * G + c; }
  struct Sc { float f[4], g[4]; int hb; };  // hb = 4n: this group's high-mask bits
  __device__ static Sc prep(const Raw &r, int G) {
    const int n = G >> 1, a = G & 1;
    const float d = lo_f16(r.d);
    Sc s;
    s.hb = 4 * n;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = 2 * j + a;  // scale index minus 8n
      const uint32_t lb = (r.lo[k >> 2] >> (8 * (k & 3))) & 0xFFu;
      const int low4 = (int)(n ? lb >> 4 : lb & 15u);
      const int high2 = (int)((r.hi >> (8 * (k & 3) + 2 * (2 * n + (j >> 1)))) & 3u);
      const float ds = d * (float)((low4 | (high2 << 4)) - 32);
      s.f[j] = ds * 16777216.0f;
      s.g[j] = -4.0f * ds;
    }
    return s;
  }
  __device__ static half8 bop(const Raw &r, const Sc &s, int st) {
    const int j = st >> 1, b = st & 1;
    const uint32_t v0 = (b ? r.q.z : r.q.x) >> (2 * j), v1 = (b ? r.q.w : r.q.y) >> (2 * j);
    const int hs = s.hb + j;
    const uint32_t h0 = (b ? r.hm.z : r.hm.x) >> hs, h1 = (b ? r.hm.w : r.hm.y) >> hs;
    const uint32_t cm = 0x00030003u, hm = 0x00040004u;
    return pack8(and_or(h0 << 2, hm, v0 & cm), and_or(h0 >> 6, hm, (v0 >> 8) & cm), and_or(h1 << 2, hm, v1 & cm),
                 and_or(h1 >> 6, hm, (v1 >> 8) & cm));
  }
  __device__ static float post(float acc, floatx4 D, floatx4 X, const Sc &s) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc += s.f[q] * D[q] + s.g[q] * X[q];
    return acc;
  }
};

// Step-scaled kinds: eight steps, eight A rows (row s for step s, whatever
// the lane group), no minimum term.
template <int KIND>
struct T1Step {
  using Dd = Dec<KIND>;
  using Raw = typename Dd::Raw;
  static constexpr bool HAS_MIN = false;
  static constexpr int NSEL = 8;
  __device__ static int sel_of_step(int s) { return s; }
  __device__ static int arow(int c, int) { return c; }
  struct Sc { float s[4]; };
  // Lane (j, G) holds D rows 4G .. 4G + 3: blocks 4G + q for G = 0, 1, and
  // zero rows for G = 2, 3 (whatever scale they take).
  __device__ static Sc prep(const Raw &r, int G) {
    Sc o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = Dd::scale(r, q), hi = Dd::scale(r, 4 + q);
      o.s[q] = (G & 1) ? hi : lo;
    }
    return o;
  }
  __device__ static half8 bop(const Raw &r, const Sc &, int st) { return Dd::bop(r, typename Dd::Sc{}, st, 0); }
  __device__ static float post(float acc, floatx4 D, floatx4, const Sc &s) {
    return acc + s.s[0] * D[0] + s.s[1] * D[1] + s.s[2] * D[2] + s.s[3] * D[3];
  }
};
template <> struct T1<Q4_0> : T1Step<Q4_0> {};
template <> struct T1<Q5_0> : T1Step<Q5_0> {};
template <> struct T1<Q8_0> : T1Step<Q8_0> {};
template <> struct T1<IQ4_NL> : T1Step<IQ4_NL> {};
template <> struct T1<MXFP4> : T1Step<MXFP4> {};
template <> struct T1<IQ4_XS> : T1Step<IQ4_XS> {};

}  // namespace gv
}  // namespace qmm
