// qmm_gemm_ks.h -- weight decoders of the wave-private prefill GEMM
// (qmm_gemm_ks.hip, the super-block kinds Q2_K, Q3_K, Q4_K, Q5_K, IQ4_XS): per lane, the sixteen weights one 64-element k-step of
// one weight row feeds into two v_mfma_f32_16x16x32_f16 B operands.
//
// Lane l of a wave belongs to lane group G = l / 16.  In a 16x16x32 f16
// product, lane group G supplies k-slots 8G .. 8G+7 of both operands.  Which
// eight weights of the 64-element step sit in those slots is free, as long
// as the activation operand holds the same k: a dot product does not depend
// on the order of its terms.  Each kind picks the assignment that makes its
// lane's bytes contiguous, and koff(G, s) gives the first of the eight k of
// sub-step s (s = 0, 1) so that the activation reads follow:
//   kBlock32 (IQ4_XS)          k = 32(G>>1) + 8(G&1) + 16s + t: code bytes
//                              8(G&1) .. +7 of 32-element group G>>1, whose
//                              low nibbles are elements 8(G&1)+t and high
//                              nibbles 16+8(G&1)+t (the low nibble of byte j
//                              is element j, the high nibble j + 16;
//                              ferrox-cuda 0.20.0 codebook.rs, the IQ4_NL and
//                              IQ4_XS rows);
//   kHalf64  (Q4_K, Q5_K, Q2_K, Q3_K)
//                              k = 8G + 32s + t: within the step, sub-step
//                              0 is the first 32 elements and sub-step 1 the
//                              second, and lane group G takes positions
//                              8G .. 8G+7 of each, which are the same code
//                              bytes in the super-block layouts.
//
// The weight bytes pass through LDS before they are decoded.  A kind lists,
// per step, the byte runs of a row that the step needs (run_start(k, st),
// run_len(k, st), at most kRunMax[k] bytes, each at least 16).  A run is
// copied as 16-byte pieces at run offsets min(16 c, len - 16): contiguous
// lanes take consecutive pieces of a few rows, every piece lies inside the
// run (so no load reaches past the weights), and the last piece overlaps
// the one before it with the same bytes.  In LDS the run's bytes sit at the
// same offsets, so gather() reads a lane's fields by their offset within
// the run (Rd::get<k, T>(offset)) into Raw, and decode() turns Raw into the
// two B operands.
//
// Every weight is rounded once to f16 from its exact value, or from its f32
// value where the exact value needs more than 24 bits (within 2^-11 + 2^-24
// relative).
#pragma once

#include "qmm_gemm_dec.h"

namespace qmm {
namespace gk {

using gm::affine;
using gm::bits;
using gm::h2;
using gm::half2v;
using gm::ld16;
using gm::ld2;
using gm::ld4;
using gm::ld8;
using gm::splat;
using gm::spread;
using gm::u32x2;
using gm::u32x4;

enum Pattern { kBlock32, kHalf64 };

template <int PAT>
__device__ __forceinline__ int koff(int G, int s) {
  if constexpr (PAT == kBlock32) return 32 * (G >> 1) + 8 * (G & 1) + 16 * s;
  else return 8 * G + 32 * s;
}

// An f16 pair (each an exact small value) times a, plus b, each element
// formed in f32 and rounded to f16 (v_fma_mixlo/mixhi_f16).
__device__ __forceinline__ uint32_t mix2(uint32_t p, float a, float b) {
  const half2v h = h2(p);
  return bits(half2v{(_Float16)__builtin_fmaf((float)h[0], a, b), (_Float16)__builtin_fmaf((float)h[1], a, b)});
}

// Four bytes (0..255 each) as the exact f16 pairs (b0 - c, b1 - c),
// (b2 - c, b3 - c); `c1024` is the f16 pair (1024 + c, 1024 + c).
__device__ __forceinline__ void bytes_minus(uint32_t v, half2v c1024, uint32_t &p01, uint32_t &p23) {
  uint32_t a, b;
  spread(v, a, b);
  p01 = bits(h2(a) - c1024);
  p23 = bits(h2(b) - c1024);
}

__device__ __forceinline__ u32x4 pack4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) { return u32x4{a, b, c, d}; }

template <int KIND> struct Frag;


// Eight code bytes of a lane as two four-code words of low nibbles
// (sub-step 0) and of high nibbles (sub-step 1), one code per byte.
__device__ __forceinline__ void nib_words(u32x2 q, uint32_t (&lo)[2], uint32_t (&hi)[2]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    lo[i] = q[i] & 0x0F0F0F0Fu;
    hi[i] = (q[i] >> 4) & 0x0F0F0F0Fu;
  }
}

// Table values plus 128 (one per byte) times dl, formed as
// fma(1152 + t, dl, -1152 dl) = t dl, exact in f32 (dl has at most 17
// significant bits, t at most 7), then rounded to f16.
__device__ __forceinline__ u32x4 table_op(const uint32_t (&c)[2], float dl, float nb) {
  uint32_t a0, b0, a1, b1;
  spread(c[0], a0, b0);
  spread(c[1], a1, b1);
  return pack4(mix2(a0, dl, nb), mix2(b0, dl, nb), mix2(a1, dl, nb), mix2(b1, dl, nb));
}

// IQ4_XS (136 B / 256): f16 d, u16 scales_h, scales_l[4], eight 32-element
// groups packed as IQ4_NL blocks; group ib has ls = nibble (ib&1) of
// scales_l[ib/2] | ((scales_h >> 2ib) & 3) << 4 and w = d*(ls-32)*table[code]
// (codebook.rs, the IQ4_XS row).  Step st covers groups 2(st%4), +1.
template <> struct Frag<IQ4_XS> {
  static constexpr int kPat = kBlock32;
  struct Raw { u32x2 h, q; };
  static constexpr int kRuns = 2;
  static constexpr int kRunMax[kRuns] = {16, 32};
  static __device__ __forceinline__ int run_start(int k, int st) {
    return (st >> 2) * 136 + (k == 0 ? 0 : 8 + 32 * (st & 3));
  }
  static __device__ __forceinline__ int run_len(int k, int st) {
    (void)st;
    return k == 0 ? 16 : 32;
  }
  template <class Rd>
  static __device__ __forceinline__ void gather(const Rd &rd, int st, int G, Raw &r) {
    (void)st;
    r.h = rd.template get<0, u32x2>(0);
    r.q = rd.template get<1, u32x2>(16 * (G >> 1) + 8 * (G & 1));
  }
  static __device__ __forceinline__ void decode(const Raw &r, int st, int G, u32x4 &b0, u32x4 &b1) {
    const int ib = 2 * (st & 3) + (G >> 1);
    const float d = f16_bits_to_f32(r.h[0] & 0xFFFFu);
    const uint32_t sh = r.h[0] >> 16;
    const uint32_t sl = (r.h[1] >> (8 * (ib >> 1) + 4 * (ib & 1))) & 15u;
    const int ls = (int)(sl | (((sh >> (2 * ib)) & 3u) << 4));
    const float dl = d * (float)(ls - 32), nb = -1152.0f * dl;
    uint32_t lo[2], hi[2];
    nib_words(r.q, lo, hi);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lo[i] = iq4_lookup(lo[i]);
      hi[i] = iq4_lookup(hi[i]);
    }
    b0 = table_op(lo, dl, nb);
    b1 = table_op(hi, dl, nb);
  }
};

// Codes (one per byte) as exact f16 values c - bias, then a * v + b each
// (f32, rounded to f16): one B operand from two four-code words.
// `c1024` = f16 pair (1024 + bias).
__device__ __forceinline__ u32x4 scaled_op(const uint32_t (&c)[2], half2v c1024, float a, float b) {
  uint32_t p0, p1, p2, p3;
  bytes_minus(c[0], c1024, p0, p1);
  bytes_minus(c[1], c1024, p2, p3);
  return pack4(mix2(p0, a, b), mix2(p1, a, b), mix2(p2, a, b), mix2(p3, a, b));
}

// The 6-bit scale and min of group j of the Q4_K/Q5_K 12-byte pack, from
// the 16-byte header h (d, dmin, pack) (Vulkore quant_test.cpp,
// ref::q4k_scale_min).
__device__ __forceinline__ uint32_t hbyte(const u32x4 &h, int i) {  // byte i of the pack
  const int b = 4 + i;
  const uint32_t w = b < 8 ? h[1] : (b < 12 ? h[2] : h[3]);
  return (w >> (8 * (b & 3))) & 0xFFu;
}
__device__ __forceinline__ void k4_sm(const u32x4 &h, int j, uint32_t &sc, uint32_t &mn) {
  if (j < 4) {
    sc = hbyte(h, j) & 63u;
    mn = hbyte(h, j + 4) & 63u;
  } else {
    sc = (hbyte(h, j + 4) & 15u) | ((hbyte(h, j - 4) >> 6) << 4);
    mn = (hbyte(h, j + 4) >> 4) | ((hbyte(h, j) >> 6) << 4);
  }
}

// Q4_K (144 B / 256): d, dmin, 12-byte scale/min pack, 128 bytes of codes;
// elements 64q .. 64q+31 are the low and 64q+32 .. +63 the high nibbles of
// code bytes 32q .. 32q+31 (Vulkore, ref::q4_k); w = d*sc*q - dmin*m.
template <> struct Frag<Q4_K> {
  static constexpr int kPat = kHalf64;
  struct Raw { u32x4 h; u32x2 q; };
  static constexpr int kRuns = 2;
  static constexpr int kRunMax[kRuns] = {16, 32};
  static __device__ __forceinline__ int run_start(int k, int st) {
    return (st >> 2) * 144 + (k == 0 ? 0 : 16 + 32 * (st & 3));
  }
  static __device__ __forceinline__ int run_len(int k, int st) {
    (void)st;
    return k == 0 ? 16 : 32;
  }
  template <class Rd>
  static __device__ __forceinline__ void gather(const Rd &rd, int st, int G, Raw &r) {
    (void)st;
    r.h = rd.template get<0, u32x4>(0);
    r.q = rd.template get<1, u32x2>(8 * G);
  }
  static __device__ __forceinline__ void decode(const Raw &r, int st, int, u32x4 &b0, u32x4 &b1) {
    const float d = f16_bits_to_f32(r.h[0] & 0xFFFFu), dmin = f16_bits_to_f32(r.h[0] >> 16);
    const int j0 = 2 * (st & 3);
    uint32_t sc0, mn0, sc1, mn1;
    k4_sm(r.h, j0, sc0, mn0);
    k4_sm(r.h, j0 + 1, sc1, mn1);
    const half2v z = {(_Float16)1024.0f, (_Float16)1024.0f};
    uint32_t lo[2], hi[2];
    nib_words(r.q, lo, hi);
    b0 = scaled_op(lo, z, d * (float)sc0, -(dmin * (float)mn0));
    b1 = scaled_op(hi, z, d * (float)sc1, -(dmin * (float)mn1));
  }
};

// Q5_K (176 B / 256): Q4_K plus qh[32] at byte 16 (codes at 48); the fifth
// bit of element r is bit r/32 of qh[r % 32].
template <> struct Frag<Q5_K> {
  static constexpr int kPat = kHalf64;
  struct Raw { u32x4 h; u32x2 qh, q; };
  static constexpr int kRuns = 3;
  static constexpr int kRunMax[kRuns] = {16, 32, 32};
  static __device__ __forceinline__ int run_start(int k, int st) {
    return (st >> 2) * 176 + (k == 0 ? 0 : k == 1 ? 16 : 48 + 32 * (st & 3));
  }
  static __device__ __forceinline__ int run_len(int k, int st) {
    (void)st;
    return k == 0 ? 16 : 32;
  }
  template <class Rd>
  static __device__ __forceinline__ void gather(const Rd &rd, int st, int G, Raw &r) {
    (void)st;
    r.h = rd.template get<0, u32x4>(0);
    r.qh = rd.template get<1, u32x2>(8 * G);
    r.q = rd.template get<2, u32x2>(8 * G);
  }
  static __device__ __forceinline__ void decode(const Raw &r, int st, int, u32x4 &b0, u32x4 &b1) {
    const float d = f16_bits_to_f32(r.h[0] & 0xFFFFu), dmin = f16_bits_to_f32(r.h[0] >> 16);
    const int j0 = 2 * (st & 3);
    uint32_t sc0, mn0, sc1, mn1;
    k4_sm(r.h, j0, sc0, mn0);
    k4_sm(r.h, j0 + 1, sc1, mn1);
    const half2v z = {(_Float16)1024.0f, (_Float16)1024.0f};
    uint32_t lo[2], hi[2];
    nib_words(r.q, lo, hi);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lo[i] |= ((r.qh[i] >> j0) & 0x01010101u) << 4;
      hi[i] |= ((r.qh[i] >> (j0 + 1)) & 0x01010101u) << 4;
    }
    b0 = scaled_op(lo, z, d * (float)sc0, -(dmin * (float)mn0));
    b1 = scaled_op(hi, z, d * (float)sc1, -(dmin * (float)mn1));
  }
};


// Q2_K (84 B / 256): scales[16] (low nibble scale, high nibble min),
// qs[64] at 16, d at 80, dmin at 82.  Element r: code bits 2j of
// qs[32n + r%32] with n = r/128, j = (r%128)/32; w = d*(s&15)*q - dmin*(s>>4)
// with s = scales[r/16].  Step st (q = st % 4) covers j = 2(q&1), +1.
template <> struct Frag<Q2_K> {
  static constexpr int kPat = kHalf64;
  struct Raw { u32x2 qs; uint32_t sc, dd; };
  static constexpr int kRuns = 2;
  static constexpr int kRunMax[kRuns] = {16, 68};
  static __device__ __forceinline__ int run_start(int k, int st) {
    const int n = (st & 3) >> 1;
    return (st >> 2) * 84 + (k == 0 ? 0 : 16 + 32 * n);
  }
  static __device__ __forceinline__ int run_len(int k, int st) {
    return k == 0 ? 16 : 68 - 32 * ((st & 3) >> 1);
  }
  template <class Rd>
  static __device__ __forceinline__ void gather(const Rd &rd, int st, int G, Raw &r) {
    const int q = st & 3, n = q >> 1;
    r.sc = rd.template get<0, uint32_t>(8 * n + 4 * (q & 1));
    r.qs = rd.template get<1, u32x2>(8 * G);
    r.dd = rd.template get<1, uint32_t>(64 - 32 * n);
  }
  static __device__ __forceinline__ void decode(const Raw &r, int st, int G, u32x4 &b0, u32x4 &b1) {
    const int sh = 4 * (st & 1);  // 2j for j = 2(q&1); q&1 = st&1
    const float d = f16_bits_to_f32(r.dd & 0xFFFFu), dmin = f16_bits_to_f32(r.dd >> 16);
    const uint32_t s0 = (r.sc >> (8 * (G >> 1))) & 0xFFu, s1 = (r.sc >> (16 + 8 * (G >> 1))) & 0xFFu;
    const half2v z = {(_Float16)1024.0f, (_Float16)1024.0f};
    uint32_t c0[2], c1[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      c0[i] = (r.qs[i] >> sh) & 0x03030303u;
      c1[i] = (r.qs[i] >> (sh + 2)) & 0x03030303u;
    }
    b0 = scaled_op(c0, z, d * (float)(s0 & 15u), -(dmin * (float)(s0 >> 4)));
    b1 = scaled_op(c1, z, d * (float)(s1 & 15u), -(dmin * (float)(s1 >> 4)));
  }
};

// The 6-bit Q3_K scale i from its 12-byte pack s[0..2]: the low four bits
// are nibble (i >= 8) of byte i % 8, the top two bits 2(i/4) of byte 8 + i%4.
__device__ __forceinline__ uint32_t scale6(const uint32_t (&s)[3], int i) {
  const int lb = i & 7;
  const uint32_t lw = lb < 4 ? s[0] : s[1];
  const uint32_t low4 = (lw >> (8 * (lb & 3) + 4 * (i >> 3))) & 15u;
  const uint32_t high2 = (s[2] >> (8 * (i & 3) + 2 * (i >> 2))) & 3u;
  return low4 | (high2 << 4);
}

// Q3_K (110 B / 256): hmask[32], qs[64] at 32 (placed as Q2_K), 12 bytes of
// 6-bit scales at 96, d at 108.  A clear bit 4n + j of hmask[r % 32]
// subtracts 4 from the 2-bit code; scale i = r/16 has its low four bits in
// nibble (i >= 8) of byte i % 8 and its top two at bits 2(i/4) of byte
// 8 + i%4; w = d * (scale - 32) * q.  The 16 bytes at 94 (two code bytes,
// the scales, d) are loaded together so no load passes the block.
template <> struct Frag<Q3_K> {
  static constexpr int kPat = kHalf64;
  struct Raw { u32x2 qs, hm; u32x4 t; };
  static constexpr int kRuns = 3;
  static constexpr int kRunMax[kRuns] = {32, 32, 16};
  static __device__ __forceinline__ int run_start(int k, int st) {
    const int n = (st & 3) >> 1;
    return (st >> 2) * 110 + (k == 0 ? 0 : k == 1 ? 32 + 32 * n : 94);
  }
  static __device__ __forceinline__ int run_len(int k, int st) {
    (void)st;
    return k == 0 ? 32 : k == 1 ? 32 : 16;
  }
  template <class Rd>
  static __device__ __forceinline__ void gather(const Rd &rd, int st, int G, Raw &r) {
    (void)st;
    r.hm = rd.template get<0, u32x2>(8 * G);
    r.qs = rd.template get<1, u32x2>(8 * G);
    r.t = rd.template get<2, u32x4>(0);
  }
  static __device__ __forceinline__ void decode(const Raw &r, int st, int G, u32x4 &b0, u32x4 &b1) {
    const int q = st & 3, n = q >> 1, j0 = 2 * (q & 1);
    const uint32_t s[3] = {__builtin_amdgcn_alignbyte(r.t[1], r.t[0], 2), __builtin_amdgcn_alignbyte(r.t[2], r.t[1], 2),
                           __builtin_amdgcn_alignbyte(r.t[3], r.t[2], 2)};
    const float d = f16_bits_to_f32(r.t[3] >> 16);
    const int i0 = 8 * n + 2 * j0 + (G >> 1);
    const float a0 = d * (float)((int)scale6(s, i0) - 32), a1 = d * (float)((int)scale6(s, i0 + 2) - 32);
    const int hb = 4 * n + j0;
    const half2v z = {(_Float16)1028.0f, (_Float16)1028.0f};
    uint32_t c0[2], c1[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      c0[i] = ((r.qs[i] >> (2 * j0)) & 0x03030303u) | (((r.hm[i] >> hb) & 0x01010101u) << 2);
      c1[i] = ((r.qs[i] >> (2 * j0 + 2)) & 0x03030303u) | (((r.hm[i] >> (hb + 1)) & 0x01010101u) << 2);
    }
    b0 = scaled_op(c0, z, a0, 0.0f);
    b1 = scaled_op(c1, z, a1, 0.0f);
  }
};

}  // namespace gk
}  // namespace qmm
