// qmm_gemm_dec.h -- weight decoders for the prefill GEMM: 32 consecutive
// elements of one weight row to f16, each rounded once.
//
// A decoder has two halves so that loads can be issued a pipeline stage
// before the values are needed:
//   Chunk<KIND>::load(row, k0, raw)   global loads of everything the 32
//                                     elements [k0, k0+32) of `row` need;
//   Chunk<KIND>::decode(raw, out)     out[p] = the f16 pair (element 2p,
//                                     element 2p+1) of the chunk.
//
// Blocks have odd strides (17, 18, 22, 34, 136 bytes), so loads are 16-byte
// vector loads at any byte offset; no load reaches past the block it serves.
//
// Integer codes become f16 without conversion instructions: a byte b placed
// in the low mantissa bits of f16 1024.0 (exponent field 0x64) reads as
// 1024 + b, and one packed subtraction leaves the exact code.  Multiplying by
// the f16 scale then rounds once: RN_f16(d * code) is the f16 rounding of the
// exact weight.  Where the scale has more significant bits than f16 can
// carry next to the code (IQ4_XS's d * (ls - 32), the K kinds' d * sc and
// dmin * m), the product is formed exactly in f32 and rounded to f16 at the
// end.
#pragma once

#include "qmm_device.h"

namespace qmm {
namespace gm {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ld16(const uint8_t *p) {
  u32x4 v;
  __builtin_memcpy(&v, p, 16);
  return v;
}
__device__ __forceinline__ u32x2 ld8(const uint8_t *p) {
  u32x2 v;
  __builtin_memcpy(&v, p, 8);
  return v;
}
__device__ __forceinline__ uint32_t ld4(const uint8_t *p) {
  uint32_t v;
  __builtin_memcpy(&v, p, 4);
  return v;
}
__device__ __forceinline__ uint32_t ld2(const uint8_t *p) {
  uint16_t v;
  __builtin_memcpy(&v, p, 2);
  return v;
}

__device__ __forceinline__ half2v h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ __forceinline__ uint32_t bits(half2v h) { return __builtin_bit_cast(uint32_t, h); }
__device__ __forceinline__ half2v splat(uint32_t f16_bits) {
  const _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)f16_bits);
  return half2v{v, v};
}

// Bytes b0..b3 of v as the f16 pairs (1024 + b0, 1024 + b1) and
// (1024 + b2, 1024 + b3).
__device__ __forceinline__ void spread(uint32_t v, uint32_t &p01, uint32_t &p23) {
  p01 = perm(0x64646464u, v, 0x04010400u);
  p23 = perm(0x64646464u, v, 0x04030402u);
}

// (1024 + c) pairs to RN_f16(d * (c - bias)); `off` holds 1024 + bias, so the
// subtraction is exact and the product rounds once.
__device__ __forceinline__ uint32_t affine(uint32_t p, half2v off, half2v d) {
  return bits((h2(p) - off) * d);
}

// Four codes (one per byte) of a low-nibble word and of a high-nibble word
// become out[2i], out[2i+1] (elements 4i..4i+3) and out[8+2i], out[9+2i]
// (elements 16+4i..16+4i+3): the 32-element nibble packing of Q4_0, Q5_0,
// IQ4_NL and MXFP4, where the low nibble of byte j is element j and the high
// nibble element j + 16.
__device__ __forceinline__ void emit(uint32_t lo, uint32_t hi, int i, half2v off, half2v d, uint32_t *out) {
  uint32_t a, b;
  spread(lo, a, b);
  out[2 * i] = affine(a, off, d);
  out[2 * i + 1] = affine(b, off, d);
  spread(hi, a, b);
  out[8 + 2 * i] = affine(a, off, d);
  out[9 + 2 * i] = affine(b, off, d);
}

template <int KIND> struct Chunk;

// Q8_0 (34 B / 32): f16 d, 32 int8 codes; w = d * q.  A code XOR 0x80 is
// q + 128 as an unsigned byte.
template <> struct Chunk<Q8_0> {
  struct Raw { uint32_t d; u32x4 q0, q1; };
  static __device__ __forceinline__ void load(const uint8_t *row, int k0, Raw &r) {
    const uint8_t *b = row + (int64_t)(k0 >> 5) * 34;
    r.d = ld2(b);
    r.q0 = ld16(b + 2);
    r.q1 = ld16(b + 18);
  }
  static __device__ __forceinline__ void decode(const Raw &r, uint32_t *out) {
    const half2v d = splat(r.d), off = {(_Float16)1152.0f, (_Float16)1152.0f};
    const uint32_t w[8] = {r.q0[0], r.q0[1], r.q0[2], r.q0[3], r.q1[0], r.q1[1], r.q1[2], r.q1[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t a, b;
      spread(w[i] ^ 0x80808080u, a, b);
      out[2 * i] = affine(a, off, d);
      out[2 * i + 1] = affine(b, off, d);
    }
  }
};

// Q4_0 (18 B / 32): f16 d, 16 bytes of nibbles; w = d * (q - 8).
template <> struct Chunk<Q4_0> {
  struct Raw { uint32_t d; u32x4 q; };
  static __device__ __forceinline__ void load(const uint8_t *row, int k0, Raw &r) {
    const uint8_t *b = row + (int64_t)(k0 >> 5) * 18;
    r.d = ld2(b);
    r.q = ld16(b + 2);
  }
  static __device__ __forceinline__ void decode(const Raw &r, uint32_t *out) {
    const half2v d = splat(r.d), off = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) emit(r.q[i] & 0x0F0F0F0Fu, (r.q[i] >> 4) & 0x0F0F0F0Fu, i, off, d, out);
  }
};

// Q5_0 (22 B / 32): f16 d, u32 qh, 16 bytes of nibbles; bit e of qh is the
// fifth bit of element e; w = d * (q - 16).
template <> struct Chunk<Q5_0> {
  struct Raw { uint32_t d, qh; u32x4 q; };
  static __device__ __forceinline__ void load(const uint8_t *row, int k0, Raw &r) {
    const uint8_t *b = row + (int64_t)(k0 >> 5) * 22;
    r.d = ld2(b);
    r.qh = ld4(b + 2);
    r.q = ld16(b + 6);
  }
  static __device__ __forceinline__ void decode(const Raw &r, uint32_t *out) {
    const half2v d = splat(r.d), off = {(_Float16)1040.0f, (_Float16)1040.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = (r.q[i] & 0x0F0F0F0Fu) | (spread4(r.qh >> (4 * i)) << 4);
      const uint32_t hi = ((r.q[i] >> 4) & 0x0F0F0F0Fu) | (spread4(r.qh >> (16 + 4 * i)) << 4);
      emit(lo, hi, i, off, d, out);
    }
  }
};

// IQ4_NL (18 B / 32): f16 d, 16 bytes of codes packed as Q4_0;
// w = d * table[code].  The table value plus 128 is an unsigned byte.
template <> struct Chunk<IQ4_NL> {
  struct Raw { uint32_t d; u32x4 q; };
  static __device__ __forceinline__ void load(const uint8_t *row, int k0, Raw &r) {
    const uint8_t *b = row + (int64_t)(k0 >> 5) * 18;
    r.d = ld2(b);
    r.q = ld16(b + 2);
  }
  static __device__ __forceinline__ void decode(const Raw &r, uint32_t *out) {
    const half2v d = splat(r.d), off = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      emit(iq4_lookup(r.q[i] & 0x0F0F0F0Fu), iq4_lookup((r.q[i] >> 4) & 0x0F0F0F0Fu), i, off, d, out);
  }
};

// MXFP4 (17 B / 32): E8M0 scale byte, 16 bytes of E2M1 codes packed as
// Q4_0; w = 2^(e-127) * e2m1[code].  The gfx950 scaled FP4 conversion turns
// the two nibbles of one byte (elements j and j + 16) into an f16 pair, each
// the f16 rounding of scale * e2m1; a byte permute regroups the pairs in k
// order.
template <> struct Chunk<MXFP4> {
  struct Raw { uint32_t e; u32x4 q; };
  static __device__ __forceinline__ void load(const uint8_t *row, int k0, Raw &r) {
    const uint8_t *b = row + (int64_t)(k0 >> 5) * 17;
    r.e = b[0];
    r.q = ld16(b + 1);
  }
  static __device__ __forceinline__ void decode(const Raw &r, uint32_t *out) {
    const float s = e8m0_to_f32(r.e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t p0 = bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r.q[i], s, 0));
      const uint32_t p1 = bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r.q[i], s, 1));
      const uint32_t p2 = bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r.q[i], s, 2));
      const uint32_t p3 = bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(r.q[i], s, 3));
      out[2 * i] = perm(p1, p0, 0x05040100u);
      out[2 * i + 1] = perm(p3, p2, 0x05040100u);
      out[8 + 2 * i] = perm(p1, p0, 0x07060302u);
      out[9 + 2 * i] = perm(p3, p2, 0x07060302u);
    }
  }
};

// Four unsigned bytes times `a`, minus `b`, each formed exactly in f32 and
// rounded once to f16: out pairs (byte0, byte1), (byte2, byte3).
__device__ __forceinline__ void fma_bytes(uint32_t v, float a, float b, uint32_t &p01, uint32_t &p23) {
  const float v0 = __builtin_fmaf(a, (float)(v & 0xFFu), b);
  const float v1 = __builtin_fmaf(a, (float)((v >> 8) & 0xFFu), b);
  const float v2 = __builtin_fmaf(a, (float)((v >> 16) & 0xFFu), b);
  const float v3 = __builtin_fmaf(a, (float)(v >> 24), b);
  p01 = bits(half2v{(_Float16)v0, (_Float16)v1});
  p23 = bits(half2v{(_Float16)v2, (_Float16)v3});
}

// IQ4_XS (136 B / 256): f16 d, u16 scales_h, scales_l[4], then eight
// 32-element groups packed as IQ4_NL blocks; w = d * (ls - 32) * table[code]
// (ferrox-cuda codebook.rs, the IQ4_XS row).  dl = d * (ls - 32) has at most
// 17 significant bits and table + 128 fits a byte, so
// fma(dl, table + 128, -128 dl) is the exact weight before the f16 rounding.
template <> struct Chunk<IQ4_XS> {
  struct Raw { u32x2 h; u32x4 q; int ib; };
  static __device__ __forceinline__ void load(const uint8_t *row, int k0, Raw &r) {
    const uint8_t *b = row + (int64_t)(k0 >> 8) * 136;
    r.ib = (k0 >> 5) & 7;
    r.h = ld8(b);
    r.q = ld16(b + 8 + 16 * r.ib);
  }
  static __device__ __forceinline__ void decode(const Raw &r, uint32_t *out) {
    const float d = f16_bits_to_f32(r.h[0] & 0xFFFFu);
    const uint32_t sh = r.h[0] >> 16;
    const uint32_t sl = (r.h[1] >> (8 * (r.ib >> 1) + 4 * (r.ib & 1))) & 15u;
    const int ls = (int)(sl | (((sh >> (2 * r.ib)) & 3u) << 4));
    const float dl = d * (float)(ls - 32), nb = -128.0f * dl;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fma_bytes(iq4_lookup(r.q[i] & 0x0F0F0F0Fu), dl, nb, out[2 * i], out[2 * i + 1]);
      fma_bytes(iq4_lookup((r.q[i] >> 4) & 0x0F0F0F0Fu), dl, nb, out[8 + 2 * i], out[9 + 2 * i]);
    }
  }
};

// Q4_K (144 B / 256): d, dmin, 12-byte 6-bit scale/min pack, 128 bytes of
// codes; group j (elements 32j..32j+31) is the low (j even) or high (j odd)
// nibbles of bytes 32*(j/2) .. +31 of the codes (Vulkore quant_test.cpp,
// ref::q4_k); w = d*sc*q - dmin*m, with d*sc and dmin*m exact in f32.
template <> struct Chunk<Q4_K> {
  struct Raw { u32x4 h, q0, q1; int j; };
  static __device__ __forceinline__ void load(const uint8_t *row, int k0, Raw &r) {
    const uint8_t *b = row + (int64_t)(k0 >> 8) * 144;
    r.j = (k0 >> 5) & 7;
    r.h = ld16(b);
    r.q0 = ld16(b + 16 + 32 * (r.j >> 1));
    r.q1 = ld16(b + 32 + 32 * (r.j >> 1));
  }
  static __device__ __forceinline__ uint32_t sbyte(const Raw &r, int i) {
    return (r.h[1 + (i >> 2)] >> (8 * (i & 3))) & 0xFFu;  // byte i of the 12-byte pack
  }
  static __device__ __forceinline__ void decode(const Raw &r, uint32_t *out) {
    const float d = f16_bits_to_f32(r.h[0] & 0xFFFFu), dmin = f16_bits_to_f32(r.h[0] >> 16);
    const int j = r.j;
    uint32_t sc, mn;
    if (j < 4) {
      sc = sbyte(r, j) & 63u;
      mn = sbyte(r, j + 4) & 63u;
    } else {
      sc = (sbyte(r, j + 4) & 15u) | ((sbyte(r, j - 4) >> 6) << 4);
      mn = (sbyte(r, j + 4) >> 4) | ((sbyte(r, j) >> 6) << 4);
    }
    const float a = d * (float)sc, b = -(dmin * (float)mn);
    const int s = 4 * (j & 1);
    const uint32_t w[8] = {r.q0[0], r.q0[1], r.q0[2], r.q0[3], r.q1[0], r.q1[1], r.q1[2], r.q1[3]};
#pragma unroll
    for (int i = 0; i < 8; ++i) fma_bytes((w[i] >> s) & 0x0F0F0F0Fu, a, b, out[2 * i], out[2 * i + 1]);
  }
};

// The other kinds decode through the shared f32 decoders straight from
// global memory (each value exact or rounded once in f32, then to f16).
template <int KIND> struct Chunk {
  struct Raw { const uint8_t *b; int sub; };
  static __device__ __forceinline__ void load(const uint8_t *row, int k0, Raw &r) {
    r.b = row + (int64_t)(k0 / Geometry<KIND>::elems) * Geometry<KIND>::bytes;
    r.sub = (k0 % Geometry<KIND>::elems) >> 4;
  }
  static __device__ __forceinline__ void decode(const Raw &r, uint32_t *out) {
    float w[32];
    decode16<KIND>(r.b, r.sub, w);
    decode16<KIND>(r.b, r.sub + 1, w + 16);
#pragma unroll
    for (int p = 0; p < 16; ++p) out[p] = bits(half2v{(_Float16)w[2 * p], (_Float16)w[2 * p + 1]});
  }
};

}  // namespace gm
}  // namespace qmm
