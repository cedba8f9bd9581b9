// qmm_device.h -- device-side block geometry and the per-kind element
// decoders shared by the dequant, GEMV, GEMM and expert kernels.
//
// A decoder turns the bytes of one GGUF block into the f32 values of sixteen
// consecutive elements (sub-block `sub` covers elements [16*sub, 16*sub+16)).
// Sixteen elements is the smallest unit every kind decodes without touching a
// neighbouring scale field (ferrox-cuda 0.21.0 mul_mm.rs, SUB and nl(); the
// 16-element split of a 32-element block picks the low or the high nibbles,
// ferrox-cuda 0.20.0 codebook.rs, the IQ4_NL row).
//
// Every value is the f32 rounding of the exact element value.  Each product
// of a scale and an integer is exact in f32 (an f16 significand has 11 bits,
// the integer factors at most 8, 6 and 5 bits), so only the final subtraction
// of the kinds with a minimum rounds.  Factors are multiplied scale first, as
// in (d * sc) * q - dmin * m, so a zero result carries the IEEE sign of that
// product (MXFP4 code 8 is -0.0).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

enum Kind : int {
  Q4_0 = 2, Q5_0 = 6, Q8_0 = 8, Q2_K = 10, Q3_K = 11, Q4_K = 12,
  Q5_K = 13, Q6_K = 14, IQ4_NL = 20, IQ4_XS = 23, MXFP4 = 39
};

template <int KIND> struct Geometry;
template <> struct Geometry<Q8_0>   { static constexpr int bytes = 34,  elems = 32;  };
template <> struct Geometry<Q4_0>   { static constexpr int bytes = 18,  elems = 32;  };
template <> struct Geometry<Q5_0>   { static constexpr int bytes = 22,  elems = 32;  };
template <> struct Geometry<Q2_K>   { static constexpr int bytes = 84,  elems = 256; };
template <> struct Geometry<Q3_K>   { static constexpr int bytes = 110, elems = 256; };
template <> struct Geometry<Q4_K>   { static constexpr int bytes = 144, elems = 256; };
template <> struct Geometry<Q5_K>   { static constexpr int bytes = 176, elems = 256; };
template <> struct Geometry<Q6_K>   { static constexpr int bytes = 210, elems = 256; };
template <> struct Geometry<IQ4_NL> { static constexpr int bytes = 18,  elems = 32;  };
template <> struct Geometry<IQ4_XS> { static constexpr int bytes = 136, elems = 256; };
template <> struct Geometry<MXFP4>  { static constexpr int bytes = 17,  elems = 32;  };

template <int KIND> constexpr int kSubs = Geometry<KIND>::elems / 16;

// ---------------------------------------------------------------------------
// Scalar field reads.  Blocks have odd strides (17, 22, 34, 110, 210 bytes),
// so nothing here assumes more than byte alignment.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t rd8(const uint8_t *p) { return p[0]; }
__device__ __forceinline__ uint32_t rd16(const uint8_t *p) { return (uint32_t)p[0] | ((uint32_t)p[1] << 8); }
__device__ __forceinline__ uint32_t rd32(const uint8_t *p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

// binary16 bits -> f32 with the hardware conversion (exact, subnormals kept).
__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// E8M0 scale byte -> 2^(e-127).  The byte is an f32 exponent field, so
// shifting it into place is exact; e = 0 is the subnormal 2^-127 and e = 255
// is NaN (OCP MX v1.0; ferrox-cuda codebook.rs, ferrox_e8m0_to_f32).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  if (e == 0u) return __builtin_bit_cast(float, 0x00400000u);
  if (e == 255u) return __builtin_bit_cast(float, 0x7fc00000u);
  return __builtin_bit_cast(float, e << 23);
}

__device__ __forceinline__ int sext8(uint32_t b) { return (int)(int8_t)(uint8_t)b; }

// The 16-entry table IQ4_NL and IQ4_XS index (ferrox-cuda codebook.rs,
// KVALUES_IQ4NL) and the E2M1 values MXFP4 indexes (KVALUES_MXFP4; code 8 is
// negative zero).
__device__ __forceinline__ float iq4_value(uint32_t code) {
  constexpr float t[16] = {-127.f, -104.f, -83.f, -65.f, -49.f, -35.f, -22.f, -10.f,
                           1.f, 13.f, 25.f, 38.f, 53.f, 69.f, 89.f, 113.f};
  return t[code & 15u];
}
__device__ __forceinline__ float e2m1_value(uint32_t code) {
  constexpr float t[16] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f,
                           -0.0f, -0.5f, -1.0f, -1.5f, -2.0f, -3.0f, -4.0f, -6.0f};
  return t[code & 15u];
}

// v_perm_b32: byte i of the result is byte sel[i] of the eight bytes
// {hi:lo} (0..3 from lo, 4..7 from hi); selector 12 gives 0x00, 13 gives 0xFF.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// The IQ4_NL table plus 128, one unsigned byte per entry, in four words.
constexpr uint32_t kIq4T0 = 0x3F2D1801u, kIq4T1 = 0x766A5D4Fu, kIq4T2 = 0xA6998D81u, kIq4T3 = 0xF1D9C5B5u;

// Table lookup of four 4-bit indices (one per byte) giving table + 128 per
// byte: entries 0..7 and 8..15 are looked up separately with v_perm and bit 3
// of each index chooses.
__device__ __forceinline__ uint32_t iq4_lookup(uint32_t idx) {
  const uint32_t low3 = idx & 0x07070707u;
  const uint32_t a = perm(kIq4T1, kIq4T0, low3);
  const uint32_t b = perm(kIq4T3, kIq4T2, low3);
  const uint32_t m = perm(0u, 0u, ((idx >> 3) & 0x01010101u) | 0x0C0C0C0Cu);
  return (b & m) | (a & ~m);
}

// Bits 0..3 of x to bit 0 of bytes 0..3 (the four shifted copies of x
// occupy disjoint bit ranges, so the product carries nothing).
__device__ __forceinline__ uint32_t spread4(uint32_t x) { return ((x & 15u) * 0x00204081u) & 0x01010101u; }

// 6-bit scale and min of 32-element group j of the Q4_K/Q5_K 12-byte pack
// (Vulkore quant_test.cpp, ref::q4k_scale_min).
__device__ __forceinline__ void k4_scale_min(const uint8_t *s, int j, int &sc, int &mn) {
  if (j < 4) {
    sc = s[j] & 63;
    mn = s[j + 4] & 63;
  } else {
    sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
    mn = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
  }
}

// ---------------------------------------------------------------------------
// decode16<KIND>(blk, sub, out): elements [16*sub, 16*sub + 16) of the block.
// ---------------------------------------------------------------------------
template <int KIND>
__device__ __forceinline__ void decode16(const uint8_t *__restrict__ b, int sub, float *out);

// Q8_0: f16 d, 32 int8 codes; w = d * q (Vulkore, ref::q8_0).
template <>
__device__ __forceinline__ void decode16<Q8_0>(const uint8_t *__restrict__ b, int sub, float *out) {
  const float d = f16_bits_to_f32(rd16(b));
#pragma unroll
  for (int i = 0; i < 16; ++i) out[i] = d * (float)sext8(b[2 + 16 * sub + i]);
}

// Q4_0: f16 d, 16 bytes of nibbles; sub 0 takes the low nibbles (elements
// 0..15), sub 1 the high nibbles (16..31); w = d * (q - 8).
template <>
__device__ __forceinline__ void decode16<Q4_0>(const uint8_t *__restrict__ b, int sub, float *out) {
  const float d = f16_bits_to_f32(rd16(b));
  const int sh = 4 * sub;
#pragma unroll
  for (int i = 0; i < 16; ++i) out[i] = d * (float)((int)((b[2 + i] >> sh) & 15u) - 8);
}

// Q5_0: f16 d, u32 qh, 16 bytes of nibbles; bit e of qh is element e's fifth
// bit; w = d * (q - 16) (Vulkore, ref::q5_0).
template <>
__device__ __forceinline__ void decode16<Q5_0>(const uint8_t *__restrict__ b, int sub, float *out) {
  const float d = f16_bits_to_f32(rd16(b));
  const uint32_t qh = rd32(b + 2) >> (16 * sub);
  const int sh = 4 * sub;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int q = (int)(((b[6 + i] >> sh) & 15u) | (((qh >> i) & 1u) << 4));
    out[i] = d * (float)(q - 16);
  }
}

// IQ4_NL: f16 d, 16 bytes of codes packed as Q4_0; w = d * table[code].
template <>
__device__ __forceinline__ void decode16<IQ4_NL>(const uint8_t *__restrict__ b, int sub, float *out) {
  const float d = f16_bits_to_f32(rd16(b));
  const int sh = 4 * sub;
#pragma unroll
  for (int i = 0; i < 16; ++i) out[i] = d * iq4_value(b[2 + i] >> sh);
}

// MXFP4: E8M0 byte, 16 bytes of E2M1 codes packed as Q4_0;
// w = 2^(e-127) * e2m1[code].
template <>
__device__ __forceinline__ void decode16<MXFP4>(const uint8_t *__restrict__ b, int sub, float *out) {
  const float s = e8m0_to_f32(b[0]);
  const int sh = 4 * sub;
#pragma unroll
  for (int i = 0; i < 16; ++i) out[i] = s * e2m1_value(b[1 + i] >> sh);
}

// Q4_K: d, dmin, 12-byte scale/min pack, 128 bytes of nibbles in 64-element
// chunks (low nibbles first); w = d*sc*q - dmin*m (Vulkore, ref::q4_k).
template <>
__device__ __forceinline__ void decode16<Q4_K>(const uint8_t *__restrict__ b, int sub, float *out) {
  const float d = f16_bits_to_f32(rd16(b));
  const float dmin = f16_bits_to_f32(rd16(b + 2));
  int sc, mn;
  k4_scale_min(b + 4, sub >> 1, sc, mn);
  const float ds = d * (float)sc, dm = dmin * (float)mn;
  const uint8_t *q = b + 16 + 32 * (sub >> 2) + 16 * (sub & 1);
  const int sh = (sub & 2) ? 4 : 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) out[i] = ds * (float)((q[i] >> sh) & 15u) - dm;
}

// Q5_K: Q4_K plus qh[32] at byte 16 (codes at 48); the fifth bit of element r
// is bit r/32 of qh[r % 32].
template <>
__device__ __forceinline__ void decode16<Q5_K>(const uint8_t *__restrict__ b, int sub, float *out) {
  const float d = f16_bits_to_f32(rd16(b));
  const float dmin = f16_bits_to_f32(rd16(b + 2));
  int sc, mn;
  k4_scale_min(b + 4, sub >> 1, sc, mn);
  const float ds = d * (float)sc, dm = dmin * (float)mn;
  const uint8_t *q = b + 48 + 32 * (sub >> 2) + 16 * (sub & 1);
  const uint8_t *qh = b + 16 + 16 * (sub & 1);
  const int sh = (sub & 2) ? 4 : 0;
  const int hb = sub >> 1;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t v = ((q[i] >> sh) & 15u) | (((uint32_t)(qh[i] >> hb) & 1u) << 4);
    out[i] = ds * (float)v - dm;
  }
}

// Q6_K: ql[128], qh[64], int8 scales[16], f16 d at 208.  Element
// r = 16*sub + i has h = r/128, l = r%32, g = (r%128)/32; its scale is byte
// 192 + sub (Vulkore, ref::q6_k); w = d * sc * (q - 32).
template <>
__device__ __forceinline__ void decode16<Q6_K>(const uint8_t *__restrict__ b, int sub, float *out) {
  const float d = f16_bits_to_f32(rd16(b + 208));
  const int h = sub >> 3, g = (sub & 7) >> 1, l0 = 16 * (sub & 1);
  const float ds = d * (float)sext8(b[192 + sub]);
  const uint8_t *ql = b + 64 * h + 32 * (g & 1) + l0;
  const uint8_t *qh = b + 128 + 32 * h + l0;
  const int sh = (g >= 2) ? 4 : 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int q = (int)(((ql[i] >> sh) & 15u) | (((uint32_t)(qh[i] >> (2 * g)) & 3u) << 4));
    out[i] = ds * (float)(q - 32);
  }
}

// Q2_K: scales[16] (low nibble scale, high nibble min), qs[64], d at 80,
// dmin at 82.  Element r = 16*sub + i: code bits 2*((r%128)/32) of
// qs[32*(r/128) + r%32]; w = d*(s&15)*q - dmin*(s>>4) with s = scales[sub].
template <>
__device__ __forceinline__ void decode16<Q2_K>(const uint8_t *__restrict__ b, int sub, float *out) {
  const float d = f16_bits_to_f32(rd16(b + 80));
  const float dmin = f16_bits_to_f32(rd16(b + 82));
  const uint32_t s = b[sub];
  const float ds = d * (float)(s & 15u), dm = dmin * (float)(s >> 4);
  const int n = sub >> 3, j = (sub & 7) >> 1;
  const uint8_t *q = b + 16 + 32 * n + 16 * (sub & 1);
#pragma unroll
  for (int i = 0; i < 16; ++i) out[i] = ds * (float)((q[i] >> (2 * j)) & 3u) - dm;
}

// Q3_K: hmask[32], qs[64] (placed as Q2_K), 12 bytes of 6-bit scales, d at
// 108.  A clear high-mask bit 4n + j of hmask[r % 32] subtracts 4 from the
// 2-bit code; scale i = sub has its low four bits in byte i (low nibble) or
// byte i-8 (high nibble) and its top two at bits 2*(i/4) of byte 8 + i%4;
// w = d * (scale - 32) * q.
template <>
__device__ __forceinline__ void decode16<Q3_K>(const uint8_t *__restrict__ b, int sub, float *out) {
  const float d = f16_bits_to_f32(rd16(b + 108));
  const uint8_t *sc = b + 96;
  const int low4 = sub < 8 ? (sc[sub] & 15) : (sc[sub - 8] >> 4);
  const int high2 = (sc[8 + (sub & 3)] >> (2 * (sub >> 2))) & 3;
  const float ds = d * (float)((low4 | (high2 << 4)) - 32);
  const int n = sub >> 3, j = (sub & 7) >> 1, l0 = 16 * (sub & 1);
  const uint8_t *q = b + 32 + 32 * n + l0;
  const uint8_t *hm = b + l0;
  const int hb = 4 * n + j;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int q2 = (int)((q[i] >> (2 * j)) & 3u);
    const int v = q2 - (((hm[i] >> hb) & 1u) ? 0 : 4);
    out[i] = ds * (float)v;
  }
}

// IQ4_XS: f16 d, u16 scales_h, scales_l[4], 128 bytes of codes; eight
// 32-element groups packed as IQ4_NL blocks, each with the 6-bit scale
// ls = nibble (ib&1) of scales_l[ib/2] | ((scales_h >> 2ib) & 3) << 4;
// w = d * (ls - 32) * table[code] (ferrox-cuda codebook.rs, the IQ4_XS row).
template <>
__device__ __forceinline__ void decode16<IQ4_XS>(const uint8_t *__restrict__ b, int sub, float *out) {
  const float d = f16_bits_to_f32(rd16(b));
  const uint32_t scales_h = rd16(b + 2);
  const int ib = sub >> 1;
  const uint32_t ls = ((uint32_t)(b[4 + (ib >> 1)] >> (4 * (ib & 1))) & 15u) |
                      (((scales_h >> (2 * ib)) & 3u) << 4);
  const float dl = d * (float)((int)ls - 32);
  const uint8_t *q = b + 8 + 16 * ib;
  const int sh = 4 * (sub & 1);
#pragma unroll
  for (int i = 0; i < 16; ++i) out[i] = dl * iq4_value(q[i] >> sh);
}

// ---------------------------------------------------------------------------
// Wave-level helpers (wave64).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

}  // namespace qmm

// Calls FN.template operator()<KIND>() for the runtime kind.
#define QMM_FOR_EACH_KIND(X) \
  X(Q8_0) X(Q4_0) X(Q5_0) X(Q2_K) X(Q3_K) X(Q4_K) X(Q5_K) X(Q6_K) X(IQ4_NL) X(IQ4_XS) X(MXFP4)
