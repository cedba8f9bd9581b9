// qmm_gemv_mfma.h -- decode GEMV on the matrix cores, for M <= 8 tokens.
//
// Roles.  y[t][n] = sum_k x[t][k] w[n][k] is computed as D = A . B with
// v_mfma_f32_16x16x32_f16: A (16 x 32) holds activations (row i = token i,
// rows >= M are zero), B (32 x 16) holds weights (column j = weight row j of a
// 16-row tile).  In the D layout lane l holds D[4*(l/16) + q][l % 16], so
// every lane's outputs belong to one weight row -- the row whose bytes that
// lane decoded -- and per-row scales are applied with no data exchange.
//
// Exact weights.  The B operand is an exact f16 integer: the block's code
// with its integer sub-block scale folded in where the product fits in f16's
// 11-bit significand (Q4_K: sc*q <= 63*15), or split into two exactly
// representable parts (Q6_K: sc*(q-32) = 16*sh*(q-32) + sl*(q-32), each part
// accumulated on its own and scaled by 16d or d).  The
// remaining f16 super-block scale d multiplies each super-block's partial
// sum in f32, and the Q4_K minimum term -dmin*m_j*X_j runs on
// v_mfma_f32_16x16x4_f32 with exact f32 operands.  The sub-block sums X_j of
// the activations come from extra MFMAs of the same activation fragments
// against a 0/1 indicator, so they cost no vector-ALU work.
//
// Activations.  f32 activations are rounded once to f16 (relative error
// <= 2^-11 per product); f16 activations are used as they are.  With exact
// weights this keeps every output within 1e-3 * sum|w||x| (worst case
// 2^-11 + the f32 accumulation error), and a unit-vector x still returns the
// weight exactly.
//
// Codes to f16 without conversions: OR-ing a nibble into the mantissa of
// f16 1024.0 (0x6400) gives 1024 + q (or 1024 + 16q for a high nibble left in
// place); one packed FMA per pair then removes the offset and applies the
// folded integer scale exactly.
#pragma once

#include "qmm_device.h"

namespace qmm {
namespace gv {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16 bytes from any address (the target allows unaligned vector loads).
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

// Four consecutive activations as loaded (one 16- or 8-byte load).
template <typename XT> struct XVec;
template <> struct XVec<float> { typedef float type __attribute__((ext_vector_type(4))); };
template <> struct XVec<_Float16> { typedef _Float16 type __attribute__((ext_vector_type(4))); };

__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ __forceinline__ uint32_t as_u(half2v h) { return __builtin_bit_cast(uint32_t, h); }

constexpr uint32_t kMagic = 0x64006400u;  // f16 pair (1024, 1024)

// (v & mask) | c.  A gfx9 VOP3 instruction cannot encode two literal
// constants, so with mask and c known the compiler splits this into an AND
// and an OR; the empty asm statements (no instruction) hide their values and
// leave them in registers, and the compiler selects one v_and_or_b32 and
// tracks it like any other VALU write.
__device__ __forceinline__ uint32_t and_or(uint32_t v, uint32_t mask, uint32_t c) {
  asm("" : "+v"(mask));
  asm("" : "+v"(c));
  return (v & mask) | c;
}
// Two f16 values 1024 + field, field = v & mask.
__device__ __forceinline__ uint32_t mag(uint32_t v, uint32_t mask) { return and_or(v, mask, kMagic); }

// Exact fold: fma(e, f, b) is computed exactly and rounded once, and every
// result here is an integer that f16 represents exactly.
__device__ __forceinline__ uint32_t fold(uint32_t e, uint32_t f, uint32_t b) {
  return as_u(__builtin_elementwise_fma(as_h2(e), as_h2(f), as_h2(b)));
}

__device__ __forceinline__ half8 pack8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}

// f32 value of the low or high f16 of a dword.
__device__ __forceinline__ float lo_f16(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu)); }
__device__ __forceinline__ float hi_f16(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16)); }

__device__ __forceinline__ floatx4 mfma16(half8 a, half8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma4f32(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Each decoder describes one k-block (the elements that share the f32
// post-scale) as seen by lane group G = lane / 16 of a 16-row tile:
//   KB, NSTEP            elements per k-block and MFMA steps per k-block
//   NPART                B operands per step (2 for a split fold)
//   HAS_MIN              a minimum term runs on the f32 MFMA
//   x_off(s, G, h)       first of the 4 consecutive elements of half h (0, 1)
//                        of the 8 elements step s gives G; inside a half the
//                        pairs are ordered (0,2), (1,3)
//   STEP_SCALE           every step has its own f32 scale, scale(raw, s):
//                        post_step(acc, D, raw, s) adds it times D after
//                        each step's MFMA (which starts from zero); otherwise
//                        post() below
//   Raw / load           the lane's bytes of one k-block
//   Sc / prep            the lane's scales for that k-block
//   bop(raw, sc, s, p)   B operand p of step s
//   ind(s, G, i)         1 if A-row i collects the sub-block that step s of
//                        group G belongs to (indicator for the sums X_j)
//   post(acc, D, X, sc)  acc += d * D[part] (- dmin * sum m_j X_j)

// Reads from a wave-private LDS copy of the tile's k-block (CHUNKED decoders
// below: the kernel loads the k-block as contiguous 16-byte chunks and stages
// it there), at the natural alignment of each field in the block layout.
// The folded Q4_K and Q6_K decoders load their few 16-byte fields straight
// from global memory instead.
__device__ __forceinline__ uint32_t s16(const uint8_t *p) {
  return *reinterpret_cast<const uint16_t *>(__builtin_assume_aligned(p, 2));
}
__device__ __forceinline__ uint32_t s32a2(const uint8_t *p) { return s16(p) | (s16(p + 2) << 16); }
__device__ __forceinline__ uint32_t s32a1(const uint8_t *p) {
  return (uint32_t)p[0] | (s16(p + 1) << 8) | ((uint32_t)p[3] << 24);  // p odd: p + 1 is even
}

// ---------------------------------------------------------------------------
// Q4_K.  Group G decodes the 32 bytes 32G..32G+31 of the codes: low nibbles
// are elements 64G + [0,32) (sub-block 2G), high nibbles 64G + 32 + [0,32)
// (sub-block 2G+1).  Step s < 4 takes low nibbles of bytes 8s..8s+7, step
// s >= 4 the high nibbles of bytes 8(s-4)..; the B value is sc_j * q.
// ---------------------------------------------------------------------------
struct DecQ4K {
  static constexpr int KB = 256, NSTEP = 8, NPART = 1, BYTES = 144;
  static constexpr bool HAS_MIN = true, CHUNKED = false;
  struct Raw { u32x4 hdr, q0, q1; };
  struct Sc { uint32_t f_lo, b_lo, f_hi, b_hi; float d, mn_lo, mn_hi; };

  static constexpr bool STEP_SCALE = false;
  __device__ static int x_off(int s, int G, int h) { return 64 * G + (s < 4 ? 8 * s : 32 + 8 * (s - 4)) + 4 * h; }

  __device__ static void load(const uint8_t *blk, int G, Raw &r) {
    r.hdr = ld16(blk);
    r.q0 = ld16(blk + 16 + 32 * G);
    r.q1 = ld16(blk + 32 + 32 * G);
  }

  __device__ static Sc prep(const Raw &r, int G) {
    // Scales and mins of sub-blocks 2G, 2G+1 from the 12-byte pack
    // (Vulkore quant_test.cpp, ref::q4k_scale_min), two 8-bit lanes at once.
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
    Sc s;
    // (1024 + sc_lo, 1024 + sc_hi) as an f16 pair, then the integers.
    const half2v scs = as_h2(__builtin_amdgcn_perm(0x64646464u, sc2, 0x07010600u)) - half2v{1024, 1024};
    const half2v f = scs * half2v{1.0f16, 0.0625f16};       // (sc_lo, sc_hi / 16)
    const half2v b2 = scs * half2v{-1024.0f16, -64.0f16};   // offsets to remove
    s.f_lo = as_u(half2v{f[0], f[0]});
    s.b_lo = as_u(half2v{b2[0], b2[0]});
    s.f_hi = as_u(half2v{f[1], f[1]});
    s.b_hi = as_u(half2v{b2[1], b2[1]});
    s.d = lo_f16(r.hdr.x);
    const float dmin = hi_f16(r.hdr.x);
    s.mn_lo = -dmin * (float)(mn2 & 0xFFu);
    s.mn_hi = -dmin * (float)((mn2 >> 8) & 0xFFu);
    return s;
  }

  __device__ static half8 bop(const Raw &r, const Sc &s, int st, int) {
    const int w = st & 3;
    const uint32_t v0 = w < 2 ? (w == 0 ? r.q0.x : r.q0.z) : (w == 2 ? r.q1.x : r.q1.z);
    const uint32_t v1 = w < 2 ? (w == 0 ? r.q0.y : r.q0.w) : (w == 2 ? r.q1.y : r.q1.w);
    const uint32_t mask = st < 4 ? 0x000F000Fu : 0x00F000F0u;
    const uint32_t f = st < 4 ? s.f_lo : s.f_hi, b = st < 4 ? s.b_lo : s.b_hi;
    return pack8(fold(mag(v0, mask), f, b), fold(mag(v0 >> 8, mask), f, b), fold(mag(v1, mask), f, b),
                 fold(mag(v1 >> 8, mask), f, b));
  }

  // A-row 4G' + h collects sub-block 2G' + h; step s of group G is in
  // sub-block 2G + (s >= 4).
  __device__ static bool ind(int s, int G, int i) { return i == 4 * G + (s >= 4 ? 1 : 0); }

  __device__ static floatx4 post(floatx4 acc, const floatx4 *D, floatx4 X, const Sc &s) {
    acc = acc + s.d * D[0];
    acc = mfma4f32(X[0], s.mn_lo, acc);
    acc = mfma4f32(X[1], s.mn_hi, acc);
    return acc;
  }
};

// ---------------------------------------------------------------------------
// Q6_K.  Group G = 2h + a covers half h and byte lane l in 16a..16a+15 of all
// four quarters g (elements 128h + 32g + 16a + [0,16)).  Step s takes
// quarter g = s/2, bytes 8(s%2)..+7 of that range, all in sub-block
// 8h + 2g + a.  The int8 sub-block scale sc = 16*sh + sl (sh in -8..7, sl in
// 0..15) is folded as two exact parts, sh*(q-32) and sl*(q-32), that
// accumulate separately and are scaled by 16d and d.
// ---------------------------------------------------------------------------
struct DecQ6K {
  static constexpr int KB = 256, NSTEP = 8, NPART = 2, BYTES = 210;
  static constexpr bool HAS_MIN = false, CHUNKED = false;
  struct Raw { u32x4 ql0, ql1, qh; u32x2 sc; uint32_t d; };
  struct Sc { uint32_t f[2][4], b[2][4]; float d; };

  static constexpr bool STEP_SCALE = false;
  __device__ static int x_off(int s, int G, int h) {
    return 128 * (G >> 1) + 32 * (s >> 1) + 16 * (G & 1) + 8 * (s & 1) + 4 * h;
  }

  __device__ static void load(const uint8_t *blk, int G, Raw &r) {
    const int h = G >> 1, a = G & 1;
    r.ql0 = ld16(blk + 64 * h + 16 * a);
    r.ql1 = ld16(blk + 64 * h + 32 + 16 * a);
    r.qh = ld16(blk + 128 + 32 * h + 16 * a);
    r.sc = ld8(blk + 192 + 8 * h);
    r.d = rd16(blk + 208);
  }

  __device__ static Sc prep(const Raw &r, int G) {
    // The sub-block of quarter g is 8h + 2g + a: byte a + 2g of the 8 loaded.
    const int a = G & 1;
    const uint32_t lo = a ? (r.sc.x >> 8) : r.sc.x;  // g = 0, 1 at bits 0, 16
    const uint32_t hi = a ? (r.sc.y >> 8) : r.sc.y;  // g = 2, 3
    Sc s;
    s.d = lo_f16(r.d);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int sc = (int)(int8_t)(uint8_t)(((g < 2 ? lo : hi) >> (16 * (g & 1))) & 0xFFu);
      const int part[2] = {sc >> 4, sc & 15};  // sc = 16*sh + sl
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        // Codes arrive as e = 1024 + q (g < 2) or 1024 + 16q (g >= 2):
        // c*(q - 32) = e*c - 1056c, or e*(c/16) - 96c.
        const float c = (float)part[p];
        const _Float16 f = (_Float16)(g < 2 ? c : c * 0.0625f);
        const _Float16 b = (_Float16)(g < 2 ? -1056.0f * c : -96.0f * c);
        s.f[p][g] = as_u(half2v{f, f});
        s.b[p][g] = as_u(half2v{b, b});
      }
    }
    return s;
  }

  __device__ static half8 bop(const Raw &r, const Sc &s, int st, int part) {
    const int g = st >> 1, w = 2 * (st & 1);
    const u32x4 &ql = (g & 1) ? r.ql1 : r.ql0;
    const uint32_t q0 = w == 0 ? ql.x : ql.z, q1 = w == 0 ? ql.y : ql.w;
    const uint32_t h0 = w == 0 ? r.qh.x : r.qh.z, h1 = w == 0 ? r.qh.y : r.qh.w;
    // Low case: nibble at bits 0-3, the two high bits go to 4-5.
    // High case: nibble stays at 4-7, the two high bits go to 8-9.
    const uint32_t qm = g < 2 ? 0x000F000Fu : 0x00F000F0u;
    const uint32_t hm = g < 2 ? 0x00300030u : 0x03000300u;
    const int up = (g & 1) ? 2 : 4;  // moves bits 2g, 2g+1 to 4 (low case) or 8 (high case)
    const uint32_t e0 = and_or(h0 << up, hm, mag(q0, qm));
    const uint32_t e1 = and_or(h0 >> (8 - up), hm, mag(q0 >> 8, qm));
    const uint32_t e2 = and_or(h1 << up, hm, mag(q1, qm));
    const uint32_t e3 = and_or(h1 >> (8 - up), hm, mag(q1 >> 8, qm));
    const uint32_t f = s.f[part][g], b = s.b[part][g];
    return pack8(fold(e0, f, b), fold(e1, f, b), fold(e2, f, b), fold(e3, f, b));
  }

  __device__ static bool ind(int, int, int) { return false; }

  __device__ static floatx4 post(floatx4 acc, const floatx4 *D, floatx4, const Sc &s) {
    return acc + (16.0f * s.d) * D[0] + s.d * D[1];
  }
};

// ---------------------------------------------------------------------------
// The 32-element kinds (and IQ4_XS's 32-element groups).  Every block has its
// own scale, so a step is exactly one block: the B operand holds the block's
// exact integer codes (or table values), the MFMA starts from zero, and the
// block scale multiplies the step's D in f32.  A k-block is 8 blocks.
//
// Nibble kinds: group G takes code bytes 4G..4G+3, whose low nibbles are
// elements 4G..4G+3 and high nibbles 16+4G..16+4G+3 (half 0 and half 1 of
// the group's 8 elements).  Q8_0: group G takes bytes 8G..8G+7.
// ---------------------------------------------------------------------------
struct StepBase {
  static constexpr int KB = 256, NSTEP = 8, NPART = 1;
  static constexpr bool HAS_MIN = false, STEP_SCALE = true, CHUNKED = true;
  struct Sc {};
  __device__ static int x_off(int s, int G, int h) { return 32 * s + 16 * h + 4 * G; }
  __device__ static bool ind(int, int, int) { return false; }
  __device__ static floatx4 post(floatx4 acc, const floatx4 *, floatx4, const Sc &) { return acc; }
};

// Four unsigned bytes u (low-nibble word) and four more (high-nibble word) as
// the B fragment (1024 + u) - off in the order (0,2), (1,3) of each half.
__device__ __forceinline__ half8 bytes_b(uint32_t lo, uint32_t hi, uint32_t off) {
  const uint32_t m = 0x00FF00FFu, one = 0x3C003C00u;
  return pack8(fold(mag(lo, m), one, off), fold(mag(lo >> 8, m), one, off), fold(mag(hi, m), one, off),
               fold(mag(hi >> 8, m), one, off));
}

constexpr uint32_t kNeg1032 = 0xE408E408u;  // f16 pair (-1032, -1032)
constexpr uint32_t kNeg1040 = 0xE410E410u;  // (-1040, -1040)
constexpr uint32_t kNeg1152 = 0xE480E480u;  // (-1152, -1152)

// Q4_0 (18 B): f16 d, 16 code bytes; w = d * (q - 8).
struct DecQ4_0 : StepBase {
  static constexpr int BYTES = 8 * 18;
  struct Raw { uint32_t d[8], q[8]; };
  __device__ static void load(const uint8_t *blk, int G, Raw &r) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      r.d[s] = s16(blk + 18 * s);
      r.q[s] = s32a2(blk + 18 * s + 2 + 4 * G);
    }
  }
  __device__ static Sc prep(const Raw &, int) { return Sc{}; }
  __device__ static half8 bop(const Raw &r, const Sc &, int s, int) {
    return bytes_b(r.q[s] & 0x0F0F0F0Fu, (r.q[s] >> 4) & 0x0F0F0F0Fu, kNeg1032);
  }
  __device__ static float scale(const Raw &r, int s) { return lo_f16(r.d[s]); }
  __device__ static floatx4 post_step(floatx4 acc, floatx4 D, const Raw &r, int s) { return acc + scale(r, s) * D; }
};

// Q5_0 (22 B): f16 d, u32 qh (bit e: fifth bit of element e), 16 code
// bytes; w = d * (q - 16).
struct DecQ5_0 : StepBase {
  static constexpr int BYTES = 8 * 22;
  struct Raw { uint32_t d[8], qh[8], q[8]; };
  __device__ static void load(const uint8_t *blk, int G, Raw &r) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      r.d[s] = s16(blk + 22 * s);
      r.qh[s] = s32a2(blk + 22 * s + 2) >> (4 * G);  // bits 0-3, 16-19: this group's fifth bits
      r.q[s] = s32a2(blk + 22 * s + 6 + 4 * G);
    }
  }
  __device__ static Sc prep(const Raw &, int) { return Sc{}; }
  __device__ static half8 bop(const Raw &r, const Sc &, int s, int) {
    const uint32_t lo = (r.q[s] & 0x0F0F0F0Fu) | (spread4(r.qh[s]) << 4);
    const uint32_t hi = ((r.q[s] >> 4) & 0x0F0F0F0Fu) | (spread4(r.qh[s] >> 16) << 4);
    return bytes_b(lo, hi, kNeg1040);
  }
  __device__ static float scale(const Raw &r, int s) { return lo_f16(r.d[s]); }
  __device__ static floatx4 post_step(floatx4 acc, floatx4 D, const Raw &r, int s) { return acc + scale(r, s) * D; }
};

// Q8_0 (34 B): f16 d, 32 int8 codes; w = d * q.  Code XOR 0x80 = q + 128.
struct DecQ8_0 : StepBase {
  static constexpr int BYTES = 8 * 34;
  struct Raw { uint32_t d[8]; u32x2 q[8]; };
  __device__ static int x_off(int s, int G, int h) { return 32 * s + 8 * G + 4 * h; }
  __device__ static void load(const uint8_t *blk, int G, Raw &r) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      r.d[s] = s16(blk + 34 * s);
      r.q[s] = u32x2{s32a2(blk + 34 * s + 2 + 8 * G), s32a2(blk + 34 * s + 6 + 8 * G)};
    }
  }
  __device__ static Sc prep(const Raw &, int) { return Sc{}; }
  __device__ static half8 bop(const Raw &r, const Sc &, int s, int) {
    return bytes_b(r.q[s].x ^ 0x80808080u, r.q[s].y ^ 0x80808080u, kNeg1152);
  }
  __device__ static float scale(const Raw &r, int s) { return lo_f16(r.d[s]); }
  __device__ static floatx4 post_step(floatx4 acc, floatx4 D, const Raw &r, int s) { return acc + scale(r, s) * D; }
};

// IQ4_NL (18 B): f16 d, 16 code bytes packed as Q4_0; w = d * table[code];
// the B operand is the exact table value.
struct DecIQ4NL : StepBase {
  static constexpr int BYTES = 8 * 18;
  struct Raw { uint32_t d[8], q[8]; };
  __device__ static void load(const uint8_t *blk, int G, Raw &r) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      r.d[s] = s16(blk + 18 * s);
      r.q[s] = s32a2(blk + 18 * s + 2 + 4 * G);
    }
  }
  __device__ static Sc prep(const Raw &, int) { return Sc{}; }
  __device__ static half8 bop(const Raw &r, const Sc &, int s, int) {
    return bytes_b(iq4_lookup(r.q[s] & 0x0F0F0F0Fu), iq4_lookup((r.q[s] >> 4) & 0x0F0F0F0Fu), kNeg1152);
  }
  __device__ static float scale(const Raw &r, int s) { return lo_f16(r.d[s]); }
  __device__ static floatx4 post_step(floatx4 acc, floatx4 D, const Raw &r, int s) { return acc + scale(r, s) * D; }
};

// MXFP4 (17 B): E8M0 byte, 16 E2M1 code bytes packed as Q4_0;
// w = 2^(e-127) * e2m1[code].  The gfx950 scaled FP4 conversion with scale 2
// gives 2 * e2m1 exactly as f16 (an integer of at most 12) for the two
// nibbles of a byte; the block scale 2^(e-128) is applied in f32.
struct DecMXFP4 : StepBase {
  static constexpr int BYTES = 8 * 17;
  struct Raw { uint32_t e[8], q[8]; };
  __device__ static void load(const uint8_t *blk, int G, Raw &r) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      r.e[s] = blk[17 * s];
      r.q[s] = (s & 1) ? s32a2(blk + 17 * s + 1 + 4 * G) : s32a1(blk + 17 * s + 1 + 4 * G);
    }
  }
  __device__ static Sc prep(const Raw &, int) { return Sc{}; }
  __device__ static half8 bop(const Raw &r, const Sc &, int s, int) {
    const uint32_t v = r.q[s];
    const uint32_t p0 = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, 0));
    const uint32_t p1 = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, 1));
    const uint32_t p2 = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, 2));
    const uint32_t p3 = as_u(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 2.0f, 3));
    // p_i = (element 4G+i, element 16+4G+i); regroup as (0,2), (1,3) per half.
    return pack8(perm(p2, p0, 0x05040100u), perm(p3, p1, 0x05040100u), perm(p2, p0, 0x07060302u),
                 perm(p3, p1, 0x07060302u));
  }
  __device__ static float scale(const Raw &r, int s) { return e8m0_to_f32(r.e[s]) * 0.5f; }
  __device__ static floatx4 post_step(floatx4 acc, floatx4 D, const Raw &r, int s) { return acc + scale(r, s) * D; }
};

// IQ4_XS (136 B / 256): f16 d, u16 scales_h, scales_l[4], then eight
// 32-element groups packed as IQ4_NL blocks; one k-block is one super-block
// and step s is group s, scaled by the exact f32 d * (ls_s - 32).
struct DecIQ4XS : StepBase {
  static constexpr int BYTES = 136;
  struct Raw { u32x2 h; uint32_t q[8]; };
  __device__ static void load(const uint8_t *blk, int G, Raw &r) {
    r.h = *reinterpret_cast<const u32x2 *>(__builtin_assume_aligned(blk, 8));
#pragma unroll
    for (int s = 0; s < 8; ++s)
      r.q[s] = *reinterpret_cast<const uint32_t *>(__builtin_assume_aligned(blk + 8 + 16 * s + 4 * G, 4));
  }
  __device__ static Sc prep(const Raw &, int) { return Sc{}; }
  __device__ static half8 bop(const Raw &r, const Sc &, int s, int) {
    return bytes_b(iq4_lookup(r.q[s] & 0x0F0F0F0Fu), iq4_lookup((r.q[s] >> 4) & 0x0F0F0F0Fu), kNeg1152);
  }
  __device__ static float scale(const Raw &r, int s) {
    const float d = lo_f16(r.h.x);
    const uint32_t sh = r.h.x >> 16;
    const uint32_t sl = (r.h.y >> (4 * s)) & 15u;  // nibble s of scales_l
    const int ls = (int)(sl | (((sh >> (2 * s)) & 3u) << 4));
    return d * (float)(ls - 32);
  }
  __device__ static floatx4 post_step(floatx4 acc, floatx4 D, const Raw &r, int s) { return acc + scale(r, s) * D; }
};

// ---------------------------------------------------------------------------
// Q5_K (176 B: d, dmin, the Q4_K scale/min pack, qh[32], qs[128]).  As Q4_K,
// group G decodes code bytes 32G .. 32G + 31 (sub-blocks 2G, 2G + 1); the
// fifth bit of element 64G + l (+ 32) is bit 2G (2G + 1) of qh[l].  The
// B value sc * q, q < 32, is an exact f16 integer (sc * q <= 63 * 31).
// ---------------------------------------------------------------------------
struct DecQ5K {
  static constexpr int KB = 256, NSTEP = 8, NPART = 1, BYTES = 176;
  static constexpr bool HAS_MIN = true, CHUNKED = false, STEP_SCALE = false;
  struct Raw { u32x4 hdr, q0, q1, h0, h1; };
  struct Sc : DecQ4K::Sc { int sh; };  // sh = 2G: this group's fifth-bit position
  __device__ static int x_off(int s, int G, int h) { return DecQ4K::x_off(s, G, h); }
  __device__ static void load(const uint8_t *blk, int G, Raw &r) {
    r.hdr = ld16(blk);
    r.h0 = ld16(blk + 16);
    r.h1 = ld16(blk + 32);
    r.q0 = ld16(blk + 48 + 32 * G);
    r.q1 = ld16(blk + 64 + 32 * G);
  }
  __device__ static Sc prep(const Raw &r, int G) {
    Sc s;
    static_cast<DecQ4K::Sc &>(s) = DecQ4K::prep(DecQ4K::Raw{r.hdr, r.q0, r.q1}, G);
    s.sh = 2 * G;
    return s;
  }
  __device__ static half8 bop(const Raw &r, const Sc &s, int st, int) {
    const int w = st & 3;
    const uint32_t v0 = w < 2 ? (w == 0 ? r.q0.x : r.q0.z) : (w == 2 ? r.q1.x : r.q1.z);
    const uint32_t v1 = w < 2 ? (w == 0 ? r.q0.y : r.q0.w) : (w == 2 ? r.q1.y : r.q1.w);
    // qh bytes 8w .. 8w + 7 hold the fifth bits of these eight elements.
    const uint32_t g0 = w < 2 ? (w == 0 ? r.h0.x : r.h0.z) : (w == 2 ? r.h1.x : r.h1.z);
    const uint32_t g1 = w < 2 ? (w == 0 ? r.h0.y : r.h0.w) : (w == 2 ? r.h1.y : r.h1.w);
    const uint32_t a0 = g0 >> s.sh, a1 = g1 >> s.sh;
    // Low case: the nibble at bits 0-3, the fifth bit (bit 0 of a) to bit 4:
    // e = 1024 + q.  High case: the nibble left at bits 4-7, the fifth bit
    // (bit 1 of a) to bit 8: e = 1024 + 16 q.
    const bool lo = st < 4;
    const uint32_t qm = lo ? 0x000F000Fu : 0x00F000F0u, hm = lo ? 0x00100010u : 0x01000100u;
    const uint32_t e0 = and_or(lo ? a0 << 4 : a0 << 7, hm, mag(v0, qm));
    const uint32_t e1 = and_or(lo ? a0 >> 4 : a0 >> 1, hm, mag(v0 >> 8, qm));
    const uint32_t e2 = and_or(lo ? a1 << 4 : a1 << 7, hm, mag(v1, qm));
    const uint32_t e3 = and_or(lo ? a1 >> 4 : a1 >> 1, hm, mag(v1 >> 8, qm));
    const uint32_t f = lo ? s.f_lo : s.f_hi, b = lo ? s.b_lo : s.b_hi;
    return pack8(fold(e0, f, b), fold(e1, f, b), fold(e2, f, b), fold(e3, f, b));
  }
  __device__ static bool ind(int s, int G, int i) { return DecQ4K::ind(s, G, i); }
  __device__ static floatx4 post(floatx4 acc, const floatx4 *D, floatx4 X, const Sc &s) {
    return DecQ4K::post(acc, D, X, s);
  }
};

// ---------------------------------------------------------------------------
// Q2_K (84 B: scales[16] (low nibble scale, high nibble min), qs[64], d,
// dmin) and Q3_K (110 B: hmask[32], qs[64], twelve bytes of 6-bit scales,
// d).  Element 128n + 32j + l holds bits 2j, 2j + 1 of qs[32n + l]
// (Q3_K: plus the high-mask bit 4n + j of hmask[l]); sixteen sub-blocks of
// 16 elements.  Group G = 2n + a decodes qs bytes 32n + 16a .. + 15, so
// step s = 2j + b (bytes 8b .. 8b + 7, shift 2j) lies in sub-block
// 8n + 2j + a, and group G's four sub-blocks (j = 0 .. 3) take A rows
// 4G + j for their activation sums.
// ---------------------------------------------------------------------------
struct DecQ2K {
  static constexpr int KB = 256, NSTEP = 8, NPART = 1, BYTES = 84;
  static constexpr bool HAS_MIN = true, CHUNKED = false, STEP_SCALE = false;
  struct Raw { u32x4 sc, q; uint32_t dd; };
  struct Sc { uint32_t f[4], b[4]; float d, mn[4]; };
  __device__ static int x_off(int s, int G, int h) { return DecQ6K::x_off(s, G, h); }
  __device__ static void load(const uint8_t *blk, int G, Raw &r) {
    r.sc = ld16(blk);
    r.q = ld16(blk + 16 + 16 * G);
    r.dd = rd32(blk + 80);
  }
  __device__ static Sc prep(const Raw &r, int G) {
    Sc s;
    const float d = lo_f16(r.dd), dmin = hi_f16(r.dd);
    s.d = d;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 8 * (G >> 1) + 2 * j + (G & 1);  // the step's sub-block
      const uint32_t byte = (r.sc[i >> 2] >> (8 * (i & 3))) & 0xFFu;
      const _Float16 c = (_Float16)(float)(byte & 15u);
      s.f[j] = as_u(half2v{c, c});
      s.b[j] = as_u(half2v{-1024.0f16 * c, -1024.0f16 * c});  // c <= 15: exact
      s.mn[j] = -dmin * (float)(byte >> 4);
    }
    return s;
  }
  __device__ static half8 bop(const Raw &r, const Sc &s, int st, int) {
    const int j = st >> 1, b = st & 1;
    const uint32_t v0 = (b ? r.q.z : r.q.x) >> (2 * j), v1 = (b ? r.q.w : r.q.y) >> (2 * j);
    const uint32_t m = 0x00030003u, f = s.f[j], c = s.b[j];
    return pack8(fold(mag(v0, m), f, c), fold(mag(v0 >> 8, m), f, c), fold(mag(v1, m), f, c),
                 fold(mag(v1 >> 8, m), f, c));
  }
  __device__ static bool ind(int s, int G, int i) { return i == 4 * G + (s >> 1); }
  __device__ static floatx4 post(floatx4 acc, const floatx4 *D, floatx4 X, const Sc &s) {
    acc = acc + s.d * D[0];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = mfma4f32(X[q], s.mn[q], acc);
    return acc;
  }
};

struct DecQ3K {
  static constexpr int KB = 256, NSTEP = 8, NPART = 1, BYTES = 110;
  static constexpr bool HAS_MIN = false, CHUNKED = false, STEP_SCALE = false;
  struct Raw { u32x4 hm, q; u32x2 lo; uint32_t hi, d; };
  struct Sc { uint32_t f[4], b[4]; float d; int hb; };  // hb = 4n: this group's high-mask bits
  __device__ static int x_off(int s, int G, int h) { return DecQ6K::x_off(s, G, h); }
  __device__ static void load(const uint8_t *blk, int G, Raw &r) {
    r.hm = ld16(blk + 16 * (G & 1));
    r.q = ld16(blk + 32 + 16 * G);
    r.lo = ld8(blk + 96);
    r.hi = rd32(blk + 104);
    r.d = rd16(blk + 108);
  }
  __device__ static Sc prep(const Raw &r, int G) {
    // Scale i = 8n + 2j + a: low four bits in byte i (n = 0, low nibble) or
    // byte i - 8 (n = 1, high nibble), top two at bits 2 (i / 4) of byte
    // 8 + i % 4; used as sc - 32.  The code v = q2 + 4 h (0 .. 7) arrives
    // at mantissa bits 3-5 (e = 1024 + 8 v), so (sc - 32)(v - 4) =
    // e (sc - 32) / 8 - 132 (sc - 32), both factors exact f16 values.
    const int n = G >> 1, a = G & 1;
    Sc s;
    s.d = lo_f16(r.d);
    s.hb = 4 * n;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = 2 * j + a;  // i - 8n
      const uint32_t lb = (r.lo[k >> 2] >> (8 * (k & 3))) & 0xFFu;
      const int low4 = (int)(n ? lb >> 4 : lb & 15u);
      const int high2 = (int)((r.hi >> (8 * (k & 3) + 2 * (2 * n + (j >> 1)))) & 3u);
      const float v = (float)((low4 | (high2 << 4)) - 32);
      const _Float16 f = (_Float16)(v * 0.125f), c = (_Float16)(v * -132.0f);
      s.f[j] = as_u(half2v{f, f});
      s.b[j] = as_u(half2v{c, c});
    }
    return s;
  }
  __device__ static half8 bop(const Raw &r, const Sc &s, int st, int) {
    const int j = st >> 1, b = st & 1;
    const uint32_t v0 = (b ? r.q.z : r.q.x) >> (2 * j), v1 = (b ? r.q.w : r.q.y) >> (2 * j);
    // The high-mask bits 4n + j of the same eight bytes of hmask.
    const int hs = s.hb + j;
    const uint32_t h0 = (b ? r.hm.z : r.hm.x) >> hs, h1 = (b ? r.hm.w : r.hm.y) >> hs;
    const uint32_t cm = 0x00180018u, hm = 0x00200020u;
    const uint32_t e0 = and_or(h0 << 5, hm, and_or(v0 << 3, cm, kMagic));
    const uint32_t e1 = and_or(h0 >> 3, hm, and_or(v0 >> 5, cm, kMagic));
    const uint32_t e2 = and_or(h1 << 5, hm, and_or(v1 << 3, cm, kMagic));
    const uint32_t e3 = and_or(h1 >> 3, hm, and_or(v1 >> 5, cm, kMagic));
    const uint32_t f = s.f[j], c = s.b[j];
    return pack8(fold(e0, f, c), fold(e1, f, c), fold(e2, f, c), fold(e3, f, c));
  }
  __device__ static bool ind(int, int, int) { return false; }
  __device__ static floatx4 post(floatx4 acc, const floatx4 *D, floatx4, const Sc &s) { return acc + s.d * D[0]; }
};

// A CHUNKED decoder's k-block of one row as 16-byte chunks: lane (j, G)
// loads chunks G, G+4, ... of row j (past the last chunk it re-reads it),
// then stores them into a wave-private LDS copy of the row, from which the
// decoder's load() reads its fields at their natural alignment.
template <typename Dd>
struct Chunks {
  static constexpr int C = (Dd::BYTES + 15) / 16;  // chunks per row (the last may overlap)
  static constexpr int L = (C + 3) / 4;            // chunks per lane
  static constexpr int RS = 16 * C;                // staging bytes per row
  struct Held { u32x4 c[L]; };
  __device__ static int offset(int c) { return c < C - 1 ? 16 * c : Dd::BYTES - 16; }
  __device__ static void load(const uint8_t *blk, int G, Held &h) {
#pragma unroll
    for (int i = 0; i < L; ++i) h.c[i] = ld16(blk + offset(min(4 * i + G, C - 1)));
  }
  __device__ static void stage(uint8_t *row, const Held &h, int G) {
    constexpr int rem = Dd::BYTES - 16 * (C - 1);  // new bytes in the last chunk
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const int c = 4 * i + G;
      if (c >= C) continue;
      const u32x4 v = h.c[i];
      if constexpr (rem == 16) {
        *reinterpret_cast<u32x4 *>(row + 16 * c) = v;
      } else {
        if (c < C - 1) {
          *reinterpret_cast<u32x4 *>(row + 16 * c) = v;
        } else if constexpr (rem == 8) {  // the last chunk overlaps: store its new bytes
          *reinterpret_cast<u32x2 *>(row + 16 * c) = u32x2{v[2], v[3]};
        } else {
          static_assert(rem == 2, "last chunk layout");
          *reinterpret_cast<uint16_t *>(row + 16 * c) = (uint16_t)(v[3] >> 16);
        }
      }
    }
  }
};

template <int KIND> struct Dec;
template <> struct Dec<Q4_K> : DecQ4K {};
template <> struct Dec<Q6_K> : DecQ6K {};
template <> struct Dec<Q4_0> : DecQ4_0 {};
template <> struct Dec<Q5_0> : DecQ5_0 {};
template <> struct Dec<Q8_0> : DecQ8_0 {};
template <> struct Dec<IQ4_NL> : DecIQ4NL {};
template <> struct Dec<MXFP4> : DecMXFP4 {};
template <> struct Dec<IQ4_XS> : DecIQ4XS {};
template <> struct Dec<Q5_K> : DecQ5K {};
template <> struct Dec<Q2_K> : DecQ2K {};
template <> struct Dec<Q3_K> : DecQ3K {};

// ---------------------------------------------------------------------------
// The repacked layout written by qmm_repack.  Tile t (rows 16t .. 16t+15) and
// k-block b form one record of 16 * BYTES bytes at (t * n_kblocks + b) * 16 *
// BYTES.  A record is a run of sections: a lane section is 1024 bytes, slot
// 16 G + j holding the 16 bytes that lane (j, G) decodes; a row section holds
// one field run per row, read alike by the four lanes of that row.  Every
// load below is aligned, and a wave's load of a lane section is 1024
// contiguous bytes.  Rec<KIND>::Packed is what a lane holds between issue and
// decode; unpack() rebuilds the decoder's Raw from it with register moves and
// shifts only.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 lda16(const uint8_t *p) {
  return *reinterpret_cast<const u32x4 *>(__builtin_assume_aligned(p, 16));
}
__device__ __forceinline__ u32x2 lda8(const uint8_t *p) {
  return *reinterpret_cast<const u32x2 *>(__builtin_assume_aligned(p, 8));
}

// Two lane sections of 4-bit codes (Q4_0, IQ4_NL, MXFP4, Q5_0, IQ4_XS): slot
// (G, j) of section c holds code bytes 4G .. 4G+3 of blocks 4c .. 4c+3, one
// dword per block.
struct NibCodes {
  u32x4 c0, c1;
  __device__ void load(const uint8_t *rec, int lane) {
    c0 = lda16(rec + 16 * lane);
    c1 = lda16(rec + 1024 + 16 * lane);
  }
  __device__ uint32_t q(int s) const { return s < 4 ? c0[s] : c1[s - 4]; }
};

template <int KIND> struct Rec;

// Q4_0 and IQ4_NL: codes, then a row section of the eight f16 scales.
template <typename Dd>
struct RecD16 {
  struct Packed { NibCodes c; u32x4 d; };
  __device__ static void load(const uint8_t *rec, int lane, int j, int, Packed &p) {
    p.c.load(rec, lane);
    p.d = lda16(rec + 2048 + 16 * j);
  }
  __device__ static typename Dd::Raw unpack(const Packed &p, int) {
    typename Dd::Raw r;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      r.q[s] = p.c.q(s);
      r.d[s] = p.d[s >> 1] >> (16 * (s & 1));  // the decoder reads the low half
    }
    return r;
  }
};
template <> struct Rec<Q4_0> : RecD16<DecQ4_0> {};
template <> struct Rec<IQ4_NL> : RecD16<DecIQ4NL> {};

// MXFP4: codes, then a row section of the eight E8M0 bytes.
template <> struct Rec<MXFP4> {
  struct Packed { NibCodes c; u32x2 e; };
  __device__ static void load(const uint8_t *rec, int lane, int j, int, Packed &p) {
    p.c.load(rec, lane);
    p.e = lda8(rec + 2048 + 8 * j);
  }
  __device__ static DecMXFP4::Raw unpack(const Packed &p, int) {
    DecMXFP4::Raw r;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      r.q[s] = p.c.q(s);
      r.e[s] = (p.e[s >> 2] >> (8 * (s & 3))) & 0xFFu;
    }
    return r;
  }
};

// Q5_0: codes, the eight 32-bit qh words of the row, then the f16 scales.
template <> struct Rec<Q5_0> {
  struct Packed { NibCodes c; u32x4 h0, h1, d; };
  __device__ static void load(const uint8_t *rec, int lane, int j, int, Packed &p) {
    p.c.load(rec, lane);
    p.h0 = lda16(rec + 2048 + 32 * j);
    p.h1 = lda16(rec + 2048 + 32 * j + 16);
    p.d = lda16(rec + 2560 + 16 * j);
  }
  __device__ static DecQ5_0::Raw unpack(const Packed &p, int G) {
    DecQ5_0::Raw r;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      r.q[s] = p.c.q(s);
      r.qh[s] = (s < 4 ? p.h0[s] : p.h1[s - 4]) >> (4 * G);
      r.d[s] = p.d[s >> 1] >> (16 * (s & 1));
    }
    return r;
  }
};

// Q8_0: four lane sections, section c holding code bytes 8G .. 8G+7 of
// blocks 2c and 2c+1; then the f16 scales.
template <> struct Rec<Q8_0> {
  struct Packed { u32x4 c[4]; u32x4 d; };
  __device__ static void load(const uint8_t *rec, int lane, int j, int, Packed &p) {
#pragma unroll
    for (int c = 0; c < 4; ++c) p.c[c] = lda16(rec + 1024 * c + 16 * lane);
    p.d = lda16(rec + 4096 + 16 * j);
  }
  __device__ static DecQ8_0::Raw unpack(const Packed &p, int) {
    DecQ8_0::Raw r;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      r.q[s] = u32x2{p.c[s >> 1][2 * (s & 1)], p.c[s >> 1][2 * (s & 1) + 1]};
      r.d[s] = p.d[s >> 1] >> (16 * (s & 1));
    }
    return r;
  }
};

// IQ4_XS: codes of the eight groups, then the row's 8-byte header (d,
// scales_h, scales_l).
template <> struct Rec<IQ4_XS> {
  struct Packed { NibCodes c; u32x2 h; };
  __device__ static void load(const uint8_t *rec, int lane, int j, int, Packed &p) {
    p.c.load(rec, lane);
    p.h = lda8(rec + 2048 + 8 * j);
  }
  __device__ static DecIQ4XS::Raw unpack(const Packed &p, int) {
    DecIQ4XS::Raw r;
    r.h = p.h;
#pragma unroll
    for (int s = 0; s < 8; ++s) r.q[s] = p.c.q(s);
    return r;
  }
};

// Q4_K: code bytes 32G .. 32G+15 and 32G+16 .. 32G+31 (sections 0, 1), then
// the row's 16-byte header (d, dmin, the packed scales and mins).
template <> struct Rec<Q4_K> {
  using Packed = DecQ4K::Raw;
  __device__ static void load(const uint8_t *rec, int lane, int j, int, Packed &p) {
    p.q0 = lda16(rec + 16 * lane);
    p.q1 = lda16(rec + 1024 + 16 * lane);
    p.hdr = lda16(rec + 2048 + 16 * j);
  }
  __device__ static Packed unpack(const Packed &p, int) { return p; }
};

// Q6_K: for half h = G/2 and byte lane a = G%2, the low-nibble runs
// 64h + 16a and 64h + 32 + 16a and the high-bit run 128 + 32h + 16a
// (sections 0-2); then the row's sixteen int8 scales and its f16 d.
template <> struct Rec<Q6_K> {
  using Packed = DecQ6K::Raw;
  __device__ static void load(const uint8_t *rec, int lane, int j, int G, Packed &p) {
    p.ql0 = lda16(rec + 16 * lane);
    p.ql1 = lda16(rec + 1024 + 16 * lane);
    p.qh = lda16(rec + 2048 + 16 * lane);
    p.sc = lda8(rec + 3072 + 16 * j + 8 * (G >> 1));
    p.d = *reinterpret_cast<const uint16_t *>(__builtin_assume_aligned(rec + 3328 + 2 * j, 2));
  }
  __device__ static Packed unpack(const Packed &p, int) { return p; }
};

// Q5_K: the Q4_K code sections, then the row's 32 qh bytes and its 16-byte
// header as row sections.
template <> struct Rec<Q5_K> {
  using Packed = DecQ5K::Raw;
  __device__ static void load(const uint8_t *rec, int lane, int j, int, Packed &p) {
    p.q0 = lda16(rec + 16 * lane);
    p.q1 = lda16(rec + 1024 + 16 * lane);
    p.h0 = lda16(rec + 2048 + 32 * j);
    p.h1 = lda16(rec + 2048 + 32 * j + 16);
    p.hdr = lda16(rec + 2560 + 16 * j);
  }
  __device__ static Packed unpack(const Packed &p, int) { return p; }
};

// Q2_K: group G's sixteen code bytes (one lane section), then the row's
// sixteen scale bytes and its f16 d, dmin.
template <> struct Rec<Q2_K> {
  using Packed = DecQ2K::Raw;
  __device__ static void load(const uint8_t *rec, int lane, int j, int, Packed &p) {
    p.q = lda16(rec + 16 * lane);
    p.sc = lda16(rec + 1024 + 16 * j);
    p.dd = *reinterpret_cast<const uint32_t *>(__builtin_assume_aligned(rec + 1280 + 4 * j, 4));
  }
  __device__ static Packed unpack(const Packed &p, int) { return p; }
};

// Q3_K: group G's sixteen code bytes, then the row's hmask (group G reads
// the half 16 (G & 1) ..), scale bytes 0-7 and 8-11, and f16 d.
template <> struct Rec<Q3_K> {
  using Packed = DecQ3K::Raw;
  __device__ static void load(const uint8_t *rec, int lane, int j, int G, Packed &p) {
    p.q = lda16(rec + 16 * lane);
    p.hm = lda16(rec + 1024 + 32 * j + 16 * (G & 1));
    p.lo = lda8(rec + 1536 + 8 * j);
    p.hi = *reinterpret_cast<const uint32_t *>(__builtin_assume_aligned(rec + 1664 + 4 * j, 4));
    p.d = *reinterpret_cast<const uint16_t *>(__builtin_assume_aligned(rec + 1728 + 2 * j, 2));
  }
  __device__ static Packed unpack(const Packed &p, int) { return p; }
};


}  // namespace gv
}  // namespace qmm
