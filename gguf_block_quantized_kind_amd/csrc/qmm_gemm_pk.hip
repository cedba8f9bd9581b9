// qmm_gemm_pk.hip -- prefill GEMM over repacked weights (the records of
// qmm_repack): every operand reaches the matrix cores straight from global
// memory, with no LDS staging in the main loop.
//
// C[M][N] = A[M][K] . W^T.  A workgroup of four waves owns a tile of
// 16 TM tokens by 16 TN weight rows; each wave computes the whole tile over
// its own quarter of K, and the four partial tiles are summed through LDS
// at the end in a fixed order (deterministic).  A record holds a 16-row
// tile's 256-element k-block with its code bytes already in the lanes'
// order: lane section c, 16-byte slot 16 G + j is what lane (j, G) of
// v_mfma_f32_16x16x32_f16 needs for row j, so one wave-wide 16-byte load of
// a section is one contiguous kilobyte.  The activations are loaded in the
// matching order (lane (i, G): token i, the eight elements its weight lane
// holds), 16 bytes per lane.  Per stage (one lane section) a wave issues the
// next stage's loads, then decodes each row tile's codes to f16 in registers
// and runs its products against the TM token tiles.
//
// Rows of a partial last tile are padding in the records (zero codes) and
// are never stored; tokens past M read token M - 1 and are never stored.
// Workgroups are numbered so that the token tiles of one weight tile run on
// one XCD (workgroup i runs on XCD i mod 8) and read it through one L2.
//
// Numerics: each weight is rounded once to f16 (d * q, the exact code times
// the f16 block scale); f16 activations are exact; f32 activations are split
// into hi = RN_f16(a) and lo = RN_f16(a - hi), both multiplied; f32
// accumulation.
#include <stdlib.h>

#include "qmm_gemm_dec.h"
#include "qmm_internal.h"

namespace qmm {
namespace pk {

using gm::half2v;
using gm::u32x2;
using gm::u32x4;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;  // buffer descriptor word 3 (raw 32-bit data)
// s_waitcnt immediate that waits until at most n vector-memory operations
// are outstanding (expcnt and lgkmcnt at their maxima: no wait on them).
__host__ __device__ constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kRing = 4;  // stages in flight: the one computed and three loading

__device__ __forceinline__ half8 as_h8(u32x4 v) { return __builtin_bit_cast(half8, v); }

// Per-kind view of a record (qmm_repack): a k-block of 256 elements is
// kRing stages of two matrix-core steps (32 elements, one GGUF block) each.
// Rows<KIND, TN> holds a wave's weight registers for TN row tiles: what it
// loads at each ring position u of a k-block (into k-block buffer p), how
// many vector-memory operations that is per row tile (loads(u)), and the
// f16 B operand of step h of stage u, whose eight elements per lane group
// G are the k-block elements given by a_part(u, h, G, e) (activation parts
// e of kParts, each kPartElems elements long).
template <int KIND, int TN> struct Rows;

__device__ __forceinline__ u32x4 ld_b128(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ u32x2 ld_b64(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// Q8_0: lane section c, slot (G, j) holds codes 8G .. 8G+7 of blocks 2c and
// 2c+1 of row j (one section per stage); row j's row section holds its
// eight f16 block scales at 4096 + 16 j.  Step h of stage u is block 2u + h,
// lane group G's elements 8G .. 8G+7 of it.
template <int TN> struct Rows<Q8_0, TN> {
  static constexpr int kRec = 16 * 272;
  static constexpr bool kPostScale = false;
  static constexpr int kParts = 1, kPartElems = 8;
  static __device__ __forceinline__ int a_part(int u, int h, int G, int) { return 64 * u + 32 * h + 8 * G; }
  static constexpr int loads(int u) { return u == 0 ? 2 : 1; }
  u32x4 w[kRing][TN], s[2][TN];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int lane, int j, const int (&rec)[TN], int wk, int u,
                                       int p) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) w[u][tn] = ld_b128(r, 16 * lane, rec[tn] + wk + 1024 * u);
    if (u == 0) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) s[p][tn] = ld_b128(r, 4096 + 16 * j, rec[tn] + wk);
    }
  }
  __device__ __forceinline__ u32x4 b(int u, int p, int tn, int h, int) const {
    const uint32_t sc = s[p][tn][u];
    const half2v d = gm::splat(h ? sc >> 16 : sc & 0xFFFFu), off = {(_Float16)1152.0f, (_Float16)1152.0f};
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t p01, p23;
      gm::spread(w[u][tn][2 * h + q] ^ 0x80808080u, p01, p23);
      out[2 * q] = gm::affine(p01, off, d);
      out[2 * q + 1] = gm::affine(p23, off, d);
    }
    return out;
  }
};

// The 32-element nibble kinds: lane section c, slot (G, j), dword w holds
// code bytes 4G .. 4G+3 of block 4c + w of row j, i.e. elements 4G .. 4G+3
// (low nibbles) and 16+4G .. 16+4G+3 (high nibbles).  Sections 0 and 1 are
// loaded at ring positions 0 and 2; step h of stage u is block 2u + h, dword
// 2 (u mod 2) + h of section u / 2, and lane group G's activations are the
// two runs of four at 4G and 16 + 4G of that block.
template <int KIND, int TN> struct NibRows {
  static constexpr int kParts = 2, kPartElems = 4;
  static constexpr bool kPostScale = false;  // B carries the block scale
  static __device__ __forceinline__ int a_part(int u, int h, int G, int e) { return 64 * u + 32 * h + 16 * e + 4 * G; }
  u32x4 w[2][2][TN];
  __device__ __forceinline__ void load_sections(__amdgpu_buffer_rsrc_t r, int lane, const int (&rec)[TN], int wk, int u,
                                                int p) {
    if (u == 0 || u == 2) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) w[p][u / 2][tn] = ld_b128(r, 16 * lane, rec[tn] + wk + 512 * u);
    }
  }
  __device__ __forceinline__ uint32_t codes(int u, int p, int tn, int h) const { return w[p][u / 2][tn][2 * (u & 1) + h]; }
  // The f16 pairs of (lo, hi): four biased integer codes per byte of each,
  // minus `off`, times d, each rounded once.
  static __device__ __forceinline__ u32x4 affine8(uint32_t lo, uint32_t hi, half2v off, half2v d) {
    uint32_t a, c, e, f;
    gm::spread(lo, a, c);
    gm::spread(hi, e, f);
    return u32x4{gm::affine(a, off, d), gm::affine(c, off, d), gm::affine(e, off, d), gm::affine(f, off, d)};
  }
};

// Q4_0: row section at 2048 + 16 j, the eight f16 block scales; w = d (q - 8).
template <int TN> struct Rows<Q4_0, TN> : NibRows<Q4_0, TN> {
  using B = NibRows<Q4_0, TN>;
  static constexpr int kRec = 16 * 144;
  static constexpr int loads(int u) { return u == 0 ? 2 : u == 2 ? 1 : 0; }
  u32x4 s[2][TN];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int lane, int j, const int (&rec)[TN], int wk, int u,
                                       int p) {
    B::load_sections(r, lane, rec, wk, u, p);
    if (u == 0) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) s[p][tn] = ld_b128(r, 2048 + 16 * j, rec[tn] + wk);
    }
  }
  __device__ __forceinline__ u32x4 b(int u, int p, int tn, int h, int) const {
    const uint32_t sc = s[p][tn][u], q = B::codes(u, p, tn, h);
    const half2v d = gm::splat(h ? sc >> 16 : sc & 0xFFFFu), off = {(_Float16)1032.0f, (_Float16)1032.0f};
    return B::affine8(q & 0x0F0F0F0Fu, (q >> 4) & 0x0F0F0F0Fu, off, d);
  }
};

// IQ4_NL: as Q4_0, w = d * table[code] (the table value plus 128 is a byte).
template <int TN> struct Rows<IQ4_NL, TN> : Rows<Q4_0, TN> {
  using B = NibRows<IQ4_NL, TN>;
  __device__ __forceinline__ u32x4 b(int u, int p, int tn, int h, int) const {
    const uint32_t sc = this->s[p][tn][u], q = this->w[p][u / 2][tn][2 * (u & 1) + h];
    const half2v d = gm::splat(h ? sc >> 16 : sc & 0xFFFFu), off = {(_Float16)1152.0f, (_Float16)1152.0f};
    return B::affine8(iq4_lookup(q & 0x0F0F0F0Fu), iq4_lookup((q >> 4) & 0x0F0F0F0Fu), off, d);
  }
};

// Q5_0: row sections at 2048 + 32 j (eight 32-bit qh words, bit e the fifth
// bit of element e) and 2560 + 16 j (eight f16 scales); w = d (q - 16).  Each
// stage loads the two qh words of its blocks.
template <int TN> struct Rows<Q5_0, TN> : NibRows<Q5_0, TN> {
  using B = NibRows<Q5_0, TN>;
  static constexpr int kRec = 16 * 176;
  static constexpr int loads(int u) { return u == 0 ? 3 : u == 2 ? 2 : 1; }
  u32x4 s[2][TN];
  u32x2 qh[kRing][TN];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int lane, int j, const int (&rec)[TN], int wk, int u,
                                       int p) {
    B::load_sections(r, lane, rec, wk, u, p);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) qh[u][tn] = ld_b64(r, 2048 + 32 * j, rec[tn] + wk + 8 * u);
    if (u == 0) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) s[p][tn] = ld_b128(r, 2560 + 16 * j, rec[tn] + wk);
    }
  }
  __device__ __forceinline__ u32x4 b(int u, int p, int tn, int h, int G) const {
    const uint32_t sc = s[p][tn][u], q = B::codes(u, p, tn, h), hb = qh[u][tn][h];
    const half2v d = gm::splat(h ? sc >> 16 : sc & 0xFFFFu), off = {(_Float16)1040.0f, (_Float16)1040.0f};
    const uint32_t lo = (q & 0x0F0F0F0Fu) | (spread4(hb >> (4 * G)) << 4);
    const uint32_t hi = ((q >> 4) & 0x0F0F0F0Fu) | (spread4(hb >> (16 + 4 * G)) << 4);
    return B::affine8(lo, hi, off, d);
  }
};

// MXFP4: row section at 2048 + 8 j, the eight E8M0 bytes; w = 2^(e - 127)
// e2m1[code], each the f16 rounding of the scaled value (gfx950's scaled FP4
// conversion takes a byte's two nibbles, elements 4G + i and 16 + 4G + i).
template <int TN> struct Rows<MXFP4, TN> : NibRows<MXFP4, TN> {
  using B = NibRows<MXFP4, TN>;
  static constexpr int kRec = 16 * 136;
  static constexpr int loads(int u) { return u == 0 ? 2 : u == 2 ? 1 : 0; }
  u32x2 s[2][TN];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int lane, int j, const int (&rec)[TN], int wk, int u,
                                       int p) {
    B::load_sections(r, lane, rec, wk, u, p);
    if (u == 0) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) s[p][tn] = ld_b64(r, 2048 + 8 * j, rec[tn] + wk);
    }
  }
  __device__ __forceinline__ u32x4 b(int u, int p, int tn, int h, int) const {
    const int blk = 2 * u + h;
    const float sc = e8m0_to_f32((s[p][tn][blk >> 2] >> (8 * (blk & 3))) & 0xFFu);
    const uint32_t q = B::codes(u, p, tn, h);
    const uint32_t p0 = gm::bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, sc, 0));
    const uint32_t p1 = gm::bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, sc, 1));
    const uint32_t p2 = gm::bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, sc, 2));
    const uint32_t p3 = gm::bits(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, sc, 3));
    return u32x4{perm(p1, p0, 0x05040100u), perm(p3, p2, 0x05040100u), perm(p1, p0, 0x07060302u),
                 perm(p3, p2, 0x07060302u)};
  }
};

// IQ4_XS: row section at 2048 + 8 j, the super-block header (f16 d,
// scales_h, scales_l).  Group s's scale d * (ls_s - 32) is exact in f32 but
// not in f16, so B is the exact table value and the scale multiplies each
// step's product in f32 (kPostScale).
template <int TN> struct Rows<IQ4_XS, TN> : NibRows<IQ4_XS, TN> {
  using B = NibRows<IQ4_XS, TN>;
  static constexpr int kRec = 16 * 136;
  static constexpr bool kPostScale = true;
  static constexpr int loads(int u) { return u == 0 ? 2 : u == 2 ? 1 : 0; }
  u32x2 s[2][TN];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int lane, int j, const int (&rec)[TN], int wk, int u,
                                       int p) {
    B::load_sections(r, lane, rec, wk, u, p);
    if (u == 0) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) s[p][tn] = ld_b64(r, 2048 + 8 * j, rec[tn] + wk);
    }
  }
  __device__ __forceinline__ u32x4 b(int u, int p, int tn, int h, int) const {
    const uint32_t q = B::codes(u, p, tn, h);
    const half2v one = {(_Float16)1.0f, (_Float16)1.0f}, off = {(_Float16)1152.0f, (_Float16)1152.0f};
    return B::affine8(iq4_lookup(q & 0x0F0F0F0Fu), iq4_lookup((q >> 4) & 0x0F0F0F0Fu), off, one);
  }
  __device__ __forceinline__ float scale(int u, int p, int tn, int h) const {
    const int g = 2 * u + h;
    const uint32_t x = s[p][tn][0], y = s[p][tn][1];
    const uint32_t ls = ((y >> (4 * g)) & 15u) | (((x >> (16 + 2 * g)) & 3u) << 4);
    return f16_bits_to_f32(x & 0xFFFFu) * (float)((int)ls - 32);
  }
};

// Direct-to-LDS 16-byte buffer load: lane l's 16 bytes land at lds + 16 l.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t *lds, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}

// Activation staging of one k part for one stage (64 elements of K for
// each of the 16 TM tokens): CPT 16-byte chunks per token, stored
// token-major with chunk p of token t at position p ^ (t mod KEYP), so that
// the tokens one fragment read touches fall in different banks (KEYP divides
// the tokens per load, so one lane offset serves every load of a stage).
template <typename AT, int TM>
struct AStage {
  static constexpr int CPT = 64 * (int)sizeof(AT) / 16;  // chunks per token
  static constexpr int TPL = 64 / CPT;                   // tokens per wave-wide load
  static constexpr int KEYP = CPT < TPL ? CPT : TPL;     // swizzle period
  static constexpr int NLD = 16 * TM / TPL;              // loads per stage
  static constexpr int BYTES = 16 * TM * 64 * (int)sizeof(AT);
};

// Workgroup of KQ x NH waves: wave (q, h) = (wave / NH, wave % NH) computes
// token rows m0 .. m0 + 16 TM - 1 against weight rows n0 + 16 TN h ..
// + 16 TN - 1 over k-blocks q nkb / KQ .. (q + 1) nkb / KQ - 1 (KQ divides
// nkb, so every wave runs as many stages).  The NH waves of one part share
// its activation staging: each issues 1 / NH of the loads, and a workgroup
// barrier per stage makes the others' loads visible.
//
// Pipeline: kRing stages in flight.  Stage t issues the loads of stage
// t + kRing - 1 (its share of the activations into the part's LDS buffer,
// its weight sections into register slot (t + kRing - 1) mod kRing, and at
// a k-block's first section that k-block's scale rows), multiplies its two
// steps, then waits for stage t + 1's loads, passes the barrier and reads
// stage t + 1's first fragments, so that LDS reads overlap the products in
// flight.  Stage s of a wave is section s mod kRing of its k-block
// kb0 + s / kRing (kRing equals the section count), so the register slots
// and scale-row buffers are fixed per unrolled position.
template <int KIND, typename AT, int TM, int TN, int KQ, int NH>
__global__ __launch_bounds__(64 * KQ * NH, 1) void gemm_pk_kernel(const uint8_t *__restrict__ P,
                                                                  const AT *__restrict__ A, float *__restrict__ C,
                                                                  int M, int N, int K, int tiles_m) {
  using R = Rows<KIND, TN>;
  using AS = AStage<AT, TM>;
  constexpr bool kF32 = sizeof(AT) == 4;
  constexpr int KW = KQ * NH;
  static_assert(AS::NLD % NH == 0, "staging loads split evenly");
  // One LDS array per ring position (the k parts' buffers side by side),
  // so that the compiler, which orders LDS reads after direct-to-LDS loads
  // into the same array only, lets a stage's fragment reads run while the
  // loads into the other positions are in flight.  The empty asm makes the
  // arrays escape: the direct loads write them.
  __shared__ __attribute__((aligned(16))) uint8_t ring0[KQ * AS::BYTES], ring1[KQ * AS::BYTES],
      ring2[KQ * AS::BYTES], ring3[KQ * AS::BYTES];
  asm volatile("" ::"v"(ring0), "v"(ring1), "v"(ring2), "v"(ring3) : "memory");
  auto ring = [&](int u) -> uint8_t * { return u == 0 ? ring0 : u == 1 ? ring1 : u == 2 ? ring2 : ring3; };
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wq = wave / NH, wh = wave % NH;
  const int G = lane >> 4, j = lane & 15;

  // Tile of this workgroup: XCD x = i mod 8 receives a contiguous range of
  // tile numbers, token tiles fastest.
  const int T = gridDim.x, L = blockIdx.x;
  const int xcd = L & 7, jx = L >> 3, q8 = T >> 3, r8 = T & 7;
  const int V = xcd < r8 ? xcd * (q8 + 1) + jx : r8 * (q8 + 1) + (xcd - r8) * q8 + jx;
  const int m0 = (V % tiles_m) * 16 * TM, n0 = (V / tiles_m) * 16 * TN * NH + 16 * TN * wh;

  // This wave's k-blocks and stages.
  const int nkb = K / 256, kbn = nkb / KQ, kb0 = kbn * wq;
  const int nst = kbn * kRing;

  // Loads go through buffer descriptors (32-bit offsets, range-checked by
  // the hardware): a lane-constant VGPR offset plus a wave-uniform SGPR
  // offset.  Record of row tile tn at k-block kb: (tile * nkb + kb) * kRec;
  // tiles past the last read the last one (never stored).
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(P), 0, (int)(((uint32_t)(N + 15) / 16) * (uint32_t)nkb * (uint32_t)R::kRec), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<AT *>(A), 0, (int)((uint32_t)M * (uint32_t)K * (uint32_t)sizeof(AT)), kRsrcWord3);
  const int last_tile = (N + 15) / 16 - 1;
  int rec0[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) rec0[tn] = min(n0 / 16 + tn, last_tile) * nkb * R::kRec;
  // Activation staging loads: load q of a stage brings tokens m0 + TPL q ..
  // + TPL - 1 (clamped to M - 1, never stored), lane l the chunk that goes
  // to position l mod CPT of token TPL q + l / CPT.
  const int at = lane / AS::CPT, ap = lane % AS::CPT;
  const int acol = 16 * (ap ^ (at % AS::KEYP));
  // Fragment reads (bytes within a stage buffer): lane (i, G) of token tile
  // tm, step h reads part e of its eight elements, kPartElems elements at
  // a_part(0, h, G, e), as one or two 16-byte pieces or one 8-byte piece.
  constexpr int PB = R::kPartElems * (int)sizeof(AT);  // bytes per part
  constexpr int NP = PB >= 16 ? PB / 16 : 1;           // pieces per part
  int frd[2][R::kParts][NP];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < R::kParts; ++e)
#pragma unroll
      for (int q = 0; q < NP; ++q) {
        const int b0 = R::a_part(0, h, G, e) * (int)sizeof(AT) + 16 * q;
        frd[h][e][q] = j * AS::CPT * 16 + 16 * ((b0 >> 4) ^ (j % AS::KEYP)) + (b0 & 15);
      }
  const int grp = wq * AS::BYTES;  // this part's buffer in each ring array

  R rows;
  // Vector-memory operations a wave issues for the stage at ring position u
  // (its activation share and its weight rows), and those of the two stages
  // after ring position u.
  constexpr auto count = [](int u) { return AS::NLD / NH + R::loads(u) * TN; };
  constexpr auto more = [count](int u) { return count((u + 1) % kRing) + count((u + 2) % kRing); };

  // Loads of stage t (clamped to the last stage: a re-read never used) into
  // ring position u = t mod kRing and scale buffer p.
  auto load = [&](int t, int u, int p) {
    t = min(t, nst - 1);
    const int kb = kb0 + t / kRing;
    const int ak = (256 * kb + 64 * u) * (int)sizeof(AT);  // wave-uniform
    uint8_t *dst = ring(u) + grp;
#pragma unroll
    for (int i = 0; i < AS::NLD / NH; ++i) {
      const int q = wh * (AS::NLD / NH) + i;
      dma16(ars, dst + 1024 * q, min(m0 + AS::TPL * q + at, M - 1) * K * (int)sizeof(AT) + acol, ak);
    }
    rows.load(prs, lane, j, rec0, kb * R::kRec, u, p);
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = floatx4{0.f, 0.f, 0.f, 0.f};

  // Activation fragments of step h of the stage in ring position u.
  auto frags = [&](int u, int h, half8 (&ahi)[TM], half8 (&alo)[TM]) {
    const uint8_t *src = ring(u) + grp;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
      const uint8_t *row = src + 16 * tm * AS::CPT * 16;
      if constexpr (kF32) {
        float a[8];
#pragma unroll
        for (int e = 0; e < R::kParts; ++e)
#pragma unroll
          for (int q = 0; q < NP; ++q) {
            const f32x4 v = __builtin_bit_cast(f32x4, *reinterpret_cast<const u32x4 *>(row + frd[h][e][q]));
#pragma unroll
            for (int i = 0; i < 4; ++i) a[e * R::kPartElems + 4 * q + i] = v[i];
          }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const _Float16 hv = (_Float16)a[e];
          ahi[tm][e] = hv;
          alo[tm][e] = (_Float16)(a[e] - (float)hv);
        }
      } else if constexpr (PB == 16) {
        ahi[tm] = as_h8(*reinterpret_cast<const u32x4 *>(row + frd[h][0][0]));
      } else {
        const u32x2 x0 = *reinterpret_cast<const u32x2 *>(row + frd[h][0][0]);
        const u32x2 x1 = *reinterpret_cast<const u32x2 *>(row + frd[h][1][0]);
        ahi[tm] = as_h8(u32x4{x0[0], x0[1], x1[0], x1[1]});
      }
    }
  };
  auto products = [&](int u, int p, int h, const half8 (&ahi)[TM], const half8 (&alo)[TM]) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const half8 bf = as_h8(rows.b(u, p, tn, h, G));
      if constexpr (R::kPostScale) {
        // The step is one group: its product, then its f32 scale.
        const float sc = rows.scale(u, p, tn, h);
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          floatx4 D = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[tm], bf, floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          if constexpr (kF32) D = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[tm], bf, D, 0, 0, 0);
          acc[tm][tn] += sc * D;
        }
      } else {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[tm], bf, acc[tm][tn], 0, 0, 0);
          if constexpr (kF32)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[tm], bf, acc[tm][tn], 0, 0, 0);
        }
      }
    }
  };
  // Wait until the loads of the stage at ring position u have landed: the
  // loads of the two stages after it (positions u + 1 and u + 2; the one at
  // position 0 also carries scale rows) may still be outstanding.  Then
  // let the part's waves arrive: a bare barrier, since every wave has
  // waited for its own direct-to-LDS loads (a fenced barrier would make
  // the compiler wait for all of them, the later stages' too).
  auto arrive = [&](int u) {
    __builtin_amdgcn_sched_barrier(0);
    constexpr int kMore[kRing] = {more(0), more(1), more(2), more(3)};
    switch (u) {
      case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm(kMore[0])); break;
      case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm(kMore[1])); break;
      case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm(kMore[2])); break;
      default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(kMore[3])); break;
    }
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  half8 a0hi[TM], a0lo[TM], a1hi[TM], a1lo[TM];
  // Stage t at ring position u, scale buffer p (its k-block's parity); the
  // loads it issues are for stage t + kRing - 1.
  auto stage = [&](int t, int u, int p) {
    // Stage t + kRing - 1 lies in the next k-block unless this stage opens
    // one (ring position 0).
    const int un = (u + kRing - 1) % kRing;
    load(t + kRing - 1, un, u == 0 ? p : p ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    products(u, p, 0, a0hi, a0lo);
    frags(u, 1, a1hi, a1lo);
    products(u, p, 1, a1hi, a1lo);
    arrive((u + 1) % kRing);
    frags((u + 1) % kRing, 0, a0hi, a0lo);
  };

  // Prologue: stages 0 .. kRing - 2 in flight, stage 0's first fragments.
#pragma unroll
  for (int s = 0; s < kRing - 1; ++s) load(s, s, 0);
  arrive(0);
  frags(0, 0, a0hi, a0lo);
  // Two k-blocks (scale buffers 0, 1) per turn of the unrolled loop, then
  // the last k-block when their number is odd.
  int t = 0;
  for (; t + 2 * kRing <= nst; t += 2 * kRing) {
#pragma unroll
    for (int u = 0; u < 2 * kRing; ++u) stage(t + u, u % kRing, u / kRing);
  }
  if (t < nst) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) stage(t + u, u, 0);
  }
  // The last direct-to-LDS loads may still be landing: wait for every
  // memory operation of this wave before the LDS is reused below.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Sum the KQ partial tiles of each row half through LDS, kRedChunk
  // accumulator values per lane at a time: wave (q, h) writes
  // red[q NH + h][v][lane]; then thread (wave, lane) adds, for row half
  // h' = wave % NH and values v = c0 + wave / NH + (KW / NH) r, the KQ
  // partials in part order for its own lane position and stores the sum.
  float *red = reinterpret_cast<float *>(ring0);
  constexpr int NV = TM * TN * 4;
  constexpr int VS = KW / NH;  // values per round step
  constexpr int kRedChunk = (KQ * AS::BYTES) / (KW * 64 * 4) < 32 ? (KQ * AS::BYTES) / (KW * 64 * 4) : 32;
  static_assert(kRedChunk % VS == 0 && NV % kRedChunk == 0, "reduction rounds");
#pragma unroll
  for (int c0 = 0; c0 < NV; c0 += kRedChunk) {
    if (c0) __syncthreads();
#pragma unroll
    for (int v = c0; v < c0 + kRedChunk && v < NV; ++v)
      red[(wave * kRedChunk + (v - c0)) * 64 + lane] = acc[(v >> 2) / TN][(v >> 2) % TN][v & 3];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRedChunk / VS; ++r) {
      const int vl = wq + VS * r, v = c0 + vl;
      if (v < NV) {
        float sum = red[(wh * kRedChunk + vl) * 64 + lane];
#pragma unroll
        for (int q = 1; q < KQ; ++q) sum += red[((q * NH + wh) * kRedChunk + vl) * 64 + lane];
        const int tm = (v >> 2) / TN, tn = (v >> 2) % TN;
        const int m = m0 + 16 * tm + 4 * G + (v & 3), n = n0 + 16 * tn + j;
        if (m < M && n < N) C[(int64_t)m * N + n] = sum;
      }
    }
  }
}

template <int KIND, typename AT, int TM, int TN, int KQ, int NH>
static hipError_t run(const uint8_t *P, const void *A, float *C, int64_t M, int64_t N, int64_t K, hipStream_t s) {
  constexpr int KW = KQ * NH;
  const int64_t tm = (M + 16 * TM - 1) / (16 * TM), tn = (N + 16 * TN * NH - 1) / (16 * TN * NH);
  static_assert((size_t)KQ * kRing * AStage<AT, TM>::BYTES <= 160 * 1024, "one workgroup per compute unit");
  hipLaunchKernelGGL((gemm_pk_kernel<KIND, AT, TM, TN, KQ, NH>), dim3((unsigned)(tm * tn)), dim3(64 * KW), 0, s,
                     P, (const AT *)A, C, (int)M, (int)N, (int)K, (int)tm);
  return hipGetLastError();
}

// The k parts must divide the k-block count: four where they do (two for
// f32 activations, whose staging is twice the size), else two, else one.
template <int KIND, int TM, int TN, int NH>
static hipError_t run_any(const uint8_t *P, const void *A, int a_f16, float *C, int64_t M, int64_t N, int64_t K,
                          hipStream_t s) {
  const int64_t nkb = K / 256;
  if (a_f16) {
    if (nkb % 4 == 0) return run<KIND, _Float16, TM, TN, 4, NH>(P, A, C, M, N, K, s);
    if (nkb % 2 == 0) return run<KIND, _Float16, TM, TN, 2, NH>(P, A, C, M, N, K, s);
    return run<KIND, _Float16, TM, TN, 1, NH>(P, A, C, M, N, K, s);
  }
  if (nkb % 2 == 0) return run<KIND, float, TM, TN, 2, NH>(P, A, C, M, N, K, s);
  return run<KIND, float, TM, TN, 1, NH>(P, A, C, M, N, K, s);
}

template <int KIND>
static hipError_t run_kind(const uint8_t *P, const void *A, int a_f16, float *C, int64_t M, int64_t N, int64_t K,
                           hipStream_t s) {
#ifdef QMM_TUNING
  static const int cfg = [] {
    const char *e = getenv("QMM_GEMM_PK_CFG");
    return e ? atoi(e) : 0;
  }();
  const int64_t nkb = K / 256;
  switch (cfg) {
    case 1: return run_any<KIND, 4, 8, 1>(P, A, a_f16, C, M, N, K, s);
    case 2: return run_any<KIND, 2, 4, 2>(P, A, a_f16, C, M, N, K, s);
    case 3: if (a_f16 && nkb % 2 == 0) return run<KIND, _Float16, 4, 3, 2, 4>(P, A, C, M, N, K, s); break;
    case 5: if (a_f16 && nkb % 4 == 0) return run<KIND, _Float16, 4, 3, 4, 2>(P, A, C, M, N, K, s); break;
    case 6: if (a_f16 && nkb % 2 == 0) return run<KIND, _Float16, 4, 2, 2, 4>(P, A, C, M, N, K, s); break;
    case 7: if (a_f16 && nkb % 2 == 0) return run<KIND, _Float16, 4, 4, 2, 4>(P, A, C, M, N, K, s); break;
    default: break;
  }
#endif
  // 64 x 128 tiles, or 64 x 192 (two k parts of four waves over three row
  // tiles each) when the 64 x 128 grid would take more than one round of
  // the compute units and the 64 x 192 grid takes one: 256 x 11008 x 4096,
  // IQ4_NL 61.9 -> 48.4 us, MXFP4 53.9 -> 41.7 us (the 64 x 192 grid is
  // slower where 64 x 128 already fits one round: 512 x 4096 x 4096 Q8_0
  // 29.4 -> 34.0 us).
  const int64_t cus = device_cus(), tm = (M + 63) / 64;
  if (a_f16 && (K / 256) % 2 == 0 && tm * ((N + 127) / 128) > cus && tm * ((N + 191) / 192) <= cus)
    return run<KIND, _Float16, 4, 3, 2, 4>(P, A, C, M, N, K, s);
  return run_any<KIND, 4, 4, 2>(P, A, a_f16, C, M, N, K, s);
}

}  // namespace pk

bool gemm_packed_supported(int kind) {
  return kind == Q8_0 || kind == Q4_0 || kind == Q5_0 || kind == IQ4_NL || kind == MXFP4 || kind == IQ4_XS;
}

hipError_t launch_gemm_packed(int kind, const uint8_t *P, const void *A, int a_f16, float *C, int64_t M, int64_t N,
                              int64_t K, hipStream_t s) {
  switch (kind) {
    case Q8_0: return pk::run_kind<Q8_0>(P, A, a_f16, C, M, N, K, s);
    case Q4_0: return pk::run_kind<Q4_0>(P, A, a_f16, C, M, N, K, s);
    case Q5_0: return pk::run_kind<Q5_0>(P, A, a_f16, C, M, N, K, s);
    case IQ4_NL: return pk::run_kind<IQ4_NL>(P, A, a_f16, C, M, N, K, s);
    case MXFP4: return pk::run_kind<MXFP4>(P, A, a_f16, C, M, N, K, s);
    case IQ4_XS: return pk::run_kind<IQ4_XS>(P, A, a_f16, C, M, N, K, s);
    default: break;
  }
  return hipErrorNotSupported;
}

}  // namespace qmm
