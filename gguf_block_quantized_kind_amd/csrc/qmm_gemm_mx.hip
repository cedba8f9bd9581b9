// qmm_gemm_mx.hip -- prefill GEMM for MXFP4 weights on gfx950's scaled
// FP8 x FP4 matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// This is the separately toleranced variant of the MXFP4 prefill GEMM.  The
// weights need no decode at all: for one 128-k step, lane (j, G) of a 16-row
// tile holds weight row j, k = 32G .. 32G+31 -- exactly one MXFP4 block,
// whose 16 code bytes are the FP4 B operand and whose E8M0 byte is the
// lane's B scale.  The activations are quantized once, before the GEMM,
// to two MX FP8 terms per row and 32-element block:
//   hi = E4M3(a / 2^e1), 2^e1 the smallest power of two with
//        max |a| / 2^e1 <= 448 (E4M3's largest value), so no element
//        saturates;
//   lo = E4M3(r / 2^e2) of the residual r = a - 2^e1 hi, on the scale of the
//        block's residuals,
// each rounded to nearest, ties to even, and each matrix-core step runs
// twice, on hi and on lo, into the same accumulator.  The scalings and the
// residual are exact in f32, so the two E4M3 roundings are the only ones
// besides the f32 accumulation: |a - 2^e1 hi - 2^e2 lo| <= 2^-8 |a| (plus
// 2^(e1 - 14) where hi is subnormal).  A single term would lose up to 2^-4
// of |a| (a block of 1.0625s rounds 5.9 % low).
//
// Operand layout of one 16 x 16 x 128 step (k counted within the step):
//   B (FP4, 4 registers): lane (j, G) holds column j, k = 32G + p in nibble p
//     of its 16 bytes, low nibble first;
//   A (FP8, 8 registers): lane (j, G) holds row j, k = 16G + b in byte b of
//     its first 16 bytes and k = 64 + 16G + b in byte b of the next 16;
//   scales: lane group G gives the E8M0 scale of k = 32G .. 32G + 31, for A
//     and for B, whichever lanes hold that block's A elements.
// A GGUF MXFP4 block keeps element e < 16 in the low nibble of byte e and
// element e + 16 in its high nibble, so nibble p is element p / 2 (p even)
// or 16 + p / 2 (p odd).  The quantizer stores each block's activations in
// that order, the weight bytes are used as they are, and a step's 128 FP8
// bytes of a token are read as 16-byte chunks G and G + 4.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {
namespace mx {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 64;   // tokens per tile (the workspace pads rows to this)
// Weight rows per tile: 4 waves x TN tiles of 16 rows.  Three tiles per
// wave (192 rows) keep a wave within 256 registers, so two workgroups share
// a compute unit; that beats four tiles per wave (256 rows, one workgroup
// per compute unit) at every size measured: 256 tokens x 11008 rows, 35.5
// against 43.1 us; 1024 tokens, 102 against 119 us.  Memory parallelism per
// compute unit bounds this kernel, and the second workgroup adds to it.
// Two tiles per wave (128 rows) pay off only when 192-row tiles would leave
// most compute units idle: 128 tokens, 27.9 against 33.8 us, but 41.0
// against 35.5 us at 256 tokens.
constexpr int kTN = 3;
constexpr int kTNSmall = 2;
constexpr int kKS = 128;  // k per matrix-core step
constexpr int kPD = 3;    // loads run this many steps ahead

// Workspace: hi codes [Mp][K], lo codes [Mp][K], hi scales [Mp][K / 32], lo
// scales [Mp][K / 32], all bytes.
struct Layout {
  int64_t Mp, K;
  Layout(int64_t M, int64_t K_) : Mp((M + kBM - 1) / kBM * kBM), K(K_) {}
  int64_t lo_codes() const { return Mp * K; }
  int64_t scales() const { return 2 * Mp * K; }
  int64_t lo_scales() const { return 2 * Mp * K + Mp * (K / 32); }
  int64_t bytes() const { return 2 * (Mp * K + Mp * (K / 32)); }
};

// Element of a 32-element block stored at position p (nibble p of the weights).
__device__ __forceinline__ int src_of(int p) { return (p & 1) ? 16 + (p >> 1) : (p >> 1); }

// The E8M0 exponent of a block whose largest magnitude is amax: the
// smallest e with amax / 2^e <= 448, clamped to [-127, 127]; -127 for zero.
// amax = f * 2^x with f in [0.5, 1): 2^(x - 9) brings amax to [256, 512),
// one more step when that exceeds 448 (f > 0.875).
__device__ __forceinline__ int mx_exponent(float amax) {
  int e = -127;
  if (amax > 0.f) {
    const int x = __builtin_amdgcn_frexp_expf(amax);
    e = x - 9 + (__builtin_amdgcn_frexp_mantf(amax) > 0.875f ? 1 : 0);
  }
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Eight E4M3 codes per pair of words: v[i] / 2^e, clamped to +-448, each
// rounded to nearest even (the hardware conversion); the codes of elements
// src_of(4w + q) go to byte q of word w.
__device__ __forceinline__ void mx_encode(const float (&v)[32], int e, uint32_t (&out)[8]) {
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    float s[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) s[q] = fminf(fmaxf(__builtin_amdgcn_ldexpf(v[src_of(4 * w + q)], -e), -448.f), 448.f);
    uint32_t packed = 0u;
    packed = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s[0], s[1], (int)packed, false);
    packed = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s[2], s[3], (int)packed, true);
    out[w] = packed;
  }
}

// One thread per (row, block): both terms' codes and scale bytes.
template <typename AT>
__global__ __launch_bounds__(256) void quantize_kernel(const AT *__restrict__ A, int M, int64_t Mp, int K,
                                                       uint8_t *__restrict__ codes_hi, uint8_t *__restrict__ codes_lo,
                                                       uint8_t *__restrict__ scales_hi,
                                                       uint8_t *__restrict__ scales_lo) {
  const int nb = K / 32;
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (row, block)
  if (id >= Mp * nb) return;
  const int64_t m = id / nb;
  const int b = (int)(id % nb);
  uint32_t hi[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u}, lo[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  int e1 = -127, e2 = -127;  // rows past M: zero codes under the smallest scale
  if (m < M) {
    float a[32];
    const AT *src = A + m * K + 32 * b;
#pragma unroll
    for (int i = 0; i < 32; ++i) a[i] = (float)src[i];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(a[i]));
    e1 = mx_exponent(amax);
    mx_encode(a, e1, hi);
    // Residuals: a - 2^e1 * E4M3 value, exact in f32.
    float r[32];
    float rmax = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const float d[4] = {__builtin_amdgcn_cvt_f32_fp8((int)hi[w], 0), __builtin_amdgcn_cvt_f32_fp8((int)hi[w], 1),
                          __builtin_amdgcn_cvt_f32_fp8((int)hi[w], 2), __builtin_amdgcn_cvt_f32_fp8((int)hi[w], 3)};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = src_of(4 * w + q);
        r[i] = a[i] - __builtin_amdgcn_ldexpf(d[q], e1);
        rmax = fmaxf(rmax, fabsf(r[i]));
      }
    }
    e2 = mx_exponent(rmax);
    mx_encode(r, e2, lo);
  }
  u32x4 *dh = reinterpret_cast<u32x4 *>(codes_hi + m * K + 32 * b);
  dh[0] = u32x4{hi[0], hi[1], hi[2], hi[3]};
  dh[1] = u32x4{hi[4], hi[5], hi[6], hi[7]};
  u32x4 *dl = reinterpret_cast<u32x4 *>(codes_lo + m * K + 32 * b);
  dl[0] = u32x4{lo[0], lo[1], lo[2], lo[3]};
  dl[1] = u32x4{lo[4], lo[5], lo[6], lo[7]};
  scales_hi[m * nb + b] = (uint8_t)(e1 + 127);
  scales_lo[m * nb + b] = (uint8_t)(e2 + 127);
}

// One workgroup: 64 tokens x 64 TN weight rows; wave w owns rows
// 16 TN w .. 16 TN (w + 1) - 1 (TN 16-row tiles) against all 64 tokens (four
// 16-token tiles), 8 TN scaled matrix-core steps per 128-k step (4 TN on
// the first activation term, then 4 TN on the second).
//
// Loads.  Per step a row contributes four blocks, a 68-byte span starting at
// a multiple of 4; the wave fetches each of its rows' spans as the five
// aligned 16-byte chunks that cover it (80 TN chunks, adjacent lanes on
// adjacent chunks; the last lanes repeat the last chunk when 64 does not
// divide them), and each thread fetches its share of the
// tokens' FP8 codes and scales of both terms.  Everything is loaded PD steps ahead into a
// ring of PD + 1 register slots and written to LDS one step ahead of use:
// activations to a shared tile, weight chunks to a wave-private copy from
// which each lane picks its 17-byte block at any byte offset.  Load
// completion is counted in issue order, so both kinds of load keep one
// distance.  Loads past the last step are clamped to it (a repeated read of
// cached data), which keeps the loop body free of branches.
template <int PD, int TN, int TM>
__global__ __launch_bounds__(256) void gemm_mx_kernel(const uint8_t *__restrict__ W, int64_t row_bytes,
                                                      const uint8_t *__restrict__ codes,
                                                      const uint8_t *__restrict__ scales, float *__restrict__ C,
                                                      int M, int N, int K, int n_tiles, int m_tiles) {
  constexpr int NS = PD + 1;                    // ring slots
  constexpr int U = NS % 2 == 0 ? NS : 2 * NS;  // unroll: whole ring turns and LDS buffer pairs
  constexpr int kChunks = 5;                    // 16-byte chunks per row and step
  constexpr int kWave = 16 * TN * kChunks;      // chunks per wave and step
  constexpr int LC = (kWave + 63) / 64;         // per lane
  constexpr int BM = 16 * TM;                   // tokens per tile
  constexpr int TPT = 256 / BM;                 // threads per token loading activations
  constexpr int CPT = 8 / TPT;                  // 16-byte chunks per thread and term
  // Term h, token t, 16-byte chunk c at [h][t * 8 + (c ^ (t & 7))].
  __shared__ u32x4 a_lds[2][2][BM * 8];
  __shared__ uint32_t s_lds[2][2 * BM];  // term h, token t: the step's four E8M0 bytes at h * BM + t
  // Wave w, row r, chunk q at [w][5r + q]; one spare chunk past the end (a
  // block read at the very end of a row window touches one dword beyond it).
  __shared__ u32x4 b_lds[2][4 * kWave + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j = lane & 15, G = lane >> 4;
  // Workgroups go to the eight XCDs in turn (id % 8).  Each XCD takes one
  // contiguous run of tiles, token tiles fastest, so the token tiles that
  // share a weight tile run on one XCD and read it through one L2.
  const int64_t tiles = (int64_t)n_tiles * m_tiles, per = (tiles + 7) / 8;
  const int64_t tile = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (tile >= tiles) return;  // the whole workgroup: no barrier is reached
  const int64_t m0 = (tile % m_tiles) * BM;
  const int64_t n0 = (tile / m_tiles) * (64 * TN) + 16 * TN * wave;
  const int nb = K / 32, steps = K / kKS;
  auto row_start = [&](int r) {  // byte offset of wave row r in W; rows past N read row N - 1
    int64_t row = n0 + r;
    if (row >= N) row = N - 1;
    return row * row_bytes;
  };

  // This lane's chunks: chunk c = lane + 64 i is row c / 5, chunk c % 5.
  int64_t cbase[LC];
#pragma unroll
  for (int i = 0; i < LC; ++i) {
    const int c = min(lane + 64 * i, kWave - 1);
    cbase[i] = row_start(c / kChunks) + 16 * (c % kChunks);
  }
  // The rows this lane multiplies: 16 tn + j; their spans start at byte
  // (rs + 68 st) mod 16 of the first chunk.
  int rs16[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn) rs16[tn] = (int)(row_start(16 * tn + j) & 15);
  // This thread's share of a step's activation tiles: token at, chunks
  // ac .. ac + CPT - 1 of both terms (the second term's codes one plane of
  // Mp K bytes further), and the scale word of token tid % BM, term
  // tid / BM % 2.
  const int64_t Mp = (int64_t)m_tiles * BM;
  const int at = tid / TPT, ac = CPT * (tid % TPT);
  const uint8_t *asrc = codes + (m0 + at) * K + 16 * ac;
  const int64_t lo_plane = Mp * K;
  const uint8_t *ssrc = scales + ((tid / BM) & 1) * (Mp * nb) + (m0 + (tid & (BM - 1))) * nb;

  u32x4 areg[NS][2 * CPT];
  uint32_t sreg[NS];
  u32x4 breg[NS][LC];
  auto load = [&](int st, int slot) {
    st = st < steps ? st : steps - 1;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      areg[slot][c] = *reinterpret_cast<const u32x4 *>(asrc + (int64_t)st * kKS + 16 * c);
      areg[slot][CPT + c] = *reinterpret_cast<const u32x4 *>(asrc + lo_plane + (int64_t)st * kKS + 16 * c);
    }
    sreg[slot] = *reinterpret_cast<const uint32_t *>(ssrc + 4 * st);
#pragma unroll
    for (int i = 0; i < LC; ++i) {
      // Aligned down to 16: the span starts at (row start + 68 st), a
      // multiple of 4, so five chunks from there cover its 68 bytes.
      const int64_t off = (cbase[i] + (int64_t)st * 68) & ~(int64_t)15;
      breg[slot][i] = *reinterpret_cast<const u32x4 *>(W + off);
    }
  };
  auto store = [&](int slot, int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < CPT; ++c) a_lds[buf][h][at * 8 + ((ac + c) ^ (at & 7))] = areg[slot][CPT * h + c];
    // Several threads load each scale word; all store the same value, which
    // keeps the step free of branches (a branch here lets the compiler sink
    // the matrix-core chain past the later steps' barriers).
    s_lds[buf][tid & (2 * BM - 1)] = sreg[slot];
#pragma unroll
    for (int i = 0; i < LC; ++i) b_lds[buf][wave * kWave + min(lane + 64 * i, kWave - 1)] = breg[slot][i];
  };

  floatx4 acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = floatx4{0.f, 0.f, 0.f, 0.f};

  // The step's products from this lane's weight blocks: the first term of
  // all four token tiles, then the second, so that 4 TN products separate
  // two that update one accumulator.
  auto products = [&](const uint32_t (&bq)[TN][4], const uint32_t (&be)[TN], int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int t = 16 * tm + j;
        const u32x4 c0 = a_lds[buf][h][t * 8 + (G ^ (t & 7))];
        const u32x4 c1 = a_lds[buf][h][t * 8 + ((G + 4) ^ (t & 7))];
        const v8i af = v8i{(int)c0[0], (int)c0[1], (int)c0[2], (int)c0[3], (int)c1[0], (int)c1[1], (int)c1[2], (int)c1[3]};
        const int sa = (int)((s_lds[buf][h * BM + t] >> (8 * G)) & 0xFFu);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const v8i bf = v8i{(int)bq[tn][0], (int)bq[tn][1], (int)bq[tn][2], (int)bq[tn][3], 0, 0, 0, 0};
          // Format codes: 0 = FP8 E4M3 (A), 4 = FP4 E2M1 (B); scales are E8M0.
          acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf, acc[tm][tn], 0, 4, 0, sa, 0,
                                                                         (int)be[tn]);
        }
      }
  };

  auto compute = [&](int st, int buf) {
    // This lane's weight block of each tile: E8M0 byte and 16 code bytes at
    // byte x of the wave's copy, read as the five dwords from x & ~3.
    uint32_t bq[TN][4], be[TN];
    const uint32_t *wl = reinterpret_cast<const uint32_t *>(&b_lds[buf][wave * kWave]);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int x = 80 * (16 * tn + j) + ((rs16[tn] + 4 * st) & 15) + 17 * G;
      const uint32_t *d = wl + (x >> 2);
      uint32_t w[5];
#pragma unroll
      for (int i = 0; i < 5; ++i) w[i] = d[i];
      const int sh = 8 * (x & 3);
      be[tn] = (w[0] >> sh) & 0xFFu;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bq[tn][i] = (uint32_t)((((uint64_t)w[i + 1] << 32) | w[i]) >> (sh + 8));
    }
    products(bq, be, buf);
  };
  // The same step when every row starts on a 16-byte boundary (row_bytes a
  // multiple of 16, i.e. K a multiple of 512) and st0 is a multiple of 4:
  // a row's span then starts at byte 4 (st % 4) of its first chunk for every
  // row, so all addresses are a lane constant plus an immediate offset, and
  // a lane's 16 code bytes sit at byte (G + 1) % 4 of five dwords, two by two
  // joined with v_alignbyte.
  const int bq_dw = 20 * j + 4 * G + ((G + 1) >> 2);  // dword of the codes, tile 0, step % 4 = 0
  const int be_b = 80 * j + 17 * G;                     // byte of the E8M0 scale
  const int bsh = (G + 1) & 3;
  auto compute_fast = [&](int u, int buf) {
    uint32_t bq[TN][4], be[TN];
    const uint32_t *wl = reinterpret_cast<const uint32_t *>(&b_lds[buf][wave * kWave]);
    const uint8_t *bl = reinterpret_cast<const uint8_t *>(wl);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const uint32_t *d = wl + bq_dw + 320 * tn + u;
      uint32_t w[5];
#pragma unroll
      for (int i = 0; i < 5; ++i) w[i] = d[i];
      be[tn] = bl[be_b + 1280 * tn + 4 * u];
#pragma unroll
      for (int i = 0; i < 4; ++i) bq[tn][i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], bsh);
    }
    products(bq, be, buf);
  };
  // Loads of step st0 + PD + u for that case: pointers advance once per
  // group of U steps; within the group every offset is an immediate.
  auto load_fast = [&](int st0, int u, int slot) {
    const int64_t sp = st0 + PD;  // st0 % 4 == 0, so 68 * st0 is a multiple of 16
    const uint8_t *ag = asrc + sp * kKS + u * kKS;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      areg[slot][c] = *reinterpret_cast<const u32x4 *>(ag + 16 * c);
      areg[slot][CPT + c] = *reinterpret_cast<const u32x4 *>(ag + lo_plane + 16 * c);
    }
    sreg[slot] = *reinterpret_cast<const uint32_t *>(ssrc + 4 * sp + 4 * u);
    const int delta = 16 * ((68 * (PD + u)) >> 4);
#pragma unroll
    for (int i = 0; i < LC; ++i)
      breg[slot][i] = *reinterpret_cast<const u32x4 *>(W + cbase[i] + (int64_t)st0 * 68 + delta);
  };
  // Step st: operands in LDS buffer st % 2.  The step issues the loads of
  // step st + PD and, after its products, stages step st + 1 from slot
  // (st + 1) % NS.
  auto step = [&](int st, int u) {
    load(st + PD, (u + PD) % NS);
    __builtin_amdgcn_sched_barrier(0);
    compute(st, u % 2);
    __builtin_amdgcn_sched_barrier(0);
    store((u + 1) % NS, (u + 1) % 2);
    __syncthreads();
  };

#pragma unroll
  for (int p = 0; p < PD; ++p) load(p, p);
  store(0, 0);
  __syncthreads();
  int st0 = 0;
  if ((row_bytes & 15) == 0) {
    static_assert(U % 4 == 0, "the aligned path walks groups of four steps");
    // Every load of these groups lies before the last step: no clamping.
    for (; st0 + U + PD <= steps; st0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        load_fast(st0, u, (u + PD) % NS);
        __builtin_amdgcn_sched_barrier(0);
        compute_fast(u, u % 2);
        __builtin_amdgcn_sched_barrier(0);
        store((u + 1) % NS, (u + 1) % 2);
        __syncthreads();
      }
    }
  }
  for (; st0 + U <= steps; st0 += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) step(st0 + u, u);
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (st0 + u < steps) step(st0 + u, u);

  // D[i][j] of a 16x16 tile sits in lane j + 16*(i/4), register i%4.
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int64_t n = n0 + 16 * tn + j;
      if (n >= N) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t m = m0 + 16 * tm + 4 * G + q;
        if (m < M) C[m * N + n] = acc[tm][tn][q];
      }
    }
}

// One launch of the scaled GEMM with TN 16-row weight tiles per wave and
// TM 16-token tiles per workgroup; the grid is a multiple of 8 so that every
// XCD gets the same number of workgroups.
template <int TN, int TM>
hipError_t launch_tiles(const uint8_t *W, int64_t row_bytes, const uint8_t *codes, const uint8_t *scales, float *C,
                        int64_t M, int64_t N, int64_t K, int64_t Mp, hipStream_t s) {
  const int64_t m_tiles = Mp / (16 * TM);
  const int64_t n_tiles = (N + 64 * TN - 1) / (64 * TN);
  const dim3 grid((unsigned)(8 * ((n_tiles * m_tiles + 7) / 8))), block(256);
  hipLaunchKernelGGL((gemm_mx_kernel<kPD, TN, TM>), grid, block, 0, s, W, row_bytes, codes, scales, C, (int)M,
                     (int)N, (int)K, (int)n_tiles, (int)m_tiles);
  return hipGetLastError();
}

}  // namespace mx

size_t gemm_mx_workspace_bytes(int64_t M, int64_t K) { return (size_t)mx::Layout(M, K).bytes(); }

hipError_t launch_gemm_mx(const uint8_t *W, const void *A, int a_f16, float *C, int64_t M, int64_t N, int64_t K,
                          void *ws, hipStream_t s) {
  if (K % mx::kKS != 0) return launch_gemm(MXFP4, W, A, a_f16, C, M, N, K, s);
  const mx::Layout L(M, K);
  uint8_t *codes = static_cast<uint8_t *>(ws), *scales = codes + L.scales();
  uint8_t *codes_lo = codes + L.lo_codes(), *scales_lo = codes + L.lo_scales();
  const int64_t blocks = L.Mp * (K / 32);
  const dim3 qgrid((unsigned)((blocks + 255) / 256)), block(256);
  if (a_f16)
    hipLaunchKernelGGL(mx::quantize_kernel<_Float16>, qgrid, block, 0, s, (const _Float16 *)A, (int)M, L.Mp,
                       (int)K, codes, codes_lo, scales, scales_lo);
  else
    hipLaunchKernelGGL(mx::quantize_kernel<float>, qgrid, block, 0, s, (const float *)A, (int)M, L.Mp, (int)K,
                       codes, codes_lo, scales, scales_lo);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t row_bytes = (K / 32) * 17;
#ifdef QMM_TUNING
  static const int cfg = [] {
    const char *e = getenv("QMM_GEMM_MX_CFG");
    return e ? atoi(e) : 0;
  }();
  switch (cfg) {
    case 1: return mx::launch_tiles<3, 4>(W, row_bytes, codes, scales, C, M, N, K, L.Mp, s);
    case 2: return mx::launch_tiles<2, 4>(W, row_bytes, codes, scales, C, M, N, K, L.Mp, s);
    case 3: return mx::launch_tiles<3, 2>(W, row_bytes, codes, scales, C, M, N, K, L.Mp, s);
    case 4: return mx::launch_tiles<2, 2>(W, row_bytes, codes, scales, C, M, N, K, L.Mp, s);
    case 5: return mx::launch_tiles<4, 2>(W, row_bytes, codes, scales, C, M, N, K, L.Mp, s);
    default: break;
  }
#endif
  // 192-row tiles, or 128-row tiles when there would be fewer than 128 of
  // the larger ones (half the compute units).
  const bool small = (N + 64 * mx::kTN - 1) / (64 * mx::kTN) * (L.Mp / 64) < 128;
  if (small) return mx::launch_tiles<mx::kTNSmall, 4>(W, row_bytes, codes, scales, C, M, N, K, L.Mp, s);
  return mx::launch_tiles<mx::kTN, 4>(W, row_bytes, codes, scales, C, M, N, K, L.Mp, s);
}

}  // namespace qmm
