// qmm_gemv_i8.hip -- the integer-activation decode GEMV: activations
// quantized per 32-element block to int8, weight codes multiplied as int8 on
// the matrix cores (v_mfma_i32_16x16x64_i8), one f32 scale product per block.
// This is the integer dot-product path that the ferrox-cuda mul_mm page names
// (llama.cpp's mmq) and leaves out; here it reads repacked Q8_0, Q4_0, Q5_0
// IQ4_NL or MXFP4 weights (the records of qmm_repack): the 32-element kinds
// whose codes, table values or doubled E2M1 values are integers that fit in
// int8.
//
// Quantization (32 lanes per token and block): amax = max |x|,
// d = amax / 127 and each x / d rounded to f32 (both through binary64, whose
// 53 bits make the double rounding to f32 exact for a quotient of two f32
// values), then to the nearest integer, ties to even.  An all-zero block has
// d = 0 and zero codes.  The codes are stored per block in the order the
// weight codes sit in a lane (below), with the block's scale and code sum.
//
// Product.  A k-block (eight blocks) is four MFMA steps of 64 k.  In step c,
// bytes 0-7 of every lane's operands belong to block 2c and bytes 8-15 to
// block 2c+1 of the k-block, in both operands, so each k index pairs the
// same element of x and w whatever the instruction's k order.  A row 2t + p
// holds token t's codes in the half of block 2c + p and zeros in the other
// half; D row 2t + p is then token t's exact integer dot product with block
// 2c + p alone.  Lane (j, G) holds D rows 4G .. 4G+3 of weight row j, i.e.
// tokens 2G and 2G+1, both blocks: it subtracts the code bias (Q4_0's 8 times
// the block's code sum, in integers) and adds d_w d_x times the sum in f32.
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "qmm.h"
#include "qmm_gemv_mfma.h"
#include "qmm_internal.h"

namespace qmm {
namespace i8 {

typedef int v4i __attribute__((ext_vector_type(4)));
using gv::floatx4;
using gv::u32x2;
using gv::u32x4;

// Position of element e of a block in the lane order of the weight codes:
// Q8_0 keeps element order (lane group G holds code bytes 8G .. 8G+7); for
// Q4_0, position 8G + j holds element 4G + j (j < 4, the low nibbles of code
// bytes 4G ..) and position 8G + 4 + j element 16 + 4G + j (their high
// nibbles).
template <int KIND>
__device__ __forceinline__ int position_of(int e) {
  if constexpr (KIND == Q8_0) {
    return e;
  } else {
    const int h = e >> 4, r = e & 15;  // low nibbles (h = 0) or high nibbles (h = 1)
    return 8 * (r >> 2) + 4 * h + (r & 3);
  }
}

// One thread per element, 32 consecutive threads per (token, block): the
// block maximum and the code sum are reduced across the 32 lanes, so the
// quantization takes a few steps instead of a 32-element loop per thread.
template <int KIND, typename XT>
__global__ __launch_bounds__(256) void quantize_kernel(const XT *__restrict__ X, int8_t *__restrict__ q,
                                                       float *__restrict__ d, int32_t *__restrict__ s,
                                                       int64_t blocks, int nb) {
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i = gi >> 5;  // (token, block)
  const int e = (int)(gi & 31);
  const bool live = i < blocks;
  const int64_t t = live ? i / nb : 0, b = live ? i - t * nb : 0;
  const float v = live ? (float)X[t * (int64_t)nb * 32 + 32 * b + e] : 0.f;
  float amax = fabsf(v);
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 32));
  const float db = (float)((double)amax / 127.0);
  const float r = db > 0.f ? (float)((double)v / (double)db) : 0.f;
  const int c = (int)__builtin_rintf(r);
  int sum = c;
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 32);
  if (!live) return;
  q[i * 32 + position_of<KIND>(e)] = (int8_t)c;
  if (e == 0) {
    d[i] = db;
    s[i] = sum;
  }
}

// B operand of step c: the 8 codes of block 2c, then the 8 of block 2c+1.
// Twice the E2M1 value of each of four 4-bit codes (one per byte), as signed
// bytes: 0, 1, 2, 3, 4, 6, 8, 12 and their negatives (code 8, -0, gives 0).
// Entries 0..7 and 8..15 are looked up with v_perm; bit 3 of each code picks.
constexpr uint32_t kE2T0 = 0x03020100u, kE2T1 = 0x0C080604u, kE2T2 = 0xFDFEFF00u, kE2T3 = 0xF4F8FAFCu;
__device__ __forceinline__ uint32_t e2m1x2_lookup(uint32_t idx) {
  const uint32_t low3 = idx & 0x07070707u;
  const uint32_t a = perm(kE2T1, kE2T0, low3);
  const uint32_t b = perm(kE2T3, kE2T2, low3);
  const uint32_t m = perm(0u, 0u, ((idx >> 3) & 0x01010101u) | 0x0C0C0C0Cu);
  return (b & m) | (a & ~m);
}

// Q4_0 and Q5_0 codes enter unsigned (their bias is applied through the
// activation code sums); IQ4_NL enters as the signed table value, MXFP4 as
// twice its E2M1 value (the block scale is halved to match).
template <int KIND>
__device__ __forceinline__ v4i bop(const typename gv::Rec<KIND>::Packed &p, int c, int G) {
  if constexpr (KIND == Q8_0) {
    return __builtin_bit_cast(v4i, p.c[c]);
  } else {
    uint32_t lo[2], hi[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int blk = 2 * c + h;
      const uint32_t w = p.c.q(blk);
      lo[h] = w & 0x0F0F0F0Fu;          // elements 4G .. 4G+3
      hi[h] = (w >> 4) & 0x0F0F0F0Fu;   // elements 16 + 4G ..
      if constexpr (KIND == Q5_0) {     // fifth bits: qh bits 4G.. and 16 + 4G..
        const uint32_t qh = (blk < 4 ? p.h0[blk] : p.h1[blk - 4]) >> (4 * G);
        lo[h] |= spread4(qh) << 4;
        hi[h] |= spread4(qh >> 16) << 4;
      } else if constexpr (KIND == IQ4_NL) {  // table value + 128, made signed
        lo[h] = iq4_lookup(lo[h]) ^ 0x80808080u;
        hi[h] = iq4_lookup(hi[h]) ^ 0x80808080u;
      } else if constexpr (KIND == MXFP4) {
        lo[h] = e2m1x2_lookup(lo[h]);
        hi[h] = e2m1x2_lookup(hi[h]);
      }
    }
    return v4i{(int)lo[0], (int)hi[0], (int)lo[1], (int)hi[1]};
  }
}

// f32 scales of blocks 2c and 2c+1 of a record: the f16 d of each block, or
// for MXFP4 2^(e-127) / 2 (its codes enter doubled).
template <int KIND>
__device__ __forceinline__ void block_scales(const typename gv::Rec<KIND>::Packed &p, int c, float &w0, float &w1) {
  if constexpr (KIND == MXFP4) {
    const uint32_t e = p.e[c >> 1] >> (16 * (c & 1));
    w0 = e8m0_to_f32(e & 0xFFu) * 0.5f;
    w1 = e8m0_to_f32((e >> 8) & 0xFFu) * 0.5f;
  } else {
    w0 = gv::lo_f16(p.d[c]);
    w1 = gv::hi_f16(p.d[c]);
  }
}

template <int KIND, int S, int PD>
__global__ __launch_bounds__(64 * S) void gemv_i8_kernel(const uint8_t *__restrict__ P, const int8_t *__restrict__ q,
                                                        const float *__restrict__ dx, const int32_t *__restrict__ sx,
                                                        float *__restrict__ Y, int M, int64_t N, int K) {
  using Rc = gv::Rec<KIND>;
  using Packed = typename Rc::Packed;
  constexpr int kBias = KIND == Q4_0 ? 8 : KIND == Q5_0 ? 16 : 0;
  constexpr int64_t kRec = 16 * gv::Dec<KIND>::BYTES;
  extern __shared__ u32x4 lds[];
  const int nb = K / 32, nkb = K / 256;
  float *ldx = reinterpret_cast<float *>(lds);       // [M][nb] scales, then [M][nb] code sums
  int32_t *lsx = reinterpret_cast<int32_t *>(ldx + M * nb);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 15, G = lane >> 4;
  const int64_t tile = blockIdx.x;
  const uint8_t *wt = P + tile * nkb * kRec;

  // A-row of this lane: token ta, block parity pa.
  const int ta = j >> 1, pa = j & 1;
  const bool alive = ta < M;
  const int8_t *xa = q + (int64_t)(alive ? ta : 0) * K + 8 * G;

  constexpr int NS = PD + 1;
  const int kb0 = (int)((int64_t)wave * nkb / S), kb1 = (int)((int64_t)(wave + 1) * nkb / S);
  Packed raw[NS];
  u32x2 xq[NS][4];
  auto issue = [&](int kb, int slot) {
    Rc::load(wt + kb * kRec, lane, j, G, raw[slot]);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x2 v = {0u, 0u};
      if (alive) v = *reinterpret_cast<const u32x2 *>(xa + 32 * (8 * kb + 2 * c + pa));
      xq[slot][c] = v;
    }
  };
#pragma unroll
  for (int d = 0; d < PD; ++d)
    if (kb0 + d < kb1) issue(kb0 + d, d);
  // The scales and code sums of every token's blocks, staged once.
  for (int i = threadIdx.x; i < M * nb; i += 64 * S) {
    ldx[i] = dx[i];
    lsx[i] = sx[i];
  }
  __syncthreads();

  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  const int t0 = min(2 * G, M - 1), t1 = min(2 * G + 1, M - 1);  // tokens of D rows 4G.., clamped
  for (int kb = kb0; kb < kb1; kb += NS) {
#pragma unroll
    for (int d = 0; d < NS; ++d) {
      if (kb + d >= kb1) break;
      if (kb + d + PD < kb1) issue(kb + d + PD, (d + PD) % NS);
      const int k = kb + d;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x2 xv = xq[d][c];
        const v4i a = pa == 0 ? v4i{(int)xv.x, (int)xv.y, 0, 0} : v4i{0, 0, (int)xv.x, (int)xv.y};
        const v4i D = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bop<KIND>(raw[d], c, G), v4i{0, 0, 0, 0}, 0, 0, 0);
        const int b0 = 8 * k + 2 * c;
        float w0, w1;  // d_w of blocks 2c and 2c+1
        block_scales<KIND>(raw[d], c, w0, w1);
        const int i00 = t0 * nb + b0, i10 = t1 * nb + b0;
        acc[0] += (w0 * ldx[i00]) * (float)(D[0] - kBias * lsx[i00]);
        acc[1] += (w1 * ldx[i00 + 1]) * (float)(D[1] - kBias * lsx[i00 + 1]);
        acc[2] += (w0 * ldx[i10]) * (float)(D[2] - kBias * lsx[i10]);
        acc[3] += (w1 * ldx[i10 + 1]) * (float)(D[3] - kBias * lsx[i10 + 1]);
      }
    }
  }
  // Tokens 2G and 2G+1 of row j: both block parities.
  float y0 = acc[0] + acc[1], y1 = acc[2] + acc[3];
  if constexpr (S > 1) {
    __syncthreads();  // every wave is done with the staged scales
    float *red = reinterpret_cast<float *>(lds);
    if (wave > 0) {
      red[((wave - 1) * 64 + lane) * 2] = y0;
      red[((wave - 1) * 64 + lane) * 2 + 1] = y1;
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 0; w < S - 1; ++w) {
      y0 += red[(w * 64 + lane) * 2];
      y1 += red[(w * 64 + lane) * 2 + 1];
    }
  }
  const int64_t row = tile * 16 + j;
  if (row >= N) return;
  if (2 * G < M) Y[(int64_t)(2 * G) * N + row] = y0;
  if (2 * G + 1 < M) Y[(int64_t)(2 * G + 1) * N + row] = y1;
}

template <int KIND, int S, int PD>
hipError_t run(const uint8_t *P, const int8_t *q, const float *d, const int32_t *s, float *y, int M, int64_t N,
               int64_t K, hipStream_t st) {
  const size_t stage = (size_t)M * (K / 32) * 8;
  const size_t red = (size_t)(S - 1) * 64 * 8;
  const size_t lds = std::max(stage, red);
  const unsigned tiles = (unsigned)((N + 15) / 16);
  hipLaunchKernelGGL((gemv_i8_kernel<KIND, S, PD>), dim3(tiles), dim3(64 * S), lds, st, P, q, d, s, y, M, N, (int)K);
  return hipGetLastError();
}

// Launch shape: S waves split K, PD k-blocks in flight.  A tuning build
// (-DQMM_TUNING) can pick another from QMM_GEMV_I8_CFG.
template <int KIND>
hipError_t run_shape(const uint8_t *P, const int8_t *q, const float *d, const int32_t *s, float *y, int M,
                     int64_t N, int64_t K, hipStream_t st) {
#ifdef QMM_TUNING
  static const int cfg = [] {
    const char *e = getenv("QMM_GEMV_I8_CFG");
    return e ? atoi(e) : 0;
  }();
  switch (cfg) {
    case 1: return run<KIND, 2, 2>(P, q, d, s, y, M, N, K, st);
    case 2: return run<KIND, 8, 1>(P, q, d, s, y, M, N, K, st);
    case 3: return run<KIND, 4, 1>(P, q, d, s, y, M, N, K, st);
    case 4: return run<KIND, 16, 1>(P, q, d, s, y, M, N, K, st);
    case 5: return run<KIND, 8, 2>(P, q, d, s, y, M, N, K, st);
    case 6: return run<KIND, 2, 3>(P, q, d, s, y, M, N, K, st);
    default: break;
  }
#endif
  // Measured at 4096 and 14336 rows: more waves per tile when tiles are few.
  if (N <= 4096) return run<KIND, 16, 1>(P, q, d, s, y, M, N, K, st);
  return run<KIND, 4, 1>(P, q, d, s, y, M, N, K, st);
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

template <int KIND>
void quantize(const void *x, int x_f16, int8_t *q, float *d, int32_t *s, int64_t blocks, int nb, unsigned grid,
              hipStream_t st) {
  if (x_f16)
    hipLaunchKernelGGL((quantize_kernel<KIND, _Float16>), dim3(grid), dim3(256), 0, st, (const _Float16 *)x, q, d, s,
                       blocks, nb);
  else
    hipLaunchKernelGGL((quantize_kernel<KIND, float>), dim3(grid), dim3(256), 0, st, (const float *)x, q, d, s,
                       blocks, nb);
}

}  // namespace i8

bool gemv_i8_supported(int kind) {
  return kind == Q8_0 || kind == Q4_0 || kind == Q5_0 || kind == IQ4_NL || kind == MXFP4;
}

size_t gemv_i8_workspace_bytes(int64_t M, int64_t K) {
  return i8::align256((size_t)M * K) + 2 * i8::align256((size_t)M * (K / 32) * 4);
}

}  // namespace qmm

// Device scratch of the allocation-free int8 GEMV: the largest workspace that
// gemv_i8_workspace_bytes gives for M * K <= QMM_GEMV_I8_MAX_MK (262144 code
// bytes, then 32768 bytes each of scales and code sums).  Every GPU holds its
// own copy at its own address; host code reaches it only through the address
// looked up below, never through this name.
static __device__ __align__(256) uint8_t scratch[QMM_GEMV_I8_SCRATCH_BYTES];

namespace qmm {

hipError_t gemv_i8_scratch(void **ptr) {
  static_assert(QMM_GEMV_I8_SCRATCH_BYTES == 262144 + 2 * 32768, "scratch = codes + scales + code sums at the largest M * K");
  constexpr int kMaxDevices = 64;
  static std::atomic<void *> addr[kMaxDevices];
  static std::mutex mu;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    // Once per device, with that device current (hipGetDevice above).
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_gemv_i8(int kind, const uint8_t *P, const void *x, int x_f16, float *y, int M, int64_t N,
                          int64_t K, void *ws, hipStream_t st) {
  int8_t *q = static_cast<int8_t *>(ws);
  float *d = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + i8::align256((size_t)M * K));
  int32_t *s = reinterpret_cast<int32_t *>(reinterpret_cast<uint8_t *>(d) + i8::align256((size_t)M * (K / 32) * 4));
  const int nb = (int)(K / 32);
  const int64_t blocks = (int64_t)M * nb;
  const unsigned grid = (unsigned)((blocks * 32 + 255) / 256);
  // The quantizer's code order: Q8_0's, or the nibble order the other
  // kinds share.
  if (kind == Q8_0)
    i8::quantize<Q8_0>(x, x_f16, q, d, s, blocks, nb, grid, st);
  else
    i8::quantize<Q4_0>(x, x_f16, q, d, s, blocks, nb, grid, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (kind) {
    case Q8_0: return i8::run_shape<Q8_0>(P, q, d, s, y, M, N, K, st);
    case Q4_0: return i8::run_shape<Q4_0>(P, q, d, s, y, M, N, K, st);
    case Q5_0: return i8::run_shape<Q5_0>(P, q, d, s, y, M, N, K, st);
    case IQ4_NL: return i8::run_shape<IQ4_NL>(P, q, d, s, y, M, N, K, st);
    case MXFP4: return i8::run_shape<MXFP4>(P, q, d, s, y, M, N, K, st);
    default: break;
  }
  return hipErrorNotSupported;
}

}  // namespace qmm
