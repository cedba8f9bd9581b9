// qmm_repack.hip -- the load-time repack of native GGUF rows into the
// lane-ordered records that the repacked GEMV reads (Vulkore quant_test.cpp,
// section 4, "repacked fast path": a one-time transform at load so that the
// matvec reads aligned planes).
//
// Record layout (also described at Rec in qmm_gemv_mfma.h): rows are grouped
// in tiles of 16, the last tile padded with zero rows; K in k-blocks of 256
// elements, B bytes per row per k-block.  Tile t, k-block b is one record of
// 16 B bytes at (t * n_kblocks + b) * 16 B.  A record is n_lane lane sections
// of 1024 bytes (slot 16 G + j: 16 bytes of row j chosen by G), then row
// sections (slot j: w bytes of row j).  The repack is a byte permutation, so
// it is lossless and the repacked tensor is the native size plus padding.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {
namespace rp {

struct Shape {
  int B;            // bytes of one row's k-block
  int n_lane;       // lane sections
  int n_row;        // row sections
  int width[4];     // bytes per row of each row section
};

template <int KIND> struct Map;

// The 4-bit-code kinds: lane section c, slot (G, j), byte i holds code byte
// 4G + i%4 of block 4c + i/4 (code bytes start at `at` in a block of `bb`).
template <int BB, int AT>
struct NibMap {
  __device__ static int lane(int c, int G, int i) { return BB * (4 * c + i / 4) + AT + 4 * G + i % 4; }
};

template <> struct Map<Q4_0> : NibMap<18, 2> {
  static constexpr Shape shape{144, 2, 1, {16, 0}};
  __device__ static int row(int, int i) { return 18 * (i / 2) + i % 2; }  // the f16 scales
};
template <> struct Map<IQ4_NL> : Map<Q4_0> {};
template <> struct Map<MXFP4> : NibMap<17, 1> {
  static constexpr Shape shape{136, 2, 1, {8, 0}};
  __device__ static int row(int, int i) { return 17 * i; }  // the E8M0 bytes
};
template <> struct Map<Q5_0> : NibMap<22, 6> {
  static constexpr Shape shape{176, 2, 2, {32, 16}};
  __device__ static int row(int sec, int i) {
    return sec == 0 ? 22 * (i / 4) + 2 + i % 4   // the 32-bit qh words
                    : 22 * (i / 2) + i % 2;      // the f16 scales
  }
};
template <> struct Map<Q8_0> {
  static constexpr Shape shape{272, 4, 1, {16, 0}};
  // Section c: code bytes 8G .. 8G+7 of blocks 2c and 2c+1.
  __device__ static int lane(int c, int G, int i) { return 34 * (2 * c + i / 8) + 2 + 8 * G + i % 8; }
  __device__ static int row(int, int i) { return 34 * (i / 2) + i % 2; }
};
template <> struct Map<IQ4_XS> {
  static constexpr Shape shape{136, 2, 1, {8, 0}};
  __device__ static int lane(int c, int G, int i) { return 8 + 16 * (4 * c + i / 4) + 4 * G + i % 4; }
  __device__ static int row(int, int i) { return i; }  // d, scales_h, scales_l
};
template <> struct Map<Q4_K> {
  static constexpr Shape shape{144, 2, 1, {16, 0}};
  __device__ static int lane(int c, int G, int i) { return 16 + 32 * G + 16 * c + i; }
  __device__ static int row(int, int i) { return i; }  // d, dmin, scales and mins
};
template <> struct Map<Q6_K> {
  static constexpr Shape shape{210, 3, 2, {16, 2}};
  __device__ static int lane(int c, int G, int i) {
    const int h = G >> 1, a = G & 1;
    return c == 0 ? 64 * h + 16 * a + i : c == 1 ? 64 * h + 32 + 16 * a + i : 128 + 32 * h + 16 * a + i;
  }
  __device__ static int row(int sec, int i) { return sec == 0 ? 192 + i : 208 + i; }  // scales, d
};

// Q5_K: the Q4_K code sections, then qh[32] and the 16-byte header as row
// sections (every group of a row reads all 32 fifth-bit bytes).
template <> struct Map<Q5_K> {
  static constexpr Shape shape{176, 2, 2, {32, 16}};
  __device__ static int lane(int c, int G, int i) { return 48 + 32 * G + 16 * c + i; }
  __device__ static int row(int sec, int i) { return sec == 0 ? 16 + i : i; }  // qh, then d, dmin, scales
};
// Q2_K and Q3_K: group G = 2n + a takes code bytes 32n + 16a .. + 15.
template <> struct Map<Q2_K> {
  static constexpr Shape shape{84, 1, 2, {16, 4}};
  __device__ static int lane(int, int G, int i) { return 16 + 16 * G + i; }
  __device__ static int row(int sec, int i) { return sec == 0 ? i : 80 + i; }  // scales, then d, dmin
};
template <> struct Map<Q3_K> {
  static constexpr Shape shape{110, 1, 4, {32, 8, 4, 2}};
  __device__ static int lane(int, int G, int i) { return 32 + 16 * G + i; }
  __device__ static int row(int sec, int i) {  // hmask, scale bytes 0-7, scale bytes 8-11, d
    return sec == 0 ? i : sec == 1 ? 96 + i : sec == 2 ? 104 + i : 108 + i;
  }
};

// Row j (in the tile) and offset in its k-block of record byte o.
template <int KIND>
__device__ void source(int o, int &j, int &off) {
  using Mp = Map<KIND>;
  constexpr Shape sh = Mp::shape;
  if (o < 1024 * sh.n_lane) {
    const int c = o >> 10, slot = (o & 1023) >> 4;
    j = slot & 15;
    off = Mp::lane(c, slot >> 4, o & 15);
    return;
  }
  o -= 1024 * sh.n_lane;
#pragma unroll
  for (int sec = 0; sec < sh.n_row; ++sec) {
    if (o < 16 * sh.width[sec] || sec == sh.n_row - 1) {
      j = o / sh.width[sec];
      off = Mp::row(sec, o % sh.width[sec]);
      return;
    }
    o -= 16 * sh.width[sec];
  }
}

// One thread per 4 bytes of the repacked tensor (records are multiples of
// 16 bytes).  Rows past N read as zero.
template <int KIND>
__global__ __launch_bounds__(256) void repack_kernel(const uint8_t *__restrict__ W, uint32_t *__restrict__ P,
                                                     int64_t N, int64_t nkb, int64_t words) {
  constexpr int B = Map<KIND>::shape.B;
  constexpr int kRec = 16 * B;
  const int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (w >= words) return;
  const int64_t byte = 4 * w;
  const int64_t rec = byte / kRec;
  const int o = (int)(byte - rec * kRec);
  const int64_t tile = rec / nkb, kb = rec - tile * nkb;
  const int64_t row_bytes = nkb * B;
  uint32_t v = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    int j, off;
    source<KIND>(o + b, j, off);
    const int64_t row = tile * 16 + j;
    const uint32_t x = row < N ? W[row * row_bytes + kb * B + off] : 0u;
    v |= x << (8 * b);
  }
  P[w] = v;
}

template <int KIND>
hipError_t run(const uint8_t *W, void *P, int64_t N, int64_t K, hipStream_t s) {
  const int64_t nkb = K / 256;
  const int64_t words = packed_bytes_of(KIND, N, K) / 4;
  const int64_t blocks = (words + 255) / 256;
  hipLaunchKernelGGL(repack_kernel<KIND>, dim3((unsigned)blocks), dim3(256), 0, s, W, (uint32_t *)P, N, nkb, words);
  return hipGetLastError();
}

}  // namespace rp

int64_t packed_bytes_of(int kind, int64_t N, int64_t K) {
  int B;
  switch (kind) {
    case Q4_0: case IQ4_NL: case Q4_K: B = 144; break;
    case MXFP4: case IQ4_XS: B = 136; break;
    case Q5_0: B = 176; break;
    case Q8_0: B = 272; break;
    case Q6_K: B = 210; break;
    case Q5_K: B = 176; break;
    case Q2_K: B = 84; break;
    case Q3_K: B = 110; break;
    default: return -1;
  }
  if (K <= 0 || K % 256 != 0 || N <= 0) return -1;
  return (N + 15) / 16 * 16 * (K / 256) * B;
}

hipError_t launch_repack(int kind, const uint8_t *W, void *P, int64_t N, int64_t K, hipStream_t s) {
  switch (kind) {
    case Q4_0: return rp::run<Q4_0>(W, P, N, K, s);
    case IQ4_NL: return rp::run<IQ4_NL>(W, P, N, K, s);
    case MXFP4: return rp::run<MXFP4>(W, P, N, K, s);
    case Q5_0: return rp::run<Q5_0>(W, P, N, K, s);
    case Q8_0: return rp::run<Q8_0>(W, P, N, K, s);
    case IQ4_XS: return rp::run<IQ4_XS>(W, P, N, K, s);
    case Q4_K: return rp::run<Q4_K>(W, P, N, K, s);
    case Q6_K: return rp::run<Q6_K>(W, P, N, K, s);
    case Q5_K: return rp::run<Q5_K>(W, P, N, K, s);
    case Q2_K: return rp::run<Q2_K>(W, P, N, K, s);
    case Q3_K: return rp::run<Q3_K>(W, P, N, K, s);
    default: break;
  }
  return hipErrorNotSupported;
}

}  // namespace qmm
