// qmm_internal.h -- host-side launchers behind the C ABI (not exported).
// Each launcher assumes its arguments were validated by qmm_api.hip and
// returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qmm {

// out[i] for i < n_blocks * block_elems.
hipError_t launch_dequant(int kind, const uint8_t *W, float *out, int64_t n_blocks, hipStream_t s);

// y[M][N] = x[M][K] . W^T, 1 <= M <= 8, x f32 (x_f16 == 0) or f16.
hipError_t launch_gemv(int kind, const uint8_t *W, const void *x, int x_f16, float *y,
                       int M, int64_t N, int64_t K, hipStream_t s);

// The matrix-core GEMV; hipErrorNotSupported for kinds it does not decode.
hipError_t launch_gemv_mfma(int kind, const uint8_t *W, const void *x, int x_f16, float *y,
                            int M, int64_t N, int64_t K, hipStream_t s);

// The repacked layout (qmm_repack): its size in bytes, or -1 for a kind
// without one or K not a multiple of 256; the repack launch; the GEMV over
// it (1 <= M <= 8).
int64_t packed_bytes_of(int kind, int64_t N, int64_t K);
bool packed_supported(int kind);
hipError_t launch_repack(int kind, const uint8_t *W, void *P, int64_t N, int64_t K, hipStream_t s);
hipError_t launch_gemv_packed(int kind, const uint8_t *P, const void *x, int x_f16, float *y, int M, int64_t N,
                              int64_t K, hipStream_t s);
// The 2-to-8-token form of that GEMV (qmm_gemv_xs.hip): activations staged
// once per workgroup; cfg picks a tuning shape in -DQMM_TUNING builds (0: the
// default shape).
hipError_t launch_gemv_xs(int kind, const uint8_t *P, const void *x, int x_f16, float *y, int M, int64_t N,
                          int64_t K, hipStream_t s, int cfg = 0);
// Its single-token form for Q4_K and Q6_K (qmm_gemv_t1.hip): sub-blocks
// kept apart in the rows of the matrix-core product, scales applied after it;
// W repacked (packed) or native rows.
bool gemv_t1_supported(int kind, bool packed = true);
hipError_t launch_gemv_t1(int kind, const uint8_t *W, const void *x, int x_f16, float *y, int64_t N, int64_t K,
                          hipStream_t s, int cfg = 0, bool packed = true);

// The prefill GEMM over repacked weights (any M; qmm_gemm_pk.hip), for the
// kinds gemm_packed_supported names; P offsets must fit in 32 bits.
// Compute units of the current device (looked up once per device).
int device_cus();

bool gemm_packed_supported(int kind);
hipError_t launch_gemm_packed(int kind, const uint8_t *P, const void *A, int a_f16, float *C, int64_t M, int64_t N,
                              int64_t K, hipStream_t s);

// The int8-activation GEMV over repacked Q8_0 / Q4_0 weights (1 <= M <= 8):
// activations quantized into `ws` (gemv_i8_workspace_bytes(M, K) bytes,
// 256-byte aligned), then the integer matrix-core product.
bool gemv_i8_supported(int kind);
size_t gemv_i8_workspace_bytes(int64_t M, int64_t K);
hipError_t launch_gemv_i8(int kind, const uint8_t *P, const void *x, int x_f16, float *y, int M, int64_t N,
                          int64_t K, void *ws, hipStream_t s);
// The current device's copy of the library-owned scratch of
// QMM_GEMV_I8_SCRATCH_BYTES bytes (256-byte aligned) that stands in for `ws`
// in the allocation-free entry point; looked up once per device.
hipError_t gemv_i8_scratch(void **ptr);

// C[M][N] = A[M][K] . W^T, any M >= 1, A f32 (a_f16 == 0) or f16.  Runs
// the wave-private GEMM (qmm_gemm_ks.hip) where gemm_ks_supported, else the
// LDS-tiled GEMM (qmm_gemm.hip, launch_gemm_lds).
bool gemm_ks_supported(int kind, int64_t M, int64_t N, int64_t K, int a_f16);
hipError_t launch_gemm_ks(int kind, const uint8_t *W, const void *A, int a_f16, float *C, int64_t M, int64_t N,
                          int64_t K, hipStream_t s);
hipError_t launch_gemm_lds(int kind, const uint8_t *W, const void *A, int a_f16, float *C, int64_t M, int64_t N,
                           int64_t K, hipStream_t s);
hipError_t launch_gemm(int kind, const uint8_t *W, const void *A, int a_f16, float *C,
                       int64_t M, int64_t N, int64_t K, hipStream_t s);

// Routed SiLU-gated expert FFN with a weighted top-k combine; see
// qmm_moe_ffn in qmm.h.
size_t moe_ffn_workspace_bytes(int64_t E, int64_t M, int64_t topk, int64_t N_ff, int64_t K);
hipError_t launch_moe_ffn(int kind, const uint8_t *W_gu, const uint8_t *W_d, int64_t E, const int32_t *ids,
                          const float *topk_w, int64_t topk, const void *X, int x_f16, float *Y, int64_t M,
                          int64_t N_ff, int64_t K, void *ws, hipStream_t s, bool packed = false);

// MXFP4 weights on the scaled FP8 x FP4 matrix cores (activations quantized
// to MX FP8 into `ws`, gemm_mx_workspace_bytes(M, K) bytes); K not a multiple
// of 128 takes the f16 GEMM.
size_t gemm_mx_workspace_bytes(int64_t M, int64_t K);
hipError_t launch_gemm_mx(const uint8_t *W, const void *A, int a_f16, float *C, int64_t M, int64_t N, int64_t K,
                          void *ws, hipStream_t s);

// Routed expert products; see qmm_moe in qmm.h.  `ws` holds
// moe_workspace_bytes(E, M, topk) bytes.
size_t moe_workspace_bytes(int64_t E, int64_t M, int64_t topk);
// packed: W is E experts in the repacked layout (qmm_moe_packed); the
// matrix-core kernel must then apply (moe_mfma_supported and 32-bit
// activation offsets), which the caller has checked.
// routed: the workspace already holds the routing of these ids for the same
// number of pairs per work item (moe_item_pairs), so it is not recomputed.
hipError_t launch_moe(int kind, const uint8_t *W, int64_t E, const int32_t *ids, int64_t topk,
                      const void *X, int x_f16, int x_per_slot, float *Y, int64_t M, int64_t N,
                      int64_t K, void *ws, hipStream_t s, bool packed = false, bool routed = false);
// Pairs per work item launch_moe uses for these arguments (N does not enter).
int moe_item_pairs(int kind, int64_t E, int64_t M, int64_t topk, int64_t K, bool packed);

// Largest expert count the routing prologue handles.
constexpr int64_t kMoeMaxExperts = 4096;

// Where the grouped expert kernel finds the routing in the workspace (int32
// offsets into it): per-expert offsets, the pair order, the number of work
// items and the items themselves (expert, first pair index).
// With `ids` set (items of one pair), work item i is pair i itself, its
// expert read from ids[i], and the workspace lists are not used.
struct MoeRoute {
  const int32_t *ws;
  int offsets_at, order_at, nwork_at, work_at;
  int topk, x_per_slot;
  const int32_t *ids;
  int E, pairs;
};

// The matrix-core expert kernel: one workgroup per (work item, 16-row
// tile); a work item is up to `mt` (1, 8 or 16) pairs of one expert.
bool moe_mfma_supported(int kind, int64_t K);
// Grouped expert products (work items of mt = 8 or 16 pairs of one expert),
// with each activation k-block staged once per workgroup for several tiles
// (qmm_gemv_xs.hip); repacked experts, or native rows of the kinds
// xs_native_supported names.
hipError_t launch_moe_xs(int kind, const uint8_t *P, const void *X, int x_f16, float *Y, int mt, int64_t N,
                         int64_t K, const MoeRoute &rt, int items, hipStream_t s, bool packed);
// Kinds whose staged-activation kernels also read native rows (decoders that
// load their fields straight from global memory), and its 2-to-8-token GEMV
// over native rows.
bool xs_native_supported(int kind);
hipError_t launch_gemv_xs_native(int kind, const uint8_t *W, const void *x, int x_f16, float *y, int M, int64_t N,
                                 int64_t K, hipStream_t s);
// The routed single-token form of launch_gemv_t1: one pair per workgroup,
// the pair's expert read from rt.ids (MoeRoute below).
hipError_t launch_moe_t1(int kind, const uint8_t *W, const void *X, int x_f16, float *Y, int64_t N, int64_t K,
                         const MoeRoute &rt, int items, hipStream_t s, bool packed);
// packed: W holds the experts' repacked records (expert e at
// e * packed_bytes_of(kind, N, K)).
hipError_t launch_moe_mfma(int kind, const uint8_t *W, const void *X, int x_f16, float *Y, int mt, int64_t N,
                           int64_t K, const MoeRoute &rt, int items, hipStream_t s, bool packed = false);

}  // namespace qmm
