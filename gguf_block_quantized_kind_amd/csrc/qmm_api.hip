// qmm_api.hip -- the exported C ABI: argument checks in the documented
// order, then dispatch to the launchers.  Nothing here allocates.
#include <stdarg.h>
#include <string.h>

#include <cstdio>
#include <string>

#include "../../include/qmm.h"
#include "qmm_internal.h"

#define QMM_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return QMM_OK;
}

struct KindInfo {
  int id;
  const char *name;
  int block_bytes;
  int block_elems;
};

// The kind table (GGUF type ids; ferrox-cuda 0.21.0 mul_mm.rs, KINDS).
constexpr KindInfo kKinds[] = {
    {QMM_Q8_0, "Q8_0", 34, 32},     {QMM_Q4_0, "Q4_0", 18, 32},     {QMM_Q5_0, "Q5_0", 22, 32},
    {QMM_Q2_K, "Q2_K", 84, 256},    {QMM_Q3_K, "Q3_K", 110, 256},   {QMM_Q4_K, "Q4_K", 144, 256},
    {QMM_Q5_K, "Q5_K", 176, 256},   {QMM_Q6_K, "Q6_K", 210, 256},   {QMM_IQ4_NL, "IQ4_NL", 18, 32},
    {QMM_IQ4_XS, "IQ4_XS", 136, 256}, {QMM_MXFP4, "MXFP4", 17, 32},
};

const KindInfo *find_kind(int kind) {
  for (const KindInfo &k : kKinds)
    if (k.id == kind) return &k;
  return nullptr;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Empty shape, then kind, then K alignment: the order of ferrox-cuda
// mul_mm.rs validate_shape.  K and the per-launch sizes must also fit the
// kernels' 32-bit indices.
int check_shape(int kind, int64_t M, int64_t N, int64_t K, const KindInfo **out) {
  if (M <= 0 || N <= 0 || K <= 0)
    return fail(QMM_ERR_EMPTY_SHAPE, "empty shape: M=%lld N=%lld K=%lld", (long long)M, (long long)N,
                (long long)K);
  const KindInfo *k = find_kind(kind);
  if (!k) return fail(QMM_ERR_UNSUPPORTED_KIND, "kind %d is not one of the eleven supported kinds", kind);
  if (K % k->block_elems != 0)
    return fail(QMM_ERR_K_NOT_BLOCK_ALIGNED, "K=%lld is not a whole number of %s blocks (%d elements)",
                (long long)K, k->name, k->block_elems);
  if (K > (int64_t)1 << 30 || N > (int64_t)INT32_MAX)
    return fail(QMM_ERR_BAD_ARG, "K=%lld or N=%lld exceeds the supported range", (long long)K,
                (long long)N);
  *out = k;
  return QMM_OK;
}

int check_dtype(int dtype) {
  if (dtype != QMM_F32 && dtype != QMM_F16) return fail(QMM_ERR_BAD_DTYPE, "dtype %d is neither QMM_F32 nor QMM_F16", dtype);
  return QMM_OK;
}

int check_act(const void *x, int dtype, const char *what) {
  if (!x) return fail(QMM_ERR_BAD_ARG, "%s is NULL", what);
  if (!aligned(x, dtype == QMM_F32 ? 4 : 2))
    return fail(QMM_ERR_BAD_ARG, "%s is not aligned to its element size", what);
  return QMM_OK;
}

int hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(QMM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

QMM_EXPORT int qmm_gemv_ex(int kind, const void *W, const void *x, int x_dtype, float *y, int64_t M,
                           int64_t N, int64_t K, void *stream) {
  const KindInfo *k;
  int st = check_shape(kind, M, N, K, &k);
  if (st) return st;
  if ((st = check_dtype(x_dtype))) return st;
  if (!W || !y) return fail(QMM_ERR_BAD_ARG, "W or y is NULL");
  if ((st = check_act(x, x_dtype, "x"))) return st;
  if (!aligned(y, 4)) return fail(QMM_ERR_BAD_ARG, "y is not 4-byte aligned");
  if (M > QMM_GEMV_MAX_M) return fail(QMM_ERR_BAD_ARG, "GEMV takes 1..%d tokens, got M=%lld", QMM_GEMV_MAX_M, (long long)M);
  return hip_status(qmm::launch_gemv(kind, (const uint8_t *)W, x, x_dtype == QMM_F16, y, (int)M, N, K,
                                     (hipStream_t)stream),
                    "gemv launch");
}

QMM_EXPORT int qmm_gemv(int kind, const void *W, const float *x, float *y, int64_t N, int64_t K) {
  return qmm_gemv_ex(kind, W, x, QMM_F32, y, 1, N, K, nullptr);
}

QMM_EXPORT int qmm_gemm_ex(int kind, const void *W, const void *A, int a_dtype, float *C, int64_t M,
                           int64_t N, int64_t K, void *stream) {
  const KindInfo *k;
  int st = check_shape(kind, M, N, K, &k);
  if (st) return st;
  if ((st = check_dtype(a_dtype))) return st;
  if (!W || !C) return fail(QMM_ERR_BAD_ARG, "W or C is NULL");
  if ((st = check_act(A, a_dtype, "A"))) return st;
  if (!aligned(C, 4)) return fail(QMM_ERR_BAD_ARG, "C is not 4-byte aligned");
  if (M > (int64_t)65535 * 64) return fail(QMM_ERR_BAD_ARG, "M=%lld exceeds the supported range", (long long)M);
  return hip_status(qmm::launch_gemm(kind, (const uint8_t *)W, A, a_dtype == QMM_F16, C, M, N, K,
                                     (hipStream_t)stream),
                    "gemm launch");
}

QMM_EXPORT int qmm_gemm(int kind, const void *W, const void *A, float *C, int64_t M, int64_t N, int64_t K) {
  return qmm_gemm_ex(kind, W, A, QMM_F16, C, M, N, K, nullptr);
}

QMM_EXPORT int qmm_matmul(int kind, const void *W, const void *A, int a_dtype, float *C, int64_t M,
                          int64_t N, int64_t K, void *stream) {
  if (M >= 1 && M <= QMM_GEMV_MAX_M) return qmm_gemv_ex(kind, W, A, a_dtype, C, M, N, K, stream);
  return qmm_gemm_ex(kind, W, A, a_dtype, C, M, N, K, stream);
}

QMM_EXPORT size_t qmm_moe_ffn_workspace_bytes(int64_t E, int64_t M, int64_t topk, int64_t N_ff, int64_t K) {
  if (E <= 0 || M <= 0 || topk <= 0 || N_ff <= 0 || K <= 0) return 0;
  return qmm::moe_ffn_workspace_bytes(E, M, topk, N_ff, K);
}

// Kind, then K % 256 (the repacked layout's k-block), after the usual shape
// checks.
static int check_packed(int kind, int64_t M, int64_t N, int64_t K) {
  const KindInfo *k;
  int st = check_shape(kind, M, N, K, &k);
  if (st) return st;
  if (!qmm::packed_supported(kind))
    return fail(QMM_ERR_UNSUPPORTED_KIND, "%s has no repacked layout", k->name);
  if (K % 256 != 0)
    return fail(QMM_ERR_K_NOT_BLOCK_ALIGNED, "the repacked layout needs K a multiple of 256, got K=%lld",
                (long long)K);
  if (qmm::packed_bytes_of(kind, N, K) > ((int64_t)1 << 40))
    return fail(QMM_ERR_BAD_ARG, "N=%lld, K=%lld exceed the supported range", (long long)N, (long long)K);
  return QMM_OK;
}

static int moe_ffn_checked(int kind, const void *W_gu, const void *W_d, int64_t E, const int32_t *ids,
                           const float *topk_w, int64_t topk, const void *X, int x_dtype, float *Y, int64_t M,
                           int64_t N_ff, int64_t K, void *workspace, size_t workspace_bytes, void *stream,
                           bool packed) {
  const KindInfo *k;
  if (E <= 0 || topk <= 0 || N_ff <= 0)
    return fail(QMM_ERR_EMPTY_SHAPE, "empty shape: E=%lld topk=%lld N_ff=%lld", (long long)E, (long long)topk,
                (long long)N_ff);
  int st = check_shape(kind, M, 2 * N_ff, K, &k);  // gate/up: 2 N_ff rows of K
  if (st) return st;
  if ((st = check_shape(kind, M, K, N_ff, &k))) return st;  // down: K rows of N_ff
  if (packed) {
    if ((st = check_packed(kind, M, 2 * N_ff, K))) return st;
    if ((st = check_packed(kind, M, K, N_ff))) return st;
  }
  if ((st = check_dtype(x_dtype))) return st;
  if (!W_gu || !W_d || !ids || !topk_w || !Y) return fail(QMM_ERR_BAD_ARG, "W_gu, W_d, ids, topk_w or Y is NULL");
  if (packed && (!aligned(W_gu, 16) || !aligned(W_d, 16)))
    return fail(QMM_ERR_BAD_ARG, "the repacked W_gu or W_d is not 16-byte aligned");
  if ((st = check_act(X, x_dtype, "X"))) return st;
  if (!aligned(ids, 4) || !aligned(topk_w, 4)) return fail(QMM_ERR_BAD_ARG, "ids or topk_w is not 4-byte aligned");
  if (!aligned(Y, 16)) return fail(QMM_ERR_BAD_ARG, "Y is not 16-byte aligned");
  if (E > qmm::kMoeMaxExperts) return fail(QMM_ERR_BAD_ARG, "E=%lld exceeds %lld experts", (long long)E, (long long)qmm::kMoeMaxExperts);
  const int64_t P = M * topk;
  if (P > ((int64_t)1 << 31) - 1 || P * (N_ff > K ? 2 * N_ff : K) > ((int64_t)1 << 38) ||
      2 * N_ff > ((int64_t)1 << 31) / 4 || K > ((int64_t)1 << 31) / 4)
    return fail(QMM_ERR_BAD_ARG, "M*topk=%lld with N_ff=%lld, K=%lld exceeds the supported range", (long long)P,
                (long long)N_ff, (long long)K);
  // Repacked experts always run on the matrix cores, whose activation
  // offsets are 32-bit.
  if (packed && P * (N_ff > K ? N_ff : K) >= ((int64_t)1 << 31))
    return fail(QMM_ERR_BAD_ARG, "M*topk*max(K, N_ff)=%lld exceeds 2^31-1", (long long)(P * (N_ff > K ? N_ff : K)));
  const size_t need = qmm::moe_ffn_workspace_bytes(E, M, topk, N_ff, K);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(QMM_ERR_WORKSPACE, "workspace needs %zu bytes (256-byte aligned), got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  return hip_status(qmm::launch_moe_ffn(kind, (const uint8_t *)W_gu, (const uint8_t *)W_d, E, ids, topk_w, topk, X,
                                        x_dtype == QMM_F16, Y, M, N_ff, K, workspace, (hipStream_t)stream, packed),
                    "moe_ffn launch");
}

QMM_EXPORT int qmm_moe_ffn(int kind, const void *W_gu, const void *W_d, int64_t E, const int32_t *ids,
                           const float *topk_w, int64_t topk, const void *X, int x_dtype, float *Y, int64_t M,
                           int64_t N_ff, int64_t K, void *workspace, size_t workspace_bytes, void *stream) {
  return moe_ffn_checked(kind, W_gu, W_d, E, ids, topk_w, topk, X, x_dtype, Y, M, N_ff, K, workspace,
                         workspace_bytes, stream, false);
}

QMM_EXPORT int qmm_moe_ffn_packed(int kind, const void *P_gu, const void *P_d, int64_t E, const int32_t *ids,
                                  const float *topk_w, int64_t topk, const void *X, int x_dtype, float *Y, int64_t M,
                                  int64_t N_ff, int64_t K, void *workspace, size_t workspace_bytes, void *stream) {
  return moe_ffn_checked(kind, P_gu, P_d, E, ids, topk_w, topk, X, x_dtype, Y, M, N_ff, K, workspace,
                         workspace_bytes, stream, true);
}

QMM_EXPORT size_t qmm_gemm_mx_workspace_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || K % 32 != 0) return 0;
  return qmm::gemm_mx_workspace_bytes(M, K);
}

QMM_EXPORT int qmm_gemm_mx(int kind, const void *W, const void *A, int a_dtype, float *C, int64_t M, int64_t N,
                           int64_t K, void *workspace, size_t workspace_bytes, void *stream) {
  const KindInfo *k;
  int st = check_shape(kind, M, N, K, &k);
  if (st) return st;
  if (kind != QMM_MXFP4)
    return fail(QMM_ERR_UNSUPPORTED_KIND, "the scaled FP4 GEMM takes MXFP4 weights only, not kind %d", kind);
  if ((st = check_dtype(a_dtype))) return st;
  if (!W || !C) return fail(QMM_ERR_BAD_ARG, "W or C is NULL");
  if (!aligned(W, 16)) return fail(QMM_ERR_BAD_ARG, "W is not 16-byte aligned");
  if ((st = check_act(A, a_dtype, "A"))) return st;
  if (!aligned(C, 4)) return fail(QMM_ERR_BAD_ARG, "C is not 4-byte aligned");
  // One workgroup per 64 x 128 or 64 x 192 tile in a one-dimensional grid.
  const int64_t Mp = (M + 63) / 64 * 64;
  if (M > (int64_t)65535 * 64 || (Mp / 64) * ((N + 127) / 128) > (int64_t)INT32_MAX - 7 ||
      Mp * K > ((int64_t)1 << 40))
    return fail(QMM_ERR_BAD_ARG, "M=%lld, N=%lld, K=%lld exceed the supported range", (long long)M,
                (long long)N, (long long)K);
  const size_t need = qmm::gemm_mx_workspace_bytes(M, K);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 16))
    return fail(QMM_ERR_WORKSPACE, "workspace needs %zu bytes at 16-byte alignment, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  return hip_status(qmm::launch_gemm_mx((const uint8_t *)W, A, a_dtype == QMM_F16, C, M, N, K, workspace,
                                        (hipStream_t)stream),
                    "gemm_mx launch");
}

QMM_EXPORT size_t qmm_moe_workspace_bytes(int64_t E, int64_t M, int64_t topk) {
  if (E <= 0 || M < 0 || topk <= 0) return 0;
  return qmm::moe_workspace_bytes(E, M, topk);
}

QMM_EXPORT int qmm_moe(int kind, const void *W, int64_t E, const int32_t *ids, int64_t topk, const void *X,
                       int x_dtype, int x_per_slot, float *Y, int64_t M, int64_t N, int64_t K, void *workspace,
                       size_t workspace_bytes, void *stream) {
  const KindInfo *k;
  if (E <= 0 || topk <= 0)
    return fail(QMM_ERR_EMPTY_SHAPE, "empty shape: E=%lld topk=%lld", (long long)E, (long long)topk);
  int st = check_shape(kind, M, N, K, &k);
  if (st) return st;
  if ((st = check_dtype(x_dtype))) return st;
  if (!W || !ids || !Y) return fail(QMM_ERR_BAD_ARG, "W, ids or Y is NULL");
  if ((st = check_act(X, x_dtype, "X"))) return st;
  if (!aligned(ids, 4) || !aligned(Y, 4)) return fail(QMM_ERR_BAD_ARG, "ids or Y is not 4-byte aligned");
  if (x_per_slot != 0 && x_per_slot != 1) return fail(QMM_ERR_BAD_ARG, "x_per_slot must be 0 or 1");
  if (E > qmm::kMoeMaxExperts) return fail(QMM_ERR_BAD_ARG, "E=%lld exceeds %lld experts", (long long)E, (long long)qmm::kMoeMaxExperts);
  if (M * topk > ((int64_t)1 << 31) - 1) return fail(QMM_ERR_BAD_ARG, "M*topk exceeds 2^31-1");
  if (N > ((int64_t)1 << 31) / 4) return fail(QMM_ERR_BAD_ARG, "N=%lld exceeds the supported range", (long long)N);
  const size_t need = qmm::moe_workspace_bytes(E, M, topk);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 4))
    return fail(QMM_ERR_WORKSPACE, "workspace needs %zu bytes (4-byte aligned), got %zu", need, workspace_bytes);
  return hip_status(qmm::launch_moe(kind, (const uint8_t *)W, E, ids, topk, X, x_dtype == QMM_F16, x_per_slot,
                                    Y, M, N, K, workspace, (hipStream_t)stream),
                    "moe launch");
}

QMM_EXPORT int64_t qmm_packed_bytes(int kind, int64_t N, int64_t K) {
  if (!qmm::packed_supported(kind)) return -1;
  return qmm::packed_bytes_of(kind, N, K);
}

QMM_EXPORT int qmm_repack(int kind, const void *W, void *P, int64_t N, int64_t K, void *stream) {
  int st = check_packed(kind, 1, N, K);
  if (st) return st;
  if (!W || !P) return fail(QMM_ERR_BAD_ARG, "W or P is NULL");
  if (!aligned(P, 16)) return fail(QMM_ERR_BAD_ARG, "P is not 16-byte aligned");
  return hip_status(qmm::launch_repack(kind, (const uint8_t *)W, P, N, K, (hipStream_t)stream), "repack launch");
}

QMM_EXPORT int qmm_gemv_packed(int kind, const void *P, const void *x, int x_dtype, float *y, int64_t M, int64_t N,
                               int64_t K, void *stream) {
  int st = check_packed(kind, M, N, K);
  if (st) return st;
  if ((st = check_dtype(x_dtype))) return st;
  if (!P || !y) return fail(QMM_ERR_BAD_ARG, "P or y is NULL");
  if (!aligned(P, 16)) return fail(QMM_ERR_BAD_ARG, "P is not 16-byte aligned");
  if ((st = check_act(x, x_dtype, "x"))) return st;
  if (!aligned(y, 4)) return fail(QMM_ERR_BAD_ARG, "y is not 4-byte aligned");
  if (M > QMM_GEMV_MAX_M) return fail(QMM_ERR_BAD_ARG, "GEMV takes 1..%d tokens, got M=%lld", QMM_GEMV_MAX_M, (long long)M);
  if (M * K >= ((int64_t)1 << 31)) return fail(QMM_ERR_BAD_ARG, "M*K=%lld exceeds 2^31-1", (long long)(M * K));
  return hip_status(qmm::launch_gemv_packed(kind, (const uint8_t *)P, x, x_dtype == QMM_F16, y, (int)M, N, K,
                                            (hipStream_t)stream),
                    "gemv_packed launch");
}

QMM_EXPORT int qmm_matmul_packed(int kind, const void *P, const void *A, int a_dtype, float *C, int64_t M, int64_t N,
                                 int64_t K, void *stream) {
  int st = check_packed(kind, M, N, K);
  if (st) return st;
  if ((st = check_dtype(a_dtype))) return st;
  if (!P || !C) return fail(QMM_ERR_BAD_ARG, "P or C is NULL");
  if (!aligned(P, 16)) return fail(QMM_ERR_BAD_ARG, "P is not 16-byte aligned");
  if ((st = check_act(A, a_dtype, "A"))) return st;
  if (!aligned(C, 4)) return fail(QMM_ERR_BAD_ARG, "C is not 4-byte aligned");
  if (M * K >= ((int64_t)1 << 31)) return fail(QMM_ERR_BAD_ARG, "M*K=%lld exceeds 2^31-1", (long long)(M * K));
  if (M <= QMM_GEMV_MAX_M)
    return hip_status(qmm::launch_gemv_packed(kind, (const uint8_t *)P, A, a_dtype == QMM_F16, C, (int)M, N, K,
                                              (hipStream_t)stream),
                      "matmul_packed launch (GEMV)");
  if (!qmm::gemm_packed_supported(kind))
    return fail(QMM_ERR_UNSUPPORTED_KIND, "the prefill GEMM over repacked weights does not take kind %d (M > %d)",
                kind, QMM_GEMV_MAX_M);
  // The GEMM addresses P and A through buffer descriptors with signed 32-bit
  // byte offsets.
  const int64_t a_bytes = M * K * (a_dtype == QMM_F16 ? 2 : 4);
  if (qmm::packed_bytes_of(kind, N, K) >= ((int64_t)1 << 31) || a_bytes >= ((int64_t)1 << 31) ||
      M >= ((int64_t)1 << 24))
    return fail(QMM_ERR_BAD_ARG, "N=%lld, K=%lld, M=%lld exceed the GEMM's 32-bit offsets", (long long)N,
                (long long)K, (long long)M);
  return hip_status(qmm::launch_gemm_packed(kind, (const uint8_t *)P, A, a_dtype == QMM_F16, C, M, N, K,
                                            (hipStream_t)stream),
                    "matmul_packed launch (GEMM)");
}

QMM_EXPORT size_t qmm_gemv_i8_workspace_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0 || K % 32 != 0) return 0;
  return qmm::gemv_i8_workspace_bytes(M, K);
}

namespace {

// The checks qmm_gemv_i8 and qmm_gemv_i8_noalloc share, in the documented order.
int check_gemv_i8(int kind, const void *P, const void *x, int x_dtype, const float *y, int64_t M, int64_t N,
                  int64_t K) {
  int st = check_packed(kind, M, N, K);
  if (st) return st;
  if (!qmm::gemv_i8_supported(kind))
    return fail(QMM_ERR_UNSUPPORTED_KIND,
                "the int8-activation GEMV takes Q8_0, Q4_0, Q5_0, IQ4_NL or MXFP4 weights, not kind %d", kind);
  if ((st = check_dtype(x_dtype))) return st;
  if (!P || !y) return fail(QMM_ERR_BAD_ARG, "P or y is NULL");
  if (!aligned(P, 16)) return fail(QMM_ERR_BAD_ARG, "P is not 16-byte aligned");
  if ((st = check_act(x, x_dtype, "x"))) return st;
  if (!aligned(y, 4)) return fail(QMM_ERR_BAD_ARG, "y is not 4-byte aligned");
  if (M > QMM_GEMV_MAX_M) return fail(QMM_ERR_BAD_ARG, "GEMV takes 1..%d tokens, got M=%lld", QMM_GEMV_MAX_M, (long long)M);
  if (M * K > (int64_t)QMM_GEMV_I8_MAX_MK)
    return fail(QMM_ERR_BAD_ARG, "M*K=%lld exceeds %d (the block scales are staged in LDS)", (long long)(M * K),
                QMM_GEMV_I8_MAX_MK);
  return QMM_OK;
}

}  // namespace

QMM_EXPORT int qmm_gemv_i8(int kind, const void *P, const void *x, int x_dtype, float *y, int64_t M, int64_t N,
                           int64_t K, void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_gemv_i8(kind, P, x, x_dtype, y, M, N, K);
  if (st) return st;
  const size_t need = qmm::gemv_i8_workspace_bytes(M, K);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
    return fail(QMM_ERR_WORKSPACE, "workspace needs %zu bytes (256-byte aligned), got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  return hip_status(qmm::launch_gemv_i8(kind, (const uint8_t *)P, x, x_dtype == QMM_F16, y, (int)M, N, K, workspace,
                                        (hipStream_t)stream),
                    "gemv_i8 launch");
}

QMM_EXPORT int qmm_gemv_i8_noalloc(int kind, const void *P, const void *x, int x_dtype, float *y, int64_t M,
                                   int64_t N, int64_t K, void *stream) {
  int st = check_gemv_i8(kind, P, x, x_dtype, y, M, N, K);
  if (st) return st;
  const size_t need = qmm::gemv_i8_workspace_bytes(M, K);
  if (need > (size_t)QMM_GEMV_I8_SCRATCH_BYTES)  // excluded by the M * K limit; kept as the scratch's own bound
    return fail(QMM_ERR_BAD_ARG, "M=%lld K=%lld needs %zu bytes of scratch, more than the %d the library holds",
                (long long)M, (long long)K, need, QMM_GEMV_I8_SCRATCH_BYTES);
  void *scratch = nullptr;
  hipError_t e = qmm::gemv_i8_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "locating the gemv_i8 scratch on the current device");
  return hip_status(qmm::launch_gemv_i8(kind, (const uint8_t *)P, x, x_dtype == QMM_F16, y, (int)M, N, K, scratch,
                                        (hipStream_t)stream),
                    "gemv_i8_noalloc launch");
}

QMM_EXPORT int qmm_moe_packed(int kind, const void *P, int64_t E, const int32_t *ids, int64_t topk, const void *X,
                              int x_dtype, int x_per_slot, float *Y, int64_t M, int64_t N, int64_t K, void *workspace,
                              size_t workspace_bytes, void *stream) {
  if (E <= 0 || topk <= 0)
    return fail(QMM_ERR_EMPTY_SHAPE, "empty shape: E=%lld topk=%lld", (long long)E, (long long)topk);
  int st = check_packed(kind, M, N, K);
  if (st) return st;
  if ((st = check_dtype(x_dtype))) return st;
  if (!P || !ids || !Y) return fail(QMM_ERR_BAD_ARG, "P, ids or Y is NULL");
  if (!aligned(P, 16)) return fail(QMM_ERR_BAD_ARG, "P is not 16-byte aligned");
  if ((st = check_act(X, x_dtype, "X"))) return st;
  if (!aligned(ids, 4) || !aligned(Y, 4)) return fail(QMM_ERR_BAD_ARG, "ids or Y is not 4-byte aligned");
  if (x_per_slot != 0 && x_per_slot != 1) return fail(QMM_ERR_BAD_ARG, "x_per_slot must be 0 or 1");
  if (E > qmm::kMoeMaxExperts) return fail(QMM_ERR_BAD_ARG, "E=%lld exceeds %lld experts", (long long)E, (long long)qmm::kMoeMaxExperts);
  if (M * topk > ((int64_t)1 << 31) - 1 || M * topk * K >= ((int64_t)1 << 31))
    return fail(QMM_ERR_BAD_ARG, "M*topk*K=%lld exceeds 2^31-1", (long long)(M * topk * K));
  if (N > ((int64_t)1 << 31) / 4) return fail(QMM_ERR_BAD_ARG, "N=%lld exceeds the supported range", (long long)N);
  if (E * qmm::packed_bytes_of(kind, N, K) > ((int64_t)1 << 40))
    return fail(QMM_ERR_BAD_ARG, "E=%lld experts of N=%lld, K=%lld exceed the supported range", (long long)E,
                (long long)N, (long long)K);
  const size_t need = qmm::moe_workspace_bytes(E, M, topk);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 4))
    return fail(QMM_ERR_WORKSPACE, "workspace needs %zu bytes (4-byte aligned), got %zu", need, workspace_bytes);
  return hip_status(qmm::launch_moe(kind, (const uint8_t *)P, E, ids, topk, X, x_dtype == QMM_F16, x_per_slot, Y, M,
                                    N, K, workspace, (hipStream_t)stream, true),
                    "moe_packed launch");
}

QMM_EXPORT int qmm_dequant(int kind, const void *W, float *out, int64_t n_elems, void *stream) {
  if (n_elems <= 0) return fail(QMM_ERR_EMPTY_SHAPE, "empty shape: n_elems=%lld", (long long)n_elems);
  const KindInfo *k = find_kind(kind);
  if (!k) return fail(QMM_ERR_UNSUPPORTED_KIND, "kind %d is not one of the eleven supported kinds", kind);
  if (n_elems % k->block_elems != 0)
    return fail(QMM_ERR_K_NOT_BLOCK_ALIGNED, "n_elems=%lld is not a whole number of %s blocks", (long long)n_elems, k->name);
  if (!W || !out) return fail(QMM_ERR_BAD_ARG, "W or out is NULL");
  if (!aligned(out, 4)) return fail(QMM_ERR_BAD_ARG, "out is not 4-byte aligned");
  if (n_elems > ((int64_t)1 << 40)) return fail(QMM_ERR_BAD_ARG, "n_elems exceeds the supported range");
  return hip_status(qmm::launch_dequant(kind, (const uint8_t *)W, out, n_elems / k->block_elems, (hipStream_t)stream),
                    "dequant launch");
}

QMM_EXPORT int64_t qmm_row_bytes(int kind, int64_t K) {
  const KindInfo *k = find_kind(kind);
  if (!k || K < 0 || K % k->block_elems != 0) return -1;
  return (K / k->block_elems) * k->block_bytes;
}

QMM_EXPORT int qmm_block_geometry(int kind, int *block_bytes, int *block_elems) {
  const KindInfo *k = find_kind(kind);
  if (!k) return fail(QMM_ERR_UNSUPPORTED_KIND, "kind %d is not one of the eleven supported kinds", kind);
  if (block_bytes) *block_bytes = k->block_bytes;
  if (block_elems) *block_elems = k->block_elems;
  return ok();
}

QMM_EXPORT int qmm_kind_from_name(const char *name) {
  if (!name) return -1;
  for (const KindInfo &k : kKinds)
    if (strcmp(k.name, name) == 0) return k.id;
  return -1;
}

QMM_EXPORT const char *qmm_kind_name(int kind) {
  const KindInfo *k = find_kind(kind);
  return k ? k->name : nullptr;
}

QMM_EXPORT const char *qmm_status_string(int status) {
  switch (status) {
    case QMM_OK: return "ok";
    case QMM_ERR_EMPTY_SHAPE: return "empty shape";
    case QMM_ERR_UNSUPPORTED_KIND: return "unsupported kind";
    case QMM_ERR_K_NOT_BLOCK_ALIGNED: return "K is not a whole number of blocks";
    case QMM_ERR_BAD_DTYPE: return "bad activation dtype";
    case QMM_ERR_BAD_ARG: return "bad argument";
    case QMM_ERR_HIP: return "HIP launch failed";
    case QMM_ERR_WORKSPACE: return "workspace missing or too small";
  }
  return "unknown status";
}

QMM_EXPORT const char *qmm_last_error(void) { return g_last_error.c_str(); }
