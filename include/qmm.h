/*
 * qmm.h -- matrix multiply against GGUF block-quantized weights on AMD
 * MI355X (gfx950).  C ABI: plain pointers and sizes, no framework types.
 *
 * The operation (all entry points):  y[m][n] = sum_k x[m][k] * w[n][k]
 *   W  the weight matrix, N rows of K elements.  Each row is K / block_elems
 *      consecutive GGUF blocks and rows are stored back to back, so row n
 *      starts at byte n * qmm_row_bytes(kind, K).  ("One output row's blocks
 *      are contiguous": redgpu/Vulkore examples/llm/quant_test.cpp, the fused
 *      dequant-matvec section; ferrox-cuda 0.21.0 mul_mm.rs, BODY_SRC and
 *      validate_shape.)  Any byte alignment of W is accepted.
 *   x  activations, row-major [M][K], f32 or f16 (QMM_F32 / QMM_F16), aligned
 *      to their element size.
 *   y  output, row-major [M][N] f32 (y[m * N + n]; ferrox-cuda mul_mm.rs,
 *      BODY_SRC, writes dst[token * n_rows + row]).  Overwritten, never
 *      accumulated into.
 * Each weight element w[n][k] is decoded from its block by its kind's rule:
 * scale * code + bias for the affine kinds, scale * table[code] for the
 * codebook kinds (ferrox-cuda 0.20.0 mul_mm_kinds/codebook.rs, module docs).
 *
 * Numerics.  Accumulation is in f32 and at most one factor of each product
 * is rounded, once, to f16 (relative error <= 2^-11).  The decode GEMV keeps
 * every weight exact (an exact f16 integer times an f32 scale) and, on its
 * matrix-core path, rounds f32 activations once to f16.  The prefill GEMM
 * rounds each decoded weight once to f16 and, for f32 activations, splits
 * each activation into two f16 parts so that the activation stays exact to
 * about 2^-22.  Results satisfy |y - y_exact| <= 1e-3 * sum_k |w||x| + 1e-6
 * per element.  Activations are taken in f16 on the matrix-core paths (the
 * GEMV at M <= 8 for every kind but Q2_K, Q3_K and Q5_K, qmm_moe, the GEMM),
 * so an f32 activation must lie within the f16 range, |x| <= 65504; a larger
 * one overflows to infinity there.  qmm_moe_ffn scales its intermediate
 * activations into that range itself.
 *
 * Ownership and asynchrony.  The caller owns every buffer; the library never
 * allocates device memory.  W, x and ids are read only.  Calls that take a
 * `stream` (a hipStream_t; NULL is the default stream) enqueue their kernels
 * there and return without synchronizing; a fault inside a kernel surfaces at
 * the caller's next synchronization.
 *
 * Errors.  Shape and argument errors are returned before anything is
 * launched, checked in this order: empty shape -> unsupported kind -> K not a
 * whole number of blocks -> K > 2^30 or N > INT32_MAX -> bad dtype -> null
 * pointer, misaligned activation or out-of-range M -> workspace too small.  A refused call computes nothing
 * (ferrox-cuda mul_mm.rs: kind_by_name and MulMmUnsupported -- a kind or
 * shape the kernel cannot do must be refused by name, never computed some
 * other way).  A failed launch returns QMM_ERR_HIP.  qmm_last_error() gives
 * the calling thread's most recent message.
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The eleven kinds, by GGUF type id (ferrox-cuda mul_mm.rs, KINDS; MXFP4 is
 * ggml type tag 39 per codebook.rs, the MXFP4 row). */
enum qmm_kind {
    QMM_Q4_0 = 2,    /*  18 B /  32: f16 d, 16 B nibbles; d*(q-8)               */
    QMM_Q5_0 = 6,    /*  22 B /  32: f16 d, u32 qh, 16 B nibbles; d*(q-16)      */
    QMM_Q8_0 = 8,    /*  34 B /  32: f16 d, 32 int8; d*q                        */
    QMM_Q2_K = 10,   /*  84 B / 256: 16 scale/min bytes, 64 B 2-bit, d, dmin    */
    QMM_Q3_K = 11,   /* 110 B / 256: 32 B hmask, 64 B 2-bit, 12 B scales, d    */
    QMM_Q4_K = 12,   /* 144 B / 256: d, dmin, 12 B 6-bit scales/mins, 128 B     */
    QMM_Q5_K = 13,   /* 176 B / 256: d, dmin, 12 B scales/mins, 32 B qh, 128 B  */
    QMM_Q6_K = 14,   /* 210 B / 256: 128 B ql, 64 B qh, 16 int8 scales, d       */
    QMM_IQ4_NL = 20, /*  18 B /  32: f16 d, 16 B codes into a 16-entry table    */
    QMM_IQ4_XS = 23, /* 136 B / 256: d, scales_h, scales_l[4], 128 B codes      */
    QMM_MXFP4 = 39   /*  17 B /  32: E8M0 scale byte, 16 B of E2M1 codes        */
};

enum qmm_dtype { QMM_F32 = 0, QMM_F16 = 1 };

enum qmm_status {
    QMM_OK = 0,
    QMM_ERR_EMPTY_SHAPE = 1,          /* a zero dimension: nothing to launch   */
    QMM_ERR_UNSUPPORTED_KIND = 2,     /* not one of the eleven kinds           */
    QMM_ERR_K_NOT_BLOCK_ALIGNED = 3,  /* K is not a whole number of blocks     */
    QMM_ERR_BAD_DTYPE = 4,            /* activation dtype not QMM_F32/QMM_F16  */
    QMM_ERR_BAD_ARG = 5,              /* null/misaligned pointer, bad M, ids   */
    QMM_ERR_HIP = 6,                  /* a HIP launch failed                   */
    QMM_ERR_WORKSPACE = 7             /* workspace missing or too small        */
};

/* Largest M the decode GEMV takes in one call. */
#define QMM_GEMV_MAX_M 8

/* Decode GEMV, M = 1: y[N] = W . x[K], f32 x, on the default stream.
 * ferrox-cuda mul_mm.rs worth_a_gemm: one token is a matvec. */
int qmm_gemv(int kind, const void *W, const float *x, float *y, int64_t N, int64_t K);

/* Decode GEMV, 1 <= M <= QMM_GEMV_MAX_M tokens, f32 or f16 x, on `stream`.
 * The few-token product below the GEMM threshold of ferrox-cuda mul_mm.rs
 * (worth_a_gemm: a batch that small stays on the matvec arm) and the
 * one-row-per-output decode matvec of inferencelayer cublas_prefill.rs (the
 * q4_0 GEMV family, y[row] = sum over blocks of scale * code . x).
 * Every weight is decoded exactly; f32 x may be rounded once to f16;
 * products accumulate in f32. */
int qmm_gemv_ex(int kind, const void *W, const void *x, int x_dtype, float *y,
                int64_t M, int64_t N, int64_t K, void *stream);

/* Prefill GEMM: C[M][N] = A[M][K] . W^T with f16 A, on the default stream.
 * Weight tiles are decoded to f16 and multiplied on the matrix cores with f32
 * accumulation (inferencelayer cublas_prefill.rs, CublasPrefill::gemm: f16
 * in, f32 accumulate, y = x . W^T).  A decoded weight beyond the f16 range
 * (|w| > 65504) becomes an infinity; the decode GEMV and qmm_moe keep every
 * weight exact instead. */
int qmm_gemm(int kind, const void *W, const void *A, float *C, int64_t M, int64_t N, int64_t K);

/* Prefill GEMM for any M >= 1 with f32 or f16 A, on `stream`: the same
 * contract (inferencelayer cublas_prefill.rs, CublasPrefill::gemm: y = x . W^T,
 * beta 0, f32 accumulate), and ferrox-cuda mul_mm.rs's batched product
 * (BODY_SRC: every token of the batch against every row, dst[token * n_rows
 * + row]).  f32 A is split into two f16 parts (see Numerics above). */
int qmm_gemm_ex(int kind, const void *W, const void *A, int a_dtype, float *C,
                int64_t M, int64_t N, int64_t K, void *stream);

/* Either path, chosen by the number of tokens as ferrox-cuda mul_mm.rs
 * worth_a_gemm chooses between its matvec arm and its GEMM: the GEMV for
 * M <= QMM_GEMV_MAX_M, the GEMM above.  Numerics and errors as the path
 * taken. */
int qmm_matmul(int kind, const void *W, const void *A, int a_dtype, float *C,
               int64_t M, int64_t N, int64_t K, void *stream);

/* Routed SiLU-gated expert FFN with a weighted top-k combine (model
 * semantics beyond the pages, which stop at the routed expert products of
 * qmm_moe).  W_gu holds E experts of 2 * N_ff rows of K elements (rows
 * [0, N_ff) are the gate, [N_ff, 2 N_ff) the up projection); W_d holds E
 * experts of K rows of N_ff elements; both in the layout of qmm_moe.  For
 * token t and slot s with e = ids[t][s] in [0, E):
 *   h = silu(W_gate[e] . X[t]) * (W_up[e] . X[t]),  silu(v) = v / (1 + e^-v)
 *   Y[t] = sum over such slots of topk_w[t][s] * (W_d[e] . h)
 * X is [M][K] f32 or f16; topk_w is [M][topk] f32; Y is [M][K] f32, 16-byte
 * aligned, overwritten.  Slots whose id lies outside [0, E) add nothing.
 * The products run as qmm_moe (each within 1e-3 sum|w||x| + 1e-6), h and
 * the combine in f32; each pair's h is divided by a power of two that
 * brings max|h| to 2^14 or below before the down product (whose matrix-core
 * path takes f16 activations), and the combine multiplies it back, exactly.
 * The sum over slots runs in a fixed order (the same call gives the same
 * bits).  With fewer than four pairs per expert on average (M * topk < 4 E),
 * whole k-blocks (N_ff, K multiples of 256), topk <= 64 and a kind with a
 * matrix-core decoder over the layout given (repacked: as qmm_gemv_packed;
 * native: Q2_K, Q3_K, Q4_K, Q5_K, Q6_K), the FFN runs in two launches:
 * gate/up with the SiLU-product in its epilogue, then down with the combine
 * in its epilogue.
 * workspace: qmm_moe_ffn_workspace_bytes(E, M, topk, N_ff, K) bytes,
 * 256-byte aligned, overwritten; calls sharing it must not overlap.  Errors as qmm_moe, with both matrices' shapes checked (gate/up
 * first) and a NULL topk_w or misaligned Y as QMM_ERR_BAD_ARG. */
int qmm_moe_ffn(int kind, const void *W_gu, const void *W_d, int64_t E, const int32_t *ids,
                const float *topk_w, int64_t topk, const void *X, int x_dtype, float *Y,
                int64_t M, int64_t N_ff, int64_t K, void *workspace, size_t workspace_bytes,
                void *stream);
/* qmm_moe_ffn over repacked experts: P_gu holds E experts' gate/up records
 * (expert e at e * qmm_packed_bytes(kind, 2 N_ff, K)), P_d their down
 * records (at e * qmm_packed_bytes(kind, K, N_ff)), each from qmm_repack of
 * that expert's rows; both 16-byte aligned.  Kinds as qmm_gemv_packed; K
 * and N_ff multiples of 256; M * topk * max(K, N_ff) below 2^31.  Semantics,
 * numerics, workspace and the remaining errors as qmm_moe_ffn. */
int qmm_moe_ffn_packed(int kind, const void *P_gu, const void *P_d, int64_t E, const int32_t *ids,
                       const float *topk_w, int64_t topk, const void *X, int x_dtype, float *Y,
                       int64_t M, int64_t N_ff, int64_t K, void *workspace, size_t workspace_bytes,
                       void *stream);
/* Workspace of qmm_moe_ffn: the routing words of qmm_moe plus f32 gate/up,
 * h, per-slot down outputs and per-pair scales; 0 for a non-positive
 * argument. */
size_t qmm_moe_ffn_workspace_bytes(int64_t E, int64_t M, int64_t topk, int64_t N_ff, int64_t K);

/* Prefill GEMM for MXFP4 weights on the scaled FP8 x FP4 matrix cores, a
 * separately toleranced variant of qmm_gemm_ex for kind QMM_MXFP4 only (the
 * block: an E8M0 scale byte and 32 E2M1 codes; codebook.rs, the MXFP4 row).
 * The weight blocks go to the matrix cores as they are stored; W must be
 * 16-byte aligned, and its rows are fetched as aligned 16-byte pieces, so the
 * last piece may cover up to 12 bytes past the end of W (never past its
 * 16-byte granule, hence never onto another page).  A (f32 or f16,
 * [M][K]) is first quantized into `workspace` to two MX FP8 terms: per row
 * and 32-element block, hi = E4M3(a / 2^e1) with 2^e1 the smallest power of
 * two with max|a| / 2^e1 <= 448, and lo = E4M3(r / 2^e2) of the residual
 * r = a - 2^e1 hi on its own such scale, both rounded to nearest even; the
 * matrix cores multiply both terms by the weights into one f32 sum.  The
 * two roundings (|a - 2^e1 hi - 2^e2 lo| <= 2^-8 |a|, plus 2^(e1 - 14) where
 * hi is subnormal) are the only difference from the exact product besides
 * f32 accumulation, so |C - exact| <= about 2^-8 . sum|w||a|; blocks whose
 * elements are E4M3 values times one power of two come through exactly.
 * Workspace layout (bytes; Mp = M rounded up to 64, rows past M are zero
 * codes with scale byte 0): hi codes [Mp][K], lo codes [Mp][K], hi scale
 * bytes e1 + 127 [Mp][K/32], lo scale bytes e2 + 127 [Mp][K/32]; within
 * each 32-element block the code at position p is element p / 2 (p even)
 * or 16 + p / 2 (p odd), the order of the MXFP4 nibbles.
 * K a multiple of 128 runs the scaled path; any other K runs qmm_gemm_ex's
 * f16 GEMM.  workspace is device memory of at least
 * qmm_gemm_mx_workspace_bytes(M, K) bytes at 16-byte alignment, overwritten by
 * the call; calls that share it must not overlap.  Errors: kinds other than
 * MXFP4 give QMM_ERR_UNSUPPORTED_KIND, a short workspace QMM_ERR_WORKSPACE,
 * M > 65535 * 64 or more than 2^31 - 8 tiles of 64 x 128 QMM_ERR_BAD_ARG,
 * the rest as qmm_gemm_ex. */
int qmm_gemm_mx(int kind, const void *W, const void *A, int a_dtype, float *C,
                int64_t M, int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                void *stream);
/* Bytes of workspace qmm_gemm_mx needs: M rounded up to 64, times
 * 2 * K * 33 / 32; 0 for M <= 0, K <= 0 or K not a multiple of 32. */
size_t qmm_gemm_mx_workspace_bytes(int64_t M, int64_t K);

/* Routed expert products, every expert in one grouped launch (plus a small
 * routing prologue when an expert may receive several pairs).  No page
 * defines this operation: the pages name expert routing only as model
 * context (ferrox-cuda 0.20.0 codebook.rs, the MXFP4 row: gpt-oss expert
 * weights; inferencelayer cublas_prefill.rs, the Qwen3-30B-A3B decode
 * estimate).  It is the batched/expert product of a 128-expert top-8
 * mixture with per-pair semantics and nothing more (no gating weights, no
 * combine).  W holds E experts of N rows each, back to back: expert
 * e's row n starts at byte (e * N + n) * qmm_row_bytes(kind, K).
 * ids is [M][topk] int32 in [0, E).  For token t and slot s with
 * e = ids[t][s]:  Y[t][s][:] = W_e . x, where x is X[t] when x_per_slot is 0
 * (X is [M][K]) and X[t][s] when it is 1 (X is [M][topk][K]).  Y is
 * [M][topk][N] f32.  A pair whose id lies outside [0, E) is skipped and its Y
 * row is left as it was; W is never read outside its E experts.
 * workspace is device memory of at least
 * qmm_moe_workspace_bytes(E, M, topk) bytes, overwritten by the call; calls
 * that share a workspace must not overlap. */
int qmm_moe(int kind, const void *W, int64_t E, const int32_t *ids, int64_t topk,
            const void *X, int x_dtype, int x_per_slot, float *Y,
            int64_t M, int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
            void *stream);
size_t qmm_moe_workspace_bytes(int64_t E, int64_t M, int64_t topk);

/* Load-time repack (Vulkore quant_test.cpp, section 4, "repacked fast
 * path": weights are transformed once when loaded so the decode matvec reads
 * aligned planes; values rebuilt from the repacked bytes must equal the
 * native dequantization bit for bit).  The layout is this library's: rows
 * in tiles of 16 (the last padded with zero rows), K in k-blocks of 256
 * elements; tile t and k-block b form one record of 16 * B bytes at
 * (t * K/256 + b) * 16 * B, B being one row's k-block in native bytes (144
 * for Q4_0, IQ4_NL, Q4_K; 136 for MXFP4, IQ4_XS; 176 Q5_0, Q5_K; 272 Q8_0;
 * 210 Q6_K; 84 Q2_K; 110 Q3_K).  A record holds exactly the bytes of its sixteen native row pieces,
 * permuted: first lane sections of 1024 bytes (16-byte slot 16 G + j holds
 * the code bytes that lane j + 16 G of a wave decodes for row j), then row
 * sections (per row: its scales and headers).  The per-kind byte tables are
 * in qmm_repack.hip.
 *
 * Kinds: all eleven (Q4_0, Q5_0, Q8_0, IQ4_NL, MXFP4, IQ4_XS, Q2_K, Q3_K,
 * Q4_K, Q5_K, Q6_K).  Size in bytes of
 * the repacked tensor of N rows of K elements: qmm_packed_bytes (-1 for any
 * other kind, K not a multiple of 256, or N <= 0). */
int64_t qmm_packed_bytes(int kind, int64_t N, int64_t K);

/* Repack N native rows W (byte-aligned, N * qmm_row_bytes(kind, K) bytes)
 * into P (qmm_packed_bytes(kind, N, K) bytes, 16-byte aligned, overwritten)
 * on `stream`.  Errors: the shape checks of qmm_gemv_ex, then a kind without
 * a repacked layout (QMM_ERR_UNSUPPORTED_KIND), K not a multiple of 256
 * (QMM_ERR_K_NOT_BLOCK_ALIGNED), NULL or misaligned pointers
 * (QMM_ERR_BAD_ARG). */
int qmm_repack(int kind, const void *W, void *P, int64_t N, int64_t K, void *stream);

/* Decode GEMV over repacked weights P (from qmm_repack with the same kind,
 * N and K): y[M][N] = x[M][K] . W^T, 1 <= M <= QMM_GEMV_MAX_M, f32 or f16
 * x, on `stream`; the numerics of qmm_gemv_ex (exact weights, x rounded once
 * to f16, f32 accumulation).  Errors as qmm_repack, plus those of
 * qmm_gemv_ex for x, y and M, and M * K >= 2^31 (QMM_ERR_BAD_ARG). */
int qmm_gemv_packed(int kind, const void *P, const void *x, int x_dtype, float *y,
                    int64_t M, int64_t N, int64_t K, void *stream);

/* Matmul over repacked weights, any M: C[M][N] = A[M][K] . W^T with W given
 * as its qmm_repack records P (16-byte aligned).  This is the prefill-GEMM
 * contract of inferencelayer cublas_prefill.rs (CublasPrefill::gemm: a
 * batch of M tokens against one weight matrix, f32 output, beta = 0) over
 * the repacked fast path of Vulkore quant_test.cpp, section 4.  M <=
 * QMM_GEMV_MAX_M runs qmm_gemv_packed; larger M runs the prefill GEMM over
 * the records, which takes Q8_0, Q4_0, Q5_0, IQ4_NL, MXFP4 and IQ4_XS (other
 * kinds give QMM_ERR_UNSUPPORTED_KIND there).  A is [M][K] f32 or f16, C
 * [M][N] f32, overwritten.  Numerics of the GEMM: each weight rounded once
 * to f16 (the f16 product of the code and the block scale; IQ4_XS instead
 * multiplies each 32-element group's product by its exact f32 scale
 * d * (ls - 32), so its weights are not rounded), f16 activations exact, f32
 * activations split into two
 * f16 halves (hi = RN_f16(a), lo = RN_f16(a - hi)) that are both multiplied,
 * f32 accumulation in a fixed order (deterministic):
 * |C - exact| <= 1e-3 . sum|w||a| + 1e-6; as in qmm_gemm_ex, a weight beyond
 * the f16 range (|w| > 65504) becomes an infinity.  Errors: as qmm_gemv_packed for
 * kind, K, dtype and pointers (without its M limit), M * K >= 2^31
 * QMM_ERR_BAD_ARG; above QMM_GEMV_MAX_M tokens also packed bytes >= 2^31 or
 * A bytes (M * K * 2 for f16, * 4 for f32) >= 2^31 QMM_ERR_BAD_ARG. */
int qmm_matmul_packed(int kind, const void *P, const void *A, int a_dtype, float *C,
                      int64_t M, int64_t N, int64_t K, void *stream);

/* Routed expert products (as qmm_moe) over repacked experts: P holds E
 * experts, expert e's records (qmm_repack of its N rows) at byte
 * e * qmm_packed_bytes(kind, N, K).  Kinds and K as qmm_gemv_packed; every
 * pair runs on the matrix cores, so M * topk * K must stay below 2^31.
 * Semantics, workspace and the remaining errors as qmm_moe. */
int qmm_moe_packed(int kind, const void *P, int64_t E, const int32_t *ids, int64_t topk,
                   const void *X, int x_dtype, int x_per_slot, float *Y,
                   int64_t M, int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                   void *stream);

/* Largest M * K of qmm_gemv_i8 (its per-block scales and code sums are
 * staged in 64 KiB of LDS). */
#define QMM_GEMV_I8_MAX_MK 262144

/* Decode GEMV with integer activations, a separately toleranced variant of
 * qmm_gemv_packed for repacked Q8_0, Q4_0, Q5_0, IQ4_NL or MXFP4 weights,
 * whose codes, table values or doubled E2M1 values are integers that fit in
 * int8 (the integer dot-product
 * path that the ferrox-cuda mul_mm page names and leaves out).  x (f32 or
 * f16, [M][K], finite) is first quantized into `workspace`, per token and
 * 32-element block: amax = max |x|, d = amax / 127 and x / d each rounded to
 * f32 (correctly rounded), then q = x / d rounded to the nearest integer,
 * ties to even (|q| <= 127); an all-zero block has d = 0.  Then
 *   y[t][n] = sum over blocks b of d_w[n][b] d[t][b] (sum_i w_i q_i)
 * with each block's integer dot product exact (Q4_0 as code - 8, Q5_0 as
 * code - 16, IQ4_NL as the table value, MXFP4 as twice its E2M1 value with
 * half the block scale) and the scaling and accumulation in
 * f32: for K <= 32768, y is within 2e-5 * sum |w| |d q| + 1e-6 of the exact
 * product with the rebuilt activations d q (the f32 accumulation adds about
 * K * 2^-31 of that sum beyond), and those lie within d / 2 of x.
 * Workspace (qmm_gemv_i8_workspace_bytes(M, K) bytes, 256-byte aligned,
 * overwritten; calls sharing it must not overlap): the codes [M][K] int8,
 * each block's 32 codes in the lane order of the weight codes (Q8_0: element
 * order; the others: position 8G + e holds element 4G + e for e < 4
 * and 16 + 4G + e - 4 otherwise, G = 0..3); at the next multiple of 256
 * bytes the scales d [M][K/32] f32; at the next, the code sums [M][K/32]
 * int32.  1 <= M <= QMM_GEMV_MAX_M and M * K <= QMM_GEMV_I8_MAX_MK.  Errors:
 * as qmm_gemv_packed, other kinds QMM_ERR_UNSUPPORTED_KIND, a larger M * K
 * QMM_ERR_BAD_ARG, a missing, short or misaligned workspace
 * QMM_ERR_WORKSPACE. */
int qmm_gemv_i8(int kind, const void *P, const void *x, int x_dtype, float *y,
                int64_t M, int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                void *stream);
/* Bytes of workspace qmm_gemv_i8 needs; 0 for M <= 0, K <= 0 or K not a
 * multiple of 32. */
size_t qmm_gemv_i8_workspace_bytes(int64_t M, int64_t K);

/* Bytes of the device scratch that qmm_gemv_i8_noalloc uses on each GPU:
 * qmm_gemv_i8_workspace_bytes at the largest M * K. */
#define QMM_GEMV_I8_SCRATCH_BYTES 327680

/* qmm_gemv_i8 without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It calls no allocating routine;
 * the quantized activations go to a scratch of QMM_GEMV_I8_SCRATCH_BYTES
 * that the library holds in each GPU's memory (a static device array, in
 * place from library load until the process ends; its address on the
 * current device is looked up on the first call there).  Same kernels,
 * arguments, numerics and results bit for bit as qmm_gemv_i8.  Nothing in
 * the scratch needs to start at zero: every call writes all it reads, and
 * the scratch keeps the last call's contents.  Calls that overlap on one
 * GPU (two streams, or two host threads) race on the scratch and must be
 * serialized by the caller; calls on different GPUs do not share it.
 * Errors: as qmm_gemv_i8 without its workspace checks (M * K above
 * QMM_GEMV_I8_MAX_MK, whose workspace would exceed the scratch, gives
 * QMM_ERR_BAD_ARG), and QMM_ERR_HIP when the scratch cannot be located on
 * the current device. */
int qmm_gemv_i8_noalloc(int kind, const void *P, const void *x, int x_dtype, float *y,
                        int64_t M, int64_t N, int64_t K, void *stream);

/* Dequantize n_elems consecutive elements (whole blocks) of W to f32 on
 * `stream`: the GPU dequantization that redgpu/Vulkore quant_test.cpp checks
 * bit for bit against its CPU references (its dequant_q8_0 / _q5_0 / _q4_k /
 * _q6_k kernels, the per-kind dequant test), and ferrox-cuda mul_mm.rs's
 * dequant_twin, one block's elements to f32 by the kind's rule.  Every value
 * is the f32 rounding of the exact value, evaluated scale first with IEEE
 * signed zeros (so MXFP4 code 8 gives -0.0; codebook.rs, the E2M1 table).
 * Errors: as qmm_gemv_ex's kind check, then n_elems not a whole number of
 * blocks (QMM_ERR_K_NOT_BLOCK_ALIGNED), NULL pointers (QMM_ERR_BAD_ARG). */
int qmm_dequant(int kind, const void *W, float *out, int64_t n_elems, void *stream);

/* Geometry and names.  qmm_row_bytes is the expected row length of
 * ferrox-cuda mul_mm.rs validate_shape ((K / block_elems) * block_bytes),
 * -1 for a bad kind or K not a whole number of blocks.  qmm_block_geometry
 * gives a kind's block_bytes and block_elems, the two geometry columns of
 * mul_mm.rs's KINDS rows (QMM_OK, or QMM_ERR_UNSUPPORTED_KIND with the
 * outputs untouched).  qmm_kind_from_name is mul_mm.rs's kind_by_name over
 * the GGUF quant names ("Q4_0", "MXFP4", ...): -1 where kind_by_name gives
 * None, so a caller must fall back and say so.  qmm_kind_name is its
 * inverse (NULL for an unsupported kind).  qmm_status_string names a
 * status; qmm_last_error gives the calling thread's most recent message
 * (the refused check, in the order of validate_shape, or the HIP error). */
int64_t qmm_row_bytes(int kind, int64_t K);
int qmm_block_geometry(int kind, int *block_bytes, int *block_elems);
int qmm_kind_from_name(const char *gguf_name);
const char *qmm_kind_name(int kind);
const char *qmm_status_string(int status);
const char *qmm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QMM_H */
