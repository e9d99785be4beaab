/*
 * fa.h — C ABI of libfa.so: exact, IO-aware tiled attention on AMD Instinct
 * MI355X (gfx950).
 *
 * The operation.  For every (batch b, head h) pair, with Q, K, V of shape N x d:
 *     S = scale * Q K^T,   A = softmax(S) row-wise,   O = A V
 * (the three-step definition of the CMU 11-868 FlashAttention guest-lecture
 * notes on quidproquo.cc, section "The scenario", slide page 5, with the
 * caller's scale on the scores).  With causal != 0, key j is visible to query
 * i only when j <= i; masked scores take no weight.  The N x N matrices S and
 * A never exist in device memory: the forward pass walks K/V tiles with the
 * online-softmax rescaling of the Lecture 9 notes on cs2680.com, section 9.4,
 * keeping a running row max and running denominator on chip, and stores one
 * float per row, the natural log-sum-exp of the scaled, masked scores
 * (LSE_i = m_i + ln l_i).  The backward pass recomputes score tiles from Q, K
 * and LSE instead of storing them (Lecture 9 section 9.6; CMU notes slide page
 * 14), after a preprocess D_i = sum_c dO_ic * O_ic.
 *
 * Layout.  Q, K, V, O, dO, dQ, dK, dV are contiguous row-major [B, H, N, d]
 * arrays of `dtype` (d is the fastest index).  LSE and the backward workspace
 * are contiguous float32 [B, H, N].
 *
 * Ownership and execution.  Every pointer is device memory owned by the
 * caller.  Inputs are only read; outputs must not alias inputs (not checked).
 * The library never allocates, frees or synchronises device memory; every call
 * enqueues its kernels on `hip_stream` (a hipStream_t; NULL = the null stream)
 * and returns without waiting.  Calls are thread-safe; the last error text is
 * kept per thread.
 *
 * Errors.  All validation happens before anything is launched; a failing call
 * returns a negative fa_status and launches nothing.  FA_ERR_HIP reports a
 * launch failure (text via fa_last_error()).  Unsupported combinations return
 * FA_ERR_UNSUPPORTED rather than a wrong answer.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null pointer, B/H/N <= 0, bad dtype, non-finite scale,
                              misaligned pointer (tensors 16-byte aligned, LSE 4-byte;
                              the FP8 entry points state their own), size overflow,
                              key/value head count not dividing H */
  FA_ERR_UNSUPPORTED = -2, /* d not in {64, 128}; scale <= 0; fp32 backward or decode;
                              decode with more than 32 query rows per key/value head;
                              N * d >= 2^30 (N = Nk for decode: one head of K or V
                              must stay below 2 GB) */
  FA_ERR_WORKSPACE = -3,   /* workspace NULL, misaligned, or smaller than
                              fa_backward_workspace_size / fa_decode_workspace_size */
  FA_ERR_HIP = -4          /* a HIP launch failed; see fa_last_error() */
} fa_status;

/*
 * Forward pass.  Writes O ([B,H,N,d], dtype) and LSE ([B,H,N], float32, natural
 * log of the sum of exp of the scaled masked scores of each row).  Any N >= 1 is
 * accepted; d must be 64 or 128; scale must be finite and > 0 (the kernels fold
 * scale * log2(e) into a single fused multiply-add ahead of exp2, which assumes
 * the row maximum of the scaled scores is scale times that of the raw scores).
 * Accumulation is float32 throughout; for fp16/bf16 the probabilities are
 * rounded to the input dtype (round-to-nearest-even) before the PV product and
 * O is rounded once at the end.
 * Defined by: CMU 11-868 notes slide page 5 (the operation), Lecture 9 section
 * 9.4 (online softmax, divide by the denominator once at the end).
 */
int fa_forward(const void* Q, const void* K, const void* V, void* O, float* LSE,
               int B, int H, int N, int d, int causal, float scale, int dtype,
               void* hip_stream);

/*
 * Forward pass with grouped key/value heads: Q and O are [B,H,N,d], K and V are
 * [B,Hkv,N,d] with Hkv dividing H, and query head h reads key/value head
 * h / (H / Hkv) (the g = H / Hkv query heads sharing one key/value head are
 * adjacent).  Hkv = H is exactly fa_forward.  Hkv <= 0 or not dividing H is
 * FA_ERR_INVALID_ARG; otherwise as fa_forward.
 * Defined by: CMU 11-868 notes slide pages 57-60 (in MQA/GQA several query heads
 * share one set of keys and values); each query head's output is the
 * definition of fa_forward over its key/value head.
 */
int fa_forward_gqa(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   int B, int H, int Hkv, int N, int d, int causal, float scale, int dtype,
                   void* hip_stream);

/*
 * Same computation as fa_forward, instrumented: additionally writes the class of
 * every (query tile, key tile) pair the forward kernel considered into
 * tile_codes ([B,H,nQ,nK] uint8, nQ = ceil(N/Br), nK = ceil(N/Bc) with Br, Bc
 * from fa_tile_config(causal ? 0 : 3, ...)): 0 = skipped (no visible element), 1 = full
 * (every element visible), 2 = partially masked (causal diagonal or ragged
 * tail), with bit 4 set on partial tiles that reach past N.  O and LSE are
 * bitwise identical to fa_forward's.  Intended for tests.
 * Defined by: CMU 11-868 notes slide page 5 (the operation, as fa_forward) and
 * slide page 12 (attention is computed block by block over tiles of keys);
 * which tiles hold no visible element, only visible elements or both follows
 * from the causal mask (key j visible to query i iff j <= i) and from N.
 */
int fa_forward_blockmap(const void* Q, const void* K, const void* V, void* O, float* LSE,
                        int B, int H, int N, int d, int causal, float scale, int dtype,
                        unsigned char* tile_codes, void* hip_stream);

/* Bytes of device workspace fa_backward needs: two float32 per row, D and
 * LSE * log2(e). */
size_t fa_backward_workspace_size(int B, int H, int N, int d);

/*
 * Backward pass of L = <dO, O>: given Q, K, V, the forward's O and LSE, and dO,
 * writes dQ, dK, dV ([B,H,N,d], same dtype as the inputs).  Runs two kernels
 * on hip_stream: a dQ kernel (one workgroup per query tile, walking key tiles
 * and recomputing P = exp(scale*QK^T - LSE) on chip), which also forms
 * D = rowsum(dO * O) and LSE * log2(e) of its rows into the workspace (float32
 * [B,H,N] each, in that order); then a dK/dV kernel (one workgroup per key
 * tile, walking query tiles, reading D and LSE * log2(e) from the workspace).
 * No atomics: results are deterministic.  fp16/bf16 only;
 * d must be 64 or 128.  Defined by: Lecture 9 section 9.6 and CMU 11-868 notes
 * slide page 14 (recompute instead of store); the gradients are the chain rule
 * through the row softmax.
 */
int fa_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                const float* LSE, void* dQ, void* dK, void* dV,
                int B, int H, int N, int d, int causal, float scale, int dtype,
                void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * fa_backward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): D and LSE * log2(e) go to a static 8 MiB array the
 * library holds in each device's memory for the life of the process, so
 * B * H * N may be at most 2^20 (1048576) rows; larger inputs return
 * FA_ERR_WORKSPACE before anything is launched.  The array's device address is
 * looked up on the first call on each device (the device of hip_stream, or
 * the current device for the null stream).  The call allocates, frees and
 * synchronises nothing; the same kernels as fa_backward run, so dQ, dK, dV are
 * bitwise those of fa_backward.  Every call on one device shares that
 * device's array: calls that overlap on one device (e.g. on two streams)
 * race and must be ordered by the caller.  Arguments, layouts and other
 * errors as fa_backward.
 */
int fa_backward_noalloc(const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                        int B, int H, int N, int d, int causal, float scale, int dtype,
                        void* hip_stream);

/* Bytes of device workspace fa_backward_gqa needs: fa_backward_workspace_size
 * (B, H, N, d) when the grouped dK/dV pass runs one workgroup per key/value head
 * and key tile; when the grid would be small (fewer than 512 workgroups) each
 * group is split over several workgroups, and the workspace also holds their
 * fp32 partial dK and dV.  Returns 0 for invalid shapes. */
size_t fa_backward_gqa_workspace_size(int B, int H, int Hkv, int N, int d);

/*
 * Backward pass with grouped key/value heads (layouts as fa_forward_gqa): dQ is
 * [B,H,N,d], dK and dV are [B,Hkv,N,d] and hold, for each key/value head, the
 * sum of the gradients of the g query heads that share it (the chain rule for a
 * shared input).  The dK/dV kernel walks the query heads of a group one after
 * the other inside one workgroup, so the sum is formed in registers without
 * atomics.  When the grid would be small the group is split over several
 * workgroups; each writes fp32 partial sums to the workspace and a reduction
 * kernel adds the parts in a fixed order.  Runs are deterministic.  The
 * workspace must hold fa_backward_gqa_workspace_size(B, H, Hkv, N, d) bytes.
 * Hkv = H is exactly fa_backward.
 * Hkv <= 0 or not dividing H is FA_ERR_INVALID_ARG; otherwise as fa_backward.
 * Defined by: as fa_backward, per query head, with the sharing of fa_forward_gqa.
 */
int fa_backward_gqa(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                    const float* LSE, void* dQ, void* dK, void* dV,
                    int B, int H, int Hkv, int N, int d, int causal, float scale, int dtype,
                    void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Same computation as fa_backward, instrumented: additionally writes the class
 * of every (query tile, key tile) pair each backward kernel considered, coded as
 * in fa_forward_blockmap (0 skipped above the causal diagonal, 1 full, 2
 * partial, | 4 past N).  The dK/dV kernel walks query tiles inside a key tile:
 * dkdv_codes is [B,H,nK1,nQ1] uint8, key tile major, with (Br, Bc) =
 * fa_tile_config(1, ...), nQ1 = ceil(N/Br), nK1 = ceil(N/Bc).  The dQ kernel
 * walks key tiles inside a query tile: dq_codes is [B,H,nQ2,nK2] with (Br, Bc) =
 * fa_tile_config(2, ...).  Both buffers are device memory owned by the caller;
 * NULL is FA_ERR_INVALID_ARG.  dQ, dK, dV are bitwise identical to fa_backward's.
 * Defined by: CMU 11-868 notes slide page 14 (the backward recomputes
 * attention tile by tile from Q, K and V); which tiles are skipped or masked
 * follows from the causal mask exactly as in the forward.  Intended for tests.
 */
int fa_backward_blockmap(const void* Q, const void* K, const void* V, const void* O,
                         const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                         int B, int H, int N, int d, int causal, float scale, int dtype,
                         void* workspace, size_t workspace_bytes, unsigned char* dkdv_codes,
                         unsigned char* dq_codes, void* hip_stream);

/*
 * One stage of the backward, for callers that schedule or time the stages
 * separately: stage 0 = preprocess (reads O, dO, LSE; writes D = rowsum(dO * O)
 * and LSE * log2(e) per query row to the workspace), 1 = dK/dV (reads Q, K, V,
 * dO and the workspace; writes dK, dV), 2 = dQ (reads Q, K, V, O, dO, LSE;
 * forms D and LSE * log2(e) of its own rows, writes them to the workspace and
 * writes dQ).  Pointers a stage does not touch may be NULL.  fa_backward is
 * exactly stage 2 then stage 1 on one stream; stage 1 needs stage 0 or stage 2
 * to have filled the workspace first (0, 1, 2 in order also works, with D
 * summed in the preprocess's order for dK/dV).  Errors as fa_backward; an
 * unknown stage is FA_ERR_INVALID_ARG.
 */
int fa_backward_stage(int stage, const void* Q, const void* K, const void* V, const void* O,
                      const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                      int B, int H, int N, int d, int causal, float scale, int dtype,
                      void* workspace, size_t workspace_bytes, void* hip_stream);

/*
 * Split-K decode: attention of a short block of Nq queries (e.g. one new token
 * per sequence) against a key/value cache of Nk >= Nq keys, with H query heads
 * and Hkv key/value heads (Hkv divides H; query head h reads key/value head
 * h / (H / Hkv): grouped-query attention, Hkv = H for multi-head attention).
 * Q and O are [B,H,Nq,d], K and V are [B,Hkv,Nk,d] (fp16 or bf16, d fastest,
 * contiguous, 16-byte aligned); LSE is float32 [B,H,Nq] (natural log, as in
 * fa_forward).  The queries are the last Nq positions of the sequence: with
 * causal != 0, query i sees keys j <= Nk - Nq + i (for Nq = Nk this is
 * fa_forward's mask; for Nq = 1 every key is visible).  The (H/Hkv) * Nq query
 * rows of one key/value head are packed into one block of at most 32 rows and
 * processed together, so every cache is read once.  The cache is split into
 * num_splits slices of whole 32-key tiles (0 = the library's choice, see
 * fa_decode_num_splits; larger counts are clamped to the tile count and to
 * 512); every slice is reduced by its own workgroup, which leaves an
 * unnormalised partial output, running max and two denominators per query row
 * in the workspace, and a second kernel merges the slices' partials with the
 * running-max rescaling (with a single slice the split kernel writes O and LSE
 * itself and no combine is launched, bitwise the same result as the two-kernel
 * path).  The result does not depend on the split beyond float32 rounding.
 * Accumulation and rounding as in fa_forward.
 * Errors: Hkv not dividing H, Nq > Nk or num_splits < 0 is FA_ERR_INVALID_ARG;
 * (H/Hkv) * Nq > 32, fp32, or d outside {64, 128} is FA_ERR_UNSUPPORTED; a
 * workspace smaller than fa_decode_workspace_size(...), NULL or not 16-byte
 * aligned is FA_ERR_WORKSPACE; otherwise as fa_forward.
 * Defined by: Lecture 9 notes section 9.8 (decode reads the whole cache for one
 * FLOP per byte; split-K spreads one sequence's cache over many compute units
 * and merges the partial softmax statistics with the rescaling of section 9.4);
 * CMU 11-868 notes slide pages 57-60 (Flash-Decoding splits along the key/value
 * length; GQA packing fills the matrix tile with the query heads that share a
 * key/value head) and slide page 12 (the rescaling identity the merge uses).
 */
int fa_decode(const void* Q, const void* K, const void* V, void* O, float* LSE,
              int B, int H, int Hkv, int Nq, int Nk, int d, int causal, float scale,
              int dtype, int num_splits, void* workspace, size_t workspace_bytes,
              void* hip_stream);

/* The slice count fa_decode uses for num_splits = 0: enough workgroups (one
 * per key/value head and slice) for every compute unit of the chip (256), with
 * at least 16 tiles of 32 keys per slice (four per wave), never more slices than
 * tiles or than 512.  Negative fa_status for invalid shapes. */
int fa_decode_num_splits(int B, int H, int Hkv, int Nq, int Nk, int d);

/* Bytes of device workspace fa_decode needs for these shapes and num_splits
 * (0 = the default): (d + 4) float32 per query row per slice.  Returns 0 for
 * invalid shapes. */
size_t fa_decode_workspace_size(int B, int H, int Hkv, int Nq, int Nk, int d, int num_splits);

/* One kernel of fa_decode, for callers that time them separately: stage 0 = the
 * split kernel (reads Q, K, V; writes the workspace; O and LSE may be NULL), 1 =
 * the combine (reads the workspace; writes O and LSE; Q, K, V may be NULL).
 * Running 0 then 1 on one stream is exactly fa_decode.  An unknown stage is
 * FA_ERR_INVALID_ARG; otherwise errors as fa_decode. */
int fa_decode_stage(int stage, const void* Q, const void* K, const void* V, void* O,
                    float* LSE, int B, int H, int Hkv, int Nq, int Nk, int d, int causal,
                    float scale, int dtype, int num_splits, void* workspace,
                    size_t workspace_bytes, void* hip_stream);

/*
 * Tile shape of a kernel: kernel_id 0 = forward with the causal mask, 1 = dK/dV,
 * 2 = dQ, 3 = forward without the causal mask (512 query rows per tile for
 * 16-bit inputs at d = 64, else as 0).  Writes the query-tile rows (*Br) and
 * key-tile columns (*Bc) the kernel uses for this d and dtype.  Returns
 * FA_ERR_INVALID_ARG / FA_ERR_UNSUPPORTED like the kernels do.
 */
int fa_tile_config(int kernel_id, int d, int dtype, int* Br, int* Bc);

/* Static text for a status code. */
const char* fa_strerror(int status);

/* Text of the last error on the calling thread ("" if none). */
const char* fa_last_error(void);

/*
 * FP8 input stage of incoherent processing (CMU 11-868 FlashAttention notes,
 * "FlashAttention-3: asynchrony and FP8 on Hopper", slide page 24: multiply Q
 * and K by one random orthogonal Hadamard matrix before quantising, which
 * keeps QK^T and spreads outliers).  Each of the `rows` rows of X (row-major
 * [rows][d], fp16 or bf16, d = 64 or 128, e.g. a [B,H,N,d] Q or K as B*H*N rows)
 * becomes y = x J with J = diag(signs) H / sqrt(d), H the Sylvester Hadamard
 * matrix (H[i][j] = (-1)^popcount(i & j)); with signs == NULL, y = x (no
 * rotation).  Then scales[r] = max_j |y_j| / 448 (1 for an all-zero row), and
 * codes[r][j] is the E4M3 byte (bias 7, 3 mantissa bits, largest finite 448)
 * nearest to y_j / scales[r], ties to even, so y ~= code * scale.  The kernel
 * forms y_j * (448 / max_j |y_j|) in fp32 rather than dividing by the scale, so
 * where that product lies within one fp32 rounding of a midpoint between two
 * E4M3 values the code may be either neighbour.  Rows whose largest magnitude
 * is below 2^-100 are scaled up by an exact power of two first, so tiny rows
 * get finite codes; their scale is then an fp32 subnormal.
 *
 * Device pointers: X (16-byte aligned), signs (d floats, each +1 or -1, not
 * checked; 16-byte aligned) or NULL, codes ([rows][d] bytes, 8-byte aligned)
 * and scales (rows floats) written; codes and scales must not overlap X or
 * signs (not checked).  Each row is independent, so Q and K may be passed as
 * one call if they lie in one buffer.  rows = 0 launches nothing and returns
 * FA_OK (the pointers may then be NULL; dtype and d are still checked).
 * Errors, before any launch: FA_ERR_INVALID_ARG for null pointers,
 * negative or too many (>= 2^31) rows, an unknown dtype or misalignment;
 * FA_ERR_UNSUPPORTED for fp32 rows or d not 64 / 128.  Asynchronous on
 * hip_stream; nothing is allocated.
 */
int fa_fp8_quantize_rows(const void* X, long long rows, int d, int dtype, const float* signs,
                         unsigned char* codes, float* scales, void* hip_stream);

/*
 * FP8 forward pass on the output of fa_fp8_quantize_rows: Qc, Kc are the E4M3
 * codes ([B,H,N,d] bytes, 16-byte aligned) of Q J and K J, Qs, Ks their row
 * scales ([B,H,N] float32), so the scores are
 *     S_ij = scale * (Qs_i Qc_i) . (Ks_j Kc_j)     (= scale * Q_i . K_j up to the FP8 rounding,
 *                                                   since (QJ)(KJ)^T = QK^T for orthogonal J).
 * V is [B,H,N,d] in `dtype` (fp16 or bf16); O ([B,H,N,d], dtype) and LSE
 * ([B,H,N] float32) are as fa_forward's: the softmax, the causal mask (key j
 * visible to query i iff j <= i), the online rescaling, the rounding of the
 * probabilities to dtype before P V and the stored log-sum-exp follow
 * fa_forward; only Q K^T runs on FP8 (E4M3 x E4M3 products, fp32 accumulation).
 * Multi-head only (K and V have H heads).  Device pointers owned by the
 * caller; nothing is allocated; asynchronous on hip_stream.
 * Errors, before any launch: FA_ERR_INVALID_ARG for null pointers, B/H/N <= 0,
 * an unknown dtype, a non-finite scale or misalignment (codes, V, O 16 bytes;
 * scales and LSE 4 bytes); FA_ERR_UNSUPPORTED for fp32, d not 64 / 128,
 * scale <= 0, or N * d >= 2^30.
 * Defined by: CMU 11-868 FlashAttention notes, "FlashAttention-3: asynchrony
 * and FP8 on Hopper", slide page 24 (Q K^T in FP8 after one random orthogonal
 * Hadamard matrix multiplies Q and K) and pages 47-49 (the FP8 forward); the
 * rest as fa_forward.
 */
int fa_forward_fp8(const void* Qc, const float* Qs, const void* Kc, const float* Ks,
                   const void* V, void* O, float* LSE, int B, int H, int N, int d, int causal,
                   float scale, int dtype, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
