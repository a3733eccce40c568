/*
 * fa2.h -- C ABI of the gfx950 (MI355X) exact-attention library libfa2.so.
 *
 * The library computes exact attention the FlashAttention-2 way: the forward
 * pass tiles the query rows across workgroups, streams K/V tiles through LDS
 * and keeps an online softmax with a deferred rescale of an unnormalized fp32
 * accumulator, emitting the per-row logsumexp L = m + log(l); the backward
 * pass rebuilds P = exp(S - L) from L and produces dK, dV looping over K/V
 * tiles on the outside, and dQ either in a separate pass over query tiles
 * (default) or with fp32 atomics inside the K/V loop.
 * (FlashAttention-2 summary page, zhaifeiyue.github.io: section 2 "Q2
 * method" -- deferred rescaling, logsumexp, sequence parallelism, split-Q;
 * section 3 "Target operation" -- O = softmax(QK^T)V, optional causal mask,
 * FP16/BF16 inputs with an FP32 accumulator; section 4 symbol table -- L and
 * D = rowsum(dO o O); section 4 checks -- GQA/MQA by shared K/V heads with
 * dK/dV summed over the sharing heads; section 7 -- dQ accumulated with
 * atomic adds.  Head dimensions up to 256 and MQA/GQA: ai.oldpan.me, "New
 * features".)
 *
 * Definition computed, per batch b and query head hq, with key/value head
 * hk = hq / (Hq / Hkv):
 *     S = scale * Q K^T,   S_ij = -inf for j > i when causal,
 *     L_i = ln sum_j exp(S_ij),   P = exp(S - L),   O = P V,
 *     dV = P^T dO,  dP = dO V^T,  D = rowsum(dO o O),  dS = P o (dP - D),
 *     dQ = scale * dS K,  dK = scale * dS^T Q   (dK, dV summed over the
 *     query heads that share a key/value head).
 *
 * Data layout (all tensors contiguous, row-major, device memory):
 *     Q, O, dO, dQ : bf16 [B, Hq,  N, d]     (bf16 = raw 16-bit storage)
 *     K, V, dK, dV : bf16 [B, Hkv, N, d]
 *     L            : fp32 [B, Hq,  N]        natural-log logsumexp of the
 *                                             scaled, masked scores
 * Every device pointer must be 16-byte aligned.  Query and key sequence
 * lengths are equal (N).  d must be 64, 128 or 256.  Hq must be a multiple
 * of Hkv.  scale must be finite and > 0 (typically 1/sqrt(d)).  Rounding to
 * bf16 is round-to-nearest-even.
 *
 * Ownership: the caller owns every buffer; the library keeps no pointer
 * after a call returns and allocates no device memory.  Outputs are fully
 * overwritten (no zeroing needed).  Inputs are never written.  An output may
 * not alias an input.
 *
 * Streams and errors: `stream` is a hipStream_t passed as void* (NULL = the
 * default stream).  Calls are asynchronous: argument errors are reported
 * before anything is launched (nothing is written then); a launch failure
 * returns FA2_ERR_HIP; a fault inside a kernel surfaces at the caller's next
 * synchronization with the stream, not as a return value.  The library is
 * thread-safe (no mutable global state beyond a per-thread error message and
 * the per-device address of fa2_bwd_noalloc's static scratch).
 *
 * Determinism: the forward pass and fa2_bwd are bitwise reproducible.  The
 * optional atomic-dQ mode of fa2_bwd_stages sums dQ with fp32 atomics and is
 * reproducible only up to the order of those additions.
 */
#ifndef FA2_H
#define FA2_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa2_status {
    FA2_OK = 0,
    FA2_ERR_INVALID_ARGUMENT = 1, /* null/misaligned/aliased pointer, bad size or scale */
    FA2_ERR_UNSUPPORTED = 2,      /* valid request this library does not implement (d) */
    FA2_ERR_HIP = 3               /* the HIP runtime rejected a launch */
} fa2_status;

/*
 * Forward pass: O = softmax(scale * Q K^T [+ causal mask]) V and L.
 *   Q [B,Hq,N,d], K/V [B,Hkv,N,d] bf16 inputs; O [B,Hq,N,d] bf16 and
 *   L [B,Hq,N] fp32 outputs.  causal != 0 masks keys j > i.
 * Any of B, Hq, N equal to 0 is an empty problem: FA2_OK, nothing launched
 * (pointers may then be NULL).
 * Errors: FA2_ERR_INVALID_ARGUMENT for a negative size, Hkv < 1 with work,
 * Hq % Hkv != 0, a NULL or non-16-byte-aligned pointer, O or L aliasing an
 * input, O aliasing L, a non-finite or non-positive scale, or sizes whose
 * element counts overflow 64 bits; FA2_ERR_UNSUPPORTED for d not in
 * {64, 128, 256}; FA2_ERR_HIP if the launch fails.
 */
fa2_status fa2_fwd(const void *Q, const void *K, const void *V, void *O, float *L,
                   int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                   void *stream);

/*
 * Bytes of device workspace fa2_bwd needs: two fp32 [B,Hq,Npad] arrays
 * (Npad = N rounded up to a multiple of 64) holding -D = -rowsum(dO o O) and
 * L * log2(e) per query row, each starting on a 256-byte boundary.  Returns 0
 * for an empty problem and for sizes fa2_bwd rejects (negative, Hq % Hkv != 0,
 * N above 2^30, byte counts that overflow).
 */
size_t fa2_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d);

/*
 * Bytes of device workspace fa2_bwd_stages / fa2_bwd_stages_f16 need for a
 * given stage mask (the bits below): those of fa2_bwd_workspace_bytes, plus,
 * when FA2_BWD_DQ_ATOMIC is set, an fp32 [B,Hq,N,d] dQ accumulator on a
 * 256-byte boundary after them.  0 for an invalid mask or as above.
 */
size_t fa2_bwd_stages_workspace_bytes(unsigned stages, int B, int Hq, int Hkv, int N, int d);

/*
 * Backward pass: dQ, dK, dV of sum(dO o O) for the forward defined above.
 *   Q, K, V: the forward's inputs; O [B,Hq,N,d] bf16 and L [B,Hq,N] fp32:
 *   the forward's outputs (P is rebuilt from L); dO [B,Hq,N,d] bf16.
 *   dQ [B,Hq,N,d], dK and dV [B,Hkv,N,d]: bf16 outputs (for GQA, dK/dV are
 *   summed over the Hq/Hkv query heads sharing each key/value head).
 *   workspace: caller-allocated device memory, 256-byte aligned, of at least
 *   fa2_bwd_workspace_bytes(...) bytes; contents undefined on entry and exit.
 * Errors: as fa2_fwd, plus FA2_ERR_INVALID_ARGUMENT when the workspace is
 * NULL, misaligned or too small, or when an output aliases an input or
 * another output.
 */
fa2_status fa2_bwd(const void *Q, const void *K, const void *V, const void *O,
                   const float *L, const void *dO, void *dQ, void *dK, void *dV,
                   void *workspace, size_t workspace_bytes,
                   int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                   void *stream);

/*
 * The backward pass as its three launches, selected by a bit mask, with the
 * same arguments and checks as fa2_bwd:
 *   FA2_BWD_PREPROCESS  D = rowsum(dO o O) (section 4 symbol table of the
 *                       FlashAttention-2 summary page) and L * log2(e)
 *                       into the workspace;
 *   FA2_BWD_MAIN        the loop over K/V tiles that writes dK and dV
 *                       (same page, section 2: the backward's outer loop runs
 *                       over K/V column blocks);
 *   FA2_BWD_FINALIZE    dQ.
 * By default dQ has its own pass (one workgroup per query tile summing the
 * contributions of all K/V tiles in registers; S and dP are recomputed),
 * which is deterministic and, on this GPU, faster than the alternative.
 * With FA2_BWD_DQ_ATOMIC also set -- the pages' design (same page, section
 * 7) -- the K/V loop adds every tile's dQ contribution into an fp32
 * accumulator in the workspace with atomic adds (PREPROCESS zeroes it,
 * FINALIZE converts it to bf16); dQ is then reproducible only up to the
 * order of those additions, and the workspace must hold
 * fa2_bwd_stages_workspace_bytes(mask, ...) bytes.  The mode bit must be the
 * same in every call of one backward pass.
 * Running the three stages in order on one stream, with the same workspace
 * untouched in between, is exactly fa2_bwd (mask FA2_BWD_ALL) or its atomic
 * variant (FA2_BWD_ALL | FA2_BWD_DQ_ATOMIC).  Stages may be issued by
 * separate calls, e.g. to time or overlap them.  A mask without any stage
 * bit, or with bits other than these four, is FA2_ERR_INVALID_ARGUMENT.
 */
#define FA2_BWD_PREPROCESS 1u
#define FA2_BWD_MAIN 2u
#define FA2_BWD_FINALIZE 4u
#define FA2_BWD_ALL 7u
#define FA2_BWD_DQ_ATOMIC 8u
fa2_status fa2_bwd_stages(unsigned stages, const void *Q, const void *K, const void *V,
                          const void *O, const float *L, const void *dO, void *dQ, void *dK,
                          void *dV, void *workspace, size_t workspace_bytes, int B, int Hq,
                          int Hkv, int N, int d, int causal, float scale, void *stream);

/*
 * fa2_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments (minus the workspace), layouts,
 * checks, kernels, results (bitwise those of fa2_bwd) and errors as fa2_bwd.
 * The per-row scratch (-D and L * log2(e), 8 bytes per query row, rows padded
 * to 64 per head) lives in a static device array of FA2_NOALLOC_SCRATCH_BYTES
 * bytes that each GPU holds until the process ends; its address is looked up
 * on the first call made with that device current (the device the stream
 * belongs to).  The call allocates nothing.  A problem needing more than the
 * array (B * Hq * round_up(N, 64) above FA2_NOALLOC_SCRATCH_BYTES / 8 rows)
 * returns FA2_ERR_UNSUPPORTED before any HIP call.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (two streams,
 * or two threads) race on it and must be ordered by the caller.  The array
 * needs no clearing between calls: each call writes every entry it reads.
 */
#define FA2_NOALLOC_SCRATCH_BYTES (16u << 20)
fa2_status fa2_bwd_noalloc(const void *Q, const void *K, const void *V, const void *O,
                           const float *L, const void *dO, void *dQ, void *dK, void *dV,
                           int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                           void *stream);

/*
 * FP16 inputs and outputs (the pages' problem statement allows FP16 or BF16).
 * Same arguments, layouts, workspace, checks, errors and determinism as
 * fa2_fwd / fa2_bwd / fa2_bwd_stages, with Q, K, V, O, dO, dQ, dK and dV
 * holding IEEE binary16 values (L stays fp32).  The same kernels run with f16
 * matrix products, fp32 accumulation and round-to-nearest-even f16 outputs.
 */
fa2_status fa2_fwd_f16(const void *Q, const void *K, const void *V, void *O, float *L,
                       int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                       void *stream);
fa2_status fa2_bwd_f16(const void *Q, const void *K, const void *V, const void *O,
                       const float *L, const void *dO, void *dQ, void *dK, void *dV,
                       void *workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                       int N, int d, int causal, float scale, void *stream);
fa2_status fa2_bwd_stages_f16(unsigned stages, const void *Q, const void *K, const void *V,
                              const void *O, const float *L, const void *dO, void *dQ,
                              void *dK, void *dV, void *workspace, size_t workspace_bytes,
                              int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                              void *stream);

/*
 * Split O: the forward's output carried to the backward at about 16
 * significant bits instead of bf16's 8 (bf16 only, dense attention).
 * The backward's D = rowsum(dO o O) (section 4 symbol table of the
 * FlashAttention-2 summary page) is formed from the O it is given; from a
 * bf16 O it inherits O's rounding, which moves dS = P o (dP - D) by
 * P * dD on every key a row attends to and, summed over many rows, dK by
 * more than the rounding of the products themselves.
 *   fa2_fwd_olo: fa2_fwd that also writes O_lo [B,Hq,N,d] bf16, the
 *     rounding residual of each output element, bf16(x - O) with x the fp32
 *     value before its rounding to O (|O_lo| is at most half an ulp of O).
 *     O and L are bitwise those of fa2_fwd.
 *   fa2_bwd_olo / fa2_bwd_stages_olo: fa2_bwd / fa2_bwd_stages with
 *     D = rowsum(dO o (O + O_lo)) (only FA2_BWD_PREPROCESS reads O_lo).
 * O_lo must be a device buffer like O (16-byte aligned, [B,Hq,N,d] bf16),
 * owned by the caller.  Errors: as fa2_fwd / fa2_bwd, plus
 * FA2_ERR_INVALID_ARGUMENT when O_lo is NULL or misaligned, overlaps Q, K
 * or V, in the forward overlaps O or L, or in the backward overlaps an
 * output or the workspace.
 */
fa2_status fa2_fwd_olo(const void *Q, const void *K, const void *V, void *O, void *O_lo,
                       float *L, int B, int Hq, int Hkv, int N, int d, int causal, float scale,
                       void *stream);
fa2_status fa2_bwd_olo(const void *Q, const void *K, const void *V, const void *O,
                       const void *O_lo, const float *L, const void *dO, void *dQ, void *dK,
                       void *dV, void *workspace, size_t workspace_bytes, int B, int Hq,
                       int Hkv, int N, int d, int causal, float scale, void *stream);
fa2_status fa2_bwd_stages_olo(unsigned stages, const void *Q, const void *K, const void *V,
                              const void *O, const void *O_lo, const float *L, const void *dO,
                              void *dQ, void *dK, void *dV, void *workspace,
                              size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d,
                              int causal, float scale, void *stream);

/*
 * Block-sparse attention (FlashAttention paper page, aipaper.jasonlin.tech,
 * key contributions: the exact kernel restricted to a predefined block
 * sparsity pattern, skipping the blocks the pattern leaves out; limitations:
 * the pattern is fixed in advance).
 *   block_mask: device memory, FA2_SPARSE_BLOCK x FA2_SPARSE_BLOCK blocks,
 *   unsigned bytes [nb, nb] with nb = ceil(N / 128), row-major by query
 *   block, shared by every batch and head, any alignment.  A zero byte at
 *   (r, c) masks the scores of query rows 128r..128r+127 against keys
 *   128c..128c+127 (set to -inf before the softmax, as the causal mask does;
 *   both apply when causal != 0).  Masked blocks cost no matrix products:
 *   every kernel's workgroup covers one mask row (forward, dQ pass) or one
 *   mask column (the backward's K/V-tile loop) and walks only the blocks it
 *   keeps.
 *   A query row with no unmasked score gets O = 0 and L = -inf; its dQ is 0
 *   and it adds nothing to dK or dV.
 * Same layouts, workspace, outputs and errors as fa2_fwd / fa2_bwd, for every
 * head dim (64, 128, 256), plus FA2_ERR_INVALID_ARGUMENT for a NULL block_mask
 * (with work) or an output overlapping it, and FA2_ERR_UNSUPPORTED for N above
 * FA2_SPARSE_MAX_N.  fa2_bwd_block_sparse takes the forward's O and L of the
 * same mask; it always computes dQ in its own pass (bitwise reproducible).
 * The _f16 variants take IEEE binary16 tensors, as fa2_fwd_f16 / fa2_bwd_f16.
 */
#define FA2_SPARSE_BLOCK 128
#define FA2_SPARSE_MAX_N 262144
fa2_status fa2_fwd_block_sparse(const void *Q, const void *K, const void *V, void *O, float *L,
                                const unsigned char *block_mask, int B, int Hq, int Hkv, int N,
                                int d, int causal, float scale, void *stream);
fa2_status fa2_bwd_block_sparse(const void *Q, const void *K, const void *V, const void *O,
                                const float *L, const void *dO, void *dQ, void *dK, void *dV,
                                const unsigned char *block_mask, void *workspace,
                                size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d,
                                int causal, float scale, void *stream);
fa2_status fa2_fwd_block_sparse_f16(const void *Q, const void *K, const void *V, void *O, float *L,
                                    const unsigned char *block_mask, int B, int Hq, int Hkv, int N,
                                    int d, int causal, float scale, void *stream);
fa2_status fa2_bwd_block_sparse_f16(const void *Q, const void *K, const void *V, const void *O,
                                    const float *L, const void *dO, void *dQ, void *dK, void *dV,
                                    const unsigned char *block_mask, void *workspace,
                                    size_t workspace_bytes, int B, int Hq, int Hkv, int N, int d,
                                    int causal, float scale, void *stream);

/*
 * The argument checks of fa2_fwd / fa2_bwd alone: no HIP call is made, so
 * they run without a GPU.  Same return codes as the full calls.
 */
fa2_status fa2_validate_fwd(const void *Q, const void *K, const void *V, const void *O,
                            const float *L, int B, int Hq, int Hkv, int N, int d,
                            int causal, float scale);
fa2_status fa2_validate_bwd(const void *Q, const void *K, const void *V, const void *O,
                            const float *L, const void *dO, const void *dQ,
                            const void *dK, const void *dV, const void *workspace,
                            size_t workspace_bytes, int B, int Hq, int Hkv, int N,
                            int d, int causal, float scale);

/* Static, human-readable name of a status code: any int, so that a value that
 * is not an fa2_status (e.g. from a newer library) gives "unknown status". */
const char *fa2_status_string(int status);

/*
 * Detail of the last non-OK status returned on the calling thread (which
 * check failed, or the HIP error string); "" if none.  Valid until the next
 * call on the same thread.
 */
const char *fa2_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */
