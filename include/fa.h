/*
 * fa.h - C ABI of the gfx950 exact tiled attention library (libfa.so).
 *
 * The operation is exact scaled-dot-product attention,
 *     O = softmax(scale * Q K^T) V,
 * the formula of "Flash Attention: بهینه‌سازی مکانیزم توجه در ترنسفورمرها"
 * (deepfa.ir), section on the structure of the attention mechanism, computed
 * tile by tile with a running row maximum and row sum so that the N x N
 * score matrix is never written to memory ("Flash Attention: Rivoluzionando
 * l'Efficienza dei Modelli Transformer" (unite.ai), sections "L'Algoritmo di
 * Flash Attention" and "La Matematica dietro Flash Attention"). The backward
 * pass recomputes the probabilities from a stored per-row logsumexp instead
 * of storing them (deepfa.ir page, recomputation technique).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are DEVICE pointers owned by the caller, laid out [B, H, N, d]
 *   contiguous row-major (d innermost), one head after another. Row vectors
 *   (lse, the backward workspace) are fp32 [B, H, N].
 * - bf16 tensors are passed as void* to 16-bit storage (bfloat16 bit
 *   patterns). All tensor pointers must be 16-byte aligned.
 * - Heads are independent; query i sees key j iff causal == 0 or j <= i
 *   (equal query and key lengths, lower-triangular mask).
 * - scale is any finite float (callers normally pass 1/sqrt(d)).
 * - Supported head dims: d in {64, 128}. N >= 0, B >= 0, H >= 0, any N
 *   (a multiple of 128 is the fast case). If B, H or N is 0 the call does
 *   nothing and returns FA_OK; null pointers are then accepted.
 * - Calls are asynchronous: they enqueue kernels on `stream` (NULL means the
 *   null stream) and return. The library never allocates, frees or
 *   synchronises and keeps no mutable global state, so it is reentrant.
 * - Errors: invalid arguments are reported by a nonzero status BEFORE any
 *   HIP call, and nothing is written. A launch failure returns FA_ERR_HIP.
 *   Device faults surface at the caller's next synchronisation.
 * - Sizes: B*H*N*d may exceed 2^31 elements (64-bit offsets between
 *   heads); within one head N*d*4 must be below 2^31 (N < 4194304 at
 *   d = 128), and B*H*ceil(N/128) below 2^31. Otherwise FA_ERR_SHAPE.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,      /* a required pointer is NULL */
    FA_ERR_SHAPE = 2,     /* B, H or N negative, or the grid would overflow */
    FA_ERR_HEADDIM = 3,   /* d not in {64, 128} */
    FA_ERR_ALIGN = 4,     /* a tensor pointer is not 16-byte aligned */
    FA_ERR_ARG = 5,       /* causal not 0/1, or scale not finite */
    FA_ERR_WORKSPACE = 6, /* backward workspace missing or too small */
    FA_ERR_HIP = 7        /* the HIP runtime reported an error at launch */
} fa_status;

/*
 * Forward pass, bf16 in / bf16 out.
 *   q, k, v : [B,H,N,d] bf16 inputs.
 *   o       : [B,H,N,d] bf16 output, O = softmax(scale Q K^T) V, rounded to
 *             nearest even from an fp32 accumulator.
 *   lse     : [B,H,N] fp32 output, lse_i = ln sum_{visible j} exp(scale q_i.k_j)
 *             (natural log of the scaled scores).
 * Arithmetic: bf16 MFMA products with fp32 accumulation; the probabilities
 * are rounded to bf16 before the product with V; row max, row sum and lse
 * are fp32.
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal,
               hipStream_t stream);

/*
 * Forward pass with fp32 inputs and an fp32 output. q, k, v are rounded to
 * bf16 (nearest even) as they are loaded, then follow the fa_forward path;
 * o receives the fp32 result before any output rounding. Arguments and
 * errors as for fa_forward.
 */
int fa_forward_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal,
                   hipStream_t stream);

/*
 * Bytes of device workspace fa_backward needs: 2*B*H*N*sizeof(float), for
 * the row terms D_i = sum_k dO_ik O_ik followed by lse_i * log2(e), each
 * [B,H,N] fp32. Returns 0 for empty or invalid shapes.
 */
size_t fa_backward_workspace_size(int B, int H, int N, int d);

/*
 * Backward pass: gradients of sum(dout * O) with respect to q, k and v,
 * O = softmax(scale Q K^T) V. The probabilities are recomputed from lse; no
 * N x N matrix is stored (deepfa.ir page, recomputation technique). The
 * pages print no backward equations; the ones used are the derivative of
 * the forward definition: with P the softmax, D_i = sum_k dout_ik O_ik,
 * dS = P * (dout V^T - D), dq = scale dS K, dk = scale dS^T Q, dv = P^T dout.
 *   q, k, v, o, dout : [B,H,N,d] bf16 inputs; o and lse are the outputs of
 *                      fa_forward on the same q, k, v, scale and causal.
 *   lse              : [B,H,N] fp32 input.
 *   dq, dk, dv       : [B,H,N,d] bf16 outputs, overwritten (not accumulated);
 *                      fp32 accumulation, rounded to nearest even once.
 *   workspace        : device buffer of at least
 *                      fa_backward_workspace_size(B,H,N,d) bytes, 16-byte
 *                      aligned; contents ignored on entry, holds the row
 *                      terms of fa_backward_prep on return.
 * Equivalent to fa_backward_prep followed by fa_backward_grads on the same
 * stream. Every output element is written by exactly one workgroup: dk and
 * dv by a pass over key blocks, dq by a pass over query-row blocks, with no
 * atomics, so results are bitwise reproducible.
 */
int fa_backward(const void* q, const void* k, const void* v, const void* o,
                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                int B, int H, int N, int d, float scale, int causal,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * First stage of fa_backward: for every row, D_i = sum_k dout_ik O_ik and
 * lse_i * log2(e), into the workspace (the first and second [B,H,N] fp32
 * halves). o, dout and lse as for fa_backward. Errors as for fa_backward
 * (scale and causal are not arguments here).
 */
int fa_backward_prep(const void* o, const void* dout, const float* lse, int B, int H, int N,
                     int d, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Second stage of fa_backward: dq, dk, dv from q, k, v, dout and the row
 * terms fa_backward_prep left in `workspace` (read only here; lse enters
 * through them). `lse` must still be a valid pointer. Arguments, layouts and
 * errors as for fa_backward.
 */
int fa_backward_grads(const void* q, const void* k, const void* v, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv,
                      int B, int H, int N, int d, float scale, int causal,
                      const void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
