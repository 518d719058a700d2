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
 * - Supported head dims: d in {64, 128, 256} (the FP8 calls: {64, 128}).
 *   N >= 0, B >= 0, H >= 0, any N
 *   (a multiple of 128 is the fast case). If B, H or N is 0 the call does
 *   nothing and returns FA_OK; null pointers are then accepted.
 * - Calls are asynchronous: they enqueue kernels on `stream` (NULL means the
 *   null stream) and return. The library never allocates, frees or
 *   synchronises and keeps no mutable global state, so it is reentrant
 *   (fa_backward_noalloc alone shares one static scratch array per GPU
 *   between its calls, see there).
 *   A call only launches kernels (no allocation, no memset), so it can be
 *   captured into a HIP graph on `stream` and replayed; a replay reads the
 *   buffers' contents at replay time. The FP8 sign vector, read from host
 *   memory during the call, is fixed at capture.
 * - Errors: invalid arguments are reported by a nonzero status BEFORE any
 *   HIP call, and nothing is written. A launch failure returns FA_ERR_HIP.
 *   Device faults surface at the caller's next synchronisation.
 * - Sizes: B*H*N*d may exceed 2^31 elements (64-bit offsets between
 *   heads); within one head N*d*4 must be below 2^31 (N < 4194304 at
 *   d = 128, N < 2097152 at d = 256), and B*H*ceil(N/128) below 2^31.
 *   Otherwise FA_ERR_SHAPE.
 * - Head dim 256 (the nearauto.com FlashAttention-2 article, section
 *   "新機能", lists head dimensions up to 256 among FlashAttention-2's
 *   additions) uses the same arithmetic and results as 64 and 128, with
 *   workgroups of one wave per SIMD (a wave's accumulators need the whole
 *   register file).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,      /* a required pointer is NULL */
    FA_ERR_SHAPE = 2,     /* B, H or N negative, K/V heads not dividing H, or too large */
    FA_ERR_HEADDIM = 3,   /* d not in {64, 128, 256} ({64, 128} for the FP8 calls) */
    FA_ERR_ALIGN = 4,     /* a tensor pointer is not 16-byte aligned */
    FA_ERR_ARG = 5,       /* causal not 0/1, a window bound below -1, scale not finite,
                             an FP8 sign not +1/-1, or a negative block-mask head stride */
    FA_ERR_WORKSPACE = 6, /* workspace missing, misaligned or too small */
    FA_ERR_HIP = 7,       /* the HIP runtime reported an error at launch */
    FA_ERR_SCRATCH = 8    /* fa_backward_noalloc: B*H*N above its static scratch (2097152) */
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
 * fa_backward without the workspace arguments, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The row terms go to a static scratch
 * array inside the library instead: 16 MiB on each GPU the library runs on,
 * taken when the library is loaded and held until the process ends, enough
 * for B*H*N <= 2097152 rows; larger problems return FA_ERR_SCRATCH before any
 * HIP call. The call allocates nothing; on its first use on a device it looks
 * up that device's address of the array (the device current at the call,
 * which `stream` must belong to). Results are bitwise those of fa_backward.
 * Every call on one GPU uses the same array, and the row-term launch
 * rewrites every row the gradient launch reads, so nothing needs clearing
 * between calls; but calls whose kernels can overlap on one GPU (on
 * different streams, from different threads, graph replays in flight) race
 * on it and must be ordered by the caller. Arguments and other errors as
 * for fa_backward.
 */
int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        int B, int H, int N, int d, float scale, int causal,
                        hipStream_t stream);

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

/*
 * Grouped-query and multi-query attention (nearauto.com FlashAttention-2
 * article, section "新機能": each set of query heads shares a single key
 * and value head, between multi-head and multi-query attention). H query
 * heads share H_kv key/value heads: query head h reads K/V head
 * h / (H / H_kv), i.e. consecutive groups of H / H_kv query heads share one
 * K/V head (the page does not say which heads form a set; this is the plain
 * reading). H_kv = H is multi-head attention, H_kv = 1 multi-query
 * attention. H_kv < 1, or H_kv not dividing H, returns FA_ERR_SHAPE (when
 * H > 0); everything else as for the calls without _gqa.
 *
 * fa_forward_gqa: q, o [B,H,N,d]; k, v [B,H_kv,N,d]; lse [B,H,N].
 */
int fa_forward_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int H_kv, int N, int d, float scale, int causal,
                   hipStream_t stream);

/*
 * fa_backward_gqa: q, o, dout, dq [B,H,N,d]; k, v, dk, dv [B,H_kv,N,d];
 * lse [B,H,N]; workspace of fa_backward_workspace_size(B,H,N,d) bytes (the
 * row terms are per query row). dk and dv of a K/V head are the sums of the
 * gradients of its query heads (the chain rule for a shared input), formed
 * inside one workgroup per K/V head and key block, with no atomics: results
 * stay bitwise reproducible. fa_backward_prep (per query head, unchanged)
 * followed by fa_backward_grads_gqa is equivalent.
 */
int fa_backward_gqa(const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    int B, int H, int H_kv, int N, int d, float scale, int causal,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

int fa_backward_grads_gqa(const void* q, const void* k, const void* v, const void* dout,
                          const float* lse, void* dq, void* dk, void* dv,
                          int B, int H, int H_kv, int N, int d, float scale, int causal,
                          const void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Local (sliding-window) attention: the pages name local attention only as a
 * coming variant (nearauto.com FlashAttention-2 article, section
 * "今後の仕事"; aiunderstanding.org, "Il futuro dell'attenzione flash").
 * The mask used generalises the causal one: key j is visible to query i iff
 *     (window_left  < 0 or j >= i - window_left) and
 *     (window_right < 0 or j <= i + window_right),
 * -1 meaning no bound on that side. (-1, 0) is the causal mask, (-1, -1) no
 * mask, (W-1, 0) a causal window of W keys. Bounds below -1 return
 * FA_ERR_ARG. A bound of N-1 or more cuts no key and is the same mask as
 * -1 (any int is accepted, INT_MAX included; the results are bitwise those
 * of -1). Every row sees at least its own key whenever both bounds are
 * >= 0, and key 0 or key N-1 otherwise, so no row is empty. Query tiles and
 * key tiles that no visible pair touches are skipped, like the tiles above
 * the diagonal under the causal mask.
 *
 * These calls take the grouped K/V heads of the _gqa calls (H_kv = H:
 * multi-head attention) and otherwise behave as them.
 */
int fa_forward_window(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int H_kv, int N, int d, float scale, int window_left,
                      int window_right, hipStream_t stream);

int fa_backward_window(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       int B, int H, int H_kv, int N, int d, float scale, int window_left,
                       int window_right, void* workspace, size_t workspace_bytes,
                       hipStream_t stream);

int fa_backward_grads_window(const void* q, const void* k, const void* v, const void* dout,
                             const float* lse, void* dq, void* dk, void* dv,
                             int B, int H, int H_kv, int N, int d, float scale, int window_left,
                             int window_right, const void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * Block-sparse attention. The nearauto.com FlashAttention-2 article names
 * block-sparse attention only as coming work (section "今後の仕事"); the
 * library reads it as a mask over blocks of 128 query rows x 128 keys:
 *   block_mask : DEVICE bytes, for query head (b, h) at
 *                block_mask + (b*H + h) * block_mask_head_stride, an
 *                nb x nb row-major array, nb = ceil(N / 128): byte (I, J)
 *                covers query rows 128I .. 128I+127 and keys 128J ..
 *                128J+127. Zero: every key of block J is masked for every
 *                row of block I; nonzero: the block is computed under the
 *                window mask of window_left, window_right (as the _window
 *                calls; -1, -1 for none, -1, 0 for causal).
 *   block_mask_head_stride : bytes between the masks of consecutive query
 *                heads, >= 0; 0 shares one mask among all heads. The caller
 *                keeps (B*H - 1) * stride + nb*nb bytes readable. Grouped
 *                K/V heads (H_kv < H) keep a mask per query head.
 * A row that sees no key at all (its blocks all zero, or its window keys
 * all in zero blocks) gets O = 0 and lse = -inf, and contributes nothing to
 * dq, dk, dv; its own dq row is 0. Zero blocks are neither loaded nor
 * computed: the work follows the number of nonzero blocks.
 * Inputs are bf16 as in fa_forward_window / fa_backward_window, whose
 * argument rules, workspace and results these calls share; a NULL
 * block_mask returns FA_ERR_NULL (checked after the tensor pointers), a
 * negative stride, or one so large that (B*H - 1) * stride + nb*nb
 * overflows 64 bits, FA_ERR_ARG. The mask takes no alignment. The backward
 * calls take the lse of the forward call with the same mask.
 */
int fa_forward_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int H_kv, int N, int d, float scale, int window_left,
                            int window_right, const uint8_t* block_mask,
                            long long block_mask_head_stride, hipStream_t stream);

int fa_backward_block_sparse(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             int B, int H, int H_kv, int N, int d, float scale, int window_left,
                             int window_right, const uint8_t* block_mask,
                             long long block_mask_head_stride, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

int fa_backward_grads_block_sparse(const void* q, const void* k, const void* v,
                                   const void* dout, const float* lse, void* dq, void* dk,
                                   void* dv, int B, int H, int H_kv, int N, int d, float scale,
                                   int window_left, int window_right, const uint8_t* block_mask,
                                   long long block_mask_head_stride, const void* workspace,
                                   size_t workspace_bytes, hipStream_t stream);

/*
 * FP8 forward with incoherent processing. The pages describe FlashAttention-3
 * computing in FP8 and multiplying Q and K by a Hadamard transform with
 * random signs, which spreads outliers over the channels and lowers the
 * quantisation error ("Flash Attention: بهینه‌سازی مکانیزم توجه در
 * ترنسفورمرها" (deepfa.ir), FlashAttention 3, section "پردازش ناهمدوس برای
 * FP8"; unite.ai FlashAttention page, section on FlashAttention-3, items 2
 * and 3). They give no formulas; the readings implemented:
 *   - M = diag(s) H, s the caller's random signs, H the d x d Sylvester
 *     Hadamard matrix (H H^T = d I); Q~ = Q M, K~ = K M, so that
 *     Q~ K~^T / d = Q K^T. signs == NULL: no rotation (plain FP8).
 *   - FP8 is OCP e4m3 (largest finite 448, subnormals), rounded to nearest
 *     even. Scales are powers of two: a_i per query row of Q~, b_t per tile
 *     of 64 keys of K~, s_{g,c} per column c and block g of 32 keys of V
 *     (not rotated); each the smallest 2^e with max|x| <= 448 * 2^e
 *     (1 for an all-zero set), and the codes are e4m3(x / scale).
 *   - S_ij = scale * a_i b_t(j) (q8_i . k8_j) / d (without the / d when not
 *     rotated); the mask and lse follow S exactly as in fa_forward.
 *   - O_i = sum_j P~_ij s_{g(j),c} v8_jc / sum_j P_ij with the probabilities
 *     taken relative to the row maximum rounded up to a whole power of two,
 *     P_ij = 2^(log2(e) S_ij - m_i), m_i = ceil(log2(e) max_j S_ij), so
 *     P_ij lies in (0, 1], and rounded with the power-of-two scale 2^-8:
 *     P~_ij = 2^-8 e4m3(2^8 P_ij) (the tile-by-tile kernel rounds P against
 *     its running reference, which may sit up to 2^2 above m_i and then
 *     differs from this only below P = 2^-12, by at most 2^-16); the row sum
 *     uses the unrounded P. These quantisation choices (scale sets, the
 *     power-of-two reference, the 2^-8 scale) are this library's design, not
 *     something the pages specify.
 * Arithmetic: Q~ and K~ in fp32 (butterflies), both products on the fp8
 * MFMA with fp32 accumulation, softmax in fp32; o is bf16 (nearest even),
 * lse fp32. Inputs must be finite (a NaN or infinity is not propagated).
 * Block scales of V below 2^-127 (block maxima below about 2^-118) are
 * raised to 2^-127.
 *
 *   q : [B,H,N,d] bf16; k, v : [B,H_kv,N,d] bf16 (H_kv divides H, as in the
 *       _gqa calls); o : [B,H,N,d] bf16 output; lse : [B,H,N] fp32 output.
 *   signs : HOST pointer to d values, each +1 or -1 (anything else:
 *       FA_ERR_ARG), or NULL. Read during the call only.
 *   causal : 0 or 1, as in fa_forward.
 *   workspace : device buffer, 16-byte aligned, of at least
 *       fa_forward_fp8_workspace_size(B,H,H_kv,N,d) bytes (FA_ERR_WORKSPACE
 *       otherwise); overwritten.
 * fa_forward_fp8 = fa_fp8_prepare (rotation and quantisation into the
 * workspace) followed by fa_forward_fp8_prepared (the attention) on the same
 * stream; the two stages can also be called separately, e.g. to reuse the
 * quantised K and V for several calls (prepare quantises Q too).
 *
 * Workspace layout (byte offsets, every region starting on a multiple of 256
 * bytes, in this order; T = ceil(N / 64), e4m3 codes as bytes):
 *   q8 : [B,H,N,d] codes of Q~ / a_i, row-major;
 *   qs : [B,H,N] fp32 row factors, a_i / d (a_i without rotation);
 *   k8 : [B,H_kv,T] tiles of 64*d bytes: the code of key 64t+r, column c at
 *        r*d + 16*((c/16) ^ sk(r)) + c%16, with sk(r) = ((r>>1)&3)|((r>>2)&4)
 *        for d = 128 and ((r>>2)&1)|((r>>3)&2) for d = 64 (keys past N: 0);
 *   ks : [B,H_kv,T] fp32 tile scales b_t;
 *   v8 : [B,H_kv,T] tiles of 64*d bytes holding V^T: the code of key 64t+j,
 *        column c at c*64 + 16*((j/16) ^ ((c>>2)&3)) + j%16 (keys past N: 0);
 *   vs : [B,H_kv,T] blocks of 256 bytes: the scale of column c, keys
 *        64t+32g .. +31 as the byte 127 + e (scale 2^e) at 4*(32g + c%32) + c/32
 *        (for d = 64 the bytes with c/32 >= 2 are unused).
 */
size_t fa_forward_fp8_workspace_size(int B, int H, int H_kv, int N, int d);

int fa_forward_fp8(const void* q, const void* k, const void* v, const signed char* signs,
                   void* o, float* lse, int B, int H, int H_kv, int N, int d, float scale,
                   int causal, void* workspace, size_t workspace_bytes, hipStream_t stream);

int fa_fp8_prepare(const void* q, const void* k, const void* v, const signed char* signs,
                   int B, int H, int H_kv, int N, int d, void* workspace,
                   size_t workspace_bytes, hipStream_t stream);

int fa_forward_fp8_prepared(const void* workspace, size_t workspace_bytes, void* o, float* lse,
                            int B, int H, int H_kv, int N, int d, float scale, int causal,
                            hipStream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
