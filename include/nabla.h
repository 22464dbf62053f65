/*
 * nabla.h - C ABI of the MI355X (gfx950) NABLA block-sparse attention library.
 *
 * The operation is the forward pass of NABLA (Neighborhood-Adaptive Block-Level
 * Attention) as the technical summary "NABLA - Atenção de Bloco Adaptativa de
 * Vizinhança para Geração de Vídeo Eficiente" (gist.science, paper 2507.13546)
 * states it in its section "Metodologia: NABLA":
 *   1. fractal flattening of the T x H x W token grid,
 *   2. block-mean pooling of Q and K, a reduced attention map with a row softmax,
 *      per-row CDF thresholding to a binary block mask, expansion to N x N tiles,
 *   3. an optional OR with a static Sliding Tile (STA) window,
 * followed by softmax attention evaluated only on the kept N x N tiles (the
 * summary runs that step through FlexAttention; here it is a HIP kernel).
 *
 * Conventions for every entry point
 *   - Tensors are dense, row-major [batch, heads, L, d] (d innermost), in device
 *     memory, 16-byte aligned.  Q, K, V, O of one call share one dtype.
 *   - The caller owns every buffer, including the workspace; the library allocates
 *     no device memory and keeps no per-call state.  The one exception is the device
 *     array behind nabla_build_mask_raster_noalloc, a fixed NABLA_NOALLOC_SCRATCH_BYTES
 *     per GPU that exists from the library's load on.
 *   - Every call is asynchronous on `stream` (0 = the null stream) and never
 *     synchronises the host.  Calls on distinct streams may run concurrently as long
 *     as they do not write the same buffers.
 *   - Arguments are validated on the host before anything is launched; a call that
 *     returns an error other than NABLA_E_HIP has launched nothing and left every
 *     output untouched.  NABLA_E_HIP reports a launch failure; errors raised later
 *     by a kernel surface on the next synchronisation of the stream.
 *   - nabla_last_error() returns a message for the calling thread's last failure.
 */
#ifndef NABLA_H
#define NABLA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NABLA_OK = 0,
    NABLA_E_INVAL = 1,        /* bad pointer, shape, threshold, window or scale */
    NABLA_E_UNSUPPORTED = 2,  /* valid request without a kernel (N != 64, d not 64/128, nb too large) */
    NABLA_E_HIP = 3,          /* HIP launch or runtime error */
    NABLA_E_WORKSPACE = 4     /* workspace missing or smaller than nabla_build_mask_workspace_size() */
} nabla_status;

typedef enum { NABLA_F32 = 0, NABLA_BF16 = 1 } nabla_dtype;

/* Sliding Tile window, in tiles of 1 frame x P x P tokens; each size odd and >= 1.
 * Block j is inside the window of block i when |dt| <= (wt-1)/2, |dh| <= (wh-1)/2
 * and |dw| <= (ww-1)/2 between their tile coordinates; the window is centred and
 * truncated at the grid border. */
typedef struct { int wt, wh, ww; } nabla_sta_window;

/* Largest number of N-token blocks per head that nabla_build_mask (and its raster, SIP
 * and allocation-free forms), the attention entry points and the backward accept (4096
 * blocks of 64: 262,144 tokens per head), and the smaller limit of the IBCS entry points,
 * whose score rows are held in LDS. */
#define NABLA_MAX_BLOCKS 4096
#define NABLA_IBCS_MAX_BLOCKS 2048

/*
 * nabla_reorder - fractal flattening of the token axis ("Metodologia: NABLA", item 1,
 * "Reordenação de Tokens (Fractal Flattening)").
 *
 * src, dst  [batch, heads, L, d] with L = T*H*W; src != dst (no in-place).
 * inverse=0 moves raster order (token (t, y, x) at l = (t*H + y)*W + x) to fractal
 * order: frames in time order, inside a frame the P x P patches row-major, each
 * patch's P*P tokens contiguous and row-major.  Position of raster token l:
 *   ((t*(H/P) + y/P)*(W/P) + x/P)*P*P + (y%P)*P + x%P.
 * inverse=1 applies the inverse permutation.  Bit-exact copy of every element.
 * Errors: NABLA_E_INVAL for null or aliased pointers, non-positive sizes, H or W not
 * a multiple of P, inverse not 0/1, a bad dtype, misaligned pointers;
 * NABLA_E_UNSUPPORTED when d * sizeof(dtype) is not a multiple of 16 bytes.
 */
nabla_status nabla_reorder(const void* src, void* dst, int batch, int heads, int T, int H,
                           int W, int d, int P, nabla_dtype dtype, int inverse,
                           hipStream_t stream);

/*
 * nabla_build_mask_workspace_size - bytes of device workspace nabla_build_mask (and its
 * raster and SIP forms) needs (BH = batch*heads, nb = L/N, nb16 = nb rounded up to a
 * multiple of 16): the pooled K, BH*nb16*d*4 bytes, then one 4-byte exponent per block,
 * each part rounded up to 256 bytes.  After a call it holds the block means of K in a
 * two-term half-precision form (mean = (hi + lo / 2048) * 2^e, e the block's exponent),
 * laid out in tiles of 16 blocks in the order the map kernel reads them; the pooled Q is
 * formed inside the map kernel and not stored.  Returns 0 for non-positive sizes or L
 * not a multiple of N.
 */
size_t nabla_build_mask_workspace_size(int batch, int heads, int L, int d, int N);

/*
 * nabla_build_mask - adaptive block mask ("Metodologia: NABLA", item 2, plus the
 * STA union of item 3) for Q and K already in fractal order.
 *
 *   Qp, Kp  = mean of each run of N consecutive tokens (float32)      ("Downsampling")
 *   S       = Qp Kp^T * scale, A = row softmax of S                   ("Atenção Reduzida")
 *   F_ij    = sum of A_ik over k with A_ik <= A_ij (ties share one F)
 *   keep    = F_ij > thr                                              ("Limiarização CDF")
 *   mask    = keep OR (sta != NULL and block j inside the window of block i)
 * so thr = 0 keeps every block, and the blocks dropped from a row carry at most thr
 * of its pooled probability mass.  The largest block of each row is always kept.
 *
 * q, k        [batch, heads, L, d], L = T*H*W, fractal order, dtype `dtype`.
 * N           tokens per block; nb = L / N blocks per head.
 * thr         in [0, 1).
 * sta         NULL for no window, else the window (requires N == P*P, one tile per block).
 * scale       logit scale of the reduced map; <= 0 selects 1/sqrt(d).
 * kv_count    out, int32 [batch, heads, nb]: kept blocks per query block.
 * kv_index    out, int32 [batch, heads, nb, nb]: row (b, h, i) lists its kept KV blocks
 *             in ascending order in its first kv_count entries; later entries are
 *             not written.
 * bitmap      optional out (NULL to skip), uint32 [batch, heads, nb, ceil(nb/32)]:
 *             bit (j % 32) of word j / 32 of row i is the mask bit (i, j); unused high
 *             bits of the last word are zero.
 * schedule    optional out (NULL to skip), int32 [batch*heads*nb]: every query block
 *             (b*heads + h)*nb + i exactly once, as a start order for
 *             block_sparse_attn_fwd, which computes entries 2j and 2j+1 in one
 *             workgroup.  Entries 2j, 2j+1 are a pair of blocks at the same patch
 *             position in neighbouring frames t, t+1 (t even; with an odd frame count
 *             the last frame's blocks pair side by side; frames that do not hold whole
 *             blocks pair blocks 2i, 2i+1), whose kept lists largely coincide.  Heads in
 *             order, each head's pairs by decreasing combined kv_count (order among equal
 *             counts unspecified); the one block per head left without a partner (odd
 *             frame count and odd blocks per frame) goes after all heads' pairs.
 *             Consecutive workgroups spread over all XCDs, so the whole GPU works on one
 *             or two heads at a time (their K/V stay in the last-level cache) and each
 *             head's short lists run last.  It never changes results.
 * workspace   device buffer of at least nabla_build_mask_workspace_size() bytes.
 * Errors: NABLA_E_INVAL (null pointers, L != T*H*W, H or W not a multiple of P,
 * L not a multiple of N, thr outside [0,1) or NaN, a window size even or < 1, a window
 * with N != P*P, NaN or infinite scale, misaligned pointers); NABLA_E_UNSUPPORTED
 * (N != 64, d not 64 or 128, nb > NABLA_MAX_BLOCKS); NABLA_E_WORKSPACE.
 */
nabla_status nabla_build_mask(const void* q, const void* k, int batch, int heads, int T, int H,
                              int W, int d, int P, int N, float thr,
                              const nabla_sta_window* sta, float scale, nabla_dtype dtype,
                              int32_t* kv_count, int32_t* kv_index, uint32_t* bitmap,
                              int32_t* schedule, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/*
 * block_sparse_attn_fwd - softmax attention restricted to the kept N x N tiles
 * ("Metodologia: NABLA", item 2, "Expansão": the expanded mask says which N x N
 * blocks of the attention are computed; a dropped block leaves both the numerator
 * and the softmax normaliser, as the AB-Attention page's section "Onde os esquemas
 * esparsos anteriores falham" spells out).  Non-causal.
 *
 *   O[b,h,a,:] = sum over tokens t of kept blocks of row blk(a) of
 *                softmax_t(scale * q_a . k_t) * v_t
 *
 * q, k, v, o  [batch, heads, L, d], any token order as long as blocks are runs of N
 *             consecutive tokens (fractal order from nabla_reorder in the NABLA path).
 * kv_count, kv_index  as written by nabla_build_mask (any lists with entries in
 *             [0, nb) are accepted; duplicates are summed twice).  A query block with
 *             kv_count 0 gets zero output.
 * schedule    optional (NULL for natural order): a permutation of the batch*heads*nb
 *             query blocks giving the order in which they are started, e.g. the one
 *             nabla_build_mask writes.  With bf16 the kernel computes two query blocks
 *             per workgroup, entries 2j and 2j+1 (natural order: blocks 2j, 2j+1), and
 *             copies each KV tile that both keep once; pairing blocks whose lists
 *             overlap saves copies.  Results depend on neither the order nor the
 *             pairing.
 * scale       <= 0 selects 1/sqrt(d).
 * bf16: scores and the running softmax in float32, P rounded to bf16 for the P V
 * product, float32 accumulation, output rounded to nearest-even bf16.
 * f32: float32 throughout.
 * Errors: NABLA_E_INVAL (null pointers, L not a multiple of N, NaN or infinite scale,
 * misaligned pointers, bad dtype); NABLA_E_UNSUPPORTED (N != 64, d not 64 or 128).
 */
nabla_status block_sparse_attn_fwd(const void* q, const void* k, const void* v, void* o,
                                   int batch, int heads, int L, int d, int N,
                                   const int32_t* kv_count, const int32_t* kv_index,
                                   const int32_t* schedule, float scale, nabla_dtype dtype,
                                   hipStream_t stream);

/*
 * nabla_build_mask_raster - nabla_build_mask for Q and K in raster order
 * (token (t, y, x) at l = (t*H + y)*W + x): the fractal flattening ("Metodologia: NABLA",
 * item 1) is applied in the addressing instead of by a separate nabla_reorder pass.
 * Block b is the P x P patch that fractal order would place at rows [N b, N b + N),
 * read as P runs of P consecutive tokens; requires N == P*P.  Results (counts, lists,
 * bitmap, schedule) are identical to nabla_reorder followed by nabla_build_mask.
 * Errors: as nabla_build_mask, plus NABLA_E_INVAL when N != P*P.
 */
nabla_status nabla_build_mask_raster(const void* q, const void* k, int batch, int heads, int T,
                                     int H, int W, int d, int P, int N, float thr,
                                     const nabla_sta_window* sta, float scale, nabla_dtype dtype,
                                     int32_t* kv_count, int32_t* kv_index, uint32_t* bitmap,
                                     int32_t* schedule, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/*
 * nabla_build_mask_raster_noalloc - nabla_build_mask_raster for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): no workspace argument, and no allocation of any kind.  The
 * pooled K lives in a device array of the library, NABLA_NOALLOC_SCRATCH_BYTES per
 * GPU, held from the library's load until the process ends; heads are processed in
 * chunks whose pooled K fits in it (nb16 * d * 4 + nb * 4 bytes per head), one launch
 * sequence per chunk on `stream`.  Results (counts, lists, bitmap, schedule) are those of
 * nabla_build_mask_raster on the same arguments.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different threads without ordering) race and give undefined
 * lists.  Nothing in the array needs clearing between calls: each chunk writes its pooled
 * means before reading them.
 * Errors: as nabla_build_mask_raster (without the workspace errors), plus
 * NABLA_E_UNSUPPORTED when one head's pooled K exceeds the array.
 */
#define NABLA_NOALLOC_SCRATCH_BYTES (32u << 20)
nabla_status nabla_build_mask_raster_noalloc(const void* q, const void* k, int batch, int heads, int T,
                                             int H, int W, int d, int P, int N, float thr,
                                             const nabla_sta_window* sta, float scale, nabla_dtype dtype,
                                             int32_t* kv_count, int32_t* kv_index, uint32_t* bitmap,
                                             int32_t* schedule, hipStream_t stream);

/*
 * block_sparse_attn_fwd_raster - block_sparse_attn_fwd for Q, K, V and O in raster order,
 * with blocks numbered as fractal order numbers them (the lists of
 * nabla_build_mask_raster): the permutation is applied while reading tiles and writing
 * rows, so no reorder pass runs before or after.  The output equals nabla_reorder of Q,
 * K, V, block_sparse_attn_fwd, and the inverse nabla_reorder of O, bit for bit.
 * T, H, W     token grid, L = T*H*W; P patch size with N == P*P.
 * Errors: as block_sparse_attn_fwd, plus NABLA_E_INVAL for non-positive T, H, W, P, H or
 * W not a multiple of P, or N != P*P.
 */
nabla_status block_sparse_attn_fwd_raster(const void* q, const void* k, const void* v, void* o,
                                          int batch, int heads, int T, int H, int W, int d, int P,
                                          int N, const int32_t* kv_count, const int32_t* kv_index,
                                          const int32_t* schedule, float scale, nabla_dtype dtype,
                                          hipStream_t stream);

/*
 * nabla_build_mask_sip - sampled block selection with inclusion-probability weights
 * (SIP), the second feature of the AB-Attention page ("Os três recursos do
 * AB-Attention"), on NABLA's block scores: the pooled, row-softmaxed map A of
 * nabla_build_mask ("Downsampling", "Atenção Reduzida"), Q and K in fractal order.
 * For each row, block j gets the inclusion probability
 *   pi_j = 1 for the row's top block (smallest index among equal maxima),
 *   pi_j = min(1, c A_j) for the others, c such that their pi sum to budget - 1
 *          (every block is certain when budget >= nb),
 * and is kept iff uniforms[b,h,i,j] < pi_j.  A kept block's list entry carries
 * kv_logw = log(1 / pi_j) (natural log), the additive logit shift that makes
 * block_sparse_attn_fwd_weighted the Horvitz-Thompson estimate of the numerator and
 * the normaliser of the full softmax (a block with pi = 1/4 counts four times).
 * budget      expected number of kept blocks per row, >= 1.
 * uniforms    float32 [batch, heads, nb, nb] draws in [0, 1), caller's random numbers.
 * kv_count, kv_index, bitmap, schedule  as nabla_build_mask.
 * kv_logw     out, float32 [batch, heads, nb, nb]: first kv_count entries of each row,
 *             aligned with kv_index.
 * No STA window.  Errors: as nabla_build_mask, plus NABLA_E_INVAL for a null or
 * misaligned uniforms / kv_logw or budget < 1.
 */
nabla_status nabla_build_mask_sip(const void* q, const void* k, int batch, int heads, int T, int H,
                                  int W, int d, int P, int N, int budget, const float* uniforms,
                                  float scale, nabla_dtype dtype, int32_t* kv_count,
                                  int32_t* kv_index, float* kv_logw, uint32_t* bitmap,
                                  int32_t* schedule, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * nabla_build_mask_ibcs_workspace_size - bytes of device workspace nabla_build_mask_ibcs
 * needs (BH = batch*heads, nb = L/N, nb16 = nb rounded up to a multiple of 16,
 * groups = L/q_group), four sections in this order, each rounded up to 256 bytes: the
 * pooled K (BH*nb16*d floats, in tiles of 16 blocks laid out in the order the score
 * kernel's MFMA reads them), 8 centroids per query group (BH*groups*8*d floats), their
 * weights (BH*groups*8 floats) and the score rows A (BH*groups*nb floats).  After a call
 * the sections hold those values, float32; the last three row-major [batch, heads, ...].
 * Returns 0 for non-positive sizes, L not a multiple of N or of q_group, or q_group not a
 * multiple of N.
 */
size_t nabla_build_mask_ibcs_workspace_size(int batch, int heads, int L, int d, int N, int q_group);

/*
 * nabla_build_mask_ibcs - nabla_build_mask with IBCS block scores, the first feature of
 * the AB-Attention page ("Os três recursos do AB-Attention": the queries are taken in
 * blocks of 128 tokens, each clustered into 8 groups, and the groups' centroids,
 * weighted by group size, score the KV blocks) in place of the mean query of NABLA's
 * "Downsampling"; the keys are still pooled over N-token blocks, and the CDF cut, STA
 * window, lists, bitmap and schedule are NABLA's.  Q and K in fractal order.
 * For each group of q_group consecutive queries (q_group = 128 as on the page, or 64 =
 * one query block):
 *   Lloyd's k-means of its queries into k = 8 clusters: the first centroids are the
 *   queries at rows 0, q_group/8, 2 q_group/8, ...; four rounds of assigning every query
 *   to its nearest centroid (squared Euclidean distance, ties to the lower index) and
 *   moving each centroid to the mean of its queries (an empty cluster keeps its
 *   centroid); mu_c the centroids, w_c = (queries in cluster c) / q_group under the last
 *   assignment;
 *   A_gj = sum_c w_c softmax_j(scale * mu_c . Kp_j),  Kp_j the mean key of block j;
 * every query block i of group g = i / (q_group/N) takes row A_g, and
 *   keep  = F_ij > thr with F the CDF of that row, as nabla_build_mask.
 * Distances and means are float32 in a fixed order (per coordinate, in index order,
 * the rounded difference, then its square added to the running sum by one fused
 * multiply-add; a running sum over the cluster's queries in row order, then one
 * division), so the clustering is reproducible bit for bit by any implementation that
 * follows the same order.
 * Arguments, outputs and errors as nabla_build_mask, plus q_group and the workspace of
 * nabla_build_mask_ibcs_workspace_size(); NABLA_E_INVAL when q_group is not a positive
 * multiple of N or does not divide L, NABLA_E_UNSUPPORTED when q_group is not 64 or
 * 128 or nb exceeds NABLA_IBCS_MAX_BLOCKS.
 */
nabla_status nabla_build_mask_ibcs(const void* q, const void* k, int batch, int heads, int T, int H,
                                   int W, int d, int P, int N, int q_group, float thr,
                                   const nabla_sta_window* sta, float scale, nabla_dtype dtype,
                                   int32_t* kv_count, int32_t* kv_index, uint32_t* bitmap,
                                   int32_t* schedule, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/*
 * nabla_build_mask_ibcs_raster - nabla_build_mask_ibcs for Q and K in raster order (the
 * fractal flattening, "Metodologia: NABLA" item 1, applied in the addressing as in
 * nabla_build_mask_raster: query block b is the P x P patch fractal order places at
 * rows [N b, N b + N), read as P runs of P tokens; a query group is q_group / N such
 * blocks).  Results, including the workspace's centroids and scores, are identical to
 * nabla_reorder followed by nabla_build_mask_ibcs.  Arguments and errors as
 * nabla_build_mask_ibcs, plus NABLA_E_INVAL when N != P*P.
 */
nabla_status nabla_build_mask_ibcs_raster(const void* q, const void* k, int batch, int heads, int T, int H,
                                          int W, int d, int P, int N, int q_group, float thr,
                                          const nabla_sta_window* sta, float scale, nabla_dtype dtype,
                                          int32_t* kv_count, int32_t* kv_index, uint32_t* bitmap,
                                          int32_t* schedule, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);

/*
 * nabla_build_mask_ibcs_sip - the AB-Attention page's two selectors together: IBCS
 * block scores (as nabla_build_mask_ibcs: q_group-query clusters, weighted centroid
 * attention to the mean keys) sampled by SIP (as nabla_build_mask_sip: inclusion
 * probabilities pi_j = min(1, c A_j) with the row's top block certain and an expected
 * `budget` blocks per row, block j kept iff uniforms[b,h,i,j] < pi_j, list entries
 * carrying kv_logw = log(1 / pi_j) for block_sparse_attn_fwd_weighted).  Block i
 * samples from its group's score row with its own draws.
 * Arguments and outputs as nabla_build_mask_sip, plus q_group; the workspace of
 * nabla_build_mask_ibcs_workspace_size().  Errors: as nabla_build_mask_sip and
 * nabla_build_mask_ibcs.
 */
nabla_status nabla_build_mask_ibcs_sip(const void* q, const void* k, int batch, int heads, int T, int H, int W,
                                       int d, int P, int N, int q_group, int budget, const float* uniforms,
                                       float scale, nabla_dtype dtype, int32_t* kv_count, int32_t* kv_index,
                                       float* kv_logw, uint32_t* bitmap, int32_t* schedule, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/*
 * block_sparse_attn_fwd_weighted - block_sparse_attn_fwd with an additive logit shift
 * per kept tile: the logits of the tokens of list entry e of row i are
 * scale * q . k + kv_logw[b,h,i,e] (the SIP weights of nabla_build_mask_sip; the
 * computation stays an ordinary softmax).  kv_logw float32 [batch, heads, nb, nb].
 * Errors: as block_sparse_attn_fwd, plus NABLA_E_INVAL for a null or misaligned
 * kv_logw.
 */
nabla_status block_sparse_attn_fwd_weighted(const void* q, const void* k, const void* v, void* o,
                                            int batch, int heads, int L, int d, int N,
                                            const int32_t* kv_count, const int32_t* kv_index,
                                            const float* kv_logw, const int32_t* schedule,
                                            float scale, nabla_dtype dtype, hipStream_t stream);

/*
 * block_sparse_attn_fwd_lse - block_sparse_attn_fwd that also writes what the gradient
 * needs: the natural-log log-sum-exp of every query row over its kept keys,
 *   lse[b,h,a] = log( sum over tokens t of kept blocks of row blk(a) of exp(scale * q_a . k_t) ),
 * -inf for the rows of a query block with no kept block.
 * lse         out, float32 [batch, heads, L], 16-byte aligned.
 * Other arguments, results and errors as block_sparse_attn_fwd (a null lse is
 * NABLA_E_INVAL).
 */
nabla_status block_sparse_attn_fwd_lse(const void* q, const void* k, const void* v, void* o,
                                       int batch, int heads, int L, int d, int N,
                                       const int32_t* kv_count, const int32_t* kv_index,
                                       const int32_t* schedule, float scale, nabla_dtype dtype,
                                       float* lse, hipStream_t stream);

/*
 * block_sparse_attn_fwd_lse_raster - block_sparse_attn_fwd_raster that also writes the
 * log-sum-exp of block_sparse_attn_fwd_lse, in raster order like O: lse[b,h,l] belongs
 * to raster token l.  Equals nabla_reorder of Q, K, V, block_sparse_attn_fwd_lse and the
 * inverse reorder of O and of lse, bit for bit (the fractal reorder of the NABLA summary,
 * "Metodologia: NABLA", item 1, folded into the addressing).
 * Arguments, results and errors as block_sparse_attn_fwd_raster and
 * block_sparse_attn_fwd_lse.
 */
nabla_status block_sparse_attn_fwd_lse_raster(const void* q, const void* k, const void* v, void* o,
                                              int batch, int heads, int T, int H, int W, int d, int P,
                                              int N, const int32_t* kv_count, const int32_t* kv_index,
                                              const int32_t* schedule, float scale, nabla_dtype dtype,
                                              float* lse, hipStream_t stream);

/*
 * nabla_attn_bwd_workspace_size - bytes of device workspace block_sparse_attn_bwd needs
 * (nb = L/N, BH = batch*heads): the row dots D (BH*L floats), the transposed mask
 * (BH*nb*ceil(nb/32) words), the transposed lists (BH*nb counts, BH*nb*nb entries) and
 * two start orders (2*BH*nb ints), each section rounded up to 256 bytes.
 * Returns 0 for non-positive sizes or L not a multiple of N.
 */
size_t nabla_attn_bwd_workspace_size(int batch, int heads, int L, int N);

/*
 * block_sparse_attn_bwd - gradient of the block-sparse attention: for
 * O = block_sparse_attn_fwd(Q, K, V) under the lists kv_count / kv_index and an
 * upstream gradient dO, the gradients of sum(O * dO) with respect to Q, K and V.  The
 * summary claims the method speeds up training as well as inference (section
 * "Principais Contribuições", dual-phase acceleration; "Resultados Experimentais",
 * item 2, pre-training); the backward pass uses the same kept tiles, and a dropped
 * tile passes no gradient.
 * With P_at = exp(scale q_a . k_t - lse_a) on the kept tiles:
 *   D_a  = sum_c dO_ac O_ac
 *   dV_t = sum_a P_at dO_a
 *   dS_at = P_at (dO_a . v_t - D_a)
 *   dQ_a = scale * sum_t dS_at k_t,   dK_t = scale * sum_a dS_at q_a
 * q, k, v, o, dout  [batch, heads, L, d], dtype `dtype` (o and lse from
 *             block_sparse_attn_fwd_lse on the same inputs and lists).
 * lse         float32 [batch, heads, L], 16-byte aligned.
 * dq, dk, dv  out, [batch, heads, L, d], dtype `dtype`; every element is written.
 * kv_count, kv_index  the forward's lists; entries in [0, nb), no duplicates within a
 *             row (nabla_build_mask writes them that way).  dQ follows each row's list;
 *             dK and dV follow its transpose, which records a block once per row.
 * scale       <= 0 selects 1/sqrt(d); must equal the forward's.
 * bf16: S, dP in float32 from bf16 MFMAs, P and dS rounded to bf16 as operands of the
 * second products, float32 accumulation, gradients rounded to nearest-even bf16.
 * f32: float32 throughout.  Deterministic: no atomics on the gradients.
 * workspace   device buffer of at least nabla_attn_bwd_workspace_size() bytes.
 * Errors: as block_sparse_attn_fwd, plus NABLA_E_INVAL for a null or misaligned lse,
 * output aliasing an input, nb > NABLA_MAX_BLOCKS giving NABLA_E_UNSUPPORTED, and
 * NABLA_E_WORKSPACE.
 */
nabla_status block_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                   int batch, int heads, int L, int d, int N,
                                   const int32_t* kv_count, const int32_t* kv_index, float scale,
                                   nabla_dtype dtype, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/*
 * block_sparse_attn_bwd_raster - block_sparse_attn_bwd for Q, K, V, O, dO, lse and the
 * gradients in raster order (lse from block_sparse_attn_fwd_lse_raster), with blocks
 * numbered as fractal order numbers them (the lists of nabla_build_mask_raster).  The
 * permutation is applied while reading tiles and rows and writing gradients, so no
 * reorder pass runs before or after; the gradients equal those of block_sparse_attn_bwd
 * on the reordered tensors, inverse-reordered, bit for bit.
 * T, H, W     token grid, L = T*H*W; P patch size with N == P*P.
 * workspace   nabla_attn_bwd_workspace_size(batch, heads, T*H*W, N) bytes.
 * Errors: as block_sparse_attn_bwd, plus NABLA_E_INVAL for non-positive T, H, W, P, H or
 * W not a multiple of P, or N != P*P.
 */
nabla_status block_sparse_attn_bwd_raster(const void* q, const void* k, const void* v, const void* o,
                                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                          int batch, int heads, int T, int H, int W, int d, int P, int N,
                                          const int32_t* kv_count, const int32_t* kv_index, float scale,
                                          nabla_dtype dtype, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream);

/* Static name of a status code ("NABLA_OK", ...). */
const char* nabla_status_string(nabla_status status);

/* Message describing the calling thread's last failed call ("" if none). */
const char* nabla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NABLA_H */
