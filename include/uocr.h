/*
 * uocr.h -- C ABI of libuocr.so: single-step decode attention for Reference
 * Sliding Window Attention (R-SWA) and its sparse variant (SR-SWA) on AMD
 * Instinct MI355X (gfx950).
 *
 * The method (sources are web pages, cited by title and section):
 *   - R-SWA: each decode query attends to a permanent reference prefix of m
 *     tokens (visual tokens + prompt; always visible, never evicted, never
 *     updated) and to a causal window of the last n generated tokens, default
 *     n = 128, so the cache holds m + min(n, T) tokens after T generated
 *     tokens.  ["百度Unlimited OCR" paper summary, lshu.cn/news/33052,
 *     section 二 (R-SWA), parts 1 and 2; "百度 Unlimited OCR 深度实战",
 *     chenxutan.com/d/4055.html, sections 2.2.1 and 3.3.1.]
 *   - The window is a ring buffer: the new token overwrites the oldest slot
 *     in place and the write pointer advances circularly.  [Unlimited-OCR-2
 *     explainer, nxmr.cn/news/162408, section "环形缓冲"; the chenxutan.com
 *     page, section 3.3.2, keeps it as a deque of maximum length n.]
 *   - SR-SWA: the prefix is cut into 32-token blocks; a light low-dimensional
 *     index projection scores every block against the query; 1.5-entmax over
 *     the scores picks the top-k (16) blocks, 16 x 32 = 512 reference tokens;
 *     each block's weight enters the attention logits of its tokens as a log
 *     bias.  [nxmr.cn/news/162408, section "稀疏路由", steps 1-4.]
 *
 * Conventions for every call
 *   - All tensors are device pointers to contiguous arrays, innermost
 *     dimension last; q, k, v and out share the element type of
 *     uocr_shape.dtype (fp32 or bf16, bf16 = upper 16 bits of an IEEE fp32,
 *     rounded to nearest even).  Arithmetic is fp32 with fp32 softmax
 *     accumulation; routing (index, scores, entmax) accumulates in fp64.
 *   - Unit = one (sequence b, head h) pair; units are ordered b-major.
 *   - Layouts: q, out, k_new, v_new [B][H][D]; k_prefix, v_prefix
 *     [B][H][prefix_cap][D]; k_ring, v_ring [B][H][window][D];
 *     prefix_len, t_gen [B] int32; proj [D][idx_dim] fp32; kbar_idx
 *     [B][H][nb_cap][idx_dim] fp32 with nb_cap = ceil(prefix_cap/block_size);
 *     scores [B][H][nb_cap] fp32; sel_idx [B][H][topk] int32; sel_prob,
 *     sel_bias [B][H][topk] fp32.
 *   - Pointers to q/k/v/out/ring/prefix/kbar/proj must be 16-byte aligned.
 *   - Device-side values are clamped, never trusted for addressing:
 *     prefix_len[b] to [0, prefix_cap], t_gen[b] below 0 to 0, sel_idx
 *     entries outside [0, ceil(prefix_len[b]/block_size)) are skipped.
 *   - Ownership: the caller allocates and owns every buffer; the library
 *     allocates nothing and keeps no state except a thread-local error string
 *     (and, for uocr_rswa_decode_static, a static device workspace per GPU
 *     and its address), never synchronises the stream, and returns as soon as the work is
 *     enqueued on `stream` (a hipStream_t passed as void*; NULL = default
 *     stream).
 *   - Errors: every call validates its arguments on the host before any
 *     launch and returns a negative uocr_status without launching anything
 *     on failure; uocr_last_error() then describes it.  A launch failure
 *     reported by the runtime returns UOCR_ERR_HIP.  Faults inside kernels
 *     surface at the caller's next synchronisation.
 */
#ifndef UOCR_H
#define UOCR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define UOCR_VERSION 10000 /* 1.0.0 */

typedef enum {
  UOCR_OK = 0,
  UOCR_ERR_NULL = -1,        /* a required pointer is NULL                     */
  UOCR_ERR_SHAPE = -2,       /* a size is out of the supported range           */
  UOCR_ERR_DTYPE = -3,       /* unknown element type                           */
  UOCR_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required     */
  UOCR_ERR_ALIGN = -5,       /* a tensor pointer is not 16-byte aligned        */
  UOCR_ERR_UNSUPPORTED = -6, /* a valid but unimplemented configuration        */
  UOCR_ERR_HIP = -7          /* the HIP runtime rejected a launch              */
} uocr_status;

typedef enum { UOCR_F32 = 0, UOCR_BF16 = 1 } uocr_dtype;

/* Problem shape shared by every call.
 *   batch B >= 1, heads H >= 1 (one KV head per query head), head_dim D in
 *   {64, 128}; prefix_cap = token capacity of the prefix arrays per unit
 *   (0 .. 2^20); window n in 1 .. 1024; dtype a uocr_dtype; scale = logit
 *   scale (normally 1/sqrt(D)), finite.  B*H must not exceed 2^24.        */
typedef struct {
  int32_t batch;
  int32_t heads;
  int32_t head_dim;
  int32_t prefix_cap;
  int32_t window;
  int32_t dtype;
  float scale;
} uocr_shape;

/* Routing configuration of SR-SWA.  block_size must be 32 (the pages'
 * sparse_block_size), idx_dim must be 32, topk in 1 .. 64; topk >= the number
 * of blocks selects every block.  nb_cap = ceil(prefix_cap / 32) <= 4096.   */
typedef struct {
  int32_t block_size;
  int32_t idx_dim;
  int32_t topk;
} uocr_route;

/* ---------------------------------------------------------------------------
 * uocr_ring_append -- append one generated token per sequence to the ring.
 * [nxmr.cn/news/162408 "环形缓冲": overwrite the oldest slot in place, the
 * write pointer advances circularly; chenxutan.com 3.3.2: deque(maxlen=n).]
 *   For every b: slot = t_gen[b] mod window; k_ring[b][h][slot][:] =
 *   k_new[b][h][:] and the same for v, for all h; then t_gen[b] += 1.
 *   Token tau therefore always lives in slot tau mod window.  Mutates
 *   k_ring, v_ring, t_gen (in place); t_gen[b] must stay below 2^31 - 1.
 *   Call it before the decode of the same step (append-then-attend).       */
int uocr_ring_append(const uocr_shape* shape, void* k_ring, void* v_ring,
                     const void* k_new, const void* v_new, int32_t* t_gen,
                     void* stream);

/* ---------------------------------------------------------------------------
 * Workspace of the dense decode: when a unit's keys are cut into several
 * workgroups (splits), each leaves its (max, sum, partial output) in the
 * caller's workspace and a second kernel in the same stream merges them.
 * Size from uocr_rswa_workspace_bytes (0 when one split suffices: then the
 * workspace may be NULL).  No initialisation is needed.  Calls that overlap
 * in time on one workspace race: give concurrent streams their own.        */
/* Workgroups per unit of the dense decode: num_splits > 0 is taken as given
 * (bounded to one workgroup per 64 keys), 0 picks one from the shape.        */
int32_t uocr_rswa_splits(const uocr_shape* shape, int32_t num_splits);
size_t uocr_rswa_workspace_bytes(const uocr_shape* shape, int32_t num_splits);

/* ---------------------------------------------------------------------------
 * uocr_rswa_decode -- dense R-SWA decode attention for one step.
 * [lshu.cn/news/33052 section 二.1-2; chenxutan.com 2.2.1 and 3.3.1.]
 *   For unit (b, h) with m = prefix_len[b] and w = min(window, t_gen[b]):
 *   keys = k_prefix[b][h][0..m) followed by ring slots 0..w-1 (the visible
 *   window; order does not affect the result), logits l_j = scale * q.k_j,
 *   out = sum_j softmax(l)_j v_j.  An empty key set (m = 0 and t_gen = 0)
 *   gives out = 0.  The key set is cut into splits processed in parallel and
 *   merged by log-sum-exp.                                                  */
int uocr_rswa_decode(const uocr_shape* shape, const void* q,
                     const void* k_prefix, const void* v_prefix,
                     const int32_t* prefix_len, const void* k_ring,
                     const void* v_ring, const int32_t* t_gen, void* out,
                     void* workspace, size_t ws_bytes, int32_t num_splits,
                     void* stream);

/* ---------------------------------------------------------------------------
 * uocr_rswa_decode_static -- uocr_rswa_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * hosts that forbid allocation): the split partials go to a workspace of
 * 16 MiB that the library keeps in a static device array, one per GPU, held
 * until the process ends.  Nothing is allocated and no workspace is passed.
 *   Arguments, layouts and results as for uocr_rswa_decode with the same
 *   num_splits (the same kernels run).  num_splits = 0 picks the split count
 *   of uocr_rswa_decode, reduced if need be until the partials fit in 16 MiB;
 *   an explicit num_splits whose partials need more returns
 *   UOCR_ERR_WORKSPACE before anything is launched.  The first call on a
 *   device looks up that device's copy of the array (with the device
 *   current); a failure there returns UOCR_ERR_HIP.
 *   Every call on one GPU shares that GPU's array: calls that overlap in time
 *   on one GPU (concurrent streams, or host threads) race and must be
 *   serialised by the caller.  The array needs no clearing: each split
 *   writes its partial before the merge reads it.                           */
int uocr_rswa_decode_static(const uocr_shape* shape, const void* q,
                            const void* k_prefix, const void* v_prefix,
                            const int32_t* prefix_len, const void* k_ring,
                            const void* v_ring, const int32_t* t_gen, void* out,
                            int32_t num_splits, void* stream);

/* ---------------------------------------------------------------------------
 * uocr_block_index_build -- block keys of the prefix, once after prefill.
 * [nxmr.cn/news/162408 "稀疏路由" steps 1-2: 32-token blocks, low-dimensional
 * index projection.]
 *   kbar_idx[b][h][j][:] = proj^T * mean_{t in block j} k_prefix[b][h][t][:]
 *   for j < ceil(m/32) (a last partial block averages its valid tokens);
 *   rows j >= ceil(m/32) up to nb_cap are set to 0.  fp64 accumulation,
 *   stored as fp32.  The prefix is static, so this runs once per sequence. */
int uocr_block_index_build(const uocr_shape* shape, const uocr_route* route,
                           const void* k_prefix, const int32_t* prefix_len,
                           const float* proj, float* kbar_idx, void* stream);

/* uocr_block_index_range -- the same, for blocks [first_block, last_block) of
 * every unit only; rows outside the range are left as they are.  For a
 * prefix that grows by chunks (chunked prefill): after the tokens
 * [m_old, m_new) are written, a call with prefix_len = m_new and the range
 * [floor(m_old/32), ceil(m_new/32)) brings kbar_idx to what a full build at
 * m_new gives, bit for bit, reading only the new tokens and the partial
 * block before them.  0 <= first_block <= last_block <= nb_cap (else
 * UOCR_ERR_SHAPE); an empty range does nothing.                             */
int uocr_block_index_range(const uocr_shape* shape, const uocr_route* route,
                           const void* k_prefix, const int32_t* prefix_len,
                           const float* proj, float* kbar_idx,
                           int32_t first_block, int32_t last_block,
                           void* stream);

/* ---------------------------------------------------------------------------
 * uocr_block_score -- relevance of every prefix block to the query.
 * [nxmr.cn/news/162408 "稀疏路由" step 2.]
 *   q_idx = proj^T q; scores[b][h][j] = q_idx . kbar_idx[b][h][j] for
 *   j < ceil(m/32), -inf for the rest of nb_cap.  No scale.  fp64
 *   accumulation, rounded once to fp32.                                     */
int uocr_block_score(const uocr_shape* shape, const uocr_route* route,
                     const void* q, const float* proj, const float* kbar_idx,
                     const int32_t* prefix_len, float* scores, void* stream);

/* ---------------------------------------------------------------------------
 * uocr_entmax15_topk -- 1.5-entmax over the block scores and top-k selection.
 * [nxmr.cn/news/162408 "稀疏路由" steps 3-4; 1.5-entmax as in Peters,
 * Niculae & Martins 2019, exact threshold by sorting.]
 *   p = entmax_1.5(scores[b][h][0..nb)) with nb = ceil(m/32), i.e.
 *   p_j = max(0, s_j/2 - tau)^2 with sum_j p_j = 1.  The min(topk, nb) blocks
 *   ranked first by (score descending, index ascending) are written to
 *   sel_idx in ascending index order with sel_prob = p_j and sel_bias = ln p_j
 *   (-inf where p_j = 0); no renormalisation over the kept blocks.  Entries
 *   past min(topk, nb) are idx -1, prob 0, bias -inf.  sel_prob may be NULL.
 *   The threshold is computed in fp64 from the fp32 scores.                 */
int uocr_entmax15_topk(const uocr_shape* shape, const uocr_route* route,
                       const float* scores, const int32_t* prefix_len,
                       int32_t* sel_idx, float* sel_prob, float* sel_bias,
                       void* stream);

/* ---------------------------------------------------------------------------
 * uocr_prefill_route -- routing of a prefill chunk: every query of the chunk
 * routed over the prefix blocks it may see.
 * [Unlimited OCR Works README mirror (git.zoyku.com), SGLang server section,
 * notes on the memory knobs: the prefill holds a temporary score tensor of
 * about [tokens, context/32]; the routing of each query is the one of
 * uocr_block_score + uocr_entmax15_topk above.]
 *   q        [B][H][tq][D] in shape->dtype: the chunk's queries;
 *   q_pos    [B] int32 (device): position of query 0 of the chunk; query i
 *            sits at q_pos[b] + i;
 *   kbar_idx [B][H][nb_cap][32] from uocr_block_index_build.
 *   Query i sees the blocks all of whose prefix tokens come before its
 *   position: ceil(m/32) blocks once q_pos[b] + i >= m, otherwise
 *   floor((q_pos[b] + i)/32) (none for a negative position).  Over those it is
 *   routed exactly as uocr_entmax15_topk routes a decode query (fp64 scores
 *   rounded once to fp32, 1.5-entmax, top-k by (score desc, index asc),
 *   ascending index order, bias = ln p).  Outputs sel_idx / sel_prob /
 *   sel_bias [B][H][tq][topk] (sel_prob may be NULL); entries past
 *   min(topk, visible blocks) are idx -1, prob 0, bias -inf.
 *   0 <= tq <= 2^20 and B*H*tq*topk < 2^31 (else UOCR_ERR_SHAPE); tq = 0
 *   does nothing.  Two launches on `stream`; the caller owns every buffer. */
int uocr_prefill_route(const uocr_shape* shape, const uocr_route* route,
                       const void* q, int32_t tq, const int32_t* q_pos,
                       const float* proj, const float* kbar_idx,
                       const int32_t* prefix_len, int32_t* sel_idx,
                       float* sel_prob, float* sel_bias, void* stream);

/* ---------------------------------------------------------------------------
 * uocr_ngram_ban -- windowed no-repeat n-gram ban and per-page output cap
 * over one decode step's logits, in place.
 * [Unlimited OCR Works README mirror (git.zoyku.com), SGLang client example:
 * the custom logit processor with ngram_size 35, window_size 128 (one page) /
 * 1024 (several), page_token_id, eos_token_id and max_page_tokens, the
 * per-page output cap; "百度 Unlimited OCR 深度实战" (chenxutan.com), the
 * inference parameters no_repeat_ngram_size / ngram_window.]
 *   tokens      [batch][ring_cap] int32: generated token of position pos at
 *               pos % ring_cap (ring_cap >= window; only the last window
 *               positions are read);
 *   n_gen       [batch] int32: tokens generated so far;
 *   page_tokens [batch] int32: tokens generated in the current page (read
 *               only when max_page_tokens > 0; may be NULL otherwise);
 *   logits      [batch][vocab], dtype UOCR_F32 or UOCR_BF16, modified in place.
 *   Ban: inside the last min(window, n_gen) generated tokens, every n-gram
 *   whose first ngram-1 tokens equal the last ngram-1 generated tokens sets
 *   the logit of its last token to -inf.  Page guard (max_page_tokens > 0
 *   and page_tokens[b] >= max_page_tokens): every logit but page_token's and
 *   eos_token's is set to -inf.  Only -inf is written; tokens outside
 *   [0, vocab) are ignored.  1 <= window <= 4096, ngram >= 1.             */
int uocr_ngram_ban(int32_t batch, const int32_t* tokens, int32_t ring_cap,
                   const int32_t* n_gen, const int32_t* page_tokens,
                   int32_t ngram, int32_t window, int32_t page_token,
                   int32_t eos_token, int32_t max_page_tokens, void* logits,
                   int32_t vocab, int32_t dtype, void* stream);

/* ---------------------------------------------------------------------------
 * uocr_rope_page2d -- page2d two-axis rotary position embedding, in place.
 * [nxmr.cn/news/162408, section "2D 位置编码": a rotary encoding with a token
 * axis (offset within the page) and a page axis (page number, page_mod 2),
 * config sparse_rope_mode page2d; the rotation of each pair of dimensions is
 * RoFormer's (Su et al., 2021).  The page gives neither the frequencies nor
 * the split of the head dimension: the choices below are this library's.]
 *   x       [B][H][tokens][D] in shape->dtype (queries or keys), rotated in
 *           place; batch, heads, head_dim and dtype of shape are used (its
 *           other fields must still pass the checks every call makes);
 *   y       NULL, or a second tensor of the same layout turned by the same
 *           positions in the same launch (e.g. x = q, y = k_new of a decode
 *           step); it must not be x;
 *   page, offset [B][tokens] int32 (device): the position of token t of
 *           sequence b, shared by its heads; negative values count as 0.
 *   Pair j < D/2 is the dims (j, j + D/2); (a, b) becomes
 *   (a cos phi - b sin phi, a sin phi + b cos phi).  Pairs j < D/4 take
 *   phi = offset * theta_j, pairs j >= D/4 take phi = pp * theta_(j - D/4)
 *   with pp = page mod page_mod (page_mod > 0) or page (page_mod = 0), and
 *   theta_i = base^(-2 i / (D/2)).  The angle is exact to ~1e-10 rad; cos,
 *   sin and the rotation are fp32, bf16 results rounded to nearest even.
 *   0 <= tokens <= 2^20, page_mod >= 0, base finite and > 0, y != x (else
 *   UOCR_ERR_SHAPE); tokens = 0 does nothing.  x and y 16-byte aligned.
 *   One launch on `stream`.                                               */
int uocr_rope_page2d(const uocr_shape* shape, void* x, void* y, int32_t tokens,
                     const int32_t* page, const int32_t* offset,
                     int32_t page_mod, float base, void* stream);

/* ---------------------------------------------------------------------------
 * uocr_srswa_decode -- SR-SWA decode: selected blocks + window, log bias.
 * [nxmr.cn/news/162408 "稀疏路由" step 4 and "环形缓冲"; 16 x 32 = 512
 * reference tokens per query.]
 *   keys = the tokens of every selected block j (sel_idx entry i >= 0), with
 *   bias sel_bias[i] added to the scaled logit of each of its tokens, plus
 *   the visible window with bias 0; out = softmax-weighted sum of values.
 *   sel_bias NULL means bias 0 for every selected block.  A block whose bias
 *   is -inf has weight exactly 0 and is not read at all.
 *   A unit's live blocks and window rows are shared among num_splits
 *   workgroups (0 = one per unit when there are at least as many units as
 *   the device has compute units (256 on MI355X), else about one workgroup
 *   per compute unit in all, at most 8 per unit; uocr_srswa_splits
 *   gives the count); with more than one, each leaves its (max, sum, partial
 *   output) in the workspace and a second kernel in the same stream merges
 *   them, as in uocr_rswa_decode.  Size the workspace with
 *   uocr_srswa_workspace_bytes for the same num_splits (0 bytes for one
 *   workgroup per unit: then workspace may be NULL); no initialisation is
 *   needed; calls that overlap on one workspace race.  Beyond the call
 *   list of the measurement plan, num_splits lets a caller fix the split
 *   count, as for the dense decode.                                         */
int32_t uocr_srswa_splits(const uocr_shape* shape, const uocr_route* route, int32_t num_splits);
size_t uocr_srswa_workspace_bytes(const uocr_shape* shape, const uocr_route* route, int32_t num_splits);
int uocr_srswa_decode(const uocr_shape* shape, const uocr_route* route,
                      const void* q, const void* k_prefix, const void* v_prefix,
                      const int32_t* prefix_len, const int32_t* sel_idx,
                      const float* sel_bias, const void* k_ring,
                      const void* v_ring, const int32_t* t_gen, void* out,
                      void* workspace, size_t ws_bytes, int32_t num_splits,
                      void* stream);

/* ---------------------------------------------------------------------------
 * Fused decode steps: one call = one whole decode step of the path above.
 * [Same passages as the calls they fuse.]
 *   uocr_rswa_step  == uocr_ring_append then uocr_rswa_decode;
 *   uocr_srswa_step == uocr_ring_append then uocr_block_score,
 *                      uocr_entmax15_topk and uocr_srswa_decode,
 * with the same results (sel_idx / sel_prob / sel_bias; out up to the order
 * of its floating-point sums, which the waves split differently), except that
 * the generated-token counts are double-buffered: t_gen_in[b] is read,
 * t_gen_out[b] = t_gen_in[b] + 1 is written and t_gen_in is left unchanged,
 * so that no workgroup can see a count another one already advanced.  The
 * two arrays must not overlap; callers alternate them between steps.  The
 * sparse step keeps the block scores on chip (no scores array).
 *   uocr_rswa_step: workspace and num_splits as for uocr_rswa_decode.
 *   uocr_srswa_step: one workgroup per unit; num_splits = waves per
 *   workgroup, 4, 8 or 16 (0 = 8).
 *
 * rope (NULL: none) fuses the page2d rotary embedding of uocr_rope_page2d
 * into the step.  [nxmr.cn/news/162408, section "2D 位置编码"; the rotation
 * and its readings as for uocr_rope_page2d.]  The step's new token of
 * sequence b sits at (rope->page[b], rope->offset[b]) ([B] int32, device,
 * 4-byte aligned); q and k_new are turned by that position before anything
 * reads them: the turned k row is what enters the ring, and the turned q is
 * both the routing query and the attention query.  q and k_new themselves
 * are left unchanged.  The results are those of uocr_rope_page2d on q and
 * k_new (x = q, y = k_new, tokens = 1) followed by the step without rope,
 * bit for bit.  page_mod >= 0 and base finite and > 0, else UOCR_ERR_SHAPE. */
typedef struct {
  const int32_t* page;
  const int32_t* offset;
  int32_t page_mod;
  float base;
} uocr_rope;

int uocr_rswa_step(const uocr_shape* shape, const void* q, const void* k_new,
                   const void* v_new, const void* k_prefix, const void* v_prefix,
                   const int32_t* prefix_len, void* k_ring, void* v_ring,
                   const int32_t* t_gen_in, int32_t* t_gen_out, void* out,
                   void* workspace, size_t ws_bytes, int32_t num_splits,
                   const uocr_rope* rope, void* stream);
int uocr_srswa_step(const uocr_shape* shape, const uocr_route* route,
                    const void* q, const void* k_new, const void* v_new,
                    const void* k_prefix, const void* v_prefix,
                    const int32_t* prefix_len, const float* proj,
                    const float* kbar_idx, void* k_ring, void* v_ring,
                    const int32_t* t_gen_in, int32_t* t_gen_out,
                    int32_t* sel_idx, float* sel_prob, float* sel_bias,
                    void* out, int32_t num_splits, const uocr_rope* rope,
                    void* stream);

/* ---------------------------------------------------------------------------
 * Diagnostics. */
const char* uocr_status_string(int status); /* static string, never NULL   */
const char* uocr_last_error(void);          /* thread-local detail, "" if none */
int uocr_version(void);                     /* UOCR_VERSION                */

#ifdef __cplusplus
}
#endif
#endif /* UOCR_H */
