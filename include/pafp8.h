/*
 * pafp8.h -- C ABI of libpafp8: FP8 (e4m3) paged decode attention on MI355X.
 *
 * What the library computes comes from Cloudflare's post "Smaller, faster,
 * safer: running Kimi and GLM at scale" (3 Aug 2026) and its restatements:
 *
 *  - section "KV 缓存量化" (KV cache quantization): decode keeps its KV cache
 *    as FP8 e4m3 instead of BF16, which halves the cache and doubles the
 *    tokens it holds; the attention kernel converts the stored format when it
 *    reads it.  A BF16-cache kernel is kept for direct comparison.
 *  - section "共享 KV 缓存保护" (shared KV cache protection): many requests
 *    read and write different pages of one physical KV cache; every physical
 *    page has a tag that changes when the page is reallocated; the server
 *    records the pages and tags each request expects and checks them before
 *    decode reads the cache, terminating a request on mismatch.  The check is
 *    a separate batched pass, not fused into attention; deployments that do
 *    not enable it use a no-op tracker.
 *  - remio.ai's analysis of the post (section on shared KV cache safety):
 *    paged attention splits the cache into reusable blocks and keeps, for
 *    every logical sequence, its mapping onto physical pages.
 *
 * The pages leave the numeric format, layout and arithmetic open; the
 * readings taken here are stated with each call.
 *
 * Conventions for every call
 *  - Pointers marked "device" are device memory owned by the caller (for
 *    example torch tensors); the library never allocates or frees memory and
 *    never keeps a pointer after the call returns.  Calls are asynchronous on
 *    the caller's HIP stream; outputs are valid once that stream has reached
 *    the call.  Pointers marked "host" are read before the call returns.
 *  - A call launches kernels on that stream and does nothing else (no
 *    allocation, no memset, no synchronisation), so it may be captured in a
 *    HIP graph; replays then read the buffers the captured call was given.
 *  - A call that finds a problem on the host (NULL pointer, bad size,
 *    unsupported shape, workspace too small) returns a status other than
 *    PAFP8_OK and launches nothing; pafp8_last_error() then describes it.
 *  - Problems in device data (page ids outside the pool, lengths outside a
 *    request's page table, stale tags) never fault: they are reported per
 *    request by page_tag_check, and the other calls neither read nor write
 *    memory outside the pool for them (see each call).
 *  - No float atomics: the same inputs and split count give bitwise
 *    identical outputs.  The library has no global mutable state apart from a
 *    thread-local error message, a per-device cache of the CU count, and the
 *    device scratch of paged_decode_attn_fp8_noalloc (with a per-device cache
 *    of its address).
 *
 * Pool layout (the "shared physical page pool"):
 *   K pool and V pool: [num_pages][num_kv_heads][block], one block of
 *   page_size * head_dim elements per (page, KV head).  Token t of request b
 *   lives in physical page page_table[b][t / page_size], slot t % page_size.
 *   Elements are e4m3 codes (e = 1 byte) or bf16 (e = 2 bytes), so the same
 *   geometry takes exactly half the bytes as e4m3.
 *   A block is cut into segments of SEG = min(page_size, 64 / e) consecutive
 *   slots (64 e4m3 or 32 bf16 tokens; the whole page when it is smaller).
 *   V segment: [head_dim][SEG], dim-major: slot u, dim d at d * SEG + u.
 *   K segment: 16-byte chunks arranged so that one 16-byte load per lane of
 *   a 64-lane wave reads 1 KiB of consecutive memory.  A K row of head_dim * e
 *   bytes is R = head_dim * e / 16 chunks; chunk c = q * KL + l (KL = R / 4,
 *   q < 4 the quarter of the row).  Slot u = TG * s + 4 * j + a of a segment
 *   (TG = 16 / e tokens per group, a < 4) keeps chunk c at chunk position
 *       ((j * KL + l) * 4 + q) * (4 * SEG / TG) + 4 * s + a
 *   of the segment; byte i of the chunk holds byte i of the row's chunk.
 *   page_size is a power of two >= 16, so every segment holds a whole number
 *   of token groups.  The cache is only meant to be written by
 *   kv_quant_append / kv_quant_fill; the layout is stated for tools that read
 *   it back.
  */
#ifndef PAFP8_H
#define PAFP8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PAFP8_ABI_VERSION 2  /* 2: segmented block layout */

typedef int32_t pafp8_status;
#define PAFP8_OK 0
#define PAFP8_EINVAL 1        /* a pointer, size or value is invalid */
#define PAFP8_EUNSUPPORTED 2  /* valid but not implemented (shape, dtype) */
#define PAFP8_EHIP 3          /* a HIP runtime call or launch failed */

/* Element type of the K/V pools. */
#define PAFP8_KV_FP8_E4M3 0
#define PAFP8_KV_BF16 1

/* Per-request status flags written by page_tag_check (0 = OK). */
#define PAFP8_REQ_TAG_MISMATCH 1  /* a page's tag differs from the recorded one */
#define PAFP8_REQ_PAGE_OOB 2      /* a page id lies outside [0, num_pages) */
#define PAFP8_REQ_BAD_LEN 4       /* context length < 1 or > max_pages_per_req * page_size */

/* The shared physical page pool (layout above). */
typedef struct pafp8_cache {
    int32_t kv_dtype;      /* PAFP8_KV_FP8_E4M3 or PAFP8_KV_BF16 */
    int32_t num_pages;     /* >= 1 */
    int32_t page_size;     /* tokens per page: 16, 32, 64, 128 or 256 */
    int32_t num_kv_heads;  /* >= 1 */
    int32_t head_dim;      /* 64 or 128 */
    int32_t reserved;      /* set to 0 */
    void *k_pool;          /* device, K pool */
    void *v_pool;          /* device, V pool */
    const float *k_scale;  /* device [num_kv_heads]: value = decode(code) * k_scale[g]; e4m3 only */
    const float *v_scale;  /* device [num_kv_heads]; e4m3 only.  Scales must be finite and
                              non-zero; others give unspecified codes. */
} pafp8_cache;

/* One decode step's batch: each request's logical-to-physical page mapping. */
typedef struct pafp8_batch {
    int32_t batch;              /* number of requests B >= 0 (0: calls do nothing) */
    int32_t max_pages_per_req;  /* row length of page_table, >= 1 */
    const int32_t *page_table;  /* device [B][max_pages_per_req]: physical page ids */
    const int32_t *context_lens;/* device [B]: tokens attended this step, including the
                                   token appended this step */
    const int32_t *req_status;  /* device [B] from page_tag_check, or NULL for the
                                   no-op tracker; a non-zero entry aborts the request */
} pafp8_batch;

/* ---------------------------------------------------------------------------
 * page_tag_check -- the batched integrity check (section "共享 KV 缓存保护").
 * For every request b with L = context_lens[b]:
 *   if L < 1 or L > max_pages_per_req * page_size: status = PAFP8_REQ_BAD_LEN;
 *   else, for each page index i < ceil(L / page_size), with
 *   p = page_table[b][i]: PAFP8_REQ_PAGE_OOB if p is outside [0, num_pages),
 *   else PAFP8_REQ_TAG_MISMATCH if page_tags[p] != expected_tags[b][i].
 * req_status_out[b] is the OR of the flags (0 = the request may proceed).
 * batch->req_status is ignored.  Run it before kv_quant_append and the
 * attention call of the same step and pass req_status_out to them.
 *   page_size      tokens per page (16, 32, 64, 128, 256)
 *   page_tags      device uint32 [num_pages]: current tag of each physical page
 *   expected_tags  device uint32 [B][max_pages_per_req]: tags the request recorded
 *   req_status_out device int32 [B]
 * Exact integer work: results are bit-exact.
 * ------------------------------------------------------------------------- */
pafp8_status page_tag_check(const pafp8_batch *batch, int32_t page_size,
                            const uint32_t *page_tags, int32_t num_pages,
                            const uint32_t *expected_tags, int32_t *req_status_out,
                            hipStream_t stream);

/* ---------------------------------------------------------------------------
 * kv_quant_append -- write this step's K/V token of every request into its
 * page (section "KV 缓存量化": the cache is stored as e4m3).
 * The token goes to position pos = context_lens[b] - 1, i.e. page
 * page_table[b][pos / page_size], slot pos % page_size.
 * e4m3 pools: code = e4m3(f32(x) / scale[g]) with an IEEE single-precision
 * division and round-to-nearest-even; magnitudes >= 448 and infinities
 * saturate to +-448; NaN becomes 0x7F|sign.  bf16 pools: the bits are copied.
 *   k_new, v_new  device bf16 bit patterns [B][num_kv_heads][head_dim]
 * Requests with a non-zero batch->req_status entry, an invalid length or a
 * page id outside the pool are skipped (nothing is written for them).
 * Bit-exact.
 * ------------------------------------------------------------------------- */
pafp8_status kv_quant_append(const pafp8_cache *cache, const pafp8_batch *batch,
                             const uint16_t *k_new, const uint16_t *v_new,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------
 * kv_quant_append_checked -- page_tag_check and kv_quant_append in one launch
 * (section "共享 KV 缓存保护": the check runs before decode reads or writes
 * the cache, at a cost the post wants negligible).  Computes exactly the
 * verdict page_tag_check would (with page_size = cache->page_size and
 * num_pages = cache->num_pages), writes it to req_status_out[b], and appends
 * the token of every request whose verdict is 0, exactly as kv_quant_append.
 * batch->req_status is ignored.  Pass req_status_out to the attention call of
 * the same step (and of every other layer that shares these pages).
 *   page_tags      device uint32 [num_pages]
 *   expected_tags  device uint32 [B][max_pages_per_req]
 *   req_status_out device int32 [B]
 * Bit-exact.
 * ------------------------------------------------------------------------- */
pafp8_status kv_quant_append_checked(const pafp8_cache *cache, const pafp8_batch *batch,
                                     const uint32_t *page_tags, const uint32_t *expected_tags,
                                     const uint16_t *k_new, const uint16_t *v_new,
                                     int32_t *req_status_out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * page_tag_realloc -- give pages to new owners on the device (section
 * "共享 KV 缓存保护": a page's tag changes whenever the page is reallocated,
 * so a request still holding it under the old tag fails its next check).
 * For every k < n with p = page_ids[k] inside [0, num_pages):
 *   page_tags[p] += 1 (wrapping modulo 2^32);
 *   if owner_req is given and (b, i) = (owner_req[k], owner_slot[k]) lies in
 *   [0, batch) x [0, max_pages_per_req): expected_tags[b][i] = the new tag
 *   and, if page_table is given, page_table[b][i] = p.
 * Entries with p outside the pool change nothing.
 *   page_ids, owner_req, owner_slot  device int32 [n]; owner_* may both be NULL
 *   page_tags      device uint32 [num_pages], updated in place
 *   page_table     device int32 [batch][max_pages_per_req] or NULL
 *   expected_tags  device uint32 [batch][max_pages_per_req] (may be NULL
 *                  only without owners)
 * The pages of one call should be distinct: then the result is bit-exact.
 * A page listed m times is bumped by exactly m, but which of its owners
 * records which of the intermediate tags is unspecified.
 * ------------------------------------------------------------------------- */
pafp8_status page_tag_realloc(int32_t n, const int32_t *page_ids, const int32_t *owner_req,
                              const int32_t *owner_slot, uint32_t *page_tags, int32_t num_pages,
                              int32_t *page_table, uint32_t *expected_tags, int32_t batch,
                              int32_t max_pages_per_req, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * kv_quant_fill -- write a block of tokens per request (the prefill-to-decode
 * hand-off: prefill keeps a BF16 cache, decode stores e4m3; section
 * "KV 缓存量化").  Source token j < token_count[b] of request b goes to
 * position token_start[b] + j, encoded as in kv_quant_append.
 *   token_start, token_count  device int32 [B]
 *   src_tokens                T, the row count of the source arrays (>= 1)
 *   k_src, v_src              device bf16 [B][T][num_kv_heads][head_dim],
 *                             16-byte aligned
 * Requires token_count[b] <= T (larger counts are clipped to T) and
 * num_kv_heads * head_dim <= 2^25 (PAFP8_EUNSUPPORTED otherwise).  Positions
 * outside [0, max_pages_per_req * page_size), page ids outside the pool and
 * requests with a non-zero batch->req_status are skipped.  context_lens is
 * not read.  Bit-exact.
 * ------------------------------------------------------------------------- */
pafp8_status kv_quant_fill(const pafp8_cache *cache, const pafp8_batch *batch,
                           const int32_t *token_start, const int32_t *token_count,
                           int32_t src_tokens, const uint16_t *k_src, const uint16_t *v_src,
                           hipStream_t stream);

/* ---------------------------------------------------------------------------
 * INT4 weight streaming for decode (the post's section "模型权重压缩", model
 * weight compression: GLM weights go from FP8 to INT4 because decode streams the
 * weights from GPU memory for every token, and fewer bytes stream faster;
 * the weights are expanded before the multiplication).  The pages give no
 * grouping or zero point; the reading here: weights are signed 4-bit
 * integers q in [-8, 7] (two's complement nibbles) with one bf16 scale per
 * output row and group of 128 consecutive input features:
 *     y[m][n] = sum_k x[m][k] * q[n][k] * scales[k / 128][n].
 *
 * Packed weight layout (what int4_gemv reads): blocks of 1024 bytes, one per
 * (row tile nt of 16 output rows, group g of 128 features), ordered
 * [N / 16][K / 128].  Byte 16 * L + 4 * j + b of a block (L < 64, j < 4,
 * b < 4), with L = 16 * kq + c, holds row n = 16 * nt + c, features
 * k = 128 * g + 32 * j + 8 * kq + 2 * b (low nibble) and k + 1 (high nibble).
 * ------------------------------------------------------------------------- */

/* int4_pack_weights -- row-major weights to the packed layout.
 *   w_rowmajor  device [N][K / 2] bytes: byte k / 2 of row n holds feature k
 *               (low nibble for even k); 4-byte aligned
 *   w_packed    device [N * K / 2] bytes, 16-byte aligned (output)
 * Requires N % 16 == 0 and K % 512 == 0.  A byte permutation: bit-exact. */
pafp8_status int4_pack_weights(const uint8_t *w_rowmajor, int32_t N, int32_t K, uint8_t *w_packed,
                               hipStream_t stream);

/* int4_gemv -- y = x . W^T with W expanded on read (q * scale).
 *   x         device bf16 bit patterns [M][K], 16-byte aligned
 *   w_packed  device, the packed layout above, 16-byte aligned
 *   scales    device bf16 bit patterns [K / 128][N]
 *   y         device fp32 [M][N] (output)
 * Requires N % 16 == 0 and K % 512 == 0; any M >= 0 (64 rows of x per
 * launch).  Products are exact and summed in fp32, per group and then over
 * the K / 128 groups; in launches of at most 16 rows, and of 17 to 32 rows
 * when K is not a multiple of 1024, the sums run over x * (136 + q) and
 * 136 * sum x is taken back out.  To first order
 *     |y[m][n] - exact| <= (K / 128 + 160) * 2^-24 * sum_k |x[m][k]| (|q[n][k]| + c) s,
 * c = 272 for the rows of such a launch (M rows, or the last launch's
 * r = M mod 64 rows), c = 0 otherwise. */
pafp8_status int4_gemv(const uint16_t *x, int32_t M, const uint8_t *w_packed, const uint16_t *scales,
                       int32_t N, int32_t K, float *y, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Split-K (flash-decoding) sizing.  With num_splits = S > 1 each request's
 * pages are cut into S consecutive chunks of ceil(max_pages_per_req / S)
 * pages; each chunk produces a partial (o, lse) in the workspace and
 * splitk_combine merges them.  pafp8_default_num_splits picks S so that
 * batch * num_kv_heads * S is about one work-group per CU, with splits of at
 * least 512 tokens and none for max_pages_per_req * page_size < 2048 tokens
 * (num_cus <= 0: query the current device).
 *
 * Balanced partition, num_splits = -W (1 <= W <= 65536): for each KV head the
 * pages of all live requests, in request order, form one sequence of T pages
 * (aborted, empty and invalid requests add none), and W work-groups take
 * consecutive ranges of ceil(T / W) pages.  Every work-group then streams
 * the same bytes whatever the spread of context lengths; a request cut by a
 * range boundary is merged afterwards like split-K partials (the outputs are
 * the same attention, up to fp32 rounding order).  The ranges are found on the
 * device from context_lens, so the host needs no lengths.
 * pafp8_default_balanced_groups gives W = ceil(num_cus / num_kv_heads), one
 * work-group per CU (num_cus <= 0: query the current device).
 *
 * pafp8_decode_workspace_bytes gives the workspace size for num_splits
 * (0 when S == 1; for -W: (num_q_heads * (batch + W - 1) * (head_dim + 1))
 * floats, each part rounded up to 16 bytes, plus (batch + 1) int64).
 * Pure host functions.
 * ------------------------------------------------------------------------- */
size_t pafp8_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                    int32_t num_splits);
int32_t pafp8_default_num_splits(int32_t batch, int32_t num_kv_heads,
                                 int32_t max_pages_per_req, int32_t page_size,
                                 int32_t num_cus);
int32_t pafp8_default_balanced_groups(int32_t num_kv_heads, int32_t num_cus);

/* ---------------------------------------------------------------------------
 * paged_decode_attn_fp8 / paged_decode_attn_bf16 -- decode attention over the
 * paged cache, converting e4m3 on read (section "KV 缓存量化"); the bf16 entry
 * is the direct-comparison kernel over a bf16 pool.
 * For request b, query head h, KV head g = h / G (G = num_q_heads /
 * num_kv_heads, consecutive query heads share a KV head), L = context_lens[b]:
 *   k_t = decode(K code) * k_scale[g]   (bf16 pool: the bf16 value)
 *   s_t = sm_scale * sum_d q[b][h][d] * k_t[d]              t < L
 *   lse[b][h] = log(sum_t exp(s_t))       (natural log)
 *   out[b][h][:] = sum_t exp(s_t - lse) * v_t
 * Arithmetic: K/V are decoded exactly; products and sums accumulate in fp32.
 *   q        device bf16 bits [B][num_q_heads][head_dim]
 *   sm_scale positive, finite (typically 1/sqrt(head_dim))
 *   num_splits S >= 1 (0: pafp8_default_num_splits), or -W for the balanced
 *            partition; S > 1 and S < 0 need workspace (16-byte aligned, at
 *            least pafp8_decode_workspace_bytes; its contents are ignored)
 *   out      device fp32 [B][num_q_heads][head_dim]
 *   lse      device fp32 [B][num_q_heads], or NULL
 * G must be 1..16; cache->kv_dtype must match the entry point.
 * Aborted requests (batch->req_status[b] != 0): out = 0, lse = -inf, and
 * none of their pages are read.  With req_status NULL (no tracker) a request
 * whose length is outside [0, max_pages_per_req * page_size] or whose pages
 * include an id outside the pool gets NaN outputs instead of a fault; a
 * request with length 0 gets out = 0, lse = -inf.
 * ------------------------------------------------------------------------- */
pafp8_status paged_decode_attn_fp8(const pafp8_cache *cache, const pafp8_batch *batch,
                                   const uint16_t *q, int32_t num_q_heads, float sm_scale,
                                   int32_t num_splits, void *workspace, size_t workspace_bytes,
                                   float *out, float *lse, hipStream_t stream);

pafp8_status paged_decode_attn_bf16(const pafp8_cache *cache, const pafp8_batch *batch,
                                    const uint16_t *q, int32_t num_q_heads, float sm_scale,
                                    int32_t num_splits, void *workspace, size_t workspace_bytes,
                                    float *out, float *lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * paged_decode_attn_fp8_append / paged_decode_attn_bf16_append --
 * kv_quant_append and the attention call of the same step in one launch
 * (section "KV 缓存量化": decode writes this step's token into the e4m3 cache,
 * then reads the cache converting on read).  Exactly as kv_quant_append(cache,
 * batch, k_new, v_new) followed by paged_decode_attn_{fp8,bf16} with the same
 * arguments: the same pool bytes and bitwise the same out and lse.  The one
 * work-group of each (request, KV head) whose tokens end at the request's
 * last token writes that token before it reads its tiles; no other
 * work-group reads that slot.  Saves the append's launch and the gap after it.
 *   k_new, v_new  device bf16 bit patterns [B][num_kv_heads][head_dim]
 * Requests with a non-zero batch->req_status entry, an invalid length or a
 * page id outside the pool are skipped by the append, as by kv_quant_append.
 * ------------------------------------------------------------------------- */
pafp8_status paged_decode_attn_fp8_append(const pafp8_cache *cache, const pafp8_batch *batch,
                                          const uint16_t *q, int32_t num_q_heads, float sm_scale,
                                          int32_t num_splits, void *workspace, size_t workspace_bytes,
                                          const uint16_t *k_new, const uint16_t *v_new, float *out,
                                          float *lse, hipStream_t stream);

pafp8_status paged_decode_attn_bf16_append(const pafp8_cache *cache, const pafp8_batch *batch,
                                           const uint16_t *q, int32_t num_q_heads, float sm_scale,
                                           int32_t num_splits, void *workspace, size_t workspace_bytes,
                                           const uint16_t *k_new, const uint16_t *v_new, float *out,
                                           float *lse, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * paged_decode_attn_fp8_noalloc -- paged_decode_attn_fp8 for callers that
 * cannot allocate memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The same kernels
 * and results, bitwise, as paged_decode_attn_fp8 with the same num_splits
 * (0: the default); the split-K or balanced partials go to a device array
 * the library holds per GPU (pafp8_noalloc_scratch_bytes() = 16 MiB) instead
 * of a workspace.  Calls whose partials would exceed it (from
 * pafp8_decode_workspace_bytes) return PAFP8_EUNSUPPORTED and launch
 * nothing.  The call allocates nothing: the array's device address is looked
 * up once per device (hipGetSymbolAddress) on the first call that needs it.
 * Every call on one GPU shares that array and nothing in it is read before
 * the call writes it, so calls in stream order are independent; calls that
 * overlap on one GPU (other streams, other threads) race on it and must not
 * be issued.
 * ------------------------------------------------------------------------- */
pafp8_status paged_decode_attn_fp8_noalloc(const pafp8_cache *cache, const pafp8_batch *batch,
                                           const uint16_t *q, int32_t num_q_heads, float sm_scale,
                                           int32_t num_splits, float *out, float *lse,
                                           hipStream_t stream);
size_t pafp8_noalloc_scratch_bytes(void);

/* ---------------------------------------------------------------------------
 * splitk_combine -- merge per-split softmax partials (flash-decoding; not on
 * the pages, which leave long-context scheduling open).  For each (b, h):
 *   LSE = log sum_s exp(part_lse[b][h][s])
 *   out[b][h][:] = sum_s exp(part_lse[b][h][s] - LSE) * part_o[b][h][s][:]
 * Partials are normalised: part_o is the attention output over the split's
 * tokens alone.  Splits with lse = -inf are empty; if every split is empty,
 * out = 0 and lse = -inf.  A NaN partial lse makes (b, h) NaN.  A non-zero
 * req_status[b] (nullable) gives out = 0, lse = -inf.
 *   part_o   device fp32 [B][num_q_heads][num_splits][head_dim]
 *   part_lse device fp32 [B][num_q_heads][num_splits]
 *   out      device fp32 [B][num_q_heads][head_dim];  lse device fp32 [B][num_q_heads] or NULL
 * head_dim must be a multiple of 4 and at most 1024.
 * ------------------------------------------------------------------------- */
pafp8_status splitk_combine(const float *part_o, const float *part_lse, int32_t batch,
                            int32_t num_q_heads, int32_t num_splits, int32_t head_dim,
                            const int32_t *req_status, float *out, float *lse,
                            hipStream_t stream);

/* ---------------------------------------------------------------------------
 * pafp8_stream_read -- a measurement aid, not a step of the decode path.  The
 * KV-cache section of "Smaller, faster, safer: running Kimi and GLM at scale"
 * treats decode attention as bound by the bytes it reads; this call reads
 * `bytes` of device memory once, with the loads the attention kernels use for
 * K/V (16 bytes per lane, non-temporal, a wave's next 16 KiB tile in flight
 * while it consumes the current one), and does nothing else.  Its time is
 * what the memory system delivers for that many bytes, against which an
 * HBM-bound kernel of the same size is set beside the published peak.
 *   src        device, 16-byte aligned, `bytes` readable (not modified)
 *   bytes      a non-negative multiple of 16384
 *   work_groups number of 256-thread work-groups (>= 1); they split the
 *              buffer into equal ranges of 16 KiB tiles
 *   sink       device uint32 [sink_words], sink_words >= work_groups * 256:
 *              each thread writes the XOR of the 32-bit words it read, so the
 *              XOR over sink[0 .. work_groups * 256) is the XOR over src
 * PAFP8_EINVAL on a bad size or pointer, with nothing launched.
 * ------------------------------------------------------------------------- */
pafp8_status pafp8_stream_read(const void *src, int64_t bytes, int32_t work_groups,
                               uint32_t *sink, int64_t sink_words, hipStream_t stream);

/* pafp8_stream_read_write -- the same read of src_bytes, and a write of
 * dst_bytes = src_bytes / R (R = 1, 2 or 4) to dst with plain 16-byte stores:
 * the bare stream behind a kernel that reads and writes in that ratio (the
 * prefill-to-decode quantiser reads 2 bytes and writes 1 per element).
 * Lane l's k-th store for 16 KiB tile t goes to dst offset
 * t * 16384 / R + k * 1024 + 16 l and is the XOR of the 16-byte words it read
 * at tile offsets (kR + q) * 1024 + 16 l, q < R.
 *   src  device, 16-byte aligned, src_bytes a non-negative multiple of 16384
 *   dst  device, 16-byte aligned, dst_bytes written (0 when src_bytes is 0)
 * PAFP8_EINVAL on a bad size, ratio or pointer, with nothing launched. */
pafp8_status pafp8_stream_read_write(const void *src, int64_t src_bytes, void *dst, int64_t dst_bytes,
                                     int32_t work_groups, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * The device e4m3 codec the kernels use, exposed for conformance testing.
 * pafp8_e4m3_encode: codes[i] = e4m3(x[i]) (rounding as kv_quant_append).
 * pafp8_e4m3_decode: for each code, the value as produced by each of the
 *   three decode routes the kernels use (direct to fp32, via fp16, via
 *   bf16), widened to fp32; any output pointer may be NULL.
 * All pointers device; n >= 0 elements.
 * ------------------------------------------------------------------------- */
pafp8_status pafp8_e4m3_encode(const float *x, uint8_t *codes, int64_t n, hipStream_t stream);
pafp8_status pafp8_e4m3_decode(const uint8_t *codes, float *out_f32, float *out_via_f16,
                               float *out_via_bf16, int64_t n, hipStream_t stream);

/* Short name of a status code (static string). */
const char *pafp8_status_string(pafp8_status status);
/* Description of the last failure on the calling thread ("" if none). */
const char *pafp8_last_error(void);
/* PAFP8_ABI_VERSION of the built library, and sizeof of the two structs, so a
 * binding can check it agrees with this header. */
int32_t pafp8_abi_version(size_t *sizeof_cache, size_t *sizeof_batch);

#ifdef __cplusplus
}
#endif

#endif /* PAFP8_H */
