/*
 * pa.h - paged-KV grouped-query attention for AMD MI355X (gfx950).
 *
 * C ABI of libpa.so.  Plain pointers and sizes only.
 *
 * Sources (the pages this library implements):
 *  [ALIGN] luanjiahao.me, post on aligning the Qwen3.5 KV page from 784 to
 *          832 tokens for DCU paged attention.
 *  [PREP]  jsqmd.com/news/1214744, "2026 先导杯实战：别只盯着大算子，把
 *          Qwen3.5 vLLM 单 Token 输入准备搬上 DCU" (single-token decode
 *          input preparation).
 *  [MEAS]  luanjiahao.me, 2026-07-17, DCU long-context inference
 *          measurement (decode-time linear layers, §4-§5).
 *
 * Conventions shared by every call
 *  - Every pointer argument is a DEVICE pointer (memory the caller allocated
 *    with hipMalloc or a framework on top of it), except the size_t* outputs
 *    of pa_decode_workspace_size / pa_prefill_workspace_size and the int32_t*
 *    output of
 *    pa_page_size_for_hybrid, which are host pointers.
 *  - bf16 tensors are passed as uint16_t* holding bf16 bit patterns.  All
 *    bf16 tensors must be 16-byte aligned.
 *  - KV cache layout ([ALIGN] §4): K and V are separate tensors, each
 *    [num_pages][block_size][num_kv_heads][head_dim] with rows of
 *    num_kv_heads*head_dim contiguous elements; consecutive pages are
 *    page_stride ELEMENTS apart (page_stride >= block_size*num_kv_heads*
 *    head_dim), so the joint [num_pages][2][block_size][..] layout of the
 *    pages works with k_cache = base, v_cache = base + block_size*Hkv*D and
 *    page_stride = 2*block_size*Hkv*D.
 *  - Block tables are int32 [num_seqs][bt_stride] row-major; entry p of row s
 *    is the physical page of logical page p ([ALIGN] §1: logical_page =
 *    t / block_size, page_offset = t % block_size, physical_page =
 *    block_table[logical_page]).
 *  - Supported shapes: head_dim == 256, num_q_heads == 6 * num_kv_heads
 *    (GQA ratio 6, [ALIGN] §4), 1 <= num_kv_heads <= 64.  Others return
 *    PA_ERR_UNSUPPORTED.  Any block_size >= 1 works as long as one page of
 *    one cache, block_size * num_kv_heads * 256 * 2 bytes, stays below
 *    4 GiB (kernels address rows inside a page with 32-bit byte offsets;
 *    larger pages return PA_ERR_BLOCK_SIZE).  Prefill gathers keys in
 *    64-token logical groups that may span two pages, so a page size that
 *    is not a multiple of 64 costs no masked tail group per page; decode
 *    walks 16-token steps inside pages (784, 832 and 1024 are whole numbers
 *    of them).
 *  - Ownership: the caller owns every buffer, including the decode
 *    workspace.  The library never allocates or frees device memory.  Its
 *    only state between calls is the 16 MiB static device buffer of
 *    pa_decode_noalloc (part of the library's code object, one per GPU) and
 *    that buffer's address per device, looked up on the first call there.
 *  - Execution: each call validates its arguments on the host, then only
 *    enqueues kernels on `stream` (a hipStream_t; NULL = the null stream) and
 *    returns without synchronizing.  On any error nothing is enqueued.
 *  - Errors: 0 on success, a negative PA_ERR_* code otherwise; nothing is
 *    thrown or aborted across the ABI.  pa_strerror() names a code.
 *  - Device-side preconditions (not checkable on the host, not checked in
 *    kernels): block-table entries that a call reads (logical pages below
 *    ceil(len / block_size)) lie in [0, num_pages); entries past that are
 *    never read.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_OK 0
#define PA_ERR_NULL -1          /* a required pointer is NULL */
#define PA_ERR_BLOCK_SIZE -2    /* block_size < 1, or one page of one cache >= 4 GiB */
#define PA_ERR_UNSUPPORTED -3   /* head_dim / head counts outside the supported set */
#define PA_ERR_SIZE -4          /* a count or position is out of range */
#define PA_ERR_WORKSPACE -5     /* decode workspace NULL or too small */
#define PA_ERR_TABLE -6         /* lengths need more block-table entries than given */
#define PA_ERR_STRIDE -7        /* page_stride smaller than one page */
#define PA_ERR_ALIGN -8         /* a bf16 tensor is not 16-byte aligned */
#define PA_ERR_LAUNCH -9        /* the HIP runtime rejected a kernel launch */
#define PA_ERR_SCALE -10        /* scale is not a positive finite number */
#define PA_ERR_SCRATCH -11      /* pa_decode_noalloc: batch too large for the static scratch */

/*
 * Slot mapping ([PREP] §3.2 and §5): for each token i,
 *   slot[i] = block_table[seq][pos / block_size] * block_size + pos % block_size
 * with pos = positions[i] and seq = token_seq[i] (token_seq NULL => seq 0).
 *
 * slot_out   int64 [num_tokens], written.
 * positions  int64 [num_tokens].  A negative position, or one whose logical
 *            page is >= bt_stride, yields slot -1 (no table read).
 * token_seq  int32 [num_tokens] or NULL.
 * block_table int32 [*][bt_stride].
 * num_tokens >= 0 (0 enqueues nothing).
 * Errors: PA_ERR_NULL, PA_ERR_BLOCK_SIZE, PA_ERR_SIZE (num_tokens < 0 or
 * bt_stride < 1), PA_ERR_LAUNCH.
 */
int pa_slot_mapping(int64_t* slot_out, const int64_t* positions, const int32_t* token_seq,
                    int32_t num_tokens, const int32_t* block_table, int32_t bt_stride,
                    int32_t block_size, void* stream);

/*
 * KV-cache write through a slot mapping ([PREP] §2-§3: the KV-cache write
 * position of each new token is its slot): copies k_new[i] (num_kv_heads *
 * head_dim bf16) to row slot % block_size of page slot / block_size of
 * k_cache, and v_new[i] likewise to v_cache.  Bit copy, no arithmetic.
 * Slots outside [0, num_pages * block_size) (e.g. -1 padding) are skipped.
 * Two tokens with the same slot: which one lands is unspecified.
 *
 * k_cache, v_cache  bf16 caches (layout above), modified in place.
 * k_new, v_new      bf16 [num_tokens][num_kv_heads][head_dim].
 * slot_mapping      int64 [num_tokens].
 * Errors: PA_ERR_NULL, PA_ERR_BLOCK_SIZE, PA_ERR_UNSUPPORTED, PA_ERR_SIZE
 * (num_tokens < 0, num_pages < 1), PA_ERR_STRIDE, PA_ERR_ALIGN, PA_ERR_LAUNCH.
 */
int pa_kv_write(uint16_t* k_cache, uint16_t* v_cache, int64_t page_stride, int32_t num_pages,
                int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                const uint16_t* k_new, const uint16_t* v_new, int32_t num_tokens,
                const int64_t* slot_mapping, void* stream);

/*
 * Fused slot mapping + KV-cache write: one launch computes each token's slot
 * from positions / token_seq / block_table exactly as pa_slot_mapping does,
 * optionally stores it to slot_out (NULL = do not store), and writes the
 * token's K/V rows as pa_kv_write does.  Same errors as both.
 */
int pa_kv_write_fused(uint16_t* k_cache, uint16_t* v_cache, int64_t page_stride,
                      int32_t num_pages, int32_t block_size, int32_t num_kv_heads,
                      int32_t head_dim, const uint16_t* k_new, const uint16_t* v_new,
                      int32_t num_tokens, const int64_t* positions, const int32_t* token_seq,
                      const int32_t* block_table, int32_t bt_stride, int64_t* slot_out,
                      void* stream);

/*
 * Bytes of device workspace pa_decode needs for this batch shape (split-K
 * partial results and per-sequence merge metadata).  The workspace needs no
 * initialisation: every pa_decode call writes what it later reads.  Two
 * pa_decode calls that share a workspace must not run concurrently (calls
 * queued on one stream are fine).  bytes_out: host pointer.
 * Errors: PA_ERR_NULL, PA_ERR_BLOCK_SIZE, PA_ERR_UNSUPPORTED, PA_ERR_SIZE.
 */
int pa_decode_workspace_size(int32_t num_seqs, int32_t max_seq_len, int32_t block_size,
                             int32_t num_kv_heads, size_t* bytes_out);

/*
 * Single-token (q = 1) paged GQA decode ([ALIGN] §7 defines it: every page
 * of each sequence, one block_table lookup per page, online softmax; no page
 * skipped, causal range not shortened.  The pages' kernel iterates 64-token
 * groups inside a page; this one splits each sequence's keys into 16-token
 * steps inside pages, spread over the GPU's CUs, and merges the per-CU
 * partial results in a second launch, in a fixed order).  For each sequence
 * s and query head h (KV head g = h / 6):
 *   out[s][h] = sum_j softmax_j(scale * q[s][h] . K_j) * V_j
 * over the seq_lens[s] keys j = 0 .. seq_lens[s]-1 of sequence s; the query
 * is the token at position seq_lens[s]-1, whose K/V must already be in the
 * cache (seq_lens = position + 1, [PREP] §2).  Computed in fp32 from bf16
 * inputs, written as bf16 (round to nearest even).
 *
 * out           bf16 [num_seqs][num_q_heads][256], written.
 * q             bf16 [num_seqs][num_q_heads][256].
 * seq_lens      int32 [num_seqs]; values are clamped to [0, max_seq_len];
 *               a sequence of length 0 gets an all-zero output.
 * max_seq_len   host-side bound on seq_lens, >= 1, and
 *               <= bt_stride * block_size.
 * workspace     device buffer of >= pa_decode_workspace_size(...) bytes,
 *               256-byte aligned, contents arbitrary (see above).
 * scale         positive and finite (1/sqrt(256) for the usual softmax).
 * Errors: PA_ERR_NULL, PA_ERR_BLOCK_SIZE, PA_ERR_UNSUPPORTED, PA_ERR_SIZE
 * (num_seqs < 1, max_seq_len < 1), PA_ERR_TABLE, PA_ERR_STRIDE,
 * PA_ERR_WORKSPACE, PA_ERR_ALIGN, PA_ERR_SCALE, PA_ERR_LAUNCH.
 */
int pa_decode(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
              const uint16_t* v_cache, int64_t page_stride, const int32_t* block_table,
              int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs,
              int32_t max_seq_len, int32_t block_size, float scale, int32_t num_q_heads,
              int32_t num_kv_heads, int32_t head_dim, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * pa_decode without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops or harnesses that forbid hipMalloc).  Same arguments,
 * semantics, kernels and output bits as pa_decode; the split-K partials and
 * merge metadata go to a file-scope device buffer of the library, 16 MiB per
 * GPU (held by every GPU the library runs on until the process ends; its
 * address is looked up once per device on the first call there, with that
 * device current).  The call runs on the CURRENT device; `stream` must
 * belong to it.  Calls no hipMalloc / hipFree.
 * Limit: batches whose pa_decode_workspace_size exceeds 16 MiB return
 * PA_ERR_SCRATCH (about 1300 sequences at 4 KV heads; fewer with more KV
 * heads).  Every call on one GPU shares the buffer: two calls that overlap
 * in time on one GPU (different streams, or different threads) race and
 * give wrong results; calls queued on one stream are fine.  Nothing in the
 * buffer needs to start at zero.
 * Errors: those of pa_decode except PA_ERR_WORKSPACE, plus PA_ERR_SCRATCH.
 */
int pa_decode_noalloc(uint16_t* out, const uint16_t* q, const uint16_t* k_cache,
                      const uint16_t* v_cache, int64_t page_stride, const int32_t* block_table,
                      int32_t bt_stride, const int32_t* seq_lens, int32_t num_seqs,
                      int32_t max_seq_len, int32_t block_size, float scale, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, void* stream);

/*
 * One decode step with the new token's KV write in the same launch: for
 * each sequence s with seq_lens[s] >= 1, the token at position
 * pos = seq_lens[s] - 1 is appended and attended.  Equivalent to
 *   pa_kv_write_fused(positions[s] = seq_lens[s] - 1, token_seq[s] = s, ...)
 * followed by pa_decode(...) on the same stream, with identical output bits
 * and identical cache contents afterwards ([PREP] §2: the new token's slot
 * is its KV-cache write position; [ALIGN] §7 for the attention).
 *
 * k_cache, v_cache  modified in place: row pos % block_size of page
 *                   block_table[s][pos / block_size] receives k_new[s] /
 *                   v_new[s].  That page must be a valid page (it is read
 *                   by the decode as well); sequences of length <= 0 write
 *                   nothing.  A sequence with seq_lens[s] > max_seq_len
 *                   attends its first max_seq_len cached keys unchanged
 *                   (as pa_decode does) and its new token is stored at
 *                   pos = seq_lens[s] - 1 when pos / block_size < bt_stride
 *                   (that entry must then be a valid page), otherwise not
 *                   stored (slot -1), exactly as the fused write above.
 * k_new, v_new      bf16 [num_seqs][num_kv_heads][256], 16-byte aligned.
 * slot_out          int64 [num_seqs] or NULL: the slot of each appended
 *                   token (-1 when its logical page is past the table row;
 *                   not written for sequences of length <= 0).
 * Other arguments, the workspace and errors: as pa_decode.
 */
int pa_decode_append(uint16_t* out, const uint16_t* q, uint16_t* k_cache, uint16_t* v_cache,
                     int64_t page_stride, const int32_t* block_table, int32_t bt_stride,
                     const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                     int32_t block_size, float scale, int32_t num_q_heads,
                     int32_t num_kv_heads, int32_t head_dim, const uint16_t* k_new,
                     const uint16_t* v_new, int64_t* slot_out, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * Attention for one chunk of a chunked prefill of a single sequence
 * ([ALIGN] §6: q_len query tokens at positions start_pos .. start_pos +
 * q_len - 1, with the paged KV of the first start_pos + q_len tokens,
 * complete causal attention).  The chunk's own K/V must already be in the
 * cache.  For chunk row i and query head h (KV head g = h / 6):
 *   out[i][h] = sum_j softmax_j(scale * q_chunk[i][h] . K_j) * V_j
 * over keys j <= start_pos + i when causal != 0, over all start_pos + q_len
 * keys when causal == 0.  bf16 MFMA products with fp32 accumulation; the
 * softmax weights are rounded to bf16 before the PV product; output bf16.
 *
 * out, q_chunk   bf16 [q_len][num_q_heads][256].
 * block_table    int32 [num_table_entries] (one sequence's row);
 *                ceil((start_pos + q_len) / block_size) <= num_table_entries.
 * q_len >= 1, start_pos >= 0, start_pos + q_len < 2^31.
 * scale          positive and finite.
 * workspace      device buffer of >= pa_prefill_workspace_size(...) bytes for
 *                this chunk shape, 256-byte aligned, contents arbitrary; NULL
 *                allowed when that size is 0.  Items (query head x 128-row
 *                tile) run one per workgroup, heaviest first; when their count
 *                leaves the last round of 256 workgroups (one per CU)
 *                incomplete, the items of that round are cut along their key
 *                groups and a second launch combines the parts (fixed order:
 *                results are bitwise repeatable).  The workspace holds those
 *                partial results.  Calls sharing a workspace must not run
 *                concurrently.
 * Errors: PA_ERR_NULL, PA_ERR_BLOCK_SIZE, PA_ERR_UNSUPPORTED, PA_ERR_SIZE,
 * PA_ERR_TABLE, PA_ERR_STRIDE, PA_ERR_ALIGN, PA_ERR_SCALE, PA_ERR_WORKSPACE,
 * PA_ERR_LAUNCH.
 */
int pa_prefill_chunk(uint16_t* out, const uint16_t* q_chunk, int32_t q_len, int32_t start_pos,
                     int32_t causal, const uint16_t* k_cache, const uint16_t* v_cache,
                     int64_t page_stride, const int32_t* block_table, int32_t num_table_entries,
                     int32_t block_size, float scale, int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Prefill attention for several sequences in one launch, in the vendor
 * interface's form ([ALIGN] §6: q, k, v, cu_seqlens_q, seqused_k,
 * block_table, max_seqlen_q, max_seqlen_k, causal; the page itself calls it
 * for one sequence).  Sequence s has query rows cu_seqlens_q[s] ..
 * cu_seqlens_q[s+1]-1 of q and out and seqused_k[s] keys (its own chunk's K/V
 * included, already in the cache); its rows are the last q_len_s positions:
 * row i sits at position seqused_k[s] - q_len_s + i, so with causal != 0 it
 * attends keys 0 .. seqused_k[s] - q_len_s + i and otherwise all
 * seqused_k[s] keys.  The same kernel as pa_prefill_chunk.
 *
 * out, q         bf16 [total_q][num_q_heads][256].
 * cu_seqlens_q   int32 [num_seqs + 1], non-decreasing, cu_seqlens_q[num_seqs]
 *                <= total_q.  seqused_k int32 [num_seqs].
 * block_table    int32 [num_seqs][bt_stride]; bt_stride * block_size >=
 *                max_seqlen_k.
 * max_seqlen_q, max_seqlen_k   host bounds of the device lengths (lengths
 *                above them are clamped to them).  A sequence with no rows,
 *                or with fewer keys than rows, is left unwritten.
 * Device offsets are clamped to [0, total_q]; if they decrease somewhere,
 * which sequences get written is unspecified, but no access leaves q, out or
 * a sequence's block-table row.  The launch has (total_q / 128 + num_seqs) *
 * num_q_heads workgroups: its size follows the rows batched, not num_seqs
 * times the longest sequence.  With up to 64 sequences, the sequences with
 * the most keys run first (the order changes no result).
 * Errors: PA_ERR_NULL, PA_ERR_BLOCK_SIZE, PA_ERR_UNSUPPORTED, PA_ERR_SIZE
 * (also when that workgroup count exceeds 2^31 - 1), PA_ERR_TABLE,
 * PA_ERR_STRIDE, PA_ERR_ALIGN, PA_ERR_SCALE, PA_ERR_LAUNCH.
 */
int pa_prefill_varlen(uint16_t* out, const uint16_t* q, int32_t total_q,
                      const int32_t* cu_seqlens_q, const int32_t* seqused_k, int32_t num_seqs,
                      int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t causal,
                      const uint16_t* k_cache, const uint16_t* v_cache, int64_t page_stride,
                      const int32_t* block_table, int32_t bt_stride, int32_t block_size,
                      float scale, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      void* stream);

/*
 * Bytes of device workspace pa_prefill_chunk needs for this chunk shape (0
 * when the chunk's items fill whole rounds of workgroups).  bytes_out: host
 * pointer.  Errors: PA_ERR_NULL, PA_ERR_BLOCK_SIZE, PA_ERR_UNSUPPORTED,
 * PA_ERR_SIZE.
 */
int pa_prefill_workspace_size(int32_t q_len, int32_t start_pos, int32_t causal, int32_t block_size,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              size_t* bytes_out);

/*
 * Model inputs and attention metadata of one single-request, single-token
 * decode step, written by one launch ([PREP] §2: when one request advances
 * by one token every entry is a closed form; §4, §5: the sampled token stays
 * on the device and one launch, one workgroup per KV-cache group, writes
 * everything; §3.2: the slot formula).  Writes
 *   input_ids[0]           = (int32) sampled_token_ids[0]
 *   positions[0]           = position                       (mrope == 0)
 *   positions[r * positions_stride] = position + mrope_delta,  r = 0, 1, 2
 *                                                            (mrope != 0)
 *   query_start_loc[0 .. query_start_loc_len) = 0, 1, 1, ..., 1
 *   seq_lens[0 .. seq_lens_len)               = position + 1, 0, ..., 0
 *   discard_request_mask[0 .. discard_len)    = 0 (false)
 *   is_token_ids[0]        = 1                               (if not NULL)
 *   for each KV-cache group g < num_kv_groups, with B = block_sizes[g],
 *   bt = (const int32_t*) block_table_ptrs[g] (the request's block-table
 *   row) and sm = (int64_t*) slot_mapping_ptrs[g]:
 *     sm[0] = bt[position / B] * B + position % B   (-1 when B <= 0)
 * and nothing else.  Every pointer, and every address inside the two
 * uint64 arrays, is a device address; block_sizes, block_table_ptrs and
 * slot_mapping_ptrs may be NULL when num_kv_groups == 0.  position is the
 * number of tokens already computed (the new token's index); position / B
 * must index a valid entry of each group's row (not checked).
 * Errors: PA_ERR_NULL, PA_ERR_SIZE (position < 0 or >= 2^31 - 1,
 * query_start_loc_len < 2, seq_lens_len < 1, discard_len < 1, num_kv_groups
 * outside [0, 65535], mrope with positions_stride < 1), PA_ERR_LAUNCH.
 */
int pa_decode_input_prep(const int64_t* sampled_token_ids, int64_t position, int32_t* input_ids,
                         int64_t* positions, int32_t mrope, int64_t positions_stride,
                         int64_t mrope_delta, int32_t* query_start_loc,
                         int32_t query_start_loc_len, int32_t* seq_lens, int32_t seq_lens_len,
                         uint8_t* discard_request_mask, int32_t discard_len,
                         uint8_t* is_token_ids, int32_t num_kv_groups, const int32_t* block_sizes,
                         const uint64_t* block_table_ptrs, const uint64_t* slot_mapping_ptrs,
                         void* stream);

/*
 * KV page size (tokens) of a hybrid attention / Mamba-state model ([ALIGN]
 * §3): the attention page must hold at least one Mamba state page, in whole
 * groups of alignment_tokens tokens,
 *   block_size = ceil(mamba_page_bytes /
 *                     (alignment_tokens * attn_page_bytes_per_token))
 *                * alignment_tokens,
 * the abstraction the page prints (its minimum comparison and later padding
 * branches are left out).  attn_page_bytes_per_token is one token's K and V
 * of one attention layer: 2 * num_kv_heads * head_dim * sizeof(element), 4096
 * bytes for 4 KV heads of 256 bf16 values ([ALIGN] §4).  With alignment 16 a
 * Mamba page in (3 145 728, 3 211 264] bytes gives 784 tokens, with alignment
 * 64 (the wave64 access group, [ALIGN] §2) 832.  Host-only arithmetic, no
 * device work; block_size_out is a host pointer.
 * Errors: PA_ERR_NULL, PA_ERR_SIZE (an argument <= 0, or a result above
 * 2^31 - 1).
 */
int pa_page_size_for_hybrid(int64_t mamba_page_bytes, int64_t attn_page_bytes_per_token,
                            int32_t alignment_tokens, int32_t* block_size_out);

/*
 * bf16 M=1 linear layer (GEMV) y = W x for decode ([MEAS] §4: y[j] =
 * sum_k x[k] * W[j, k], bf16 weights and input, fp32 accumulation; §5: the
 * 14336 / 16384 / 34816 x 5120 weight shapes).
 *   y    [N] output: bf16 when y_f32 == 0, float32 when y_f32 != 0
 *   W    [N, K] bf16, row-major, row stride ldw elements (ldw >= K)
 *   x    [K] bf16
 * Summation order, fixed for every launch shape so results are bitwise
 * repeatable: row j is cut into chunks of 8 consecutive elements; 64 partial
 * fp32 sums start at +0, sum l takes chunks l, l + 64, l + 128, ... in order
 * and inside a chunk the elements in order, adding each exact bf16 product
 * with one rounding (a fused multiply-add); the 64 sums are combined by a
 * butterfly over index distances 32, 16, 8, 4, 2, 1 (sum_l += sum_(l xor d));
 * the result is written as fp32 or rounded to bf16 (nearest, ties to even).
 * W is read once, with streaming (non-temporal) loads; y is written once.
 * K = 0 gives +0 everywhere; N = 0 launches nothing and checks no pointer.
 * Errors: PA_ERR_NULL (y, or W / x when N > 0 and K > 0), PA_ERR_SIZE (N < 0,
 * K < 0, K % 8 != 0, ldw < K, ldw % 8 != 0), PA_ERR_ALIGN (W or x not
 * 16-byte aligned, y not aligned to its element), PA_ERR_LAUNCH.
 */
int pa_gemv_bf16(void* y, int32_t y_f32, const void* W, const void* x, int32_t N, int32_t K,
                 int64_t ldw, void* stream);

/* Static string naming an error code (never NULL). */
const char* pa_strerror(int code);

/* Static string: library version, gfx target and kernel variant ids. */
const char* pa_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
