/*
 * pkv.h -- C ABI of libpkv: paged KV storage and paged attention on MI355X.
 *
 * A sequence's keys and values live in fixed-size pages of a device page pool
 * and are reached through its block table: position p sits in page
 * block_table[p / page_size] at offset p % page_size (TileInfer.jl docs,
 * "KV cache", section "Pages and block tables"; "KV Cache Management and
 * PagedAttention", section "Connect token order to storage locations",
 * Figure 2; indices are 0-based as in the latter).
 *
 * The library has two halves.
 *   Host:   a page allocator (free stack, block tables, reference counts,
 *           reserve / truncate / release / share) and the prefix-sharing
 *           planner.  Pure C++ on the CPU; never touches the GPU.
 *   Device: pkv_store_kv, pkv_decode and pkv_prefill_append (plus
 *           pkv_copy_pages, the group-wise codec and a streaming-read
 *           probe), hand-written HIP kernels for gfx950, enqueued on a
 *           caller-provided stream.
 *
 * Conventions for every function:
 *   - Every function returns int (PKV_OK = 0 or a negative PKV_ERR_* code),
 *     except pkv_alloc_destroy, pkv_last_error and pkv_workspace_bytes.
 *     No C++ exception crosses the ABI.  After a failure, pkv_last_error()
 *     returns a message for the calling thread.
 *   - Host calls check every argument and are all-or-nothing: on error the
 *     allocator is unchanged.
 *   - The library never allocates device memory.  Pools, queries, outputs,
 *     slots, block tables, lengths and workspace are caller-owned device
 *     buffers (any allocator; PyTorch tensors in the Python binding).  Device
 *     calls check scalars and pointer alignment on the host, enqueue work on
 *     `stream` (a hipStream_t passed as void*, NULL = the null stream) and
 *     return without synchronising.  They do not read device arrays on the
 *     host.  Kernels skip (never dereference) out-of-range slots, page ids,
 *     block-table indices and query rows, so malformed device arrays give
 *     wrong values but no out-of-bounds access; pkv_validate_tables checks
 *     such arrays on the host.
 *   - A pkv_alloc handle is not thread-safe; distinct handles are
 *     independent.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------------------
 * Status codes
 * ------------------------------------------------------------------------- */
enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1,      /* argument contradicts the state or the rules below */
  PKV_ERR_OUT_OF_PAGES = -2,     /* reserve needs more pages than are free: the
                                    OutOfPagesError of TileInfer.jl "Growing,
                                    rolling back, releasing" */
  PKV_ERR_UNSUPPORTED = -3,      /* dtype / head_dim / page_size / head counts not built */
  PKV_ERR_DEVICE = -4,           /* a HIP launch failed */
  PKV_ERR_BUFFER_TOO_SMALL = -5, /* workspace or output array too small */
  PKV_ERR_SHARED_PAGE = -6       /* pkv_reserve would write into a page another
                                    sequence references (pkv_reserve_cow copies
                                    the page instead) */
};

/* Message describing the last failing call on this thread ("" if none). */
const char* pkv_last_error(void);

/* ---------------------------------------------------------------------------
 * Host page allocator
 *
 * Source: TileInfer.jl "KV cache" -- a BlockManager keeps a stack of free
 * page ids and each sequence owns a block table ("Pages and block tables");
 * reserve! / truncate! / release! ("Growing, rolling back, releasing").
 * Quail docs "KV" -- several documents may reference one page, which is free
 * when nothing references it ("Paged KV"); a document references its
 * parent's shared pages without copying ("Execution").  "KV Cache Management
 * and PagedAttention" -- blocks are taken only when needed (Figures 1, 3) and
 * reference counts decide when a block returns to the pool ("Return blocks
 * after a request ends").
 * ------------------------------------------------------------------------- */
typedef struct pkv_alloc pkv_alloc;

/* Create an allocator over pages 0..num_pages-1 of page_size positions each.
 * free_order: NULL, or a permutation of 0..num_pages-1 giving the order pages
 * leave the free stack (free_order[0] first).  NULL means 0, 1, 2, ...
 * Errors: INVALID_ARG (num_pages < 0, page_size < 1, free_order not a
 * permutation, out == NULL). */
int pkv_alloc_create(int32_t num_pages, int32_t page_size, const int32_t* free_order,
                     pkv_alloc** out);
void pkv_alloc_destroy(pkv_alloc* a);

/* New empty sequence; its id (>= 0, never reused) goes to *seq_out. */
int pkv_seq_new(pkv_alloc* a, int32_t* seq_out);

/* Extend a sequence by n positions (n >= 0), popping a page from the free
 * stack only when the last page is full.  All-or-nothing: OUT_OF_PAGES when
 * fewer pages are free than needed; SHARED_PAGE when position len would be
 * written into a partially filled page whose reference count exceeds 1 (see
 * pkv_reserve_cow). */
int pkv_reserve(pkv_alloc* a, int32_t seq, int32_t n);

/* Keep the first n_keep positions (0 <= n_keep <= len).  Pages of logical
 * blocks >= ceil(n_keep / page_size) lose one reference; a page left with
 * none is pushed back on the free stack, last logical block first, so a
 * following reserve hands back the same pages.  No data is copied or cleared:
 * later writes overwrite the stale slots (TileInfer.jl, truncate!). */
int pkv_truncate(pkv_alloc* a, int32_t seq, int32_t n_keep);

/* truncate(seq, 0) and retire the id (TileInfer.jl, release!). */
int pkv_release(pkv_alloc* a, int32_t seq);

/* Make the empty sequence `child` reference the first n_tokens positions of
 * `parent` (n_tokens a multiple of page_size, <= len(parent)): its block
 * table becomes the parent's first n_tokens / page_size pages, each gaining
 * one reference; nothing is copied (Quail docs "KV", "Execution"). */
int pkv_share_prefix(pkv_alloc* a, int32_t child, int32_t parent, int32_t n_tokens);

/* Make the empty sequence `child` reference every page of `parent`, its
 * partially filled last page included, each page gaining one reference; the
 * child's length becomes the parent's.  Two responses to one input then share
 * the input's KV ("KV Cache Management and PagedAttention", "Share common KV
 * across responses", Figure 5).  A later write into the shared partial page
 * needs pkv_reserve_cow. */
int pkv_fork(pkv_alloc* a, int32_t child, int32_t parent);

/* pkv_reserve with copy-on-write ("KV Cache Management and PagedAttention",
 * "Split shared blocks when a write is needed", Figure 6): when the first new
 * position falls in a partially filled page that other sequences also
 * reference, the sequence first takes a fresh page (popped before any page
 * the growth needs), its block table points there, and the shared page loses
 * this reference.  copy_out[0] = the shared page, copy_out[1] = the fresh
 * one, *n_copies = 1; the caller must copy the page on the device
 * (pkv_copy_pages) before storing into it.  Otherwise *n_copies = 0.  A
 * shared page that is already full stays shared.  All-or-nothing:
 * OUT_OF_PAGES (counting the copy's page) leaves the allocator unchanged. */
int pkv_reserve_cow(pkv_alloc* a, int32_t seq, int32_t n, int32_t* copy_out, int32_t* n_copies);

/* ---------------------------------------------------------------------------
 * KV retention pool (on the allocator)
 *
 * Source: Quail docs "KV", section "KV retention".  KV that a later consumer
 * may reuse is retained within a memory limit; when the pool is over its
 * limit the KV with the lowest priority = probability_of_reuse *
 * recompute_seconds / pages (estimated compute saved per page) is removed
 * first, and a consumer that finds its KV removed computes it again.  Here a
 * retained unit is a sequence; `pages` is its page count when it enters the
 * pool; equal priorities leave in entry order; removal is pkv_release.
 * ------------------------------------------------------------------------- */

/* Retain a live, non-empty sequence (not already retained).  INVALID_ARG for
 * a negative or non-finite probability or time.  The caller keeps the
 * sequence unchanged while it is retained. */
int pkv_retention_add(pkv_alloc* a, int32_t seq, double probability_of_reuse, double recompute_seconds);

/* Release lowest-priority retained sequences until the retained page count
 * is at most limit_pages (the caller's limit: for instance the pool's pages
 * minus the pages two forward passes need).  Their ids go to evicted[],
 * eviction order, and their count to *n_evicted.  All-or-nothing:
 * BUFFER_TOO_SMALL when more than max_evicted would leave. */
int pkv_retention_evict(pkv_alloc* a, int64_t limit_pages, int32_t* evicted, int32_t max_evicted,
                        int32_t* n_evicted);

/* A consumer reuses `seq`: *available = 1 when its KV is still retained (it
 * leaves the pool and stays live), 0 when it was evicted or never retained
 * (the consumer recomputes it). */
int pkv_retention_take(pkv_alloc* a, int32_t seq, int32_t* available);

/* Sum of the retained sequences' page counts. */
int pkv_retention_pages(const pkv_alloc* a, int64_t* pages);

/* Queries of the allocator's state.  These four are helpers with no source
 * passage of their own: they read back what the calls above maintain (for
 * tests, sizing and callers' bookkeeping) and change nothing.  Errors:
 * INVALID_ARG (null pointer, unknown sequence or page). */
/* Positions stored in `seq`. */
int pkv_seq_len(const pkv_alloc* a, int32_t seq, int32_t* len);
/* Pages on the free stack. */
int pkv_num_free(const pkv_alloc* a, int32_t* n);
/* Reference count of one page (0 = free). */
int pkv_page_refcount(const pkv_alloc* a, int32_t page, int32_t* count);
/* Number of pages in a sequence's block table. */
int pkv_seq_num_blocks(const pkv_alloc* a, int32_t seq, int32_t* n);

/* Block tables of n_seqs sequences into host array out[n_seqs][stride],
 * row b = the pages of seqs[b] in logical order, the tail padded with 0.
 * BUFFER_TOO_SMALL if a table has more than `stride` pages. */
int pkv_block_tables(const pkv_alloc* a, const int32_t* seqs, int32_t n_seqs, int32_t stride,
                     int32_t* out);

/* Slots of positions start .. start+n-1 of a sequence into host array out[n]:
 * out[i] = block_table[p / page_size] * page_size + p % page_size with
 * p = start + i (the flat pool index of page and offset that TileInfer.jl's
 * prepare_step! computes for each new token).  Requires start + n <= len. */
int pkv_slots(const pkv_alloc* a, int32_t seq, int32_t start, int32_t n, int64_t* out);

/* One serving step's host preparation, the prepare_step! of TileInfer.jl
 * ("Pages and block tables": compute each new token's slot, then upload the
 * slots and the block table).  For b = 0..n_seqs-1: reserve n_new[b]
 * positions for seqs[b]; write the slots of its new positions (old length ..
 * old length + n_new[b] - 1) to slots_out, packed in b order (capacity
 * sum(n_new)); its block table to bt_out[b][bt_stride] (tail padded with 0);
 * its new length to seq_lens_out[b].  Any of slots_out, bt_out and
 * seq_lens_out may be NULL to skip it.  All-or-nothing across the batch: on
 * OUT_OF_PAGES, SHARED_PAGE or BUFFER_TOO_SMALL (a table longer than
 * bt_stride) every reserve made by this call is undone and the free stack is
 * back in its previous order.  INVALID_ARG for unknown or repeated sequence
 * ids or a negative n_new. */
int pkv_prepare_step(pkv_alloc* a, const int32_t* seqs, int32_t n_seqs, const int32_t* n_new,
                     int32_t bt_stride, int64_t* slots_out, int32_t* bt_out,
                     int32_t* seq_lens_out);

/* ---------------------------------------------------------------------------
 * Prefix-sharing planner (pure function on host arrays)
 *
 * Source: Quail docs "KV", section "The sharing plan".  Documents are sorted
 * by token sequence (lexicographically, a prefix before its extensions, ties
 * in input order); each is compared with its predecessor in that order; only
 * whole pages are shared and a document's final token is always computed
 * (shared = page_size * floor(min(lcp, len - 1) / page_size)); when the
 * predecessor itself reuses the whole shared prefix, parent links are
 * followed to the document that supplies the pages.
 *
 * tokens: all documents' token ids, concatenated; offsets[n_docs + 1]: doc d
 * is tokens[offsets[d] .. offsets[d+1]).  Outputs (caller-owned, n_docs
 * each): order[k] = document at sorted position k; parent[d] = document id
 * whose pages d adopts, or -1; shared[d] = number of adopted positions.
 * Errors: INVALID_ARG (n_docs < 0, page_size < 1, offsets not
 * non-decreasing from 0, a NULL array with n_docs > 0).
 * ------------------------------------------------------------------------- */
int pkv_plan_prefix(const int32_t* tokens, const int64_t* offsets, int32_t n_docs,
                    int32_t page_size, int32_t* order, int32_t* parent, int32_t* shared);

/* ---------------------------------------------------------------------------
 * Device operations
 *
 * Pools: separate K and V pools, each laid out row-major
 * [num_pages][num_kv_heads][page_size][head_dim] -- the TileInfer.jl pool
 * shape (head_dim, page_size, kv_heads, num_pages) in column-major order --
 * so one KV head's page is a contiguous page_size * head_dim block.
 * Supported: dtype PKV_F32, PKV_BF16 or PKV_I8; head_dim 64 or 128;
 * 1 <= page_size <= 256; num_q_heads a multiple of num_kv_heads with
 * group = num_q_heads / num_kv_heads <= 16; query head h reads KV head
 * h / group.  All device arrays must be 16-byte aligned.
 *
 * PKV_I8 (TileInfer.jl docs, "KV cache", section "INT8 cache"): each cached
 * vector (one KV head at one position) is held as head_dim int8 codes and one
 * fp32 scale, value ~ scale * code.  A pool is num_pages * num_kv_heads
 * blocks of pkv_i8_block_bytes(page_size, head_dim) bytes, block
 * (page, g) at byte (page * num_kv_heads + g) * block_bytes: first the codes
 * of offsets 0..page_size-1 (head_dim bytes each), then their page_size fp32
 * scales, then zero to 15 bytes of padding up to a multiple of 16.  So a
 * vector costs head_dim + 4 bytes (132 for head_dim 128; the padding is 0
 * when page_size is a multiple of 4).  New K/V, queries and outputs are bf16.
 * ------------------------------------------------------------------------- */
enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_I8 = 2 };

typedef struct {
  int32_t dtype;        /* PKV_F32 or PKV_BF16: pools, new K/V, q and out;
                           PKV_I8: INT8 pools, bf16 new K/V, q and out */
  int32_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
} pkv_pool_desc;

/* Bytes of one (page, KV head) block of a PKV_I8 pool:
 * page_size * head_dim + (4 * page_size rounded up to a multiple of 16);
 * 0 when page_size or head_dim is below 1. */
size_t pkv_i8_block_bytes(int32_t page_size, int32_t head_dim);

/* Bytes of one pool (K or V) for this descriptor; 0 when the descriptor is
 * not supported. */
size_t pkv_pool_bytes(const pkv_pool_desc* desc);

/* Write each new token's keys and values into the pools at its slot
 * (TileInfer.jl "Pages and block tables": store_kv! writes the new keys and
 * values at their slots).  k_new, v_new: device [n_tokens][num_kv_heads]
 * [head_dim]; slots: device int64 [n_tokens], slot = page * page_size +
 * offset.  Token t's vector for KV head g goes to pool element
 * ((page * num_kv_heads + g) * page_size + offset) * head_dim.  A slot
 * outside [0, num_pages * page_size) is skipped (padding tokens may use -1).
 * Two tokens with the same slot race: the result is one of them.
 * PKV_I8: each bf16 vector is quantized once, here ("INT8 cache"), in fp32:
 * scale = max|x| / 127, code = x / scale rounded to nearest, ties to even,
 * clamped to [-127, 127]; a zero vector gets scale 0 and codes 0.  Inputs
 * must be finite. */
int pkv_store_kv(const pkv_pool_desc* desc, void* k_pool, void* v_pool, const void* k_new,
                 const void* v_new, const int64_t* slots, int32_t n_tokens, void* stream);

/* The device half of copy-on-write: for each i < n_copies, page
 * copies[2 i + 1] of both pools becomes a byte copy of page copies[2 i] (every
 * KV head and offset; for PKV_I8 pools codes and scales).  copies: device
 * int32 [n_copies][2] = (source, destination), as pkv_reserve_cow returns
 * them.  A pair with a page outside [0, num_pages) or source == destination
 * is skipped.  Destination pages must differ from each other and from every
 * source page of the same call (pages fresh from pkv_reserve_cow do);
 * otherwise the result is undefined. */
int pkv_copy_pages(const pkv_pool_desc* desc, void* k_pool, void* v_pool, const int32_t* copies,
                   int32_t n_copies, void* stream);

/* ---------------------------------------------------------------------------
 * Group-wise low-bit KV codec (ReKV, section 2.2: the prefix KV is quantized
 * in groups of 64 elements along the last dimension and sent as packed codes
 * with one FP16 scale per group, eq. (7); the receiver dequantizes it)
 *
 * Symmetric groups: scale = fp16(max|x| / q_max), q_max = 127 (bits 8) or 7
 * (bits 4); code = x * (1 / scale) rounded to nearest (ties to even) in
 * fp32, one reciprocal per group, clamped to [-q_max, q_max]; a zero scale
 * gives zero codes.  Restoring
 * writes bf16(scale * code).  Payload: the codes of K then V (position,
 * KV head, element order; bits 8: one byte each; bits 4: two's-complement
 * nibbles, element 2i in the low nibble of byte i), then the fp16 scales of
 * K then V in the same order.  bf16 pools; head_dim 64 or 128.
 * ------------------------------------------------------------------------- */

/* Payload bytes of n_positions positions: 2 n Hkv D bits/8 + 2 (2 n Hkv D /
 * 64); 0 for unsupported arguments. */
size_t pkv_codec_payload_bytes(int32_t n_positions, int32_t num_kv_heads, int32_t head_dim, int32_t bits);

/* Encode positions 0..n_positions-1 of one sequence, read in place through
 * its device block table (>= ceil(n_positions / page_size) entries), into
 * `payload` (device, 16-byte aligned, pkv_codec_payload_bytes).  A position
 * whose table entry is not a page of the pool (< 0 or >= num_pages) encodes
 * as zeros.  Errors: INVALID_ARG, UNSUPPORTED (dtype other than PKV_BF16,
 * bits), DEVICE. */
int pkv_codec_encode(const pkv_pool_desc* desc, const void* k_pool, const void* v_pool, const int32_t* block_table,
                     int32_t n_positions, int32_t bits, void* payload, void* stream);

/* Restore a payload written by pkv_codec_encode into positions
 * 0..n_positions-1 of a sequence whose block table names the destination
 * pages (bf16(scale * code) per element; other slots untouched).  Positions
 * whose table entry is not a page of the pool are skipped, never written
 * elsewhere.  Errors: INVALID_ARG, UNSUPPORTED, DEVICE. */
int pkv_codec_decode(const pkv_pool_desc* desc, void* k_pool, void* v_pool, const int32_t* block_table,
                     int32_t n_positions, int32_t bits, const void* payload, void* stream);

/* Bytes of device workspace pkv_decode / pkv_prefill_append need for these
 * sizes (0 when a launch needs none).  Pass the same scalars to the call.
 * Returns 0 for unsupported descriptors as well; the call then reports it.
 * A helper with no source passage: it sizes the caller-owned scratch
 * (split partial states, schedule offsets) that the library never allocates. */
size_t pkv_workspace_bytes(const pkv_pool_desc* desc, int32_t n_seqs, int32_t num_q_heads,
                           int32_t max_q_per_seq, int32_t max_seq_len);

/* Paged decode: one new query per sequence attends to every stored position
 * of its sequence, reading K/V in place through its block table ("KV Cache
 * Management and PagedAttention", "Compute attention over scattered KV",
 * Figure 4: positions 0..p including the query's own, just stored; other
 * sequences' pages and unused slots take no part).
 *   q:            device [n_seqs][num_q_heads][head_dim]
 *   block_tables: device int32 [n_seqs][bt_stride]
 *   seq_lens:     device int32 [n_seqs], positions stored, the new one included
 *                 (>= 1, <= bt_stride * page_size)
 *   max_seq_len:  host upper bound of seq_lens (sizes the grid and the split);
 *                 positions at or past min(max_seq_len, bt_stride * page_size)
 *                 are never read, whatever seq_lens holds
 *   scale:        softmax scale (1/sqrt(head_dim) in the usual model)
 *   out:          device [n_seqs][num_q_heads][head_dim], dtype of q
 *                 (q and out are bf16 for PKV_I8 pools, whose key scales
 *                 multiply the scores and value scales the probabilities,
 *                 "INT8 cache")
 *   workspace:    device, >= pkv_workspace_bytes(desc, n_seqs, num_q_heads, 1,
 *                 max_seq_len) bytes (may be NULL when that is 0)
 * Long contexts are split across workgroups at fixed logical positions and
 * merged by log-sum-exp, so the result depends on the logical sequence only,
 * never on which physical pages hold it.  Errors: INVALID_ARG, UNSUPPORTED,
 * BUFFER_TOO_SMALL (workspace), DEVICE. */
int pkv_decode(const pkv_pool_desc* desc, const void* k_pool, const void* v_pool, const void* q,
               int32_t n_seqs, int32_t num_q_heads, const int32_t* block_tables,
               int32_t bt_stride, const int32_t* seq_lens, int32_t max_seq_len, float scale,
               void* out, void* workspace, size_t ws_bytes, void* stream);

/* pkv_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and the same result as pkv_decode, with the workspace taken
 * from a static device array of PKV_NOALLOC_SCRATCH_BYTES (32 MiB) that each
 * device holds from the library's load until the process ends.  Nothing is
 * allocated or freed: the array's device address is looked up once per
 * device (hipGetSymbolAddress) on the first call made with that device
 * current, and the call's stream must belong to the current device.
 * Arguments as for pkv_decode, without the workspace.  A batch whose
 * workspace (pkv_workspace_bytes(desc, n_seqs, num_q_heads, 1, max_seq_len))
 * exceeds the array is refused with BUFFER_TOO_SMALL before anything is
 * enqueued.  Every call on one device shares that device's array and nothing
 * in it needs clearing between calls; calls that can overlap on one device
 * (different streams without ordering between them) race on it.  Errors as
 * for pkv_decode. */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int pkv_decode_noalloc(const pkv_pool_desc* desc, const void* k_pool, const void* v_pool, const void* q,
                       int32_t n_seqs, int32_t num_q_heads, const int32_t* block_tables, int32_t bt_stride,
                       const int32_t* seq_lens, int32_t max_seq_len, float scale, void* out, void* stream);

/* Paged prefill / append: sequence b has n_b = cu_q[b+1] - cu_q[b] new queries
 * (packed rows cu_q[b] .. cu_q[b+1]-1 of q and out) at positions
 * seq_lens[b] - n_b .. seq_lens[b] - 1; new query i attends causally to
 * positions 0 .. seq_lens[b] - n_b + i.  The earlier positions are whatever
 * the block table names: pages adopted from a parent that shares the prefix
 * (Quail docs "KV", "The sharing plan" / "Execution"), or a document's pages
 * kept after its previous question was truncated ("KV rewind").  The new
 * positions' K/V must already be stored (pkv_store_kv).
 *   q, out:       device [total_q][num_q_heads][head_dim]; rows >= total_q are
 *                 never touched
 *   total_q:      host row count of q and out.  Not in the statement of the
 *                 problem: cu_q lives in device memory, which the host does
 *                 not read before launching, so this host bound is what
 *                 keeps every kernel's rows inside q and out whatever cu_q
 *                 holds (and it sizes the grid)
 *   cu_q:         device int32 [n_seqs + 1], non-decreasing, cu_q[0] = 0
 *   max_q_per_seq: host upper bound of n_b (queries beyond it are not computed)
 *   other arguments as for pkv_decode; workspace >= pkv_workspace_bytes(desc,
 *   n_seqs, num_q_heads, max_q_per_seq, max_seq_len).  On PKV_I8 pools the
 *   scales are folded as for pkv_decode ("INT8 cache"): codes enter the
 *   products as exact bf16 integers, the key scale multiplies the scores and
 *   the value scale the probabilities; no dequantized key or value is formed.
 * Errors: INVALID_ARG, UNSUPPORTED, BUFFER_TOO_SMALL, DEVICE. */
int pkv_prefill_append(const pkv_pool_desc* desc, const void* k_pool, const void* v_pool,
                       const void* q, int32_t total_q, const int32_t* cu_q, int32_t n_seqs,
                       int32_t num_q_heads, const int32_t* block_tables, int32_t bt_stride,
                       const int32_t* seq_lens, int32_t max_q_per_seq, int32_t max_seq_len,
                       float scale, void* out, void* workspace, size_t ws_bytes, void* stream);

/* Host-side check of device-call inputs copied to the host: every
 * seq_lens[b] in 1 .. bt_stride * page_size, every block-table entry a
 * sequence uses in [0, num_pages), and, when cu_q is not NULL, cu_q[0] = 0,
 * non-decreasing, n_b <= seq_lens[b] and n_b <= max_q_per_seq (ignored when
 * max_q_per_seq <= 0).  Returns PKV_OK or INVALID_ARG with a message. */
int pkv_validate_tables(const pkv_pool_desc* desc, const int32_t* block_tables, int32_t n_seqs,
                        int32_t bt_stride, const int32_t* seq_lens, const int32_t* cu_q,
                        int32_t max_q_per_seq);

/* ---------------------------------------------------------------------------
 * Measurement aid (not part of the paged method): the HBM read bandwidth a
 * plain streaming kernel reaches on this device, the practical ceiling the
 * memory-bound kernels above are compared with.
 *
 * Reads `bytes` (a multiple of 16) of device memory at `buf` (16-byte
 * aligned) once, with coalesced, non-temporal 16-byte loads from a
 * grid-stride loop of n_partials workgroups (1..65535).  Workgroup i writes partial_sums[i] =
 * the sum modulo 2^32 of the 32-bit words it read, so the sum of all
 * partials is the sum of every word of the buffer modulo 2^32 (which keeps
 * the loads from being elided and lets a test check that every byte was
 * read once).  partial_sums: device uint32 [n_partials], caller-owned.
 * Errors: INVALID_ARG, DEVICE. */
int pkv_stream_read(const void* buf, size_t bytes, uint32_t* partial_sums, int32_t n_partials, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
