/*
 * paged_attn.h -- C ABI of the MI355X (gfx950) paged grouped-query attention
 * library: a KV cache kept in fixed 256-position pages behind a per-stream
 * page table, with split-K decode (partials plus a log-sum-exp merge) and
 * causal prompt-chunk prefill over the paged prefix.
 *
 * Sources the operations follow (TensorFold pull requests and issue):
 *   - pull request #1373, "What changes": decode tiles and prompt rows read
 *     key rows through the stream's page table when it has one, else from a
 *     contiguous slab, with the same arithmetic either way;
 *   - pull request #2011, "What this changes" and review section "Is paged
 *     output the same as windowed output?": pages of 256 positions, the page
 *     looked up once per page, addresses change and the bytes do not;
 *   - pull request #2011, review section "Memory admission": pages claimed
 *     up front, all or nothing, lowest ids for KV;
 *   - issue #1344, "Mechanism" and "Conclusion": decode is a split partial
 *     plus a merge, and a stream's result must not depend on what else is in
 *     the batch (one arithmetic for paged and contiguous streams).
 *
 * Conventions for every entry point:
 *   - "device" pointers point into GPU memory the caller owns; the library
 *     never allocates, frees or synchronises device memory.  Work is enqueued
 *     on the HIP stream passed as `hip_stream` (a hipStream_t; NULL is the
 *     default stream) and completes asynchronously.
 *   - Descriptor arrays (pa_kv_cache, pa_stream) are host memory and are
 *     read only during the call.
 *   - All validation happens on the host before anything is enqueued.  On a
 *     negative status nothing has been launched and no output byte changed.
 *   - A query row i of a stream is at absolute position first_pos + i and
 *     attends keys 0 .. first_pos + i inclusive (causal).  Q and the output
 *     are bf16 [total_rows][n_q_heads][head_dim], row-major; a stream's rows
 *     are rows row_offset .. row_offset + n_rows - 1.  Query head h reads kv
 *     head h / (n_q_heads / n_kv_heads).
 *   - Page ids read from a device page table are checked on the device: an
 *     id outside [0, n_pages) is never dereferenced.  Attention rows that
 *     would read it come out NaN (so may other rows of the same stream that
 *     one workgroup computes with them); other streams are unaffected.
 *     write_kv skips a row whose page id is rejected.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define PA_API __attribute__((visibility("default")))
#else
#define PA_API
#endif

/* Positions per page; fixed at compile time in every kernel. */
#define PA_PAGE_POSITIONS 256
/* Default split-K size of decode, in keys (a multiple of the page). */
#define PA_DEFAULT_SPLIT_KEYS 4096
/* Most query rows per stream one decode call serves (verify rows). */
#define PA_DECODE_MAX_ROWS 16
/* Most rows of a stream that carries an ancestor table (one 32-bit word per row). */
#define PA_TREE_MAX_ROWS 32

typedef enum pa_status {
  PA_OK = 0,
  PA_EINVAL = -1,        /* a null pointer, bad enum, bad count or bad shape */
  PA_ERANGE = -2,        /* rows past the stream's context, overlapping rows */
  PA_ENOSPC = -3,        /* page pool: not enough free pages right now */
  PA_ETOOBIG = -4,       /* page pool: more pages than the pool will ever hold */
  PA_EWORKSPACE = -5,    /* decode workspace missing or smaller than required */
  PA_EDEVICE = -6,       /* a HIP launch failed (hipGetLastError after launch) */
  PA_EUNSUPPORTED = -7   /* head_dim or group size this build has no kernel for */
} pa_status;

typedef enum pa_kv_dtype {
  PA_KV_BF16 = 0,        /* bf16 keys and values */
  PA_KV_FP8_E4M3 = 1     /* OCP E4M3FN codes times a per-tensor scale */
} pa_kv_dtype;

typedef enum pa_layout {
  PA_LAYOUT_PAGED = 0,   /* rows live in pool pages named by page_table */
  PA_LAYOUT_SLAB = 1     /* rows live in a per-stream contiguous slab */
} pa_layout;

/*
 * The page pool as the kernels see it (one layer's pool, or one layer's
 * block inside a multi-layer pool when page_stride is larger).
 *
 * K, page p, kv head g, slot j (position 256*t + j of the page's stream),
 * dim d: element  p*page_stride + (g*256 + j)*head_dim + d            (head-major)
 * V, same: element  p*page_stride + g*256*head_dim
 *                   + ((j/VB)*head_dim + d)*VB + j%VB               (key blocks)
 * with VB = 64 / element size (32 keys for bf16, 64 for fp8): V is kept in
 * 64-byte key blocks, dim-major inside a block.
 *
 * Elements are bf16 (2 bytes) or E4M3FN codes (1 byte) per `dtype`.  The V
 * layout makes the MFMA operand of P.V (eight consecutive keys of one dim)
 * one 16-byte load, and makes a chunk of VB keys one contiguous run of
 * head_dim*64 bytes, so every HBM line a chunk reads is used whole.
 */
typedef struct pa_kv_cache {
  void *k_pages;         /* device, may be NULL if no stream is paged */
  void *v_pages;         /* device, may be NULL if no stream is paged */
  int64_t page_stride;   /* elements between pages, >= n_kv_heads*256*head_dim */
  int32_t n_pages;       /* pages in the pool */
  int32_t n_kv_heads;    /* >= 1 */
  int32_t head_dim;      /* 128 or 256 */
  int32_t dtype;         /* pa_kv_dtype */
  float k_scale;         /* fp8: value = code * k_scale; ignored for bf16 */
  float v_scale;         /* fp8: value = code * v_scale; ignored for bf16 */
} pa_kv_cache;

/*
 * One stream (sequence) of a launch.  Slab layout, capacity C positions (a
 * multiple of 256), same dtype as the cache: K element (g*C + t)*head_dim + d;
 * V element g*C*head_dim + ((t/VB)*head_dim + d)*VB + t%VB (the page layout
 * of V repeated over the slab).
 *
 * Ancestor table (tree-shaped speculative verify; TensorFold pull request
 * #1355, follow-up checks, "Indexing", names a per-row ancestor table beside
 * the query rows): when tree_mask is set (device, n_rows 32-bit words,
 * n_rows <= PA_TREE_MAX_ROWS), row i attends every key before first_pos and,
 * of the rows' own keys, position first_pos + j (j <= i) only when bit j of
 * word i is set; bits above i are ignored.  The rows' K/V are stored in
 * topological order (a node after its parent).  Every row must attend at
 * least one key (set bit i, or have first_pos > 0).  NULL: the causal chain.
 */
typedef struct pa_stream {
  int32_t layout;          /* pa_layout */
  int32_t ctx_len;         /* positions stored for the stream (>= 1) */
  int32_t n_rows;          /* query rows in this call (>= 0) */
  int32_t row_offset;      /* index of the stream's first row in q / out */
  int32_t first_pos;       /* absolute position of the first row; first_pos + n_rows <= ctx_len */
  int32_t reserved;        /* must be 0 */
  const int32_t *page_table; /* device, ceil(ctx_len/256) page ids (paged layout) */
  void *k_slab;            /* device (slab layout) */
  void *v_slab;            /* device (slab layout) */
  int64_t slab_cap;        /* slab capacity in positions (slab layout) */
  const uint32_t *tree_mask; /* device ancestor words, or NULL (see above) */
} pa_stream;

/* Text for a pa_status value (static storage). */
PA_API const char *pa_status_string(int status);

/* Library ABI version: (major << 16) | minor. */
PA_API int pa_version(void);

/* A plain streaming read of `bytes` of device memory at `buf`, for
 * measuring the device's achievable HBM read rate beside the attention
 * kernels (the pages time their arms against such a reference, interleaved:
 * pull request #2011, the author's A/A comment).  Not part of attention.
 * buf: device, 16-byte aligned; bytes: a positive multiple of 16; every
 * 16-byte chunk is read once with nontemporal loads.  sink: device, one
 * uint32 that the kernel XORs a fold of the data into (so that no load is
 * dead); its value carries no meaning.  Enqueued on hip_stream (null: the
 * null stream); PA_EINVAL on a bad argument, PA_EDEVICE if the launch
 * fails. */
PA_API int pa_hbm_read_probe(const void *buf, size_t bytes, uint32_t *sink, void *hip_stream);

/* ---------------------------------------------------------------- page pool
 * Host-side bookkeeping of which page ids are free (pull request #2011,
 * "Memory admission").  The pool's device memory is the caller's.  A pool
 * handle is not thread-safe; serialise calls on one handle. */
typedef struct pa_page_pool pa_page_pool;

/* Create a pool of n_pages free pages (ids 0..n_pages-1).  *out receives the
 * handle.  PA_EINVAL if n_pages < 1 or out is NULL. */
PA_API int page_pool_create(int32_t n_pages, pa_page_pool **out);

/* Release the handle (NULL is allowed). */
PA_API void page_pool_destroy(pa_page_pool *pool);

/* Claim n pages, all or nothing, lowest free ids first, written in
 * ascending order to ids_out (host, n entries).  PA_ETOOBIG if n exceeds the
 * pool's size (it can never fit), PA_ENOSPC if fewer than n are free now
 * (nothing is claimed), PA_EINVAL for n < 0 or null pointers. */
PA_API int page_pool_alloc(pa_page_pool *pool, int32_t n, int32_t *ids_out);

/* Shared prefix pages (TensorFold pull request #2011 and the review of #1355
 * name prefix sharing and a prompt cache that keeps KV pages on the device):
 * every claimed page carries a reference count, 1 after page_pool_alloc.
 * page_pool_share adds one reference per occurrence of an id (a second
 * stream's page table now names the page); page_pool_free drops one per
 * occurrence, and a page returns to the free set when its count reaches 0.
 * A stream that must write into a shared partial last page copies it first
 * (page_copy) into a page of its own: copy on write. */

/* Drop one reference per occurrence of each id.  PA_ERANGE if an id is out
 * of range or would drop below zero references (nothing changes then). */
PA_API int page_pool_free(pa_page_pool *pool, const int32_t *ids, int32_t n);

/* Add one reference per occurrence of each id.  PA_ERANGE if an id is out of
 * range or not claimed (nothing changes then). */
PA_API int page_pool_share(pa_page_pool *pool, const int32_t *ids, int32_t n);

/* References held on page id (0: free), or a negative status. */
PA_API int32_t page_pool_refcount(const pa_page_pool *pool, int32_t id);

/* Number of free pages, or a negative status for a NULL pool. */
PA_API int32_t page_pool_free_count(const pa_page_pool *pool);

/* ----------------------------------------------------------- whole pages
 * A page is page_stride contiguous elements of K (and of V) starting at
 * element page*page_stride: every kv head of it, and, when the pool holds
 * several layers per page (a layer's view is k_pages/v_pages advanced by
 * its block and the same page_stride: the layer block inside a page of
 * TensorFold pull request #2011, review section "Is paged output the same
 * as windowed output?", the bullet on the decode tiles), every layer.
 * page_stride * element size must be a multiple of 16 bytes.  Page ids are
 * host arrays of n entries, each in [0, n_pages).
 *
 * page_copy: device copy of page src_ids[i] onto dst_ids[i] (K and V) for
 * every i, enqueued on hip_stream.  Destinations must be distinct and no
 * destination may be a source of the same call (PA_ERANGE otherwise).
 *
 * page_save / page_restore: copies between pages and host memory, one
 * contiguous block per page (TensorFold pull request #2011, the author's
 * A/A comment, its list of three local fixes).  Page
 * ids[i] occupies bytes [i*P, (i+1)*P) of host_k and of host_v, P =
 * page_stride * element size; host memory should be pinned for the copies to
 * run asynchronously on hip_stream.  The caller synchronises before reading
 * saved pages or reusing restored ones. */
PA_API int page_copy(const pa_kv_cache *cache, const int32_t *src_ids, const int32_t *dst_ids,
                     int32_t n, void *hip_stream);
PA_API int page_save(const pa_kv_cache *cache, const int32_t *ids, int32_t n, void *host_k,
                     void *host_v, void *hip_stream);
PA_API int page_restore(const pa_kv_cache *cache, const int32_t *ids, int32_t n,
                        const void *host_k, const void *host_v, void *hip_stream);

/* ----------------------------------------------------------------- write_kv
 * Store new key/value rows (the step the pages call the rope stores, with
 * RoPE already applied by the caller): for each stream, rows
 * row_offset .. row_offset+n_rows-1 of k_new / v_new (bf16, device,
 * [total_rows][n_kv_heads][head_dim]) go to positions first_pos .. of the
 * stream, through its page table or into its slab.  fp8 caches quantise
 * each element as RNE_E4M3FN(clamp(fl32(x) / scale, -448, 448)) (NaN stays
 * NaN).  Streams must not write the same position twice in one call. */
PA_API int write_kv(const pa_kv_cache *cache, const pa_stream *streams, int32_t n_streams,
             const void *k_new, const void *v_new, void *hip_stream);

/* ----------------------------------------------------------------- decode
 * Split-K decode (issue #1344, "Mechanism"): each stream's keys
 * 0 .. first_pos+n_rows-1 are cut into splits of split_keys keys from
 * position 0; one partial (m, l, o) per (row, q head, split) is written to
 * the workspace, then a fixed-order log-sum-exp merge writes
 * out = v_scale * sum_j e^(m_j-M) o_j / sum_j e^(m_j-M) l_j  as bf16 (RNE).
 * The split count of a stream depends on that stream alone, so a stream's
 * output bytes do not depend on the other streams in the call.
 * Which kernel computes a stream's partials depends on that stream alone
 * too: a stream with at most 32 (row, q head) pairs per kv head (for a group
 * of 6, up to 5 rows) streams K/V from HBM into registers, one 16-column
 * MFMA tile per workgroup; a wider one (verify rows) runs on the row-tile
 * kernel, one workgroup per (split, kv head) whose LDS K/V tiles serve every
 * row and q head of the group, so each split is read from HBM once.
 * When the register-streaming workgroups of a call would take two or more
 * rounds of the device's 256 compute units, one workgroup computes several
 * consecutive splits of its stream (pa_decode_plan.narrow_splits_per_wg);
 * every split is still computed as by a workgroup of its own, so no
 * partial's bytes depend on that grouping.
 * n_rows per stream <= PA_DECODE_MAX_ROWS; sm_scale > 0 (1/sqrt(head_dim)
 * is the usual value); split_keys a positive multiple of 256.
 * The workspace (device, >= paged_attn_decode_workspace_size bytes, 256-byte
 * aligned) holds the partials; it is fully overwritten before it is read.
 * When every stream of a launch group streams through registers and has a
 * single split, the merge would weigh that split by exactly 1: the partial
 * kernel then writes out (o / l * v_scale, in the merge's operation order,
 * so the same bytes) and no merge runs; the group's workspace slots are not
 * written. */
PA_API size_t paged_attn_decode_workspace_size(const pa_stream *streams, int32_t n_streams,
                                        int32_t n_q_heads, int32_t head_dim, int32_t split_keys);

PA_API int paged_attn_decode(const pa_kv_cache *cache, const pa_stream *streams, int32_t n_streams,
                      const void *q, void *out, int32_t n_q_heads, float sm_scale,
                      int32_t split_keys, void *workspace, size_t workspace_bytes,
                      void *hip_stream);

/* The two halves of paged_attn_decode, for callers that place work
 * between them (for example partials computed on several devices for one
 * stream's key shards and gathered into one workspace before the merge).
 * paged_attn_decode_partials writes every (row, q head, split) triple of the
 * call into the workspace: m (fp32, a reference logit in log2 units), then
 * l = sum_t 2^(s_t - m) and o = sum_t 2^(s_t - m) v_t over the split's
 * visible keys t, with s_t the logit times log2(e), o (fp32 [D]) in units of
 * the stored V values (the merge applies v_scale for fp8).  m is the split's
 * largest s_t for narrow streams and lies at most 8 below it for wide ones
 * (their running maximum moves only when a logit passes it by more than 8),
 * so every term is at most 2^8.  A split wholly masked for a row stores
 * m = -inf, l = 0, o = 0.  Triple (r, h, j) of the
 * i-th stream lives at slot  S_i + (r*n_q_heads + h)*n_splits_i + j, where S_i
 * is the sum of n_rows*n_q_heads*n_splits over earlier streams; o at float
 * offset slot*head_dim, (m, l) at the second region (byte offset
 * align256(slots*head_dim*4)) as floats 2*slot and 2*slot+1.
 * paged_attn_decode_merge reads them back for the same stream descriptors
 * and split_keys and writes out.  Same validation and errors as
 * paged_attn_decode. */
PA_API int paged_attn_decode_partials(const pa_kv_cache *cache, const pa_stream *streams,
                                      int32_t n_streams, const void *q, int32_t n_q_heads,
                                      float sm_scale, int32_t split_keys, void *workspace,
                                      size_t workspace_bytes, void *hip_stream);

PA_API int paged_attn_decode_merge(const pa_kv_cache *cache, const pa_stream *streams,
                                   int32_t n_streams, void *out, int32_t n_q_heads,
                                   int32_t split_keys, const void *workspace,
                                   size_t workspace_bytes, void *hip_stream);

/* paged_attn_decode without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The partials live in a fixed
 * device array of PA_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends; the call allocates and frees
 * nothing.  Same validation, arguments and output bytes as
 * paged_attn_decode; PA_EWORKSPACE when the call's partials
 * (paged_attn_decode_workspace_size) exceed the array.  All calls on one
 * GPU share that array: calls that overlap on one GPU (from several host
 * threads, or on several HIP streams at once) race and must be serialised by
 * the caller.  The first call on a device looks the array's address up
 * (PA_EDEVICE if that fails). */
#define PA_NOALLOC_SCRATCH_BYTES (128u << 20)

PA_API int paged_attn_decode_noalloc(const pa_kv_cache *cache, const pa_stream *streams,
                                     int32_t n_streams, const void *q, void *out,
                                     int32_t n_q_heads, float sm_scale, int32_t split_keys,
                                     void *hip_stream);

/* Launch plan of a decode call, for callers that size grids or check
 * scheduling: per stream its split count (splits_out, n_streams entries, may
 * be NULL), and the totals.  kv_dtype (pa_kv_dtype) selects the kernels the
 * block counts refer to; split counts and workspace size do not depend on
 * it.  Host only; validates like paged_attn_decode minus the device
 * pointers. */
typedef struct pa_decode_plan {
  int32_t n_launch_groups;   /* launch groups (streams are grouped, at most 32 a group) */
  int32_t total_splits;      /* sum over streams of their split counts */
  int32_t col_tiles;         /* 16-column MFMA tiles per (split, kv head), narrow streams */
  int32_t partial_blocks;    /* workgroups of all partial kernels */
  int32_t merge_blocks;      /* workgroups of the merge kernel(s) */
  int32_t wide_blocks;       /* of partial_blocks: those of the LDS-shared row-tile kernel */
  int32_t narrow_splits_per_wg; /* consecutive splits a register-streaming workgroup computes
                                   (largest over launch groups; 0 when there is none) */
  size_t workspace_bytes;
} pa_decode_plan;

PA_API int paged_attn_decode_plan(const pa_stream *streams, int32_t n_streams, int32_t n_q_heads,
                           int32_t n_kv_heads, int32_t head_dim, int32_t split_keys,
                           int32_t kv_dtype, int32_t *splits_out, pa_decode_plan *plan);

/* ----------------------------------------------------------------- prefill
 * Prompt-chunk prefill (pull request #1373, prompt rows; pull request #2011,
 * hpattn_p256_kernel): every row of every stream, causal against the
 * stream's stored prefix, one launch, page size 256 fixed.  A workgroup
 * covers a tile of a stream's rows for some q heads of one kv head (tiles
 * never span streams); a row's bytes do not depend on which other rows
 * share its tile, so any slicing of a stream's rows into calls gives the
 * same bytes as one call.
 *
 * Finite inputs: this kernel (also the one behind the partials of bf16
 * decode streams with more than a few rows) is built without NaN semantics.
 * Q, the scales, and K and V at every key a row sees must be finite; a NaN
 * or infinity there leaves that row's output unspecified (not necessarily
 * NaN).  Keys a row does not see, and slots past the stream's context, may
 * hold anything, NaN codes included: they are replaced by selects before
 * any arithmetic.  A rejected page id still poisons its rows with NaN bit
 * patterns (written as integers). */
PA_API int paged_attn_prefill(const pa_kv_cache *cache, const pa_stream *streams, int32_t n_streams,
                       const void *q, void *out, int32_t n_q_heads, float sm_scale,
                       void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
