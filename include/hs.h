/*
 * hs.h -- C ABI of the MI355X (gfx950) HiSparse hot-path library (libhs.so).
 *
 * What the library does (HiSparse paper abstract, arXiv 2608.07009; "HiSparse"
 * note, sections 2 and 3): every request keeps its full KV history in pinned
 * host memory and only a fixed number B of device slots per layer in HBM.  At
 * each decode step and layer, the top-k token selection of a sparse-attention
 * indexer is resolved against that buffer -- hit detection through a
 * token->slot page table, LRU replacement among the slots not selected in the
 * step, page-table and recency update, host-to-device fetch of the missing
 * rows -- and a sparse MLA decode attention then reads only the resolved slots.
 * The exact replacement rule (the pages say "LRU"): a slot's recency stamp is
 * the step at which it was last selected (a fill counts as a selection); the
 * candidates for a step are the slots holding no token selected in that step,
 * least recent first, ties to the lower slot index; missing tokens are served
 * in ascending token order, the i-th missing token taking the i-th candidate.
 *
 * Page-granular selections (paper abstract: the method serves the NSA and Quest
 * families, whose indexers select blocks of consecutive tokens): with
 * hs_config.page_tokens = P > 1 the cached unit is a page of P consecutive
 * tokens (page c = tokens cP .. cP + P - 1).  Selections, top_k,
 * device_buffer_size, capacity and the page table then count pages, a slot holds
 * the P rows of its page in position order, a miss fetches the whole page, and
 * the same replacement rule applies with "page" for "token".  The host history
 * stays one row per token (hs_host_kv, hs_offload), and hs_attend /
 * hs_attend_pages read every token of the resolved pages.
 *
 * Conventions for every function:
 *   - device pointers ("d_" prefix) are HIP device addresses; host pointers are
 *     ordinary process addresses;
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream);
 *   - argument errors are detected on the host and returned before any device
 *     work is queued; nothing is written in that case;
 *   - hs_resolve and hs_attend only enqueue kernels: they never allocate, copy
 *     synchronously or synchronise, so they may be captured in a hipGraph;
 *   - a handle is not thread-safe; calls on one handle must be serialised by
 *     the caller.
 */
#ifndef HS_H
#define HS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hs_status {
  HS_OK = 0,
  HS_ERR_INVALID_ARG = 1,   /* bad configuration or call argument (message: hs_last_error_message) */
  HS_ERR_OUT_OF_MEMORY = 2, /* a host or device allocation failed */
  HS_ERR_UNSUPPORTED = 3,   /* valid request the library does not implement (e.g. no attention heads) */
  HS_ERR_HIP = 4,           /* a HIP runtime call failed (message has the HIP error string) */
  HS_ERR_DEVICE = 5         /* the device flagged invalid input (see hs_get_device_error) */
} hs_status;

/* KV entry layouts (bytes per token).  Rows are stored as given, byte for byte. */
typedef enum hs_kv_layout {
  HS_KV_BF16_576 = 0,   /* 576 bf16: 512 latent + 64 rope                                  = 1152 B */
  HS_KV_FP8_MLA_656 = 1 /* 512 E4M3FN latent codes, 4 fp32 scales (one per 128 latent
                           values), 64 bf16 rope                                            =  656 B */
} hs_kv_layout;

/* Handle flags (hs_config.flags). */
#define HS_FLAG_NO_IO 0x1u /* resolve updates every table but moves no row: measures the
                              resolution cost alone (the paper's no-IO oracle); no host
                              pool is allocated (hs_host_bytes reports 0, hs_host_kv and
                              hs_offload return HS_ERR_UNSUPPORTED) */
#define HS_FLAG_ATTN_OUT_F32 0x2u /* hs_attend / hs_attend_pages write fp32 output, with P
                                     carried in fp32 through the P V product (the 1e-5 tier)
                                     instead of rounded to bf16 */
#define HS_FLAG_RESIDENT_TAIL 0x4u /* 656-byte token rows only (HS_KV_FP8_MLA_656, page_tokens
                                      0 or 1, not with HS_FLAG_NO_IO).  The host pool keeps the
                                      first 640 bytes of each row, at a 640-byte stride, so a row
                                      read over the host link covers five whole 128-byte lines
                                      instead of six; the last 16 bytes of every row (the last 8
                                      rope values) stay in a device-resident tail plane
                                      (hs_state_view.tail_plane, 16 bytes per token of history,
                                      [max_requests][capacity] per layer, part of
                                      hs_device_bytes).  Misses are assembled from both into the
                                      slot, so slot rows, tables and attention are those of the
                                      packed layout; hs_host_kv reports the 640-byte stride, and
                                      hs_append / hs_offload write both parts.  Callers that
                                      write history rows themselves write the tails into the
                                      plane.  Cost: 16 bytes of HBM per token of history (2.4 %
                                      of the rows).  Measured on 256 requests of fp8 rows: the
                                      fused resolve with its row copies 16 % shorter (387 against
                                      461 us per step). */

/*
 * Eviction policies.  LRU is the method (paper abstract; note, section 2); the others exist
 * for the policy study the note describes (section 3: LRU is steadier than a policy that does
 * not exploit locality).
 *   HS_EVICT_LRU     candidates by (stamp of last selection, slot)
 *   HS_EVICT_FIFO    candidates by (stamp of the fill, slot): a hit does not refresh a slot
 *   HS_EVICT_RANDOM  the non-hit slots in slot order; the i-th miss (ascending token) takes
 *                    candidate perm(i), perm a pseudo-random permutation of the candidate
 *                    ranks: a 4-round Feistel network on 2h-bit values (4^h the smallest
 *                    power of four >= the candidate count), round i XORing the left half
 *                    with the low h bits of SplitMix64 output (i << 32 | right half) under
 *                    key = SplitMix64 output ((request * layers + layer) << 32 | step) of
 *                    eviction_seed, re-encrypting values outside the range (cycle walking).
 *                    Stamps follow LRU; lru_order is not maintained; hs_append is
 *                    unsupported.
 */
typedef enum hs_eviction { HS_EVICT_LRU = 0, HS_EVICT_FIFO = 1, HS_EVICT_RANDOM = 2 } hs_eviction;

/* Device error bits, accumulated (OR) until read by hs_get_device_error. */
#define HS_DEVERR_TOKEN_RANGE 0x1 /* a selected token outside [0, capacity) and not -1 */
#define HS_DEVERR_DUPLICATE 0x2   /* a token selected twice in one row */

/*
 * Configuration.  top_k, device_buffer_size and host_to_device_ratio are the
 * three tuning parameters the note names (section 3); the host capacity per
 * (request, layer) is host_to_device_ratio * device_buffer_size tokens.
 */
typedef struct hs_config {
  int32_t top_k;                /* k: selections per request and step, >= 1                  */
  int32_t device_buffer_size;   /* B: device slots per (request, layer), B >= top_k           */
  int32_t host_to_device_ratio; /* >= 1; capacity = ratio * B tokens (pages) of history      */
  int32_t max_requests;         /* request slots 0..max_requests-1                           */
  int32_t num_layers;           /* layers, each with its own buffer and tables               */
  int32_t layout;               /* hs_kv_layout                                              */
  int32_t num_heads;            /* query heads for hs_attend (0: resolve only), <= 16        */
  uint32_t flags;               /* HS_FLAG_*                                                 */
  void* device_mem;             /* optional caller-owned device block of hs_device_bytes()
                                   bytes, 256-byte aligned; NULL: the library allocates     */
  size_t device_mem_bytes;      /* size of device_mem                                        */
  int32_t eviction;             /* hs_eviction; 0 = LRU                                      */
  uint64_t eviction_seed;       /* HS_EVICT_RANDOM: key of its permutation                   */
  int32_t page_tokens;          /* tokens per cached unit: 0 or 1 = token-granular; P > 1, a
                                   power of two <= 256, = pages of P tokens (see above);
                                   with num_heads > 0, top_k * P <= 65536                    */
} hs_config;

typedef struct hs_handle hs_handle;

/* Device-side state of one layer; all pointers are device addresses owned by the handle. */
typedef struct hs_state_view {
  int32_t* page_table;   /* [max_requests][capacity] token (page) -> slot, -1 = not resident */
  int32_t* slot_owner;   /* [max_requests][B] slot -> token (page), -1 = empty         */
  int32_t* slot_stamp;   /* [max_requests][B] step of last selection, -1 = never       */
  int32_t* lru_order;    /* [max_requests][B] slots sorted by (stamp, slot) ascending  */
                         /* (not maintained under HS_EVICT_RANDOM)                     */
  int32_t* step;         /* [max_requests] resolves done so far (the next stamp)        */
  uint8_t* kv_buffer;    /* per request (request_stride bytes apart): B slot rows of    */
                         /* slot_stride bytes, then one row of zeros the attention     */
                         /* kernel reads for padded selection entries (never written)  */
  int64_t capacity;      /* page-table entries per (request, layer): tokens, or pages    */
  int64_t slot_stride;   /* bytes between slots in kv_buffer (page_tokens * entry_bytes) */
  int64_t entry_bytes;   /* bytes of one token's KV entry                               */
  int64_t request_stride; /* bytes between requests in kv_buffer ((B + 1) * slot_stride) */
  int64_t page_tokens;   /* tokens per slot (1 = token-granular)                        */
  uint32_t* fresh_slots; /* [max_requests][(B + 31) / 32] bits: slots appended since the  */
                         /* last resolve (their stamp is already the next step's)        */
  uint8_t* tail_plane;   /* HS_FLAG_RESIDENT_TAIL: [max_requests][capacity][tail_bytes], the */
                         /* last tail_bytes bytes of each history row; NULL otherwise     */
  int64_t tail_bytes;    /* 16 with HS_FLAG_RESIDENT_TAIL, else 0                         */
} hs_state_view;

/* Bytes the device block must have for this configuration (0 and an error if invalid). */
hs_status hs_device_bytes(const hs_config* cfg, size_t* bytes);

/* Bytes of the pinned host pool for this configuration (0 with HS_FLAG_NO_IO). */
hs_status hs_host_bytes(const hs_config* cfg, size_t* bytes);

/*
 * Create a handle: validates cfg (B >= top_k, ratio >= 1, known layout, sizes
 * without overflow, tables within the resolver's on-chip limits) before any HIP
 * call, then allocates the pinned host pool (hipHostMalloc, mapped) and the
 * device state, and sets every request to the empty state (no token resident,
 * all stamps -1, step 0).  On error *out is NULL.
 */
hs_status hs_create(const hs_config* cfg, hs_handle** out);

/*
 * Resolve one layer's selections for requests 0..n_req-1 (paper abstract:
 * hit detection, LRU replacement and host-to-device fetch for each layer's
 * selections; note, section 3: identify the misses, pick LRU victims, update
 * the page table, pull the rows from host memory).
 *   d_sel   [n_req][top_k] int32 token positions, -1 = padding
 *   d_slots [n_req][top_k] int32 out: slot now holding d_sel[r][i], -1 for padding or
 *           rejected entries
 *   d_miss  [n_req] int32 out: number of rows fetched for the request, or NULL
 * Ends with every selected token resident and its row in kv_buffer (unless
 * HS_FLAG_NO_IO).  Entries outside [0, capacity) or repeated in a row are
 * skipped (slot -1) and set the device error word; the library never reads or
 * writes outside its tables.  Ordering: resolve(l, t) must complete before
 * attend(l, t) and attend(l, t) before resolve(l, t+1) on the caller's streams;
 * different layers may run concurrently.
 */
hs_status hs_resolve(hs_handle* h, int32_t layer, int32_t n_req, const int32_t* d_sel, int32_t* d_slots,
                     int32_t* d_miss, void* stream);

/*
 * hs_resolve in two halves, for schedulers that overlap the host-to-device copy with other
 * work (layer-wise prefetch runs the copies of later layers beside the attention of earlier
 * ones).  hs_resolve_tables does everything hs_resolve does except moving rows, and records
 * each request's miss list (token, slot) in the handle; hs_fetch_misses then copies those
 * rows with a kernel of 128 small workgroups that keeps the link busy beside other work (each
 * workgroup reserves 96 KiB of LDS it does not use, so that attention workgroups run on the
 * other compute units rather than at the pace of the copy's host reads).  The pair must run
 * in this order on the caller's streams,
 * with no other resolve of the same layer in between; together they equal hs_resolve.
 * hs_fetch_misses returns HS_ERR_INVALID_ARG (and enqueues nothing) unless the layer's last
 * resolve, append or reset call was an hs_resolve_tables of at least n_req requests: other
 * calls change the tables, and copying an older miss list would write rows into slots that
 * now belong to other tokens.  With HS_FLAG_NO_IO, hs_fetch_misses enqueues nothing.
 */
hs_status hs_resolve_tables(hs_handle* h, int32_t layer, int32_t n_req, const int32_t* d_sel, int32_t* d_slots,
                            int32_t* d_miss, void* stream);
hs_status hs_fetch_misses(hs_handle* h, int32_t layer, int32_t n_req, void* stream);

/*
 * Write-through append of newly generated tokens (the note's introduction: KV not in use is
 * actively offloaded to host memory; paper abstract: each request's full KV history lives in
 * host memory).  For each request r < n_req with d_pos[r] >= 0:
 *   - the row at d_rows + r * row_stride (entry_bytes bytes, device memory) is written to
 *     position d_pos[r] of the request's history in the host pool (with
 *     HS_FLAG_RESIDENT_TAIL its last 16 bytes to the tail plane);
 *   - the token becomes resident before the next resolve: it keeps its slot if it has one,
 *     otherwise it takes the first slot in (stamp, slot) order -- empty slots first -- whose
 *     token leaves the page table; the slot's bytes become the row and its stamp the step
 *     number the next resolve will use (the step counter does not move).
 *   d_pos      [n_req] int32 token positions, -1 = no token for this request
 *   d_rows     device rows, 16-byte aligned; row_stride >= entry bytes, a multiple of 16
 *   d_slot_out [n_req] int32 out: the slot now holding the token (-1 if none), or NULL
 * A position outside [0, capacity) is skipped and sets HS_DEVERR_TOKEN_RANGE.  With
 * HS_FLAG_NO_IO the tables change but no row moves.  Enqueue-only, graph-capturable.
 * A selection that names the token in the next resolve finds it resident (a hit).
 * HS_ERR_UNSUPPORTED under HS_EVICT_RANDOM (token-granular handles).
 * With page_tokens = P > 1 the append writes through only: the row goes to the history and,
 * when its page d_pos[r] / P is resident, into that page's slot at row offset d_pos[r] mod P;
 * no table changes (a page that is not resident arrives whole, new row included, when a
 * selection names it), and d_slot_out gets the page's slot or -1.  Any eviction policy.
 */
hs_status hs_append(hs_handle* h, int32_t layer, int32_t n_req, const int32_t* d_pos, const void* d_rows,
                    int64_t row_stride, int32_t* d_slot_out, void* stream);

/*
 * Top-k selection from indexer scores, the step that feeds hs_resolve (the note, section 2:
 * the backend's indexer decides the selected set; paper abstract: indexer-agnostic).  For
 * each request r < n_req, among positions 0 .. d_len[r]-1 of its score row (fp32, row r at
 * d_scores + r * score_stride), the top_k positions of largest score, a tie going to the
 * smaller position, are written to d_sel[r][0 .. top_k) in ascending position order; when
 * d_len[r] < top_k every position is selected and the row is padded with -1.  The output is
 * a valid hs_resolve selection.
 *   d_scores  16-byte aligned; score_stride a multiple of 4, >= every d_len[r]; no NaN
 *   d_len     [n_req] int32 in [0, min(capacity, score_stride, 2^18)]; otherwise the row is
 *             all -1 and HS_DEVERR_TOKEN_RANGE is set
 *   d_sel     [n_req][top_k] int32 out
 * Enqueue-only, graph-capturable; touches no table.
 */
hs_status hs_topk(hs_handle* h, int32_t n_req, const float* d_scores, int64_t score_stride, const int32_t* d_len,
                  int32_t* d_sel, void* stream);

/*
 * hs_topk for a decode loop: the same selection, computed with one pass over the score row
 * instead of two when a guess of where the k-th largest score lies is right.  Consecutive
 * steps of a request and layer have nearly the same scores (the note, section 2: the indexer
 * scores every token at every step), so the previous call's result is such a guess.
 *   d_hint  [n_req] int32 in/out: in, the value this call wrote for the same request and layer
 *           at the previous step (or -1: no guess); out, the value for the next call (-1 when
 *           len[r] <= top_k or the row is rejected).  It is the top 12 bits of the k-th largest
 *           score's order key (scores mapped to 32-bit keys whose unsigned order is the float
 *           order, -0 joined with +0); a guess g is used when that score's 12-bit digit lies
 *           within g - 1 .. g + 1, and otherwise costs one extra pass over the row.
 * d_sel is bit for bit that of hs_topk for any d_hint contents.  HS_ERR_INVALID_ARG for a
 * NULL d_hint; other arguments as hs_topk.  Enqueue-only, graph-capturable.
 */
hs_status hs_topk_hinted(hs_handle* h, int32_t n_req, const float* d_scores, int64_t score_stride,
                         const int32_t* d_len, int32_t* d_sel, int32_t* d_hint, void* stream);

/*
 * Prefill offload: copies count rows (device memory, row_stride bytes apart) into positions
 * first .. first + count - 1 (token positions, also with pages) of request `request`'s
 * history in the host pool (the note's
 * introduction: KV is actively offloaded to host memory).  Device tables are untouched: the
 * tokens arrive on the device as misses when a selection names them.  Stream-ordered: one
 * flat device-to-host copy when row_stride equals the entry size, a zero-copy store kernel
 * for 16-byte-aligned padded rows, a 2-D copy otherwise.  With HS_FLAG_RESIDENT_TAIL each
 * row's last 16 bytes go to the tail plane instead (the store kernel for 16-byte-aligned
 * rows, else two 2-D copies).  HS_ERR_INVALID_ARG for a range
 * outside [0, capacity * page_tokens) or row_stride < entry bytes.
 */
hs_status hs_offload(hs_handle* h, int32_t layer, int32_t request, int64_t first, int64_t count,
                     const void* d_rows, int64_t row_stride, void* stream);

/*
 * Sparse MLA decode attention over the resolved slots (paper abstract: each
 * step reads only the selected KV entries; only placement changes, so the
 * result equals attention over the selected tokens of the full history).
 *   d_q     [n_req][num_heads][576] bf16 queries (512 latent + 64 rope)
 *   d_slots [n_req][top_k] int32 slots from hs_resolve (-1 entries skipped)
 *   scale   softmax scale applied to q.K
 *   d_out   [n_req][num_heads][512] bf16 (fp32 with HS_FLAG_ATTN_OUT_F32):
 *           sum_j softmax_j(scale q.K_j) V_j, with K_j all 576 decoded values of
 *           slot j and V_j its first 512
 *   d_lse   [n_req][num_heads] fp32 log-sum-exp of the scaled scores, or NULL
 * A row with no valid slot gives out = 0 and lse = -inf.  HS_ERR_UNSUPPORTED
 * when the handle was created with num_heads = 0.  With page_tokens = P > 1,
 * d_slots holds page slots and the attended tokens are the P rows of each valid
 * page slot (top_k * P tokens).
 */
hs_status hs_attend(hs_handle* h, int32_t layer, int32_t n_req, const void* d_q, const int32_t* d_slots,
                    float scale, void* d_out, float* d_lse, void* stream);

/*
 * hs_attend cut at each request's context length, for page-granular selections whose last
 * page is partly written (paper abstract: NSA and Quest select blocks of tokens; a block past
 * the newest token holds no KV yet).  Token o of the i-th selected page takes part iff its
 * page slot is valid, d_sel[r][i] >= 0 and d_sel[r][i] * page_tokens + o < d_len[r].
 *   d_sel   [n_req][top_k] int32, the selection d_slots was resolved from
 *   d_len   [n_req] int32 context length in tokens
 * Other arguments and errors as hs_attend; valid for token-granular handles too.
 */
hs_status hs_attend_pages(hs_handle* h, int32_t layer, int32_t n_req, const void* d_q, const int32_t* d_slots,
                          const int32_t* d_sel, const int32_t* d_len, float scale, void* d_out, float* d_lse,
                          void* stream);

/*
 * Measurement helper, not a step of the method: a dense streaming read of `bytes` bytes of
 * device memory at d_src (16-byte aligned, bytes a multiple of 16), enqueued on `stream`.
 * Timing it gives the HBM read rate the attention and resolver kernels are compared with.
 * d_sink: one device uint32 that the kernel may overwrite (it keeps the loads alive).
 * HS_ERR_INVALID_ARG for NULL pointers or misaligned sizes; no allocation, no sync.
 */
hs_status hs_stream_read(const void* d_src, size_t bytes, uint32_t* d_sink, void* stream);

/*
 * hs_attend for callers that cannot allocate device memory (code under graph capture, tight
 * serving loops, harnesses that forbid hipMalloc), also on handles created with
 * num_heads = 0, which reserve no attention partials: the same computation and kernels as
 * hs_attend with num_heads (1..16) query heads per call, the split partials of requests
 * spread over several workgroups kept in a static device array of 256 partials (8.4 MB),
 * one copy per GPU, held until the process ends, instead of the handle's block.  Its address
 * on the handle's device is resolved when the handle is created.  Allocates nothing.
 *   d_q, d_slots, scale, d_out, d_lse   as hs_attend, with num_heads in place of the handle's
 * HS_ERR_UNSUPPORTED when the launch would need more than 256 partials: it needs n_req x s
 * of them when hs_attend would spread each request over s > 1 workgroups (s = 256 / n_req,
 * at most 16 and at most tokens / 64, at least tokens / 2048 for fp8 rows and tokens / 1024
 * for bf16 rows, tokens = top_k x page_tokens), none when s = 1.  The handle's own partials
 * are untouched.
 * Calls that overlap on one GPU -- on any handle -- race on the shared array.
 */
hs_status hs_attend_noalloc(hs_handle* h, int32_t layer, int32_t n_req, int32_t num_heads, const void* d_q,
                            const int32_t* d_slots, float scale, void* d_out, float* d_lse, void* stream);

/*
 * A step's attention split by residency, so that the attention of the selected tokens
 * already in the device buffer runs while the misses are still being copied in (paper
 * abstract: host-device IO is the only price of bounded residency; the note, section 3:
 * the missing KV is pulled from host memory before the step can attend).  The two parts
 * together equal hs_attend (or hs_attend_pages, with d_len) over the same slots, up to the
 * order in which fp32 partial sums are merged.  Order on the caller's streams:
 *   hs_resolve_tables(l)  ->  { hs_attend_resident(l)  ||  hs_fetch_misses(l) }  ->  hs_attend_fetched(l)
 * with no other resolve, attend part or append of layer l in between.
 * hs_attend_resident attends the entries of d_slots (from that hs_resolve_tables) whose slot
 * is not one of the step's victims -- those rows are resident and the copy does not touch
 * them -- and leaves split partials in the handle; it reads the handle's miss list.
 * hs_attend_fetched attends the step's misses (the rows hs_fetch_misses copied), merges them
 * with the resident partials in a fixed order and writes d_out / d_lse as hs_attend does.
 *   d_sel, d_len  both NULL (no cut), or as hs_attend_pages (the fetched part takes each
 *                 miss's unit from the miss list and needs only d_len, the same array)
 * Other arguments, outputs and errors as hs_attend; HS_ERR_UNSUPPORTED with HS_FLAG_NO_IO
 * (no rows are copied, so there is nothing to overlap); HS_ERR_INVALID_ARG when the layer's
 * last resolve, append or reset call was not an hs_resolve_tables of at least n_req requests
 * (the handle tracks the order of the calls, not of the device work).  hs_attend_fetched
 * also returns HS_ERR_INVALID_ARG unless an hs_attend_resident of the same layer and the same
 * n_req came after that hs_resolve_tables with no hs_attend / hs_attend_pages of the layer in
 * between (they reuse the space of the resident partials).  Enqueue-only, graph-capturable.
 */
hs_status hs_attend_resident(hs_handle* h, int32_t layer, int32_t n_req, const void* d_q, const int32_t* d_slots,
                             const int32_t* d_sel, const int32_t* d_len, float scale, void* stream);
hs_status hs_attend_fetched(hs_handle* h, int32_t layer, int32_t n_req, const void* d_q, const int32_t* d_len,
                            float scale, void* d_out, float* d_lse, void* stream);

/*
 * Wait for the work this handle's calls enqueued (not for the rest of the device) and free
 * everything the handle owns.  NULL is accepted.  Work the caller captured into a graph runs
 * on whatever stream the graph is launched on, which the handle never sees: the caller
 * waits for such replays before destroying the handle.
 */
hs_status hs_destroy(hs_handle* h);

/*
 * Host rows of (layer, request): *ptr = first of `*capacity` token rows (the
 * page-table capacity times page_tokens), `*row_stride` bytes apart, in pinned
 * memory owned by the handle (valid until hs_destroy).  With HS_FLAG_RESIDENT_TAIL a
 * host row is the row's first 640 bytes (row_stride 640) and the rest is in the tail
 * plane.
 * The caller writes a token's row before any selection names it, directly or
 * through hs_offload / hs_append; resolves read it for misses.
 * HS_ERR_UNSUPPORTED with HS_FLAG_NO_IO (no host pool).
 */
hs_status hs_host_kv(hs_handle* h, int32_t layer, int32_t request, void** ptr, int64_t* capacity,
                     int64_t* row_stride);

/* Device pointers of one layer's tables and slot buffer.  Together with the host rows
 * (hs_host_kv) they are the whole state carried from one step to the next: copying them
 * into another handle of the same configuration, between steps, resumes the run there. */
hs_status hs_device_state(hs_handle* h, int32_t layer, hs_state_view* view);

/* Return requests first..first+count-1 of every layer to the empty state (enqueued on stream). */
hs_status hs_reset_requests(hs_handle* h, int32_t first, int32_t count, void* stream);

/*
 * Wait for the work this handle's calls enqueued (as hs_destroy; graph replays are the
 * caller's to wait for), then return the accumulated HS_DEVERR_* bits in *bits and clear
 * them.  Other streams of the process are not synchronised.
 */
hs_status hs_get_device_error(hs_handle* h, int32_t* bits);

/* Static description of a status code. */
const char* hs_status_string(hs_status s);

/* Message of the last failed call on this thread ("" if none). */
const char* hs_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* HS_H */
