/*
 * g4attn -- Gemma-4-style attention over a device-resident KV cache on
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * Sources of the operations (cited by page title and section):
 *   [FR]   "Porting Gemma-4 (2B / 4B / 12B) to AWS Inferentia2": introduction
 *          table (sliding + global layers, head counts, windows); 2.1
 *          (cross-layer KV-sharing: shared layers read an earlier owner's K/V
 *          and hold no cache); 2.2 (GQA: each KV head serves a contiguous group
 *          of query heads); 2.3 (12B mixed attention types); 4 (the in-place
 *          masked write of the new token's K/V); 5 (KV cache resident on the
 *          device, filled by a prefill graph and read by a decode graph).
 *   [12B]  "Gemma-4 12B on AWS Inferentia2 -- Tensor-Parallel (TP=2), device
 *          prefill": "Why this is its own port" (global layers: one KV head,
 *          head_dim 512, K reused as V; sliding window 1024) and "The recipe"
 *          (a 64-token prefill bucket and a 1-token decode bucket sharing one
 *          resident cache).
 *   [E4B]  "Gemma-4-E4B-it on AWS Inferentia2 -- Tensor-Parallel (TP=2)":
 *          "Limitations" (single-stream batch-1 decode: neither continuous
 *          batching nor a paged KV cache).
 *
 * Conventions for every call:
 *   - Return value: G4ATTN_OK (0) or a negative G4ATTN_ERR_* code.  On error
 *     nothing is launched and nothing is written; g4attn_last_error() gives a
 *     message (thread-local, valid until the next call on that thread).
 *     No C++ exception or abort crosses this ABI.
 *   - Device pointers (q, k, v, out, length arrays, cache, workspace) are
 *     owned by the caller.  The library owns only the host-side plan.
 *   - Compute calls are asynchronous on the given HIP stream (hipStream_t
 *     passed as void*; NULL = the default stream) and never synchronize.
 *     They allocate nothing, so they may be captured into a HIP graph.
 *   - Tensors are dense, row-major, bf16 (IEEE binary32's upper 16 bits), and
 *     16-byte aligned.  Length / position arrays are int32 on the device.
 *   - Device length arrays must respect the host-side hints passed with them.
 *     The kernels clamp each length or start position to its hint (and every
 *     cache access into the cache), so a violation gives wrong numbers for
 *     that sequence, never an out-of-bounds access, and leaves no state that
 *     affects later calls.
 *   - Calls that use one stack's workspace (decode, prefill) must be ordered
 *     on one stream; calls on different streams that touch disjoint cache
 *     regions and different workspaces are safe.
 */
#ifndef G4ATTN_H
#define G4ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define G4ATTN_OK 0
#define G4ATTN_ERR_NULL -1         /* a required pointer is NULL */
#define G4ATTN_ERR_DESC -2         /* invalid layer descriptor or stack size */
#define G4ATTN_ERR_OWNER -3        /* invalid kv_owner_layer */
#define G4ATTN_ERR_SHARED_LAYER -4 /* append on a KV-shared layer */
#define G4ATTN_ERR_RANGE -5        /* layer, batch, length or position out of range */
#define G4ATTN_ERR_UNBOUND -6      /* cache / workspace not bound */
#define G4ATTN_ERR_UNSUPPORTED -7  /* head_dim or size the kernels do not build */
#define G4ATTN_ERR_HIP -8          /* a HIP runtime call failed */

/*
 * Per-layer attention geometry.
 *   n_q_heads, n_kv_heads: n_q_heads % n_kv_heads == 0; query head h reads KV
 *       head h / (n_q_heads / n_kv_heads) ([FR] 2.2, contiguous groups).
 *   head_dim: 32, 64, 128, 256 or 512 ([12B]: 256 sliding, 512 global).
 *   window: 0 = global causal; W > 0 = a query at position p sees keys
 *       p - W < k <= p ([FR] introduction table: sliding windows 512/1024;
 *       the window counts the query's own key).
 *   k_eq_v: 1 = values are the cached key rows; the layer has no V plane
 *       ([12B] "Why this is its own port").
 *   kv_owner_layer: -1 or the layer's own index = the layer owns a cache;
 *       otherwise an earlier layer that owns its cache and has equal
 *       (n_kv_heads, head_dim, k_eq_v, window).  The layer then reads that
 *       cache and writes none ([FR] 2.1).
 *   scale: multiplies q.k before the softmax; must be finite.
 *   softcap: attention-logit cap c.  0 = none; c > 0 replaces each scaled
 *       score s by c * tanh(s / c) before the softmax (an attention softcap
 *       is one of the recipe's pieces on the E4B Inferentia2 model card,
 *       "Architecture", which gives no value; the c * tanh(x / c) form is the
 *       one the pages give for Gemma-4's final-logit cap).  Must be 0, or
 *       finite and positive with scale / c finite in fp32 (G4ATTN_ERR_DESC
 *       otherwise).  A KV-shared layer uses its own cap, like its scale.
 */
typedef struct g4attn_layer_desc {
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t window;
  int32_t k_eq_v;
  int32_t kv_owner_layer;
  float scale;
  float softcap;
} g4attn_layer_desc;

typedef struct g4attn_stack g4attn_stack; /* opaque, host-side plan */

/*
 * Validate the descriptors, resolve owners ([FR] 2.1: a KV-shared layer names
 * an earlier owning layer) and plan the one resident cache ([FR] 5: a fixed
 * buffer on the device, sized once for the largest context).  Host only; no
 * HIP call.  max_batch: sequences per call; kv_max: positions per sequence
 * (every position < kv_max); max_chunk: new tokens per append/prefill call.
 * Errors: G4ATTN_ERR_NULL, _DESC, _OWNER, _UNSUPPORTED.  *out is set only on
 * success and must be released with g4attn_stack_destroy.
 */
int32_t g4attn_stack_create(const g4attn_layer_desc* layers, int32_t n_layers,
                            int32_t max_batch, int32_t kv_max, int32_t max_chunk,
                            g4attn_stack** out);
void g4attn_stack_destroy(g4attn_stack* stack);

/*
 * Cache layout ([FR] 5: one static buffer per owning layer; [FR] 2.1: only
 * owning layers allocate).  Each owning layer gets a K plane and, unless
 * k_eq_v, a V plane, each max_batch x n_kv_heads segments of cap x head_dim
 * bf16, 256-byte aligned.  cap is a multiple of 64: roundup64(kv_max) for
 * global layers and min(roundup64(kv_max), roundup64(window + max_chunk - 1))
 * for sliding ones (a ring: enough for a window plus one chunk of new tokens,
 * independent of context length).  Position p lives in slot p mod cap.
 * Within a segment the rows are stored in matrix-core operand order, so that
 * each 16-key (K) or 32-key (V) block is contiguous and every kernel load is a
 * contiguous 1 KiB per wavefront; g4attn_kv_offset gives the byte offset of
 * any element.  Shared layers get no planes.
 * g4attn_cache_bytes: bytes of the single cache buffer to pass to bind.
 * g4attn_workspace_bytes: bytes of device scratch for split partial results
 *   and arrival counters.  The workspace must be zero-filled once before the
 *   first compute call; the kernels leave the counters at zero afterwards.
 */
int32_t g4attn_cache_bytes(const g4attn_stack* stack, uint64_t* bytes);
int32_t g4attn_workspace_bytes(const g4attn_stack* stack, uint64_t* bytes);

/* Attach caller-owned device buffers (256-byte aligned): the resident cache
 * that every prefill and decode call of the stack reads and appends write
 * ([FR] 5: one device buffer filled by the prefill graph and read by the
 * decode graph, never copied back to the host) and the workspace.  Host only.
 * Errors: G4ATTN_ERR_NULL, G4ATTN_ERR_RANGE (misaligned). */
int32_t g4attn_bind(g4attn_stack* stack, void* cache, void* workspace);

/* Host-side lookups, bit-exact with what the kernels do (test hooks). */
/* Layer whose cache `layer` reads ([FR] 2.1). */
int32_t g4attn_resolve_owner(const g4attn_stack* stack, int32_t layer, int32_t* owner);
/* Slots per (sequence, KV head) of the cache `layer` reads: the full context
 * on global layers, a window-plus-chunk ring on sliding ones ([FR]
 * introduction table: sliding windows of 512 / 1024 positions; [12B] "Why
 * this is its own port": window 1024). */
int32_t g4attn_layer_capacity(const g4attn_stack* stack, int32_t layer, int32_t* cap);
/* Keys [lo, hi) visible to a query at q_pos when n_keys positions exist:
 * hi = min(q_pos + 1, n_keys) (causal); lo = max(0, q_pos - window + 1) on a
 * sliding layer, else 0 ([FR] introduction table: sliding vs global layers
 * and their windows). */
int32_t g4attn_key_range(const g4attn_stack* stack, int32_t layer, int64_t q_pos,
                         int64_t n_keys, int64_t* lo, int64_t* hi);
/* Byte offsets in the cache of element d of the K row and of the V row
 * (== the K element when k_eq_v, [12B] "Why this is its own port": K reused
 * as V) of (sequence b, KV head, position pos) read by `layer` (the owner's
 * planes, [FR] 2.1).  Errors: _NULL, _RANGE, _UNSUPPORTED (paged stack). */
int32_t g4attn_kv_offset(const g4attn_stack* stack, int32_t layer, int32_t b, int32_t kv_head,
                         int64_t pos, int32_t d, int64_t* off_k, int64_t* off_v);

/*
 * Write new K (and V) rows into the owning layer's planes ([FR] 4 and 5: the
 * new token's K/V is written in place into the resident cache).
 *   k, v: [batch][n_new][n_kv_heads][head_dim] bf16; v must be NULL when
 *         k_eq_v (the V role is played by K) and non-NULL otherwise.
 *   start_pos: int32[batch], position of row 0 of each sequence.
 *   n_valid: int32[batch] or NULL; rows t >= n_valid[b] are skipped (ragged
 *         appends); NULL means all n_new rows.
 *   max_end_pos: host bound on start_pos[b] + n_valid[b]; must be <= kv_max.
 * Errors: _NULL, _RANGE (layer, batch > max_batch, n_new > max_chunk,
 * max_end_pos > kv_max), _SHARED_LAYER (layer reads another layer's cache),
 * _UNBOUND, _HIP.
 */
int32_t g4attn_append_kv(const g4attn_stack* stack, int32_t layer, const void* k,
                         const void* v, const int32_t* start_pos, const int32_t* n_valid,
                         int32_t batch, int32_t n_new, int32_t max_end_pos, void* stream);

/*
 * Single-token decode ([12B] "The recipe": the 1-token decode bucket).
 *   q:   [batch][n_q_heads][head_dim] bf16, the current token's queries.
 *   seq_lens: int32[batch], keys cached for each sequence INCLUDING the
 *        current token (already appended); the query sits at seq_lens[b]-1.
 *        A length <= 0 gives a zero output row.
 *   max_seq_len: host bound on seq_lens[b]; 1 <= max_seq_len <= kv_max.  The
 *        key splits are planned from it; a larger seq_lens[b] is treated as
 *        max_seq_len.
 *   out: [batch][n_q_heads][head_dim] bf16.
 * Output = softmax(s) V over the visible keys, s = scale * q K^T (each score
 * replaced by softcap * tanh(s / softcap) when the layer sets a cap), fp32
 * accumulation, rounded to bf16 (round to nearest even).
 * Errors: _NULL, _RANGE, _UNBOUND, _HIP.
 */
int32_t g4attn_decode(const g4attn_stack* stack, int32_t layer, const void* q,
                      const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, void* out,
                      void* stream);

/*
 * g4attn_decode for callers that cannot allocate device memory or use a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, results and errors as
 * g4attn_decode on an unpaged stack whose cache is bound; the bound workspace
 * is not touched.  The split partials and arrival counters live instead in a
 * scratch array the library holds on each GPU it runs on (16 MiB, of which
 * 256 KiB are counters; kept until the process ends).  A call whose split
 * plan needs more (about batch x n_q_heads x splits x (head_dim + 2) x 4
 * bytes, or more than 65536 (sequence, KV head, head block) counters) returns
 * G4ATTN_ERR_UNSUPPORTED before any launch.  No hipMalloc or other
 * allocation happens in this call; its first call on a GPU looks up that
 * GPU's scratch address and clears the counters with one small kernel on
 * `stream`.  Every call on one GPU shares that GPU's scratch: calls that
 * overlap in time on one GPU (different streams, or several host threads)
 * race and must be ordered by the caller.
 */
int32_t g4attn_decode_noalloc(const g4attn_stack* stack, int32_t layer, const void* q,
                              const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                              void* out, void* stream);

/*
 * Decode step with the current token's K/V write fused in ([FR] 4 and 5: the
 * decode graph writes the new token's K/V into the resident cache in place
 * and attends over it).  Same as g4attn_append_kv of one token at position
 * seq_lens[b] - 1 followed by g4attn_decode, in one launch, with bit-identical
 * results and cache contents.
 *   k_new: [batch][n_kv_heads][head_dim] bf16, the current token's K rows.
 *   v_new: same shape, or NULL on a k_eq_v layer (and non-NULL otherwise).
 *   q, seq_lens, max_seq_len, out: as for g4attn_decode; seq_lens[b] counts
 *        the current token, whose row is written at position seq_lens[b] - 1
 *        (nothing is written for a length <= 0).
 * Errors: _NULL, _RANGE, _SHARED_LAYER (the layer reads another layer's
 * cache), _UNBOUND, _HIP.
 */
int32_t g4attn_decode_append(const g4attn_stack* stack, int32_t layer, const void* q,
                             const void* k_new, const void* v_new, const int32_t* seq_lens,
                             int32_t batch, int32_t max_seq_len, void* out, void* stream);

/*
 * Prefill of a chunk of n_tok new tokens per sequence ([12B] "The recipe":
 * the 64-token prefill bucket; causal with the layer's window).
 *   q:   [batch][n_tok][n_q_heads][head_dim] bf16.
 *   start_pos: int32[batch]; token t of sequence b sits at start_pos[b] + t.
 *        The chunk's own K/V must already be appended (to the owning layer).
 *   max_start_pos: host bound on start_pos[b]; max_start_pos + n_tok <= kv_max.
 *        A larger start_pos[b] is treated as max_start_pos.
 *   out: [batch][n_tok][n_q_heads][head_dim] bf16.
 * Errors: _NULL, _RANGE (n_tok > max_chunk, ...), _UNBOUND, _HIP.
 */
int32_t g4attn_prefill(const g4attn_stack* stack, int32_t layer, const void* q,
                       const int32_t* start_pos, int32_t batch, int32_t n_tok,
                       int32_t max_start_pos, void* out, void* stream);

/*
 * Paged KV cache, for continuous batching ([E4B] "Limitations" names its
 * absence; [FR] closing section: batching as the next step).  Each owning
 * layer's planes hold n_pages pages of page_size slots for every KV head.
 * Position p of sequence b lives in page block_table[b * max_pages_per_seq +
 * p / page_size] at slot p % page_size; all layers of a stack share one block
 * table (page ids index each owning layer's own planes).  Within a page the
 * slots of one KV head are laid out like a cap-slot segment of the unpaged
 * layout.  There is no sliding-window ring: a sequence needs pages for the
 * positions a call reads or writes, and pages wholly before every window it
 * will read again may be reused by the caller.
 *   page_size: a multiple of 64 in [64, 65536].
 *   max_pages_per_seq: block-table entries per sequence; kv_max becomes
 *       max_pages_per_seq * page_size.  A key range of kv_max + max_chunk
 *       positions may span at most 1022 pages (else _UNSUPPORTED).
 * Unpaged entry points reject a paged stack and the _paged ones an unpaged
 * stack (G4ATTN_ERR_UNSUPPORTED); g4attn_kv_offset is unpaged only.  g4attn_layer_capacity returns page_size for a paged stack.
 * Block tables are int32 device arrays [batch][max_pages_per_seq]; ids outside
 * [0, n_pages) are clamped into it (wrong numbers, never an out-of-bounds
 * access).  Errors: as for the unpaged calls, plus _NULL for a NULL table.
 */
int32_t g4attn_stack_create_paged(const g4attn_layer_desc* layers, int32_t n_layers,
                                  int32_t max_batch, int32_t page_size, int32_t n_pages,
                                  int32_t max_pages_per_seq, int32_t max_chunk,
                                  g4attn_stack** out);
/* Byte offsets in the cache of element d of (page, kv_head, slot)'s K row and
 * V row for `layer`.  Errors: _NULL, _RANGE, _UNSUPPORTED (unpaged stack). */
int32_t g4attn_page_offset(const g4attn_stack* stack, int32_t layer, int32_t page, int32_t kv_head,
                           int32_t slot, int32_t d, int64_t* off_k, int64_t* off_v);
/* g4attn_append_kv through a block table. */
int32_t g4attn_append_kv_paged(const g4attn_stack* stack, int32_t layer, const void* k,
                               const void* v, const int32_t* start_pos, const int32_t* n_valid,
                               int32_t batch, int32_t n_new, int32_t max_end_pos,
                               const int32_t* block_table, void* stream);
/* g4attn_decode through a block table. */
int32_t g4attn_decode_paged(const g4attn_stack* stack, int32_t layer, const void* q,
                            const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                            const int32_t* block_table, void* out, void* stream);
/* g4attn_decode_append through a block table: the current token's K/V row is
 * written at position seq_lens[b] - 1 of the page the table maps it to, then
 * attended, in one launch.  The table must map that position.  The results
 * (outputs and cache contents) are those of g4attn_append_kv_paged followed by
 * g4attn_decode_paged; the errors those of g4attn_decode_append, plus _NULL
 * for a NULL table. */
int32_t g4attn_decode_append_paged(const g4attn_stack* stack, int32_t layer, const void* q,
                                   const void* k_new, const void* v_new,
                                   const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                   const int32_t* block_table, void* out, void* stream);
/* g4attn_prefill through a block table. */
int32_t g4attn_prefill_paged(const g4attn_stack* stack, int32_t layer, const void* q,
                             const int32_t* start_pos, int32_t batch, int32_t n_tok,
                             int32_t max_start_pos, const int32_t* block_table, void* out,
                             void* stream);

/* Message of the last error on this thread ("" if none). */
const char* g4attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* G4ATTN_H */
