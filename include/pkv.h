/*
 * pkv.h — C ABI of libpkv: PagedAttention decode on AMD MI355X (gfx950).
 *
 * The KV cache of every sequence is cut into fixed blocks of block_size
 * tokens (16) that sit anywhere in one shared pool; a per-sequence block
 * table maps logical block -> physical block, the way an OS page table maps
 * pages (ahmedhaies.com, "PagedAttention: why LLM serving wastes most GPU
 * memory", section "The solution: borrow virtual memory from the OS";
 * thienlv.com, "PagedAttention là gì?", section "How does PagedAttention
 * work?"). One decode step appends each sequence's new key/value and attends
 * its new query over the whole cache (news.hamidun.com glossary "KV-Cache",
 * prefill/decode paragraph).
 *
 * Conventions for every call:
 *  - Return value: PKV_OK (0) or a negative PKV_E* code. No exception or
 *    abort crosses the ABI. pkv_last_error() gives a message for the last
 *    failing call on this host thread.
 *  - Device memory (the pool, q, out, k_new, v_new, slots, workspace) is
 *    owned by the caller (e.g. torch tensors) and must outlive the calls
 *    that use it. Host metadata (free list, reference counts, the device
 *    copies of tables, lengths and schedules, pinned staging) is owned by the
 *    library and released by pkv_kv_pool_free.
 *  - Streams are passed as uintptr_t (a hipStream_t; 0 = null stream). All
 *    device work is asynchronous on that stream; no call synchronises the
 *    device except pkv_kv_pool_free.
 *  - A pool handle must not be used from two host threads at once, and its
 *    device work must be ordered: issue it on one stream, or order the
 *    streams, since an upload rewrites device copies that earlier launches read.
 *
 * Pool layout in device memory (dev_base, dev_bytes >= pkv_pool_bytes):
 *   K region: [layers][num_blocks][kv_heads][block_size][head_dim] elements,
 *   V region: the same shape, starting right after the K region.
 * A physical block id names the same block in every layer. One
 * (block, kv_head) tile of K (or V) is block_size * head_dim contiguous
 * elements: 4 KiB for bf16/fp16 x 128 or fp32 x 64.
 *
 * q8_0 cache (PKV_Q8_0): the quantised cache type ssdnodes.com ("KV cache vs
 * prompt cache", "Four ways to make the KV cache smaller", item 2) names as
 * halving an f16 cache, in llama.cpp's Q8_0 block format: every 32
 * consecutive head_dim elements of a row are one fp16 scale d and 32 int8
 * codes c, value d * c. A tile is block_size * head_dim int8 codes followed
 * by block_size * head_dim/32 fp16 scales, ordered [row][group] in the K
 * region and [group][row] in the V region (2176 bytes for head_dim 128). The
 * codes are placed so that every 16-byte load of the decode kernel reads a
 * contiguous run: rows are taken R = min(block_size, 16) at a time (u = r/R,
 * rr = r%R), and with P = head_dim/8 chunks of 8 codes per row and NV = P/4,
 * chunk w = 4k + q (codes 8w .. 8w+7) of row r starts at byte
 *   K: u*R*head_dim + (k/2)*R*64 + (q*R + rr)*16 + (k%2)*8,
 *   V: u*R*head_dim + ((rr%NV)/2)*R*64 + ((rr/NV)*P + w)*16 + (rr%2)*8. q, k_new and v_new are bf16 for a q8_0 cache; appends quantise each
 * group with d = max|x| / 127 and c = round(x * (1/d)) (halves away from
 * zero, fp32 arithmetic, d stored rounded to fp16).
 *
 * q4_0 cache (PKV_Q4_0): the 4-bit cache type of the same passage (about a
 * quarter of an f16 cache), in llama.cpp's Q4_0 block format: every 32
 * consecutive elements of a row are one fp16 scale d and 32 4-bit codes q,
 * value (q - 8) * d. A tile is block_size rows of CB = head_dim/2 code bytes
 * followed by the scales as for q8_0 (1152 bytes for head_dim 128). Codes are
 * kept in 4-byte words of 8 consecutive elements (element j of a word in byte
 * j/2, low nibble for even j); with G = head_dim/32, word w = 4k + q of row r
 * (group k, quarter q) is at byte r*CB + 4*(q*G + k) of a K tile and at
 * (r - r%G)*CB + 4*(w*G + r%G) of a V tile, so that the decode kernel reads a
 * lane's share of each tile with one 16-byte (head_dim 64: 8-byte) load.
 * q, k_new and v_new are bf16; appends take m,
 * the group's element of largest magnitude (the first on ties, +0 for an
 * all-zero group), d = m / -8 and q = min(15, trunc(x * (1/d) + 8.5)) (fp32,
 * product and sum rounded separately, 1/d taken as 0 when d is 0), d stored
 * rounded to fp16.
 *
 * Supported: block_size 8, 16 or 32, head_dim 64 or 128, dtype
 * fp32/fp16/bf16/q8_0/q4_0, q_heads / kv_heads (the GQA group) from 1 to 8.
 * Other shapes return PKV_EUNSUPPORTED.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_pool pkv_pool; /* opaque */

enum { PKV_F32 = 0, PKV_F16 = 1, PKV_BF16 = 2, PKV_Q8_0 = 3, PKV_Q4_0 = 4 };

enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,          /* bad argument or inconsistent table              */
  PKV_ECAPACITY = -2,       /* pool cannot hold max_seq_len tokens             */
  PKV_EOUT_OF_BLOCKS = -3,  /* free list exhausted: the caller should queue    */
  PKV_EUNSUPPORTED = -4,    /* shape outside the supported set                 */
  PKV_EHIP = -5             /* HIP runtime error (allocation, copy, launch)    */
};

typedef struct {
  int32_t layers;      /* layers sharing one block id space                      */
  int32_t num_blocks;  /* physical blocks per layer                              */
  int32_t block_size;  /* tokens per block: 8, 16 (the pages' default) or 32     */
  int32_t kv_heads;    /* stored K/V heads                                       */
  int32_t head_dim;    /* 64 or 128                                              */
  int32_t dtype;       /* PKV_F32 | PKV_F16 | PKV_BF16 | PKV_Q8_0 | PKV_Q4_0     */
  int32_t max_seq_len; /* longest context any sequence may reach (< 2^30)        */
  int32_t max_seqs;    /* largest batch passed to upload/prepare                 */
} pkv_shape;

/*
 * Bytes of device memory the pool needs:
 *   layers * num_blocks * block_size * 2 * kv_heads * head_dim * elem_bytes,
 * i.e. num_blocks * block_size tokens at the per-token size
 * 2 * layers * kv_heads * head_dim * elem_bytes (ssdnodes.com, "KV cache vs
 * prompt cache", section "How much memory does the KV cache use?").
 * Returns 0 for an invalid shape.
 */
size_t pkv_pool_bytes(const pkv_shape* shape);

/*
 * Create a pool over caller-owned device memory dev_base[0, dev_bytes).
 * Startup capacity check: if max_seq_len > num_blocks * block_size the call
 * fails with PKV_ECAPACITY and a message naming both numbers (the check
 * described on ssdnodes.com, "KV cache vs prompt cache", section "Why a model
 * that works at 2k refuses to load at 32k").
 * dev_base == NULL creates a host-only pool: the block manager works, every
 * device call returns PKV_EINVAL. Otherwise the library allocates its device
 * metadata (tables, lengths, slots, schedules) and pinned staging here.
 * On success *out receives the handle; on failure *out is untouched.
 */
int pkv_kv_pool_alloc(const pkv_shape* shape, void* dev_base, size_t dev_bytes, pkv_pool** out);

/* Synchronise the device, release library-owned memory and the handle. NULL is a no-op. */
int pkv_kv_pool_free(pkv_pool* pool);

/* ---- host block manager: ids are physical block ids shared by all layers ---- */

/*
 * Take n free blocks (refcount 1 each) into ids_out[n]. Blocks are handed out
 * only on demand (thienlv.com, "PagedAttention là gì?", "How does
 * PagedAttention work?"). If fewer than n are free nothing is taken and
 * PKV_EOUT_OF_BLOCKS is returned: the caller queues the request (ssdnodes.com,
 * "KV cache vs prompt cache", section "What concurrency does").
 */
int pkv_block_alloc(pkv_pool* pool, int n, int32_t* ids_out);

/* Take the given free blocks (refcount 1): restores a known placement. All-or-nothing. */
int pkv_block_claim(pkv_pool* pool, const int32_t* ids, int n);

/*
 * Add one reference to each allocated block: a sequence starts sharing it
 * (shared prompt, parallel sampling; ahmedhaies.com, "PagedAttention: why LLM
 * serving wastes most GPU memory", the copy-on-write paragraph). All-or-nothing.
 */
int pkv_block_ref(pkv_pool* pool, const int32_t* ids, int n);

/*
 * Drop one reference from each block; a block returns to the free list at
 * zero (a request's cache is released when it ends: ssdnodes.com, "KV cache
 * vs prompt cache", FAQ). All-or-nothing.
 */
int pkv_block_free(pkv_pool* pool, const int32_t* ids, int n);

/* Reference count of one block (>= 0), or PKV_EINVAL for an out-of-range id. */
int pkv_block_refcount(const pkv_pool* pool, int32_t id);

/*
 * Slot assignment for one decode step: each sequence's new token gets the
 * row after its cached ones, in a block taken on demand when the token starts
 * a new one (thienlv.com, "PagedAttention là gì?", "How does PagedAttention
 * work?": physical blocks are handed out only when needed and recorded in the
 * block table), and a block still shared by other sequences is copied before
 * it is written (ahmedhaies.com, "PagedAttention: why LLM serving wastes most
 * GPU memory", the copy-on-write paragraph after "The solution: borrow virtual
 * memory from the OS"). host_bt is the caller's block table,
 * int32 [batch][max_blocks] row-major, -1 for absent entries; ctx_lens[s] is
 * the context length with the new token included (>= 1). For each sequence in
 * batch order, with p = ctx_lens[s] - 1 and j = p / block_size:
 *   - host_bt[s][j] == -1: a free block is taken and written there;
 *   - host_bt[s][j] shared (refcount > 1): copy-on-write — a free block is
 *     taken, the pair (old, new) is appended to cow_pairs_out, the old block
 *     loses one reference and host_bt[s][j] becomes the new block;
 *   - otherwise the block is written in place.
 * slot_out[s] = host_bt[s][j] * block_size + p % block_size (int64).
 * cow_pairs_out receives n_cow (old, new) int32 pairs; cow_capacity is its
 * capacity in pairs (batch always suffices). Every check and the count of
 * blocks the call needs come before any change, so a failing call (including
 * PKV_EOUT_OF_BLOCKS) changes nothing: no table entry, reference count or
 * prefix-cache entry.
 */
int pkv_prepare_append(pkv_pool* pool, int32_t* host_bt, int batch, int max_blocks,
                       const int32_t* ctx_lens, int64_t* slot_out, int32_t* cow_pairs_out,
                       int cow_capacity, int* n_cow);

/*
 * Slot assignment for writing several tokens per sequence, e.g. a prompt or a
 * chunk of one in prefill, whose K/V rows are all written to the cache
 * (news.hamidun.com "KV-Cache", prefill/decode paragraph). Sequence s writes
 * n_new[s] >= 0 tokens at logical positions ctx_before[s] ..
 * ctx_before[s] + n_new[s] - 1. In batch order, every block index j those
 * positions touch is handled once as pkv_prepare_append handles its one
 * block: absent -> a free block is taken; shared -> copy-on-write pair;
 * otherwise in place. slot_out (capacity slot_capacity) receives
 * sum(n_new) int64 slots, sequence by sequence in position order:
 * host_bt[s][p / block_size] * block_size + p % block_size. The slots are
 * distinct and can be passed (on the device) to pkv_kv_append as its
 * per-row slots. pkv_prepare_append is the case n_new = 1,
 * ctx_before = ctx_lens - 1. All-or-nothing, as pkv_prepare_append.
 */
int pkv_prepare_write(pkv_pool* pool, int32_t* host_bt, int batch, int max_blocks,
                      const int32_t* ctx_before, const int32_t* n_new, int64_t* slot_out,
                      int64_t slot_capacity, int32_t* cow_pairs_out, int cow_capacity,
                      int* n_cow);

/*
 * Block-table upload: the per-sequence map from logical block to physical
 * block that the decode kernels read the cache through (thienlv.com,
 * "PagedAttention là gì?", "How does PagedAttention work?"; ahmedhaies.com,
 * "PagedAttention: why LLM serving wastes most GPU memory", "The solution:
 * borrow virtual memory from the OS", where it plays the role of the page
 * table). Upload the block table int32 [batch][max_blocks] (-1 padded), the context
 * lengths int32 [batch] and optionally the slots int64 [batch] (NULL: keep
 * none) to the library's device copies, asynchronously on `stream`: the
 * data is packed into coherent pinned staging (a ring of four buffers, each
 * reused once the copy that last read it has finished) and copied by a small
 * kernel on `stream`, together with the decode schedule for the partition
 * setting and group of the previous decode call. Checked on the host first: 1 <= batch <= max_seqs,
 * max_blocks * block_size <= the pool's table width, 1 <= ctx <= max_seq_len, every
 * entry j < ceil(ctx / block_size) in [0, num_blocks); a non-negative slot must be the
 * table position of the sequence's new token (row ctx-1), as
 * pkv_prepare_append produces; negative slots skip the append.
 * Later kv_append / decode calls use this upload.
 */
int pkv_block_table_upload(pkv_pool* pool, const int32_t* host_bt, int batch, int max_blocks,
                           const int32_t* ctx_lens, const int64_t* host_slots, uintptr_t stream);

/*
 * Copy-on-write copies: for each host pair (src, dst) int32 [n][2], copy the
 * whole K and V block src -> dst in every layer (ahmedhaies.com,
 * "PagedAttention: why LLM serving wastes most GPU memory", copy-on-write
 * paragraph). Pairs are uploaded through pinned staging. Must run before the
 * kv_append that writes into dst. n == 0 is a no-op.
 */
int pkv_copy_blocks(pkv_pool* pool, const int32_t* host_pairs, int n, uintptr_t stream);

/*
 * Append: each decode step stores the new token's key and value in the cache
 * (news.hamidun.com glossary "KV-Cache", prefill/decode paragraph), here at
 * the slot the block table gives it. For s < batch and every kv head g, write k_new[s][g][:] and
 * v_new[s][g][:] (cache dtype, [batch][kv_heads][head_dim]; bf16 when quantised)
 * into the pool row of layer `layer` at slot[s] (block slot / block_size, row
 * slot % block_size); slot < 0 skips. dev_slots: device int64 [batch], or NULL for the
 * slots of the last upload (batch must then equal the uploaded batch). Bytes
 * are copied unchanged (q8_0 / q4_0: quantised as described above). With device
 * slots, "batch" is any number of rows: the multi-token write of a prefill
 * passes one row and one slot (from pkv_prepare_write) per token; the slots
 * must be distinct. Device slots are not checked on the host; a slot outside
 * [0, num_blocks * block_size) is skipped by the kernel (nothing is written
 * for that row). The kernels index their work items with 32-bit integers:
 * batch * kv_heads * 2 * head_dim may reach 2^37 elements for q8_0 / q4_0 and
 * 2^43 / (element bytes) otherwise; a larger call returns PKV_EHIP without
 * writing.
 */
int pkv_kv_append(pkv_pool* pool, int layer, const void* k_new, const void* v_new,
                  const int64_t* dev_slots, int batch, uintptr_t stream);

/*
 * Decode attention of layer `layer` for the uploaded batch:
 *   out[s][h][:] = sum_t softmax_t(scale * q[s][h] . K_s[t][g]) * V_s[t][g],
 *   g = h / (q_heads / kv_heads), t < ctx[s],
 * where K_s[t] is row t % block_size of block bt[s][t / block_size] (news.hamidun.com
 * "KV-Cache", mechanism and prefill/decode paragraphs; the GQA head sharing of
 * ssdnodes.com, "KV cache vs prompt cache").
 * q: device [batch][q_heads][head_dim] in the cache dtype (bf16 when quantised,
 * whose K/V values are scale * code). out: device fp32
 * [batch][q_heads][head_dim]. Softmax and accumulation are fp32.
 * partition_tokens: 0 = balanced split — every wavefront of a full-chip launch
 * takes an equal share of all (sequence, kv head, block) tiles and partial
 * results are merged by a reduce kernel; > 0 (multiple of 16) = fixed split-K
 * partitions of that many tokens per sequence, each keeping its own max/sum,
 * merged by the same reduce (a partition >= the longest context is the
 * single-pass form, no reduce).
 * With a 2-byte cache of head_dim 128 (at most 4 q heads per kv head),
 * sequences whose tables name the same blocks for their
 * first tiles (a shared prompt, thienlv.com "Sharing") are grouped, up to
 * 16 / group per group, and those shared tiles are read once per group; their
 * partial results are merged with each sequence's own tiles by the reduce.
 * workspace / ws_bytes: device scratch of at least
 * pkv_decode_workspace_bytes(...) bytes, 16-byte aligned, for the split
 * partials (unused, may be NULL, when no sequence is split and no prompt is
 * shared). Calls sharing one workspace must not overlap.
 */
int pkv_paged_attn_decode(pkv_pool* pool, int layer, const void* q, int q_heads, float scale,
                          float* out, int partition_tokens, void* workspace, size_t ws_bytes,
                          uintptr_t stream);

/*
 * kv_append followed by paged_attn_decode of the same layer, in one launch:
 * the wavefront that reads a sequence's last block takes the new token's row
 * from k_new / v_new ([batch][kv_heads][head_dim], cache dtype; bf16 for
 * quantised caches: quantised as pkv_kv_append does), writes it to the pool at the
 * uploaded slot and attends over it. The last upload must
 * carry slots. Same results, bit for bit in the pool, as the two calls.
 */
int pkv_append_paged_attn_decode(pkv_pool* pool, int layer, const void* k_new, const void* v_new,
                                 const void* q, int q_heads, float scale, float* out,
                                 int partition_tokens, void* workspace, size_t ws_bytes,
                                 uintptr_t stream);

/*
 * pkv_paged_attn_decode without a workspace, for callers that cannot
 * allocate device memory around the call (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation). Same arguments, results
 * and errors as pkv_paged_attn_decode; the split partials live in a static
 * device array of PKV_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, held from the
 * library's first pool on that GPU until the process ends, and the call
 * allocates nothing (no hipMalloc, hipFree or pinned host memory). A decode
 * whose partials need more than that array (pkv_decode_workspace_bytes gives
 * the bound) returns PKV_EUNSUPPORTED; a decode whose schedule or staging
 * would have to grow returns PKV_EINVAL. Every call on one GPU shares its
 * array: calls that overlap on one GPU (other streams, other pools) race and
 * must be ordered by the caller. Nothing in the array needs to start at zero.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)
int pkv_paged_attn_decode_noalloc(pkv_pool* pool, int layer, const void* q, int q_heads,
                                  float scale, float* out, int partition_tokens,
                                  uintptr_t stream);

/* Workspace bytes a decode of `batch` sequences with these settings may need (upper bound). */
size_t pkv_decode_workspace_bytes(const pkv_pool* pool, int batch, int q_heads,
                                  int partition_tokens);

/*
 * Automatic prefix caching (ahmedhaies.com, "PagedAttention: why LLM serving
 * wastes most GPU memory", the enable-prefix-caching flag and the prefix
 * caching trade-off; thienlv.com, "PagedAttention là gì?", "Sharing";
 * ssdnodes.com, "KV cache vs prompt cache", "When local and remote caching
 * intersect"): a full block's K/V depend on every token up to its end, so a
 * block is keyed by its token ids together with the key of the block before
 * it. A block is found through a chained FNV-1a 64-bit hash of the prefix and
 * then confirmed exactly: its stored token ids must equal the request's, and
 * the block it was cached behind must be the block matched just before (the
 * same id with the same cache generation; a block id keyed again for other
 * content gets a new generation). Cached blocks whose last reference is released stay reusable
 * ("evictable") instead of returning to the free list; when the free list is
 * empty, allocation takes the least recently released evictable block and
 * drops its cache entry. Writing into a cached block held by one sequence
 * drops its entry (its content changes).
 *
 * pkv_prefix_match: walk the full blocks of tokens[0 .. n_tokens) from the
 * start and return how many leading blocks (at most max_ids) are cached;
 * their ids go to ids_out and each gains one reference (the caller puts them
 * at the front of the sequence's table and writes only the remaining tokens).
 * pkv_prefix_insert: register the full blocks of a sequence whose first
 * n_tokens tokens are written, bt_row[0 .. n_entries) being its table row;
 * blocks already cached, or whose content is already cached in another
 * block, are skipped. Returns the number of blocks added.
 * pkv_prefix_stats: stats_out[0] cached blocks, [1] of them evictable,
 * [2] blocks matched so far, [3] evictions so far.
 */
int pkv_prefix_match(pkv_pool* pool, const int32_t* tokens, int n_tokens, int32_t* ids_out,
                     int max_ids);
int pkv_prefix_insert(pkv_pool* pool, const int32_t* tokens, int n_tokens,
                      const int32_t* bt_row, int n_entries);
int pkv_prefix_stats(const pkv_pool* pool, int64_t stats_out[4]);

/*
 * stats_out[0] free blocks (including evictable cached ones), [1] blocks in
 * use, [2] blocks with refcount > 1,
 * [3] internal waste in tokens of the last upload: sum over sequences of
 * 16 * ceil(ctx/16) - ctx (only the last block of a sequence is partly empty;
 * ahmedhaies.com, "PagedAttention: why LLM serving wastes most GPU memory",
 * "The solution: borrow virtual memory from the OS").
 */
int pkv_pool_stats(const pkv_pool* pool, int64_t stats_out[4]);

/*
 * Decode schedule counters (diagnostics): stats_out[0] schedules built in
 * full, [1] bins schedules updated in place for an upload whose sequences
 * only gained tokens (the previous packing and cuts kept, new tiles given to
 * the wave holding each segment's last tile), [2] 1 when the current
 * schedule is the bins form, [3] its waves.
 */
int pkv_schedule_stats(const pkv_pool* pool, int64_t stats_out[4]);

/*
 * Bandwidth probes (measurements that bound the decode from above; not part
 * of the decode path). Both read with the decode's 16-byte nontemporal loads,
 * do no arithmetic beyond an XOR of what they read, and write one uint32 per
 * lane to dev_out (device memory of waves * 64 uint32, caller-owned); they
 * are asynchronous on `stream`.
 * pkv_probe_stream_read: `bytes` (a multiple of 16, dev_buf 16-byte aligned)
 *   of a contiguous device buffer, each of `waves` waves reading one
 *   contiguous share.
 * pkv_probe_gather: every K and V tile (16 tokens of one kv head) the decode
 *   of `layer` reads for the last upload, through the uploaded block table,
 *   the (kv head, sequence, tile) space split into `waves` equal shares: the
 *   decode's access pattern with perfect balance and no compute. 2-byte caches
 *   in blocks of 16 tokens (PKV_EUNSUPPORTED otherwise); PKV_EINVAL before an
 *   upload or for bad arguments.
 */
int pkv_probe_stream_read(const void* dev_buf, int64_t bytes, uint32_t* dev_out, int waves,
                          uintptr_t stream);
int pkv_probe_gather(const pkv_pool* pool, int layer, uint32_t* dev_out, int waves,
                     uintptr_t stream);

/* Message for the last failing call on this host thread ("" if none). */
const char* pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
