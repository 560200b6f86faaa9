/*
 * pkv.h -- C ABI of a paged, prefix-sharing KV attention library for
 * MI355X (gfx950).
 *
 * The problem, as the pages state it:
 *   - K/V activations live in fixed-size token blocks taken from one shared
 *     pool; each sequence holds an ordered list of block ids instead of a
 *     contiguous array, and a sequence that shares a prefix acquires the
 *     existing blocks (refcount + 1) instead of allocating and recomputing
 *     them ("Introducing RadixAttention into Trellis", section "RadixAttention
 *     in Trellis").
 *   - A fork copies block-table pointers, not K/V data, so it costs O(1) in
 *     the context length; blocks are shared copy-on-write (Dendrite page,
 *     section details and glossary entry "Copy-on-Write").
 *   - Decode is bound by memory bandwidth and PagedAttention splits the cache
 *     into fixed-size blocks like virtual-memory pages (SGLang RadixAttention
 *     page, section on the KV-cache lifecycle; Dendrite glossary).
 *   - Speculative decoding checks a draft tree's tokens in one target pass
 *     (CAST page, technical summary, "Problem").
 *
 * Conventions for every call:
 *   - Status codes, never exceptions or aborts.  On any error the host state
 *     (tables, refcounts, free list, sequence ids) is exactly as before the
 *     call and no device work has been enqueued -- except PKV_ERR_HIP from a
 *     kernel launch itself (a runtime or device failure, not an argument
 *     the library checks): work enqueued before it in the same call (a plan
 *     upload, the earlier sequences of a commit that runs them one by one)
 *     may have run, so the device contents of the pool are then undefined
 *     and the pool should be destroyed.  pkv_last_error() gives a message
 *     for the calling thread's last failure.
 *   - Ownership: every device pointer (the two K/V pools, the workspace, new
 *     K/V, Q, out, lse) is owned by the caller and must stay valid until the
 *     work enqueued on the stream has finished.  The pool handle owns its host
 *     metadata and any device memory it allocates itself (a workspace when
 *     the caller gives none, the append / commit lists); kv_pool_destroy
 *     releases both after synchronising the device.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *     stream).  Device work of one pool must be issued on a single stream, or
 *     the caller must order the streams: calls reuse the pool's scratch.
 *   - Threading: a pool is not thread-safe.
 *   - Sequence ids are int64, handed out in increasing order and never reused.
 *
 * Device layout of the pool (caller-allocated, bf16, each of K and V):
 *     [num_layers][num_blocks][num_kv_heads][block_size][head_dim]
 * so one (block, kv head) tile of one layer is contiguous.  Physical slot s
 * of a sequence's token t is (table[t / block_size], t % block_size).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_pool pkv_pool;

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_ARG = -1,         /* bad argument, pointer or shape */
  PKV_ERR_OOM = -2,         /* the free list cannot supply the blocks a call needs, or a
                               call's plan / partial states do not fit the pool's workspace */
  PKV_ERR_SEQ = -3,         /* unknown or freed sequence id */
  PKV_ERR_HIP = -4,         /* a HIP runtime call failed (message says which) */
  PKV_ERR_EMPTY = -5,       /* attention over a sequence with no tokens */
  PKV_ERR_UNSUPPORTED = -6  /* a shape the kernels do not handle */
} pkv_status;

typedef struct pkv_desc {
  int32_t num_blocks;    /* physical blocks in the pool, >= 1 */
  int32_t block_size;    /* tokens per block: a power of two, 1..128 */
  int32_t num_layers;    /* layers sharing one block table per sequence, >= 1 */
  int32_t num_q_heads;   /* query heads, a multiple of num_kv_heads */
  int32_t num_kv_heads;  /* key/value heads; q head h reads kv head h / (Hq / Hkv) */
  int32_t head_dim;      /* 64 or 128 for device pools; any >= 1 for host-only pools */
} pkv_desc;

/* Bytes of ONE of the two device pool arrays (K or V) for `desc`. 0 if invalid. */
size_t kv_pool_bytes(const pkv_desc* desc);

/*
 * Device workspace of a pool: the work lists ("plans") of its decode,
 * tree-verify and prefill calls and their partial softmax states.
 *   ptr:   device memory on the pool's device, 256-byte aligned, of `bytes`
 *          bytes, owned by the caller; or NULL: the pool allocates its own
 *          buffers and grows them when a call needs more (hipMalloc inside
 *          that call; an outgrown buffer is freed once the work enqueued
 *          before it has finished, with no device-wide synchronisation).
 *   bytes: at least kv_workspace_bytes(desc, max_seqs, max_tree_nodes).
 *   max_seqs:       sequences per attention call at most (0: 256).
 *   max_tree_nodes: query tokens per sequence at most -- the draft-tree
 *          nodes of a verify call, the new tokens of a prefill call (0: 64).
 * With a caller workspace, decode / verify / prefill calls allocate no
 * device memory: a call over more sequences or query tokens than these
 * limits returns PKV_ERR_ARG; a call whose work lists would not fit is
 * planned again with fewer, longer work items (no partial states where a
 * whole sequence fits one item) and returns PKV_ERR_OOM only if even that
 * plan does not fit -- never for calls within the limits when `bytes` is
 * the bound below.  Both errors come before any work is enqueued.
 */
typedef struct pkv_workspace {
  void* ptr;
  size_t bytes;
  int32_t max_seqs;
  int32_t max_tree_nodes;
} pkv_workspace;

/* Bytes of workspace that make every attention call within (max_seqs,
 * max_tree_nodes) on a pool of this shape fit, at any context length the
 * pool can hold: the decode, verify and prefill work lists (regions of their
 * own, so a cached decode plan survives the other calls) and the partial
 * states, each region 256-byte aligned.  0 for an invalid desc or limits
 * outside 1 .. 65536. */
size_t kv_workspace_bytes(const pkv_desc* desc, int32_t max_seqs, int32_t max_tree_nodes);

/* The regions of that workspace, in order: regions[0] decode work lists,
 * [1] verify work lists, [2] prefill work lists, [3] partial states (bytes;
 * they sum to kv_workspace_bytes). */
pkv_status kv_workspace_layout(const pkv_desc* desc, int32_t max_seqs, int32_t max_tree_nodes,
                               size_t* regions);

/*
 * Create a pool over caller-owned device arrays k_pool / v_pool (bf16, layout
 * above, each kv_pool_bytes(desc) bytes, on the device current at this call).
 * Passing NULL for both makes a host-only pool: the same allocator and block
 * tables with no device storage, for planning and tests (kv_append then takes
 * NULL K/V and attention calls return PKV_ERR_ARG).
 * Device pools also need one layer of one array (num_blocks * num_kv_heads *
 * block_size * head_dim * 2 bytes) under 64 GiB and fewer than 2^24 blocks;
 * else PKV_ERR_UNSUPPORTED.
 * ws: the device workspace (see pkv_workspace); NULL is {NULL, 0, 0, 0}.  A
 * caller workspace smaller than kv_workspace_bytes(desc, max_seqs,
 * max_tree_nodes) or not 256-byte aligned is PKV_ERR_ARG.  Host-only pools
 * take none.
 * free_order: NULL for the initial free list 0..num_blocks-1, else a host
 * array holding a permutation of 0..num_blocks-1 (head first).
 * Blocks are taken from the head of the free list; a block whose refcount
 * drops to zero is appended at the tail (SGLang RadixAttention page,
 * source-level sketch: free page pool, extend on reclaim).
 */
pkv_status kv_pool_create(const pkv_desc* desc, void* k_pool, void* v_pool, const pkv_workspace* ws,
                          const int32_t* free_order, pkv_pool** out);

/*
 * 4-bit pools.  The Dendrite page keeps the KV cache in 4 bits (TurboQuant)
 * for 3.88x less memory and computes from the quantized indices instead of
 * dequantizing the cache on every call (Dendrite page: summary and the
 * TurboQuant integration line).  Format of one token's K (or V) vector x of
 * one kv head: its norm in fp16 and head_dim 4-bit codes of the rotated
 * direction R x / |x|, R = H diag(signs) / sqrt(head_dim) (H the Sylvester
 * Hadamard matrix), each coordinate times sqrt(head_dim) quantized to the
 * 16-level Lloyd-Max levels of the unit normal (Max 1960).  2 + head_dim / 2
 * bytes per vector: 66 against 256 bf16 bytes at head_dim 128.
 * Device arrays (caller-owned, 16-byte aligned), for K and for V:
 *   codes u8   [num_layers][num_blocks][num_kv_heads][block_size][head_dim / 2]
 *              (byte j: dim 2j in the low nibble, dim 2j + 1 in the high one;
 *              code c names the c-th level in ascending order),
 *   norms fp16 [num_layers][num_blocks][num_kv_heads][block_size].
 * kv_pool_q4_bytes returns the bytes of one codes array and writes those of
 * one norms array to *norm_bytes (0 if desc is invalid).
 */
size_t kv_pool_q4_bytes(const pkv_desc* desc, size_t* norm_bytes);

/*
 * Create a 4-bit pool: same allocator and calls as kv_pool_create, but
 * kv_append quantizes the new bf16 K/V into codes and norms (copy-on-write
 * copies codes and norms), and paged_attn_decode computes attention from the
 * codes: in the rotated space a key's score is its norm times the dot
 * product of the rotated query with the levels its codes name, so MFMA
 * contracts the rotated query with the levels (fp16) directly; V is summed
 * in the rotated space and rotated back once.  The result is attention over
 * the dequantized K/V (fp16 operands: max |error| about 1e-3 against float64
 * on N(0,1) data).  One workgroup per query and kv head, no merge.
 * signs: host int8 [head_dim] of +1 / -1 (the rotation's random signs).
 * head_dim 64 or 128 and at most 16 query heads per kv head, else
 * PKV_ERR_UNSUPPORTED.  paged_attn_tree_verify, paged_attn_prefill and
 * kv_tree_commit return PKV_ERR_UNSUPPORTED on a 4-bit pool.  A 4-bit pool
 * manages its own workspace (as kv_pool_create with ws NULL).
 */
pkv_status kv_pool_create_q4(const pkv_desc* desc, void* k_codes, void* v_codes, void* k_norms,
                             void* v_norms, const int8_t* signs, const int32_t* free_order,
                             pkv_pool** out);

/* Synchronise the pool's device, then free its scratch and metadata. NULL is a no-op. */
void kv_pool_destroy(pkv_pool* pool);

/* New empty sequence (no blocks, length 0).  Host only. (Dendrite page,
 * first code listing: allocate_sequence.) */
pkv_status seq_allocate(pkv_pool* pool, int64_t* out_seq);

/*
 * Fork: the child gets a copy of the parent's block table and length and
 * every block's refcount goes up by one.  No K/V data moves and no device
 * work is enqueued (Dendrite page, section details and first code listing:
 * fork_sequence).  Cost is linear in the table length only.
 */
pkv_status seq_fork(pkv_pool* pool, int64_t parent, int64_t* out_child);

/* Drop a sequence: refcount - 1 for each block in table order; blocks that
 * reach zero go to the tail of the free list.  Host only. */
pkv_status seq_free(pkv_pool* pool, int64_t seq);

/*
 * Append n_tok new tokens to each of the n_seqs (distinct) sequences.
 * k_new / v_new: device bf16 [num_layers][n_seqs][n_tok][num_kv_heads][head_dim].
 * Host planning happens now and is all-or-nothing (PKV_ERR_OOM changes
 * nothing).  Per sequence in call order, per token in order:
 *   len % B == 0                 -> take a fresh block;
 *   else last block refcount > 1 -> copy-on-write: a fresh block receives the
 *                                   last block's filled slots (all layers, K
 *                                   and V), the sequence's table points at it
 *                                   and the old block loses one reference;
 *   then the token goes to slot (table[len / B], len % B) and len += 1.
 * (Dendrite glossary, Copy-on-Write; the cache is append-only: Trellis page,
 * section "LLM prefill and KV cache".)
 * Device work, in one launch on `stream`: the copy-on-write copies and the
 * scatter of the new K/V into their slots (they touch disjoint slots).
 */
pkv_status kv_append(pkv_pool* pool, const int64_t* seqs, int32_t n_seqs,
                     int32_t n_tok, const void* k_new, const void* v_new,
                     void* stream);

/*
 * Draft-tree commit: keep the accepted path of each sequence's draft tree
 * and drop the other nodes (CAST page: the target model checks the draft
 * tree in one pass and keeps the tokens it accepts -- lay summary part 2
 * and the technical summary's accept length).  The tree is the sequence's
 * last n_nodes tokens in node order, as for paged_attn_tree_verify.
 * parent:   host int32 [n_seqs][n_nodes], parent[0] = -1, 0 <= parent[i] < i;
 * path_len: host int32 [n_seqs], 0..n_nodes accepted nodes;
 * paths:    host int32 [n_seqs][n_nodes], row i starting with path_len[i]
 *           nodes: the root first, each node the parent of the next.
 * Afterwards sequence i has length ctx + path_len[i] (ctx = len - n_nodes):
 * its context, then the accepted nodes' K/V (all layers) in path order.
 * Per sequence in call order, blocks past the new length lose a reference
 * (table order; freed blocks go to the free-list tail), then each shared
 * block that receives a moved token is copied first (copy-on-write, table
 * order), taking only blocks that were free before the call.
 * All-or-nothing (PKV_ERR_OOM / PKV_ERR_ARG / PKV_ERR_SEQ change nothing).
 * Device work (device pools): one launch on `stream` (one per sequence
 * when a block one sequence writes in place is read by another).
 * 1 <= n_nodes <= 64; n_seqs <= 65535 (PKV_ERR_ARG beyond); sequences must
 * be distinct.
 */
pkv_status kv_tree_commit(pkv_pool* pool, const int64_t* seqs, int32_t n_seqs, int32_t n_nodes,
                          const int32_t* parent, const int32_t* path_len, const int32_t* paths,
                          void* stream);

/*
 * Decode attention at one layer: one query per sequence, GQA.
 * q:   device bf16 [n_seqs][num_q_heads][head_dim]
 * out: device fp32 [n_seqs][num_q_heads][head_dim]
 * lse: device fp32 [n_seqs][num_q_heads] (natural-log log-sum-exp), or NULL.
 * Each query attends to all `len` cached tokens of its sequence, its own
 * newest token included (Trellis page, section "LLM prefill and KV cache":
 * producing token t+1 reads K/V of tokens 0..t).
 *   out = sum_t softmax_t(sm_scale * q.k_t) v_t,  lse = ln sum_t exp(sm_scale * q.k_t)
 * Blocks shared by several of the sequences (a common prefix) are read once
 * per query group and the partial softmax states are merged by log-sum-exp.
 * Calls of short queries (by default every query at most 1024 keys and at
 * most 768 query x kv-head pairs) instead run one workgroup per query and
 * kv head over all of its keys, in a single launch with no merge; the
 * environment variables PKV_DIRECT_MAX_TOKENS / PKV_DIRECT_MAX_WGS, read at
 * kv_pool_create, move these limits (0 turns that mode off).
 * Sequences may repeat.  n_seqs == 0 is a no-op.  An empty sequence gives
 * PKV_ERR_EMPTY.
 */
pkv_status paged_attn_decode(pkv_pool* pool, int32_t layer, const int64_t* seqs,
                             int32_t n_seqs, const void* q, float sm_scale,
                             float* out, float* lse, void* stream);

/*
 * paged_attn_decode over the consecutive layers layer0 .. layer0 +
 * n_layers - 1 in one call, for schedules that hold the queries of several
 * layers at once: layer l's queries at q + l * n_seqs * num_q_heads *
 * head_dim (bf16 [n_layers][n_seqs][num_q_heads][head_dim]), its output and
 * lse rows likewise ([n_layers][n_seqs][num_q_heads][head_dim] fp32,
 * [n_layers][n_seqs][num_q_heads] or NULL).  One plan serves every layer
 * (the layers share the block tables); a call of short queries (the direct
 * plan) is ONE kernel launch over all its layers, other plans launch once
 * per layer.  Results equal n_layers paged_attn_decode calls bit for bit.
 * A layer range outside the pool: PKV_ERR_ARG; 4-bit pools:
 * PKV_ERR_UNSUPPORTED; otherwise as paged_attn_decode.
 */
pkv_status paged_attn_decode_layers(pkv_pool* pool, int32_t layer0, int32_t n_layers, const int64_t* seqs,
                                    int32_t n_seqs, const void* q, float sm_scale, float* out, float* lse,
                                    void* stream);

/*
 * paged_attn_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid it):
 * the same arguments and results, and the same kernels except that none of
 * them uses private (scratch) memory, which the runtime would size at its
 * first launch (for 256-row dense tiles at head_dim 128 this entry takes
 * the eight-wave kernel instead of the sixteen-wave one, which spills a few
 * registers).  The call's work lists and
 * partial softmax states live in a file-scope device array of the library
 * (32 MiB per device: 8 MiB of work lists, 24 MiB of partial states), held
 * by each device the library runs on until the process ends.  The call
 * allocates no device or pinned memory: it plans afresh each time (reusing
 * the pool's host buffers), uploads the work lists from pageable host memory
 * on `stream`, and launches.  A call whose work lists or partial states
 * exceed the array even when planned coarse returns PKV_ERR_OOM before any
 * work is enqueued.  Nothing in the array needs to start at zero (every
 * partial state is written before it is read).  Every call on one device
 * shares that device's array: calls that overlap on a device, from any pool
 * or stream, race.  4-bit pools: PKV_ERR_UNSUPPORTED.  With kernel timing on
 * (pkv_timing_enable) a call may create HIP events.
 */
pkv_status paged_attn_decode_scratch(pkv_pool* pool, int32_t layer, const int64_t* seqs, int32_t n_seqs,
                                     const void* q, float sm_scale, float* out, float* lse, void* stream);

/*
 * Draft-tree verify at one layer (CAST page, technical summary, "Problem":
 * the target model checks the draft tree's tokens in one pass; EAGLE-style
 * dynamic trees keep alternative branches).  For each sequence the last
 * n_nodes tokens are the tree's nodes in node order (appended by kv_append);
 * the context is the first len - n_nodes tokens.
 * parent: host int32 [n_seqs][n_nodes], parent[0] == -1, 0 <= parent[i] < i.
 * q:   device bf16 [n_seqs][n_nodes][num_q_heads][head_dim]
 * out: device fp32 [n_seqs][n_nodes][num_q_heads][head_dim]
 * lse: device fp32 [n_seqs][n_nodes][num_q_heads], or NULL.
 * Node i attends to the whole context, to its ancestors and to itself.
 * 1 <= n_nodes <= 64.
 */
pkv_status paged_attn_tree_verify(pkv_pool* pool, int32_t layer,
                                  const int64_t* seqs, int32_t n_seqs,
                                  int32_t n_nodes, const int32_t* parent,
                                  const void* q, float sm_scale, float* out,
                                  float* lse, void* stream);

/*
 * Causal prefill at one layer: attention of each sequence's newest tokens
 * over its whole cache.  After a prefix-cache hit only the prompt's
 * unmatched tokens are computed (SGLang RadixAttention page, the radix
 * tree's core operations, prefix matching: the forward pass covers the
 * n - k tokens that missed); they are appended with kv_append first, and
 * token t attends to tokens 0..t, the causal rule (Trellis page, section
 * "LLM prefill and KV cache").
 * n_new: host int32 [n_seqs]; the last n_new[i] tokens of seqs[i] are new
 *        (0 <= n_new[i] <= len; 0 contributes no queries).
 * q:   device bf16 [sum n_new][num_q_heads][head_dim], sequence after
 *      sequence, tokens in order.
 * out: device fp32 [sum n_new][num_q_heads][head_dim];
 * lse: device fp32 [sum n_new][num_q_heads] (natural log), or NULL.
 * Query j of sequence i (at position len - n_new[i] + j) attends to tokens
 * 0 .. len - n_new[i] + j.  At most 65536 queries per call (PKV_ERR_ARG
 * beyond).  A call whose n_new are all 0 is a no-op (q and out may then be
 * NULL).  Sequences may repeat.  A call with the same sequences and counts
 * as the previous prefill call, on a pool no call has changed since (the
 * next layer of the same step), reuses that call's plan.
 */
pkv_status paged_attn_prefill(pkv_pool* pool, int32_t layer, const int64_t* seqs,
                              int32_t n_seqs, const int32_t* n_new, const void* q,
                              float sm_scale, float* out, float* lse, void* stream);

/* ---- radix prefix cache (host only) ------------------------------------ */

/*
 * A block-granular radix tree from token-id sequences to the pool blocks
 * holding their K/V (SGLang RadixAttention page: node and edge structure,
 * the core operations match / split / insert, reference counting and
 * leaf-first LRU eviction; block-paged as on the Trellis page, section
 * "RadixAttention in Trellis": a session sharing a prefix acquires the
 * existing blocks, refcount + 1).  Edges hold whole blocks; a prompt matches
 * whole blocks only, so a prompt differing inside a block shares the blocks
 * before it (Trellis page, hit rate at most (L/B - 1)/(L/B) when the probe
 * differs in the last block).  The cache holds one reference on every block
 * it caches; blocks leave the pool only when their refcount reaches zero.
 * A cache borrows its pool.  Destroying the pool first detaches its caches:
 * their calls then fail with PKV_ERR_ARG and radix_destroy only frees the
 * cache.  Not thread-safe.
 * Access order for eviction is a counter bumped per touched node.
 * None of these calls enqueues device work.
 */
typedef struct pkv_radix pkv_radix;

pkv_status radix_create(pkv_pool* pool, pkv_radix** out);

/* Drops the cache's block references; NULL is a no-op. */
void radix_destroy(pkv_radix* cache);

/*
 * Longest cached whole-block prefix of tokens[0..n_tokens): a new sequence
 * (*out_seq) holds those blocks (refcount + 1 each) with length
 * *out_matched (a multiple of block_size, possibly 0).  The caller appends
 * the other n_tokens - *out_matched tokens with kv_append and computes only
 * them (paged_attn_prefill).  Every tree node on the matched path is locked
 * (protected from eviction) until radix_release(out_seq).
 */
pkv_status radix_match(pkv_radix* cache, const int32_t* tokens, int32_t n_tokens,
                       int64_t* out_seq, int32_t* out_matched);

/*
 * Cache the whole blocks of `seq` (its first n_tokens / block_size blocks)
 * under tokens[0..n_tokens), 0 <= n_tokens <= the sequence's length; the
 * caller vouches that those blocks hold the K/V of these tokens.  An edge
 * that diverges part-way is split at the block boundary (block ids are
 * re-sliced, no data moves); blocks under tokens already cached are left as
 * the tree has them; the rest become a new leaf (cache reference + 1 each).
 */
pkv_status radix_insert(pkv_radix* cache, int64_t seq, const int32_t* tokens, int32_t n_tokens);

/* The request that radix_match made `seq` for is done: unlock its path.
 * The sequence itself is untouched (seq_free it separately).
 * PKV_ERR_SEQ if `seq` holds no unreleased match of this cache. */
pkv_status radix_release(pkv_radix* cache, int64_t seq);

/*
 * Evict until the pool's free list holds at least want_free blocks: the
 * unlocked leaf touched longest ago goes first (its blocks lose the cache's
 * reference); a parent left without children becomes a leaf candidate.
 * *n_free (may be NULL) receives the free-list length afterwards.
 * PKV_ERR_OOM when only locked nodes remain and the target is not reached
 * (what could be evicted has been).
 */
pkv_status radix_evict(pkv_radix* cache, int32_t want_free, int32_t* n_free);

/* Tree nodes (root excluded), blocks referenced by the tree, locked nodes. */
pkv_status radix_stats(const pkv_radix* cache, int32_t* nodes, int32_t* cached_blocks,
                       int32_t* locked_nodes);

/* The tree in preorder (children ordered by their first block's tokens,
 * root excluded), per node: depth, token count t, lock count, t tokens,
 * t / block_size block ids.  Up to cap entries are copied; *n receives the
 * full length. */
pkv_status radix_dump(const pkv_radix* cache, int32_t* out, int32_t cap, int32_t* n);

/* ---- introspection (host only) ---------------------------------------- */

/* Block table (up to cap entries copied to out; out may be NULL when cap is 0),
 * number of blocks and length of a sequence. */
pkv_status seq_block_table(const pkv_pool* pool, int64_t seq, int32_t* out,
                           int32_t cap, int32_t* n_blocks, int32_t* len);

/* Refcount of one physical block. */
pkv_status block_refcount(const pkv_pool* pool, int32_t block, int32_t* rc);

/* The free list, head first (up to cap entries), and its length. */
pkv_status free_list(const pkv_pool* pool, int32_t* out, int32_t cap, int32_t* n);

/* Where the last successful kv_append put each token and which copies it
 * made: slots[i * n_tok + j] = block * block_size + offset for token j of
 * sequence i; cow = (src, dst, slots copied) triples in the order taken. */
pkv_status kv_last_append(const pkv_pool* pool, int32_t* slots, int32_t slot_cap,
                          int32_t* n_slots, int32_t* cow, int32_t cow_cap,
                          int32_t* n_cow);

typedef struct pkv_plan_stats {
  int64_t unique_tokens;   /* filled slots of the distinct blocks the call reads */
  int64_t logical_tokens;  /* sum over queries of the keys each attends to */
  int32_t unique_blocks;   /* distinct physical blocks the call reads */
  int32_t segments;        /* shared-prefix segments (runs of blocks with one query set) */
  int32_t work_items;      /* workgroups per kv head (MFMA, VALU, direct and path items) */
  int32_t merged_rows;     /* query rows whose partial states are merged */
  int32_t direct;          /* 1: one workgroup per query and kv head (direct kernel) */
  int32_t max_parts;       /* most partial states merged into one query (0: no merge) */
  int64_t plan_bytes;      /* device bytes of the call's work lists */
  int64_t partial_bytes;   /* device bytes of its partial softmax states */
} pkv_plan_stats;

/* What paged_attn_decode would read and launch for these sequences (host
 * only; planned as the call would be, before any fitting to a workspace). */
pkv_status paged_attn_decode_plan_stats(pkv_pool* pool, const int64_t* seqs,
                                        int32_t n_seqs, pkv_plan_stats* out);

/* Likewise for paged_attn_tree_verify (parent as there) and
 * paged_attn_prefill (n_new as there); segments is the number of sequences. */
pkv_status paged_attn_verify_plan_stats(pkv_pool* pool, const int64_t* seqs, int32_t n_seqs,
                                        int32_t n_nodes, const int32_t* parent, pkv_plan_stats* out);
pkv_status paged_attn_prefill_plan_stats(pkv_pool* pool, const int64_t* seqs, int32_t n_seqs,
                                         const int32_t* n_new, pkv_plan_stats* out);

/* ---- kernel timing (benchmarks) --------------------------------------- */

/* enable = n > 0: every n-th paged_attn_decode / paged_attn_tree_verify call
 * times its attention kernel with a pair of HIP events attached to that
 * kernel's own dispatch (hipExtLaunchKernel: they take the kernel's start and
 * end, not the time of separate markers; the plan upload and the
 * partial-state merge kernel stay outside); sampling keeps the timing from
 * slowing the calls it measures.  enable = 0 turns timing off and drops
 * pending pairs; negative values are an error. */
pkv_status pkv_timing_enable(pkv_pool* pool, int32_t enable);

/* Synchronise the recorded events and return the summed kernel time in ms
 * and the number of bracketed calls since the last reset; reset != 0 starts
 * a new count. */
pkv_status pkv_timing_read(pkv_pool* pool, double* total_ms, int64_t* calls,
                           int32_t reset);

/* ---- measurement ------------------------------------------------------ */

/* Enqueue one streaming read of `bytes` (a multiple of 16) of device memory
 * at `src` (16-byte aligned) by `blocks` workgroups of 256 threads, 128-bit
 * loads (sink: a device word the kernel writes only when the data fold to
 * a fixed 32-bit value, so the loads cannot be optimised away).  Timed by the caller with events on `stream`: the
 * HBM read ceiling the attention kernels are compared with. */
pkv_status pkv_hbm_read_probe(const void* src, size_t bytes, void* sink, int32_t blocks, void* stream);

/* Message of the calling thread's last error ("" if none). */
const char* pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
