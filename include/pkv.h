/*
 * pkv.h — C ABI of the paged-KV append and paged-attention library for AMD MI355X (gfx950).
 *
 * The library implements one hot path: new K/V rows are scattered into paged pools through an
 * int32 slot mapping, then a flat ragged step of decode rows and chunked-prefill rows attends
 * over the paged cache. Sources of the operations:
 *   [P3]  "P3: native paged-KV continuous-batching sampler" (align, code/docs/P3_ENGINE.md),
 *         section "Design > paged.py" (BlockAllocator, PagedKVCache, TritonPagedAttention
 *         contract) and "Design > engine.py" (Scheduler, Prefix sharing).
 *   [PKV] "Optional paged KV cache (vLLM-style) — v1 design" (mlx-bun docs/design/
 *         paged-kv-cache.md), section "Design" (BlockPool, typed PagedPoolExhausted).
 *   [BC]  "Finish RL Training Faster: Bitwise-Consistent ..." section 2 (kernel determinism,
 *         batch independence).
 *
 * Conventions for every entry point
 *   - Returns PKV_OK (0) or a negative status; pkv_last_error() then gives a message. The
 *     message is kept per thread: the next call on that thread that fails replaces it and a
 *     call that succeeds may clear it, so read (or copy) it right after the failure.
 *   - Arguments are validated on the host before anything happens: on any error nothing is
 *     launched, nothing is copied and no allocator state changes.
 *   - No exception crosses the ABI. No entry point allocates device memory: device buffers
 *     are owned by the caller; the library owns only allocator handles, a small ring of
 *     pinned host staging buffers for work lists (allocated by the first call on a device and
 *     grown only by a call larger than any before it: see pkv_staging_info) and, per device,
 *     one stream and two events.
 *   - Device work is enqueued on the caller's stream (a hipStream_t passed as void*; NULL is
 *     the default stream) and is asynchronous with respect to the host. An attention step with
 *     a large prefill pass (over 512 workgroups: the segments' tiles of 128 / group query
 *     rows, times num_kv_heads) and a large decode pass (at least 1024 workgroups: the decode
 *     rows' KV splits, times num_kv_heads) enqueues its decode pass on the library's stream,
 *     forked from the caller's stream after the step's append and joined back to it before
 *     the call returns: work enqueued later on the caller's stream sees the whole result, and
 *     the output bits are those of the unforked path. Such calls from several threads on one
 *     device serialise their decode passes on that stream.
 *   - Element type codes: PKV_F32 (float32) and PKV_BF16 (bfloat16). q, k_new, v_new and both
 *     pools share one element type; attention output is always float32.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status and element types ------------------------------------------------------- */
enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = -1,         /* malformed argument, shape, or id */
  PKV_ERR_POOL_EXHAUSTED = -2,  /* [PKV] typed exhaustion: never a silent truncation */
  PKV_ERR_DOUBLE_FREE = -3,     /* [P3] free of a block whose refcount is already 0 */
  PKV_ERR_SHARED_WRITE = -4,    /* [P3] write into a block with refcount > 1 */
  PKV_ERR_UNSUPPORTED = -5,     /* valid request outside the built kernel set */
  PKV_ERR_HIP = -6,             /* HIP runtime error (launch, copy, event) */
  PKV_ERR_INCONSISTENT = -7     /* allocator books do not add up */
};

/* Element types. PKV_E4M3 (one-byte E4M3 codes) names the pools of the _fp8 entry points and
 * is accepted as a pool type by pkv_copy_blocks only; the other entry points take PKV_F32 or
 * PKV_BF16. */
enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_E4M3 = 2 };

/* Flag bits of pkv_attention_ex / pkv_attention_workspace_size_ex. */
enum { PKV_ATTN_PHASE_CONSISTENT = 1 };

/* Message for the calling thread's last failure ("" if none). */
const char* pkv_last_error(void);
/* Library version string. */
const char* pkv_version(void);

/* ---- host block allocator [P3 "Design > paged.py": BlockAllocator] -------------------
 * A LIFO free list plus one refcount per block. A fresh pool hands out ids 0, 1, 2, ...
 * (the stack is [NB-1, ..., 1, 0] with 0 on top). Multi-id calls apply ids in array order
 * and are all-or-nothing. The handle is not thread-safe: serialise calls on one handle.
 */
typedef struct pkv_alloc pkv_alloc;

/* New allocator over num_blocks >= 0 blocks; *out receives the handle (caller destroys). */
int32_t pkv_alloc_create(int32_t num_blocks, pkv_alloc** out);
/* Release a handle (NULL is ignored). */
void pkv_alloc_destroy(pkv_alloc* a);
/* Pop n ids into out_ids[0..n) in pop order, each with refcount 1. All or nothing: if fewer
 * than n blocks are free, returns PKV_ERR_POOL_EXHAUSTED and changes nothing [PKV "Design"]. */
int32_t pkv_alloc_allocate(pkv_alloc* a, int32_t n, int32_t* out_ids);
/* Share: +1 reference on each of ids[0..n). Every id must be live (refcount >= 1), else
 * PKV_ERR_INVALID [P3 "Prefix sharing": only a running sequence's blocks are adopted]. */
int32_t pkv_alloc_incref(pkv_alloc* a, int32_t n, const int32_t* ids);
/* -1 reference on each of ids[0..n) in array order; a block reaching 0 is pushed on the free
 * stack. A free at refcount 0 (counting repeats within the call) is PKV_ERR_DOUBLE_FREE. */
int32_t pkv_alloc_free(pkv_alloc* a, int32_t n, const int32_t* ids);
/* Refcount of block id (>= 0), or PKV_ERR_INVALID for an id outside the pool. */
int32_t pkv_alloc_refcount(const pkv_alloc* a, int32_t id);
/* Number of free blocks. */
int32_t pkv_alloc_num_free(const pkv_alloc* a);
/* Number of blocks in the pool. */
int32_t pkv_alloc_num_blocks(const pkv_alloc* a);
/* PKV_OK iff free + referenced == total, no id twice on the free stack and no free-stack
 * member referenced [P3 "Design > paged.py": check_consistent]; else PKV_ERR_INCONSISTENT. */
int32_t pkv_alloc_check_consistent(const pkv_alloc* a);
/* Copy the free stack (bottom to top, pkv_alloc_num_free entries) and all refcounts
 * (pkv_alloc_num_blocks entries) into caller buffers; either pointer may be NULL. */
int32_t pkv_alloc_snapshot(const pkv_alloc* a, int32_t* free_stack_out, int32_t* refcounts_out);

/* Slot mapping [P3 "Design > paged.py": slots()]: for positions start_pos .. start_pos+n_new-1
 * of one sequence whose block-table row is bt_row[0..n_bt), writes
 *   slots_out[i] = bt_row[p / block_size] * block_size + p % block_size.
 * Refuses (PKV_ERR_SHARED_WRITE) a position whose block has refcount > 1: a shared block is
 * read-only for everyone, owner included. A free block or a position past the row is
 * PKV_ERR_INVALID. Host only; slots_out is host memory. */
int32_t pkv_slot_mapping(const pkv_alloc* a, const int32_t* bt_row, int32_t n_bt,
                         int32_t block_size, int32_t start_pos, int32_t n_new,
                         int32_t* slots_out);

/* Slot mapping of a whole step: for each sequence b < B, positions start_pos[b] ..
 * start_pos[b] + n_new[b] - 1 through row b of block_tables_host ([B, max_blocks], host int32),
 * written contiguously in sequence order to slots_out (sum of n_new entries). Same rules as
 * pkv_slot_mapping; all sequences are validated before any slot is written. Host only. */
int32_t pkv_slot_mapping_step(const pkv_alloc* a, const int32_t* block_tables_host, int32_t B,
                              int32_t max_blocks, int32_t block_size, const int32_t* start_pos,
                              const int32_t* n_new, int32_t* slots_out);

/* Host check of a slot array before pkv_write_kv: every slot is negative (padding, skipped)
 * or in [0, num_slots), and no non-negative slot appears twice. PKV_OK or PKV_ERR_INVALID. */
int32_t pkv_validate_slots(const int32_t* slots_host, int32_t n, int64_t num_slots);

/* ---- host step builder [P3 "Design > engine.py": Scheduler, Prefix sharing; "Optional
 *      paged KV cache (vLLM-style) — v1 design", sections "Design" (trim) and "Follow-ups"
 *      (block-level copy-on-write)] ------------------------------------------------------
 * Turns requests into the flat ragged steps the device path consumes (cu_seqlens_q, ctx_lens,
 * block tables, slots). A sequence is a token count plus num_computed; a step gives each
 * scheduled sequence n_new = min(remaining, chunk_size, budget) new rows: decodes (remaining
 * == 1) first, oldest first, then the others, oldest first, while the token budget lasts.
 * Admission is FIFO and takes the first waiting sequence only if its whole token list fits in
 * the free blocks not promised to sequences admitted earlier in the same step (at most
 * max_num_seqs running). When a scheduled sequence cannot get its blocks, the youngest running
 * sequence that holds blocks and is not yet scheduled in this step is preempted by recompute
 * (its blocks are freed, num_computed drops to 0, its tokens are kept); it may be the asking
 * sequence, which then waits for a later step. With prefix sharing, a waiting sequence adopts
 * the first (prompt_len - 1) / block_size blocks of the oldest running sequence of its group
 * and prompt length once that one has computed them (it waits until then), and recomputes its
 * last prompt token. A chunk that writes into a block with refcount > 1 first gets a fresh copy
 * of it (copy-on-write): the step lists (src, dst) block pairs the caller copies before the
 * append. After the forward pass, pkv_sched_complete advances num_computed; a sequence whose
 * tokens are all computed samples: it finishes (blocks freed) if listed in `finished` or at
 * max_blocks_per_seq * block_size tokens, else it grows by one token.
 * The handle owns its block allocator (pkv_sched_allocator returns it for queries and slot
 * mapping; do not destroy it separately). Not thread-safe. Errors: PKV_ERR_INVALID. */
typedef struct pkv_sched pkv_sched;

/* New scheduler over a fresh pool of num_blocks blocks; every size >= 1 (num_blocks >= 0);
 * prefix_sharing != 0 enables adoption. *out receives the handle (caller destroys). */
int32_t pkv_sched_create(int32_t num_blocks, int32_t block_size, int32_t chunk_size,
                         int32_t token_budget, int32_t max_num_seqs, int32_t max_blocks_per_seq,
                         int32_t prefix_sharing, pkv_sched** out);
void pkv_sched_destroy(pkv_sched* s);
/* The scheduler's allocator (owned by the handle). */
pkv_alloc* pkv_sched_allocator(pkv_sched* s);
/* Queue a request: a new id, prompt_len in [1, max_blocks_per_seq * block_size], group >= 0
 * to take part in prefix sharing (-1: none). */
int32_t pkv_sched_add(pkv_sched* s, int32_t seq_id, int32_t prompt_len, int32_t group);
/* Build the next step (refused while the previous one awaits pkv_sched_complete). Writes the
 * number of scheduled sequences B, rows T, copy-on-write pairs and preempted sequences; the
 * plan itself is read with pkv_sched_plan. */
int32_t pkv_sched_step(pkv_sched* s, int32_t* B, int32_t* T, int32_t* n_copies,
                       int32_t* n_preempted);
/* Copy the pending plan into caller buffers (any may be NULL): seq_ids, n_new, ctx_lens [B];
 * cu_seqlens_q [B + 1]; block_tables [B, max_blocks_per_seq] (whole tables after the step,
 * -1 past each sequence's blocks); slots [T] in step order; copies [2 * n_copies] as (src, dst)
 * pairs; preempted [n_preempted]. */
int32_t pkv_sched_plan(const pkv_sched* s, int32_t* seq_ids, int32_t* n_new, int32_t* ctx_lens,
                       int32_t* cu_seqlens_q, int32_t* block_tables, int32_t* slots,
                       int32_t* copies, int32_t* preempted);
/* Apply the pending plan after its forward pass; `finished` lists sequences whose sampled token
 * ends them. Writes the sequences that sampled, in plan order, to sampled [<= B] (may be NULL)
 * and their count to *n_sampled. */
int32_t pkv_sched_complete(pkv_sched* s, const int32_t* finished, int32_t n_finished,
                           int32_t* sampled, int32_t* n_sampled);
/* Rewind a running sequence to n_tokens in [1, its token count]: num_computed becomes
 * min(num_computed, n_tokens - 1) (the last kept token is fed again) and the blocks past
 * ceil(num_computed / block_size) are freed. Refused while a step is pending. */
int32_t pkv_sched_trim(pkv_sched* s, int32_t seq_id, int32_t n_tokens);
/* Fork a running sequence into new_id: the fork shares every block (refcount + 1) and is
 * admitted now; the first write into a shared block copies it. Refused while a step is pending
 * or at max_num_seqs. */
int32_t pkv_sched_fork(pkv_sched* s, int32_t src_id, int32_t new_id);
/* Per-sequence state (0 waiting, 1 running, 2 finished), token count, num_computed, blocks held;
 * any pointer may be NULL. pkv_sched_seq_blocks copies the held block ids (n_blocks entries). */
int32_t pkv_sched_seq_info(const pkv_sched* s, int32_t seq_id, int32_t* state,
                           int32_t* n_tokens, int32_t* num_computed, int32_t* n_blocks);
int32_t pkv_sched_seq_blocks(const pkv_sched* s, int32_t seq_id, int32_t* blocks);
/* Counters: preemptions so far, tokens adopted through prefix sharing, running and waiting
 * sequences. */
int32_t pkv_sched_stats(const pkv_sched* s, int64_t* preemptions, int64_t* shared_tokens,
                        int32_t* n_running, int32_t* n_waiting);
/* PKV_OK iff the allocator is consistent, refcounts equal the references held by the live
 * tables and no running sequence has computed past its blocks; else PKV_ERR_INCONSISTENT. */
int32_t pkv_sched_check(const pkv_sched* s);

/* ---- KV append [P3 "Design > paged.py": copy-free append, write scatters into
 *      (block, offset) in place] -----------------------------------------------------------
 * k_new, v_new: device [n_rows, num_kv_heads, head_dim] contiguous, element type dtype.
 * slots_dev:    device int32 [n_rows]; row t goes to slot s = slots_dev[t] (= block *
 *               block_size + offset), i.e. k_cache[s / block_size][s % block_size] = k_new[t].
 *               A negative slot skips its row. A slot >= num_blocks * block_size is skipped
 *               too (never written out of bounds). Duplicate non-negative slots leave the
 *               destination undefined: check host copies with pkv_validate_slots.
 * k_cache, v_cache: device [num_blocks, block_size, num_kv_heads, head_dim], written in place.
 * Bytes are copied exactly. Enqueued on stream. n_rows == 0 is a no-op. */
int32_t pkv_write_kv(const void* k_new, const void* v_new, const int32_t* slots_dev,
                     int32_t n_rows, void* k_cache, void* v_cache, int32_t num_blocks,
                     int32_t block_size, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                     void* stream);

/* ---- block copy for copy-on-write ["Optional paged KV cache (vLLM-style) — v1 design",
 *      section "Follow-ups": block-level copy-on-write, a fork copies a shared block on its
 *      first divergent write] ------------------------------------------------------------
 * For each pair i, block pairs_host[2i + 1] of both pools becomes a byte copy of block
 * pairs_host[2i] (all block_size slots, all heads): the (src, dst) pairs pkv_sched_step lists,
 * applied before the step's append. Validated on the host before anything is enqueued: ids in
 * [0, num_blocks), no destination twice, no destination that is also a source
 * (PKV_ERR_INVALID). The pairs go to the device through the library's pinned staging into
 * workspace (device, >= 8 * n_pairs bytes rounded up to 256, caller-owned; untouched until the
 * copy has run). Pools as in pkv_write_kv, or E4M3 pools (dtype PKV_E4M3). Enqueued on stream;
 * n_pairs == 0 is a no-op. */
int32_t pkv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs_host,
                        int32_t n_pairs, int32_t num_blocks, int32_t block_size,
                        int32_t num_kv_heads, int32_t head_dim, int32_t dtype, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ---- ragged paged attention [P3 "Design > paged.py": TritonPagedAttention contract —
 *      q, k/v cache blocks, block tables, cu_seqlens_q, ctx_lens, slot mapping; fixed KV
 *      split per context length, no atomics] ---------------------------------------------
 *
 * Semantics. Sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1; they are the
 * LAST q_len = cu[b+1]-cu[b] positions of its ctx_lens[b] cached tokens (ctx_lens counts the
 * cache after this step's append, new tokens included). The row at position pos attends over
 * keys 0..pos of its own sequence (causal inside a prefill chunk, prior context fully
 * visible). Query head h reads kv head h / (num_q_heads / num_kv_heads) [P3 "Tensor
 * parallelism > Design": blocked GQA map]. out[t][h] = sum_j softmax_j(scale * q.k_j) v_j,
 * accumulated in float32 and written as float32.
 *
 * Batch invariance [BC section 2]: a row's bits depend only on its own query, its sequence's
 * K/V values, its position, ctx_len and its kind (decode = segment with q_len == 1, prefill =
 * q_len > 1). They do not depend on the other sequences, the row's index in the step, the
 * physical placement of blocks, the stream or the run. Decode rows are cut into fixed splits
 * of kv_split tokens aligned at position 0 and merged in ascending split order; prefill rows
 * visit 64-token key tiles aligned at position 0 in ascending order. No atomics anywhere.
 *
 * Arguments.
 *   q:             device [T, num_q_heads, head_dim], element type dtype.
 *   k_cache, v_cache: device [num_blocks, block_size, num_kv_heads, head_dim], dtype.
 *   block_tables_dev: device int32 [B, max_blocks]; entries at and past ceil(ctx_lens[b] /
 *                  block_size) are never read. A read entry outside [0, num_blocks) is never
 *                  dereferenced: the rows that need it come out NaN.
 *   ctx_lens_host, cu_seqlens_q_host: host int32 [B] and [B + 1]; they drive the host work
 *                  planner. Need cu[0] == 0, cu non-decreasing, cu[B] == T,
 *                  0 <= q_len <= ctx_len <= max_blocks * block_size.
 *   head_dim:      64 or 128. num_q_heads / num_kv_heads in {1, 2, 4, 8}.
 *   kv_split:      positive multiple of 64, at most 2048 (512 is the default; part of the
 *                  numeric contract, so keep it fixed for bitwise comparisons). The
 *                  phase-consistent mode below takes any positive multiple of 64.
 *   out:           device float32 [T, num_q_heads, head_dim].
 *   workspace:     device buffer of at least pkv_attention_workspace_size() bytes, owned by
 *                  the caller, not read by the caller; it must stay untouched until the
 *                  enqueued work has finished. Calls that share a workspace must be ordered
 *                  on one stream.
 * Errors: PKV_ERR_INVALID (shapes, lengths, workspace too small), PKV_ERR_UNSUPPORTED
 * (head_dim or group size outside the built set), PKV_ERR_HIP. */
int32_t pkv_attention_workspace_size(const int32_t* ctx_lens_host,
                                     const int32_t* cu_seqlens_q_host, int32_t B,
                                     int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t kv_split, int32_t dtype,
                                     size_t* bytes);

int32_t pkv_attention(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables_dev, int32_t max_blocks,
                      const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host,
                      int32_t B, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                      int32_t kv_split, int32_t dtype, float* out, void* workspace,
                      size_t workspace_bytes, void* stream);

/* ---- phase-consistent attention ------------------------------------------------------
 * Same as pkv_attention / pkv_attention_workspace_size with a flags word. flags = 0 is exactly
 * pkv_attention. PKV_ATTN_PHASE_CONSISTENT routes every segment, decode rows (q_len == 1)
 * included, through the prefill tile path (64-key tiles aligned at position 0, visited in
 * ascending order, bf16 MFMA for both contractions), so a token's output bits are the same
 * whether it is computed inside a prefill chunk of any size or as a decode row (phase
 * consistency, [BC section 2]; the page names the shared path as the main cost of the
 * consistent version). In this mode every row, decode or prefill, has its keys cut into
 * splits of kv_split keys on the tile path: a tile item covers one split of its rows, and a row
 * whose keys reach past the first split writes one partial per split, which the merge combines
 * in ascending split order, exactly as for the split decode pass. The same kv_split must be
 * used for the calls whose rows are compared. Here kv_split has no upper bound: a split longer
 * than every context gives each row one pass over its whole context (no partials, fewer
 * workgroups for long decode rows). The extra cost over the split decode pass is measured, not
 * hidden.
 * Errors: as pkv_attention, plus PKV_ERR_INVALID for unknown flag bits and PKV_ERR_UNSUPPORTED
 * when the flag is set for float32 inputs (the tile path is bf16 MFMA only). */
int32_t pkv_attention_workspace_size_ex(const int32_t* ctx_lens_host,
                                        const int32_t* cu_seqlens_q_host, int32_t B,
                                        int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t kv_split, int32_t dtype,
                                        uint32_t flags, size_t* bytes);

int32_t pkv_attention_ex(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables_dev, int32_t max_blocks,
                         const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host,
                         int32_t B, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                         int32_t kv_split, int32_t dtype, uint32_t flags, float* out,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ---- fused step: KV append + attention in one call [P3 "Design > paged.py": the
 *      TritonPagedAttention contract takes the slot mapping together with q, the cache
 *      blocks, block tables, cu_seqlens_q and ctx_lens; it writes the new K/V and returns
 *      [T, H, D]] -----------------------------------------------------------------------
 * Same result as pkv_write_kv(k_new, v_new, <slots>, n_rows, k_cache, v_cache, ...) followed
 * by pkv_attention_ex(..., flags, ...) on the same stream, but the slots are read from host
 * memory: they are staged with the attention work lists in the library's pinned buffer, and
 * one launch copies the lists to the workspace and appends the rows, reading the slots from
 * the pinned buffer in place (no separate host-to-device copy).
 *   slots_host:   host int32 [n_rows]; row t of k_new / v_new ([n_rows, num_kv_heads,
 *                 head_dim], device, dtype) goes to slot slots_host[t]. A negative slot skips
 *                 its row; a slot >= num_blocks * block_size, or a non-negative slot that appears
 *                 twice, is PKV_ERR_INVALID (the rules of pkv_validate_slots, checked before
 *                 anything is enqueued: two rows sent to one slot would leave it undefined).
 *                 The array is copied before the call returns.
 *   workspace:    at least pkv_write_kv_attention_workspace_size() bytes (the attention
 *                 workspace plus the staged slots); same ownership rules as pkv_attention.
 * Every other argument as in pkv_write_kv and pkv_attention_ex. n_rows == 0 is the plain
 * attention call; T == 0 is the plain KV append.
 * Errors: as pkv_write_kv and pkv_attention_ex. */
int32_t pkv_write_kv_attention_workspace_size(const int32_t* ctx_lens_host,
                                              const int32_t* cu_seqlens_q_host, int32_t B,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t kv_split, int32_t dtype,
                                              uint32_t flags, int32_t n_rows, size_t* bytes);

int32_t pkv_write_kv_attention(const void* q, const void* k_new, const void* v_new,
                               const int32_t* slots_host, int32_t n_rows, void* k_cache,
                               void* v_cache, const int32_t* block_tables_dev,
                               int32_t max_blocks, const int32_t* ctx_lens_host,
                               const int32_t* cu_seqlens_q_host, int32_t B, int32_t T,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks, float scale,
                               int32_t kv_split, int32_t dtype, uint32_t flags, float* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ---- fused step with shared reads [P3 "Design > engine.py", Prefix sharing: G samples of a
 *      prompt share its full blocks read-only; "Optional paged KV cache (vLLM-style) — v1
 *      design", "Motivation": block-level sharing of a common prefix] --------------------
 * pkv_write_kv_attention with a host copy of the block tables for the work planner:
 *   block_tables_host: host int32 [B, max_blocks], the same entries as block_tables_dev over
 *                 every row's context (the planner reads entries below ceil(ctx_lens[b] /
 *                 block_size) only).
 * A decode split (kv_split keys aligned at a multiple of kv_split) that lies wholly inside the
 * contexts of several decode rows and covers the same physical blocks in each is read once per
 * group of up to min(4, 16 / (num_q_heads / num_kv_heads)) of those rows, instead of once per
 * row: one work item loads its K/V tiles once and runs every row's arithmetic of the per-row
 * decode item on them (the rows' query heads side by side in the matrix-core tile). So every
 * output bit is the same as with pkv_write_kv_attention (and as each row alone): only HBM and
 * cache traffic change. Applies to bfloat16 pools with num_q_heads / num_kv_heads in
 * {1, 2, 4, 8} on the split decode pass (not in the phase-consistent mode, where decode rows
 * run on the tile path); otherwise the call is exactly pkv_write_kv_attention. If the device tables name other blocks than the host copy
 * for a row of a group, that row is written as NaN (never from another row's keys).
 * The workspace comes from pkv_write_kv_attention_shared_workspace_size with the same host
 * tables (the group items take the place of per-row items in the lists).
 * Errors: as pkv_write_kv_attention, plus PKV_ERR_INVALID for NULL host tables (B > 0),
 * max_blocks < 0 or a ctx_len beyond max_blocks * block_size. */
int32_t pkv_write_kv_attention_shared_workspace_size(
    const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host, int32_t B,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t kv_split,
    int32_t dtype, uint32_t flags, int32_t n_rows, const int32_t* block_tables_host,
    int32_t max_blocks, int32_t block_size, size_t* bytes);

int32_t pkv_write_kv_attention_shared(const void* q, const void* k_new, const void* v_new,
                                      const int32_t* slots_host, int32_t n_rows,
                                      void* k_cache, void* v_cache,
                                      const int32_t* block_tables_dev,
                                      const int32_t* block_tables_host, int32_t max_blocks,
                                      const int32_t* ctx_lens_host,
                                      const int32_t* cu_seqlens_q_host, int32_t B, int32_t T,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                      float scale, int32_t kv_split, int32_t dtype,
                                      uint32_t flags, float* out, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* ---- FP8 (OCP E4M3) KV pools with per-tensor scales [BC section 4.2: the KV cache kept in
 *      FP8, about 57 % of the BF16 bytes, one write path; P3 "Design > paged.py" and its
 *      single-device notes: a K/V dtype other than the model's is dequantised on read, and
 *      FP8 without per-tensor scales is visibly lossy] -------------------------------------
 * A pool element is one byte, an E4M3 code (bias 7, largest finite 448, S.1111.111 NaN, no
 * infinities); the value it stands for is decode(code) * scale, with one float32 scale for
 * the whole K pool (k_scale) and one for the V pool (v_scale), both finite and > 0.
 *
 * pkv_write_kv_fp8: quantises and scatters. For row t and element e, with x the bfloat16
 * input, the code stored is E4M3(clamp(float32(x) * float32(1 / scale), -448, 448)) rounded to
 * nearest, ties to even (saturating; -0 keeps its sign). NaN inputs are not supported.
 *   k_new, v_new: device bfloat16 [n_rows, num_kv_heads, head_dim] contiguous.
 *   slots_dev, k_cache, v_cache: as pkv_write_kv, the pools uint8 [num_blocks, block_size,
 *                 num_kv_heads, head_dim]. num_kv_heads * head_dim a multiple of 16.
 * Errors: PKV_ERR_INVALID (sizes, NULL pointers, scales), PKV_ERR_UNSUPPORTED (row width),
 * PKV_ERR_HIP. n_rows == 0 is a no-op.
 *
 * pkv_attention_fp8: pkv_attention_ex over E4M3 pools, q bfloat16, out float32, with the same
 * routing, splits, tiles and merge order, hence the same batch invariance: decode rows on the
 * split decode pass over the codes, prefill rows (and with PKV_ATTN_PHASE_CONSISTENT every
 * row) on the MFMA tile path, which widens each tile's codes to bfloat16 in LDS. Codes widen
 * exactly (every E4M3 value is a bfloat16 value); k_scale folds into the score scale, v_scale
 * multiplies each split numerator (decode) or output (tiles) once. head_dim 64 or 128,
 * num_q_heads / num_kv_heads in {1, 2, 4, 8}; flags as pkv_attention_ex. Workspace from
 * pkv_attention_fp8_workspace_size (same flags), same ownership rules as pkv_attention.
 * Errors: as pkv_attention_ex, plus PKV_ERR_INVALID for scales that are not finite and > 0. */
int32_t pkv_write_kv_fp8(const void* k_new, const void* v_new, const int32_t* slots_dev,
                         int32_t n_rows, void* k_cache, void* v_cache, int32_t num_blocks,
                         int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                         float k_scale, float v_scale, void* stream);

int32_t pkv_attention_fp8_workspace_size(const int32_t* ctx_lens_host,
                                         const int32_t* cu_seqlens_q_host, int32_t B,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t kv_split, uint32_t flags,
                                         size_t* bytes);

int32_t pkv_attention_fp8(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables_dev, int32_t max_blocks,
                          const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host,
                          int32_t B, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                          float k_scale, float v_scale, int32_t kv_split, uint32_t flags,
                          float* out, void* workspace, size_t workspace_bytes, void* stream);

/* Fused E4M3 step: pkv_write_kv_fp8 of k_new / v_new through host slots followed by
 * pkv_attention_fp8, with the slots in the same host-to-device copy as the work lists, as
 * pkv_write_kv_attention does for bfloat16 / float32 pools (same slot rules: negative skips,
 * >= num_blocks * block_size or a repeated non-negative slot is PKV_ERR_INVALID). Workspace from
 * pkv_write_kv_attention_fp8_workspace_size (same flags, n_rows >= 0). Errors: as
 * pkv_write_kv_fp8 and pkv_attention_fp8. */
int32_t pkv_write_kv_attention_fp8_workspace_size(const int32_t* ctx_lens_host,
                                                  const int32_t* cu_seqlens_q_host, int32_t B,
                                                  int32_t num_q_heads, int32_t num_kv_heads,
                                                  int32_t head_dim, int32_t kv_split,
                                                  uint32_t flags, int32_t n_rows,
                                                  size_t* bytes);

int32_t pkv_write_kv_attention_fp8(const void* q, const void* k_new, const void* v_new,
                                   const int32_t* slots_host, int32_t n_rows, void* k_cache,
                                   void* v_cache, const int32_t* block_tables_dev,
                                   int32_t max_blocks, const int32_t* ctx_lens_host,
                                   const int32_t* cu_seqlens_q_host, int32_t B, int32_t T,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks, float scale,
                                   float k_scale, float v_scale, int32_t kv_split,
                                   uint32_t flags, float* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Fused E4M3 step with shared reads [P3 "Design > engine.py", Prefix sharing; "Finish RL
 * Training Faster: Bitwise-Consistent ...", section 4.2, one read path for FP8 storage]:
 * pkv_write_kv_attention_fp8 with a host copy of the block tables, exactly as
 * pkv_write_kv_attention_shared is pkv_write_kv_attention with one: decode splits that lie
 * wholly in the same physical blocks for several rows are read once per group of rows, every
 * output bit the same as pkv_write_kv_attention_fp8 on the same step (and as each row alone).
 * Arguments as pkv_write_kv_attention_fp8 plus block_tables_host / max_blocks as in
 * pkv_write_kv_attention_shared; the workspace comes from
 * pkv_write_kv_attention_shared_fp8_workspace_size with the same host tables. Errors: as
 * pkv_write_kv_attention_fp8, plus those of the host tables in pkv_write_kv_attention_shared. */
int32_t pkv_write_kv_attention_shared_fp8_workspace_size(
    const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host, int32_t B,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t kv_split,
    uint32_t flags, int32_t n_rows, const int32_t* block_tables_host, int32_t max_blocks,
    int32_t block_size, size_t* bytes);

int32_t pkv_write_kv_attention_shared_fp8(
    const void* q, const void* k_new, const void* v_new, const int32_t* slots_host,
    int32_t n_rows, void* k_cache, void* v_cache, const int32_t* block_tables_dev,
    const int32_t* block_tables_host, int32_t max_blocks, const int32_t* ctx_lens_host,
    const int32_t* cu_seqlens_q_host, int32_t B, int32_t T, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
    float k_scale, float v_scale, int32_t kv_split, uint32_t flags, float* out, void* workspace,
    size_t workspace_bytes, void* stream);

/* ---- allocation-free attention ---------------------------------------------------------
 * For callers that cannot allocate device memory during a call: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.
 * pkv_attention_noalloc is pkv_attention_ex (same arguments, semantics, kernels and bits)
 * without the workspace arguments: its work lists and split partials live in a device array
 * of PKV_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on until the process
 * ends. The first call with a device current sets that device up (the array's address, and the
 * pinned staging ring of 16 x 1 MiB if the device has none yet); every later call allocates
 * nothing (no hipMalloc, hipFree, hipHostMalloc or torch allocation).
 * Limits: a step whose workspace (pkv_attention_workspace_size_ex with the same arguments)
 * exceeds PKV_NOALLOC_SCRATCH_BYTES, or whose work lists exceed one staging slot (1 MiB unless
 * another entry point has grown the ring), is refused with PKV_ERR_UNSUPPORTED before
 * anything is enqueued.
 * Every call on one GPU shares that GPU's array: calls on one stream are ordered and safe;
 * calls that can overlap on one GPU (other streams, other threads without ordering) race on
 * it and give undefined results. Nothing in the array needs clearing between calls.
 * Errors: as pkv_attention_ex, plus PKV_ERR_UNSUPPORTED for the limits above. */
#define PKV_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)

int32_t pkv_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables_dev, int32_t max_blocks,
                              const int32_t* ctx_lens_host, const int32_t* cu_seqlens_q_host,
                              int32_t B, int32_t T, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              float scale, int32_t kv_split, int32_t dtype, uint32_t flags,
                              float* out, void* stream);

/* ---- diagnostics: per-kernel device time ------------------------------------------------
 * While enabled, every kernel launched by pkv_write_kv / pkv_attention is bracketed by two HIP
 * events recorded on its launch stream (the library owns the events). pkv_profile_read waits
 * for the recorded launches of one kernel kind and returns their summed elapsed time and count.
 * Kernel kinds: 0 KV append, 1 prefill tiles, 2 decode split pass, 3 split merge, 4 decode
 * group items (pkv_write_kv_attention_shared).
 * pkv_profile_enable(1) clears previous records; pkv_profile_enable(0) stops recording.
 * Not thread-safe with concurrent launches from several host threads. */
int32_t pkv_profile_enable(int32_t enable);
int32_t pkv_profile_read(int32_t kernel_kind, double* total_ms, int64_t* launches);
/* Summed over the attention calls recorded since pkv_profile_enable(1): the span from the
 * earliest start to the latest end of each call's bracketed launches whose kind bit is set in
 * kinds (launches of one call may run concurrently on two streams, e.g. the decode pass's
 * per-row items, kind 2, beside its group items, kind 4), and the number of such calls. */
int32_t pkv_profile_read_span(uint32_t kinds, double* total_ms, int64_t* calls);
/* The calling thread's current device's pinned staging ring: bytes per slot (0 before the
 * first staged call) and how many times its arena has been allocated so far. The arena (16
 * equal slots) is allocated by the first call that stages work lists on a device and replaced
 * only when a call needs more than a slot holds (the new slot size is the next power of two at
 * or above twice the old one and the request, at least 1 MiB), so steps of a size already seen
 * allocate nothing. Either pointer may be NULL. */
int32_t pkv_staging_info(size_t* slot_bytes, int64_t* allocations);
/* Kernel kinds bracketed from now on while profiling is enabled: bit k = kind k (default all,
 * 0x1F); records already taken are kept. Each event record costs the stream a few
 * microseconds, so a caller timing whole steps can bracket only the kernel it reports, or
 * only some of its launches. PKV_ERR_INVALID for bits above kind 4. */
int32_t pkv_profile_set_kinds(uint32_t kinds);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
