/*
 * pagedkv.h -- PagedAttention decode for AMD Instinct MI355X (gfx950), C ABI.
 *
 * Page citations:
 *   [Walkthrough] "LLM serving (vLLM, quantized inference): Visual walkthrough"
 *   [Serving]     "How LLM Inference Serving Works: KV Cache, PagedAttention and Continuous
 *                 Batching"
 *
 * Model of the cache ([Serving] "PagedAttention: Virtual Memory for the KV Cache";
 * [Walkthrough] "Step 7"): the keys and values of every sequence live in fixed-size blocks of
 * `bs` tokens scattered through one physical pool; a per-sequence block table maps logical
 * block j (tokens j*bs .. j*bs+bs-1) to a physical block.  A slot is physical_block*bs + offset.
 *
 * Device layouts (row-major, all owned by the caller):
 *   k_cache   [NB][Hkv][bs][D]   token-major inside each (block, KV head) tile
 *   v_cache   [NB][Hkv][D][bs]   dim-major inside each (block, KV head) tile
 *   k_scale, v_scale [NB][Hkv] fp32, quantised caches only (value = code * scale)
 *   PA_I4 caches pack two codes per byte: K [NB][Hkv][bs][D/2], V [NB][Hkv][D][bs/2] bytes;
 *     every 4-byte group holds 8 consecutive elements of its row (dims for K, tokens for V):
 *     elements 0..3 in the low nibbles of bytes 0..3, elements 4..7 in the high nibbles, each
 *     nibble code + 8, codes in [-7, 7] ([Walkthrough] "Step 1": bytes per element set the
 *     cache size; INT4 halves INT8 again)
 *   q, out    [B][Hq][D]; out is always fp32
 *   block_tables [B][max_blocks] int32, unused entries may hold anything (e.g. -1)
 *   seq_lens  [B] int32
 *
 * Conventions
 *   - Every function returns an int status: PA_OK (0) or a negative PA_ERR_* code.  Nothing
 *     throws across the ABI.
 *   - Arguments are checked on the host before any HIP call; a bad argument returns
 *     PA_ERR_INVALID (or PA_ERR_UNSUPPORTED for a valid but unimplemented combination) and
 *     enqueues nothing.
 *   - Device entry points enqueue on `stream` (a hipStream_t passed as void*, NULL = the null
 *     stream) and return without synchronising.  A launch error returns PA_ERR_DEVICE.
 *   - The library allocates no device memory.  Scratch space for pa_decode is a caller buffer
 *     of at least pa_decode_workspace_size() bytes.
 *   - "Device-readable" arrays (the per-step slot mappings, table indices, lengths and copy
 *     pairs below) may be device memory or pinned host memory (hipHostMalloc): the kernels read
 *     each entry once, so a step's host-made arrays need no separate upload.
 *   - Not checked on the device, the caller's contract: block ids in tables, slot mappings and
 *     copy pairs lie in [0, NB); seq_lens[b] <= max_seq_len.  Kernels clamp lengths to
 *     max_seq_len and skip table entries outside [0, NB), so a broken contract gives wrong
 *     numbers, never an out-of-bounds access.
 *   - Allocator handles are not thread-safe; use one handle per thread or lock around it.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID = -1,     /* bad argument (null pointer, size out of range, ...) */
  PA_ERR_OOM = -2,         /* allocator: not enough free blocks; state left unchanged */
  PA_ERR_DEVICE = -3,      /* a HIP call or kernel launch failed */
  PA_ERR_UNSUPPORTED = -4, /* valid arguments, combination not implemented */
  PA_ERR_STATE = -5,       /* allocator: unknown or released sequence id */
  PA_ERR_TOO_LARGE = -6    /* pa_decode_no_alloc: the call needs more than its fixed scratch */
};

enum pa_dtype { PA_F32 = 0, PA_BF16 = 1, PA_I8 = 2, PA_I4 = 3 };

/* Static text for a status code. */
const char* pa_status_string(int status);

/* ABI version, bumped on any incompatible change. */
int pa_abi_version(void);

/* ================================================================================== */
/* Host block allocator ([Serving] "PagedAttention: Virtual Memory for the KV Cache",   */
/* "Sharing comes for free", "The Life of a Request"; [Walkthrough] "Step 7", "Step 8") */
/* ================================================================================== */
/*
 * Blocks are handed out on demand, when a sequence's current block is full.  Blocks carry a
 * reference count; forks share blocks; a write into a block with more than one reference first
 * copies it (copy-on-write).  The pages fix no hand-out order; this one makes every table
 * unique: a FIFO free list, initialised from `free_order`; allocations pop the head; a block
 * whose count reaches zero is pushed to the tail, in the logical order of the table it leaves;
 * batch calls serve sequences in the order given; sequence ids count up from 0 and are never
 * reused.  When the free list is empty an allocation evicts the least recently used cached
 * block (prefix caching, below).  Calls that run out of blocks return PA_ERR_OOM and change
 * nothing.
 */
typedef struct pa_allocator pa_allocator;

/* num_blocks >= 1, block_size >= 1.  free_order: NULL for 0..num_blocks-1, else a permutation
 * of 0..num_blocks-1 (copied; anything else is PA_ERR_INVALID).  *out receives the handle. */
int pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                    pa_allocator** out);
/* Releases the handle and all its host memory.  NULL is a no-op. */
void pa_alloc_destroy(pa_allocator* a);

/* New empty sequence; its id goes to *seq. */
int pa_seq_create(pa_allocator* a, int32_t* seq);

/* New sequence sharing the first n_tokens of `parent` (0 <= n_tokens <= parent length): the
 * child's table is the parent's first ceil(n_tokens/bs) blocks, each gaining a reference. */
int pa_seq_fork(pa_allocator* a, int32_t parent, int32_t n_tokens, int32_t* child);

/* Slot of the sequence's next token.  When the write lands in a block that other sequences
 * also hold, a fresh block replaces it in this sequence's table and *cow_src / *cow_dst name
 * the copy that must reach the device before the write (pa_copy_blocks); otherwise both are -1.
 * cow_src / cow_dst may be NULL only if the caller knows no copy can arise. */
int pa_seq_append_slot(pa_allocator* a, int32_t seq, int64_t* slot, int32_t* cow_src,
                       int32_t* cow_dst);

/* n successive appends to one sequence.  slots[n] receives each slot; cow_pairs[n][2] receives
 * the (src, dst) copies in order, *n_cow their count.  All or nothing. */
int pa_seq_reserve(pa_allocator* a, int32_t seq, int32_t n, int64_t* slots, int32_t* cow_pairs,
                   int32_t* n_cow);

/* One decode step's appends for a batch ([Serving] "The Life of a Request": each step appends
 * one token per request, allocating a block only when the current one fills).  For i in 0..B-1
 * in order, one append to seqs[i]:
 *   slots[i]        its slot;
 *   seq_lens[i]     (may be NULL) the sequence length after the append;
 *   table_index[i]  (may be NULL) the logical block whose table entry now holds slots[i]/bs --
 *                   a new block or the copy that replaced a shared one -- or -1, so that a device
 *                   copy of the block tables can be patched (pa_update_block_tables,
 *                   pa_append_step);
 *   cow_pairs[*n_cow][2]  the (src, dst) copies, in batch order, that must reach the device
 *                   before any of the step's writes (pa_copy_blocks).  At most B entries.
 * All or nothing. */
int pa_step(pa_allocator* a, const int32_t* seqs, int32_t B, int64_t* slots, int32_t* seq_lens,
            int32_t* table_index, int32_t* cow_pairs, int32_t* n_cow);

/* Drop a sequence: each of its blocks loses a reference; blocks left with none go to the tail
 * of the free list in table order ([Serving] "The Life of a Request"), except published blocks,
 * which become evictable (see prefix caching below). */
int pa_seq_free(pa_allocator* a, int32_t seq);

/* ---- automatic prefix caching ([Serving] "Prefix Caching and Chunked Prefill" / "Automatic
 * prefix caching", "Putting It Together: The Life of a Request") ----
 * A sequence created by pa_seq_create_prefix knows its token ids.  Each of its blocks that is
 * full and whose ids are all known is published under a chained hash: FNV-1a (64-bit) over the
 * little-endian bytes of the parent hash followed by the block's bs token ids (int32), the first
 * block's parent being FNV-1a of the 8 salt bytes.  The hash covers the whole prefix, so a block
 * matches only when every token before it matches too; a different salt never matches.  A
 * published block whose last reference is released is not freed: it joins an LRU list of
 * evictable blocks (the sequence's blocks last-first, so prefixes outlive their extensions), can
 * still be matched, and is evicted -- oldest first, its hash dropped -- only when an allocation
 * finds the free list empty.  When two blocks hold the same content, the first published keeps
 * the hash.  Matches compare the stored ids too, so a hash collision never reuses a wrong block.
 * Sequences made by pa_seq_create never publish; with only those, nothing above changes. */

/* New sequence for a prompt of n token ids (copied), reusing the longest run of cached blocks
 * that match its leading full blocks among the first n - 1 tokens (at least one prompt token is
 * left to compute: generation needs its query).  *n_cached receives the number of tokens whose
 * K/V is already in the pool (a multiple of bs; the sequence's length); the caller reserves
 * slots for tokens n_cached..n-1 (pa_seq_reserve) and writes them.  salt: 0 or a per-tenant
 * value mixed into the first block's hash. */
int pa_seq_create_prefix(pa_allocator* a, const int32_t* tokens, int32_t n, uint64_t salt,
                         int32_t* seq, int32_t* n_cached);
/* Append n token ids to what a pa_seq_create_prefix sequence knows (generated tokens, before
 * or after their slots are reserved); newly complete blocks are published.  PA_ERR_INVALID for
 * a sequence made by pa_seq_create. */
int pa_seq_add_tokens(pa_allocator* a, int32_t seq, const int32_t* tokens, int32_t n);
/* Number of evictable cached blocks, and the list in eviction order (up to cap; *n = total). */
int pa_num_evictable(const pa_allocator* a, int32_t* n);
int pa_evictable_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n);
/* Whether a block is published, and its hash (0 when not). */
int pa_block_hash(const pa_allocator* a, int32_t block, uint64_t* hash, int32_t* cached);

/* ---- preemption by swapping ([Serving] "When memory runs out anyway": a preempted request's
 * blocks are freed; its KV is either dropped and recomputed later, or swapped out to CPU memory
 * and brought back) ----
 * The allocator also hands out blocks of a host swap pool (num_cpu_blocks blocks in the same
 * layout, e.g. pinned host memory) from a FIFO free list of its own.  A swapped-out sequence
 * keeps its length and token ids but holds no device blocks; calls that need its blocks return
 * PA_ERR_STATE until it is swapped in; pa_seq_len and pa_seq_free still work. */

/* Sets the swap pool size, once. */
int pa_alloc_set_swap(pa_allocator* a, int32_t num_cpu_blocks);
/* Swap a resident sequence out: each of its table's blocks gets a swap block (FIFO) and
 * pairs[j] = (device block, swap block) in table order, *n = count (cap must be >= the table
 * length, else PA_ERR_INVALID with *n set).  The device blocks are then released as by
 * pa_seq_free.  The caller copies the pairs device -> host (pa_swap_blocks) on the stream
 * before anything can write the released blocks.  PA_ERR_OOM (nothing changed) when the swap
 * pool is short. */
int pa_seq_swap_out(pa_allocator* a, int32_t seq, int32_t* pairs, int32_t cap, int32_t* n);
/* Swap a swapped-out sequence back in: fresh device blocks (allocated like any other, possibly
 * evicting cached ones), pairs[j] = (swap block, device block) in table order; the swap blocks
 * return to the tail of the swap free list.  The caller copies the pairs host -> device before
 * anything can reuse the swap blocks.  PA_ERR_OOM (nothing changed) when the device is short. */
int pa_seq_swap_in(pa_allocator* a, int32_t seq, int32_t* pairs, int32_t cap, int32_t* n);
int pa_num_free_swap(const pa_allocator* a, int32_t* n);

int pa_seq_len(const pa_allocator* a, int32_t seq, int32_t* len);
/* Copies up to `cap` table entries to out; *n receives the table length. */
int pa_seq_table(const pa_allocator* a, int32_t seq, int32_t* out, int32_t cap, int32_t* n);
/* Host block tables [B][max_blocks] (padded with -1) and lengths [B] for the listed sequences.
 * PA_ERR_INVALID if a table is longer than max_blocks. */
int pa_export_block_tables(const pa_allocator* a, const int32_t* seqs, int32_t B,
                           int32_t max_blocks, int32_t* tables, int32_t* seq_lens);
int pa_block_refcount(const pa_allocator* a, int32_t block, int32_t* rc);
int pa_num_free(const pa_allocator* a, int32_t* n);
/* Free list from head to tail: up to `cap` ids to out, *n receives its length. */
int pa_free_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n);

/* ================================================================================== */
/* Device entry points                                                                */
/* ================================================================================== */

/* Append one token per sequence ([Serving] "What the KV Cache Is": the cache grows by one
 * token's K and V per decode step; "The Life of a Request").  k_new, v_new: device [B][Hkv][D] in the
 * cache dtype (PA_F32 or PA_BF16; int8 caches are written by pa_kv_append_int8).
 * slot_mapping: device-readable [B] int64, -1 = skip this sequence.  Writes K into k_cache[slot/bs][g]
 * [slot%bs][:] and V into v_cache[slot/bs][g][:][slot%bs]; nothing else is touched.  Two
 * sequences must not share a slot.  Constraints: B >= 0, Hkv >= 1, D in {64, 128}, bs == 16. */
int pa_kv_append(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                 void* k_cache, void* v_cache, int32_t B, int32_t Hkv, int32_t D, int32_t bs,
                 int32_t NB, int32_t kv_dtype, void* stream);

/* Append into an int8 cache, quantising on the way (the write side of a quantised cache:
 * [Walkthrough] keeps KV as int8 with a scale per block and head).  k_new, v_new: device
 * [B][Hkv][D] in new_dtype (PA_F32 or PA_BF16); slot_mapping as for pa_kv_append; k_cache,
 * v_cache int8 in the usual layouts; k_scale, v_scale device [NB][Hkv] fp32.  Entries apply in
 * batch order; entries writing into the same block must be consecutive in the batch (one
 * token per sequence, or a sequence's chunk in order, both are).  Per (block, KV head), K and V
 * alike, all in fp32 with IEEE division and round-half-to-even: c = max|x| / 127 for the new
 * vector x; at offset 0 the block's scale becomes c; otherwise a c above the scale s grows the
 * scale to c and re-rounds the block's earlier codes, code = clamp(rint(code * (s / c)), -127,
 * 127); the new slot gets clamp(rint(x / scale), -127, 127), or 0 while the scale is 0.  So a
 * block's scale is always max|x| / 127 over its tokens; a block of zeros has scale 0. */
int pa_kv_append_int8(const void* k_new, const void* v_new, int32_t new_dtype,
                      const int64_t* slot_mapping, int8_t* k_cache, int8_t* v_cache,
                      float* k_scale, float* v_scale, int32_t B, int32_t Hkv, int32_t D,
                      int32_t bs, int32_t NB, void* stream);

/* pa_kv_append_int8 for a packed int4 cache (layout above): the same rule with 7 in place of
 * 127 -- scale = max|x| / 7 grown token by token, codes clamp(rint(x / scale), -7, 7), earlier
 * codes re-rounded by old/new when the scale grows.  k_cache, v_cache: the packed bytes. */
int pa_kv_append_int4(const void* k_new, const void* v_new, int32_t new_dtype,
                      const int64_t* slot_mapping, uint8_t* k_cache, uint8_t* v_cache,
                      float* k_scale, float* v_scale, int32_t B, int32_t Hkv, int32_t D,
                      int32_t bs, int32_t NB, void* stream);

/* Copy-on-write block copies ([Serving] "Sharing comes for free"; [Walkthrough] "Step 8").
 * pairs: device-readable [n][2] int32 (src, dst).  Copies the whole K and V tile of block src over block
 * dst, and for PA_I8 / PA_I4 also both scales (k_scale, v_scale must then be non-NULL).  Destinations
 * must be distinct and no destination may be another pair's source (the allocator never
 * produces either).  n == 0 enqueues nothing. */
int pa_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                   const int32_t* pairs, int32_t n, int32_t Hkv, int32_t D, int32_t bs,
                   int32_t NB, int32_t kv_dtype, void* stream);

/* Copy whole blocks between two pools of the same layout -- the device pool and a host swap
 * pool (pinned host memory, device-readable and -writable) for preemption by swapping, or any
 * two device pools: for i < n, block pairs[i][1] of the destination := block pairs[i][0] of the
 * source (K, V, and for PA_I8 / PA_I4 both scales, which must then all be non-NULL).  One launch for
 * the whole batch.  Pairs are device-readable int32 [n][2]; destination blocks must be
 * distinct; entries outside [0, src_blocks) or [0, dst_blocks) are skipped. */
int pa_swap_blocks(const void* src_k, const void* src_v, const float* src_k_scale,
                   const float* src_v_scale, int32_t src_blocks, void* dst_k, void* dst_v,
                   float* dst_k_scale, float* dst_v_scale, int32_t dst_blocks,
                   const int32_t* pairs, int32_t n, int32_t Hkv, int32_t D, int32_t bs,
                   int32_t kv_dtype, void* stream);

/* Patch a device block table after pa_step: for every i < B with table_index[i] >= 0,
 * block_tables[i][table_index[i]] = slots[i] / bs.  slots (int64) and table_index (int32) are
 * device-readable [B] arrays; entries outside [0, max_blocks) are skipped. */
int pa_update_block_tables(int32_t* block_tables, int32_t max_blocks, const int64_t* slots,
                           const int32_t* table_index, int32_t B, int32_t bs, void* stream);

/* The device side of a decode step's bookkeeping in one launch, once its copy-on-write copies
 * (pa_copy_blocks) are enqueued: pa_kv_append, pa_update_block_tables, and
 * seq_lens_out[b] = seq_lens_in[b] (the lengths pa_step produced, for pa_decode).  Arguments as
 * for those calls; table_index may be NULL (no table changes); seq_lens_in / seq_lens_out are
 * both NULL (no copy) or both set: a device-readable and a device [B] int32 array.  With pa_step
 * writing its arrays into pinned host memory, this call reads them there directly. */
int pa_append_step(const void* k_new, const void* v_new, const int64_t* slot_mapping,
                   const int32_t* table_index, const int32_t* seq_lens_in, int32_t* seq_lens_out,
                   void* k_cache, void* v_cache, int32_t* block_tables, int32_t max_blocks,
                   int32_t B, int32_t Hkv, int32_t D, int32_t bs, int32_t NB, int32_t kv_dtype,
                   void* stream);

/* Bytes of scratch that pa_decode needs for these sizes (same partition_tokens as the decode
 * call).  Returns 0 for invalid sizes.  The size does not depend on the lengths themselves, so a
 * buffer sized once for the largest max_seq_len serves every step. */
size_t pa_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                int32_t max_seq_len, int32_t partition_tokens);

/* Decode attention over the paged cache ([Serving] "What the KV Cache Is": the new token's
 * query is compared with the key of every cached token and the values are mixed by those
 * weights; "PagedAttention": the kernel follows the block table to gather K and V; grouped-query
 * attention: query head h reads KV head h / (Hq/Hkv)).  For every b < B and h < Hq:
 *     out[b][h] = sum_t softmax_t(scale * <q[b][h], K_t>) V_t,  t < seq_lens[b],
 * token t at block_tables[b][t/bs], offset t%bs; int8 elements are code * scale of their
 * (block, KV head).  seq_lens[b] == 0 gives out[b] = 0.
 *   q_dtype:  PA_F32 or PA_BF16.  kv_dtype: PA_F32, PA_BF16, PA_I8 or PA_I4 (then
 *   k_scale/v_scale; PA_I4 needs a PA_BF16 q and Hq/Hkv in {1, 2, 4, 8, 16}, else
 *   PA_ERR_UNSUPPORTED).
 *   Hq % Hkv == 0, Hq/Hkv <= 16, D in {64, 128}, bs == 16.
 *   max_seq_len: host bound on every seq_lens[b], 0 <= max_seq_len <= max_blocks*bs.
 *   partition_tokens: 0 = balanced schedule: the block pairs of all (sequence, KV head)
 *     segments are split into equal spans, one per resident workgroup, whatever the length
 *     mix.  It runs for a PA_BF16 q over PA_BF16, PA_I8 or PA_I4 caches with Hq/Hkv <= 8 and
 *     B <= 8192; everything else (PA_F32 q or cache, Hq/Hkv == 16, larger B) falls back to
 *     fixed partitions of 512 tokens, or of 8192 when B*Hkv >= 1024 (the batch alone then fills
 *     the device).  Otherwise a multiple of 64 in [64, 8192]: one workgroup per
 *     partition of that many tokens.  Either way a segment cut into several pieces ("split-K")
 *     is merged with the log-sum-exp identity, in a fixed order: repeated calls on the same
 *     inputs give bit-identical outputs.
 *   workspace: device buffer of workspace_bytes >= pa_decode_workspace_size(...); its contents
 *     need no initialisation and are scratch after the call.  Calls that overlap in time must
 *     not share a workspace.
 *   Quantised caches (PA_I8, PA_I4) run the products in fp16: q and P * v_scale are rounded to
 *   fp16, so |q| must stay below 65504 and v_scale below 2^14; beyond that the result is not
 *   finite.  The scales of blocks a sequence does not read (table entries past its length or
 *   outside [0, NB)) never enter its result, whatever they hold (NaN included).
 * The softmax runs in fp32 with exp computed as exp2 of a log2(e)-scaled argument. */
int pa_decode(float* out, const void* q, int32_t q_dtype, const void* k_cache,
              const void* v_cache, int32_t kv_dtype, const float* k_scale, const float* v_scale,
              const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
              int32_t max_seq_len, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs,
              int32_t NB, float scale, int32_t partition_tokens, void* workspace,
              size_t workspace_bytes, void* stream);

/* pa_decode for callers that cannot allocate device memory: code being captured into a HIP
 * graph, tight serving loops, harnesses that forbid allocation.  Same arguments, results and
 * schedules as pa_decode, without the workspace: the partial states of split segments live in
 * one fixed buffer of PA_DECODE_SCRATCH_BYTES per GPU, a file-scope device array of the library
 * (held until the process ends).  Nothing is allocated or freed.  A call whose schedule needs
 * more scratch than that (the balanced schedule needs at most ~8.4 MiB; fixed partitions need
 * B*Hq*ceil(max_seq_len/partition)*(D+2)*4 bytes) returns PA_ERR_TOO_LARGE and enqueues
 * nothing.  Every call on one GPU shares that GPU's buffer: calls that overlap in time on one
 * GPU (other streams, other threads) race and must be serialised by the caller.  The buffer's
 * contents need no initialisation and carry nothing from one call to the next. */
#define PA_DECODE_SCRATCH_BYTES (16u << 20)
int pa_decode_no_alloc(float* out, const void* q, int32_t q_dtype, const void* k_cache,
                       const void* v_cache, int32_t kv_dtype, const float* k_scale,
                       const float* v_scale, const int32_t* block_tables, int32_t max_blocks,
                       const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t Hq,
                       int32_t Hkv, int32_t D, int32_t bs, int32_t NB, float scale,
                       int32_t partition_tokens, void* stream);

/* Bytes of scratch that pa_decode_shared_prefix needs for these sizes; 0 for invalid sizes.
 * At least pa_decode_workspace_size(B, Hq, Hkv, D, max_seq_len, 0). */
size_t pa_decode_shared_prefix_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                                              int32_t max_seq_len);

/* pa_decode (balanced schedule) that reads a shared prefix once per group instead of once per
 * sequence ([Serving] "Sharing comes for free": the tables of sequences with a common prompt
 * name the same physical blocks for it; [Walkthrough] "Step 8": a shared prefix is stored
 * once).
 * Same arguments and result as pa_decode with partition_tokens = 0; the sums are taken in a
 * different order, so outputs agree with pa_decode's to rounding, not bit for bit (repeated
 * calls are bit-identical).
 *   Groups: a run of consecutive batch entries, inside an aligned window of 64, whose tables
 *     start with the same block in [0, NB).  The library finds them on the device: callers
 *     that want the saving put sequences that share a prefix next to each other.  Within a
 *     group, member b shares with the longest member (the first on ties) the tokens below
 *     min(seq_lens[b], 16 k) rounded down to a multiple of 32, k = leading table entries equal
 *     and in [0, NB) in both; those are read once per KV head for up to 16 query heads (of
 *     several members) at a time, and b's other tokens as in pa_decode.  The tables alone decide: a run of unrelated sequences costs nothing
 *     but the detection.
 *   Runs its own schedule for a PA_BF16 q over PA_BF16, PA_I8 or PA_I4 caches with Hq/Hkv in
 *     {1, 2, 4, 8} and B <= 8192; any other valid call is pa_decode(..., 0, ...).
 *   workspace: device buffer of workspace_bytes >= pa_decode_shared_prefix_workspace_size();
 *     needs no initialisation; calls that overlap in time must not share it.
 *   Four launches on `stream`: the group plan, the prefix pass, the decode of every sequence
 *   past its prefix, and a merge launch that combines split segments and folds the prefix
 *   states into every row with a shared prefix (log-sum-exp).  Errors as for pa_decode. */
int pa_decode_shared_prefix(float* out, const void* q, int32_t q_dtype, const void* k_cache,
                            const void* v_cache, int32_t kv_dtype, const float* k_scale,
                            const float* v_scale, const int32_t* block_tables, int32_t max_blocks,
                            const int32_t* seq_lens, int32_t max_seq_len, int32_t B, int32_t Hq,
                            int32_t Hkv, int32_t D, int32_t bs, int32_t NB, float scale,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Chunked-prefill attention over the paged cache ([Serving] "Two Phases: Prefill and Decode":
 * prefill runs a prompt's tokens in parallel, each attending to all earlier ones; "Prefix
 * Caching and Chunked Prefill" / "Chunked prefill": a long prefill runs as a series of chunks).
 * Sequence b's chunk is query rows cu_q[b] .. cu_q[b+1]-1 of q, the last n_b = cu_q[b+1]-cu_q[b]
 * of its seq_lens[b] tokens, whose K/V are already in the cache (pa_kv_append with one batch
 * entry per token).  Query i of the chunk sits at position p = seq_lens[b] - n_b + i:
 *     out[row][h] = sum_{t <= p} softmax_t(scale * <q[row][h], K_t>) V_t   (KV head h/(Hq/Hkv)),
 * and a row with p < 0 gets zeros.
 *   q: device [T][Hq][D] PA_BF16 (PA_F32: PA_ERR_UNSUPPORTED).
 *   k_cache / v_cache: PA_BF16, PA_I8 or PA_I4 in the layouts above (PA_F32:
 *   PA_ERR_UNSUPPORTED); for PA_I8 / PA_I4 also k_scale / v_scale, device [NB][Hkv] fp32
 *   (element = code * scale), else ignored.  Quantised caches run the products in fp16: q and
 *   P * v_scale are rounded to fp16, and v_scale must stay below 2^14 (|V| below 2^21 for int8).
 *   A PA_BF16 cache runs P . V in fp16 too: P rounded to fp16, V converted exactly, so |V| must
 *   stay below 65504 (beyond, the result is not finite); the scores stay in bf16.
 *   out: device [T][Hq][D] fp32; cu_q: device [B + 1] int32, non-decreasing, cu_q[0] = 0,
 *   cu_q[B] = T; seq_lens: device [B] int32; max_seq_len bounds every seq_lens[b];
 *   Hq/Hkv in {1, 2, 4, 8, 16}, D in {64, 128}, bs == 16.  Needs no workspace.  Compute-bound:
 *   each K/V tile is shared by 16 queries of every head of its group. */
int pa_prefill(float* out, const void* q, int32_t q_dtype, const void* k_cache,
               const void* v_cache, int32_t kv_dtype, const float* k_scale, const float* v_scale,
               const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
               const int32_t* cu_q, int32_t max_seq_len, int32_t B, int32_t T, int32_t Hq,
               int32_t Hkv, int32_t D, int32_t bs, int32_t NB, float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
