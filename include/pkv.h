/*
 * pkv.h -- C ABI of libpkv, a PagedAttention library for AMD Instinct MI355X (gfx950).
 *
 * Pages this header cites (title, then where on the page):
 *   [Shootout]         "LLM Serving Engine Shootout: vLLM vs TensorRT-LLM vs SGLang vs llama.cpp"
 *                      (initnode.dev), sections 1.1, 2.1, 3.1, 3.2, 5.1.
 *   [Serving Engines]  "Serving Engines" (inference.tusharamrit.in), part "How vLLM works".
 *   [Inference Engines] "Inference Engines: vLLM, SGLang, TensorRT-LLM" (ragyfied.com),
 *                      parts "PagedAttention" and "Prefix caching".
 *   [VRAM black hole]  zhichai.net topic 178634546 (Chinese original), section 1, the ASCII
 *                      figure of logical blocks, block table and physical blocks; section 4,
 *                      the KV-cache memory formula (FP8: one byte per element).
 *
 * What the library computes
 * -------------------------
 * The KV cache of every sequence lives in fixed-size physical blocks of `block_size` tokens
 * (16 or 32) drawn from one pool shared by all sequences [Shootout 3.1; Serving Engines].
 * A per-sequence block table maps logical block i (tokens i*B .. i*B+B-1) to a physical block
 * anywhere in the pool [Shootout 3.1; Inference Engines "PagedAttention"]. Token j of a
 * sequence therefore sits in physical block table[j / B] at offset j % B: the equation in
 * [Shootout 3.1] gives the block index, the figure in [VRAM black hole section 1] (tokens 0-15
 * in physical block #7, tokens 16-31 in #2) gives the offset. The attention kernels locate K and
 * V through the block table; new tokens are placed by a per-token slot index [Serving Engines].
 *
 * Pool layout (fixed by this ABI; the pages leave it open)
 * ---------------------------------------------------------
 *   k_pool: [num_blocks][num_kv_heads][block_size][head_dim]   (token-major inside a tile)
 *   v_pool: [num_blocks][num_kv_heads][head_dim][block_size]   (dim-major inside a tile)
 * Both row-major, element type `dtype`. One (block, kv_head) tile of either pool is one
 * contiguous run of block_size*head_dim elements. The element for token offset `o`, head `h`,
 * dimension `d` of physical block `b` is at
 *   k_pool[((b*Hkv + h)*B + o)*D + d]      v_pool[((b*Hkv + h)*D + d)*B + o]
 * (index arithmetic is done in 64-bit). V is stored dim-major because the P*V product contracts
 * over tokens, and a matrix-core operand wants its contraction index contiguous per lane.
 *
 * A slot is the flat token position blk*B + off in the pool.
 *
 * Conventions for every call
 * --------------------------
 *  - All array pointers are DEVICE pointers owned by the caller. The library allocates no
 *    device memory, keeps no device state between calls and never synchronises; each call
 *    enqueues its kernels on `stream` (a hipStream_t passed as void*; NULL = null stream) and
 *    returns. Calls are thread-safe.
 *  - Return value: a pkv_status. Arguments are validated on the host before any HIP call; a
 *    failure returns without launching anything. PKV_ERR_HIP reports a kernel launch that the
 *    HIP runtime refused (the status of that launch; a call of two kernels launches the second
 *    only if the first was accepted). Faults inside a kernel surface later, at the caller's
 *    next synchronisation, as HIP errors of the caller's own calls.
 *    pkv_last_error() returns a thread-local text for the last non-OK status of the thread.
 *  - dtype PKV_F32 or PKV_BF16 (bf16 = IEEE binary32 truncated to the top 16 bits).
 *    head_dim in {64, 128}; block_size in {16, 32}; num_q_heads % num_kv_heads == 0.
 *    Anything else returns PKV_ERR_UNSUPPORTED.
 *  - Query head h uses KV head h / (num_q_heads / num_kv_heads) (consecutive grouping, GQA
 *    [Shootout 2.1]).
 *  - Device-array preconditions the host cannot check without a synchronisation, and which
 *    the caller must guarantee (a violation is undefined behaviour):
 *      block ids in block_table[s][0 .. ceil(context_lens[s]/B)-1] lie in [0, num_blocks);
 *      0 <= context_lens[s] <= max_blocks_per_seq*B, and <= max_context_len when one is given;
 *      non-negative slots in slot_mapping are < num_blocks*B and pairwise distinct.
 *    Block-table entries past ceil(context_lens[s]/B) are never read.
 *    Debug builds (libpkv_debug.so, compiled with PKV_DEBUG=1) check them on the device: every
 *    call first runs check kernels over the arrays it was handed (block ids it would read,
 *    context lengths, slots, chunk bounds, prefix groups, copy pairs; the distinctness of slots
 *    is not checked), waits for them (so debug calls synchronise their stream), and launches its
 *    own kernels only if nothing was found; otherwise it returns PKV_ERR_DEVICE_ARG, launches
 *    nothing and leaves every output untouched. pkv_debug_found() gives what was found.
 *  - Sharing: several block tables may name the same physical block (shared prefixes,
 *    [Inference Engines "PagedAttention"; Serving Engines]). The attention calls only read the
 *    pools; writing into a shared block is the caller's error (fork it first).
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ABI_VERSION 2

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, inconsistent sizes */
  PKV_ERR_UNSUPPORTED = 2, /* dtype / head_dim / block_size / grouping not built */
  PKV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  PKV_ERR_HIP = 4,         /* a HIP runtime call failed; see pkv_last_error() */
  PKV_ERR_OUT_OF_BLOCKS = 5, /* block manager: not enough free blocks (nothing was changed) */
  PKV_ERR_DEVICE_ARG = 6     /* debug builds: a device array breaks a precondition (see above) */
} pkv_status;

/* PKV_FP8_E4M3: pools only (pkv_kv_cache_write_fp8, pkv_paged_attention_decode_fp8,
 * pkv_kv_cache_copy_blocks): one byte per element in the OCP 8-bit floating point E4M3 format
 * (1 sign, 4 exponent bits with bias 7, 3 fraction bits; no infinity; S.1111.111 is NaN;
 * largest finite 448). */
typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 } pkv_dtype;

/* Library plumbing (not defined by the pages). */
int pkv_abi_version(void);
const char* pkv_status_string(int status);
const char* pkv_last_error(void);
/* 1 in a debug build (device-array checks before every call, see above), else 0. */
int pkv_debug_build(void);
/* Debug builds: what the checks of this thread's last call found, as a mask -- 1 block id
 * outside the pool, 2 context length out of range, 4 slot outside the pool, 8 chunk bounds
 * (cu_q_lens) invalid, 16 prefix groups invalid, 32 copy pair outside its pool; 0 when the call
 * was clean. Release builds: 0. */
unsigned pkv_debug_found(void);

/*
 * pkv_kv_cache_write -- scatter new K/V rows into pool slots through a slot mapping.
 * [Serving Engines, "How vLLM works": the kernel works from a block table and a slot mapping;
 *  a sequence claims a new block only when its current one is full.]
 * [Inference Engines, "PagedAttention": blocks are allocated as the sequence grows.]
 *
 *   k_new, v_new  [T][num_kv_heads][head_dim], dtype        (read)
 *   k_pool        [num_blocks][num_kv_heads][block_size][head_dim]  (written in place)
 *   v_pool        [num_blocks][num_kv_heads][head_dim][block_size]  (written in place)
 *   slot_mapping  int32 [T]; token i goes to slot slot_mapping[i] = blk*B + off; a negative
 *                 slot skips the token.
 * For every i with slot >= 0 and every head h, dimension d:
 *   k_pool[blk][h][off][d] = k_new[i][h][d],  v_pool[blk][h][d][off] = v_new[i][h][d].
 * A pure bit copy: no rounding, NaN payloads preserved. Slots not named are left untouched.
 * T == 0 is a no-op that returns PKV_OK.
 */
pkv_status pkv_kv_cache_write(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                              const int32_t* slot_mapping, int T, int num_kv_heads, int head_dim,
                              int block_size, int num_blocks, int dtype, void* stream);

/*
 * pkv_kv_cache_write_fp8 -- pkv_kv_cache_write into E4M3 pools, quantising on the way.
 * [VRAM black hole section 4: FP8 stores a cached element in one byte; Serving Engines "What
 *  they all agree on": engines quantise the KV cache.] The pages give no scaling scheme; this
 *  call takes one float32 scale per pool.
 *
 *   k_new, v_new   [T][num_kv_heads][head_dim], in_dtype PKV_BF16 or PKV_F32   (read)
 *   k_pool, v_pool uint8 E4M3 codes, layout above                            (written in place)
 *   k_scale, v_scale  finite, > 0
 * Element x of k_new is stored as code(x / k_scale), v_new's with v_scale, where the quotient
 * is the IEEE float32 quotient (correctly rounded) and code() picks the E4M3 value nearest to
 * it, ties to the code with an even last bit; magnitudes beyond 448 (and infinities) saturate
 * to +-448; the sign bit follows the quotient's sign; NaN stores 0x7F. Placement, skipped
 * slots and preconditions are those of pkv_kv_cache_write.
 */
pkv_status pkv_kv_cache_write_fp8(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                  const int32_t* slot_mapping, int T, int num_kv_heads,
                                  int head_dim, int block_size, int num_blocks, int in_dtype,
                                  float k_scale, float v_scale, void* stream);

/*
 * pkv_kv_cache_copy_blocks -- copy whole physical blocks between two pools (or inside one).
 * ["Serving Engines", How vLLM works: copy-on-write -- when one of several sequences sharing a
 *  block writes into it, only that block is copied and the block tables split there; swap
 *  preemption moves a sequence's blocks to host memory and back.]
 *
 *   src_k, src_v   source pools, layout above (read)
 *   dst_k, dst_v   destination pools, same layout and dtype (written); may equal the sources
 *   dtype          PKV_F32, PKV_BF16 or PKV_FP8_E4M3 (only the element size matters)
 *   block_pairs    int32 [n_pairs][2]: (source block, destination block), device-accessible
 *   src_num_blocks, dst_num_blocks  pool sizes (for the caller's bookkeeping and validation)
 * For each pair every KV head's K tile and V tile of the destination block becomes a bit copy
 * of the source block's. Any of the four pools may be pinned host memory (hipHostMalloc):
 * copying a device pool to a host pool and back is the swap-out / swap-in of preemption.
 * Preconditions (unchecked, device data): ids within their pools; destination blocks pairwise
 * distinct; within one pool, no destination is also a source. n_pairs == 0 is a no-op.
 */
pkv_status pkv_kv_cache_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                                    const int32_t* block_pairs, int n_pairs, int num_kv_heads,
                                    int head_dim, int block_size, int src_num_blocks,
                                    int dst_num_blocks, int dtype, void* stream);

/*
 * Block manager -- host-side allocator of physical blocks with reference counts, for the
 * bookkeeping around the kernels. ["Serving Engines", How vLLM works: a sequence claims a new
 * block only when its current one fills; a reference count per block tracks sharing; a write
 * into a shared block copies that block only. "Inference Engines", PagedAttention: blocks are
 * freed when the sequence finishes.] Single-writer: not thread-safe.
 *
 *   pkv_bm_create(num_blocks, block_size, &bm)  all blocks free; ids handed out lowest first
 *   pkv_bm_destroy(bm)
 *   pkv_bm_num_free(bm)                         free blocks
 *   pkv_bm_add(bm, seq)                         new empty sequence (PKV_ERR_INVALID_ARG if the
 *                                               id exists)
 *   pkv_bm_fork(bm, parent, child)              child shares every block of parent (counts+1)
 *   pkv_bm_append(bm, seq, n, slots, copies, max_copies, &n_copies)
 *       reserves slots for the next n tokens of seq: slots[i] = block * B + offset of token
 *       len + i. If the last block is shared and partly filled, it is first copied to a fresh
 *       block (copy-on-write): the pair (old, new) is written to copies[0..1] and n_copies = 1;
 *       otherwise n_copies = 0. New blocks are claimed as positions cross block boundaries.
 *       All or nothing: PKV_ERR_OUT_OF_BLOCKS if the pool cannot supply the blocks.
 *   pkv_bm_free(bm, seq)                        drops seq; blocks whose count reaches 0 return
 *                                               to the pool
 *   pkv_bm_context_len(bm, seq, &len)
 *   pkv_bm_block_table(bm, seq, table, capacity, &n_blocks)  copies up to capacity ids
 *   pkv_bm_refcount(bm, block, &count)
 */
typedef struct pkv_block_manager pkv_block_manager;
pkv_status pkv_bm_create(int num_blocks, int block_size, pkv_block_manager** out);
void pkv_bm_destroy(pkv_block_manager* bm);
int pkv_bm_num_free(const pkv_block_manager* bm);
pkv_status pkv_bm_add(pkv_block_manager* bm, int64_t seq);
pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child);
pkv_status pkv_bm_append(pkv_block_manager* bm, int64_t seq, int n_tokens, int32_t* slots,
                         int32_t* copies, int max_copies, int* n_copies);
pkv_status pkv_bm_free(pkv_block_manager* bm, int64_t seq);
pkv_status pkv_bm_context_len(const pkv_block_manager* bm, int64_t seq, int* len);
pkv_status pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq, int32_t* table,
                              int capacity, int* n_blocks);
pkv_status pkv_bm_refcount(const pkv_block_manager* bm, int block, int* count);

/*
 * pkv_decode_partition_size -- the fixed partition size, in tokens, that
 * pkv_paged_attention_decode uses for these arguments; 0 when it uses the balanced split
 * (partition_size == 0 with bf16 inputs). Library plumbing.
 * Returns -1 for a partition_size that is negative or not a multiple of 16.
 */
int pkv_decode_partition_size(int partition_size, int num_seqs, int num_kv_heads,
                              int max_context_len, int dtype);

/*
 * pkv_decode_workspace_size -- bytes of device workspace pkv_paged_attention_decode needs for
 * these sizes (0 when fixed partitions leave a single partition, so no partials are stored).
 * With dtype PKV_FP8_E4M3 (partition_size ignored): what pkv_paged_attention_decode_fp8
 * needs. Library plumbing.
 */
size_t pkv_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int max_context_len, int partition_size, int dtype);

/*
 * pkv_paged_attention_decode -- one query token per sequence against its paged context.
 * [Shootout 3.1, the displayed equation: score A_ij = q_i . k_j / sqrt(d_head) with k_j fetched
 *  via BlockTable[floor(j / B_size)].] [Shootout 5.1: softmax of the scores, then the product
 *  with V.] [Shootout 2.1: grouped-query attention, fewer KV heads than query heads.]
 *
 * For sequence s with n = context_lens[s] (the count of cached tokens, including the current
 * one, whose K/V must already be written) and query head h with KV head g:
 *   a_j = scale * sum_d q[s][h][d] * K_s[g][j][d],     j = 0 .. n-1
 *   out[s][h][:] = sum_j softmax(a)_j * V_s[g][j][:]
 * where K_s, V_s are the sequence's K/V gathered through block_table (see above).
 * n == 0 writes zeros.
 *
 *   out           [num_seqs][num_q_heads][head_dim], out_dtype (written)
 *   q             [num_seqs][num_q_heads][head_dim], dtype
 *   k_pool/v_pool pool layout above, dtype
 *   block_table   int32 [num_seqs][max_blocks_per_seq]
 *   context_lens  int32 [num_seqs]
 *   scale         normally 1/sqrt(head_dim)
 *   max_context_len  host bound on context_lens (0 = max_blocks_per_seq*block_size)
 *   partition_size   how the contexts are split over the GPU's waves (split-context):
 *                    > 0: fixed partitions of that many tokens (a multiple of 16 and of
 *                         block_size); each partition of each (sequence, KV head) is one work
 *                         unit.
 *                    0:   bf16 inputs: balanced split -- the batch's 32-token tiles, in
 *                         (sequence, KV head, position) order, are dealt in equal contiguous
 *                         shares to num_waves waves, so every wave does the same work whatever
 *                         the mix of context lengths. fp32 inputs: fixed partitions of a
 *                         default size.
 *                    A context cut into several pieces is merged by a second kernel: each piece
 *                    leaves (max, sum of exponentials, normalised output) and the merge weighs
 *                    them by log-sum-exp. The result is the same softmax up to floating-point
 *                    rounding.
 *   num_waves     waves of the balanced split (0 = the default, 1024); fewer are used when the
 *                 batch has under 8 tiles per wave. Ignored with fixed partitions.
 *                 Must lie in [0, 2^20].
 *   workspace     device buffer of at least pkv_decode_workspace_size(...) bytes (may be NULL
 *                 when that size is 0); contents on entry are ignored.
 * out_dtype may differ from dtype (e.g. bf16 inputs with an fp32 output); the bf16 output is
 * rounded to nearest even from the fp32 result.
 */
pkv_status pkv_paged_attention_decode(void* out, const void* q, const void* k_pool,
                                      const void* v_pool, const int32_t* block_table,
                                      const int32_t* context_lens, int num_seqs, int num_q_heads,
                                      int num_kv_heads, int head_dim, int block_size,
                                      int max_blocks_per_seq, int num_blocks, float scale,
                                      int max_context_len, int partition_size, int num_waves,
                                      void* workspace, size_t workspace_bytes, int dtype,
                                      int out_dtype, void* stream);

/*
 * pkv_kv_cache_write_and_decode -- pkv_kv_cache_write of each sequence's new token followed by
 * pkv_paged_attention_decode, with the same results, the write folded into the attention
 * kernel (bf16 pools). [Serving Engines "How vLLM works": each decode step writes the new
 * token's K/V through the slot mapping and attends over the whole context; Shootout 3.1 and 5.1
 * for the attention.]
 *
 *   k_new, v_new  [num_seqs][num_kv_heads][head_dim] bf16: sequence s's newest token, at
 *                 position context_lens[s] - 1
 *   slot_mapping  int32 [num_seqs]: that token's slot (the block table's slot for position
 *                 n - 1), or negative when the pool already holds every token of s
 *   k_pool, v_pool  read, and written at the new tokens' slots
 *   workspace     pkv_decode_workspace_size(..., partition_size = 0, PKV_BF16) bytes
 * Other arguments (num_waves included), preconditions and errors as for
 * pkv_paged_attention_decode with the balanced split. The attention takes the newest token's
 * K/V from k_new / v_new, and the wave that does so also stores them into the pool, so no
 * kernel has to wait for the write.
 */
pkv_status pkv_kv_cache_write_and_decode(void* out, const void* q, const void* k_new,
                                         const void* v_new, const int32_t* slot_mapping,
                                         void* k_pool, void* v_pool, const int32_t* block_table,
                                         const int32_t* context_lens, int num_seqs, int num_q_heads,
                                         int num_kv_heads, int head_dim, int block_size,
                                         int max_blocks_per_seq, int num_blocks, float scale,
                                         int max_context_len, int num_waves, void* workspace,
                                         size_t workspace_bytes, int out_dtype, void* stream);

/*
 * pkv_paged_attention_decode_fp8 -- pkv_paged_attention_decode over E4M3 pools.
 * [VRAM black hole section 4: FP8 halves the bytes per cached element; Shootout 3.1 and 5.1 for
 *  the attention itself, as above.]
 * The pools hold E4M3 codes written by pkv_kv_cache_write_fp8 with the same k_scale and
 * v_scale (finite, > 0); K's value is code value * k_scale, V's is code value * v_scale, and
 * with those values the result is pkv_paged_attention_decode's. q is bf16; out_dtype PKV_BF16
 * or PKV_F32. The context is always split the balanced way over num_waves waves (0 = the
 * default, 1024); workspace: pkv_decode_workspace_size(..., dtype = PKV_FP8_E4M3) bytes.
 * Other arguments, preconditions and errors as for pkv_paged_attention_decode. Unwritten slots
 * may hold any code, NaN included.
 */
pkv_status pkv_paged_attention_decode_fp8(void* out, const void* q, const void* k_pool,
                                          const void* v_pool, const int32_t* block_table,
                                          const int32_t* context_lens, int num_seqs,
                                          int num_q_heads, int num_kv_heads, int head_dim,
                                          int block_size, int max_blocks_per_seq, int num_blocks,
                                          float scale, float k_scale, float v_scale,
                                          int max_context_len, int num_waves, void* workspace,
                                          size_t workspace_bytes, int out_dtype, void* stream);

/*
 * pkv_paged_attention_decode_shared_prefix -- decode for batches whose sequences share
 * prompt prefixes, reading each shared prefix once per group instead of once per sequence.
 * [Inference Engines "Prefix caching" and Serving Engines "How vLLM works": sequences with a
 *  common prompt prefix point their block tables at the same physical blocks; Shootout 3.2:
 *  shared blocks are copy-on-write.] The result is pkv_paged_attention_decode's (bf16 pools) or
 * pkv_paged_attention_decode_fp8's (E4M3 pools); only the order of the arithmetic differs.
 *
 *   group_start       int32 [num_groups+1], device: group i is sequences group_start[i] ..
 *                     group_start[i+1]-1 (groups are consecutive runs covering the batch:
 *                     group_start[0] = 0, non-decreasing, group_start[num_groups] = num_seqs)
 *   group_prefix_len  int32 [num_groups], device: tokens every member of group i shares, a
 *                     multiple of block_size; the first group_prefix_len[i] / block_size
 *                     entries of the members' block tables are the same physical blocks (the
 *                     kernel reads them from the first member's table); <= each member's
 *                     context_len; 0 = no sharing
 *   max_group_size, max_prefix_len  host bounds on group sizes and group_prefix_len
 *                     (max_prefix_len a multiple of block_size)
 *   kv_dtype          PKV_BF16 or PKV_FP8_E4M3 (then k_scale, v_scale as for the fp8 decode;
 *                     ignored for bf16); q is bf16; out_dtype PKV_BF16 or PKV_F32
 *   workspace         pkv_decode_shared_prefix_workspace_size(...) bytes
 * Other arguments as for pkv_paged_attention_decode (num_waves: waves of the balanced split of
 * the private suffixes, 0 = the default: as many as fill the compute units that the prefix
 * workgroups leave, eight per unit; fewer are used when the suffixes have under 3 (bf16) or 4
 * (E4M3) tiles of 32 tokens per wave). Each shared prefix is split into chunks of 256 tokens;
 * one workgroup of eight waves stages a chunk's K/V in LDS as bf16 (E4M3 codes widened exactly)
 * and attends it for up to 256 (member, query head) rows. The private rest of every context
 * goes through the balanced split, and a reduce kernel merges the pieces by log-sum-exp.
 */
size_t pkv_decode_shared_prefix_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                               int head_dim, int max_context_len,
                                               int max_prefix_len, int kv_dtype);
pkv_status pkv_paged_attention_decode_shared_prefix(void* out, const void* q, const void* k_pool,
                                                    const void* v_pool, const int32_t* block_table,
                                                    const int32_t* context_lens,
                                                    const int32_t* group_start,
                                                    const int32_t* group_prefix_len, int num_groups,
                                                    int max_group_size, int max_prefix_len,
                                                    int num_seqs, int num_q_heads, int num_kv_heads,
                                                    int head_dim, int block_size,
                                                    int max_blocks_per_seq, int num_blocks,
                                                    float scale, int max_context_len, int num_waves,
                                                    int kv_dtype, float k_scale, float v_scale,
                                                    void* workspace, size_t workspace_bytes,
                                                    int out_dtype, void* stream);

/*
 * pkv_paged_attention_prefill_chunk -- a causal chunk of query tokens against the paged cache.
 * [Serving Engines, "How vLLM works": chunked prefill slices a long prompt into pieces that run
 *  interleaved with other sequences' decode steps.] [Shootout 3.1 equation, as for decode.]
 * [Shootout 3.2; Serving Engines: shared-prefix blocks are read through the block table like
 *  any other block.]
 *
 * Sequence s owns query rows cu_q_lens[s] .. cu_q_lens[s+1]-1 (chunk length c = the
 * difference) and n = context_lens[s] cached tokens, which INCLUDE the chunk's own K/V
 * (written beforehand with pkv_kv_cache_write). The chunk follows r = n - c earlier tokens,
 * so chunk row i sits at absolute position r + i and attends to tokens 0 .. r + i (the causal
 * mask is aligned to the end of the context). Requires 0 <= c <= n for every sequence.
 *
 *   out          [total_q][num_q_heads][head_dim], out_dtype (written)
 *   q            [total_q][num_q_heads][head_dim], dtype; sequences packed in order
 *   cu_q_lens    int32 [num_seqs+1], cu_q_lens[0] = 0, non-decreasing, cu_q_lens[S] = total_q
 *   context_lens int32 [num_seqs]
 *   max_q_len, max_context_len  host bounds on c and n (0 = total_q and
 *                               max_blocks_per_seq*block_size)
 */
pkv_status pkv_paged_attention_prefill_chunk(void* out, const void* q, const int32_t* cu_q_lens,
                                             const int32_t* context_lens, const void* k_pool,
                                             const void* v_pool, const int32_t* block_table,
                                             int num_seqs, int total_q, int num_q_heads,
                                             int num_kv_heads, int head_dim, int block_size,
                                             int max_blocks_per_seq, int num_blocks, float scale,
                                             int max_q_len, int max_context_len, int dtype,
                                             int out_dtype, void* stream);

/*
 * pkv_paged_attention_decode_noalloc -- pkv_paged_attention_decode (bf16 inputs, balanced
 * split) for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. It takes no workspace and allocates nothing:
 * the partials live in a static device array of the library, 128 MiB per GPU (held from the
 * first use of the library on that GPU until the process ends), whose address is looked up once
 * per device on the first call made with it current.
 *   Arguments as for pkv_paged_attention_decode with dtype = PKV_BF16 and partition_size = 0;
 *   the results are the same bit for bit.
 *   Returns PKV_ERR_WORKSPACE, before any HIP call, when these sizes would need more than the
 *   128 MiB (pkv_decode_workspace_size(..., 0, PKV_BF16) bytes; e.g. 64 sequences of up to 4096
 *   tokens with 32/8 heads need 17 MiB, 32 of up to 32768 tokens with 64/8 heads 120 MiB).
 *   Every call on one GPU uses that GPU's one array, and the array keeps the last call's
 *   contents (nothing in it has to start at zero): calls that overlap on one GPU (other streams,
 *   other threads) race and give wrong results; calls in order on one stream do not.
 */
pkv_status pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_pool,
                                              const void* v_pool, const int32_t* block_table,
                                              const int32_t* context_lens, int num_seqs,
                                              int num_q_heads, int num_kv_heads, int head_dim,
                                              int block_size, int max_blocks_per_seq,
                                              int num_blocks, float scale, int max_context_len,
                                              int num_waves, int out_dtype, void* stream);

/*
 * pkv_decode_read_probe -- measurement only, not part of the attention path. Launches the
 * balanced split of pkv_paged_attention_decode (bf16 pools, the same num_waves rule) with the
 * same waves reading the same K/V tiles with the same loads, but without the attention
 * arithmetic: each lane folds the words it loaded into one XOR and stores it to sink. The
 * decode's time over this probe's, on the same arguments, is how close the decode comes to a
 * bare read of exactly the bytes it must read [Shootout 1.1: decode is bound by memory
 * bandwidth]. Arguments as for pkv_paged_attention_decode; sink: device buffer of at least
 * pkv_decode_read_probe_sink_size(...) bytes (contents written are meaningless).
 */
size_t pkv_decode_read_probe_sink_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                       int max_context_len, int num_waves);
pkv_status pkv_decode_read_probe(const void* k_pool, const void* v_pool, const int32_t* block_table,
                                 const int32_t* context_lens, int num_seqs, int num_q_heads,
                                 int num_kv_heads, int head_dim, int block_size,
                                 int max_blocks_per_seq, int num_blocks, int max_context_len,
                                 int num_waves, void* sink, size_t sink_bytes, void* stream);

/*
 * Kernel timing (library plumbing, for benchmarks). For every kernel selected by the mask, the
 * library passes a pair of HIP events to the kernel launch itself (hipExtLaunchKernel), so the
 * events bracket exactly that kernel on the stream it runs on and add nothing between kernels;
 * the elapsed times are accumulated per kernel name. pkv_profile_read synchronises on the
 * recorded events. Off by default; enabling, resetting and reading are not thread-safe against
 * concurrent launches.
 *   pkv_profile_enable(mask): bit k selects the k-th name of pkv_profile_kernel_names()
 *   (0 turns timing off); also clears the totals.
 *   pkv_profile_read(name, &total_ms, &launches): totals for kernel `name` since the last
 *   enable/reset; returns PKV_ERR_INVALID_ARG for an unknown name.
 *   pkv_profile_kernel_names(): the kernel names, comma-separated, in bit order.
 */
pkv_status pkv_profile_enable(int kernel_mask);
pkv_status pkv_profile_reset(void);
pkv_status pkv_profile_read(const char* kernel_name, double* total_ms, long long* launches);
const char* pkv_profile_kernel_names(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
