// Host-side block manager: physical blocks with reference counts, per-sequence block tables,
// copy-on-write on append. ("Serving Engines", How vLLM works: a sequence claims a new block only
// when its current one fills; a count per block tracks sharing; a write forks only the block
// being written. "Inference Engines", PagedAttention: blocks are freed when a sequence ends.)
// Single-writer, as the pages describe the block manager; not thread-safe.
#include <functional>
#include <queue>
#include <unordered_map>
#include <vector>

#include "../../include/pkv.h"
#include "errors.hpp"

using pkv::fail;

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t len = 0;
  };
  int num_blocks = 0;
  int block_size = 0;
  std::vector<int> refcount;
  // Free ids in a min-heap: the lowest free id is always the next one handed out.
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_list;
  std::unordered_map<int64_t, Seq> seqs;

  int32_t take() {
    const int32_t b = free_list.top();
    free_list.pop();
    refcount[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--refcount[b] == 0) free_list.push(b);
  }
};

extern "C" {

pkv_status pkv_bm_create(int num_blocks, int block_size, pkv_block_manager** out) {
  if (!out || num_blocks <= 0 || block_size <= 0)
    return fail(PKV_ERR_INVALID_ARG, "bm_create: num_blocks %d, block_size %d", num_blocks,
                block_size);
  auto* bm = new pkv_block_manager;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->refcount.assign(num_blocks, 0);
  for (int b = 0; b < num_blocks; ++b) bm->free_list.push(b);
  *out = bm;
  return PKV_OK;
}

void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

int pkv_bm_num_free(const pkv_block_manager* bm) {
  return bm ? static_cast<int>(bm->free_list.size()) : -1;
}

pkv_status pkv_bm_add(pkv_block_manager* bm, int64_t seq) {
  if (!bm) return fail(PKV_ERR_INVALID_ARG, "bm_add: null manager");
  if (bm->seqs.count(seq)) return fail(PKV_ERR_INVALID_ARG, "bm_add: sequence %lld exists",
                                       static_cast<long long>(seq));
  bm->seqs[seq] = pkv_block_manager::Seq{};
  return PKV_OK;
}

pkv_status pkv_bm_fork(pkv_block_manager* bm, int64_t parent, int64_t child) {
  if (!bm || !bm->seqs.count(parent) || bm->seqs.count(child))
    return fail(PKV_ERR_INVALID_ARG, "bm_fork: parent %lld must exist and child %lld must not",
                static_cast<long long>(parent), static_cast<long long>(child));
  const pkv_block_manager::Seq copy = bm->seqs.at(parent);
  for (int32_t b : copy.blocks) ++bm->refcount[b];
  bm->seqs[child] = copy;
  return PKV_OK;
}

pkv_status pkv_bm_append(pkv_block_manager* bm, int64_t seq, int n_tokens, int32_t* slots,
                         int32_t* copies, int max_copies, int* n_copies) {
  if (!bm || !n_copies || n_tokens < 0 || !bm->seqs.count(seq))
    return fail(PKV_ERR_INVALID_ARG, "bm_append: bad arguments for sequence %lld",
                static_cast<long long>(seq));
  if (n_tokens > 0 && !slots) return fail(PKV_ERR_INVALID_ARG, "bm_append: slots is null");
  auto& q = bm->seqs.at(seq);
  const int64_t B = bm->block_size;
  const int64_t len = q.len;
  const bool cow = len % B != 0 && bm->refcount[q.blocks.back()] > 1;
  const int64_t fresh = (len + n_tokens + B - 1) / B - (len + B - 1) / B;
  const int64_t need = fresh + (cow ? 1 : 0);
  if (n_tokens > 0 && cow && (!copies || max_copies < 1))
    return fail(PKV_ERR_INVALID_ARG, "bm_append: a block copy is due and copies has no room");
  if (need > static_cast<int64_t>(bm->free_list.size()))
    return fail(PKV_ERR_OUT_OF_BLOCKS, "bm_append: %lld blocks needed, %zu free",
                static_cast<long long>(need), bm->free_list.size());
  *n_copies = 0;
  if (n_tokens == 0) return PKV_OK;
  if (cow) {  // the last block is shared and partly filled: write into a private copy
    const int32_t old = q.blocks.back();
    const int32_t fresh_block = bm->take();
    bm->drop(old);
    q.blocks.back() = fresh_block;
    copies[0] = old;
    copies[1] = fresh_block;
    *n_copies = 1;
  }
  for (int i = 0; i < n_tokens; ++i) {
    const int64_t pos = len + i;
    if (pos % B == 0) q.blocks.push_back(bm->take());
    slots[i] = static_cast<int32_t>(q.blocks[pos / B] * B + pos % B);
  }
  q.len = len + n_tokens;
  return PKV_OK;
}

pkv_status pkv_bm_free(pkv_block_manager* bm, int64_t seq) {
  if (!bm || !bm->seqs.count(seq))
    return fail(PKV_ERR_INVALID_ARG, "bm_free: unknown sequence %lld", static_cast<long long>(seq));
  for (int32_t b : bm->seqs.at(seq).blocks) bm->drop(b);
  bm->seqs.erase(seq);
  return PKV_OK;
}

pkv_status pkv_bm_context_len(const pkv_block_manager* bm, int64_t seq, int* len) {
  if (!bm || !len || !bm->seqs.count(seq))
    return fail(PKV_ERR_INVALID_ARG, "bm_context_len: unknown sequence %lld",
                static_cast<long long>(seq));
  *len = static_cast<int>(bm->seqs.at(seq).len);
  return PKV_OK;
}

pkv_status pkv_bm_block_table(const pkv_block_manager* bm, int64_t seq, int32_t* table,
                              int capacity, int* n_blocks) {
  if (!bm || !n_blocks || capacity < 0 || !bm->seqs.count(seq))
    return fail(PKV_ERR_INVALID_ARG, "bm_block_table: unknown sequence %lld",
                static_cast<long long>(seq));
  const auto& blocks = bm->seqs.at(seq).blocks;
  *n_blocks = static_cast<int>(blocks.size());
  if (capacity > 0 && !table) return fail(PKV_ERR_INVALID_ARG, "bm_block_table: table is null");
  for (int i = 0; i < capacity && i < static_cast<int>(blocks.size()); ++i) table[i] = blocks[i];
  return PKV_OK;
}

pkv_status pkv_bm_refcount(const pkv_block_manager* bm, int block, int* count) {
  if (!bm || !count || block < 0 || block >= bm->num_blocks)
    return fail(PKV_ERR_INVALID_ARG, "bm_refcount: block %d out of range", block);
  *count = bm->refcount[block];
  return PKV_OK;
}

}  // extern "C"
