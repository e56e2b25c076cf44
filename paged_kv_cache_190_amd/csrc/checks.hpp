// Device-array preconditions of the C ABI (include/pkv.h, "Device-array preconditions"), as
// predicates that the debug build's check kernels run on the device and that a CPU harness runs
// on the host. Each returns a mask of DebugBits; 0 means the item is valid. They only read
// inside the arrays they are handed: a context length past the table's width is reported, and
// only the row's max_blocks_per_seq entries are looked at.
// ("Serving Engines", How vLLM works: the workers run against the block tables and slot mappings
// the scheduler hands them, so a bad table reaches the kernels unchecked in a release build.)
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define PKV_HD __host__ __device__
#else
#define PKV_HD
#endif

namespace pkv {

enum DebugBits : unsigned {
  kBadBlockId = 1u,     // a block id the call would read lies outside [0, num_blocks)
  kBadContextLen = 2u,  // context length < 0, > max_blocks_per_seq * B, or > max_context_len
  kBadSlot = 4u,        // a non-negative slot >= num_blocks * B
  kBadChunk = 8u,       // cu_q_lens not a partition of [0, total_q), or a chunk longer than n
  kBadGroup = 16u,      // group_start / group_prefix_len break their documented form
  kBadPair = 32u,       // a block-copy pair names a block outside its pool
};

// Sequence of a decode or prefill call: n = context_lens[s], row = block_table[s].
PKV_HD inline unsigned check_sequence(const int32_t* row, int n, int MB, int B, int NB,
                                      int max_ctx) {
  unsigned bits = 0;
  if (n < 0 || static_cast<long long>(n) > static_cast<long long>(MB) * B || n > max_ctx)
    bits |= kBadContextLen;
  const int need = n > 0 ? (n + B - 1) / B : 0;
  const int nblk = need < MB ? need : MB;
  for (int i = 0; i < nblk; ++i)
    if (row[i] < 0 || row[i] >= NB) {
      bits |= kBadBlockId;
      break;
    }
  return bits;
}

// One entry of a slot mapping (negative = skip the token).
PKV_HD inline unsigned check_slot(int32_t slot, int NB, int B) {
  return (slot >= 0 && static_cast<long long>(slot) >= static_cast<long long>(NB) * B)
             ? kBadSlot : 0u;
}

// Chunk of sequence s in a prefill: rows [lo, hi) of total_q, context n.
PKV_HD inline unsigned check_chunk(int s, int S, int lo, int hi, int n, int total_q) {
  unsigned bits = 0;
  if (lo < 0 || hi < lo || hi > total_q || (s == 0 && lo != 0) || (s == S - 1 && hi != total_q))
    bits |= kBadChunk;
  if (hi - lo > n) bits |= kBadChunk;
  return bits;
}

// Group i of a prefix-aware decode: members [first, last), shared prefix of pre tokens; n_first
// is the context length of the group's first member (every member's must be >= pre).
PKV_HD inline unsigned check_group(int i, int NG, int first, int last, int S, int pre, int B,
                                   int max_prefix, int min_member_ctx) {
  unsigned bits = 0;
  if (first < 0 || last < first || last > S || (i == 0 && first != 0) ||
      (i == NG - 1 && last != S))
    bits |= kBadGroup;
  if (pre < 0 || pre % B != 0 || pre > max_prefix || (last > first && pre > min_member_ctx))
    bits |= kBadGroup;
  return bits;
}

// One (source, destination) pair of a block copy.
PKV_HD inline unsigned check_pair(int32_t src, int32_t dst, int src_nb, int dst_nb) {
  return (src < 0 || src >= src_nb || dst < 0 || dst >= dst_nb) ? kBadPair : 0u;
}

}  // namespace pkv
