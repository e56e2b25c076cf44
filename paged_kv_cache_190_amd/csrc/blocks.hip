// kv_cache_copy_blocks: bit copies of whole physical blocks, between two pools or inside one.
//
// ("Serving Engines", How vLLM works: a copy-on-write fork copies exactly the block being
// written; swap preemption moves a sequence's blocks out to host memory and back.)
// A block of either pool is one contiguous run of Hkv*B*D elements (the KV-head tiles of that
// block), so a pair copies two runs: the K run and the V run. The pools may be device memory or
// pinned host memory; the kernel reads and writes them through their pointers.
// Grid: (chunk groups, pairs); each thread copies 16-byte words.
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

__global__ __launch_bounds__(256) void copy_blocks_kernel(const u32x4* __restrict__ src_k,
                                                          const u32x4* __restrict__ src_v,
                                                          u32x4* __restrict__ dst_k,
                                                          u32x4* __restrict__ dst_v,
                                                          const int32_t* __restrict__ pairs,
                                                          int64_t words_per_block) {
  const int p = blockIdx.y;
  const int64_t s = pairs[2 * p];
  const int64_t d = pairs[2 * p + 1];
  const u32x4* sk = src_k + s * words_per_block;
  const u32x4* sv = src_v + s * words_per_block;
  u32x4* dk = dst_k + d * words_per_block;
  u32x4* dv = dst_v + d * words_per_block;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       i < words_per_block; i += stride) {
    // streamed: nothing copied is read again by this kernel (non-temporal loads and stores
    // took the copy of half the 8B-shaped batch's blocks from 116 to 100 us)
    const u32x4 a = __builtin_nontemporal_load(sk + i);
    const u32x4 b = __builtin_nontemporal_load(sv + i);
    __builtin_nontemporal_store(a, dk + i);
    __builtin_nontemporal_store(b, dv + i);
  }
}

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream) {
  if (a.n_pairs == 0) return hipSuccess;
  const int64_t words = static_cast<int64_t>(a.Hkv) * a.B * a.D * a.elem_bytes / 16;
  const int64_t groups = (words + 4 * 256 - 1) / (4 * 256);  // about four words per thread
  dim3 grid(static_cast<unsigned>(groups < 64 ? groups : 64), a.n_pairs);
  return launch_kernel(K_COPY_BLOCKS, copy_blocks_kernel, grid, dim3(256), stream,
                      static_cast<const u32x4*>(a.src_k), static_cast<const u32x4*>(a.src_v),
                      static_cast<u32x4*>(a.dst_k), static_cast<u32x4*>(a.dst_v), a.pairs,
                      words);
}

}  // namespace pkv
