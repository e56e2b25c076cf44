// Debug-build checks of the device arrays a call receives (the predicates are in checks.hpp).
// A build with PKV_DEBUG=1 runs these kernels first in every entry point, reads back what they
// found and launches the call's own kernels only when nothing was found, so arrays that break the
// documented preconditions are reported instead of being read out of bounds. Release builds
// compile these kernels too but never launch them.
#include "checks.hpp"
#include "launch.hpp"

namespace pkv {

// OR of the DebugBits found since the last reset, one word per GPU.
static __device__ unsigned debug_bits;

__device__ __forceinline__ void note(unsigned b) {
  if (b) atomicOr(&debug_bits, b);
}

__global__ __launch_bounds__(64) void debug_reset_kernel() {
  if (threadIdx.x == 0) debug_bits = 0u;
}

// One thread per sequence.
__global__ __launch_bounds__(256) void debug_tables_kernel(const int32_t* __restrict__ bt,
                                                           const int32_t* __restrict__ ctx,
                                                           int S, int MB, int B, int NB,
                                                           int max_ctx) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s < S) note(check_sequence(bt + static_cast<int64_t>(s) * MB, ctx[s], MB, B, NB, max_ctx));
}

__global__ __launch_bounds__(256) void debug_slots_kernel(const int32_t* __restrict__ slots,
                                                          int T, int NB, int B) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < T) note(check_slot(slots[i], NB, B));
}

__global__ __launch_bounds__(256) void debug_chunks_kernel(const int32_t* __restrict__ cu,
                                                           const int32_t* __restrict__ ctx, int S,
                                                           int total_q) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s < S) note(check_chunk(s, S, cu[s], cu[s + 1], ctx[s], total_q));
}

// One thread per group; the members' context lengths are read only inside [0, S).
__global__ __launch_bounds__(256) void debug_groups_kernel(const int32_t* __restrict__ gs,
                                                           const int32_t* __restrict__ gp,
                                                           const int32_t* __restrict__ ctx,
                                                           int NG, int S, int B, int max_prefix) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= NG) return;
  const int first = gs[i];
  const int last = gs[i + 1];
  int min_ctx = 0x7fffffff;
  const int lo = first < 0 ? 0 : first;
  const int hi = last > S ? S : last;
  for (int s = lo; s < hi; ++s) min_ctx = ctx[s] < min_ctx ? ctx[s] : min_ctx;
  note(check_group(i, NG, first, last, S, gp[i], B, max_prefix, min_ctx));
}

__global__ __launch_bounds__(256) void debug_pairs_kernel(const int32_t* __restrict__ pairs,
                                                          int n, int src_nb, int dst_nb) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) note(check_pair(pairs[2 * i], pairs[2 * i + 1], src_nb, dst_nb));
}

static unsigned groups_of(long long n) { return static_cast<unsigned>((n + 255) / 256); }

hipError_t debug_check(const DebugCheckArgs& a, hipStream_t st, unsigned* bits) {
  hipError_t e = launch_kernel(K_DEBUG_CHECK, debug_reset_kernel, dim3(1), dim3(64), st);
  if (e == hipSuccess && a.block_table && a.S > 0)
    e = launch_kernel(K_DEBUG_CHECK, debug_tables_kernel, dim3(groups_of(a.S)), dim3(256), st,
                      a.block_table, a.context_lens, a.S, a.MB, a.B, a.NB, a.max_ctx);
  if (e == hipSuccess && a.slots && a.T > 0)
    e = launch_kernel(K_DEBUG_CHECK, debug_slots_kernel, dim3(groups_of(a.T)), dim3(256), st,
                      a.slots, a.T, a.slot_NB, a.B);
  if (e == hipSuccess && a.cu_q_lens && a.S > 0)
    e = launch_kernel(K_DEBUG_CHECK, debug_chunks_kernel, dim3(groups_of(a.S)), dim3(256), st,
                      a.cu_q_lens, a.context_lens, a.S, a.total_q);
  if (e == hipSuccess && a.group_start && a.NG > 0)
    e = launch_kernel(K_DEBUG_CHECK, debug_groups_kernel, dim3(groups_of(a.NG)), dim3(256), st,
                      a.group_start, a.group_prefix_len, a.context_lens, a.NG, a.S, a.B,
                      a.max_prefix);
  if (e == hipSuccess && a.pairs && a.n_pairs > 0)
    e = launch_kernel(K_DEBUG_CHECK, debug_pairs_kernel, dim3(groups_of(a.n_pairs)), dim3(256),
                      st, a.pairs, a.n_pairs, a.src_nb, a.dst_nb);
  if (e != hipSuccess) return e;
  unsigned found = 0;
  e = hipMemcpyFromSymbolAsync(&found, HIP_SYMBOL(debug_bits), sizeof(found), 0,
                               hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  *bits = found;
  return hipSuccess;
}

}  // namespace pkv
