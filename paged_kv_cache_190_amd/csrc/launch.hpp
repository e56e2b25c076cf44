// Internal launch interface between the C ABI (api.cpp) and the kernel files.
// Arguments arrive validated; each launcher only computes its grid and launches.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>

namespace pkv {

// Kernel ids for the timing registry (api.cpp owns the registry).
enum KernelId {
  K_KV_WRITE = 0,
  K_DECODE_PARTITION = 1,
  K_DECODE_REDUCE = 2,
  K_PREFILL = 3,
  K_COPY_BLOCKS = 4,
  K_READ_PROBE = 5,
  K_DEBUG_CHECK = 6,
  K_COUNT = 7
};
const char* kernel_name(int id);

// Timing: when kernel `id` is being timed, a pair of events (registered with the timing
// registry) that the launch records as part of the kernel dispatch; otherwise nulls.
struct TimingEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
TimingEvents timing_events(int id);

// Every kernel of the library is launched through here: hipExtLaunchKernel takes the timing
// events with the dispatch itself, so timing adds no packets between kernels. The status is the
// one this launch returned (a launch the runtime refuses, e.g. no code object for the device or
// an invalid configuration); on failure the runtime's sticky copy of the error is cleared, since
// the caller reports it.
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(int id, void (*kernel)(KArgs...), dim3 grid, dim3 block,
                         hipStream_t stream, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
  const TimingEvents ev = timing_events(id);
  std::tuple<KArgs...> vals{static_cast<KArgs>(args)...};
  void* argv[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
  std::apply(
      [&argv](auto&... v) {
        int i = 0;
        ((argv[i++] = static_cast<void*>(&v)), ...);
      },
      vals);
  const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block,
                                          argv, 0, stream, ev.start, ev.stop, 0);
  if (e != hipSuccess) (void)hipGetLastError();
  return e;
}

struct KvWriteArgs {
  const void* k_new;
  const void* v_new;
  void* k_pool;
  void* v_pool;
  const int32_t* slot_mapping;
  int T, Hkv, D, B, NB, elem_bytes;
};
hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream);
// E4M3 pools: inputs bf16 (in_bf16) or fp32, stored as the codes of x / scale.
hipError_t launch_kv_write_fp8(const KvWriteArgs& a, int in_bf16, float k_scale, float v_scale,
                               hipStream_t stream);

struct CopyBlocksArgs {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  const int32_t* pairs;
  int n_pairs, Hkv, D, B, elem_bytes;
};
hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t stream);

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* context_lens;
  int S, Hq, Hkv, D, B, MB, NB;
  float scale;
  int max_ctx;   // resolved host bound
  // Fixed partitions (balanced == 0): P tokens each, NP = ceil(max_ctx / P); NP == 1 stores no
  // partials. Balanced split (balanced == 1): `waves` waves share the batch's 32-token tiles
  // equally, each taking at least min_tiles; a row has at most KMAX partials.
  int balanced;
  int P;
  int NP;
  int waves;
  int min_tiles;
  int KMAX;
  float* part_o;       // [S][Hq][NP or KMAX][D]
  float* part_m;       // [S][Hq][NP or KMAX]
  float* part_l;       // [S][Hq][NP or KMAX]
  int32_t* seg_count;  // [S][Hkv][ceil(G/16)] (balanced)
  int bf16_in;
  int bf16_out;
  // E4M3 pools (always balanced; q is bf16): K value = code * k_scale, V value = code * v_scale.
  int fp8_kv;
  float k_scale;
  float v_scale;
  // Shared prefixes (num_groups > 0; balanced): group i is sequences group_start[i] ..
  // group_start[i+1]-1 sharing their first group_prefix_len[i] tokens. prefix_units units
  // (group, KV head, chunk, block of query columns; prefix_col_blocks blocks per chunk), each a
  // workgroup of kPrefixWgWaves waves, run beside the `waves` suffix waves. KMAX is then the row
  // stride of the partials (prefix chunks first).
  int num_groups;
  const int32_t* group_start;
  const int32_t* group_prefix_len;
  int prefix_units;
  int prefix_col_blocks;
  int prefix_chunks;
  // Fused write + decode (bf16, balanced): token s's newest K/V come from k_new / v_new when
  // slot_mapping[s] >= 0, and the same launch stores them into the pool.
  int step;
  const void* k_new;
  const void* v_new;
  const int32_t* slot_mapping;
};
constexpr int kPrefixChunkTokens = 256;  // tokens of the shared prefix per prefix chunk
// Prefix-aware decode: waves per workgroup, and the (member, query head) columns one prefix
// workgroup computes (32 per wave).
constexpr int kPrefixWgWaves = 8;
constexpr int kPrefixWgColumns = 32 * kPrefixWgWaves;
// Waves per workgroup of the balanced split's kernels; a launch of W waves runs
// kBalancedWavesPerGroup * ceil(W / kBalancedWavesPerGroup) of them.
constexpr int kBalancedWavesPerGroup = 4;

// Scratch of pkv_paged_attention_decode_noalloc: the balanced split's partials and segment
// counts in a file-scope device array of this many bytes (one per GPU, held until the process
// ends). noalloc_scratch returns the current device's copy: its address is looked up once per
// device and kept; nothing is allocated.
constexpr size_t kNoAllocScratchBytes = static_cast<size_t>(128) << 20;
hipError_t noalloc_scratch(void** ptr, size_t* bytes);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Read probe (measurement only): the balanced decode's waves and tiles, loads without the
// attention arithmetic; each of `waves` waves leaves 64 words in sink.
struct ReadProbeArgs {
  uint32_t* sink;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* context_lens;
  int S, Hq, Hkv, D, B, MB;
  int waves;
  int min_tiles;
};
hipError_t launch_read_probe(const ReadProbeArgs& a, hipStream_t stream);

// Debug builds (PKV_DEBUG=1): which device arrays a call hands over, for the check kernels of
// debug.hip. Null pointers and zero counts skip a check. debug_check launches the checks on the
// stream, waits for them and returns the OR of the DebugBits (checks.hpp) they found in *bits.
struct DebugCheckArgs {
  const int32_t* block_table = nullptr;
  const int32_t* context_lens = nullptr;
  int S = 0, MB = 0, B = 0, NB = 0, max_ctx = 0;
  const int32_t* slots = nullptr;
  int T = 0, slot_NB = 0;
  const int32_t* cu_q_lens = nullptr;
  int total_q = 0;
  const int32_t* group_start = nullptr;
  const int32_t* group_prefix_len = nullptr;
  int NG = 0, max_prefix = 0;
  const int32_t* pairs = nullptr;
  int n_pairs = 0, src_nb = 0, dst_nb = 0;
};
hipError_t debug_check(const DebugCheckArgs& a, hipStream_t stream, unsigned* bits);

struct PrefillArgs {
  void* out;
  const void* q;
  const int32_t* cu_q_lens;
  const int32_t* context_lens;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  int S, total_q, Hq, Hkv, D, B, MB, NB;
  float scale;
  int max_q_len, max_ctx;
  int bf16_in;
  int bf16_out;
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace pkv
