// Internal launch interface between the C ABI (api.cpp) and the kernel files.
// Arguments arrive validated; each launcher only computes its grid and launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Kernel ids for the timing registry (api.cpp owns the registry).
enum KernelId {
  K_KV_WRITE = 0,
  K_DECODE_PARTITION = 1,
  K_DECODE_REDUCE = 2,
  K_PREFILL = 3,
  K_COUNT = 4
};
const char* kernel_name(int id);

// Called by launchers around every kernel launch (no-ops unless timing is enabled).
void timing_begin(int id, hipStream_t stream);
void timing_end(int id, hipStream_t stream);

struct KvWriteArgs {
  const void* k_new;
  const void* v_new;
  void* k_pool;
  void* v_pool;
  const int32_t* slot_mapping;
  int T, Hkv, D, B, NB, elem_bytes;
};
hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream);

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
  int P;         // resolved partition size (tokens)
  int NP;        // ceil(max_ctx / P); 1 => no partials
  float* part_o; // [S][Hq][NP][D]
  float* part_m; // [S][Hq][NP]
  float* part_l; // [S][Hq][NP]
  int bf16_in;
  int bf16_out;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

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
