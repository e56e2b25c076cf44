// C ABI of libpkv: argument validation, partition sizing, kernel timing, error reporting.
// Declarations and the meaning of every argument are in include/pkv.h.
#include "../../include/pkv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "checks.hpp"
#include "errors.hpp"
#include "launch.hpp"

// PKV_DEBUG=1 builds check the device arrays of every call on the device before launching it.
#ifndef PKV_DEBUG
#define PKV_DEBUG 0
#endif

namespace {
thread_local std::string g_last_error;
thread_local unsigned g_debug_found = 0;  // DebugBits of this thread's last checked call
constexpr bool kDebugBuild = PKV_DEBUG != 0;
}  // namespace

pkv_status pkv::fail(pkv_status status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

namespace {

using pkv::fail;

pkv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Debug builds: the call's device arrays are checked on the device first (debug.hip); a call
// whose arrays break the documented preconditions launches nothing and returns
// PKV_ERR_DEVICE_ARG. Release builds: nothing.
pkv_status debug_gate(const pkv::DebugCheckArgs& d, void* stream, const char* what) {
  if constexpr (!kDebugBuild) {
    (void)d, (void)stream, (void)what;
    return PKV_OK;
  } else {
    unsigned bits = 0;
    const hipError_t e = pkv::debug_check(d, static_cast<hipStream_t>(stream), &bits);
    if (pkv_status st = hip_status(e, what)) return st;
    g_debug_found = bits;
    if (!bits) return PKV_OK;
    std::string names;
    const char* labels[] = {"block id", "context length", "slot", "chunk", "group", "pair"};
    for (int i = 0; i < 6; ++i)
      if (bits & (1u << i)) names += std::string(names.empty() ? "" : ", ") + labels[i];
    return fail(PKV_ERR_DEVICE_ARG,
                "%s: device arrays break the documented preconditions (found: %s); nothing "
                "was launched", what, names.c_str());
  }
}

pkv::DebugCheckArgs tables_check(const int32_t* bt, const int32_t* ctx, int S, int MB, int B,
                                 int NB, int max_ctx) {
  pkv::DebugCheckArgs d;
  d.block_table = bt;
  d.context_lens = ctx;
  d.S = S;
  d.MB = MB;
  d.B = B;
  d.NB = NB;
  d.max_ctx = max_ctx;
  return d;
}

bool supported_dtype(int d) { return d == PKV_F32 || d == PKV_BF16; }
int elem_bytes(int d) { return d == PKV_FP8_E4M3 ? 1 : (d == PKV_BF16 ? 2 : 4); }
bool valid_pool_scale(float s) { return std::isfinite(s) && s > 0.0f; }

constexpr int kMaxGridYZ = 65535;

// ------------------------------------------------------------------ kernel timing registry
struct TimingRecord {
  int id;
  hipEvent_t start;
  hipEvent_t stop;
};

std::mutex g_timing_mu;
unsigned g_timing_mask = 0;  // bit k: kernel id k is timed
std::vector<TimingRecord> g_pending;
std::vector<hipEvent_t> g_event_pool;
double g_total_ms[pkv::K_COUNT];
long long g_launches[pkv::K_COUNT];

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void drain_locked() {
  for (const TimingRecord& r : g_pending) {
    float ms = 0.f;
    if (r.stop && hipEventSynchronize(r.stop) == hipSuccess &&
        hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
      g_total_ms[r.id] += ms;
      g_launches[r.id] += 1;
    }
    if (r.start) g_event_pool.push_back(r.start);
    if (r.stop) g_event_pool.push_back(r.stop);
  }
  g_pending.clear();
}

}  // namespace

namespace pkv {

const char* kernel_name(int id) {
  switch (id) {
    case K_KV_WRITE: return "kv_cache_write";
    case K_DECODE_PARTITION: return "decode_partition";
    case K_DECODE_REDUCE: return "decode_reduce";
    case K_PREFILL: return "prefill_chunk";
    case K_COPY_BLOCKS: return "copy_blocks";
    case K_READ_PROBE: return "read_probe";
    case K_DEBUG_CHECK: return "debug_check";
    default: return "?";
  }
}

TimingEvents timing_events(int id) {
  TimingEvents ev;
  if (!(g_timing_mask & (1u << id))) return ev;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  ev.start = take_event();
  ev.stop = take_event();
  if (ev.start && ev.stop) {
    g_pending.push_back({id, ev.start, ev.stop});
  } else {
    if (ev.start) g_event_pool.push_back(ev.start);
    if (ev.stop) g_event_pool.push_back(ev.stop);
    ev = TimingEvents{};
  }
  return ev;
}

}  // namespace pkv

namespace {

// Fixed-partition default (fp32 inputs, or callers that ask for fixed partitions): 512 tokens,
// halved (down to 64) while the launch would have fewer than 2048 (sequence, KV head,
// partition) work units, i.e. about eight per compute unit.
int resolve_partition(int partition_size, int num_seqs, int num_kv_heads, int max_ctx) {
  if (partition_size < 0 || partition_size % 16 != 0) return -1;
  if (partition_size > 0) return partition_size;
  int p = 512;
  while (p > 64) {
    const long long parts = (max_ctx + p - 1) / p;
    if (static_cast<long long>(num_seqs) * num_kv_heads * parts >= 2048) break;
    p /= 2;
  }
  return p;
}

int num_partitions(int max_ctx, int p) { return max_ctx <= 0 ? 1 : (max_ctx + p - 1) / p; }

size_t fixed_workspace_bytes(int S, int Hq, int D, int NP) {
  if (NP <= 1) return 0;
  const size_t rows = static_cast<size_t>(S) * Hq * NP;
  return rows * D * sizeof(float) + 2 * rows * sizeof(float);
}

// Balanced split (bf16 inputs, partition_size == 0).
constexpr int kMinTilesPerWave = 8;     // 256 tokens
// The prefix-aware decode's suffix waves: its suffixes are short and its prefix chunks carry the
// rest of the work, so more, shorter suffix pieces pay there. On the shared-prefix batch: over
// E4M3 pools 4 against 8 tiles gave 20.6-20.8 against 21.0-21.2 us; over bf16 pools (suffix
// waves filling the CUs beside the prefix workgroups) 3 gave 24.0-24.6 us, 4 24.7-25.1 and 2
// 24.4-24.8.
int prefix_min_tiles(int kv_dtype) { return kv_dtype == PKV_FP8_E4M3 ? 4 : 3; }
constexpr int kDefaultDecodeWaves = 1024;
// E4M3 pools: the same count measured best (768 - 2048 tried; their tile loop keeps three
// tiles in flight instead).
constexpr int kDefaultDecodeWavesFp8 = 1024;

struct BalancedPlan {
  int waves;
  int kmax;
  size_t o_off, m_off, l_off, cnt_off, bytes;
};

// Waves of the balanced split: the caller's count, or the default for the pool type.
constexpr int kMaxDecodeWaves = 1 << 20;

// extra_slots: partial slots per row ahead of the balanced split's (the prefix chunks).
BalancedPlan balanced_plan(int S, int Hq, int Hkv, int D, int max_ctx, int waves_request,
                           int extra_slots = 0, int min_tiles = kMinTilesPerWave) {
  BalancedPlan pl{};
  const int G = Hq / Hkv;
  const long long segs = static_cast<long long>(Hkv) * ((G + 15) / 16);
  const long long seg_tiles = (std::max(max_ctx, 1) + 31) / 32;
  const long long t_upper = static_cast<long long>(S) * segs * seg_tiles;
  pl.waves = static_cast<int>(
      std::max(1LL, std::min<long long>(waves_request, t_upper / min_tiles)));
  pl.kmax = static_cast<int>((seg_tiles + min_tiles - 1) / min_tiles + 1) +
            extra_slots;
  const size_t rows = static_cast<size_t>(S) * Hq * pl.kmax;
  auto align = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  pl.o_off = 0;
  pl.m_off = align(rows * D * sizeof(float));
  pl.l_off = pl.m_off + align(rows * sizeof(float));
  pl.cnt_off = pl.l_off + align(rows * sizeof(float));
  pl.bytes = pl.cnt_off + align(static_cast<size_t>(S) * segs * sizeof(int32_t));
  return pl;
}

pkv_status check_common(int Hq, int Hkv, int D, int B, int dtype, int out_dtype) {
  if (Hq <= 0 || Hkv <= 0) return fail(PKV_ERR_INVALID_ARG, "head counts must be positive");
  if (Hq % Hkv != 0)
    return fail(PKV_ERR_UNSUPPORTED, "num_q_heads %d is not a multiple of num_kv_heads %d", Hq,
                Hkv);
  if (D != 64 && D != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", D);
  if (B != 16 && B != 32) return fail(PKV_ERR_UNSUPPORTED, "block_size %d not in {16, 32}", B);
  if (!supported_dtype(dtype) || !supported_dtype(out_dtype))
    return fail(PKV_ERR_UNSUPPORTED, "dtype %d / out_dtype %d not supported", dtype, out_dtype);
  if (Hq > kMaxGridYZ) return fail(PKV_ERR_UNSUPPORTED, "num_q_heads %d too large", Hq);
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_abi_version(void) { return PKV_ABI_VERSION; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_HIP: return "HIP runtime error";
    case PKV_ERR_OUT_OF_BLOCKS: return "not enough free blocks";
    case PKV_ERR_DEVICE_ARG: return "device array breaks a precondition (debug build)";
    default: return "unknown status";
  }
}

const char* pkv_last_error(void) { return g_last_error.c_str(); }

int pkv_debug_build(void) { return kDebugBuild ? 1 : 0; }

unsigned pkv_debug_found(void) { return g_debug_found; }

pkv_status pkv_kv_cache_write(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                              const int32_t* slot_mapping, int T, int num_kv_heads, int head_dim,
                              int block_size, int num_blocks, int dtype, void* stream) {
  if (T < 0) return fail(PKV_ERR_INVALID_ARG, "T = %d is negative", T);
  if (T == 0) return PKV_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !slot_mapping)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (num_kv_heads <= 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARG, "num_kv_heads and num_blocks must be positive");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", head_dim);
  if (block_size != 16 && block_size != 32)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d not in {16, 32}", block_size);
  if (!supported_dtype(dtype)) return fail(PKV_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
  if (num_kv_heads > kMaxGridYZ)
    return fail(PKV_ERR_UNSUPPORTED, "num_kv_heads %d too large", num_kv_heads);
  if (static_cast<long long>(num_blocks) * block_size > 0x7fffffffLL)
    return fail(PKV_ERR_UNSUPPORTED, "pool of %d blocks exceeds int32 slot numbers", num_blocks);
  pkv::KvWriteArgs a{k_new, v_new, k_pool, v_pool, slot_mapping, T, num_kv_heads, head_dim,
                     block_size, num_blocks, elem_bytes(dtype)};
  pkv::DebugCheckArgs d;
  d.slots = slot_mapping;
  d.T = T;
  d.slot_NB = num_blocks;
  d.B = block_size;
  if (pkv_status st = debug_gate(d, stream, "kv_cache_write")) return st;
  return hip_status(pkv::launch_kv_write(a, static_cast<hipStream_t>(stream)), "kv_cache_write");
}

pkv_status pkv_kv_cache_write_fp8(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                  const int32_t* slot_mapping, int T, int num_kv_heads,
                                  int head_dim, int block_size, int num_blocks, int in_dtype,
                                  float k_scale, float v_scale, void* stream) {
  if (T < 0) return fail(PKV_ERR_INVALID_ARG, "T = %d is negative", T);
  if (T == 0) return PKV_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !slot_mapping)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (num_kv_heads <= 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARG, "num_kv_heads and num_blocks must be positive");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", head_dim);
  if (block_size != 16 && block_size != 32)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d not in {16, 32}", block_size);
  if (!supported_dtype(in_dtype))
    return fail(PKV_ERR_UNSUPPORTED, "in_dtype %d not supported", in_dtype);
  if (!valid_pool_scale(k_scale) || !valid_pool_scale(v_scale))
    return fail(PKV_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
  if (num_kv_heads > kMaxGridYZ)
    return fail(PKV_ERR_UNSUPPORTED, "num_kv_heads %d too large", num_kv_heads);
  if (static_cast<long long>(num_blocks) * block_size > 0x7fffffffLL)
    return fail(PKV_ERR_UNSUPPORTED, "pool of %d blocks exceeds int32 slot numbers", num_blocks);
  pkv::KvWriteArgs a{k_new, v_new, k_pool, v_pool, slot_mapping, T, num_kv_heads, head_dim,
                     block_size, num_blocks, elem_bytes(in_dtype)};
  pkv::DebugCheckArgs d;
  d.slots = slot_mapping;
  d.T = T;
  d.slot_NB = num_blocks;
  d.B = block_size;
  if (pkv_status st = debug_gate(d, stream, "kv_cache_write_fp8")) return st;
  return hip_status(pkv::launch_kv_write_fp8(a, in_dtype == PKV_BF16, k_scale, v_scale,
                                             static_cast<hipStream_t>(stream)),
                    "kv_cache_write_fp8");
}

namespace {
// A pool handed to the copy kernel may be device memory or pinned host memory; anything else
// (pageable host memory, a stale pointer) would fault in the kernel, so it is refused here.
// Pinned memory is accepted only where the device sees it at the same address.
pkv_status check_kernel_visible(const void* p, const char* name) {
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(PKV_ERR_INVALID_ARG, "%s is not device or pinned host memory", name);
  }
  if (at.type == hipMemoryTypeHost && at.devicePointer != p)
    return fail(PKV_ERR_INVALID_ARG, "%s: pinned host memory not mapped at the same address",
                name);
  if (at.type == hipMemoryTypeUnregistered)
    return fail(PKV_ERR_INVALID_ARG, "%s is unregistered host memory", name);
  return PKV_OK;
}
}  // namespace

pkv_status pkv_kv_cache_copy_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                                    const int32_t* block_pairs, int n_pairs, int num_kv_heads,
                                    int head_dim, int block_size, int src_num_blocks,
                                    int dst_num_blocks, int dtype, void* stream) {
  if (n_pairs < 0) return fail(PKV_ERR_INVALID_ARG, "n_pairs = %d is negative", n_pairs);
  if (n_pairs == 0) return PKV_OK;
  if (!src_k || !src_v || !dst_k || !dst_v || !block_pairs)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  if (num_kv_heads <= 0 || src_num_blocks <= 0 || dst_num_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARG, "num_kv_heads and pool sizes must be positive");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", head_dim);
  if (block_size != 16 && block_size != 32)
    return fail(PKV_ERR_UNSUPPORTED, "block_size %d not in {16, 32}", block_size);
  if (!supported_dtype(dtype) && dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
  if (n_pairs > kMaxGridYZ) return fail(PKV_ERR_UNSUPPORTED, "n_pairs %d too large", n_pairs);
  const void* ptrs[5] = {src_k, src_v, dst_k, dst_v, block_pairs};
  const char* names[5] = {"src_k", "src_v", "dst_k", "dst_v", "block_pairs"};
  for (int i = 0; i < 5; ++i)
    if (pkv_status st = check_kernel_visible(ptrs[i], names[i])) return st;
  pkv::CopyBlocksArgs a{src_k, src_v, dst_k, dst_v, block_pairs, n_pairs, num_kv_heads,
                        head_dim, block_size, elem_bytes(dtype)};
  pkv::DebugCheckArgs d;
  d.pairs = block_pairs;
  d.n_pairs = n_pairs;
  d.src_nb = src_num_blocks;
  d.dst_nb = dst_num_blocks;
  if (pkv_status st = debug_gate(d, stream, "kv_cache_copy_blocks")) return st;
  return hip_status(pkv::launch_copy_blocks(a, static_cast<hipStream_t>(stream)),
                    "kv_cache_copy_blocks");
}

int pkv_decode_partition_size(int partition_size, int num_seqs, int num_kv_heads,
                              int max_context_len, int dtype) {
  if (partition_size == 0 && dtype == PKV_BF16) return 0;  // balanced split
  return resolve_partition(partition_size, num_seqs, num_kv_heads, max_context_len);
}

size_t pkv_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int max_context_len, int partition_size, int dtype) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0)
    return 0;
  if (dtype == PKV_FP8_E4M3)
    return balanced_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                         kDefaultDecodeWavesFp8).bytes;
  if (partition_size == 0 && dtype == PKV_BF16)
    return balanced_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                         kDefaultDecodeWaves).bytes;
  const int p = resolve_partition(partition_size, num_seqs, num_kv_heads, max_context_len);
  if (p <= 0) return 0;
  return fixed_workspace_bytes(num_seqs, num_q_heads, head_dim,
                               num_partitions(max_context_len, p));
}

}  // extern "C"

namespace {

// Balanced split set-up: the plan for a's sizes, and the partial buffers carved out of the
// caller's workspace.
pkv_status setup_balanced(pkv::DecodeArgs& a, void* workspace, size_t workspace_bytes,
                          int default_waves, int num_waves, int extra_slots = 0,
                          int min_tiles = kMinTilesPerWave) {
  if (num_waves < 0 || num_waves > kMaxDecodeWaves)
    return fail(PKV_ERR_INVALID_ARG, "num_waves %d outside [0, %d]", num_waves, kMaxDecodeWaves);
  const BalancedPlan pl = balanced_plan(a.S, a.Hq, a.Hkv, a.D, a.max_ctx,
                                        num_waves > 0 ? num_waves : default_waves, extra_slots,
                                        min_tiles);
  if (!workspace || workspace_bytes < pl.bytes)
    return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", pl.bytes,
                workspace ? workspace_bytes : static_cast<size_t>(0));
  char* base = static_cast<char*>(workspace);
  a.balanced = 1;
  a.waves = pl.waves;
  a.min_tiles = min_tiles;
  a.KMAX = pl.kmax;
  a.P = 32;
  a.NP = 1;
  a.part_o = reinterpret_cast<float*>(base + pl.o_off);
  a.part_m = reinterpret_cast<float*>(base + pl.m_off);
  a.part_l = reinterpret_cast<float*>(base + pl.l_off);
  a.seg_count = reinterpret_cast<int32_t*>(base + pl.cnt_off);
  return PKV_OK;
}

// Compute units of the current device, read once per device.
hipError_t device_cu_count(int* cus) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int per_device[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (per_device[dev] <= 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n <= 0) return hipErrorInvalidDevice;
    per_device[dev] = n;
  }
  *cus = per_device[dev];
  return hipSuccess;
}

// Partial slots per row taken by the prefix chunks.
int prefix_chunks(int max_prefix_len) {
  return (max_prefix_len + pkv::kPrefixChunkTokens - 1) / pkv::kPrefixChunkTokens;
}

// Checks shared by the decode entry points; fills the size fields of a.
pkv_status check_decode(pkv::DecodeArgs& a, void* out, const void* q, const void* k_pool,
                 const void* v_pool, const int32_t* block_table, const int32_t* context_lens,
                 int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                 int max_blocks_per_seq, int num_blocks, float scale, int max_context_len,
                 int dtype, int out_dtype) {
  if (!out || !q || !k_pool || !v_pool || !block_table || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  pkv_status st = check_common(num_q_heads, num_kv_heads, head_dim, block_size, dtype, out_dtype);
  if (st != PKV_OK) return st;
  if (max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq and num_blocks must be positive");
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  const long long cap = static_cast<long long>(max_blocks_per_seq) * block_size;
  if (cap > 0x7fffffffLL) return fail(PKV_ERR_UNSUPPORTED, "max_blocks_per_seq too large");
  if (max_context_len < 0 || max_context_len > cap)
    return fail(PKV_ERR_INVALID_ARG, "max_context_len %d outside [0, %lld]", max_context_len,
                cap);
  if (num_seqs > kMaxGridYZ) return fail(PKV_ERR_UNSUPPORTED, "num_seqs %d too large", num_seqs);
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.S = num_seqs;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.D = head_dim;
  a.B = block_size;
  a.MB = max_blocks_per_seq;
  a.NB = num_blocks;
  a.scale = scale;
  a.max_ctx = max_context_len > 0 ? max_context_len : static_cast<int>(cap);
  return PKV_OK;
}

}  // namespace

extern "C" {

size_t pkv_decode_shared_prefix_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                               int head_dim, int max_context_len,
                                               int max_prefix_len, int kv_dtype) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || max_prefix_len < 0)
    return 0;
  return balanced_plan(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                       kv_dtype == PKV_FP8_E4M3 ? kDefaultDecodeWavesFp8 : kDefaultDecodeWaves,
                       prefix_chunks(max_prefix_len), prefix_min_tiles(kv_dtype))
      .bytes;
}

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
                                                    int out_dtype, void* stream) {
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs = %d is negative", num_seqs);
  if (num_seqs == 0) return PKV_OK;
  pkv::DecodeArgs a{};
  pkv_status st = check_decode(a, out, q, k_pool, v_pool, block_table, context_lens, num_seqs,
                        num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                        num_blocks, scale, max_context_len, PKV_BF16, out_dtype);
  if (st != PKV_OK) return st;
  if (kv_dtype != PKV_BF16 && kv_dtype != PKV_FP8_E4M3)
    return fail(PKV_ERR_UNSUPPORTED, "kv_dtype %d: bf16 or E4M3 pools", kv_dtype);
  if (kv_dtype == PKV_FP8_E4M3) {
    if (!valid_pool_scale(k_scale) || !valid_pool_scale(v_scale))
      return fail(PKV_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
    if (!std::isfinite(scale * k_scale))
      return fail(PKV_ERR_INVALID_ARG, "scale * k_scale is not finite");
  }
  if (!group_start || !group_prefix_len)
    return fail(PKV_ERR_INVALID_ARG, "null group array");
  if (num_groups <= 0 || num_groups > num_seqs)
    return fail(PKV_ERR_INVALID_ARG, "num_groups %d outside [1, num_seqs]", num_groups);
  if (max_group_size <= 0 || max_group_size > num_seqs)
    return fail(PKV_ERR_INVALID_ARG, "max_group_size %d outside [1, num_seqs]", max_group_size);
  if (max_prefix_len < 0 || max_prefix_len % block_size != 0 || max_prefix_len > a.max_ctx)
    return fail(PKV_ERR_INVALID_ARG,
                "max_prefix_len %d must be a multiple of block_size within the context bound",
                max_prefix_len);
  const int G = num_q_heads / num_kv_heads;
  const int nch = prefix_chunks(max_prefix_len);
  // column units: a workgroup of kPrefixWgWaves waves takes kPrefixWgColumns (sequence, query
  // head) columns of a chunk
  const int cols_per_unit = pkv::kPrefixWgColumns;
  const long long col_blocks =
      (static_cast<long long>(max_group_size) * G + cols_per_unit - 1) / cols_per_unit;
  const long long units = static_cast<long long>(num_groups) * num_kv_heads * nch * col_blocks;
  const long long units_p = (units + 7) / 8 * 8;  // prefix workgroups, a multiple of 8
  const int min_tiles = prefix_min_tiles(kv_dtype);
  st = setup_balanced(a, workspace, workspace_bytes, kDefaultDecodeWaves, num_waves, nch,
                      min_tiles);
  if (st != PKV_OK) return st;
  if (num_waves == 0) {
    // Every workgroup takes one CU (the prefix chunks' LDS): by default the suffix waves fill
    // the CUs that the prefix workgroups leave, all resident from the start (more waves,
    // dispatched as CUs free up, measured 31 against 24 us on the shared-prefix batch).
    int cus = 0;
    if (pkv_status hs = hip_status(device_cu_count(&cus), "compute unit count")) return hs;
    const long long free_cus = std::max<long long>(cus - units_p, cus / 4);
    st = setup_balanced(a, workspace, workspace_bytes,
                        static_cast<int>(std::min<long long>(free_cus * pkv::kPrefixWgWaves,
                                                             kMaxDecodeWaves)),
                        0, nch, min_tiles);
    if (st != PKV_OK) return st;
  }
  if (units_p + a.waves > 0x7fffffffLL)
    return fail(PKV_ERR_UNSUPPORTED, "too many prefix units (%lld)", units);
  a.num_groups = num_groups;
  a.group_start = group_start;
  a.group_prefix_len = group_prefix_len;
  a.prefix_units = static_cast<int>(units_p);
  a.prefix_col_blocks = static_cast<int>(col_blocks);
  a.prefix_chunks = nch;
  a.fp8_kv = kv_dtype == PKV_FP8_E4M3;
  a.k_scale = a.fp8_kv ? k_scale : 1.0f;
  a.v_scale = a.fp8_kv ? v_scale : 1.0f;
  a.bf16_in = 1;
  a.bf16_out = out_dtype == PKV_BF16;
  pkv::DebugCheckArgs d = tables_check(block_table, context_lens, a.S, a.MB, a.B, a.NB, a.max_ctx);
  d.group_start = group_start;
  d.group_prefix_len = group_prefix_len;
  d.NG = num_groups;
  d.max_prefix = max_prefix_len;
  if (pkv_status dst = debug_gate(d, stream, "paged_attention_decode_shared_prefix")) return dst;
  return hip_status(pkv::launch_decode(a, static_cast<hipStream_t>(stream)),
                    "paged_attention_decode_shared_prefix");
}

pkv_status pkv_kv_cache_write_and_decode(void* out, const void* q, const void* k_new,
                                         const void* v_new, const int32_t* slot_mapping,
                                         void* k_pool, void* v_pool, const int32_t* block_table,
                                         const int32_t* context_lens, int num_seqs, int num_q_heads,
                                         int num_kv_heads, int head_dim, int block_size,
                                         int max_blocks_per_seq, int num_blocks, float scale,
                                         int max_context_len, int num_waves, void* workspace,
                                         size_t workspace_bytes, int out_dtype, void* stream) {
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs = %d is negative", num_seqs);
  if (num_seqs == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  pkv::DecodeArgs a{};
  pkv_status st = check_decode(a, out, q, k_pool, v_pool, block_table, context_lens, num_seqs,
                        num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                        num_blocks, scale, max_context_len, PKV_BF16, out_dtype);
  if (st != PKV_OK) return st;
  if (static_cast<long long>(num_blocks) * block_size > 0x7fffffffLL)
    return fail(PKV_ERR_UNSUPPORTED, "pool of %d blocks exceeds int32 slot numbers", num_blocks);
  st = setup_balanced(a, workspace, workspace_bytes, kDefaultDecodeWaves, num_waves);
  if (st != PKV_OK) return st;
  a.step = 1;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slot_mapping = slot_mapping;
  a.bf16_in = 1;
  a.bf16_out = out_dtype == PKV_BF16;
  pkv::DebugCheckArgs d = tables_check(block_table, context_lens, a.S, a.MB, a.B, a.NB, a.max_ctx);
  d.slots = slot_mapping;
  d.T = num_seqs;
  d.slot_NB = num_blocks;
  if (pkv_status dst = debug_gate(d, stream, "kv_cache_write_and_decode")) return dst;
  return hip_status(pkv::launch_decode(a, static_cast<hipStream_t>(stream)),
                    "kv_cache_write_and_decode");
}

pkv_status pkv_paged_attention_decode_fp8(void* out, const void* q, const void* k_pool,
                                          const void* v_pool, const int32_t* block_table,
                                          const int32_t* context_lens, int num_seqs,
                                          int num_q_heads, int num_kv_heads, int head_dim,
                                          int block_size, int max_blocks_per_seq, int num_blocks,
                                          float scale, float k_scale, float v_scale,
                                          int max_context_len, int num_waves, void* workspace,
                                          size_t workspace_bytes, int out_dtype, void* stream) {
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs = %d is negative", num_seqs);
  if (num_seqs == 0) return PKV_OK;
  pkv::DecodeArgs a{};
  pkv_status st = check_decode(a, out, q, k_pool, v_pool, block_table, context_lens, num_seqs,
                        num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                        num_blocks, scale, max_context_len, PKV_BF16, out_dtype);
  if (st != PKV_OK) return st;
  if (!valid_pool_scale(k_scale) || !valid_pool_scale(v_scale))
    return fail(PKV_ERR_INVALID_ARG, "k_scale and v_scale must be finite and positive");
  if (!std::isfinite(scale * k_scale))
    return fail(PKV_ERR_INVALID_ARG, "scale * k_scale is not finite");
  st = setup_balanced(a, workspace, workspace_bytes, kDefaultDecodeWavesFp8, num_waves);
  if (st != PKV_OK) return st;
  a.fp8_kv = 1;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.bf16_in = 1;
  a.bf16_out = out_dtype == PKV_BF16;
  if (pkv_status dst = debug_gate(tables_check(block_table, context_lens, a.S, a.MB, a.B, a.NB,
                                        a.max_ctx), stream, "paged_attention_decode_fp8"))
    return dst;
  return hip_status(pkv::launch_decode(a, static_cast<hipStream_t>(stream)),
                    "paged_attention_decode_fp8");
}

pkv_status pkv_paged_attention_decode(void* out, const void* q, const void* k_pool,
                                      const void* v_pool, const int32_t* block_table,
                                      const int32_t* context_lens, int num_seqs, int num_q_heads,
                                      int num_kv_heads, int head_dim, int block_size,
                                      int max_blocks_per_seq, int num_blocks, float scale,
                                      int max_context_len, int partition_size, int num_waves,
                                      void* workspace, size_t workspace_bytes, int dtype,
                                      int out_dtype, void* stream) {
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs = %d is negative", num_seqs);
  if (num_seqs == 0) return PKV_OK;
  pkv::DecodeArgs a{};
  pkv_status st = check_decode(a, out, q, k_pool, v_pool, block_table, context_lens, num_seqs,
                        num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                        num_blocks, scale, max_context_len, dtype, out_dtype);
  if (st != PKV_OK) return st;
  const int max_ctx = a.max_ctx;
  if (partition_size < 0 || partition_size % 16 != 0 || partition_size % block_size != 0)
    return fail(PKV_ERR_INVALID_ARG,
                "partition_size %d must be a non-negative multiple of 16 and of block_size",
                partition_size);
  if (partition_size == 0 && dtype == PKV_BF16) {
    st = setup_balanced(a, workspace, workspace_bytes, kDefaultDecodeWaves, num_waves);
    if (st != PKV_OK) return st;
  } else {
    const int P = resolve_partition(partition_size, num_seqs, num_kv_heads, max_ctx);
    if (P % block_size != 0)
      return fail(PKV_ERR_INVALID_ARG, "partition size %d not a multiple of block_size", P);
    const int NP = num_partitions(max_ctx, P);
    const size_t need = fixed_workspace_bytes(num_seqs, num_q_heads, head_dim, NP);
    if (need > 0 && (!workspace || workspace_bytes < need))
      return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes : static_cast<size_t>(0));
    a.P = P;
    a.NP = NP;
    if (NP > 1) {
      const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * NP;
      float* base = static_cast<float*>(workspace);
      a.part_o = base;
      a.part_m = base + rows * head_dim;
      a.part_l = a.part_m + rows;
    }
  }
  a.bf16_in = dtype == PKV_BF16;
  a.bf16_out = out_dtype == PKV_BF16;
  if (pkv_status dst = debug_gate(tables_check(block_table, context_lens, a.S, a.MB, a.B, a.NB,
                                        a.max_ctx), stream, "paged_attention_decode"))
    return dst;
  return hip_status(pkv::launch_decode(a, static_cast<hipStream_t>(stream)),
                    "paged_attention_decode");
}

}  // extern "C"

namespace {
// The probe launches whole workgroups of kBalancedWavesPerGroup waves, and every launched wave
// may store its 64 words.
size_t probe_sink_bytes(int waves) {
  const size_t per = pkv::kBalancedWavesPerGroup;
  const size_t launched = (static_cast<size_t>(waves) + per - 1) / per * per;
  return launched * 64 * sizeof(uint32_t);
}
}  // namespace

extern "C" {

pkv_status pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_pool,
                                              const void* v_pool, const int32_t* block_table,
                                              const int32_t* context_lens, int num_seqs,
                                              int num_q_heads, int num_kv_heads, int head_dim,
                                              int block_size, int max_blocks_per_seq,
                                              int num_blocks, float scale, int max_context_len,
                                              int num_waves, int out_dtype, void* stream) {
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs = %d is negative", num_seqs);
  if (num_seqs == 0) return PKV_OK;
  pkv::DecodeArgs a{};
  pkv_status st = check_decode(a, out, q, k_pool, v_pool, block_table, context_lens, num_seqs,
                        num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                        num_blocks, scale, max_context_len, PKV_BF16, out_dtype);
  if (st != PKV_OK) return st;
  if (num_waves < 0 || num_waves > kMaxDecodeWaves)
    return fail(PKV_ERR_INVALID_ARG, "num_waves %d outside [0, %d]", num_waves, kMaxDecodeWaves);
  // the size check is made before any HIP call
  const size_t need =
      balanced_plan(a.S, a.Hq, a.Hkv, a.D, a.max_ctx,
                    num_waves > 0 ? num_waves : kDefaultDecodeWaves).bytes;
  if (need > pkv::kNoAllocScratchBytes)
    return fail(PKV_ERR_WORKSPACE,
                "these sizes need %zu bytes of scratch; the library's static scratch holds %zu "
                "(use pkv_paged_attention_decode with a workspace)",
                need, pkv::kNoAllocScratchBytes);
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (pkv_status hs = hip_status(pkv::noalloc_scratch(&ws, &ws_bytes), "decode_noalloc scratch"))
    return hs;
  st = setup_balanced(a, ws, ws_bytes, kDefaultDecodeWaves, num_waves);
  if (st != PKV_OK) return st;
  a.bf16_in = 1;
  a.bf16_out = out_dtype == PKV_BF16;
  if (pkv_status dst = debug_gate(tables_check(block_table, context_lens, a.S, a.MB, a.B, a.NB,
                                        a.max_ctx), stream, "paged_attention_decode_noalloc"))
    return dst;
  return hip_status(pkv::launch_decode(a, static_cast<hipStream_t>(stream)),
                    "paged_attention_decode_noalloc");
}

size_t pkv_decode_read_probe_sink_size(int num_seqs, int num_q_heads, int num_kv_heads,
                                       int max_context_len, int num_waves) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || num_waves < 0 || num_waves > kMaxDecodeWaves)
    return 0;
  const BalancedPlan pl = balanced_plan(num_seqs, num_q_heads, num_kv_heads, 64,
                                        max_context_len,
                                        num_waves > 0 ? num_waves : kDefaultDecodeWaves);
  return probe_sink_bytes(pl.waves);
}

pkv_status pkv_decode_read_probe(const void* k_pool, const void* v_pool, const int32_t* block_table,
                                 const int32_t* context_lens, int num_seqs, int num_q_heads,
                                 int num_kv_heads, int head_dim, int block_size,
                                 int max_blocks_per_seq, int num_blocks, int max_context_len,
                                 int num_waves, void* sink, size_t sink_bytes, void* stream) {
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs = %d is negative", num_seqs);
  if (num_seqs == 0) return PKV_OK;
  pkv::DecodeArgs a{};
  pkv_status st = check_decode(a, sink, sink, k_pool, v_pool, block_table, context_lens, num_seqs,
                        num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                        num_blocks, 1.0f, max_context_len, PKV_BF16, PKV_BF16);
  if (st != PKV_OK) return st;
  if (num_waves < 0 || num_waves > kMaxDecodeWaves)
    return fail(PKV_ERR_INVALID_ARG, "num_waves %d outside [0, %d]", num_waves, kMaxDecodeWaves);
  const BalancedPlan pl = balanced_plan(a.S, a.Hq, a.Hkv, a.D, a.max_ctx,
                                        num_waves > 0 ? num_waves : kDefaultDecodeWaves);
  const size_t need = probe_sink_bytes(pl.waves);
  if (!sink || sink_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "sink of %zu bytes needed, %zu given", need, sink_bytes);
  pkv::ReadProbeArgs r{static_cast<uint32_t*>(sink), k_pool, v_pool, block_table, context_lens,
                       a.S, a.Hq, a.Hkv, a.D, a.B, a.MB, pl.waves, kMinTilesPerWave};
  if (pkv_status dst = debug_gate(tables_check(block_table, context_lens, a.S, a.MB, a.B, a.NB,
                                        a.max_ctx), stream, "decode_read_probe"))
    return dst;
  return hip_status(pkv::launch_read_probe(r, static_cast<hipStream_t>(stream)),
                    "decode_read_probe");
}

pkv_status pkv_paged_attention_prefill_chunk(void* out, const void* q, const int32_t* cu_q_lens,
                                             const int32_t* context_lens, const void* k_pool,
                                             const void* v_pool, const int32_t* block_table,
                                             int num_seqs, int total_q, int num_q_heads,
                                             int num_kv_heads, int head_dim, int block_size,
                                             int max_blocks_per_seq, int num_blocks, float scale,
                                             int max_q_len, int max_context_len, int dtype,
                                             int out_dtype, void* stream) {
  if (num_seqs < 0 || total_q < 0)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs and total_q must be non-negative");
  if (num_seqs == 0 || total_q == 0) return PKV_OK;
  if (!out || !q || !cu_q_lens || !context_lens || !k_pool || !v_pool || !block_table)
    return fail(PKV_ERR_INVALID_ARG, "null pointer argument");
  pkv_status st = check_common(num_q_heads, num_kv_heads, head_dim, block_size, dtype, out_dtype);
  if (st != PKV_OK) return st;
  if (max_blocks_per_seq <= 0 || num_blocks <= 0)
    return fail(PKV_ERR_INVALID_ARG, "max_blocks_per_seq and num_blocks must be positive");
  if (!std::isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale is not finite");
  const long long cap = static_cast<long long>(max_blocks_per_seq) * block_size;
  if (cap > 0x7fffffffLL) return fail(PKV_ERR_UNSUPPORTED, "max_blocks_per_seq too large");
  if (max_context_len < 0 || max_context_len > cap)
    return fail(PKV_ERR_INVALID_ARG, "max_context_len %d outside [0, %lld]", max_context_len,
                cap);
  if (max_q_len < 0 || max_q_len > total_q)
    return fail(PKV_ERR_INVALID_ARG, "max_q_len %d outside [0, total_q = %d]", max_q_len,
                total_q);
  if (num_seqs > kMaxGridYZ) return fail(PKV_ERR_UNSUPPORTED, "num_seqs %d too large", num_seqs);
  const long long gy = static_cast<long long>(num_q_heads);  // upper bound on grid y
  if (gy > kMaxGridYZ) return fail(PKV_ERR_UNSUPPORTED, "too many heads");
  pkv::PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.cu_q_lens = cu_q_lens;
  a.context_lens = context_lens;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.S = num_seqs;
  a.total_q = total_q;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.D = head_dim;
  a.B = block_size;
  a.MB = max_blocks_per_seq;
  a.NB = num_blocks;
  a.scale = scale;
  a.max_q_len = max_q_len > 0 ? max_q_len : total_q;
  a.max_ctx = max_context_len > 0 ? max_context_len : static_cast<int>(cap);
  a.bf16_in = dtype == PKV_BF16;
  a.bf16_out = out_dtype == PKV_BF16;
  pkv::DebugCheckArgs d = tables_check(block_table, context_lens, a.S, a.MB, a.B, a.NB, a.max_ctx);
  d.cu_q_lens = cu_q_lens;
  d.total_q = total_q;
  if (pkv_status dst = debug_gate(d, stream, "paged_attention_prefill_chunk")) return dst;
  return hip_status(pkv::launch_prefill(a, static_cast<hipStream_t>(stream)),
                    "paged_attention_prefill_chunk");
}

pkv_status pkv_profile_enable(int kernel_mask) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  drain_locked();
  for (int i = 0; i < pkv::K_COUNT; ++i) {
    g_total_ms[i] = 0.0;
    g_launches[i] = 0;
  }
  g_timing_mask = static_cast<unsigned>(kernel_mask) & ((1u << pkv::K_COUNT) - 1u);
  return PKV_OK;
}

pkv_status pkv_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  drain_locked();
  for (int i = 0; i < pkv::K_COUNT; ++i) {
    g_total_ms[i] = 0.0;
    g_launches[i] = 0;
  }
  return PKV_OK;
}

pkv_status pkv_profile_read(const char* kernel_name, double* total_ms, long long* launches) {
  if (!kernel_name) return fail(PKV_ERR_INVALID_ARG, "null kernel name");
  std::lock_guard<std::mutex> lk(g_timing_mu);
  drain_locked();
  for (int i = 0; i < pkv::K_COUNT; ++i) {
    if (std::string(kernel_name) == pkv::kernel_name(i)) {
      if (total_ms) *total_ms = g_total_ms[i];
      if (launches) *launches = g_launches[i];
      return PKV_OK;
    }
  }
  return fail(PKV_ERR_INVALID_ARG, "unknown kernel name '%s'", kernel_name);
}

const char* pkv_profile_kernel_names(void) {
  return "kv_cache_write,decode_partition,decode_reduce,prefill_chunk,copy_blocks,read_probe,"
         "debug_check";
}

}  // extern "C"
