// kv_cache_write: scatter new K/V rows into pool slots through a slot mapping.
//
// Token i with slot = slot_mapping[i] >= 0 goes to physical block slot / B at offset slot % B
// ("Serving Engines", How vLLM works: new tokens are placed through a slot mapping; the
// zhichai.net block-table figure, section 1: block-then-offset addressing). A pure copy of
// 16-bit or 32-bit words; NaN payloads are kept.
//
// E4M3 pools (kv_write_fp8_kernel): the same placement of one-byte codes, each the quantised
// quotient element / scale.
//
// Layout: k_pool [NB][Hkv][B][D] (a token's row is D contiguous elements),
//         v_pool [NB][Hkv][D][B] (a token's values are B elements apart).
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

// Work split (both kernels): a workgroup takes 16 consecutive tokens of one KV head; thread
// (token tt = tid % 16, chunk c = tid / 16) moves one 16-byte piece of the token's row. The token
// is the fastest lane index, so when consecutive tokens go to consecutive slots of a block (a
// prefill chunk) each V dimension's values of the 16 tokens form one contiguous run in the
// dim-major V tile, and the stores of a wave coalesce. Any slot mapping is still handled.
constexpr int kWriteGroup = 16;

template <typename T>
__global__ __launch_bounds__(512) void kv_write_kernel(const T* __restrict__ k_new,
                                                       const T* __restrict__ v_new,
                                                       T* __restrict__ k_pool,
                                                       T* __restrict__ v_pool,
                                                       const int32_t* __restrict__ slot_mapping,
                                                       int T_tokens, int Hkv, int D, int B) {
  constexpr int VEC = 16 / sizeof(T);
  const int i = blockIdx.x * kWriteGroup + (threadIdx.x % kWriteGroup);
  const int d0 = (threadIdx.x / kWriteGroup) * VEC;
  const int h = blockIdx.y;
  if (i >= T_tokens || d0 >= D) return;
  const int slot = slot_mapping[i];
  if (slot < 0) return;
  const int64_t blk = slot / B;
  const int off = slot - static_cast<int>(blk) * B;
  const int64_t src = (static_cast<int64_t>(i) * Hkv + h) * D + d0;
  const int64_t tile = blk * Hkv + h;
  *reinterpret_cast<u32x4*>(k_pool + (tile * B + off) * D + d0) = load16(k_new + src);
  const u32x4 vv = load16(v_new + src);
  T vals[VEC];
  __builtin_memcpy(vals, &vv, 16);
  T* vdst = v_pool + (tile * D + d0) * B + off;
#pragma unroll
  for (int e = 0; e < VEC; ++e) vdst[static_cast<int64_t>(e) * B] = vals[e];
}

// E4M3 code of a float32: the nearest representable value, ties to the even code; magnitudes
// of 448 and beyond (infinity too) saturate to the largest finite code; NaN gives 0x7F; the
// sign bit is x's. Integer steps on the binary32 word:
//   |x| < 2^-6   the E4M3 values there are the multiples of 2^-9 (subnormals, then 2^-6
//                itself), so the code is |x| * 2^9 rounded to the nearest even integer;
//   otherwise    rebias the exponent from 127 to 7 and round the 23 fraction bits to 3, to
//                nearest even; a carry out of the fraction moves the exponent up, as it should.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;  // 448 = 1.75 * 2^8
  if (a < 0x3c800000u)                        // 2^-6
    return sign | static_cast<uint32_t>(__builtin_rintf(__uint_as_float(a) * 512.0f));
  uint32_t r = a - (120u << 23);
  r += 0x7ffffu + ((r >> 20) & 1u);
  return sign | (r >> 20);
}

template <typename In>
__device__ __forceinline__ void load_row16(const In* p, float (&x)[16]) {
  if constexpr (sizeof(In) == 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 w = load16(p + 8 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[8 * h + 2 * i] = bf16_lo(w[i]);
        x[8 * h + 2 * i + 1] = bf16_hi(w[i]);
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const u32x4 w = load16(p + 4 * h);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * h + i] = __uint_as_float(w[i]);
    }
  }
}

// Same work split as kv_write_kernel; a thread quantises 16 consecutive elements of one head's
// row: K leaves as one 16-byte store, V as 16 single bytes, one per dimension.
template <typename In>
__global__ __launch_bounds__(512) void kv_write_fp8_kernel(
    const In* __restrict__ k_new, const In* __restrict__ v_new, uint8_t* __restrict__ k_pool,
    uint8_t* __restrict__ v_pool, const int32_t* __restrict__ slot_mapping, int T_tokens, int Hkv,
    int D, int B, float k_scale, float v_scale) {
  const int i = blockIdx.x * kWriteGroup + (threadIdx.x % kWriteGroup);
  const int d0 = (threadIdx.x / kWriteGroup) * 16;
  const int h = blockIdx.y;
  if (i >= T_tokens || d0 >= D) return;
  const int slot = slot_mapping[i];
  if (slot < 0) return;
  const int64_t blk = slot / B;
  const int off = slot - static_cast<int>(blk) * B;
  const int64_t src = (static_cast<int64_t>(i) * Hkv + h) * D + d0;
  const int64_t tile = blk * Hkv + h;
  float x[16];
  load_row16(k_new + src, x);
  u32x4 kw = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 16; ++e) kw[e / 4] |= e4m3_code(x[e] / k_scale) << (8 * (e % 4));
  *reinterpret_cast<u32x4*>(k_pool + (tile * B + off) * D + d0) = kw;
  load_row16(v_new + src, x);
  uint8_t* vdst = v_pool + (tile * D + d0) * B + off;
#pragma unroll
  for (int e = 0; e < 16; ++e)
    vdst[static_cast<int64_t>(e) * B] = static_cast<uint8_t>(e4m3_code(x[e] / v_scale));
}

hipError_t launch_kv_write_fp8(const KvWriteArgs& a, int in_bf16, float k_scale, float v_scale,
                               hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid((a.T + kWriteGroup - 1) / kWriteGroup, a.Hkv);
  const dim3 block(kWriteGroup * (a.D / 16));
  if (in_bf16) {
    return launch_kernel(K_KV_WRITE, kv_write_fp8_kernel<uint16_t>, grid, block, stream,
        static_cast<const uint16_t*>(a.k_new), static_cast<const uint16_t*>(a.v_new),
        static_cast<uint8_t*>(a.k_pool), static_cast<uint8_t*>(a.v_pool), a.slot_mapping, a.T,
        a.Hkv, a.D, a.B, k_scale, v_scale);
  } else {
    return launch_kernel(K_KV_WRITE, kv_write_fp8_kernel<float>, grid, block, stream,
        static_cast<const float*>(a.k_new), static_cast<const float*>(a.v_new),
        static_cast<uint8_t*>(a.k_pool), static_cast<uint8_t*>(a.v_pool), a.slot_mapping, a.T,
        a.Hkv, a.D, a.B, k_scale, v_scale);
  }
}

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const int vec = 16 / a.elem_bytes;
  const dim3 grid((a.T + kWriteGroup - 1) / kWriteGroup, a.Hkv);
  const dim3 block(kWriteGroup * (a.D / vec));
  if (a.elem_bytes == 2) {
    return launch_kernel(K_KV_WRITE, kv_write_kernel<uint16_t>, grid, block, stream,
        static_cast<const uint16_t*>(a.k_new), static_cast<const uint16_t*>(a.v_new),
        static_cast<uint16_t*>(a.k_pool), static_cast<uint16_t*>(a.v_pool), a.slot_mapping, a.T,
        a.Hkv, a.D, a.B);
  } else {
    return launch_kernel(K_KV_WRITE, kv_write_kernel<float>, grid, block, stream,
        static_cast<const float*>(a.k_new), static_cast<const float*>(a.v_new),
        static_cast<float*>(a.k_pool), static_cast<float*>(a.v_pool), a.slot_mapping, a.T, a.Hkv,
        a.D, a.B);
  }
}

}  // namespace pkv
