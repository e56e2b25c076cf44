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
// One workgroup per token; a thread copies 16 contiguous bytes of one head's row.
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

template <typename T>
__global__ __launch_bounds__(256) void kv_write_kernel(const T* __restrict__ k_new,
                                                       const T* __restrict__ v_new,
                                                       T* __restrict__ k_pool,
                                                       T* __restrict__ v_pool,
                                                       const int32_t* __restrict__ slot_mapping,
                                                       int Hkv, int D, int B) {
  constexpr int VEC = 16 / sizeof(T);
  const int i = blockIdx.x;
  const int slot = slot_mapping[i];
  if (slot < 0) return;
  const int64_t blk = slot / B;
  const int off = slot - static_cast<int>(blk) * B;
  const int chunks = Hkv * (D / VEC);
  for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
    const int h = c / (D / VEC);
    const int d0 = (c - h * (D / VEC)) * VEC;
    const int64_t src = (static_cast<int64_t>(i) * Hkv + h) * D + d0;
    const u32x4 kv = load16(k_new + src);
    const u32x4 vv = load16(v_new + src);
    const int64_t tile = blk * Hkv + h;
    *reinterpret_cast<u32x4*>(k_pool + (tile * B + off) * D + d0) = kv;
    T vals[VEC];
    __builtin_memcpy(vals, &vv, 16);
    T* vdst = v_pool + (tile * D + d0) * B + off;
#pragma unroll
    for (int e = 0; e < VEC; ++e) vdst[static_cast<int64_t>(e) * B] = vals[e];
  }
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

// One workgroup per token; a thread quantises 16 consecutive elements of one head's row: K
// leaves as one 16-byte store, V as 16 single bytes B apart.
template <typename In>
__global__ __launch_bounds__(256) void kv_write_fp8_kernel(const In* __restrict__ k_new,
                                                           const In* __restrict__ v_new,
                                                           uint8_t* __restrict__ k_pool,
                                                           uint8_t* __restrict__ v_pool,
                                                           const int32_t* __restrict__ slot_mapping,
                                                           int Hkv, int D, int B, float k_scale,
                                                           float v_scale) {
  const int i = blockIdx.x;
  const int slot = slot_mapping[i];
  if (slot < 0) return;
  const int64_t blk = slot / B;
  const int off = slot - static_cast<int>(blk) * B;
  const int chunks = Hkv * (D / 16);
  for (int c = threadIdx.x; c < chunks; c += blockDim.x) {
    const int h = c / (D / 16);
    const int d0 = (c - h * (D / 16)) * 16;
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
}

hipError_t launch_kv_write_fp8(const KvWriteArgs& a, int in_bf16, float k_scale, float v_scale,
                               hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const int chunks = a.Hkv * (a.D / 16);
  const int threads = chunks >= 256 ? 256 : ((chunks + 63) / 64) * 64;
  if (in_bf16) {
    (void)launch_kernel(K_KV_WRITE, kv_write_fp8_kernel<uint16_t>, dim3(a.T), dim3(threads),
        stream, static_cast<const uint16_t*>(a.k_new), static_cast<const uint16_t*>(a.v_new),
        static_cast<uint8_t*>(a.k_pool), static_cast<uint8_t*>(a.v_pool), a.slot_mapping, a.Hkv,
        a.D, a.B, k_scale, v_scale);
  } else {
    (void)launch_kernel(K_KV_WRITE, kv_write_fp8_kernel<float>, dim3(a.T), dim3(threads),
        stream, static_cast<const float*>(a.k_new), static_cast<const float*>(a.v_new),
        static_cast<uint8_t*>(a.k_pool), static_cast<uint8_t*>(a.v_pool), a.slot_mapping, a.Hkv,
        a.D, a.B, k_scale, v_scale);
  }
  return hipGetLastError();
}

hipError_t launch_kv_write(const KvWriteArgs& a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const int vec = 16 / a.elem_bytes;
  const int chunks = a.Hkv * (a.D / vec);
  const int threads = chunks >= 256 ? 256 : ((chunks + 63) / 64) * 64;
  if (a.elem_bytes == 2) {
    (void)launch_kernel(K_KV_WRITE, kv_write_kernel<uint16_t>, dim3(a.T), dim3(threads), stream,
        static_cast<const uint16_t*>(a.k_new), static_cast<const uint16_t*>(a.v_new),
        static_cast<uint16_t*>(a.k_pool), static_cast<uint16_t*>(a.v_pool), a.slot_mapping, a.Hkv,
        a.D, a.B);
  } else {
    (void)launch_kernel(K_KV_WRITE, kv_write_kernel<float>, dim3(a.T), dim3(threads), stream,
        static_cast<const float*>(a.k_new), static_cast<const float*>(a.v_new),
        static_cast<float*>(a.k_pool), static_cast<float*>(a.v_pool), a.slot_mapping, a.Hkv, a.D,
        a.B);
  }
  hipError_t e = hipGetLastError();
  return e;
}

}  // namespace pkv
