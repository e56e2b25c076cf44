// kv_cache_write: scatter new K/V rows into pool slots through a slot mapping.
//
// Token i with slot = slot_mapping[i] >= 0 goes to physical block slot / B at offset slot % B
// ("Serving Engines", How vLLM works: new tokens are placed through a slot mapping; the
// zhichai.net block-table figure, section 1: block-then-offset addressing). A pure copy of
// 16-bit or 32-bit words; NaN payloads are kept.
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
