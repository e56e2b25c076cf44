// paged_attention_decode: one query token per sequence against its paged K/V.
//
// What is computed ("LLM Serving Engine Shootout", 3.1 equation and 5.1 steps; 2.1 for GQA):
//   a_j = scale * q . k_j for the n cached tokens, k_j read from block table[j / B] at offset
//   j % B; out = softmax(a) . V. Query head h uses KV head h / G (G = Hq / Hkv).
//
// Split context: the context is cut into partitions of P tokens. Each partition keeps a running
// maximum m and sum l of exponentials while it walks its tiles (the online softmax), and stores
// (m, l, acc / l). A second kernel merges the partitions with weights l_p * 2^(m_p - M). With a
// single partition the first kernel writes the output itself.
//
// bf16 path (matrix cores). One wave owns (sequence, KV head, partition) and walks 32-token
// tiles (one block of 32 or two consecutive logical blocks of 16). Per tile:
//   S^T[32 tok][16 heads] = K_tile . Q^T        two 16x16x32 MFMAs per 32 dims
//   online softmax on S^T (lane = head column, 8 tokens per lane)
//   O^T[D][16 heads]     += V_tile^T . P^T     one 16x16x32 MFMA per 16 dims
// The output layout of the first product (a lane holds one head column and four consecutive
// rows) is also the B-operand layout the second product needs, so P never leaves registers. For
// that to line up, the tile's tokens are assigned to MFMA rows so that the lane in row group lg
// ends up holding tokens 8*lg .. 8*lg+7: then its V^T operand is 16 contiguous bytes of the
// dim-major V tile. Heads beyond G in the 16-wide column are zero queries whose results are
// dropped; the kernel is bound by HBM reads of K and V, so the padded MFMA work is free.
// K and V of the next tile are loaded while the current tile is computed (two register sets).
//
// fp32 path (vector ALUs): one wave owns (sequence, query head, partition); lanes take one token
// each for the scores, then one output dimension each for P.V.
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;

template <int D, int B>
struct KvTile {
  u32x4 k[2][D / 32];
  u32x4 v[D / 16];
};

template <int D, int B, bool SPLIT, typename OutT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void decode_bf16_kernel(
    OutT* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_m,
    float* __restrict__ part_l, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kpool, const uint16_t* __restrict__ vpool,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ context_lens, int Hq,
    int Hkv, int G, int HG, int MB, int P, int NP, float scale_log2) {
  constexpr int KK = D / 32;
  constexpr int DT = D / 16;
  constexpr int TILE = B * D;  // elements of one (block, head) tile

  const int lane = threadIdx.x;
  const int r16 = lane & 15;
  const int lg = lane >> 4;
  const int p = blockIdx.x;
  const int g = blockIdx.y / HG;
  const int hgrp = blockIdx.y - g * HG;
  const int s = blockIdx.z;
  const int n = context_lens[s];
  const int start = p * P;
  const int hl = hgrp * 16 + r16;
  const bool hvalid = hl < G;
  const int h = g * G + (hvalid ? hl : 0);

  if (start >= n) {
    if (!SPLIT && p == 0 && hvalid) {  // empty context: zero row
      OutT* o = out + (static_cast<int64_t>(s) * Hq + h) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) store_out(o + 16 * dt + 4 * lg + e, 0.0f);
    }
    return;
  }
  const int end = min(start + P, n);
  const int ntiles = (end - start + 31) >> 5;
  const int nblk = (n + B - 1) / B;
  const int32_t* bt = block_table + static_cast<int64_t>(s) * MB;

  // Q as the B operand: column = head, contraction slots d = 32*kk + 8*lg + e.
  u32x4 qf[KK];
  {
    const uint16_t* qrow = q + (static_cast<int64_t>(s) * Hq + h) * D + 8 * lg;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = hvalid ? load16(qrow + 32 * kk) : u32x4{0u, 0u, 0u, 0u};
  }

  // K operand row r16 of half hf holds tile token 8*(r16/4) + 4*hf + r16%4.
  int koff[2];
  int ksel = 0;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int tau = 8 * (r16 >> 2) + 4 * hf + (r16 & 3);
    koff[hf] = (tau % B) * D + 8 * lg;
    ksel = tau / B;  // same block for both halves
  }
  // V^T operand: row d = 16*dt + r16, tokens 8*lg .. 8*lg+7 of the tile.
  const int vsel = (B == 16) ? (lg >> 1) : 0;
  const int vtok = (B == 16) ? 8 * (lg & 1) : 8 * lg;
  const int voff = r16 * B + vtok;

  const int64_t head_off = static_cast<int64_t>(g) * TILE;
  const int64_t blk_stride = static_cast<int64_t>(Hkv) * TILE;

  auto load_tile = [&](KvTile<D, B>& T, int t) {
    const int lb0 = (start + 32 * t) / B;
    const int id0 = bt[min(lb0, nblk - 1)];
    const int id1 = (B == 16) ? bt[min(lb0 + 1, nblk - 1)] : id0;
    const uint16_t* kb = kpool + (ksel ? id1 : id0) * blk_stride + head_off;
    const uint16_t* vb = vpool + (vsel ? id1 : id0) * blk_stride + head_off;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) T.k[hf][kk] = load16(kb + koff[hf] + 32 * kk);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) T.v[dt] = load16(vb + voff + 16 * dt * B);
  };

  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  float l = 0.f;

  auto compute = [&](KvTile<D, B>& T, int t) {
    const int tok0 = start + 32 * t;
    f32x4 sc[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      sc[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) sc[hf] = mfma16x16x32(T.k[hf][kk], qf[kk], sc[hf]);
    }
    // lane: head column r16, tile tokens 8*lg + 4*hf + e
    const int lim = end - tok0;
    float x[8];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tt = 8 * lg + 4 * hf + e;
        x[4 * hf + e] = (tt < lim) ? sc[hf][e] * scale_log2 : -INFINITY;
      }
    float tmax = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, x[i]);
    tmax = wave_max_xor(tmax, 16);
    tmax = wave_max_xor(tmax, 32);
    const float mnew = fmaxf(m, tmax);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    float psum = 0.f;
    u32x4 pb;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float p0 = fast_exp2(x[2 * w] - mnew);
      const float p1 = fast_exp2(x[2 * w + 1] - mnew);
      psum += p0 + p1;
      pb[w] = pack_bf16x2(p0, p1);
    }
    l = l * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
    // Token slots at or past n may hold stale words (NaN) or come from a borrowed block:
    // their P is 0, but 0 * NaN is NaN, so clear the V words themselves.
    const int vlim = n - tok0;
    if (vlim < 32) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int t0 = 8 * lg + 2 * w;
        const uint32_t keep =
            (t0 < vlim ? 0x0000ffffu : 0u) | (t0 + 1 < vlim ? 0xffff0000u : 0u);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) T.v[dt][w] &= keep;
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma16x16x32(T.v[dt], pb, acc[dt]);
  };

  KvTile<D, B> ta, tb;
  load_tile(ta, 0);
  for (int t = 0; t < ntiles; t += 2) {
    if (t + 1 < ntiles) load_tile(tb, t + 1);
    compute(ta, t);
    if (t + 1 >= ntiles) break;
    if (t + 2 < ntiles) load_tile(ta, t + 2);
    compute(tb, t + 1);
  }

  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const float inv = 1.0f / l;
  if (!hvalid) return;
  const int64_t row = static_cast<int64_t>(s) * Hq + h;
  if constexpr (!SPLIT) {
    OutT* o = out + row * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) store_out(o + 16 * dt + 4 * lg + e, acc[dt][e] * inv);
  } else {
    const int64_t idx = row * NP + p;
    if (lg == 0) {
      part_m[idx] = m;
      part_l[idx] = l;
    }
    float* o = part_o + idx * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(o + 16 * dt + 4 * lg) = acc[dt] * inv;
  }
}

// fp32 path. `rows` are decode sequences (PREFILL = false) or prefill query tokens.
template <int D, int B, bool SPLIT, bool PREFILL, typename OutT>
__global__ __launch_bounds__(64) void attn_f32_kernel(
    OutT* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_m,
    float* __restrict__ part_l, const float* __restrict__ q, const float* __restrict__ kpool,
    const float* __restrict__ vpool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ cu_q_lens, int S,
    int Hq, int Hkv, int MB, int P, int NP, float scale_log2) {
  constexpr int DPL = D / 64;
  __shared__ float qs[D];
  __shared__ float ps[64];
  __shared__ int64_t vbase[64];

  const int lane = threadIdx.x;
  const int row = blockIdx.x;
  const int h = blockIdx.y;
  const int p = blockIdx.z;
  const int g = h / (Hq / Hkv);
  int s = row;
  int n;  // keys visible to this row
  if constexpr (PREFILL) {
    int lo = 0, hi = S;  // find s with cu[s] <= row < cu[s+1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu_q_lens[mid] <= row) lo = mid; else hi = mid;
    }
    s = lo;
    const int c = cu_q_lens[s + 1] - cu_q_lens[s];
    n = context_lens[s] - c + (row - cu_q_lens[s]) + 1;
  } else {
    n = context_lens[s];
  }
  const int start = p * P;
  const int64_t orow = static_cast<int64_t>(row) * Hq + h;
  if (start >= n) {
    if (!SPLIT && p == 0)
      for (int i = 0; i < DPL; ++i) store_out(out + orow * D + lane + 64 * i, 0.0f);
    return;
  }
  const int end = min(start + P, n);
  const int32_t* bt = block_table + static_cast<int64_t>(s) * MB;
  for (int i = 0; i < DPL; ++i) qs[lane + 64 * i] = q[orow * D + lane + 64 * i];
  __syncthreads();

  float acc[DPL];
  for (int i = 0; i < DPL; ++i) acc[i] = 0.f;
  float m = -INFINITY, l = 0.f;
  for (int tok0 = start; tok0 < end; tok0 += 64) {
    const int tok = tok0 + lane;
    float x = -INFINITY;
    if (tok < end) {
      const int64_t blk = bt[tok / B];
      const int off = tok % B;
      const float* krow = kpool + ((blk * Hkv + g) * B + off) * D;
      float dot = 0.f;
      for (int d = 0; d < D; d += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(krow + d);
        dot += qs[d] * kv.x + qs[d + 1] * kv.y + qs[d + 2] * kv.z + qs[d + 3] * kv.w;
      }
      x = dot * scale_log2;
      vbase[lane] = (blk * Hkv + g) * D * B + off;
    }
    float tmax = x;
    for (int mk = 32; mk >= 1; mk >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, mk));
    const float mnew = fmaxf(m, tmax);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    const float pv = (tok < end) ? fast_exp2(x - mnew) : 0.f;
    float psum = pv;
    for (int mk = 32; mk >= 1; mk >>= 1) psum += __shfl_xor(psum, mk);
    l = l * alpha + psum;
    ps[lane] = pv;
    __syncthreads();
    const int cnt = min(64, end - tok0);
    for (int i = 0; i < DPL; ++i) acc[i] *= alpha;
    for (int j = 0; j < cnt; ++j) {
      const float pj = ps[j];
      const int64_t vb = vbase[j];
      for (int i = 0; i < DPL; ++i) acc[i] += pj * vpool[vb + static_cast<int64_t>(lane + 64 * i) * B];
    }
    __syncthreads();
  }
  const float inv = 1.0f / l;
  if constexpr (!SPLIT) {
    for (int i = 0; i < DPL; ++i) store_out(out + orow * D + lane + 64 * i, acc[i] * inv);
  } else {
    const int64_t idx = orow * NP + p;
    if (lane == 0) {
      part_m[idx] = m;
      part_l[idx] = l;
    }
    for (int i = 0; i < DPL; ++i) part_o[idx * D + lane + 64 * i] = acc[i] * inv;
  }
}

// Merge of the partitions: out = sum_p w_p o_p / sum_p w_p, w_p = l_p * 2^(m_p - max m).
template <typename OutT>
__global__ __launch_bounds__(64) void decode_reduce_kernel(
    OutT* __restrict__ out, const float* __restrict__ part_o, const float* __restrict__ part_m,
    const float* __restrict__ part_l, const int32_t* __restrict__ context_lens, int Hq, int D,
    int P, int NP) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int n = context_lens[s];
  const int np = min((n + P - 1) / P, NP);  // NP bounds the workspace rows
  const int64_t row = static_cast<int64_t>(s) * Hq + h;
  OutT* o = out + row * D;
  if (np <= 0) {
    for (int d = threadIdx.x; d < D; d += 64) store_out(o + d, 0.0f);
    return;
  }
  const float* pm = part_m + row * NP;
  const float* pl = part_l + row * NP;
  float M = -INFINITY;
  for (int i = 0; i < np; ++i) M = fmaxf(M, pm[i]);
  float wsum = 0.f;
  float acc0 = 0.f, acc1 = 0.f;
  const float* po = part_o + row * NP * D;
  const int d0 = threadIdx.x, d1 = threadIdx.x + 64;
  for (int i = 0; i < np; ++i) {
    const float w = pl[i] * fast_exp2(pm[i] - M);
    wsum += w;
    acc0 += w * po[static_cast<int64_t>(i) * D + d0];
    if (d1 < D) acc1 += w * po[static_cast<int64_t>(i) * D + d1];
  }
  const float inv = 1.0f / wsum;
  store_out(o + d0, acc0 * inv);
  if (d1 < D) store_out(o + d1, acc1 * inv);
}

// ------------------------------------------------------------------------------ launchers

template <int D, int B, bool SPLIT, typename OutT>
static void launch_bf16(const DecodeArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const int HG = (G + 15) / 16;
  dim3 grid(a.NP, a.Hkv * HG, a.S);
  decode_bf16_kernel<D, B, SPLIT, OutT><<<grid, 64, 0, st>>>(
      static_cast<OutT*>(a.out), a.part_o, a.part_m, a.part_l,
      static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k_pool),
      static_cast<const uint16_t*>(a.v_pool), a.block_table, a.context_lens, a.Hq, a.Hkv, G, HG,
      a.MB, a.P, a.NP, a.scale * kLog2e);
}

template <int D, int B, bool SPLIT, typename OutT>
static void launch_f32(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.S, a.Hq, a.NP);
  attn_f32_kernel<D, B, SPLIT, false, OutT><<<grid, 64, 0, st>>>(
      static_cast<OutT*>(a.out), a.part_o, a.part_m, a.part_l, static_cast<const float*>(a.q),
      static_cast<const float*>(a.k_pool), static_cast<const float*>(a.v_pool), a.block_table,
      a.context_lens, nullptr, a.S, a.Hq, a.Hkv, a.MB, a.P, a.NP, a.scale * kLog2e);
}

template <int D, int B, bool SPLIT>
static void dispatch_out(const DecodeArgs& a, hipStream_t st) {
  if (a.bf16_in) {
    if (a.bf16_out) launch_bf16<D, B, SPLIT, uint16_t>(a, st);
    else launch_bf16<D, B, SPLIT, float>(a, st);
  } else {
    if (a.bf16_out) launch_f32<D, B, SPLIT, uint16_t>(a, st);
    else launch_f32<D, B, SPLIT, float>(a, st);
  }
}

template <int D, int B>
static void dispatch_split(const DecodeArgs& a, hipStream_t st) {
  if (a.NP > 1) dispatch_out<D, B, true>(a, st);
  else dispatch_out<D, B, false>(a, st);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  timing_begin(K_DECODE_PARTITION, st);
  if (a.D == 128) {
    if (a.B == 16) dispatch_split<128, 16>(a, st);
    else dispatch_split<128, 32>(a, st);
  } else {
    if (a.B == 16) dispatch_split<64, 16>(a, st);
    else dispatch_split<64, 32>(a, st);
  }
  hipError_t e = hipGetLastError();
  timing_end(K_DECODE_PARTITION, st);
  if (e != hipSuccess || a.NP <= 1) return e;
  timing_begin(K_DECODE_REDUCE, st);
  dim3 grid(a.Hq, a.S);
  if (a.bf16_out)
    decode_reduce_kernel<uint16_t><<<grid, 64, 0, st>>>(static_cast<uint16_t*>(a.out), a.part_o,
                                                        a.part_m, a.part_l, a.context_lens,
                                                        a.Hq, a.D, a.P, a.NP);
  else
    decode_reduce_kernel<float><<<grid, 64, 0, st>>>(static_cast<float*>(a.out), a.part_o,
                                                     a.part_m, a.part_l, a.context_lens, a.Hq,
                                                     a.D, a.P, a.NP);
  e = hipGetLastError();
  timing_end(K_DECODE_REDUCE, st);
  return e;
}

// fp32 prefill runs on the same vector kernel: chunk row i of a sequence is a decode row whose
// visible context ends at its own position (r + i + 1 keys).
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t st);

template <int D, int B, typename OutT>
static void launch_prefill_f32_t(const PrefillArgs& a, hipStream_t st) {
  dim3 grid(a.total_q, a.Hq, 1);
  attn_f32_kernel<D, B, false, true, OutT><<<grid, 64, 0, st>>>(
      static_cast<OutT*>(a.out), nullptr, nullptr, nullptr, static_cast<const float*>(a.q),
      static_cast<const float*>(a.k_pool), static_cast<const float*>(a.v_pool), a.block_table,
      a.context_lens, a.cu_q_lens, a.S, a.Hq, a.Hkv, a.MB, 1 << 30, 1, a.scale * kLog2e);
}

template <int D, int B>
static void prefill_f32_out(const PrefillArgs& a, hipStream_t st) {
  if (a.bf16_out) launch_prefill_f32_t<D, B, uint16_t>(a, st);
  else launch_prefill_f32_t<D, B, float>(a, st);
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t st) {
  if (a.D == 128) {
    if (a.B == 16) prefill_f32_out<128, 16>(a, st);
    else prefill_f32_out<128, 32>(a, st);
  } else {
    if (a.B == 16) prefill_f32_out<64, 16>(a, st);
    else prefill_f32_out<64, 32>(a, st);
  }
  return hipGetLastError();
}

}  // namespace pkv
