// paged_attention_prefill_chunk: a causal chunk of query tokens against the paged K/V.
//
// ("Serving Engines", How vLLM works: chunked prefill runs a prompt in slices interleaved with
// decode. "LLM Serving Engine Shootout" 3.1 equation for the scores, 5.1 for the fused steps.)
// Sequence s holds n tokens, the last c of which are this chunk (its K/V already written);
// chunk row i sits at position r + i, r = n - c, and attends to keys 0 .. r + i.
//
// bf16 path (matrix cores). A workgroup of four waves owns (sequence, group of query heads
// sharing one KV head, tile of chunk rows). Each wave owns 32 query rows of one head, so the
// heads of a KV group share every K/V tile the workgroup stages into LDS. Per 32-key tile:
//   S^T[32 keys][32 rows] = K_tile . Q^T      one 32x32x16 MFMA per 16 dims
//   online softmax per row (a lane owns a query row; the two lane halves hold 16 keys each)
//   O^T[D][32 rows]      += V_tile^T . P^T    two 32x32x16 MFMAs per 32 dims
// Keys are assigned to the MFMA rows of the first product so that the lane half hb ends up
// with keys 16*hb .. 16*hb+15, in order: then its P values are the B operand of the second
// product as they stand, and its V^T operand is 16 contiguous bytes of the dim-major V tile.
// K/V tiles are double-buffered in LDS: the next tile is read from HBM into registers while the
// current one is multiplied, then written to the other buffer. Tiles wholly above a wave's
// causal diagonal are skipped; only diagonal tiles apply the mask.
// Workgroups are numbered so that the row tiles of one (sequence, KV head) land on the same XCD
// (the GPU deals consecutive workgroups round-robin to its eight XCDs, each with its own L2) and
// the tiles with the most keys start first.
//
// fp32 prefill runs on the vector kernel in decode.hip.
#include "common.hpp"
#include "launch.hpp"

namespace pkv {

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t st);

constexpr float kLog2eP = 1.4426950408889634f;

__device__ __forceinline__ u32x4 lds16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

template <int D, int B, typename OutT>
__global__ __launch_bounds__(256) void prefill_bf16_kernel(
    OutT* __restrict__ out, const uint16_t* __restrict__ q, const int32_t* __restrict__ cu_q_lens,
    const int32_t* __restrict__ context_lens, const uint16_t* __restrict__ kpool,
    const uint16_t* __restrict__ vpool, const int32_t* __restrict__ block_table, int Hq, int Hkv,
    int G, int HW, int MB, int n_tiles, int n_groups, float scale_log2) {
  constexpr int KS = D + 8;    // LDS row pitch of the K tile (elements), padded
  constexpr int VS = 32 + 8;   // LDS row pitch of the V^T tile
  constexpr int KK = D / 16;   // QK MFMA steps
  constexpr int DT = D / 32;   // PV output tiles
  constexpr int CH = D / 64;   // 16-byte chunks per thread per tile (K and V each)
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][32 * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][D * VS];

  // XCD-aware numbering (see header comment).
  const int total = n_tiles * gridDim.y * gridDim.z;
  int bid = blockIdx.x + n_tiles * (blockIdx.y + gridDim.y * blockIdx.z);
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  const int tile = n_tiles - 1 - bid % n_tiles;
  const int gy = (bid / n_tiles) % gridDim.y;
  const int s = bid / (n_tiles * gridDim.y);

  const int g = gy / n_groups;
  const int grp = gy - g * n_groups;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;
  const int hb = lane >> 5;
  const int head = g * G + grp * HW + (wave % HW);
  const int WGT = 32 * (4 / HW);

  const int q0 = cu_q_lens[s];
  const int c = cu_q_lens[s + 1] - q0;
  const int n = context_lens[s];
  const int r = n - c;
  const int wg_tok0 = tile * WGT;
  if (wg_tok0 >= c) return;
  const int w_tok0 = wg_tok0 + (wave / HW) * 32;
  const bool wave_active = w_tok0 < c;
  const int my_i = w_tok0 + col;
  const bool row_valid = my_i < c;
  const int kend = r + min(wg_tok0 + WGT, c);  // keys [0, kend) are needed by this workgroup
  const int ntiles = (kend + 31) >> 5;
  const int nblk = (n + B - 1) / B;
  const int32_t* bt = block_table + static_cast<int64_t>(s) * MB;
  const int64_t blk_stride = static_cast<int64_t>(Hkv) * B * D;
  const uint16_t* kg = kpool + static_cast<int64_t>(g) * B * D;
  const uint16_t* vg = vpool + static_cast<int64_t>(g) * B * D;

  u32x4 qf[KK];
  {
    // rows past the chunk load nothing; their address is clamped into the chunk regardless
    const int qi = min(my_i, c - 1);
    const uint16_t* qrow = q + (static_cast<int64_t>(q0 + qi) * Hq + head) * D + 8 * hb;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = row_valid ? load16(qrow + 16 * kk) : u32x4{0u, 0u, 0u, 0u};
  }

  // Staging: thread tid copies CH 16-byte chunks of K ([32 keys][D]) and of V^T ([D][32 keys]).
  u32x4 kreg[CH], vreg[CH];
  auto stage_load = [&](int t) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int cid = tid + 256 * j;
      {  // K chunk: key cid / (D/8), dims 8*(cid % (D/8)) ..
        const int key = cid / (D / 8);
        const int dch = (cid % (D / 8)) * 8;
        const int ka = 32 * t + key;
        const int lb = min(ka / B, nblk - 1);
        const int64_t id = bt[lb];
        u32x4 v = load16(kg + id * blk_stride + (ka % B) * D + dch);
        if (ka >= n) v = u32x4{0u, 0u, 0u, 0u};
        kreg[j] = v;
      }
      {  // V chunk: dim cid / 4, keys 8*(cid % 4) .. +7
        const int d = cid >> 2;
        const int k8 = (cid & 3) * 8;
        const int ka = 32 * t + k8;
        const int lb = min(ka / B, nblk - 1);
        const int64_t id = bt[lb];
        u32x4 v = load16(vg + id * blk_stride + static_cast<int64_t>(d) * B + (ka % B));
        const int valid = n - ka;  // keys ka .. ka+7: keep the first `valid`
        if (valid < 8) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t keep =
                (2 * w < valid ? 0x0000ffffu : 0u) | (2 * w + 1 < valid ? 0xffff0000u : 0u);
            v[w] &= keep;
          }
        }
        vreg[j] = v;
      }
    }
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int cid = tid + 256 * j;
      const int key = cid / (D / 8);
      const int dch = (cid % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(&ks[buf][key * KS + dch]) = kreg[j];
      const int d = cid >> 2;
      const int k8 = (cid & 3) * 8;
      *reinterpret_cast<u32x4*>(&vs[buf][d * VS + k8]) = vreg[j];
    }
  };

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  float m = -INFINITY;
  float l = 0.f;
  const int qpos = r + my_i;          // this lane's query position
  const int wq_lo = r + w_tok0;       // the wave's first query position
  // MFMA row of the K operand -> key within the tile: lane half hb gets keys 16*hb + i.
  const int krow = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);

  auto compute = [&](int buf, int t) {
    const int key0 = 32 * t;
    if (!wave_active || key0 > wq_lo + 31) return;  // wholly above the diagonal
    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
    const uint16_t* kt = &ks[buf][krow * KS + 8 * hb];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) sacc = mfma32x32x16(lds16(kt + 16 * kk), qf[kk], sacc);
    float x[16];
    const bool diag = key0 + 31 > wq_lo;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float v = sacc[i] * scale_log2;
      x[i] = (diag && key0 + 16 * hb + i > qpos) ? -INFINITY : v;
    }
    float rmax = x[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) rmax = fmaxf(rmax, x[i]);
    rmax = xor32_max(rmax);
    const float mnew = fmaxf(m, rmax);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    float psum = 0.f;
    u32x4 pb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = fast_exp2(x[8 * j + 2 * w] - mnew);
        const float p1 = fast_exp2(x[8 * j + 2 * w + 1] - mnew);
        psum += p0 + p1;
        pb[j][w] = pack_bf16x2(p0, p1);
      }
    l = l * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint16_t* vt = &vs[buf][(32 * dt + col) * VS + 16 * hb];
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[dt] = mfma32x32x16(lds16(vt + 8 * j), pb[j], acc[dt]);
    }
  };

  stage_load(0);
  stage_store(0);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const bool more = t + 1 < ntiles;
    if (more) stage_load(t + 1);
    compute(t & 1, t);
    if (more) stage_store((t + 1) & 1);
    __syncthreads();
  }

  if (!wave_active) return;
  l = xor32_sum(l);
  if (!row_valid) return;
  const float inv = 1.0f / l;
  OutT* o = out + (static_cast<int64_t>(q0 + my_i) * Hq + head) * D + 4 * hb;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      store_out(o + 32 * dt + 8 * (i >> 2) + (i & 3), acc[dt][i] * inv);
}

template <int D, int B, typename OutT>
static void launch_t(const PrefillArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const int HW = (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1);
  const int WGT = 32 * (4 / HW);
  const int n_tiles = (a.max_q_len + WGT - 1) / WGT;
  const int n_groups = G / HW;
  dim3 grid(n_tiles, a.Hkv * n_groups, a.S);
  launch_kernel(K_PREFILL, prefill_bf16_kernel<D, B, OutT>, dim3(grid), dim3(256), st,
      static_cast<OutT*>(a.out), static_cast<const uint16_t*>(a.q), a.cu_q_lens, a.context_lens,
      static_cast<const uint16_t*>(a.k_pool), static_cast<const uint16_t*>(a.v_pool), a.block_table,
      a.Hq, a.Hkv, G, HW, a.MB, n_tiles, n_groups, a.scale * kLog2eP);
}

template <int D, int B>
static void launch_out(const PrefillArgs& a, hipStream_t st) {
  if (a.bf16_out) launch_t<D, B, uint16_t>(a, st);
  else launch_t<D, B, float>(a, st);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.total_q == 0 || a.max_q_len == 0) return hipSuccess;
  hipError_t e;
  if (!a.bf16_in) {
    e = launch_prefill_f32(a, st);
  } else {
    if (a.D == 128) {
      if (a.B == 16) launch_out<128, 16>(a, st);
      else launch_out<128, 32>(a, st);
    } else {
      if (a.B == 16) launch_out<64, 16>(a, st);
      else launch_out<64, 32>(a, st);
    }
    e = hipGetLastError();
  }
  return e;
}

}  // namespace pkv
