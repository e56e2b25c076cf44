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
// dim-major V tile. Heads beyond G in the 16-wide column are zero queries: their lanes skip the
// softmax and feed P = 0, and their results are dropped; the kernel is bound by HBM reads of K
// and V, so the padded MFMA work costs no time.
// K and V of the next tile are loaded while the current tile is computed (two register sets).
//
// E4M3 pools (same waves, same tiles): every E4M3 value is exactly a bf16 value, so each lane
// widens the bytes it loaded with v_cvt_scalef32_pk_bf16_fp8 (scale 1) and feeds the same bf16
// matrix products. A tile's K is 4 KB instead of 8, so the contraction slots are assigned
// differently: lane group lg holds the D/4 consecutive dimensions lg*D/4 .. (lg+1)*D/4-1 of its
// token row (one 16-byte load per 16 dimensions), and the query operand uses the same
// assignment. The pool scales are folded in: k_scale into the score scale, v_scale into the
// final normalisation. The tile loop keeps three register sets (two tiles in flight).
//
// Also here: the prefix-aware decode for batches that share prompt prefixes (see PrefixInfo),
// the write folded into the decode (see StepInfo), and the reduce kernel.
//
// fp32 path (vector ALUs): one wave owns (sequence, query head, partition); lanes take one token
// each for the scores, then one output dimension each for P.V.
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "lds_tile.hpp"

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;

template <int D, int B>
struct KvTile {
  u32x4 k[2][D / 32];
  u32x4 v[D / 16];
};

// Running online-softmax state of one wave: 16 head columns, D output dims per column.
template <int D>
struct WaveAttn {
  f32x4 acc[D / 16];
  float m;
  float l;  // per lane: sum over the lane's own tokens; reduce over rows before use
};

template <int D>
__device__ __forceinline__ void attn_init(WaveAttn<D>& st) {
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) st.acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
}

// Q as the MFMA B operand: column = head, contraction slots d = 32*kk + 8*lg + e.
template <int D>
__device__ __forceinline__ void load_q(u32x4 (&qf)[D / 32], const uint16_t* qrow, bool hvalid,
                                       int lg) {
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    qf[kk] = hvalid ? load16(qrow + 32 * kk + 8 * lg) : u32x4{0u, 0u, 0u, 0u};
}

// The online-softmax update of one tile for a lane's 8 scores x (log2 units, masked ones -inf)
// whose column maximum is tmax; leaves the bf16 weights of the P.V product in pb.
// Lazy rescaling: the running maximum m moves only when a column's scores exceed it by more
// than 2^8 (then acc and l are rescaled, a wave-uniform branch); otherwise the weights are taken
// against the stale m and are at most 2^8. That is exact: l and acc always refer to the same m,
// and the output (acc / l) and the partials (m, l, acc / l) only ever combine them consistently.
template <int D>
__device__ __forceinline__ void softmax_step(WaveAttn<D>& st, const float (&x)[8], float tmax,
                                             u32x4& pb) {
  const bool grow = tmax > st.m + 8.0f;
  if (__builtin_amdgcn_ballot_w64(grow)) {
    const float mnew = grow ? tmax : st.m;
    const float alpha = fast_exp2(st.m - mnew);
    st.m = mnew;
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) st.acc[dt] *= alpha;
  }
  float psum = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float p0 = fast_exp2(x[2 * w] - st.m);
    const float p1 = fast_exp2(x[2 * w + 1] - st.m);
    psum += p0 + p1;
    pb[w] = pack_bf16x2(p0, p1);
  }
  st.l += psum;
}

// One 32-token tile's step of the online softmax, bf16 operands already in registers: scores
// by MFMA, running max / sum / rescale, then P.V by MFMA. Tile tokens at or past lim get no
// weight; V words of tokens at or past vlim are cleared first (stale slots may hold NaN, and
// 0 * NaN is NaN).
template <int D>
__device__ __forceinline__ void tile_update(WaveAttn<D>& st, const u32x4 (&k)[2][D / 32],
                                            u32x4 (&v)[D / 16], const u32x4 (&qf)[D / 32],
                                            int lim, int vlim, float scale_log2, int lg,
                                            bool col_used = true) {
  constexpr int KK = D / 32;
  constexpr int DT = D / 16;
  f32x4 sc[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    sc[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) sc[hf] = mfma16x16x32(k[hf][kk], qf[kk], sc[hf]);
  }
  // lane: head column r16, tile tokens 8*lg + 4*hf + e. Padding columns (no query head) skip
  // the softmax and give P = 0; all four lanes of a column agree on col_used.
  u32x4 pb = {0u, 0u, 0u, 0u};
  if (col_used) {
    float x[8];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * hf + e] = sc[hf][e] * scale_log2;
    if (lim < 32) {  // wave-uniform: only a context's last tile has tokens to mask
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (8 * lg + 4 * (i >> 2) + (i & 3) >= lim) x[i] = -INFINITY;
    }
    float tmax = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, x[i]);
    tmax = xor32_max(xor16_max(tmax));
    softmax_step(st, x, tmax, pb);
  }
  if (vlim < 32) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int t0 = 8 * lg + 2 * w;
      const uint32_t keep = (t0 < vlim ? 0x0000ffffu : 0u) | (t0 + 1 < vlim ? 0xffff0000u : 0u);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) v[dt][w] &= keep;
    }
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) st.acc[dt] = mfma16x16x32(v[dt], pb, st.acc[dt]);
}

// A one-token tile from rows outside the pool (the token being added this step): the token
// takes tile row 0, i.e. K row 0 (held by the lanes of column 0) and V token 0 (element 0 of
// the lanes of row group 0); everything else is zero and masked.
template <int D>
__device__ __forceinline__ void attend_one_token(WaveAttn<D>& st, const u32x4 (&qf)[D / 32],
                                                 const uint16_t* __restrict__ krow,
                                                 const uint16_t* __restrict__ vrow,
                                                 float scale_log2) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int lg = lane >> 4;
  u32x4 k[2][D / 32];
  u32x4 v[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    k[0][kk] = (r16 == 0) ? load16(krow + 32 * kk + 8 * lg) : u32x4{0u, 0u, 0u, 0u};
    k[1][kk] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    v[dt] = u32x4{(lg == 0) ? static_cast<uint32_t>(vrow[16 * dt + r16]) : 0u, 0u, 0u, 0u};
  tile_update<D>(st, k, v, qf, 1, 1, scale_log2, lg);
}

// Walk over the 32-token tiles of one (sequence, KV head) of bf16 pools, starting at token
// tok_begin (a multiple of B): per-lane operand addresses and the block ids of the chunk being
// walked. Block ids come one chunk of up to 64 logical blocks at a time: lane i holds the id of
// block chunk_lb + i (clamped to the last block that holds tokens); tiles read them with
// readlane, so block addresses stay wave-uniform and the tile loop issues no other vector load.
template <int D, int B>
struct TileWalk {
  static constexpr int KK = D / 32;
  static constexpr int DT = D / 16;
  static constexpr int TILE = B * D;  // elements of one (block, head) tile
  static constexpr int kChunkTiles = 64 * B / 32;  // tiles whose block ids fit one VGPR
  const uint16_t* kpool;
  const uint16_t* vpool;
  int tok_begin;
  int nblk;
  int koff[2];
  int ksel;
  int vsel;
  int voff;
  int64_t head_off;
  uint32_t blk_stride;  // elements of one block of a pool (Hkv * B * D < 2^32)
  int chunk_lb = 0;
  int my_id = 0;

  __device__ __forceinline__ TileWalk(const uint16_t* kp, const uint16_t* vp, int n, int g,
                                      int Hkv, int tb)
      : kpool(kp), vpool(vp), tok_begin(tb), nblk((n + B - 1) / B) {
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15;
    const int lg = lane >> 4;
    // K operand row r16 of half hf holds tile token 8*(r16/4) + 4*hf + r16%4.
    ksel = 0;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int tau = 8 * (r16 >> 2) + 4 * hf + (r16 & 3);
      koff[hf] = (tau % B) * D + 8 * lg;
      ksel = tau / B;  // same block for both halves
    }
    // V^T operand: row d = 16*dt + r16, tokens 8*lg .. 8*lg+7 of the tile.
    vsel = (B == 16) ? (lg >> 1) : 0;
    const int vtok = (B == 16) ? 8 * (lg & 1) : 8 * lg;
    voff = r16 * B + vtok;
    head_off = static_cast<int64_t>(g) * TILE;
    blk_stride = static_cast<uint32_t>(Hkv) * TILE;
  }
  // Load the block ids of the chunk that starts at tile c0.
  __device__ __forceinline__ void begin_chunk(const int32_t* __restrict__ bt, int c0) {
    chunk_lb = (tok_begin + 32 * c0) / B;
    my_id = bt[min(chunk_lb + static_cast<int>(threadIdx.x & 63), nblk - 1)];
  }
  __device__ __forceinline__ int block_id(int lb) const {
    return __builtin_amdgcn_readlane(my_id, min(lb, nblk - 1) - chunk_lb);
  }
  // STREAM: non-temporal loads (tiles read once); without it the lines stay cached for the
  // units that read the same tile again (shared prefixes).
  template <bool STREAM = true>
  __device__ __forceinline__ void load(KvTile<D, B>& T, int t) const {
    const int lb0 = (tok_begin + 32 * t) / B;
    // both candidate block offsets are wave-uniform (block ids are non-negative); a lane
    // selects the one its rows lie in
    const uint64_t o0 = static_cast<uint64_t>(static_cast<uint32_t>(block_id(lb0))) * blk_stride;
    const uint64_t o1 =
        (B == 16) ? static_cast<uint64_t>(static_cast<uint32_t>(block_id(lb0 + 1))) * blk_stride
                  : o0;
    const uint16_t* kb = kpool + (ksel ? o1 : o0) + head_off;
    const uint16_t* vb = vpool + (vsel ? o1 : o0) + head_off;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        T.k[hf][kk] = STREAM ? load16_stream(kb + koff[hf] + 32 * kk)
                             : load16(kb + koff[hf] + 32 * kk);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      T.v[dt] = STREAM ? load16_stream(vb + voff + 16 * dt * B) : load16(vb + voff + 16 * dt * B);
  }
};

// Attend the wave's 16 head columns (KV head g) to tokens [tok_begin, tok_end) of one
// sequence with n tokens, walking 32-token tiles from tok_begin (a multiple of B).
// STREAM: the tiles' loads are non-temporal (see TileWalk::load).
template <int D, int B, bool STREAM = true>
__device__ __forceinline__ void attend_tiles(WaveAttn<D>& st, const u32x4 (&qf)[D / 32],
                                             const uint16_t* __restrict__ kpool,
                                             const uint16_t* __restrict__ vpool,
                                             const int32_t* __restrict__ bt, int n, int g,
                                             int Hkv, int tok_begin, int tok_end,
                                             float scale_log2, bool col_used = true) {
  const int lg = (threadIdx.x & 63) >> 4;
  const int ntiles = (tok_end - tok_begin + 31) >> 5;
  TileWalk<D, B> wk(kpool, vpool, n, g, Hkv, tok_begin);
  auto compute = [&](KvTile<D, B>& T, int t) {
    const int tok0 = tok_begin + 32 * t;
    tile_update<D>(st, T.k, T.v, qf, tok_end - tok0, n - tok0, scale_log2, lg, col_used);
  };

  // Software pipeline: every compute of tile t runs while the loads of tile t+1 are in
  // flight. Inside a chunk the loop body always issues exactly one tile of loads before each
  // compute, so the wait before a compute leaves the next tile's loads outstanding.
  KvTile<D, B> ta, tb;
  for (int c0 = 0; c0 < ntiles; c0 += TileWalk<D, B>::kChunkTiles) {
    const int c1 = min(ntiles, c0 + TileWalk<D, B>::kChunkTiles);
    wk.begin_chunk(bt, c0);
    wk.template load<STREAM>(ta, c0);
    int t = c0;
    for (; t + 2 < c1; t += 2) {
      wk.template load<STREAM>(tb, t + 1);
      compute(ta, t);
      wk.template load<STREAM>(ta, t + 2);
      compute(tb, t + 1);
    }
    if (t + 1 < c1) {
      wk.template load<STREAM>(tb, t + 1);
      compute(ta, t);
      compute(tb, t + 1);
    } else {
      compute(ta, t);
    }
  }
}

// Read probe (measurement only): the tiles attend_tiles would read for the same arguments,
// loaded by the same lanes through the same two-register-set pipeline, with the attention
// arithmetic replaced by an XOR of the loaded words (so no load can be dropped). Its time
// against the decode's separates the cost of reading the tile list from the cost of the math.
template <int D, int B, bool STREAM = true>
__device__ __forceinline__ uint32_t probe_tiles(const uint16_t* __restrict__ kpool,
                                                const uint16_t* __restrict__ vpool,
                                                const int32_t* __restrict__ bt, int n, int g,
                                                int Hkv, int tok_begin, int tok_end) {
  const int ntiles = (tok_end - tok_begin + 31) >> 5;
  TileWalk<D, B> wk(kpool, vpool, n, g, Hkv, tok_begin);
  uint32_t acc = 0;
  auto fold = [&](const KvTile<D, B>& T) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) acc ^= T.k[hf][kk][0] ^ T.k[hf][kk][1] ^
                                                 T.k[hf][kk][2] ^ T.k[hf][kk][3];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc ^= T.v[dt][0] ^ T.v[dt][1] ^ T.v[dt][2] ^ T.v[dt][3];
  };
  KvTile<D, B> ta, tb;
  for (int c0 = 0; c0 < ntiles; c0 += TileWalk<D, B>::kChunkTiles) {
    const int c1 = min(ntiles, c0 + TileWalk<D, B>::kChunkTiles);
    wk.begin_chunk(bt, c0);
    wk.template load<STREAM>(ta, c0);
    int t = c0;
    for (; t + 2 < c1; t += 2) {
      wk.template load<STREAM>(tb, t + 1);
      fold(ta);
      wk.template load<STREAM>(ta, t + 2);
      fold(tb);
    }
    if (t + 1 < c1) {
      wk.template load<STREAM>(tb, t + 1);
      fold(ta);
      fold(tb);
    } else {
      fold(ta);
    }
  }
  return acc;
}

// ----------------------------------------------------------------------------- E4M3 pools

template <int D, int B>
struct KvTile8 {
  u32x4 k[2][D / 64];  // per half: the lane's D/4 bytes of one token row
  u32x2 v[D / 16];     // per 16 dims: 8 tokens of one dimension row
};

// Q as the MFMA B operand for E4M3 K: contraction slot (kk, 8*lg + e) is dimension
// lg*D/4 + 8*kk + e.
template <int D>
__device__ __forceinline__ void load_q_fp8(u32x4 (&qf)[D / 32], const uint16_t* qrow,
                                           bool hvalid, int lg) {
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    qf[kk] = hvalid ? load16(qrow + (D / 4) * lg + 8 * kk) : u32x4{0u, 0u, 0u, 0u};
}

// Eight E4M3 codes (bytes 0..7 of w0, w1) as eight bf16 values, byte i -> element i. Exact.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return r;
}

__device__ __forceinline__ u32x2 load8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

// attend_tiles for E4M3 pools: the same tiles, token-to-row assignment, softmax and pipeline;
// only the loads (bytes) and the widening before each product differ.
// DEPTH: register sets in the tile pipeline (3, or 2 where registers are tighter).
// STREAM: non-temporal loads (see TileWalk::load).
template <int D, int B, int DEPTH = 3, bool STREAM = true>
__device__ __forceinline__ void attend_tiles_fp8(WaveAttn<D>& st, const u32x4 (&qf)[D / 32],
                                                 const uint8_t* __restrict__ kpool,
                                                 const uint8_t* __restrict__ vpool,
                                                 const int32_t* __restrict__ bt, int n, int g,
                                                 int Hkv, int tok_begin, int tok_end,
                                                 float scale_log2) {
  constexpr int KK = D / 32;
  constexpr int KL = D / 64;
  constexpr int DT = D / 16;
  constexpr int TILE = B * D;  // bytes of one (block, head) tile
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int lg = lane >> 4;
  const int ntiles = (tok_end - tok_begin + 31) >> 5;
  const int nblk = (n + B - 1) / B;

  int koff[2];
  int ksel = 0;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int tau = 8 * (r16 >> 2) + 4 * hf + (r16 & 3);
    koff[hf] = (tau % B) * D + (D / 4) * lg;
    ksel = tau / B;
  }
  const int vsel = (B == 16) ? (lg >> 1) : 0;
  const int vtok = (B == 16) ? 8 * (lg & 1) : 8 * lg;
  const int voff = r16 * B + vtok;
  const int64_t head_off = static_cast<int64_t>(g) * TILE;
  const uint32_t blk_stride = static_cast<uint32_t>(Hkv) * TILE;  // < 2^32

  int chunk_lb = 0;
  int my_id = 0;
  auto block_id = [&](int lb) -> int {
    return __builtin_amdgcn_readlane(my_id, min(lb, nblk - 1) - chunk_lb);
  };
  auto load_tile = [&](KvTile8<D, B>& T, int t) {
    const int lb0 = (tok_begin + 32 * t) / B;
    const uint64_t o0 = static_cast<uint64_t>(static_cast<uint32_t>(block_id(lb0))) * blk_stride;
    const uint64_t o1 =
        (B == 16) ? static_cast<uint64_t>(static_cast<uint32_t>(block_id(lb0 + 1))) * blk_stride
                  : o0;
    const uint8_t* kb = kpool + (ksel ? o1 : o0) + head_off;
    const uint8_t* vb = vpool + (vsel ? o1 : o0) + head_off;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int j = 0; j < KL; ++j)
        T.k[hf][j] = STREAM ? load16_stream(kb + koff[hf] + 16 * j)
                            : load16(kb + koff[hf] + 16 * j);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      T.v[dt] = STREAM ? load8_stream(vb + voff + 16 * dt * B) : load8(vb + voff + 16 * dt * B);
  };

  auto compute = [&](KvTile8<D, B>& T, int t) {
    const int tok0 = tok_begin + 32 * t;
    f32x4 sc[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      sc[hf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4 w = T.k[hf][kk >> 1];
        const u32x4 a = (kk & 1) ? e4m3x8_to_bf16x8(w[2], w[3]) : e4m3x8_to_bf16x8(w[0], w[1]);
        sc[hf] = mfma16x16x32(a, qf[kk], sc[hf]);
      }
    }
    const int lim = tok_end - tok0;
    float x[8];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * hf + e] = sc[hf][e] * scale_log2;
    if (lim < 32) {  // wave-uniform: only a context's last tile has tokens to mask
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (8 * lg + 4 * (i >> 2) + (i & 3) >= lim) x[i] = -INFINITY;
    }
    float tmax = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, x[i]);
    tmax = xor32_max(xor16_max(tmax));
    u32x4 pb;
    softmax_step(st, x, tmax, pb);
    u32x4 vv[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vv[dt] = e4m3x8_to_bf16x8(T.v[dt][0], T.v[dt][1]);
    // Slots at or past n may hold any code, NaN included: clear those V values (0 * NaN).
    const int vlim = n - tok0;
    if (vlim < 32) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int t0 = 8 * lg + 2 * w;
        const uint32_t keep =
            (t0 < vlim ? 0x0000ffffu : 0u) | (t0 + 1 < vlim ? 0xffff0000u : 0u);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vv[dt][w] &= keep;
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.acc[dt] = mfma16x16x32(vv[dt], pb, st.acc[dt]);
  };

  // DEPTH register sets. With three (the plain decode), two tiles' loads stay in flight during
  // each compute (an E4M3 tile is half the bytes of a bf16 one, so the bf16 loop's two-deep
  // pipeline would keep half the bytes in flight); the prefix-aware kernel, held to 256 VGPRs
  // by its eight-wave workgroups, uses two.
  constexpr int kChunkTiles = 64 * B / 32;
  if constexpr (DEPTH == 2) {
    KvTile8<D, B> ta, tb;
    for (int c0 = 0; c0 < ntiles; c0 += kChunkTiles) {
      const int c1 = min(ntiles, c0 + kChunkTiles);
      chunk_lb = (tok_begin + 32 * c0) / B;
      my_id = bt[min(chunk_lb + lane, nblk - 1)];
      load_tile(ta, c0);
      int t = c0;
      for (; t + 2 < c1; t += 2) {
        load_tile(tb, t + 1);
        compute(ta, t);
        load_tile(ta, t + 2);
        compute(tb, t + 1);
      }
      if (t + 1 < c1) {
        load_tile(tb, t + 1);
        compute(ta, t);
        compute(tb, t + 1);
      } else {
        compute(ta, t);
      }
    }
    return;
  }
  KvTile8<D, B> t0, t1, t2;
  for (int c0 = 0; c0 < ntiles; c0 += kChunkTiles) {
    const int c1 = min(ntiles, c0 + kChunkTiles);
    chunk_lb = (tok_begin + 32 * c0) / B;
    my_id = bt[min(chunk_lb + lane, nblk - 1)];
    load_tile(t0, c0);
    if (c0 + 1 < c1) load_tile(t1, c0 + 1);
    int t = c0;
    for (; t + 4 < c1; t += 3) {  // on entry t0 and t1 hold tiles t and t+1
      load_tile(t2, t + 2);
      compute(t0, t);
      load_tile(t0, t + 3);
      compute(t1, t + 1);
      load_tile(t1, t + 4);
      compute(t2, t + 2);
    }
    const int rem = c1 - t;  // 1 .. 4 tiles left
    if (rem >= 3) load_tile(t2, t + 2);
    compute(t0, t);
    if (rem == 4) load_tile(t0, t + 3);
    if (rem >= 2) compute(t1, t + 1);
    if (rem >= 3) compute(t2, t + 2);
    if (rem == 4) compute(t0, t + 3);
  }
}

// Final output of a wave whose state covers a head's whole context: out = acc / l.
// out_scale multiplies the result (the V pool's scale for E4M3 pools, else 1).
template <int D, typename OutT>
__device__ __forceinline__ void write_final(OutT* __restrict__ o, const WaveAttn<D>& st,
                                            float l_total, int lg, float out_scale = 1.0f) {
  const float inv = out_scale / l_total;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out(o + 16 * dt + 4 * lg + e, st.acc[dt][e] * inv);
}

// Partial result of part of a context: (m, l, acc / l) in fp32.
template <int D>
__device__ __forceinline__ void write_partial(float* __restrict__ part_o,
                                              float* __restrict__ part_m,
                                              float* __restrict__ part_l, int64_t idx,
                                              const WaveAttn<D>& st, float l_total, int lg,
                                              float out_scale = 1.0f) {
  const float inv = out_scale / l_total;
  if (lg == 0) {
    part_m[idx] = st.m;
    part_l[idx] = l_total;
  }
  float* o = part_o + idx * D;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    *reinterpret_cast<f32x4*>(o + 16 * dt + 4 * lg) = st.acc[dt] * inv;
}

template <int D, typename OutT>
__device__ __forceinline__ void write_zero(OutT* __restrict__ o, int lg) {
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out(o + 16 * dt + 4 * lg + e, 0.0f);
}

// Cache policy of a segment's tile loads. Tiles read once per call are streamed (non-temporal
// loads). A block that several sequences' tables name (a shared prompt prefix, as prefix caching
// and copy-on-write forks produce) is read again by those sequences' waves and should stay
// cached instead. Sharing is detected cheaply, per sequence: its first block also starts the
// table of the previous or the next sequence of the batch (the entry is read even when that
// neighbour's context is empty: it lies inside the table, and the outcome only picks a policy).
// Only the load hints depend on it, never the result.
__device__ __forceinline__ bool shares_first_block(const int32_t* __restrict__ block_table,
                                                   int s, int S, int MB) {
  const int64_t row = static_cast<int64_t>(s) * MB;
  const int first = block_table[row];
  const int prev = s > 0 ? block_table[row - MB] : -1;
  const int next = s + 1 < S ? block_table[row + MB] : -1;
  return first == prev || first == next;
}

// Fixed partitions of P tokens: grid (KV head x head group, sequence, partition). The
// partition index is the slowest, so the dispatcher hands out every sequence's first (full)
// partitions before the shorter last ones, and the launch ends on small work units.
template <int D, int B, bool SPLIT, typename OutT>
__global__ __launch_bounds__(64) void decode_fixed_kernel(
    OutT* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_m,
    float* __restrict__ part_l, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ kpool, const uint16_t* __restrict__ vpool,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ context_lens, int Hq,
    int Hkv, int G, int HG, int MB, int P, int NP, float scale_log2) {
  const int lane = threadIdx.x;
  const int lg = lane >> 4;
  const int g = blockIdx.x / HG;
  const int hgrp = blockIdx.x - g * HG;
  const int s = blockIdx.y;
  const int p = blockIdx.z;
  const int n = context_lens[s];
  const int start = p * P;
  const int hl = hgrp * 16 + (lane & 15);
  const bool hvalid = hl < G;
  const int h = g * G + (hvalid ? hl : 0);
  const int64_t row = static_cast<int64_t>(s) * Hq + h;

  if (start >= n) {
    if (!SPLIT && p == 0 && hvalid) write_zero<D>(out + row * D, lg);  // empty context
    return;
  }
  u32x4 qf[D / 32];
  load_q<D>(qf, q + row * D, hvalid, lg);
  WaveAttn<D> st;
  attn_init(st);
  const int32_t* bt = block_table + static_cast<int64_t>(s) * MB;
  if (!shares_first_block(block_table, s, gridDim.y, MB))
    attend_tiles<D, B, true>(st, qf, kpool, vpool, bt, n, g, Hkv, start, min(start + P, n),
                             scale_log2);
  else
    attend_tiles<D, B, false>(st, qf, kpool, vpool, bt, n, g, Hkv, start, min(start + P, n),
                              scale_log2);
  const float l_total = xor32_sum(xor16_sum(st.l));
  if (!hvalid) return;
  if constexpr (!SPLIT) write_final<D>(out + row * D, st, l_total, lg);
  else write_partial<D>(part_o, part_m, part_l, row * NP + p, st, l_total, lg);
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int mk = 32; mk >= 1; mk >>= 1) v += __shfl_xor(v, mk);
  return v;
}

__device__ __forceinline__ int wave_incl_scan_i(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  return v;
}

// Shared prefixes (the prefix-aware decode): sequences come in groups of consecutive ones,
// group i being sequences group_start[i] .. group_start[i+1]-1, whose first group_prefix_len[i]
// tokens (a multiple of B) are the same physical blocks. Such a prefix is attended once per
// group, in units of (group, KV head, chunk of kPrefixChunk prefix tokens, block of
// kPrefixWgColumns query columns), the columns being (member sequence, query head) pairs: a
// chunk's K/V is then read once for every member's query heads instead of once per sequence.
// A unit is a workgroup of kPrefixWgWaves waves (prefix_wg). The private rest of each context
// goes through the balanced split as usual. A row's partials: the prefix chunks at slots
// 0 .. pc-1 (pc = ceil(prefix / kPrefixChunk)), then its suffix pieces.
constexpr int kPrefixChunk = kPrefixChunkTokens;

struct PrefixInfo {
  const int32_t* group_start;       // [NG+1]
  const int32_t* group_prefix_len;  // [NG]
  int NG;
};

// Prefix length of sequence s (binary search over the group starts).
__device__ __forceinline__ int seq_prefix_len(const PrefixInfo& pf, int s) {
  int lo = 0, hi = pf.NG;  // group_start[lo] <= s < group_start[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pf.group_start[mid] <= s) lo = mid; else hi = mid;
  }
  return pf.group_prefix_len[lo];
}

// Fused decode step (kv_cache_write_and_decode): sequence s's newest token, at position n-1,
// comes from k_new / v_new (slot_mapping[s] >= 0) instead of the pool; the wave whose piece ends
// at n attends to it as a one-token tile and stores it into the pool slot. Nothing reads that
// slot in the same launch, so the store needs no ordering. (Merging the split rows inside this
// kernel as well, by the last wave to finish each row, was measured slower: publishing a
// partial across XCDs needs a device-scope release, which writes back the XCD's whole L2.)
struct StepInfo {
  const uint16_t* k_new;   // [S][Hkv][D]
  const uint16_t* v_new;
  const int32_t* slots;    // [S]
  uint16_t* kpool;         // the pools, written at the new tokens' slots
  uint16_t* vpool;
};

// Balanced split: the batch is a list of 32-token tiles ordered by (sequence, KV head x head
// group, tile); wave w of W takes tiles [w*T/W, (w+1)*T/W). A (sequence, KV head) segment that
// one wave covers whole is written as output directly; a segment shared by several waves gets
// one partial per wave, merged by the reduce kernel. Every wave does the same number of tiles
// (to within one), whatever the mix of context lengths. Wave 0 also records, per segment, how
// many partials its rows have. W is lowered on the device so that each wave gets at least
// min_tiles tiles, which bounds the partials per segment by ceil(ceil(max_ctx/32) / min_tiles) + 1.
// With PREFIX, a sequence's tiles start after its group's prefix, partial slots after the prefix
// chunks' (KSTRIDE slots per row in all), and a segment with prefix chunks is never final.
// With STEP (bf16 only), the new tokens are handled as described at StepInfo.
template <int D, int B, typename OutT, typename KvT, bool PREFIX, bool STEP = false,
          bool PROBE = false>
__device__ __forceinline__ void balanced_body(
    int w, int W, OutT* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_m,
    float* __restrict__ part_l, int32_t* __restrict__ seg_count, const uint16_t* __restrict__ q,
    const KvT* __restrict__ kpool, const KvT* __restrict__ vpool,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ context_lens, int S,
    int Hq, int Hkv, int G, int HG, int MB, int KSTRIDE, int min_tiles, float scale_log2,
    float out_scale, PrefixInfo pf, StepInfo sp = StepInfo{}, uint32_t* probe_sink = nullptr) {
  constexpr bool kFp8 = sizeof(KvT) == 1;
  static_assert(!STEP || (!PREFIX && !kFp8), "the fused step is built for plain bf16 decode");
  static_assert(!PROBE || (!PREFIX && !STEP && !kFp8), "the read probe walks plain bf16 decode");
  const int lane = threadIdx.x & 63;
  const int lg = lane >> 4;
  const int segs = Hkv * HG;
  // tiles of one segment of sequence s, and where they start
  auto prefix_of = [&](int s) -> int { return PREFIX ? seq_prefix_len(pf, s) : 0; };
  auto seq_tiles = [&](int s) -> int {
    return (s < S) ? (context_lens[s] - prefix_of(s) + 31) >> 5 : 0;
  };

  int64_t T = 0;  // tiles of the whole batch
  for (int base = 0; base < S; base += 64) T += wave_sum_i(seq_tiles(base + lane));
  T *= segs;
  const int64_t Weff = max<int64_t>(1, min<int64_t>(W, T / max(1, min_tiles)));
  // wave that owns tile x: the largest w with floor(w*T/Weff) <= x
  auto wave_of = [&](int64_t x) -> int64_t { return (x * Weff + Weff - 1) / T; };

  if (!PROBE && w == 0) {  // partial counts per segment, for the reduce
    int64_t cum = 0;
    for (int base = 0; base < S; base += 64) {
      const int s = base + lane;
      const int ts = seq_tiles(s);
      const int incl = wave_incl_scan_i(ts);
      if (s < S) {
        const int pc = PREFIX ? (prefix_of(s) + kPrefixChunk - 1) / kPrefixChunk : 0;
        const int64_t seq0 = (cum + incl - ts) * segs;
        for (int j = 0; j < segs; ++j) {
          int cnt = 0;
          if (ts > 0) {
            const int64_t a = seq0 + static_cast<int64_t>(j) * ts;
            cnt = static_cast<int>(wave_of(a + ts - 1) - wave_of(a) + 1);
          }
          seg_count[static_cast<int64_t>(s) * segs + j] = cnt + pc;
        }
      }
      cum += __shfl(incl, 63);
    }
  }
  if (w >= Weff || T == 0) return;
  const int64_t x0 = (static_cast<int64_t>(w) * T) / Weff;
  const int64_t x1 = (static_cast<int64_t>(w + 1) * T) / Weff;
  if (x0 >= x1) return;

  // Locate the sequence holding tile x0.
  int s = -1;
  int64_t sstart = 0;  // first tile of sequence s
  {
    int64_t cum = 0;
    for (int base = 0; base < S && s < 0; base += 64) {
      const int sl = base + lane;
      const int ts = seq_tiles(sl);
      const int incl = wave_incl_scan_i(ts);
      const int64_t end_l = (cum + incl) * segs;
      const uint64_t hit = __ballot(sl < S && end_l > x0);
      if (hit) {
        const int first = __ffsll(static_cast<unsigned long long>(hit)) - 1;
        s = base + first;
        sstart = (cum + __shfl(incl - ts, first)) * segs;
      }
      cum += __shfl(incl, 63);
    }
  }
  if (s < 0) return;
  int n = context_lens[s];
  int pre = prefix_of(s);
  int ts = (n - pre + 31) >> 5;
  int j = static_cast<int>((x0 - sstart) / ts);
  int64_t x = x0;
  uint32_t probe_acc = 0;
  while (x < x1) {
    const int64_t a = sstart + static_cast<int64_t>(j) * ts;  // first tile of segment (s, j)
    const int t_begin = static_cast<int>(x - a);
    const int t_end = static_cast<int>(min<int64_t>(ts, x1 - a));
    const int g = j / HG;
    const int hgrp = j - g * HG;
    const int hl = hgrp * 16 + (lane & 15);
    const bool hvalid = hl < G;
    const int h = g * G + (hvalid ? hl : 0);
    const int64_t row = static_cast<int64_t>(s) * Hq + h;
    u32x4 qf[D / 32];
    WaveAttn<D> st;
    attn_init(st);
    const int32_t* bt = block_table + static_cast<int64_t>(s) * MB;
    const int tb = pre + 32 * t_begin;
    const int te = min(pre + 32 * t_end, n);
    // the prefix kernels' suffix waves: cacheable loads (measured faster than streamed ones,
    // 24.4 against 26.1 us on the shared-prefix batch over bf16 pools)
    const bool stream = !PREFIX && !shares_first_block(block_table, s, S, MB);
    if constexpr (PROBE) {
      probe_acc ^= stream ? probe_tiles<D, B, true>(kpool, vpool, bt, n, g, Hkv, tb, te)
                          : probe_tiles<D, B, false>(kpool, vpool, bt, n, g, Hkv, tb, te);
    } else if constexpr (kFp8) {
      load_q_fp8<D>(qf, q + row * D, hvalid, lg);
      // the prefix-aware kernel is held to 256 VGPRs: two register sets there
      if constexpr (PREFIX)
        attend_tiles_fp8<D, B, 2, false>(st, qf, kpool, vpool, bt, n, g, Hkv, tb, te,
                                         scale_log2);
      else if (stream)
        attend_tiles_fp8<D, B, 3, true>(st, qf, kpool, vpool, bt, n, g, Hkv, tb, te,
                                        scale_log2);
      else
        attend_tiles_fp8<D, B, 3, false>(st, qf, kpool, vpool, bt, n, g, Hkv, tb, te,
                                         scale_log2);
    } else if constexpr (STEP) {
      load_q<D>(qf, q + row * D, hvalid, lg);
      const int slot = sp.slots[s];
      const int np = slot >= 0 ? n - 1 : n;  // tokens read from the pool
      if (stream)
        attend_tiles<D, B, true>(st, qf, kpool, vpool, bt, np, g, Hkv, tb, min(te, np),
                                 scale_log2, hvalid);
      else
        attend_tiles<D, B, false>(st, qf, kpool, vpool, bt, np, g, Hkv, tb, min(te, np),
                                  scale_log2, hvalid);
      if (slot >= 0 && te == n) {
        const int64_t src = (static_cast<int64_t>(s) * Hkv + g) * D;
        attend_one_token<D>(st, qf, sp.k_new + src, sp.v_new + src, scale_log2);
        if (hgrp == 0) {  // store the token: K row (16-byte pieces), V column (stride B)
          const int64_t blk = slot / B;
          const int off = slot - static_cast<int>(blk) * B;
          const int64_t tile = blk * Hkv + g;
          if (lane < D / 8)
            *reinterpret_cast<u32x4*>(sp.kpool + (tile * B + off) * D + 8 * lane) =
                load16(sp.k_new + src + 8 * lane);
          for (int d = lane; d < D; d += 64) sp.vpool[(tile * D + d) * B + off] = sp.v_new[src + d];
        }
      }
    } else {
      load_q<D>(qf, q + row * D, hvalid, lg);
      if (stream)
        attend_tiles<D, B, true>(st, qf, kpool, vpool, bt, n, g, Hkv, tb, te, scale_log2,
                                 hvalid);
      else
        attend_tiles<D, B, false>(st, qf, kpool, vpool, bt, n, g, Hkv, tb, te, scale_log2,
                                  hvalid);
    }
    const float l_total = xor32_sum(xor16_sum(st.l));
    const int64_t wf = wave_of(a);
    const int64_t wl = wave_of(a + ts - 1);
    const int pc = PREFIX ? (pre + kPrefixChunk - 1) / kPrefixChunk : 0;
    const float osc = kFp8 ? out_scale : 1.0f;
    if (!PROBE && hvalid) {
      if (pc == 0 && wf == wl) write_final<D>(out + row * D, st, l_total, lg, osc);
      else if (pc + (w - wf) < KSTRIDE)  // always true when context_lens respect max_context_len
        write_partial<D>(part_o, part_m, part_l, row * KSTRIDE + pc + (w - wf), st, l_total, lg,
                         osc);
    }
    x = a + t_end;
    if (++j == segs) {  // next non-empty sequence
      j = 0;
      do {
        sstart += static_cast<int64_t>(segs) * ts;
        if (++s >= S) break;
        n = context_lens[s];
        pre = prefix_of(s);
        ts = (n - pre + 31) >> 5;
      } while (ts == 0);
      if (s >= S) break;
    }
  }
  if constexpr (PROBE) probe_sink[static_cast<int64_t>(w) * 64 + lane] = probe_acc;
}

// KvT: uint16_t for bf16 pools, uint8_t for E4M3 pools (out_scale = the V scale).
// kBalancedWavesPerGroup (launch.hpp): four waves per workgroup, one per SIMD of a compute unit
// (a quarter of the workgroup dispatches of one wave per workgroup).
template <int D, int B, typename OutT, typename KvT>
__global__ __launch_bounds__(64 * kBalancedWavesPerGroup) void decode_balanced_kernel(
    OutT* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_m,
    float* __restrict__ part_l, int32_t* __restrict__ seg_count,
    const uint16_t* __restrict__ q, const KvT* __restrict__ kpool,
    const KvT* __restrict__ vpool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, int S, int Hq, int Hkv, int G, int HG, int MB,
    int KMAX, int min_tiles, float scale_log2, float out_scale) {
  balanced_body<D, B, OutT, KvT, false>(
      blockIdx.x * kBalancedWavesPerGroup + (threadIdx.x >> 6),
      gridDim.x * kBalancedWavesPerGroup, out, part_o, part_m, part_l,
                                        seg_count, q, kpool, vpool, block_table, context_lens, S,
                                        Hq, Hkv, G, HG, MB, KMAX, min_tiles, scale_log2,
                                        out_scale, PrefixInfo{nullptr, nullptr, 0});
}

// kv_cache_write_and_decode for bf16 pools (see StepInfo).
template <int D, int B, typename OutT>
__global__ __launch_bounds__(64 * kBalancedWavesPerGroup) void decode_step_kernel(
    OutT* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_m,
    float* __restrict__ part_l, int32_t* __restrict__ seg_count, const uint16_t* __restrict__ q,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ slots, uint16_t* __restrict__ kpool,
    uint16_t* __restrict__ vpool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, int S, int Hq, int Hkv, int G, int HG, int MB,
    int KMAX, int min_tiles, float scale_log2) {
  balanced_body<D, B, OutT, uint16_t, false, true>(
      blockIdx.x * kBalancedWavesPerGroup + (threadIdx.x >> 6),
      gridDim.x * kBalancedWavesPerGroup, out, part_o, part_m, part_l, seg_count, q, kpool, vpool,
      block_table, context_lens, S, Hq, Hkv, G, HG, MB, KMAX, min_tiles, scale_log2, 1.0f,
      PrefixInfo{nullptr, nullptr, 0}, StepInfo{k_new, v_new, slots, kpool, vpool});
}

// Read probe kernel: the balanced decode's launch shape and tile walk (see probe_tiles); each
// lane leaves its XOR in sink[wave][lane].
template <int D, int B>
__global__ __launch_bounds__(64 * kBalancedWavesPerGroup) void decode_read_probe_kernel(
    uint32_t* __restrict__ sink, const uint16_t* __restrict__ kpool,
    const uint16_t* __restrict__ vpool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, int S, int Hq, int Hkv, int G, int HG, int MB,
    int min_tiles) {
  balanced_body<D, B, float, uint16_t, false, false, true>(
      blockIdx.x * kBalancedWavesPerGroup + (threadIdx.x >> 6),
      gridDim.x * kBalancedWavesPerGroup, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
      kpool, vpool, block_table, context_lens, S, Hq, Hkv, G, HG, MB, 0, min_tiles, 0.f, 1.0f,
      PrefixInfo{nullptr, nullptr, 0}, StepInfo{}, sink);
}

// Prefix chunks, one workgroup of kPrefixWgWaves waves per (group, KV head, chunk, block of
// 32 * kPrefixWgWaves query columns): the columns are (member sequence, query head) pairs, 32
// per wave. The chunk's K/V tiles (kPrefixChunk tokens of the shared blocks) are staged in LDS
// as bf16 once, all of them at the start (no LDS stage is reused), and every wave computes its
// columns against each tile as the chunked prefill does against its rows, without a causal
// mask (every member's query follows the whole prefix):
//   S^T[32 keys][32 columns] = K_tile . Q^T,  online softmax per column,
//   O^T[D][32 columns] += V_tile^T . P^T      (32x32x16 MFMAs)
// Each column leaves one partial (m, l, O / l) at its row's slot for the chunk, or its final
// output when the prefix is one chunk and the whole context.
constexpr int kPrefixWgCols = kPrefixWgColumns;

// f(std::integral_constant<int, i>{}) for i = 0 .. N-1, in order (i usable as a constant).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_from(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_from<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) { static_for_from<0, N>(f); }
constexpr int kPrefixChunkTiles = kPrefixChunk / 32;

template <int D>
constexpr int prefix_stage_bytes() { return 32 * 2 * D + D * 64; }  // K tile + V tile

template <int D, int B, typename OutT, typename KvT>
__device__ __forceinline__ void prefix_wg(
    int64_t unit, unsigned char* __restrict__ smem, OutT* __restrict__ out,
    float* __restrict__ part_o, float* __restrict__ part_m, float* __restrict__ part_l,
    const uint16_t* __restrict__ q, const KvT* __restrict__ kpool,
    const KvT* __restrict__ vpool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, int Hq, int Hkv, int G, int MB, int KSTRIDE, int CB,
    int NCH, float scale_log2, int neg_scale, float out_scale, PrefixInfo pf) {
  constexpr bool kFp8 = sizeof(KvT) == 1;
  constexpr int KK = D / 16;              // QK MFMA steps
  constexpr int DT = D / 32;              // PV output tiles
  constexpr int NW = kPrefixWgWaves;
  constexpr int NCT = kPrefixChunkTiles;  // tiles per chunk, one LDS stage each
  constexpr int KROW = 2 * D;             // bytes of one K row in LDS
  constexpr int CPR = D / 8;              // 16-byte chunks per K row
  constexpr int K_BYTES = 32 * KROW;
  constexpr int STAGE = prefix_stage_bytes<D>();
  constexpr int KC = K_BYTES / 1024;      // 1 KiB DMA instructions for K (V follows at KC)
  constexpr int LPT = STAGE / 1024 / NW;  // DMA instructions per wave per tile
  static_assert(LPT >= 1 && (STAGE / 1024) % NW == 0, "DMA work must split evenly over waves");
  static_assert(NCT * LPT <= 63, "every DMA of the chunk fits the vmcnt counter");

  const int cb = static_cast<int>(unit % CB);
  int64_t r = unit / CB;
  const int ch = static_cast<int>(r % NCH);
  r /= NCH;
  const int g = static_cast<int>(r % Hkv);
  const int gi = static_cast<int>(r / Hkv);
  // (all of these are uniform over the workgroup, so whole workgroups leave together)
  if (gi >= pf.NG) return;
  const int s0 = pf.group_start[gi];
  const int ncols = (pf.group_start[gi + 1] - s0) * G;
  const int pre = pf.group_prefix_len[gi];
  const int tok0 = ch * kPrefixChunk;
  if (tok0 >= pre || cb * kPrefixWgCols >= ncols) return;
  const int te = min(pre, tok0 + kPrefixChunk);
  const int pblk = pre / B;  // the prefix's blocks (pre is a multiple of B)
  const int32_t* bt = block_table + static_cast<int64_t>(s0) * MB;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 31;
  const int hb = lane >> 5;
  const int c = cb * kPrefixWgCols + 32 * wave + col;
  const bool valid = c < ncols;
  const bool wave_active = cb * kPrefixWgCols + 32 * wave < ncols;
  const int mi = valid ? c / G : 0;
  const int64_t row = static_cast<int64_t>(s0 + mi) * Hq + g * G + (valid ? c - mi * G : 0);

  u32x4 qf[KK];
  {
    // A negative scale is applied as |scale| on -q (bf16 negation flips the sign bits), so the
    // maximum can be taken on the raw scores. A column past the group reads the group's first
    // query (its results are never stored), so that every load is unconditional and none has
    // to be waited for before the DMAs are issued.
    const uint16_t* qrow = q + row * D + 8 * hb;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = load16(qrow + 16 * kk);
  }

  // Staging: piece j of wave w fills KiB (LPT * w + j) of a stage, 16 bytes (8 bf16 values)
  // per lane. K pieces cover 64 / CPR key rows each, V pieces 16 dims x 32 keys; a lane's offset
  // inside its block is the same for every tile, so its source is a fixed address inside block
  // 0 of the pool plus the tile's block id times the block's bytes. bf16 pools: each piece is
  // one DMA (global_load_lds). E4M3 pools: each lane loads its 8 codes (8 bytes) into registers,
  // widens them to bf16 exactly and writes the 16 bytes to the same LDS place, so the tiles in
  // LDS, and everything that reads them, are the same for both pool types.
  const KvT* kg = kpool + static_cast<int64_t>(g) * B * D;
  const KvT* vg = vpool + static_cast<int64_t>(g) * B * D;
  const char* lsrc[LPT];
  bool ssel[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int ci = LPT * wave + j;
    if (ci < KC) {
      const int prow = ci * (64 / CPR) + lane / CPR;
      const int chunk = (lane % CPR) ^ kswz<D>(prow);
      lsrc[j] = reinterpret_cast<const char*>(kg + (prow % B) * D + 8 * chunk);
      ssel[j] = B == 16 && prow >= 16;
    } else {
      const int d = (ci - KC) * 16 + lane / 4;
      const int chunk = (lane & 3) ^ vswz(d);  // keys 8*chunk .. 8*chunk+7
      lsrc[j] = reinterpret_cast<const char*>(vg + d * B + (8 * chunk) % B);
      ssel[j] = B == 16 && chunk >= 2;
    }
  }
  const uint32_t blk_bytes = static_cast<uint32_t>(sizeof(KvT) * Hkv * B * D);  // < 2^32
  // Every stage is filled, also past the chunk's last tile (those repeat the prefix's last
  // blocks and are never computed), so that the count of DMAs, and each wait below, is fixed.
  // The chunk's block ids first (uniform indexes: scalar loads, which do not count in vmcnt),
  // so that their loads overlap.
  constexpr int NID = NCT * 32 / B;
  uint32_t ids[NID];
#pragma unroll
  for (int i = 0; i < NID; ++i)
    ids[i] = static_cast<uint32_t>(
        bt[__builtin_amdgcn_readfirstlane(min(tok0 / B + i, pblk - 1))]);
  // bf16: q has arrived before the DMAs start counting in the same counter (its loads overlap
  // the block ids' loads); the tile waits below then count DMAs only.
  if constexpr (!kFp8) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  {
    const uint32_t flip = neg_scale ? 0x80008000u : 0u;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] ^= flip;
  }
  [[maybe_unused]] u32x2 raw[kFp8 ? NCT : 1][LPT];  // E4M3 codes of every piece of the chunk
#pragma unroll
  for (int t = 0; t < NCT; ++t) {
    const uint32_t ida = ids[t * 32 / B];
    const uint32_t idb = B == 16 ? ids[t * 32 / B + 1] : ida;
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const uint32_t bid = (B == 16 && ssel[j]) ? idb : ida;
      const char* src = lsrc[j] + static_cast<uint64_t>(bid) * blk_bytes;
      if constexpr (kFp8)
        raw[t][j] = load8(src);
      else
        __builtin_amdgcn_global_load_lds(src, smem + t * STAGE + (LPT * wave + j) * 1024, 16, 0,
                                         0);
    }
  }

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  float m = -INFINITY;
  float m_grow_raw = -INFINITY;  // (m + 8) / scale_log2: the raw score past which m moves
  const float inv_scale_log2 = 1.0f / scale_log2;
  float l[2] = {0.f, 0.f};
  // MFMA row of the K operand -> key within the tile: lane half hb gets keys 16*hb + i.
  const int krow = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
  const int kbase = krow * KROW;
  const int kx = kswz<D>(krow);
  const int vx = vswz(col);

  auto compute = [&](int t) {
    const int key0 = tok0 + 32 * t;
    const unsigned char* st = smem + t * STAGE;
    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
    u32x4 ka[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      ka[kk] = *reinterpret_cast<const u32x4*>(st + kbase + 16 * ((2 * kk + hb) ^ kx));
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) sacc = mfma32x32x16(ka[kk], qf[kk], sacc);
    u32x4 va[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const unsigned char* vrow = st + K_BYTES + (32 * dt + col) * 64;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        va[dt][j] = *reinterpret_cast<const u32x4*>(vrow + 16 * ((2 * hb + j) ^ vx));
    }
    const int vlim = te - key0;  // keys of the tile inside the chunk
    if (vlim < 32) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (16 * hb + i >= vlim) sacc[i] = -INFINITY;
    }
    float rmax = sacc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) rmax = __builtin_elementwise_maximum(rmax, sacc[i]);
    // Lazy rescaling as in the chunked prefill: the reference max moves only when a column's
    // max grows past it by more than 2^8; each lane half tests its own keys in raw units.
    if (__builtin_amdgcn_ballot_w64(rmax > m_grow_raw)) {
      const auto rr = __builtin_amdgcn_permlane32_swap(__float_as_uint(rmax),
                                                       __float_as_uint(rmax), false, false);
      const float col_raw =
          __builtin_elementwise_maximum(__uint_as_float(rr[0]), __uint_as_float(rr[1]));
      const bool grow = col_raw > m_grow_raw;
      const float mnew = grow ? col_raw * scale_log2 : m;
      const float alpha = fast_exp2(m - mnew);
      m = mnew;
      m_grow_raw = (mnew + 8.0f) * inv_scale_log2;
      l[0] *= alpha;
      l[1] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
    }
    u32x4 pb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = fast_exp2(__builtin_fmaf(sacc[8 * j + 2 * w], scale_log2, -m));
        const float p1 = fast_exp2(__builtin_fmaf(sacc[8 * j + 2 * w + 1], scale_log2, -m));
        const bf16x2 pp = __builtin_convertvector((f32x2{p0, p1}), bf16x2);
        pb[j][w] = __builtin_bit_cast(uint32_t, pp);
        l[j] = __builtin_amdgcn_fdot2_f32_bf16(pp, bf16x2{1.0f, 1.0f}, l[j], false);
      }
    if (vlim < 32) {  // words past the chunk may hold anything: clear their V
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int k0 = 16 * hb + 8 * j + 2 * w;
          const uint32_t keep =
              (k0 < vlim ? 0x0000ffffu : 0u) | (k0 + 1 < vlim ? 0xffff0000u : 0u);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) va[dt][j][w] &= keep;
        }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[dt] = mfma32x32x16(va[dt][j], pb[j], acc[dt]);
  };

  const int ntiles = (te - tok0 + 31) >> 5;
  // Tile t: this wave's DMAs of it are done once at most (NCT - 1 - t) * LPT remain (the q loads
  // were issued first); the barrier then covers every wave's.
  static_for<NCT>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    if constexpr (kFp8) {
      // (the compiler waits for exactly this tile's codes; the LDS writes are waited for
      // before the barrier that publishes them)
#pragma unroll
      for (int j = 0; j < LPT; ++j)
        *reinterpret_cast<u32x4*>(smem + t * STAGE + (LPT * wave + j) * 1024 + 16 * lane) =
            e4m3x8_to_bf16x8(raw[t][j][0], raw[t][j][1]);
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm((NCT - 1 - t) * LPT));
    }
    __builtin_amdgcn_s_barrier();
    if (t < ntiles && wave_active) compute(t);
  });

  if (!wave_active) return;
  const float lsum = xor32_sum(l[0] + l[1]);
  if (!valid) return;
  const int pc = (pre + kPrefixChunk - 1) / kPrefixChunk;
  const int seq = s0 + mi;
  const float inv = out_scale / lsum;  // (E4M3 pools: the V scale is folded in here)
  if (pc == 1 && context_lens[seq] == pre) {
    OutT* o = out + row * D + 4 * hb;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        store_out(o + 32 * dt + 8 * (i >> 2) + (i & 3), acc[dt][i] * inv);
    return;
  }
  const int64_t idx = row * KSTRIDE + ch;
  if (hb == 0) {
    part_m[idx] = m;
    part_l[idx] = lsum;
  }
  float* o = part_o + idx * D + 4 * hb;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      *reinterpret_cast<f32x4*>(o + 32 * dt + 8 * i4) =
          f32x4{acc[dt][4 * i4], acc[dt][4 * i4 + 1], acc[dt][4 * i4 + 2], acc[dt][4 * i4 + 3]} *
          inv;
}

// Prefix-aware decode: WGp workgroups of prefix chunks (prefix_wg), then workgroups of
// kPrefixWgWaves suffix waves of the balanced split (Ws waves in all). The prefix workgroups come
// first, so that they are dispatched with the first suffix workgroups and run beside them (the
// chunks' products on the matrix cores, the suffixes streaming from HBM). Prefix workgroups are
// numbered so that the column blocks of one (group, KV head, chunk), which read the same K/V,
// land on the same XCD. The LDS that the prefix chunks take (8 stages) leaves one workgroup per
// CU. KvT: uint16_t for bf16 pools, uint8_t for E4M3 pools (out_scale = the V scale).
template <int D, int B, typename OutT, typename KvT>
__global__ __launch_bounds__(64 * kPrefixWgWaves) void decode_prefix_wg_kernel(
    OutT* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_m,
    float* __restrict__ part_l, int32_t* __restrict__ seg_count,
    const uint16_t* __restrict__ q, const KvT* __restrict__ kpool,
    const KvT* __restrict__ vpool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ group_start,
    const int32_t* __restrict__ group_prefix_len, int NG, int S, int Hq, int Hkv, int G, int HG,
    int MB, int KSTRIDE, int min_tiles, int WGp, int Ws, int CB, int NCH, float scale_log2,
    float pscale_log2, int neg_scale, float out_scale) {
  __shared__ __attribute__((aligned(16))) unsigned char
      smem[kPrefixChunkTiles * prefix_stage_bytes<D>()];
  const PrefixInfo pf{group_start, group_prefix_len, NG};
  const int b = blockIdx.x;
  if (b < WGp) {
    const int64_t unit = static_cast<int64_t>(b & 7) * (WGp >> 3) + (b >> 3);
    prefix_wg<D, B, OutT, KvT>(unit, smem, out, part_o, part_m, part_l, q, kpool, vpool,
                               block_table, context_lens, Hq, Hkv, G, MB, KSTRIDE, CB, NCH,
                               pscale_log2, neg_scale, out_scale, pf);
    return;
  }
  const int w = (b - WGp) * kPrefixWgWaves + (threadIdx.x >> 6);
  if (w >= Ws) return;
  balanced_body<D, B, OutT, KvT, true>(w, Ws, out, part_o, part_m, part_l, seg_count, q, kpool,
                                       vpool, block_table, context_lens, S, Hq, Hkv, G, HG, MB,
                                       KSTRIDE, min_tiles, scale_log2, out_scale, pf);
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
      for (int i = 0; i < DPL; ++i)
        acc[i] += pj * vpool[vb + static_cast<int64_t>(lane + 64 * i) * B];
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

// Merge of partial results: out = sum_k w_k o_k / sum_k w_k, w_k = l_k * 2^(m_k - max m).
// One workgroup per (sequence, query head). Fixed partitions (seg_count == nullptr): the row has
// ceil(n / P) partials. Balanced split: seg_count gives the number of waves that shared the
// row's segment; 1 means the output was written already, 0 an empty context.
// Latency: the row's count and the (m, l) of its first 64 slots are loaded together (slots past
// the count hold stale values and are ignored), then all partial outputs with their loads in
// flight together: two dependent round trips to memory.
template <typename OutT>
__global__ __launch_bounds__(64) void decode_reduce_kernel(
    OutT* __restrict__ out, const float* __restrict__ part_o, const float* __restrict__ part_m,
    const float* __restrict__ part_l, const int32_t* __restrict__ context_lens,
    const int32_t* __restrict__ seg_count, int Hq, int G, int HG, int D, int P, int KMAX) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t row = static_cast<int64_t>(s) * Hq + h;
  OutT* o = out + row * D;
  const float* pm = part_m + row * KMAX;
  const float* pl = part_l + row * KMAX;
  const float* po = part_o + row * KMAX * D;
  const float m0 = (tid < KMAX) ? pm[tid] : -INFINITY;
  const float l0 = (tid < KMAX) ? pl[tid] : 0.f;
  int cnt;
  if (seg_count) {
    const int g = h / G;
    const int j = g * HG + (h - g * G) / 16;
    cnt = seg_count[static_cast<int64_t>(s) * (Hq / G) * HG + j];
    if (cnt == 1) return;
  } else {
    cnt = (context_lens[s] + P - 1) / P;
  }
  cnt = min(cnt, KMAX);  // KMAX bounds the workspace rows
  if (cnt <= 0) {
    for (int d = tid; d < D; d += 64) store_out(o + d, 0.0f);
    return;
  }
  float M = (tid < cnt) ? m0 : -INFINITY;
  for (int k = tid + 64; k < cnt; k += 64) M = fmaxf(M, pm[k]);
#pragma unroll
  for (int mk = 32; mk >= 1; mk >>= 1) M = fmaxf(M, __shfl_xor(M, mk));
  const bool two = tid + 64 < D;
  float acc0 = 0.f, acc1 = 0.f, wsum = 0.f;
  for (int k0 = 0; k0 < cnt; k0 += 64) {
    const int k = k0 + tid;
    float wk = 0.f;
    if (k < cnt) wk = (k0 == 0) ? l0 * fast_exp2(m0 - M) : pl[k] * fast_exp2(pm[k] - M);
    const int kn = min(64, cnt - k0);
    const float* pk = po + static_cast<int64_t>(k0) * D;
    // Groups of G partials with their loads in flight together (G = 16 for long rows, 4 for
    // short ones); the last group is padded with the chunk's last slot at weight 0 (a written
    // slot, so its values are finite), so no partial waits for the one before it.
    auto merge = [&](auto group) {
      constexpr int GS = decltype(group)::value;
      for (int i = 0; i < kn; i += GS) {
        float a[GS], b[GS], wi[GS];
#pragma unroll
        for (int u = 0; u < GS; ++u) {
          const int iu = min(i + u, kn - 1);
          const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), iu));
          wi[u] = (i + u < kn) ? w : 0.f;
          a[u] = pk[static_cast<int64_t>(iu) * D + tid];
          b[u] = two ? pk[static_cast<int64_t>(iu) * D + tid + 64] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < GS; ++u) {
          wsum += wi[u];
          acc0 += wi[u] * a[u];
          acc1 += wi[u] * b[u];
        }
      }
    };
    if (kn > 4) merge(std::integral_constant<int, 16>{});
    else merge(std::integral_constant<int, 4>{});
  }
  const float inv = 1.0f / wsum;
  store_out(o + tid, acc0 * inv);
  if (two) store_out(o + tid + 64, acc1 * inv);
}

// The same merge for rows that can have many partials (the host picks it when a row may have
// more than 64, long contexts spread over many waves, and the rows are fewer than the GPU's
// SIMDs). Four waves per row: the row's maximum over all slots meets in LDS, then each wave
// merges a quarter of the slots, sixteen partials' loads in flight together, and the four
// waves' sums meet in LDS again.
template <typename OutT>
__global__ __launch_bounds__(256) void decode_reduce_wide_kernel(
    OutT* __restrict__ out, const float* __restrict__ part_o, const float* __restrict__ part_m,
    const float* __restrict__ part_l, const int32_t* __restrict__ context_lens,
    const int32_t* __restrict__ seg_count, int Hq, int G, int HG, int D, int P, int KMAX) {
  __shared__ float s_max[4];
  __shared__ float s_acc[4][2][64];
  __shared__ float s_sum[4];
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int64_t row = static_cast<int64_t>(s) * Hq + h;
  OutT* o = out + row * D;
  const float* pm = part_m + row * KMAX;
  const float* pl = part_l + row * KMAX;
  const float* po = part_o + row * KMAX * D;
  int cnt;
  if (seg_count) {
    const int g = h / G;
    const int j = g * HG + (h - g * G) / 16;
    cnt = seg_count[static_cast<int64_t>(s) * (Hq / G) * HG + j];
    if (cnt == 1) return;  // uniform over the workgroup
  } else {
    cnt = (context_lens[s] + P - 1) / P;
  }
  cnt = min(cnt, KMAX);  // KMAX bounds the workspace rows
  if (cnt <= 0) {
    for (int d = tid; d < D; d += 256) store_out(o + d, 0.0f);
    return;
  }
  float M = -INFINITY;
  for (int k = tid; k < cnt; k += 256) M = fmaxf(M, pm[k]);
#pragma unroll
  for (int mk = 32; mk >= 1; mk >>= 1) M = fmaxf(M, __shfl_xor(M, mk));
  if (lane == 0) s_max[wv] = M;
  __syncthreads();
  M = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const bool two = lane + 64 < D;
  const int kb = (wv * cnt) / 4;
  const int ke = ((wv + 1) * cnt) / 4;
  float acc0 = 0.f, acc1 = 0.f, wsum = 0.f;
  for (int k0 = kb; k0 < ke; k0 += 64) {
    const int k = k0 + lane;
    const float wk = (k < ke) ? pl[k] * fast_exp2(pm[k] - M) : 0.f;
    const int kn = min(64, ke - k0);
    const float* pk = po + static_cast<int64_t>(k0) * D;
    // groups of sixteen, the last one padded with the wave's last slot at weight 0 (a written
    // slot, so its values are finite), so every group's loads are in flight together
    for (int i = 0; i < kn; i += 16) {
      float a[16], b[16], wi[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int iu = min(i + u, kn - 1);
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wk), iu));
        wi[u] = (i + u < kn) ? w : 0.f;
        a[u] = pk[static_cast<int64_t>(iu) * D + lane];
        b[u] = two ? pk[static_cast<int64_t>(iu) * D + lane + 64] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        wsum += wi[u];
        acc0 += wi[u] * a[u];
        acc1 += wi[u] * b[u];
      }
    }
  }
  s_acc[wv][0][lane] = acc0;
  s_acc[wv][1][lane] = acc1;
  if (lane == 0) s_sum[wv] = wsum;
  __syncthreads();
  if (wv != 0) return;
  const float inv = 1.0f / (s_sum[0] + s_sum[1] + s_sum[2] + s_sum[3]);
  store_out(o + lane, (s_acc[0][0][lane] + s_acc[1][0][lane] + s_acc[2][0][lane] +
                       s_acc[3][0][lane]) * inv);
  if (two)
    store_out(o + lane + 64, (s_acc[0][1][lane] + s_acc[1][1][lane] + s_acc[2][1][lane] +
                              s_acc[3][1][lane]) * inv);
}

// ------------------------------------------------------------------------------ launchers

// The scratch of pkv_paged_attention_decode_noalloc (see kNoAllocScratchBytes). In host code
// `scratch` names a host-side stand-in, not device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device, looked up on the first call made with
// that device current and kept per device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!per_device[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  *bytes = kNoAllocScratchBytes;
  return hipSuccess;
}

template <int D, int B, typename OutT>
static hipError_t launch_bf16(const DecodeArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const int HG = (G + 15) / 16;
  const int groups = (a.waves + kBalancedWavesPerGroup - 1) / kBalancedWavesPerGroup;
  if (a.fp8_kv) {
    return launch_kernel(K_DECODE_PARTITION, decode_balanced_kernel<D, B, OutT, uint8_t>,
        dim3(groups), dim3(64 * kBalancedWavesPerGroup), st, static_cast<OutT*>(a.out), a.part_o,
        a.part_m, a.part_l, a.seg_count, static_cast<const uint16_t*>(a.q),
        static_cast<const uint8_t*>(a.k_pool), static_cast<const uint8_t*>(a.v_pool),
        a.block_table, a.context_lens, a.S, a.Hq, a.Hkv, G, HG, a.MB, a.KMAX, a.min_tiles,
        a.scale * a.k_scale * kLog2e, a.v_scale);
  }
  if (a.balanced) {
    return launch_kernel(K_DECODE_PARTITION, decode_balanced_kernel<D, B, OutT, uint16_t>,
        dim3(groups), dim3(64 * kBalancedWavesPerGroup), st, static_cast<OutT*>(a.out), a.part_o,
        a.part_m, a.part_l, a.seg_count, static_cast<const uint16_t*>(a.q),
        static_cast<const uint16_t*>(a.k_pool), static_cast<const uint16_t*>(a.v_pool),
        a.block_table, a.context_lens, a.S, a.Hq, a.Hkv, G, HG, a.MB, a.KMAX, a.min_tiles,
        a.scale * kLog2e, 1.0f);
  }
  dim3 grid(a.Hkv * HG, a.S, a.NP);
  if (a.NP > 1)
    return launch_kernel(K_DECODE_PARTITION, decode_fixed_kernel<D, B, true, OutT>, dim3(grid),
        dim3(64), st, static_cast<OutT*>(a.out), a.part_o, a.part_m, a.part_l,
        static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k_pool),
        static_cast<const uint16_t*>(a.v_pool), a.block_table, a.context_lens, a.Hq, a.Hkv, G, HG,
        a.MB, a.P, a.NP, a.scale * kLog2e);
  return launch_kernel(K_DECODE_PARTITION, decode_fixed_kernel<D, B, false, OutT>, dim3(grid),
        dim3(64), st, static_cast<OutT*>(a.out), a.part_o, a.part_m, a.part_l,
        static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k_pool),
        static_cast<const uint16_t*>(a.v_pool), a.block_table, a.context_lens, a.Hq, a.Hkv, G, HG,
        a.MB, a.P, a.NP, a.scale * kLog2e);
}

// Prefix-aware decode. The prefix workgroups take a positive scale (see prefix_wg; zero becomes
// a tiny one, which gives the uniform softmax of a zero scale).
template <int D, int B, typename OutT, typename KvT>
static hipError_t launch_prefix_wg_t(const DecodeArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const int HG = (G + 15) / 16;
  const float sl = a.scale * (a.fp8_kv ? a.k_scale : 1.0f) * kLog2e;
  const int wgs = (a.waves + kPrefixWgWaves - 1) / kPrefixWgWaves;
  return launch_kernel(K_DECODE_PARTITION, decode_prefix_wg_kernel<D, B, OutT, KvT>,
      dim3(a.prefix_units + wgs), dim3(64 * kPrefixWgWaves), st, static_cast<OutT*>(a.out),
      a.part_o, a.part_m, a.part_l, a.seg_count, static_cast<const uint16_t*>(a.q),
      static_cast<const KvT*>(a.k_pool), static_cast<const KvT*>(a.v_pool), a.block_table,
      a.context_lens, a.group_start, a.group_prefix_len, a.num_groups, a.S, a.Hq, a.Hkv, G, HG,
      a.MB, a.KMAX, a.min_tiles, a.prefix_units, a.waves, a.prefix_col_blocks,
      a.prefix_chunks, sl, fmaxf(fabsf(sl), 1e-30f), a.scale < 0.f ? 1 : 0,
      a.fp8_kv ? a.v_scale : 1.0f);
}

template <int D, int B, typename OutT>
static hipError_t launch_step_t(const DecodeArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const int HG = (G + 15) / 16;
  return launch_kernel(K_DECODE_PARTITION, decode_step_kernel<D, B, OutT>,
      dim3((a.waves + kBalancedWavesPerGroup - 1) / kBalancedWavesPerGroup),
      dim3(64 * kBalancedWavesPerGroup), st, static_cast<OutT*>(a.out), a.part_o, a.part_m,
      a.part_l, a.seg_count,
      static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k_new),
      static_cast<const uint16_t*>(a.v_new), a.slot_mapping,
      static_cast<uint16_t*>(const_cast<void*>(a.k_pool)),
      static_cast<uint16_t*>(const_cast<void*>(a.v_pool)), a.block_table, a.context_lens, a.S,
      a.Hq, a.Hkv, G, HG, a.MB, a.KMAX, a.min_tiles, a.scale * kLog2e);
}

template <int D, int B, bool SPLIT, typename OutT>
static hipError_t launch_f32(const DecodeArgs& a, hipStream_t st) {
  dim3 grid(a.S, a.Hq, a.NP);
  return launch_kernel(K_DECODE_PARTITION, attn_f32_kernel<D, B, SPLIT, false, OutT>, dim3(grid),
                       dim3(64),
      st, static_cast<OutT*>(a.out), a.part_o, a.part_m, a.part_l, static_cast<const float*>(a.q),
      static_cast<const float*>(a.k_pool), static_cast<const float*>(a.v_pool), a.block_table,
      a.context_lens, nullptr, a.S, a.Hq, a.Hkv, a.MB, a.P, a.NP, a.scale * kLog2e);
}

template <int D, int B, typename OutT>
static hipError_t dispatch_out_t(const DecodeArgs& a, hipStream_t st) {
  if (a.step) return launch_step_t<D, B, OutT>(a, st);
  if (a.num_groups > 0)
    return a.fp8_kv ? launch_prefix_wg_t<D, B, OutT, uint8_t>(a, st)
                    : launch_prefix_wg_t<D, B, OutT, uint16_t>(a, st);
  if (a.bf16_in || a.fp8_kv) return launch_bf16<D, B, OutT>(a, st);
  return a.NP > 1 ? launch_f32<D, B, true, OutT>(a, st) : launch_f32<D, B, false, OutT>(a, st);
}

template <int D, int B>
static hipError_t dispatch_out(const DecodeArgs& a, hipStream_t st) {
  return a.bf16_out ? dispatch_out_t<D, B, uint16_t>(a, st) : dispatch_out_t<D, B, float>(a, st);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  hipError_t e;
  if (a.D == 128) e = a.B == 16 ? dispatch_out<128, 16>(a, st) : dispatch_out<128, 32>(a, st);
  else e = a.B == 16 ? dispatch_out<64, 16>(a, st) : dispatch_out<64, 32>(a, st);
  // no merge after a refused partition launch (its partials were never written)
  if (e != hipSuccess || (!a.balanced && a.NP <= 1)) return e;
  const int G = a.Hq / a.Hkv;
  const int HG = (G + 15) / 16;
  const int kmax = a.balanced ? a.KMAX : a.NP;
  const int32_t* cnt = a.balanced ? a.seg_count : nullptr;
  dim3 grid(a.Hq, a.S);
  // Rows that may have many partials, and fewer rows than the GPU has SIMDs: four waves per
  // row. (With more rows than SIMDs the one-wave form is faster: 2048 rows of the 70B-shaped
  // batch took 4.9 us with it and 8.3 us with four waves per row.)
  if (kmax > 64 && static_cast<int64_t>(a.S) * a.Hq < 1024) {
    if (a.bf16_out)
      return launch_kernel(K_DECODE_REDUCE, decode_reduce_wide_kernel<uint16_t>, dim3(grid),
          dim3(256), st, static_cast<uint16_t*>(a.out), a.part_o, a.part_m, a.part_l,
          a.context_lens, cnt, a.Hq, G, HG, a.D, a.P, kmax);
    return launch_kernel(K_DECODE_REDUCE, decode_reduce_wide_kernel<float>, dim3(grid),
        dim3(256), st, static_cast<float*>(a.out), a.part_o, a.part_m, a.part_l,
        a.context_lens, cnt, a.Hq, G, HG, a.D, a.P, kmax);
  }
  if (a.bf16_out)
    return launch_kernel(K_DECODE_REDUCE, decode_reduce_kernel<uint16_t>, dim3(grid), dim3(64),
        st, static_cast<uint16_t*>(a.out), a.part_o, a.part_m, a.part_l, a.context_lens, cnt,
        a.Hq, G, HG, a.D, a.P, kmax);
  return launch_kernel(K_DECODE_REDUCE, decode_reduce_kernel<float>, dim3(grid), dim3(64), st,
      static_cast<float*>(a.out), a.part_o, a.part_m, a.part_l, a.context_lens, cnt, a.Hq, G, HG,
      a.D, a.P, kmax);
}

template <int D, int B>
static hipError_t launch_probe_t(const ReadProbeArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const int HG = (G + 15) / 16;
  return launch_kernel(K_READ_PROBE, decode_read_probe_kernel<D, B>,
                       dim3((a.waves + kBalancedWavesPerGroup - 1) / kBalancedWavesPerGroup),
                       dim3(64 * kBalancedWavesPerGroup), st, a.sink,
                       static_cast<const uint16_t*>(a.k_pool),
                       static_cast<const uint16_t*>(a.v_pool), a.block_table, a.context_lens, a.S,
                       a.Hq, a.Hkv, G, HG, a.MB, a.min_tiles);
}

hipError_t launch_read_probe(const ReadProbeArgs& a, hipStream_t st) {
  if (a.D == 128)
    return a.B == 16 ? launch_probe_t<128, 16>(a, st) : launch_probe_t<128, 32>(a, st);
  return a.B == 16 ? launch_probe_t<64, 16>(a, st) : launch_probe_t<64, 32>(a, st);
}

// fp32 prefill runs on the same vector kernel: chunk row i of a sequence is a decode row whose
// visible context ends at its own position (r + i + 1 keys).
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t st);

template <int D, int B, typename OutT>
static hipError_t launch_prefill_f32_t(const PrefillArgs& a, hipStream_t st) {
  dim3 grid(a.total_q, a.Hq, 1);
  return launch_kernel(K_PREFILL, attn_f32_kernel<D, B, false, true, OutT>, dim3(grid), dim3(64),
                       st,
      static_cast<OutT*>(a.out), nullptr, nullptr, nullptr, static_cast<const float*>(a.q),
      static_cast<const float*>(a.k_pool), static_cast<const float*>(a.v_pool), a.block_table,
      a.context_lens, a.cu_q_lens, a.S, a.Hq, a.Hkv, a.MB, 1 << 30, 1, a.scale * kLog2e);
}

template <int D, int B>
static hipError_t prefill_f32_out(const PrefillArgs& a, hipStream_t st) {
  return a.bf16_out ? launch_prefill_f32_t<D, B, uint16_t>(a, st)
                    : launch_prefill_f32_t<D, B, float>(a, st);
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t st) {
  if (a.D == 128)
    return a.B == 16 ? prefill_f32_out<128, 16>(a, st) : prefill_f32_out<128, 32>(a, st);
  return a.B == 16 ? prefill_f32_out<64, 16>(a, st) : prefill_f32_out<64, 32>(a, st);
}

}  // namespace pkv
