// paged_attention_prefill_chunk: a causal chunk of query tokens against the paged K/V.
//
// ("Serving Engines", How vLLM works: chunked prefill runs a prompt in slices interleaved with
// decode. "LLM Serving Engine Shootout" 3.1 equation for the scores, 5.1 for the fused steps.)
// Sequence s holds n tokens, the last c of which are this chunk (its K/V already written);
// chunk row i sits at position r + i, r = n - c, and attends to keys 0 .. r + i.
//
// bf16 path (matrix cores). A workgroup of eight waves owns (sequence, group of query heads
// sharing one KV head, tile of chunk rows). Each wave owns 32 query rows of one head, so the
// heads of a KV group, and two to eight row tiles, share every K/V tile the workgroup stages
// into LDS. Per 32-key tile:
//   S^T[32 keys][32 rows] = K_tile . Q^T      one 32x32x16 MFMA per 16 dims
//   online softmax per row (a lane owns a query row; the two lane halves hold 16 keys each)
//   O^T[D][32 rows]      += V_tile^T . P^T    two 32x32x16 MFMAs per 32 dims
// Keys are assigned to the MFMA rows of the first product so that the lane half hb ends up
// with keys 16*hb .. 16*hb+15, in order: then its P values are the B operand of the second
// product as they stand, and its V^T operand is 16 contiguous bytes of the dim-major V tile.
// K/V tiles go from HBM straight into LDS (global_load_lds: each lane's 16 bytes land at its own
// place in the wave's 1 KiB of LDS, no register round trip) through a ring of eight stages
// (128 KB of LDS: one workgroup per CU, two waves per SIMD). The ring advances two tiles per
// workgroup barrier, with up to six tiles in flight. Waits count those DMAs only (explicit
// s_waitcnt; block ids come through scalar loads, which count elsewhere); LDS rows are
// XOR-swizzled instead of padded, so that the 128-bit LDS reads are free of bank conflicts.
// Tiles wholly above a wave's causal diagonal are skipped; only diagonal tiles apply the mask.
// Workgroups are numbered so that the XCDs (the GPU deals consecutive workgroups round-robin to
// its eight XCDs, each with its own L2) get equal shares of the work, with the row tiles of one
// (sequence, KV head) on the same XCD and the tiles with the most keys first.
//
// fp32 prefill runs on the vector kernel in decode.hip.
#include "common.hpp"
#include "launch.hpp"
#include "lds_tile.hpp"

namespace pkv {

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t st);

constexpr float kLog2eP = 1.4426950408889634f;

__device__ __forceinline__ u32x4 lds16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

constexpr int kPrefillWaves = 8;  // waves per workgroup
constexpr int kStages = 8;        // K/V tiles in the LDS ring
constexpr int kTilesPerBarrier = 2;  // tiles the ring advances per workgroup barrier
constexpr int kRankMax = 64;       // largest batch whose sequences are ranked by work

// The sequence of rank j when sequences are ordered by decreasing c * (2n - c) (chunk length c,
// context length n), ties by index; j itself when the batch has more than RMAX sequences.
// Block-wide (every thread calls it, two barriers); scratch: 8 * RMAX + 4 bytes of LDS.
template <int NT, int RMAX>
__device__ __forceinline__ int seq_by_rank(int j, int S, const int32_t* __restrict__ cu_q_lens,
                                           const int32_t* __restrict__ context_lens,
                                           unsigned char* lds, int tid) {
  if (S > RMAX) return j;
  int64_t* key = reinterpret_cast<int64_t*>(lds);
  int* found = reinterpret_cast<int*>(lds + 8 * RMAX);
  for (int i = tid; i < S; i += NT) {
    const int64_t c = cu_q_lens[i + 1] - cu_q_lens[i];
    key[i] = c * (2 * static_cast<int64_t>(context_lens[i]) - c);
  }
  if (tid == 0) *found = j;  // overwritten below; keeps the result in range whatever happens
  __syncthreads();
  for (int i = tid; i < S; i += NT) {
    const int64_t ki = key[i];
    int rank = 0;
    for (int o = 0; o < S; ++o) {
      const int64_t ko = key[o];
      rank += (ko > ki || (ko == ki && o < i)) ? 1 : 0;
    }
    if (rank == j) *found = i;  // exactly one sequence has rank j
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*found);
}

template <int D, int B, typename OutT>
__global__ __launch_bounds__(64 * kPrefillWaves) void prefill_bf16_kernel(
    OutT* __restrict__ out, const uint16_t* __restrict__ q, const int32_t* __restrict__ cu_q_lens,
    const int32_t* __restrict__ context_lens, const uint16_t* __restrict__ kpool,
    const uint16_t* __restrict__ vpool, const int32_t* __restrict__ block_table, int Hq, int Hkv,
    int G, int HW, int MB, int n_tiles, int n_groups, float scale_log2, int neg_scale) {
  constexpr int KK = D / 16;             // QK MFMA steps
  constexpr int DT = D / 32;             // PV output tiles
  constexpr int NW = kPrefillWaves;
  constexpr int NT = 64 * NW;            // threads
  constexpr int NS = kStages;            // pipeline stages
  constexpr int KROW = 2 * D;            // bytes of one K row in LDS
  constexpr int CPR = D / 8;             // 16-byte chunks per K row
  constexpr int K_BYTES = 32 * KROW;     // K tile [32 keys][D]
  constexpr int V_BYTES = D * 64;        // V tile [D][32 keys]
  constexpr int STAGE = K_BYTES + V_BYTES;
  constexpr int KC = K_BYTES / 1024;     // 1 KiB DMA instructions for K (V follows at KC)
  constexpr int LPT = STAGE / 1024 / NW; // DMA instructions per wave (and per thread) per tile
  static_assert(LPT >= 1 && (STAGE / 1024) % NW == 0, "DMA work must split evenly over waves");
  static_assert(NS * STAGE >= 8 * kRankMax + 4, "the ranking scratch must fit the stages");
  __shared__ __attribute__((aligned(16))) unsigned char smem[NS * STAGE];

  // XCD-aware numbering. Workgroup b is dispatched to XCD b % 8, and each XCD works through its
  // share in order. The (head group, sequence) pairs are dealt round-robin to the XCDs (with 8
  // KV heads, XCD x takes KV head x of every sequence), so every XCD gets the same mix of
  // context lengths; all row tiles of a pair stay on one XCD and share its L2; within a pair
  // the tiles with the most keys start first.
  const int pairs = gridDim.y * gridDim.z;
  const int lin = blockIdx.x + n_tiles * (blockIdx.y + gridDim.y * blockIdx.z);
  int pair, tix;
  if ((pairs & 7) == 0) {
    const int k = lin >> 3;
    pair = (k / n_tiles) * 8 + (lin & 7);
    tix = k % n_tiles;
  } else {
    pair = lin / n_tiles;
    tix = lin % n_tiles;
  }
  const int tile = n_tiles - 1 - tix;
  const int gy = pair % gridDim.y;
  const int tid = threadIdx.x;
  // pair / gridDim.y is a rank: sequences are taken in order of decreasing work (estimated as
  // c * (2n - c), which grows with the chunk's visible (row, key) pairs), so that the longest
  // jobs start first and the short ones fill in behind them. Every workgroup ranks the batch
  // itself, in the LDS that the tile stages use later (up to kRankMax sequences; past that,
  // batch order).
  const int s = seq_by_rank<NT, kRankMax>(pair / gridDim.y, gridDim.z, cu_q_lens, context_lens,
                                          smem, tid);

  const int g = gy / n_groups;
  const int grp = gy - g * n_groups;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
  const int lane = tid & 63;
  const int col = lane & 31;
  const int hb = lane >> 5;
  const int head = g * G + grp * HW + (wave % HW);
  const int WGT = 32 * (NW / HW);

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
  const uint32_t blk_stride = static_cast<uint32_t>(Hkv) * B * D;  // < 2^32
  const uint16_t* kg = kpool + static_cast<int64_t>(g) * B * D;
  const uint16_t* vg = vpool + static_cast<int64_t>(g) * B * D;

  u32x4 qf[KK];
  {
    // rows past the chunk load nothing; their address is clamped into the chunk regardless
    const int qi = min(my_i, c - 1);
    const uint16_t* qrow = q + (static_cast<int64_t>(q0 + qi) * Hq + head) * D + 8 * hb;
    // A negative scale is applied as |scale| on -q (bf16 negation flips the sign bits), so the
    // scores' maximum can be taken on the raw MFMA results.
    const uint32_t flip = neg_scale ? 0x80008000u : 0u;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      qf[kk] = row_valid ? (load16(qrow + 16 * kk) ^ flip) : u32x4{0u, 0u, 0u, 0u};
  }

  // q must have arrived before the tile DMAs start counting in the same counter; the barrier
  // keeps the first DMAs out of the ranking scratch until every wave has read its result.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  // Block ids are wave-uniform: each is one scalar load (through the scalar cache; its wait
  // counts in lgkmcnt, so the tile loop's vector-memory waits still count DMAs only).
  auto block_id = [&](int lb) -> uint32_t {
    return static_cast<uint32_t>(bt[__builtin_amdgcn_readfirstlane(min(lb, nblk - 1))]);
  };

  // DMA of key tile t into stage t % NS: STAGE / 1 KiB instructions, LPT per wave; instruction
  // c (= LPT * wave + j) fills bytes c KiB .. of the stage. K instructions (c < KC) cover
  // 64 / CPR physical key rows each, V instructions 16 dims x 32 keys. Block ids are
  // wave-uniform per tile (two candidates when B = 16); a lane's offset inside the block tile
  // does not change from tile to tile (tiles start at multiples of 32, which B divides or
  // equals), so it is computed once. Each wave's instructions are all K or all V.
  const char* lsrc[LPT];  // the lane's 16 bytes inside block 0 of the pool it copies from
  bool ssel[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int c = LPT * wave + j;
    if (c < KC) {
      const int prow = c * (64 / CPR) + lane / CPR;
      const int chunk = (lane % CPR) ^ kswz<D>(prow);
      lsrc[j] = reinterpret_cast<const char*>(kg + (prow % B) * D + 8 * chunk);
      ssel[j] = B == 16 && prow >= 16;
    } else {
      const int d = (c - KC) * 16 + lane / 4;
      const int chunk = (lane & 3) ^ vswz(d);  // keys 8*chunk .. 8*chunk+7
      lsrc[j] = reinterpret_cast<const char*>(vg + d * B + (8 * chunk) % B);
      ssel[j] = B == 16 && chunk >= 2;
    }
  }
  // The physical block ids of key tile t (two when B = 16: the tile spans two blocks).
  struct Ids { uint32_t a, b; };
  auto ids_of = [&](int t) -> Ids {
    const int lb0 = (32 * t) / B;
    const uint32_t a = block_id(lb0);
    return Ids{a, B == 16 ? block_id(lb0 + 1) : a};
  };
  // A block of a pool is 2 * blk_stride bytes, which fits 32 bits (num_q_heads <= 65535 bounds
  // the KV heads), so a lane's address is one 32 x 32 -> 64-bit multiply-add.
  const uint32_t blk_bytes = 2u * blk_stride;
  auto issue_ids = [&](int t, int stage, Ids id) {
    unsigned char* st = smem + stage * STAGE;
    // (The source pointer is a named variable: given a conditional expression directly, the
    // builtin makes clang drop this kernel's host-side launch stub without a diagnostic.)
#pragma unroll
    for (int j = 0; j < LPT; ++j) {
      const uint32_t bid = (B == 16 && ssel[j]) ? id.b : id.a;
      const char* src = lsrc[j] + static_cast<uint64_t>(bid) * blk_bytes;
      __builtin_amdgcn_global_load_lds(src, st + (LPT * wave + j) * 1024, 16, 0, 0);
    }
  };
  auto issue = [&](int t) { issue_ids(t, t % NS, ids_of(t)); };

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;
  float m = -INFINITY;
  // (m + 8) / scale_log2: the raw score past which the reference max moves
  float m_grow_raw = -INFINITY;
  const float inv_scale_log2 = 1.0f / scale_log2;
  float l[2] = {0.f, 0.f};  // row sum, in two halves that the dot2 chains extend
  const int qpos = r + my_i;           // this lane's query position
  const int wq_lo = r + w_tok0;        // the wave's first query position
  const int klim = min(qpos, n - 1);   // last visible key of this row
  // MFMA row of the K operand -> key within the tile: lane half hb gets keys 16*hb + i.
  const int krow = 16 * ((col >> 2) & 1) + 4 * (col >> 3) + (col & 3);
  const int kbase = krow * KROW;
  const int kx = kswz<D>(krow);
  const int vx = vswz(col);

  auto compute = [&](int t, int stage) {
    const int key0 = 32 * t;
    if (!wave_active || key0 > wq_lo + 31) return;  // wholly above the diagonal
    const unsigned char* st = smem + stage * STAGE;
    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
    u32x4 ka[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      ka[kk] = *reinterpret_cast<const u32x4*>(st + kbase + 16 * ((2 * kk + hb) ^ kx));
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) sacc = mfma32x32x16(ka[kk], qf[kk], sacc);
    // Scores stay in raw units until the exponential: the row max is taken on the raw values
    // (scale_log2 >= 0 keeps the order) and p = 2^(raw * scale_log2 - m) is one fma.
    // The V operands are read from LDS now, while the score products finish.
    u32x4 va[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const unsigned char* vrow = st + K_BYTES + (32 * dt + col) * 64;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        va[dt][j] = *reinterpret_cast<const u32x4*>(vrow + 16 * ((2 * hb + j) ^ vx));
    }
    const bool edge = key0 + 31 > wq_lo || key0 + 31 >= n;  // diagonal or past the context
    if (edge) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (key0 + 16 * hb + i > klim) sacc[i] = -INFINITY;
    }
    // (IEEE maximum: a NaN score makes the row NaN either way, and this form needs no
    // canonicalising of the MFMA results before the three-input max instructions)
    float rmax = sacc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) rmax = __builtin_elementwise_maximum(rmax, sacc[i]);
    // Lazy rescaling: keep the old reference max unless the row's max grows by more than 2^8,
    // so exponentials stay <= 256 and the output is rescaled only rarely. Each lane half tests
    // its own 16 keys in raw units (a row grows exactly when one of its halves does); only
    // then are the halves combined and scaled.
    if (__builtin_amdgcn_ballot_w64(rmax > m_grow_raw)) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(rmax),
                                                      __float_as_uint(rmax), false, false);
      const float row_raw =
          __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
      const bool grow = row_raw > m_grow_raw;
      const float mnew = grow ? row_raw * scale_log2 : m;
      const float alpha = fast_exp2(m - mnew);
      m = mnew;
      m_grow_raw = (mnew + 8.0f) * inv_scale_log2;
      l[0] *= alpha;
      l[1] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
    }
    // The row sum takes the bf16-rounded weights that the P.V product uses, two per dot2; the
    // dot2 chains extend the two halves of the running sum directly.
    float* psum = l;
    u32x4 pb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float p0 = fast_exp2(__builtin_fmaf(sacc[8 * j + 2 * w], scale_log2, -m));
        const float p1 = fast_exp2(__builtin_fmaf(sacc[8 * j + 2 * w + 1], scale_log2, -m));
        const bf16x2 pp = __builtin_convertvector((f32x2{p0, p1}), bf16x2);
        pb[j][w] = __builtin_bit_cast(uint32_t, pp);
        psum[j] = __builtin_amdgcn_fdot2_f32_bf16(pp, bf16x2{1.0f, 1.0f}, psum[j], false);
      }

    const int vlim = n - key0;  // keys at or past n may hold stale words: clear their V
    if (vlim < 32) {
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

  // Pipeline: the ring advances TPB tiles per workgroup barrier. A wave waits for its DMAs of
  // tiles t .. t+TPB-1, leaving the tiles issued after them in flight; the barrier publishes
  // those tiles and frees the stages of the TPB tiles computed before it, into which tiles
  // t+NS-TPB .. t+NS-1 are issued, each just before one of the tiles t .. t+TPB-1 is computed
  // (so the waves' DMA issues spread over the iteration instead of all following the barrier).
  // Fewer barriers per tile than one per tile, with up to NS-TPB tiles in flight. The block ids
  // of the tiles to issue are loaded before the wait, so their scalar loads overlap it.
  constexpr int TPB = kTilesPerBarrier;
  constexpr int PRE = NS - TPB;  // tiles issued ahead of the loop
  static_assert(PRE - TPB >= 0 && PRE - TPB <= 4, "one wait per possible depth below");
#pragma unroll
  for (int t = 0; t < PRE; ++t)
    if (t < ntiles) issue(t);
  // The loop runs once around the ring per outer iteration, unrolled, so that every tile's stage
  // is a compile-time constant: the LDS reads then take the stage as an immediate offset instead
  // of an address add per read.
  static_assert(NS % TPB == 0, "the unrolled ring visits every stage");
  for (int t0 = 0; t0 < ntiles; t0 += NS) {
#pragma unroll
    for (int kb = 0; kb < NS; kb += TPB) {
      const int t = t0 + kb;
      if (t >= ntiles) break;
      Ids nid[TPB];  // (ids_of clamps past the context, so this is safe for any t)
#pragma unroll
      for (int k = 0; k < TPB; ++k) nid[k] = ids_of(t + PRE + k);
      // issued so far: tiles 0 .. min(t + PRE, ntiles) - 1; needed now: t .. t+TPB-1
      const int ahead = min(t + PRE, ntiles) - min(t + TPB, ntiles);
      if (ahead >= 4) __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * LPT));
      else if (ahead == 3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * LPT));
      else if (ahead == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LPT));
      else if (ahead == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPT));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int k = 0; k < TPB; ++k) {
        if (t + PRE + k < ntiles) issue_ids(t + PRE + k, (kb + PRE + k) % NS, nid[k]);
        if (t + k < ntiles) compute(t + k, kb + k);
      }
    }
  }

  if (!wave_active) return;
  const float lsum = xor32_sum(l[0] + l[1]);
  if (!row_valid) return;
  const float inv = 1.0f / lsum;
  OutT* o = out + (static_cast<int64_t>(q0 + my_i) * Hq + head) * D + 4 * hb;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      store_out(o + 32 * dt + 8 * (i >> 2) + (i & 3), acc[dt][i] * inv);
}

// The kernel takes a positive scale (a negative one flips q; zero becomes a tiny positive value,
// which keeps masked scores at -inf and gives the uniform softmax of a zero scale).
template <int D, int B, typename OutT>
static hipError_t launch_t(const PrefillArgs& a, hipStream_t st) {
  const int G = a.Hq / a.Hkv;
  const int HW = (G % 4 == 0) ? 4 : (G % 2 == 0 ? 2 : 1);
  const int WGT = 32 * (kPrefillWaves / HW);
  const int n_tiles = (a.max_q_len + WGT - 1) / WGT;
  const int n_groups = G / HW;
  dim3 grid(n_tiles, a.Hkv * n_groups, a.S);
  return launch_kernel(K_PREFILL, prefill_bf16_kernel<D, B, OutT>, dim3(grid),
      dim3(64 * kPrefillWaves), st,
      static_cast<OutT*>(a.out), static_cast<const uint16_t*>(a.q), a.cu_q_lens, a.context_lens,
      static_cast<const uint16_t*>(a.k_pool), static_cast<const uint16_t*>(a.v_pool), a.block_table,
      a.Hq, a.Hkv, G, HW, a.MB, n_tiles, n_groups, fmaxf(fabsf(a.scale) * kLog2eP, 1e-30f),
      a.scale < 0.f ? 1 : 0);
}

template <int D, int B>
static hipError_t launch_out(const PrefillArgs& a, hipStream_t st) {
  if (a.bf16_out) return launch_t<D, B, uint16_t>(a, st);
  return launch_t<D, B, float>(a, st);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.total_q == 0 || a.max_q_len == 0) return hipSuccess;
  if (!a.bf16_in) return launch_prefill_f32(a, st);
  if (a.D == 128) return a.B == 16 ? launch_out<128, 16>(a, st) : launch_out<128, 32>(a, st);
  return a.B == 16 ? launch_out<64, 16>(a, st) : launch_out<64, 32>(a, st);
}

}  // namespace pkv
