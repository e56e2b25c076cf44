"""Seeded synthetic workloads for the paged-attention calls.

This module only builds inputs: context lengths, a block allocation, block tables, slot
mappings, and pools of N(0, 1) values. It does none of the attention arithmetic, so the tests and
the benchmark can hand the same arrays both to the HIP library and to the CPU oracle.

Shapes follow the workloads the pages describe: Llama-3-style grouped-query decode with mixed
context lengths, shared system-prompt prefixes, and chunked prefill ("LLM Serving Engine
Shootout" 2.1 and 3.1; "Inference Engines: vLLM, SGLang, TensorRT-LLM", "PagedAttention" and
"Prefix caching"; "Serving Engines", "How vLLM works"). No dataset, token or weight is involved.

Array conventions are those of the C ABI: k_pool [NB][Hkv][B][D], v_pool [NB][Hkv][D][B];
"bf16" arrays are uint16 bit patterns, "f32" arrays are float32.

Allocation recipe (shared by every builder):
  * blocks needed by a sequence of n tokens: ceil(n / B); a shared prefix of P tokens (P a
    multiple of B) is P / B physical blocks named by every table;
  * pool size NB = ceil(1.1 * distinct blocks) unless given;
  * physical ids are handed out in order from one seeded permutation of range(NB), shared
    prefix first, then sequence by sequence in logical order;
  * block-table entries past a sequence's last block are -1;
  * every slot that holds no token of any sequence is NaN (so a read of a stale slot shows up),
    including the slots the new tokens will be written to.
Random draws, in order, from numpy.random.default_rng(seed): the lengths (by the config
functions), the permutation, the K pool, the V pool, q, the new K rows, the new V rows.

E4M3 pools (kv_dtype "fp8") hold codes drawn directly, field by field: a uniform sign bit, an
exponent field uniform in 8..12 (2% of elements get exponent field 0: zeros and subnormals),
a uniform 3-bit fraction; with the pool scale 1/16 the values lie within about +-0.06..3.75,
the spread of N(0, 1) rows. Unused slots hold the NaN code 0x7F. q and the new rows are bf16
N(0, 1) values; the new rows are quantised by the library's own write.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
FP8_NAN = np.uint8(0x7F)
FP8_POOL_SCALE = 1.0 / 16.0


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, rounding to nearest, ties to even (IEEE 754 rounding of
    the 24-bit significand to 8 bits). NaN maps to the canonical quiet NaN 0x7FC0."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    r[np.isnan(x)] = BF16_NAN
    return r


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """Inputs of one decode step or one prefill chunk, as host arrays."""
    kind: str                      # "decode" or "prefill"
    dtype: str                     # "f32" or "bf16"
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    scale: float
    q: np.ndarray                  # [S][Hq][D] or [Tq][Hq][D]
    k_pool: np.ndarray             # before the write of the new tokens
    v_pool: np.ndarray
    k_new: np.ndarray              # [T][Hkv][D] rows written by kv_cache_write
    v_new: np.ndarray
    slot_mapping: np.ndarray       # int32 [T]
    block_table: np.ndarray        # int32 [S][MB]
    context_lens: np.ndarray       # int32 [S], includes the new tokens
    cu_q_lens: np.ndarray | None = None   # int32 [S+1] (prefill)
    prefix_tokens: int = 0
    shared_blocks: int = 0
    name: str = ""
    meta: dict = field(default_factory=dict)
    kv_dtype: str = ""             # pool element type when it differs from dtype ("fp8")
    k_scale: float = 1.0           # E4M3 pools: value = code value * scale
    v_scale: float = 1.0

    @property
    def pool_dtype(self) -> str:
        return self.kv_dtype or self.dtype

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def max_q_len(self) -> int:
        if self.cu_q_lens is None:
            return 1
        return int(np.diff(self.cu_q_lens).max()) if self.num_seqs else 0

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])


def _allocate(rng, lens, block_size, prefix_tokens, num_blocks, max_blocks):
    """Block tables for sequences of `lens` tokens sharing `prefix_tokens` leading tokens."""
    assert prefix_tokens % block_size == 0
    shared = prefix_tokens // block_size
    per_seq = [max(0, -(-int(n) // block_size)) for n in lens]
    for n in lens:
        assert prefix_tokens == 0 or n > prefix_tokens
    private = [nb - shared if prefix_tokens else nb for nb in per_seq]
    distinct = (shared if len(lens) else 0) + sum(private)
    if num_blocks is None:
        num_blocks = max(1, math.ceil(1.1 * distinct))
    assert num_blocks >= distinct, "pool too small"
    if max_blocks is None:
        max_blocks = max(per_seq) if per_seq else 1
        max_blocks = max(max_blocks, 1)
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = np.full((len(lens), max_blocks), -1, dtype=np.int32)
    shared_ids = perm[:shared]
    nxt = shared
    for s, nb in enumerate(per_seq):
        assert nb <= max_blocks
        if prefix_tokens:
            bt[s, :shared] = shared_ids
            bt[s, shared:nb] = perm[nxt: nxt + nb - shared]
            nxt += nb - shared
        else:
            bt[s, :nb] = perm[nxt: nxt + nb]
            nxt += nb
    return bt, num_blocks, max_blocks, shared


def _fill_pools(rng, bt, lens, new_from, hkv, d, b, nb, dtype):
    """Pools of N(0,1) where a token lives, NaN elsewhere. Token positions >= new_from[s] of
    sequence s are the ones about to be written, so they start as NaN too."""
    k = rng.standard_normal((nb, hkv, b, d), dtype=np.float32)
    v = rng.standard_normal((nb, hkv, d, b), dtype=np.float32)
    live = np.zeros((nb, b), dtype=bool)
    for s, n in enumerate(lens):
        upto = int(new_from[s])
        for j in range(0, upto, b):
            blk = int(bt[s, j // b])
            live[blk, : min(b, upto - j)] = True
    dead_k = ~live[:, None, :, None]
    dead_v = ~live[:, None, None, :]
    if dtype == "fp8":
        kc, vc = fp8_codes(rng, k.shape), fp8_codes(rng, v.shape)
        np.copyto(kc, FP8_NAN, where=np.broadcast_to(dead_k, k.shape))
        np.copyto(vc, FP8_NAN, where=np.broadcast_to(dead_v, v.shape))
        return kc, vc
    np.copyto(k, np.float32(np.nan), where=np.broadcast_to(dead_k, k.shape))
    np.copyto(v, np.float32(np.nan), where=np.broadcast_to(dead_v, v.shape))
    if dtype == "bf16":
        return bf16_bits(k), bf16_bits(v)
    return k, v


def fp8_codes(rng, shape) -> np.ndarray:
    """Random E4M3 codes drawn field by field (see the module notes); never NaN."""
    sign = rng.integers(0, 2, shape, dtype=np.uint8)
    expo = rng.integers(8, 13, shape, dtype=np.uint8)
    expo[rng.random(shape) < 0.02] = 0
    frac = rng.integers(0, 8, shape, dtype=np.uint8)
    return ((sign << 7) | (expo << 3) | frac).astype(np.uint8)


def _values(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return bf16_bits(x) if dtype == "bf16" else x


def _slots(bt, positions_per_seq, b):
    out = []
    for s, positions in enumerate(positions_per_seq):
        for j in positions:
            out.append(int(bt[s, j // b]) * b + j % b)
    return np.asarray(out, dtype=np.int32)


def build_decode(seed, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, lens,
                 dtype="bf16", prefix_tokens=0, num_blocks=None, max_blocks=None, name="",
                 rng=None, kv_dtype=""):
    """One decode step: sequence s has lens[s] tokens, the last of which is new (written by
    kv_cache_write before attention). A zero length has no new token (slot -1).
    kv_dtype "fp8": E4M3 pools with scale FP8_POOL_SCALE (q and new rows stay in dtype)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    lens = np.asarray(lens, dtype=np.int32)
    assert len(lens) == num_seqs
    assert kv_dtype in ("", "fp8") and (kv_dtype == "" or dtype == "bf16")
    bt, nb, mb, shared = _allocate(rng, lens, block_size, prefix_tokens, num_blocks, max_blocks)
    new_from = np.maximum(lens - 1, 0)
    k_pool, v_pool = _fill_pools(rng, bt, lens, new_from, num_kv_heads, head_dim, block_size,
                                 nb, kv_dtype or dtype)
    q = _values(rng, (num_seqs, num_q_heads, head_dim), dtype)
    k_new = _values(rng, (num_seqs, num_kv_heads, head_dim), dtype)
    v_new = _values(rng, (num_seqs, num_kv_heads, head_dim), dtype)
    slots = np.full(num_seqs, -1, dtype=np.int32)
    for s, n in enumerate(lens):
        if n > 0:
            j = int(n) - 1
            slots[s] = int(bt[s, j // block_size]) * block_size + j % block_size
    sc = FP8_POOL_SCALE if kv_dtype == "fp8" else 1.0
    return Workload("decode", dtype, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                    nb, mb, 1.0 / math.sqrt(head_dim), q, k_pool, v_pool, k_new, v_new, slots,
                    bt, lens, None, prefix_tokens, shared, name, kv_dtype=kv_dtype, k_scale=sc,
                    v_scale=sc)


def build_grouped_decode(seed, groups, num_q_heads, num_kv_heads, head_dim, block_size,
                         dtype="bf16", kv_dtype="", name="", rng=None):
    """One decode step over groups of consecutive sequences that share prompt prefixes.
    `groups` is a list of (prefix_tokens, [context lengths of the members]); prefix_tokens is a
    multiple of B and at most each member's length. Each group's prefix blocks are allocated
    once and named by every member's table; the rest of each context has private blocks. A
    member whose context is exactly the prefix has no new token (its last token sits in a shared
    block). meta holds group_start [G+1] and group_prefix_len [G] (int32)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    b = block_size
    lens, prefix_of, starts, plens = [], [], [0], []
    for pre, members in groups:
        assert pre % b == 0 and all(n >= pre for n in members)
        lens += [int(n) for n in members]
        prefix_of += [pre] * len(members)
        starts.append(starts[-1] + len(members))
        plens.append(pre)
    lens = np.asarray(lens, dtype=np.int32)
    S = len(lens)
    per_seq = [-(-int(n) // b) for n in lens]
    distinct = sum(pre // b for pre, _ in groups) + sum(
        nb - p // b for nb, p in zip(per_seq, prefix_of))
    num_blocks = max(1, math.ceil(1.1 * distinct))
    mb = max(max(per_seq), 1)
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = np.full((S, mb), -1, dtype=np.int32)
    nxt = 0
    for gi, (pre, members) in enumerate(groups):
        shared = perm[nxt: nxt + pre // b]
        nxt += pre // b
        for s in range(starts[gi], starts[gi + 1]):
            bt[s, : pre // b] = shared
            own = per_seq[s] - pre // b
            bt[s, pre // b: per_seq[s]] = perm[nxt: nxt + own]
            nxt += own
    new = np.asarray([n > p for n, p in zip(lens, prefix_of)])
    new_from = np.where(new, lens - 1, lens)
    k_pool, v_pool = _fill_pools(rng, bt, lens, new_from, num_kv_heads, head_dim, b, num_blocks,
                                 kv_dtype or dtype)
    q = _values(rng, (S, num_q_heads, head_dim), dtype)
    k_new = _values(rng, (S, num_kv_heads, head_dim), dtype)
    v_new = _values(rng, (S, num_kv_heads, head_dim), dtype)
    slots = np.full(S, -1, dtype=np.int32)
    for s in range(S):
        if new[s]:
            j = int(lens[s]) - 1
            slots[s] = int(bt[s, j // b]) * b + j % b
    sc = FP8_POOL_SCALE if kv_dtype == "fp8" else 1.0
    meta = {"group_start": np.asarray(starts, np.int32),
            "group_prefix_len": np.asarray(plens, np.int32)}
    return Workload("decode", dtype, S, num_q_heads, num_kv_heads, head_dim, b, num_blocks, mb,
                    1.0 / math.sqrt(head_dim), q, k_pool, v_pool, k_new, v_new, slots, bt, lens,
                    None, max(plens) if plens else 0, 0, name, meta, kv_dtype=kv_dtype,
                    k_scale=sc, v_scale=sc)


def build_prefill(seed, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, prior_lens,
                  chunk_lens, dtype="bf16", prefix_tokens=0, num_blocks=None, max_blocks=None,
                  name="", rng=None):
    """One chunked-prefill call: sequence s has prior_lens[s] cached tokens followed by a
    chunk of chunk_lens[s] new tokens whose K/V kv_cache_write stores first."""
    rng = np.random.default_rng(seed) if rng is None else rng
    prior = np.asarray(prior_lens, dtype=np.int32)
    chunk = np.asarray(chunk_lens, dtype=np.int32)
    lens = prior + chunk
    bt, nb, mb, shared = _allocate(rng, lens, block_size, prefix_tokens, num_blocks, max_blocks)
    k_pool, v_pool = _fill_pools(rng, bt, lens, prior, num_kv_heads, head_dim, block_size, nb,
                                 dtype)
    tq = int(chunk.sum())
    q = _values(rng, (tq, num_q_heads, head_dim), dtype)
    k_new = _values(rng, (tq, num_kv_heads, head_dim), dtype)
    v_new = _values(rng, (tq, num_kv_heads, head_dim), dtype)
    slots = _slots(bt, [range(int(r), int(r) + int(c)) for r, c in zip(prior, chunk)],
                   block_size)
    cu = np.zeros(num_seqs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(chunk)
    return Workload("prefill", dtype, num_seqs, num_q_heads, num_kv_heads, head_dim,
                    block_size, nb, mb, 1.0 / math.sqrt(head_dim), q, k_pool, v_pool, k_new,
                    v_new, slots, bt, lens, cu, prefix_tokens, shared, name,
                    {"prior_lens": prior, "chunk_lens": chunk})


# ------------------------------------------------------------------------ the five workloads

CONFIG_NAMES = {
    1: "tiny fp32 decode: 4 seqs, ctx {1,17,33,100}, 8/8 heads, D64, B16, pool 64",
    2: "Llama-3-8B-shaped decode: 64 seqs, ctx U[512,4096], 32/8 heads, D128, B16, bf16",
    3: "Llama-3-70B-shaped decode: 32 seqs, ctx logU[1024,32768], 64/8 heads, D128, B32, bf16",
    4: "shared-prefix decode: 64 seqs, 2000-token shared prefix + U[16,512], 32/8, D128, B16",
    5: "chunked prefill: 8 seqs, 512-token chunk after U[0,8192] cached, 32/8, D128, B16, bf16",
}


def make_config(k: int, seed: int | None = None, kv_dtype: str = "", tp: int = 1) -> Workload:
    """The five workloads, k = 1..5, seeded by default with seed = k. kv_dtype "fp8" gives the
    decode workloads (2, 3, 4) with E4M3 pools and the same lengths and block tables. tp > 1
    gives one GPU's share of a decode workload split by KV head over tp GPUs (tensor
    parallelism): num_kv_heads / tp KV heads and their query heads, the same sequences and
    lengths."""
    seed = k if seed is None else seed
    if kv_dtype:
        assert k in (2, 3, 4), "E4M3 pools are built for the bf16 decode workloads"
    if tp != 1:
        assert k in (2, 3, 4) and 8 % tp == 0, "a KV-head share of the decode workloads"
    rng = np.random.default_rng(seed)
    hq, hkv = 32 // tp, 8 // tp  # workloads 2 and 4
    hq70 = 64 // tp              # workload 3 (8 KV heads as well)
    if k == 1:
        return build_decode(seed, 4, 8, 8, 64, 16, [1, 17, 33, 100], "f32", num_blocks=64,
                            max_blocks=7, name="c1", rng=rng)
    if k == 2:
        lens = rng.integers(512, 4097, 64)
        return build_decode(seed, 64, hq, hkv, 128, 16, lens, "bf16", max_blocks=256, name="c2",
                            rng=rng, kv_dtype=kv_dtype)
    if k == 3:
        lens = np.round(np.exp(rng.uniform(math.log(1024), math.log(32768), 32))).astype(int)
        return build_decode(seed, 32, hq70, hkv, 128, 32, lens, "bf16", max_blocks=1024,
                            name="c3", rng=rng, kv_dtype=kv_dtype)
    if k == 4:
        suffix = rng.integers(16, 513, 64)
        return build_decode(seed, 64, hq, hkv, 128, 16, 2000 + suffix, "bf16",
                            prefix_tokens=2000, max_blocks=157, name="c4", rng=rng,
                            kv_dtype=kv_dtype)
    if k == 5:
        prior = rng.integers(0, 8193, 8)
        return build_prefill(seed, 8, 32, 8, 128, 16, prior, [512] * 8, "bf16", max_blocks=544,
                             name="c5", rng=rng)
    raise ValueError(f"no config {k}")
