"""CPU oracle for paged attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, `__graft_entry__.smoke()` and the bench's CPU-baseline leg may import this module.
The library's product path never calls it, and it shares no code with the HIP kernels, their
host code or their binding.

It is the plain definition of what the paged-attention calls compute, in float64 NumPy, slow
and easy to check by eye. Pages cited (title, then the place on the page):

  [Shootout]          "LLM Serving Engine Shootout: vLLM vs TensorRT-LLM vs SGLang vs
                      llama.cpp" (initnode.dev): 2.1 (GQA: fewer KV heads), 3.1 (physical
                      blocks, block table, and the displayed score equation), 3.2
                      (copy-on-write sharing), 5.1 (the attention steps: Q K^T, softmax, A V).
  [Serving Engines]   "Serving Engines" (inference.tusharamrit.in), "How vLLM works": one
                      pool of fixed-size blocks, block tables, slot mapping, chunked prefill,
                      copy-on-write sharing by pointing tables at the same blocks.
  [Inference Engines] "Inference Engines: vLLM, SGLang, TensorRT-LLM" (ragyfied.com),
                      "PagedAttention": blocks grow with the sequence; two tables may name the
                      same physical block.
  [VRAM black hole]   zhichai.net topic 178634546 (Chinese original), section 1, the ASCII
                      figure: logical tokens 0-15 -> physical block #7, 16-31 -> #2.

Readings taken where the pages are silent (each is listed with its reason in the design doc):
  * offset inside a block = j mod B (the figure's tokens 0-15 / 16-31 split);
  * query head h reads KV head h // (Hq / Hkv);
  * context_len counts every cached token including the current decode token;
  * decode with context_len 0 returns zeros;
  * in a prefill chunk of c rows after r earlier tokens, row i sits at position r + i and
    sees keys 0 .. r + i;
  * softmax is the textbook one: exp(a - max a) / sum exp(a - max a) (a stabilised but exact
    rewrite of exp(a) / sum exp(a)).

  [VRAM black hole 4] the same zhichai.net topic, section 4 (the KV-cache memory formula:
                      FP8 takes one byte per element), and [Serving Engines] "What they all
                      agree on" (engines quantise the KV cache too). The pages fix no FP8
                      detail beyond one byte per element; the readings taken are the OCP 8-bit
                      floating point E4M3 ("fn") element format and one float32 scale per pool
                      (stored code = value / scale).

Array conventions (the same arrays the GPU receives):
  dtype "f32":  float32 arrays.
  dtype "bf16": uint16 arrays holding bf16 bit patterns (NumPy has no bf16 type). The oracle
                decodes them exactly to float64 itself.
  dtype "fp8":  uint8 arrays holding E4M3 codes (pools only; the value of a code is multiplied
                by the pool's scale).
  k_pool [NB][Hkv][B][D]; v_pool [NB][Hkv][D][B]; q [S][Hq][D] (decode) or [Tq][Hq][D]
  (prefill); block_table int32 [S][MB]; context_lens int32 [S]; cu_q_lens int32 [S+1];
  slot_mapping int32 [T].
"""

from __future__ import annotations

import math

import numpy as np


# ----------------------------------------------------------------------------- element types

def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of every element. bf16 is the high half of a binary32 word, so
    shifting its 16 bits up by 16 gives the binary32 with the same value."""
    if dtype == "f32":
        assert a.dtype == np.float32
        return a.astype(np.float64)
    if dtype == "bf16":
        assert a.dtype == np.uint16
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "fp8":
        return fp8_e4m3_value(a)
    if dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def fp8_e4m3_value(codes: np.ndarray) -> np.ndarray:
    """float64 value of E4M3 codes (OCP 8-bit floating point, the "fn" variant): bit 7 the
    sign, bits 6..3 a biased exponent e (bias 7), bits 2..0 a fraction f. e > 0: (1 + f/8) *
    2^(e-7); e == 0: subnormal, f/8 * 2^-6. No infinities; e == 15 with f == 7 is NaN, so the
    largest finite magnitude is 1.75 * 2^8 = 448."""
    c = np.asarray(codes)
    assert c.dtype == np.uint8
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = ((c >> 3) & 0xF).astype(np.int64)
    f = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, f / 8.0 * 2.0 ** -6, (1.0 + f / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (f == 7), np.nan, mag)
    return sign * mag


FP8_E4M3_MAX = 448.0


def fp8_e4m3_encode(x: np.ndarray) -> np.ndarray:
    """E4M3 code of each float32 x: the representable value nearest to x, ties to the code
    with an even last bit (round to nearest even); magnitudes beyond 448 saturate to +-448
    (the reading taken: the cache stays finite, as the format has no infinity). The sign
    bit follows x's sign, so -0.0 and negatives that round to zero give 0x80. NaN gives 0x7F."""
    x = np.asarray(x, dtype=np.float32)
    finite = np.arange(127, dtype=np.uint8)           # non-negative finite codes, ascending
    vals = fp8_e4m3_value(finite)
    assert np.all(np.diff(vals) > 0)
    a = np.abs(x.astype(np.float64)).reshape(-1)
    hi = np.clip(np.searchsorted(vals, a), 1, 126)    # vals[hi-1] <= a <= vals[hi] in range
    lo = hi - 1
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a >= FP8_E4M3_MAX, 126, pick)
    code = pick.astype(np.uint8) | np.where(np.signbit(x.reshape(-1)), 0x80, 0).astype(np.uint8)
    code = np.where(np.isnan(x.reshape(-1)), np.uint8(0x7F), code)
    return code.reshape(x.shape).astype(np.uint8)


# ------------------------------------------------------------------------ kv cache write

def kv_cache_write(k_pool, v_pool, k_new, v_new, slot_mapping, block_size):
    """Scatter new rows into pool slots; returns new (k_pool, v_pool), inputs untouched.

    [Serving Engines, "How vLLM works"]: a new token goes to the slot its slot-mapping entry
    names; slot = physical_block * B + offset [VRAM black hole, section 1 figure]. A pure copy of
    the stored words, so the result is compared bit for bit. Negative slots are skipped.
    """
    k_pool = k_pool.copy()
    v_pool = v_pool.copy()
    nb, hkv, b, d = k_pool.shape
    assert b == block_size and v_pool.shape == (nb, hkv, d, b)
    slots = [int(s) for s in slot_mapping]
    used = [s for s in slots if s >= 0]
    assert len(set(used)) == len(used), "non-negative slots must be distinct"
    for i, slot in enumerate(slots):
        if slot < 0:
            continue
        assert slot < nb * b, "slot outside the pool"
        blk, off = divmod(slot, b)
        k_pool[blk, :, off, :] = k_new[i]
        v_pool[blk, :, :, off] = v_new[i]
    return k_pool, v_pool


def kv_cache_copy_blocks(src_k, src_v, dst_k, dst_v, pairs):
    """Copy whole physical blocks (every KV head, K and V): dst[d] = src[s] for each (s, d).

    ["Serving Engines", How vLLM works]: a copy-on-write fork copies exactly the one block being
    written before the tables split; the same copy between a device pool and a host pool is the
    data movement of swap preemption. Returns new (dst_k, dst_v); the inputs are untouched.
    Source and destination may be the same pool; destinations must be distinct and must not be
    sources of other pairs.
    """
    dst_k = dst_k.copy()
    dst_v = dst_v.copy()
    dsts = [int(d) for _, d in pairs]
    assert len(set(dsts)) == len(dsts), "destination blocks must be distinct"
    for s_blk, d_blk in pairs:
        s_blk, d_blk = int(s_blk), int(d_blk)
        assert 0 <= s_blk < src_k.shape[0] and 0 <= d_blk < dst_k.shape[0]
        dst_k[d_blk] = src_k[s_blk]
        dst_v[d_blk] = src_v[s_blk]
    return dst_k, dst_v


def kv_cache_write_fp8(k_pool, v_pool, k_new, v_new, slot_mapping, block_size, in_dtype,
                       k_scale, v_scale):
    """kv_cache_write into E4M3 pools: each new element x (dtype in_dtype, exactly a float32)
    is stored as the code of the float32 quotient x / scale (IEEE division rounded to float32,
    then fp8_e4m3_encode), K with k_scale and V with v_scale. [VRAM black hole 4]: one byte per cached
    element. The codes are then placed exactly as kv_cache_write places words."""
    ks, vs = np.float32(k_scale), np.float32(v_scale)
    kq = fp8_e4m3_encode(to_f64(k_new, in_dtype).astype(np.float32) / ks)
    vq = fp8_e4m3_encode(to_f64(v_new, in_dtype).astype(np.float32) / vs)
    return kv_cache_write(k_pool, v_pool, kq, vq, slot_mapping, block_size)


# ----------------------------------------------------------------------------- gather

def gather(k_pool, v_pool, bt_row, n, block_size, dtype):
    """A sequence's contiguous K and V, float64 [Hkv][n][D] each.

    [Shootout 3.1]: logical block i of the sequence is physical block bt_row[i]; concatenating
    the physical blocks in logical order gives the logical view the attention math sees. The
    last block may be partly filled; only its first n - (nb-1)*B tokens are taken.
    """
    nbk = -(-n // block_size)
    nb_pool = k_pool.shape[0]
    if nbk == 0:
        hkv, d = k_pool.shape[1], k_pool.shape[3]
        return np.zeros((hkv, 0, d)), np.zeros((hkv, 0, d))
    ids = [int(x) for x in bt_row[:nbk]]
    assert all(0 <= i < nb_pool for i in ids), "block id outside the pool"
    k = np.concatenate([to_f64(k_pool[i], dtype) for i in ids], axis=1)  # [Hkv][nbk*B][D]
    v = np.concatenate([to_f64(v_pool[i], dtype).transpose(0, 2, 1) for i in ids], axis=1)
    return k[:, :n, :], v[:, :n, :]


# ----------------------------------------------------------------------------- attention

def attend(qrow, k, v, scale):
    """softmax(scale * k @ qrow) @ v for one query row, float64.

    [Shootout 3.1 equation]: a_j = q . k_j / sqrt(d) (scale = 1/sqrt(d) in every workload);
    [Shootout 5.1]: then the softmax of the scores, then their product with V.
    """
    a = scale * (k @ qrow)
    p = np.exp(a - a.max())
    return (p @ v) / p.sum()


def gather_values(k_pool, v_pool, bt_row, n, block_size, kv_dtype, k_scale=1.0, v_scale=1.0):
    """gather() for any pool type: the values of an E4M3 pool are its code values times the
    pool's scale (K with k_scale, V with v_scale); other pools hold values as they are."""
    k, v = gather(k_pool, v_pool, bt_row, n, block_size, kv_dtype)
    if kv_dtype == "fp8":
        return k * k_scale, v * v_scale
    return k, v


def decode(q, k_pool, v_pool, block_table, context_lens, scale, dtype, kv_dtype=None,
           k_scale=1.0, v_scale=1.0):
    """paged_attention_decode: one query token per sequence; float64 [S][Hq][D].
    kv_dtype (default: dtype) may be "fp8": the pools hold E4M3 codes, K's and V's value are
    code value * k_scale and * v_scale; q stays in dtype."""
    s_count, hq, d = q.shape
    hkv = k_pool.shape[1]
    b = k_pool.shape[2]
    assert hq % hkv == 0
    group = hq // hkv  # [Shootout 2.1]: G query heads per KV head, consecutive
    out = np.zeros((s_count, hq, d))
    qf = to_f64(q, dtype)
    for s in range(s_count):
        n = int(context_lens[s])
        if n == 0:
            continue  # reading: an empty context gives a zero row
        k, v = gather_values(k_pool, v_pool, block_table[s], n, b, kv_dtype or dtype, k_scale,
                             v_scale)
        for h in range(hq):
            g = h // group
            out[s, h] = attend(qf[s, h], k[g], v[g], scale)
    return out


def decode_row(q, k_pool, v_pool, block_table, context_lens, scale, dtype, s, h,
               kv_dtype=None, k_scale=1.0, v_scale=1.0):
    """One output row of decode (for sampled comparisons at full size)."""
    hq = q.shape[1]
    hkv, b = k_pool.shape[1], k_pool.shape[2]
    n = int(context_lens[s])
    if n == 0:
        return np.zeros(q.shape[2])
    k, v = gather_values(k_pool, v_pool, block_table[s], n, b, kv_dtype or dtype, k_scale,
                         v_scale)
    g = h // (hq // hkv)
    return attend(to_f64(q[s, h], dtype), k[g], v[g], scale)


def prefill_chunk(q, cu_q_lens, context_lens, k_pool, v_pool, block_table, scale, dtype,
                  rows=None):
    """paged_attention_prefill_chunk; float64 [Tq][Hq][D].

    [Serving Engines, "How vLLM works"]: chunked prefill runs a slice of a prompt. Reading:
    sequence s holds n = context_lens[s] tokens, the last c = cu[s+1] - cu[s] of which are this
    chunk; chunk row i is at position r + i (r = n - c) and attends to keys 0 .. r + i.
    Without `rows`, each (sequence, head) is the textbook masked attention of the whole chunk:
    scores of every chunk row against every key, the causal mask (key j kept for row i iff
    j <= r + i, aligned to the end of the context), a row-wise softmax, then the product with V.
    `rows`, if given, is a list of (token_row, head) pairs: only those are computed, one row at
    a time over its visible keys.
    """
    tq, hq, d = q.shape
    hkv, b = k_pool.shape[1], k_pool.shape[2]
    group = hq // hkv
    out = np.zeros((tq, hq, d))
    qf = to_f64(q, dtype)
    wanted = None if rows is None else set((int(t), int(h)) for t, h in rows)
    for s in range(len(context_lens)):
        lo, hi = int(cu_q_lens[s]), int(cu_q_lens[s + 1])
        c, n = hi - lo, int(context_lens[s])
        r = n - c
        assert c >= 0 and r >= 0, "chunk longer than the context"
        if c == 0:
            continue
        if wanted is not None and not any(lo <= t < hi for t, _ in wanted):
            continue
        k, v = gather(k_pool, v_pool, block_table[s], n, b, dtype)
        if wanted is None:
            keep = np.arange(n)[None, :] <= (r + np.arange(c))[:, None]  # [c][n] causal mask
            for h in range(hq):
                g = h // group
                a = np.where(keep, scale * (qf[lo:hi, h] @ k[g].T), -np.inf)
                p = np.exp(a - a.max(axis=1, keepdims=True))
                out[lo:hi, h] = (p @ v[g]) / p.sum(axis=1, keepdims=True)
            continue
        for i in range(c):
            for h in range(hq):
                if wanted is not None and (lo + i, h) not in wanted:
                    continue
                g = h // group
                last = r + i  # keys 0 .. r+i are visible
                out[lo + i, h] = attend(qf[lo + i, h], k[g, : last + 1], v[g, : last + 1], scale)
    return out


# ------------------------------------------------------------------------ brute force (tiny)

def _elem(pool_words, dtype):
    return float(to_f64(np.asarray([pool_words]), dtype)[0])


def brute_force_decode(q, k_pool, v_pool, block_table, context_lens, scale, dtype):
    """Scalar loops, no gather: every key element is fetched one at a time from its slot,
    slot = block_table[s][j // B] * B + j % B, and the flat pool index is written out from the
    layout. Uses math.exp. For tiny inputs only; independent of gather()/attend()."""
    s_count, hq, d = q.shape
    nb, hkv, b, _ = k_pool.shape
    kf = k_pool.reshape(-1)
    vf = v_pool.reshape(-1)
    out = [[[0.0] * d for _ in range(hq)] for _ in range(s_count)]
    for s in range(s_count):
        n = int(context_lens[s])
        for h in range(hq):
            g = h * hkv // hq
            qv = [_elem(q[s, h, x], dtype) for x in range(d)]
            scores = []
            for j in range(n):
                blk = int(block_table[s][j // b])
                off = j % b
                acc = 0.0
                for x in range(d):
                    acc += qv[x] * _elem(kf[((blk * hkv + g) * b + off) * d + x], dtype)
                scores.append(acc * scale)
            if n == 0:
                continue
            mx = max(scores)
            w = [math.exp(a - mx) for a in scores]
            tot = sum(w)
            for x in range(d):
                acc = 0.0
                for j in range(n):
                    blk = int(block_table[s][j // b])
                    off = j % b
                    acc += w[j] * _elem(vf[((blk * hkv + g) * d + x) * b + off], dtype)
                out[s][h][x] = acc / tot
    return np.asarray(out, dtype=np.float64)


def brute_force_prefill(q, cu_q_lens, context_lens, k_pool, v_pool, block_table, scale, dtype):
    """Scalar-loop chunked prefill for tiny inputs: key j is visible to chunk row i iff
    j <= n - c + i; elements fetched one by one through the block table as above."""
    tq, hq, d = q.shape
    nb, hkv, b, _ = k_pool.shape
    kf = k_pool.reshape(-1)
    vf = v_pool.reshape(-1)
    out = np.zeros((tq, hq, d))
    for s in range(len(context_lens)):
        lo, hi = int(cu_q_lens[s]), int(cu_q_lens[s + 1])
        n = int(context_lens[s])
        for i in range(hi - lo):
            pos = n - (hi - lo) + i
            for h in range(hq):
                g = h * hkv // hq
                scores = []
                for j in range(pos + 1):
                    blk, off = int(block_table[s][j // b]), j % b
                    acc = 0.0
                    for x in range(d):
                        acc += _elem(q[lo + i, h, x], dtype) * _elem(
                            kf[((blk * hkv + g) * b + off) * d + x], dtype)
                    scores.append(acc * scale)
                mx = max(scores)
                w = [math.exp(a - mx) for a in scores]
                tot = sum(w)
                for x in range(d):
                    acc = 0.0
                    for j in range(pos + 1):
                        blk, off = int(block_table[s][j // b]), j % b
                        acc += w[j] * _elem(vf[((blk * hkv + g) * d + x) * b + off], dtype)
                    out[lo + i, h, x] = acc / tot
    return out
