"""GPU parity of the E4M3 KV cache: the quantising write bit for bit against the oracle (every
bf16 input pattern, several scales), the widening of every code through a one-token decode, and
decode over E4M3 pools against the oracle's decode of code value * scale, within the bf16
tolerance (the kernel widens codes to bf16 exactly and accumulates in fp32, as on bf16 pools)."""
import functools

import numpy as np
import pytest

from oracle import paged_attention as orc
from paged_kv_cache_190_amd import binding as bd
from paged_kv_cache_190_amd import workloads as wl

from gpu_util import TOL_BF16, assert_close, bits, log, to_dev, values

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    bd.lib()


def _oracle_written(w):
    return orc.kv_cache_write_fp8(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping,
                                  w.block_size, w.dtype, w.k_scale, w.v_scale)


def _write(w, kp, vp):
    bd.kv_cache_write_fp8(to_dev(w.k_new), to_dev(w.v_new), kp, vp, to_dev(w.slot_mapping),
                          w.k_scale, w.v_scale)


def _decode(w, kp, vp, out_dtype, max_context_len=None, num_waves=0):
    import torch
    td = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = torch.full(w.q.shape, float("nan"), dtype=td, device="cuda")
    mc = w.max_context_len if max_context_len is None else max_context_len
    bd.paged_attention_decode_fp8(out, to_dev(w.q), kp, vp, to_dev(w.block_table),
                                  to_dev(w.context_lens), w.scale, w.k_scale, w.v_scale,
                                  max_context_len=mc, num_waves=num_waves)
    return out


# ------------------------------------------------------------------------------- the write

@pytest.mark.parametrize("scale", [1.0, 0.37, 1.0 / 16, 3e-3, 1e4])
def test_write_fp8_every_bf16_pattern(scale):
    """Each of the 65536 bf16 patterns is quantised once as K and once as V (NaN, infinity,
    subnormals and values far outside the E4M3 range included)."""
    log(f"kv_cache_write_fp8 every bf16 pattern, scale {scale}")
    hkv, d, b, nb = 8, 128, 16, 80
    T = 65536 // (hkv * d)
    pat = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    kn = pat.reshape(T, hkv, d)
    vn = pat[::-1].copy().reshape(T, hkv, d)
    rng = np.random.default_rng(int(scale * 1000) % 997)
    slots = rng.permutation(nb * b)[:T].astype(np.int32)
    k0 = np.full((nb, hkv, b, d), 0xA5, np.uint8)
    v0 = np.full((nb, hkv, d, b), 0x5A, np.uint8)
    ek, ev = orc.kv_cache_write_fp8(k0, v0, kn, vn, slots, b, "bf16", scale, scale)
    tk, tv = to_dev(k0), to_dev(v0)
    bd.kv_cache_write_fp8(to_dev(kn), to_dev(vn), tk, tv, to_dev(slots), scale, scale)
    assert np.array_equal(bits(tk), ek) and np.array_equal(bits(tv), ev)


def test_write_fp8_float32_edges():
    """fp32 inputs at every E4M3 midpoint (ties), just beside them, at the saturation edge,
    and the specials; D = 64, B = 32, one negative slot."""
    hkv, d, b, nb = 2, 64, 32, 12
    vals = orc.fp8_e4m3_value(np.arange(127, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        [447.0, 448.0, 463.99, 464.0, 465.0, 1e30, np.inf, np.nan, -0.0, 1e-45,
                         2.0 ** -10, 3 * 2.0 ** -11]]).astype(np.float32)
    x = np.concatenate([x, -x])
    per_tok = hkv * d
    T = -(-len(x) // per_tok)
    x = np.concatenate([x, np.zeros(T * per_tok - len(x), np.float32)]).reshape(T, hkv, d)
    rng = np.random.default_rng(4)
    slots = rng.permutation(nb * b)[:T].astype(np.int32)
    slots[1] = -1
    k0 = np.zeros((nb, hkv, b, d), np.uint8)
    v0 = np.zeros((nb, hkv, d, b), np.uint8)
    ek, ev = orc.kv_cache_write_fp8(k0, v0, x, x[::-1].copy(), slots, b, "f32", 1.0, 0.5)
    tk, tv = to_dev(k0), to_dev(v0)
    bd.kv_cache_write_fp8(to_dev(x), to_dev(x[::-1].copy()), tk, tv, to_dev(slots), 1.0, 0.5)
    assert np.array_equal(bits(tk), ek) and np.array_equal(bits(tv), ev)


# ---------------------------------------------------------------------------- the widening

def test_every_code_widens_exactly():
    """One-token contexts: the output row is the token's V row times v_scale, exactly, so each
    of the 256 codes (NaN codes give NaN) is checked through the decode kernel's widening."""
    import torch
    S, hq, hkv, d, b = 2, 4, 1, 128, 16
    codes = np.arange(256, dtype=np.uint8).reshape(S, d)
    kp = np.full((4, hkv, b, d), 0x38, np.uint8)
    vp = np.full((4, hkv, d, b), 0x7F, np.uint8)   # every unused slot NaN
    bt = np.asarray([[2], [0]], np.int32)
    for s in range(S):
        vp[bt[s, 0], 0, :, 0] = codes[s]
    q = wl.bf16_bits(np.ones((S, hq, d), np.float32))
    lens = np.asarray([1, 1], np.int32)
    out = torch.full((S, hq, d), -1.0, dtype=torch.float32, device="cuda")
    bd.paged_attention_decode_fp8(out, to_dev(q), to_dev(kp), to_dev(vp), to_dev(bt),
                                  to_dev(lens), 0.1, 1.0, 2.0, max_context_len=1)
    got = values(out)
    want = orc.fp8_e4m3_value(codes) * 2.0
    for h in range(hq):
        assert np.array_equal(np.isnan(got[:, h]), np.isnan(want))
        assert np.array_equal(got[:, h][~np.isnan(want)], want[~np.isnan(want)])


# --------------------------------------------------------------------------------- decode

FP8_CASES = [
    # name, seed, S, Hq, Hkv, D, B, lens
    ("g4_edges", 201, 9, 32, 8, 128, 16, [1, 15, 16, 17, 31, 32, 33, 700, 64]),
    ("g8_b32", 202, 4, 64, 8, 128, 32, [1, 32, 33, 1500]),
    ("g1_d64", 203, 3, 16, 16, 64, 16, [5, 100, 64]),
    ("g16_b32", 204, 3, 32, 2, 128, 32, [200, 63, 64]),
    ("g20_two_groups", 205, 2, 40, 2, 64, 16, [50, 300]),
    ("g3_zero", 206, 3, 6, 2, 128, 16, [77, 0, 9]),
    ("g2_d64_b32", 207, 3, 8, 4, 64, 32, [96, 97, 1]),
]


@functools.lru_cache(maxsize=None)
def _case(name):
    c = next(c for c in FP8_CASES if c[0] == name)
    _, seed, S, hq, hkv, d, b, lens = c
    w = wl.build_decode(seed, S, hq, hkv, d, b, lens, "bf16", kv_dtype="fp8")
    kp, vp = _oracle_written(w)
    ref = orc.decode(w.q, kp, vp, w.block_table, w.context_lens, w.scale, "bf16",
                     kv_dtype="fp8", k_scale=w.k_scale, v_scale=w.v_scale)
    return w, kp, vp, ref


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name", [c[0] for c in FP8_CASES])
def test_decode_fp8_small(name, out_dtype):
    w, kp, vp, ref = _case(name)
    log(f"decode_fp8 {name} out={out_dtype}")
    tk, tv = to_dev(w.k_pool), to_dev(w.v_pool)
    _write(w, tk, tv)
    assert np.array_equal(bits(tk), kp) and np.array_equal(bits(tv), vp)
    out = _decode(w, tk, tv, out_dtype, max_context_len=max(w.max_context_len, 1))
    assert_close(values(out), ref, TOL_BF16, f"decode_fp8 {name} out={out_dtype}")


@pytest.mark.parametrize("waves", [1, 7, 333, 4096])
def test_decode_fp8_wave_counts(waves):
    w, kp, vp, ref = _case("g4_edges")
    tk, tv = to_dev(kp), to_dev(vp)
    out = _decode(w, tk, tv, "f32", num_waves=waves)
    assert_close(values(out), ref, TOL_BF16, f"decode_fp8 waves={waves}")


def _requantised(codes, old_scale, new_scale):
    """The same values held at another pool scale: each code's value (code value * old_scale)
    re-encoded as the E4M3 code of value / new_scale (float32 quotient), by the oracle's
    encoder. NaN codes (the never-written slots) stay NaN."""
    vals = (orc.fp8_e4m3_value(codes) * old_scale).astype(np.float32)
    return orc.fp8_e4m3_encode(vals / np.float32(new_scale))


def test_decode_fp8_scales():
    """Non-power-of-two pool scales, with K and V at the workload's magnitudes: the pools'
    values are re-encoded at each (k_scale, v_scale), so the result stays the size of the
    workload's and the absolute bf16 tolerance applies unchanged. A k_scale or v_scale folded in
    wrongly (or not at all) changes the result by a factor, far beyond the tolerance."""
    w, kp, vp, _ = _case("g8_b32")
    for ks, vs in [(0.3, 0.7), (0.011, 5.0), (1.0 / 3.0, 1.0 / 7.0)]:
        kq = _requantised(kp, w.k_scale, ks)
        vq = _requantised(vp, w.v_scale, vs)
        w2 = wl.Workload(**{**w.__dict__, "k_scale": ks, "v_scale": vs})
        ref = orc.decode(w.q, kq, vq, w.block_table, w.context_lens, w.scale, "bf16",
                         kv_dtype="fp8", k_scale=ks, v_scale=vs)
        assert np.abs(ref).max() < 4.0  # the workload's magnitudes
        got = values(_decode(w2, to_dev(kq), to_dev(vq), "f32"))
        assert_close(got, ref, TOL_BF16, f"scales {ks}, {vs}")


@pytest.mark.parametrize("k", [2, 3, 4])
def test_decode_fp8_full_config(k):
    w = wl.make_config(k, kv_dtype="fp8")
    log(f"decode_fp8 config {k}: S={w.num_seqs} sum n={int(w.context_lens.sum())}")
    kp, vp = _oracle_written(w)
    ref = orc.decode(w.q, kp, vp, w.block_table, w.context_lens, w.scale, "bf16",
                     kv_dtype="fp8", k_scale=w.k_scale, v_scale=w.v_scale)
    tk, tv = to_dev(w.k_pool), to_dev(w.v_pool)
    _write(w, tk, tv)
    assert np.array_equal(bits(tk), kp) and np.array_equal(bits(tv), vp)
    assert_close(values(_decode(w, tk, tv, "bf16")), ref, TOL_BF16, f"fp8 config {k} bf16 out")
    assert_close(values(_decode(w, tk, tv, "f32")), ref, TOL_BF16, f"fp8 config {k} f32 out")


def test_decode_fp8_deterministic_and_copyable():
    """Repeated calls agree bit for bit, and block copies work on E4M3 pools."""
    w, kp, vp, _ = _case("g4_edges")
    tk, tv = to_dev(kp), to_dev(vp)
    first = bits(_decode(w, tk, tv, "bf16"))
    for _ in range(10):
        assert np.array_equal(bits(_decode(w, tk, tv, "bf16")), first)
    free = np.setdiff1d(np.arange(w.num_blocks), w.block_table[w.block_table >= 0])
    assert len(free) >= 2
    pairs = np.asarray([[int(w.block_table[0, 0]), free[0]], [int(w.block_table[7, 2]), free[-1]]],
                       np.int32)
    ek, ev = orc.kv_cache_copy_blocks(kp, vp, kp, vp, pairs)
    bd.kv_cache_copy_blocks(tk, tv, tk, tv, to_dev(pairs))
    assert np.array_equal(bits(tk), ek) and np.array_equal(bits(tv), ev)
