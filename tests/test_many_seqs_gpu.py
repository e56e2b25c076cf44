"""GPU parity for batches of more than 64 sequences: the balanced split scans the sequences
64 at a time (one per lane) when it counts tiles, locates a wave's first sequence and records
the per-segment counts, so batches of 130 and 200 ragged contexts (zero lengths included)
exercise the carry from one group of 64 to the next, for every decode entry point."""
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


def _lens(seed, n, hi):
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, hi, n)
    lens[rng.permutation(n)[: n // 10]] = 0  # some empty contexts
    return [int(x) for x in lens]


@functools.lru_cache(maxsize=None)
def _plain(kv):
    w = wl.build_decode(501, 200, 16, 4, 128, 16, _lens(501, 200, 700), "bf16", kv_dtype=kv)
    if kv == "fp8":
        kp, vp = orc.kv_cache_write_fp8(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping,
                                        w.block_size, "bf16", w.k_scale, w.v_scale)
    else:
        kp, vp = orc.kv_cache_write(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping,
                                    w.block_size)
    ref = orc.decode(w.q, kp, vp, w.block_table, w.context_lens, w.scale, "bf16",
                     kv_dtype=kv or None, k_scale=w.k_scale, v_scale=w.v_scale)
    return w, kp, vp, ref


def _out(w, dtype="f32"):
    import torch
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    return torch.full(w.q.shape, float("nan"), dtype=td, device="cuda")


@pytest.mark.parametrize("waves", [0, 97, 3000])
def test_decode_200_sequences(waves):
    w, kp, vp, ref = _plain("")
    log(f"decode 200 seqs, waves={waves or 'default'}")
    out = _out(w)
    bd.paged_attention_decode(out, to_dev(w.q), to_dev(kp), to_dev(vp), to_dev(w.block_table),
                              to_dev(w.context_lens), w.scale, max_context_len=w.max_context_len,
                              num_waves=waves)
    assert_close(values(out), ref, TOL_BF16, f"decode 200 seqs waves={waves}")


def test_decode_fp8_200_sequences():
    w, kp, vp, ref = _plain("fp8")
    out = _out(w)
    bd.paged_attention_decode_fp8(out, to_dev(w.q), to_dev(kp), to_dev(vp),
                                  to_dev(w.block_table), to_dev(w.context_lens), w.scale,
                                  w.k_scale, w.v_scale, max_context_len=w.max_context_len)
    assert_close(values(out), ref, TOL_BF16, "decode fp8 200 seqs")


def test_write_and_decode_200_sequences():
    w, kp, vp, ref = _plain("")
    tk, tv = to_dev(w.k_pool), to_dev(w.v_pool)
    out = _out(w)
    bd.kv_cache_write_and_decode(out, to_dev(w.q), to_dev(w.k_new), to_dev(w.v_new),
                                 to_dev(w.slot_mapping), tk, tv, to_dev(w.block_table),
                                 to_dev(w.context_lens), w.scale,
                                 max_context_len=w.max_context_len)
    assert np.array_equal(bits(tk), kp) and np.array_equal(bits(tv), vp)
    assert_close(values(out), ref, TOL_BF16, "write_and_decode 200 seqs")


def test_shared_prefix_130_sequences():
    rng = np.random.default_rng(502)
    groups = [(96, [96 + int(x) for x in rng.integers(0, 300, 70)]),
              (0, [int(x) for x in rng.integers(0, 200, 25)]),
              (512, [512 + int(x) for x in rng.integers(0, 100, 35)])]
    w = wl.build_grouped_decode(502, groups, 16, 4, 128, 16, "bf16")
    kp, vp = orc.kv_cache_write(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping,
                                w.block_size)
    ref = orc.decode(w.q, kp, vp, w.block_table, w.context_lens, w.scale, "bf16")
    out = _out(w)
    gs, gp = w.meta["group_start"], w.meta["group_prefix_len"]
    bd.paged_attention_decode_shared_prefix(
        out, to_dev(w.q), to_dev(kp), to_dev(vp), to_dev(w.block_table), to_dev(w.context_lens),
        to_dev(gs), to_dev(gp), w.scale, int(np.diff(gs).max()), int(gp.max()),
        max_context_len=w.max_context_len)
    assert_close(values(out), ref, TOL_BF16, "shared prefix 130 seqs")
