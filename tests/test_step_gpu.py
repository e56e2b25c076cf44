"""GPU parity of the fused decode step (kv_cache_write_and_decode): the pools after the call
equal the oracle's kv_cache_write bit for bit, and the output equals the oracle's decode over
the written pools within the bf16 tolerance."""
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


CASES = [
    # name, seed, S, Hq, Hkv, D, B, lens
    ("g4_edges", 401, 9, 32, 8, 128, 16, [1, 15, 16, 17, 31, 32, 33, 700, 64]),
    ("g8_b32", 402, 4, 64, 8, 128, 32, [1, 32, 33, 1500]),
    ("g1_d64", 403, 3, 16, 16, 64, 16, [5, 100, 64]),
    ("g20_two_groups", 404, 2, 40, 2, 64, 16, [50, 300]),
    ("zero_and_one", 405, 5, 32, 8, 128, 16, [0, 40, 0, 1, 600]),
    ("g2_d64_b32", 406, 3, 8, 4, 64, 32, [96, 97, 1]),
]


@functools.lru_cache(maxsize=None)
def _case(name):
    c = next(c for c in CASES if c[0] == name)
    _, seed, S, hq, hkv, d, b, lens = c
    w = wl.build_decode(seed, S, hq, hkv, d, b, lens, "bf16")
    return w, _ref(w)


def _ref(w):
    kp, vp = orc.kv_cache_write(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping,
                                w.block_size)
    return kp, vp, orc.decode(w.q, kp, vp, w.block_table, w.context_lens, w.scale, "bf16")


def _step(w, out_dtype="bf16", workspace=None, pools=None, num_waves=0):
    import torch
    tk, tv = pools if pools is not None else (to_dev(w.k_pool), to_dev(w.v_pool))
    td = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = torch.full(w.q.shape, float("nan"), dtype=td, device="cuda")
    bd.kv_cache_write_and_decode(out, to_dev(w.q), to_dev(w.k_new), to_dev(w.v_new),
                                 to_dev(w.slot_mapping), tk, tv, to_dev(w.block_table),
                                 to_dev(w.context_lens), w.scale,
                                 max_context_len=max(w.max_context_len, 1), workspace=workspace,
                                 num_waves=num_waves)
    return out, tk, tv


def _workspace(w):
    import torch
    need = bd.decode_workspace_size(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                    max(w.max_context_len, 1), 0, bd.PKV_BF16)
    return torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")  # contents are ignored


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name", [c[0] for c in CASES])
def test_step_small(name, out_dtype):
    w, (kp, vp, ref) = _case(name)
    log(f"write_and_decode {name} out={out_dtype}")
    out, tk, tv = _step(w, out_dtype, _workspace(w))
    assert np.array_equal(bits(tk), kp) and np.array_equal(bits(tv), vp)
    assert_close(values(out), ref, TOL_BF16, f"write_and_decode {name}")


@pytest.mark.parametrize("waves", [1, 7, 64, 333, 4096])
def test_step_wave_counts(waves):
    """Few waves (long pieces) and many (rows split into many merged pieces)."""
    w, (kp, vp, ref) = _case("g8_b32")
    ws = _workspace(w)
    for rep in range(3):  # the same workspace, reused
        out, tk, tv = _step(w, "f32", ws, num_waves=waves)
        assert_close(values(out), ref, TOL_BF16, f"waves={waves} call {rep}")


def test_step_negative_slots_read_the_pool():
    """A negative slot means the pool already holds the newest token: the result is plain
    decode over the pool (written beforehand here by the separate write)."""
    w, (kp, vp, ref) = _case("g4_edges")
    tk, tv = to_dev(kp), to_dev(vp)
    import copy
    w2 = copy.copy(w)
    w2.slot_mapping = np.where(np.arange(w.num_seqs) % 2 == 0, -1, w.slot_mapping).astype(np.int32)
    out, tk, tv = _step(w2, "f32", _workspace(w), pools=(tk, tv))
    assert np.array_equal(bits(tk), kp) and np.array_equal(bits(tv), vp)
    assert_close(values(out), ref, TOL_BF16, "negative slots")


@pytest.mark.parametrize("k", [2, 3, 4])
def test_step_full_config(k):
    w = wl.make_config(k)
    log(f"write_and_decode config {k}")
    kp, vp, ref = _ref(w)
    ws = _workspace(w)
    out, tk, tv = _step(w, "bf16", ws)
    assert np.array_equal(bits(tk), kp) and np.array_equal(bits(tv), vp)
    assert_close(values(out), ref, TOL_BF16, f"write_and_decode config {k}")
    out2, _, _ = _step(w, "bf16", ws)  # pools already hold the tokens; same inputs again
    assert np.array_equal(bits(out2), bits(out)), "a second call on the same workspace differs"
