"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that every one of
them makes at least one pin fail. This is what makes the pins worth trusting."""
import inspect
import types

import pytest

from oracle import paged_attention as orc
from oracle_pins import PINS

SOURCE = inspect.getsource(orc)

# (name, text in the oracle, replacement). Each text must occur in the oracle exactly once.
MUTANTS = [
    ("gqa_mod_instead_of_div", "            g = h // group\n            out[s, h] = attend",
     "            g = h % hkv\n            out[s, h] = attend"),
    ("scale_dropped", "a = scale * (k @ qrow)", "a = (k @ qrow)"),
    ("normalise_by_max", "return (p @ v) / p.sum()", "return (p @ v) / p.max()"),
    ("causal_off_by_one", "k[g, : last + 1], v[g, : last + 1]", "k[g, : last], v[g, : last]"),
    ("causal_top_left", "last = r + i  # keys", "last = i  # keys"),
    ("table_order_ignored", "ids = [int(x) for x in bt_row[:nbk]]",
     "ids = sorted(int(x) for x in bt_row[:nbk])"),
    ("v_layout_not_transposed", "to_f64(v_pool[i], dtype).transpose(0, 2, 1)",
     "to_f64(v_pool[i], dtype).transpose(0, 1, 2)"),
    ("last_block_not_truncated", "return k[:, :n, :], v[:, :n, :]", "return k, v"),
    ("write_k_into_v", "v_pool[blk, :, :, off] = v_new[i]", "v_pool[blk, :, :, off] = k_new[i]"),
    ("write_offset_swapped", "blk, off = divmod(slot, b)", "off, blk = divmod(slot, b)"),
    ("bf16_shift", "(a.astype(np.uint32) << np.uint32(16))",
     "(a.astype(np.uint32) << np.uint32(15))"),
    ("query_uses_kv_head", "out[s, h] = attend(qf[s, h], k[g], v[g], scale)",
     "out[s, h] = attend(qf[s, g], k[g], v[g], scale)"),
    ("context_len_excludes_current", "        n = int(context_lens[s])\n        if n == 0:\n            continue",
     "        n = int(context_lens[s]) - 1\n        if n <= 0:\n            continue"),
    ("brute_gqa", "            g = h * hkv // hq\n            qv", "            g = h % hkv\n            qv"),
    ("brute_offset", "                off = j % b\n                acc = 0.0\n                for x in range(d):\n                    acc += qv[x]",
     "                off = (j + 1) % b\n                acc = 0.0\n                for x in range(d):\n                    acc += qv[x]"),
    ("row_helper_gqa", "    g = h // (hq // hkv)\n    return attend", "    g = h % hkv\n    return attend"),
    ("copy_v_from_k", "dst_v[d_blk] = src_v[s_blk]", "dst_v[d_blk] = src_k[s_blk].reshape(dst_v[d_blk].shape)"),
    ("copy_direction", "dst_k[d_blk] = src_k[s_blk]", "dst_k[s_blk % dst_k.shape[0]] = src_k[d_blk % src_k.shape[0]]"),
    ("copy_k_skipped", "        dst_k[d_blk] = src_k[s_blk]\n", "        pass\n"),
    ("fp8_bias", "np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    ("fp8_subnormal_scale", "f / 8.0 * 2.0 ** -6", "f / 8.0 * 2.0 ** -7"),
    ("fp8_ties_up", "np.where(lo % 2 == 0, lo, hi)", "hi"),
    ("fp8_nan_code", "(e == 15) & (f == 7)", "(e == 15) & (f == 6)"),
    ("fp8_negative_zero", "np.where(np.signbit(x.reshape(-1)), 0x80, 0)",
     "np.where(x.reshape(-1) < 0, 0x80, 0)"),
    ("fp8_write_multiplies", "to_f64(k_new, in_dtype).astype(np.float32) / ks",
     "to_f64(k_new, in_dtype).astype(np.float32) * ks"),
    ("fp8_v_scale_from_k", "return k * k_scale, v * v_scale", "return k * k_scale, v * k_scale"),
    ("prefill_rows_selection", "if wanted is not None and (lo + i, h) not in wanted:",
     "if wanted is not None and (i, h) not in wanted:"),
    # the whole-chunk (matrix) form of the prefill
    ("chunk_mask_off_by_one", "np.arange(n)[None, :] <= (r + np.arange(c))[:, None]",
     "np.arange(n)[None, :] < (r + np.arange(c))[:, None]"),
    ("chunk_mask_top_left", "np.arange(n)[None, :] <= (r + np.arange(c))[:, None]",
     "np.arange(n)[None, :] <= np.arange(c)[:, None]"),
    ("chunk_gqa_mod", "                g = h // group\n                a = np.where",
     "                g = h % hkv\n                a = np.where"),
    ("chunk_scale_dropped", "np.where(keep, scale * (qf[lo:hi, h] @ k[g].T), -np.inf)",
     "np.where(keep, qf[lo:hi, h] @ k[g].T, -np.inf)"),
    ("chunk_normalise_by_max", "(p @ v[g]) / p.sum(axis=1, keepdims=True)",
     "(p @ v[g]) / p.max(axis=1, keepdims=True)"),
    ("chunk_softmax_over_rows", "p = np.exp(a - a.max(axis=1, keepdims=True))",
     "p = np.exp(a - a.max(axis=0, keepdims=True))"),
]


def _mutant(old, new):
    assert SOURCE.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SOURCE.replace(old, new), "<oracle mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    mod = _mutant(old, new)
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except Exception as e:  # an assertion or a crash both count as caught
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"planted mistake {name!r} passed every pin"
