"""Python binding of libpkv (ctypes). Argument marshalling only.

The functions take torch device tensors, check shapes, dtypes and contiguity, and pass raw
device pointers and the current HIP stream to the C ABI declared in include/pkv.h. Every step of
the computation runs in the library's HIP kernels; torch only owns device memory and streams.
The Python names drop the C prefix: kv_cache_write is pkv_kv_cache_write, and so on.

The library must have been built (python -m paged_kv_cache_190_amd.build); loading fails loudly
otherwise. There is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libpkv.so")
# The library built with PKV_DEBUG=1: device-array checks before every call (see include/pkv.h).
DEBUG_LIB_PATH = os.path.join(PKG, "lib", "libpkv_debug.so")

(PKV_OK, PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_WORKSPACE, PKV_ERR_HIP,
 PKV_ERR_OUT_OF_BLOCKS, PKV_ERR_DEVICE_ARG) = range(7)
PKV_F32, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2

_lib = None
_debug_lib = None


class PkvError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libpkv (loaded once)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def debug_lib() -> ctypes.CDLL:
    """The debug build of libpkv (loaded once), with the same C ABI."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _load(DEBUG_LIB_PATH)
    return _debug_lib


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m paged_kv_cache_190_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    L.pkv_debug_build.restype = i32
    L.pkv_debug_found.restype = ctypes.c_uint
    L.pkv_abi_version.restype = i32
    L.pkv_status_string.restype = ctypes.c_char_p
    L.pkv_status_string.argtypes = [i32]
    L.pkv_last_error.restype = ctypes.c_char_p
    L.pkv_kv_cache_write.restype = i32
    L.pkv_kv_cache_write.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    L.pkv_decode_partition_size.restype = i32
    L.pkv_decode_partition_size.argtypes = [i32, i32, i32, i32, i32]
    L.pkv_decode_workspace_size.restype = sz
    L.pkv_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.pkv_paged_attention_decode.restype = i32
    L.pkv_paged_attention_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                             i32, i32, f32, i32, i32, i32, vp, sz, i32, i32, vp]
    L.pkv_paged_attention_prefill_chunk.restype = i32
    L.pkv_paged_attention_prefill_chunk.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                                    i32, i32, i32, i32, i32, f32, i32, i32, i32,
                                                    i32, vp]
    L.pkv_paged_attention_decode_noalloc.restype = i32
    L.pkv_paged_attention_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                     i32, i32, i32, f32, i32, i32, i32, vp]
    L.pkv_decode_read_probe_sink_size.restype = sz
    L.pkv_decode_read_probe_sink_size.argtypes = [i32, i32, i32, i32, i32]
    L.pkv_decode_read_probe.restype = i32
    L.pkv_decode_read_probe.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                        i32, vp, sz, vp]
    L.pkv_profile_enable.restype = i32
    L.pkv_profile_enable.argtypes = [i32]
    L.pkv_profile_reset.restype = i32
    L.pkv_profile_read.restype = i32
    L.pkv_profile_read.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_longlong)]
    L.pkv_profile_kernel_names.restype = ctypes.c_char_p
    L.pkv_kv_cache_write_fp8.restype = i32
    L.pkv_kv_cache_write_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                         f32, vp]
    L.pkv_paged_attention_decode_fp8.restype = i32
    L.pkv_paged_attention_decode_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                                 i32, i32, f32, f32, f32, i32, i32, vp, sz, i32,
                                                 vp]
    L.pkv_decode_shared_prefix_workspace_size.restype = sz
    L.pkv_decode_shared_prefix_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    L.pkv_paged_attention_decode_shared_prefix.restype = i32
    L.pkv_paged_attention_decode_shared_prefix.argtypes = [
        vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, f32,
        i32, i32, i32, f32, f32, vp, sz, i32, vp]
    L.pkv_kv_cache_write_and_decode.restype = i32
    L.pkv_kv_cache_write_and_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                                i32, i32, i32, i32, f32, i32, i32, vp, sz, i32,
                                                vp]
    L.pkv_kv_cache_copy_blocks.restype = i32
    L.pkv_kv_cache_copy_blocks.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                           vp]
    i64, pi32 = ctypes.c_int64, ctypes.POINTER(ctypes.c_int32)
    pint = ctypes.POINTER(ctypes.c_int)
    L.pkv_bm_create.restype = i32
    L.pkv_bm_create.argtypes = [i32, i32, ctypes.POINTER(vp)]
    L.pkv_bm_destroy.restype = None
    L.pkv_bm_destroy.argtypes = [vp]
    L.pkv_bm_num_free.restype = i32
    L.pkv_bm_num_free.argtypes = [vp]
    for name in ("pkv_bm_add", "pkv_bm_free"):
        getattr(L, name).restype = i32
        getattr(L, name).argtypes = [vp, i64]
    L.pkv_bm_fork.restype = i32
    L.pkv_bm_fork.argtypes = [vp, i64, i64]
    L.pkv_bm_append.restype = i32
    L.pkv_bm_append.argtypes = [vp, i64, i32, pi32, pi32, i32, pint]
    L.pkv_bm_context_len.restype = i32
    L.pkv_bm_context_len.argtypes = [vp, i64, pint]
    L.pkv_bm_block_table.restype = i32
    L.pkv_bm_block_table.argtypes = [vp, i64, pi32, i32, pint]
    L.pkv_bm_refcount.restype = i32
    L.pkv_bm_refcount.argtypes = [vp, i32, pint]
    return L


def _check(status: int, where: str) -> None:
    if status != PKV_OK:
        L = lib()
        raise PkvError(status, where, L.pkv_last_error().decode())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype == torch.float32:
        return PKV_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _is_fp8_pool(t) -> bool:
    """E4M3 pools are uint8 tensors of codes (or torch.float8_e4m3fn views of them)."""
    import torch
    return t.dtype in (torch.uint8, torch.float8_e4m3fn)


def _pool_code(t) -> int:
    return PKV_FP8_E4M3 if _is_fp8_pool(t) else _dtype_code(t)


def _same_dtype(what: str, *ts) -> None:
    """The kernels take element types from one argument; a tensor of another type would be
    read with the wrong element size, so a mismatch is refused here."""
    if any(t.dtype != ts[0].dtype for t in ts):
        raise TypeError(f"{what} must share one dtype (got {[str(t.dtype) for t in ts]})")


def _bf16(what: str, *ts) -> None:
    import torch
    if any(t.dtype != torch.bfloat16 for t in ts):
        raise TypeError(f"{what} must be bfloat16")


def _dev(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _i32(t, name: str):
    import torch
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    return _dev(t, name)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def kv_cache_write(k_new, v_new, k_pool, v_pool, slot_mapping, stream=None) -> None:
    """Scatter k_new/v_new [T][Hkv][D] into k_pool [NB][Hkv][B][D] / v_pool [NB][Hkv][D][B]
    at slot_mapping [T] (int32, slot = block * B + offset, negative = skip). In place."""
    T, hkv, d = k_new.shape
    nb, hkv2, b, d2 = k_pool.shape
    if (hkv, d) != (hkv2, d2) or v_pool.shape != (nb, hkv, d, b) or v_new.shape != k_new.shape:
        raise ValueError("inconsistent shapes")
    if not (k_new.dtype == v_new.dtype == k_pool.dtype == v_pool.dtype):
        raise TypeError("k/v and pools must share a dtype")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [T]")
    _check(lib().pkv_kv_cache_write(_dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                    _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                    _i32(slot_mapping, "slot_mapping"), T, hkv, d, b, nb,
                                    _dtype_code(k_pool), _stream(stream)), "kv_cache_write")


def decode_partition_size(partition_size, num_seqs, num_kv_heads, max_context_len,
                          dtype=PKV_BF16) -> int:
    """Fixed partition size decode uses (0: the balanced split)."""
    return lib().pkv_decode_partition_size(partition_size, num_seqs, num_kv_heads,
                                           max_context_len, dtype)


def decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                          partition_size=0, dtype=PKV_BF16) -> int:
    return lib().pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                           max_context_len, partition_size, dtype)


def paged_attention_decode(out, q, k_pool, v_pool, block_table, context_lens, scale,
                           max_context_len=0, partition_size=0, workspace=None, stream=None,
                           num_waves=0):
    """out [S][Hq][D] = softmax(scale * q K^T) V over each sequence's paged context.
    A workspace (uint8 device tensor) is allocated when needed and not given. num_waves: waves
    of the balanced split (0 = the library's default)."""
    import torch
    S, hq, d = q.shape
    nb, hkv, b, d2 = k_pool.shape
    if d2 != d or v_pool.shape != (nb, hkv, d, b) or out.shape != q.shape:
        raise ValueError("inconsistent shapes")
    if block_table.dim() != 2 or block_table.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_table must be [S][MB], context_lens [S]")
    _same_dtype("q, k_pool and v_pool", q, k_pool, v_pool)
    mb = block_table.shape[1]
    ctx = max_context_len if max_context_len else mb * b
    need = decode_workspace_size(S, hq, hkv, d, ctx, partition_size, _dtype_code(q))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = ctypes.c_void_p(workspace.data_ptr()) if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().pkv_paged_attention_decode(
        _dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _i32(block_table, "block_table"), _i32(context_lens, "context_lens"), S, hq, hkv, d, b,
        mb, nb, float(scale), int(max_context_len), int(partition_size), int(num_waves), ws_ptr,
        ws_bytes, _dtype_code(q), _dtype_code(out), _stream(stream)), "paged_attention_decode")
    return out


def kv_cache_write_and_decode(out, q, k_new, v_new, slot_mapping, k_pool, v_pool, block_table,
                              context_lens, scale, max_context_len=0, workspace=None,
                              stream=None, num_waves=0):
    """kv_cache_write of each sequence's newest token (k_new / v_new [S][Hkv][D], slot_mapping
    [S], negative = none) and paged_attention_decode over the contexts including it, the write
    folded into the attention kernel (bf16). A workspace is allocated when needed and not
    given."""
    import torch
    S, hq, d = q.shape
    nb, hkv, b, d2 = k_pool.shape
    if d2 != d or v_pool.shape != (nb, hkv, d, b) or out.shape != q.shape:
        raise ValueError("inconsistent shapes")
    if k_new.shape != (S, hkv, d) or v_new.shape != k_new.shape or slot_mapping.shape != (S,):
        raise ValueError("k_new / v_new must be [S][Hkv][D], slot_mapping [S]")
    if block_table.dim() != 2 or block_table.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_table must be [S][MB], context_lens [S]")
    for t in (q, k_new, v_new, k_pool, v_pool):
        if t.dtype != torch.bfloat16:
            raise TypeError("q, k_new, v_new and the pools must be bfloat16")
    mb = block_table.shape[1]
    ctx = max_context_len if max_context_len else mb * b
    if workspace is None:
        need = decode_workspace_size(S, hq, hkv, d, ctx, 0, PKV_BF16)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().pkv_kv_cache_write_and_decode(
        _dev(out, "out"), _dev(q, "q"), _dev(k_new, "k_new"), _dev(v_new, "v_new"),
        _i32(slot_mapping, "slot_mapping"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _i32(block_table, "block_table"), _i32(context_lens, "context_lens"), S, hq, hkv, d, b,
        mb, nb, float(scale), int(max_context_len), int(num_waves),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
        _dtype_code(out), _stream(stream)), "kv_cache_write_and_decode")
    return out


def kv_cache_write_fp8(k_new, v_new, k_pool, v_pool, slot_mapping, k_scale, v_scale,
                       stream=None) -> None:
    """kv_cache_write into E4M3 pools (uint8 codes): each element x of k_new / v_new (bf16 or
    fp32) is stored as the E4M3 code of x / k_scale or x / v_scale."""
    T, hkv, d = k_new.shape
    nb, hkv2, b, d2 = k_pool.shape
    if (hkv, d) != (hkv2, d2) or v_pool.shape != (nb, hkv, d, b) or v_new.shape != k_new.shape:
        raise ValueError("inconsistent shapes")
    if not (_is_fp8_pool(k_pool) and _is_fp8_pool(v_pool)) or k_new.dtype != v_new.dtype:
        raise TypeError("pools must be E4M3 (uint8); k_new and v_new must share a dtype")
    if slot_mapping.shape != (T,):
        raise ValueError("slot_mapping must be [T]")
    _check(lib().pkv_kv_cache_write_fp8(_dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                        _i32(slot_mapping, "slot_mapping"), T, hkv, d, b, nb,
                                        _dtype_code(k_new), float(k_scale), float(v_scale),
                                        _stream(stream)), "kv_cache_write_fp8")


def paged_attention_decode_fp8(out, q, k_pool, v_pool, block_table, context_lens, scale, k_scale,
                               v_scale, max_context_len=0, workspace=None, stream=None,
                               num_waves=0):
    """paged_attention_decode over E4M3 pools (K value = code * k_scale, V value = code *
    v_scale); q bf16; out bf16 or fp32. A workspace is allocated when needed and not given."""
    import torch
    S, hq, d = q.shape
    nb, hkv, b, d2 = k_pool.shape
    if d2 != d or v_pool.shape != (nb, hkv, d, b) or out.shape != q.shape:
        raise ValueError("inconsistent shapes")
    if not (_is_fp8_pool(k_pool) and _is_fp8_pool(v_pool)):
        raise TypeError("pools must be E4M3 (uint8)")
    _bf16("q", q)
    if block_table.dim() != 2 or block_table.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_table must be [S][MB], context_lens [S]")
    mb = block_table.shape[1]
    ctx = max_context_len if max_context_len else mb * b
    need = decode_workspace_size(S, hq, hkv, d, ctx, 0, PKV_FP8_E4M3)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().pkv_paged_attention_decode_fp8(
        _dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _i32(block_table, "block_table"), _i32(context_lens, "context_lens"), S, hq, hkv, d, b,
        mb, nb, float(scale), float(k_scale), float(v_scale), int(max_context_len),
        int(num_waves), ctypes.c_void_p(workspace.data_ptr()),
        workspace.numel() * workspace.element_size(), _dtype_code(out), _stream(stream)),
        "paged_attention_decode_fp8")
    return out


def decode_shared_prefix_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                        max_context_len, max_prefix_len, kv_dtype=PKV_BF16):
    return lib().pkv_decode_shared_prefix_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                                         head_dim, max_context_len,
                                                         max_prefix_len, kv_dtype)


def paged_attention_decode_shared_prefix(out, q, k_pool, v_pool, block_table, context_lens,
                                         group_start, group_prefix_len, scale, max_group_size,
                                         max_prefix_len, k_scale=1.0, v_scale=1.0,
                                         max_context_len=0, workspace=None, stream=None,
                                         num_waves=0):
    """paged_attention_decode (bf16 pools) or paged_attention_decode_fp8 (uint8 E4M3 pools) for
    a batch in groups of consecutive sequences sharing prefixes: group i is sequences
    group_start[i] .. group_start[i+1]-1, sharing their first group_prefix_len[i] tokens (the
    same physical blocks). group_start / group_prefix_len are int32 device tensors."""
    import torch
    S, hq, d = q.shape
    nb, hkv, b, d2 = k_pool.shape
    if d2 != d or v_pool.shape != (nb, hkv, d, b) or out.shape != q.shape:
        raise ValueError("inconsistent shapes")
    if block_table.dim() != 2 or block_table.shape[0] != S or context_lens.shape != (S,):
        raise ValueError("block_table must be [S][MB], context_lens [S]")
    _bf16("q", q)
    _same_dtype("k_pool and v_pool", k_pool, v_pool)
    if not (_is_fp8_pool(k_pool) or k_pool.dtype == torch.bfloat16):
        raise TypeError("pools must be bfloat16 or E4M3 (uint8)")
    ng = group_prefix_len.shape[0]
    if group_start.shape != (ng + 1,):
        raise ValueError("group_start must be [num_groups + 1]")
    kvd = PKV_FP8_E4M3 if _is_fp8_pool(k_pool) else _dtype_code(k_pool)
    mb = block_table.shape[1]
    ctx = max_context_len if max_context_len else mb * b
    need = decode_shared_prefix_workspace_size(S, hq, hkv, d, ctx, max_prefix_len, kvd)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().pkv_paged_attention_decode_shared_prefix(
        _dev(out, "out"), _dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _i32(block_table, "block_table"), _i32(context_lens, "context_lens"),
        _i32(group_start, "group_start"), _i32(group_prefix_len, "group_prefix_len"), ng,
        int(max_group_size), int(max_prefix_len), S, hq, hkv, d, b, mb, nb, float(scale),
        int(max_context_len), int(num_waves), kvd, float(k_scale), float(v_scale),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
        _dtype_code(out), _stream(stream)), "paged_attention_decode_shared_prefix")
    return out


def paged_attention_prefill_chunk(out, q, cu_q_lens, context_lens, k_pool, v_pool, block_table,
                                  scale, max_q_len=0, max_context_len=0, stream=None):
    """out [Tq][Hq][D]: causal attention of each sequence's chunk rows over its paged context
    (row i of a c-row chunk after r cached tokens sees keys 0 .. r + i)."""
    tq, hq, d = q.shape
    nb, hkv, b, d2 = k_pool.shape
    S = context_lens.shape[0]
    if d2 != d or v_pool.shape != (nb, hkv, d, b) or out.shape != q.shape:
        raise ValueError("inconsistent shapes")
    if cu_q_lens.shape != (S + 1,) or block_table.dim() != 2 or block_table.shape[0] != S:
        raise ValueError("cu_q_lens must be [S+1], block_table [S][MB]")
    _same_dtype("q, k_pool and v_pool", q, k_pool, v_pool)
    _check(lib().pkv_paged_attention_prefill_chunk(
        _dev(out, "out"), _dev(q, "q"), _i32(cu_q_lens, "cu_q_lens"),
        _i32(context_lens, "context_lens"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
        _i32(block_table, "block_table"), S, tq, hq, hkv, d, b, block_table.shape[1], nb,
        float(scale), int(max_q_len), int(max_context_len), _dtype_code(q), _dtype_code(out),
        _stream(stream)), "paged_attention_prefill_chunk")
    return out


def _pool(t, name: str):
    """A pool may live in device memory or in pinned host memory (a swap space)."""
    if not (t.is_cuda or t.is_pinned()):
        raise ValueError(f"{name} must be a device tensor or a pinned host tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def kv_cache_copy_blocks(src_k, src_v, dst_k, dst_v, block_pairs, stream=None) -> None:
    """Copy whole blocks: for each row (s, d) of block_pairs [n][2] (int32, device), block s of
    src_k/src_v to block d of dst_k/dst_v. Pools are [NB][Hkv][B][D] (K) and [NB][Hkv][D][B] (V)
    in device memory or pinned host memory; source and destination may be the same pools."""
    nbs, hkv, b, d = src_k.shape
    nbd = dst_k.shape[0]
    if (src_v.shape != (nbs, hkv, d, b) or dst_k.shape[1:] != (hkv, b, d)
            or dst_v.shape != (nbd, hkv, d, b)):
        raise ValueError("inconsistent pool shapes")
    if not (src_k.dtype == src_v.dtype == dst_k.dtype == dst_v.dtype):
        raise TypeError("pools must share a dtype")
    if block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [n][2]")
    n = block_pairs.shape[0]
    _check(lib().pkv_kv_cache_copy_blocks(
        _pool(src_k, "src_k"), _pool(src_v, "src_v"), _pool(dst_k, "dst_k"),
        _pool(dst_v, "dst_v"), _i32(block_pairs, "block_pairs") if n else None, n, hkv, d, b,
        nbs, nbd, _pool_code(src_k), _stream(stream)), "kv_cache_copy_blocks")


def decode_read_probe(k_pool, v_pool, block_table, context_lens, num_q_heads,
                      max_context_len=0, num_waves=0, sink=None, stream=None):
    """Measurement only: the balanced decode's waves read exactly the decode's K/V tiles (bf16
    pools) without the attention arithmetic. Returns the sink tensor it wrote."""
    import torch
    nb, hkv, b, d = k_pool.shape
    S = context_lens.shape[0]
    if v_pool.shape != (nb, hkv, d, b) or block_table.dim() != 2 or block_table.shape[0] != S:
        raise ValueError("inconsistent shapes")
    _bf16("k_pool and v_pool", k_pool, v_pool)
    mb = block_table.shape[1]
    ctx = max_context_len if max_context_len else mb * b
    need = lib().pkv_decode_read_probe_sink_size(S, num_q_heads, hkv, ctx, int(num_waves))
    if sink is None:
        sink = torch.empty(max(need // 4, 1), dtype=torch.int32, device=k_pool.device)
    _check(lib().pkv_decode_read_probe(
        _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _i32(block_table, "block_table"),
        _i32(context_lens, "context_lens"), S, num_q_heads, hkv, d, b, mb, nb,
        int(max_context_len), int(num_waves), _dev(sink, "sink"),
        sink.numel() * sink.element_size(), _stream(stream)), "decode_read_probe")
    return sink


# ------------------------------------------------------------------------------ block manager

class BlockManager:
    """Host block manager in libpkv: reference-counted physical blocks, per-sequence block
    tables, copy-on-write when a sequence appends into a shared, partly filled block."""

    def __init__(self, num_blocks: int, block_size: int):
        self._h = ctypes.c_void_p()
        _check(lib().pkv_bm_create(num_blocks, block_size, ctypes.byref(self._h)),
               "pkv_bm_create")
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self) -> None:
        if self._h:
            lib().pkv_bm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_free(self) -> int:
        return lib().pkv_bm_num_free(self._h)

    def add(self, seq: int) -> None:
        _check(lib().pkv_bm_add(self._h, seq), "pkv_bm_add")

    def fork(self, parent: int, child: int) -> None:
        _check(lib().pkv_bm_fork(self._h, parent, child), "pkv_bm_fork")

    def append(self, seq: int, n_tokens: int):
        """Slots (list of int) for the next n_tokens of seq, and the (src, dst) block copies the
        caller must make before writing them."""
        slots = (ctypes.c_int32 * max(n_tokens, 1))()
        copies = (ctypes.c_int32 * 2)()
        n_copies = ctypes.c_int()
        _check(lib().pkv_bm_append(self._h, seq, n_tokens, slots, copies, 1,
                                   ctypes.byref(n_copies)), "pkv_bm_append")
        pairs = [(copies[0], copies[1])] if n_copies.value else []
        return list(slots[:n_tokens]), pairs

    def free(self, seq: int) -> None:
        _check(lib().pkv_bm_free(self._h, seq), "pkv_bm_free")

    def context_len(self, seq: int) -> int:
        n = ctypes.c_int()
        _check(lib().pkv_bm_context_len(self._h, seq, ctypes.byref(n)), "pkv_bm_context_len")
        return n.value

    def block_table(self, seq: int):
        n = ctypes.c_int()
        _check(lib().pkv_bm_block_table(self._h, seq, None, 0, ctypes.byref(n)),
               "pkv_bm_block_table")
        table = (ctypes.c_int32 * max(n.value, 1))()
        _check(lib().pkv_bm_block_table(self._h, seq, table, n.value, ctypes.byref(n)),
               "pkv_bm_block_table")
        return list(table[:n.value])

    def refcount(self, block: int) -> int:
        c = ctypes.c_int()
        _check(lib().pkv_bm_refcount(self._h, block, ctypes.byref(c)), "pkv_bm_refcount")
        return c.value


# ------------------------------------------------------------------------------ timing

KERNEL_NAMES = ("kv_cache_write", "decode_partition", "decode_reduce", "prefill_chunk",
                "copy_blocks", "read_probe")


def profile_enable(on: bool = True, kernels=None) -> None:
    """Time the library's kernels (all of them, or only those named in `kernels`) with HIP
    events recorded as part of each kernel dispatch; clears the totals."""
    if not on:
        mask = 0
    elif kernels is None:
        mask = (1 << len(KERNEL_NAMES)) - 1
    else:
        mask = 0
        for k in kernels:
            mask |= 1 << KERNEL_NAMES.index(k)
    _check(lib().pkv_profile_enable(mask), "profile_enable")


def profile_reset() -> None:
    _check(lib().pkv_profile_reset(), "profile_reset")


def profile_read(kernel: str):
    """(total milliseconds, launches) of `kernel` since the last enable/reset."""
    ms = ctypes.c_double()
    n = ctypes.c_longlong()
    _check(lib().pkv_profile_read(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)),
           "profile_read")
    return ms.value, n.value
