"""ctypes binding of libwedlm.so: one Python function per C entry point, same names.

Argument marshalling only: tensors are passed as device pointers
(``Tensor.data_ptr()``), the stream as torch's current HIP stream unless one
is given, and a non-zero status raises ``WedlmError``. Every step of the
computation runs in the library's HIP kernels; nothing here computes. The
library is loaded on first use and a missing library raises - there is no
fallback path.
"""

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwedlm.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "wedlm.h")

WEDLM_F32 = 0
WEDLM_BF16 = 1
WEDLM_ATTN_SHARED_PAGES = 1  # attention flag: rows of the block table share pages
WEDLM_ATTN_DEFER_COMBINE = 2  # attention flag: the split merge runs in the combine tail
MAX_WINDOW = 64

_c_int, _c_size, _c_float, _c_double, _p = (ctypes.c_int, ctypes.c_size_t, ctypes.c_float,
                                             ctypes.c_double, ctypes.c_void_p)

# argument types of every exported function (must match include/wedlm.h)
_SIGNATURES = {
    "wedlm_status_string": (ctypes.c_char_p, [_c_int]),
    "wedlm_abi_version": (_c_int, []),
    "wedlm_window_reorder": (_c_int, [_c_int, _c_int, _p, _p, _p, _p, _p, _p, _p, _p]),
    "wedlm_window_reorder_rule": (_c_int, [_c_int, _c_int, _c_int, _p, _p, _p, _p, _p, _p, _p, _p]),
    "wedlm_rope_logical": (_c_int, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _c_double,
                                    _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "wedlm_window_attn_workspace_size": (_c_size, [_c_int] * 9),
    "wedlm_window_attn": (_c_int, [_c_int] * 11 + [_c_float] + [_p] * 9 + [_c_size, _c_int, _p]),
    "wedlm_entropy_select_workspace_size": (_c_size, [_c_int] * 4),
    "wedlm_entropy_select": (_c_int, [_c_int] * 4 + [_p, _p, _c_float, _c_float, _c_int] + [_p] * 5
                             + [_c_size, _p]),
    "wedlm_entropy_select_noalloc": (_c_int, [_c_int] * 4 + [_p, _p, _c_float, _c_float, _c_int]
                                     + [_p] * 5),
    "wedlm_commit_prefix": (_c_int, [_c_int] * 9 + [_p] * 13 + [ctypes.c_int32, _p]),
    "wedlm_window_attn_rope": (_c_int, [_c_int] * 11 + [_c_float, _c_double] + [_p] * 12
                               + [_c_size, _c_int, _p]),
    "wedlm_commit_prefix_rope": (_c_int, [_c_int] * 9 + [_c_double] + [_p] * 13
                                 + [ctypes.c_int32, _p]),
    "wedlm_lm_head_packed_size": (_c_size, [_c_int] * 3),
    "wedlm_lm_head_pack": (_c_int, [_c_int] * 3 + [_p, _p, _p]),
    "wedlm_lm_head_select_workspace_size": (_c_size, [_c_int] * 5),
    "wedlm_lm_head_select": (_c_int, [_c_int] * 5 + [_p, _p, _p, _c_float, _c_float, _c_int]
                             + [_p] * 5 + [_c_size, _p]),
    "wedlm_read_probe": (_c_int, [_p, _c_size, _p, _c_int, _p, _c_int, _p]),
    "wedlm_select_commit_reorder": (_c_int, [_c_int] * 4 + [_p, _c_float, _c_float] + [_c_int] * 5
                                    + [_p] * 7 + [ctypes.c_int32] + [_p] * 9 + [_c_size, _p]),
    "wedlm_entropy_partials": (_c_int, [_c_int] * 4 + [_p, _p, _c_size, _p]),
    "wedlm_window_attn_rope_entropy": (_c_int, [_c_int] * 11 + [_c_float, _c_double] + [_p] * 12
                                       + [_c_size, _c_int, _c_int, _p, _p, _c_size, _p]),
    "wedlm_select_commit_reorder_partials": (_c_int, [_c_int] * 4 + [_c_float, _c_float]
                                             + [_c_int] * 5 + [_p] * 7 + [ctypes.c_int32]
                                             + [_p] * 9 + [_c_size, _p]),
    "wedlm_select_commit_reorder_combine": (_c_int, [_c_int] * 4 + [_c_float, _c_float]
                                            + [_c_int] * 5 + [_p] * 7 + [ctypes.c_int32]
                                            + [_p] * 9 + [_c_size] + [_c_int] * 5
                                            + [_p, _c_size, _p, _p]),
    "wedlm_block_attn_rope": (_c_int, [_c_int] * 10 + [_c_float, _c_double] + [_p] * 10),
}

_lib = None


class WedlmError(RuntimeError):
    def __init__(self, fn, status):
        msg = lib().wedlm_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status} ({msg})")
        self.status = status


def header_functions():
    """Names of the functions include/wedlm.h declares."""
    with open(HEADER) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"\b(wedlm_[a-z_0-9]+)\s*\(", text)))


def lib():
    """Load libwedlm.so once (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with causal_streaming_decoding_amd.build.build()")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("wedlm kernels take device tensors")
    if not t.is_contiguous():
        raise ValueError("wedlm kernels take contiguous tensors")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(name, status):
    if status != 0:
        raise WedlmError(name, status)


def dtype_code(t_or_dtype):
    dt = t_or_dtype.dtype if isinstance(t_or_dtype, torch.Tensor) else t_or_dtype
    if dt == torch.bfloat16:
        return WEDLM_BF16
    if dt == torch.float32:
        return WEDLM_F32
    raise ValueError(f"unsupported dtype {dt}")


def wedlm_status_string(status):
    return lib().wedlm_status_string(status).decode()


def wedlm_abi_version():
    return lib().wedlm_abi_version()


def wedlm_window_reorder(B, W, filled, prefix_len, perm, inv_perm, pos, n_obs, run_len, stream=None):
    _check("wedlm_window_reorder", lib().wedlm_window_reorder(
        B, W, _ptr(filled), _ptr(prefix_len), _ptr(perm), _ptr(inv_perm), _ptr(pos), _ptr(n_obs),
        _ptr(run_len), _stream(stream)))


COMMIT_STREAM = 0
COMMIT_BLOCK = 1


def wedlm_window_reorder_rule(B, W, commit_rule, filled, prefix_len, perm, inv_perm, pos, n_obs,
                              run_len, stream=None):
    _check("wedlm_window_reorder_rule", lib().wedlm_window_reorder_rule(
        B, W, commit_rule, _ptr(filled), _ptr(prefix_len), _ptr(perm), _ptr(inv_perm), _ptr(pos),
        _ptr(n_obs), _ptr(run_len), _stream(stream)))


def wedlm_rope_logical(dtype, n_layers, B, W, Hq, Hkv, D, theta, q, k, v, perm, pos, q_phys, k_phys,
                       v_phys, stream=None):
    _check("wedlm_rope_logical", lib().wedlm_rope_logical(
        dtype, n_layers, B, W, Hq, Hkv, D, float(theta), _ptr(q), _ptr(k), _ptr(v), _ptr(perm),
        _ptr(pos), _ptr(q_phys), _ptr(k_phys), _ptr(v_phys), _stream(stream)))


def wedlm_window_attn_workspace_size(dtype, n_layers, B, W, Hq, Hkv, D, page_size, max_prefix_len):
    return lib().wedlm_window_attn_workspace_size(dtype, n_layers, B, W, Hq, Hkv, D, page_size,
                                                  max_prefix_len)


def wedlm_window_attn(dtype, n_layers, B, W, Hq, Hkv, D, page_size, num_pages, max_pages,
                      max_prefix_len, scale, q_phys, k_phys, v_phys, k_cache, v_cache, block_table,
                      prefix_len, out_phys, workspace, workspace_bytes, flags=0, stream=None):
    _check("wedlm_window_attn", lib().wedlm_window_attn(
        dtype, n_layers, B, W, Hq, Hkv, D, page_size, num_pages, max_pages, max_prefix_len,
        float(scale), _ptr(q_phys), _ptr(k_phys), _ptr(v_phys), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_table), _ptr(prefix_len), _ptr(out_phys), _ptr(workspace), workspace_bytes,
        flags, _stream(stream)))


def wedlm_entropy_select_workspace_size(dtype, B, W, V):
    return lib().wedlm_entropy_select_workspace_size(dtype, B, W, V)


def wedlm_entropy_select(dtype, B, W, V, logits, filled, lam, tau, min_fill, entropy, score,
                         argmax_tok, selected, workspace, workspace_bytes, stream=None):
    _check("wedlm_entropy_select", lib().wedlm_entropy_select(
        dtype, B, W, V, _ptr(logits), _ptr(filled), float(lam), float(tau), int(min_fill),
        _ptr(entropy), _ptr(score), _ptr(argmax_tok), _ptr(selected), _ptr(workspace),
        workspace_bytes, _stream(stream)))


def wedlm_entropy_select_noalloc(dtype, B, W, V, logits, filled, lam, tau, min_fill, entropy,
                                 score, argmax_tok, selected, stream=None):
    _check("wedlm_entropy_select_noalloc", lib().wedlm_entropy_select_noalloc(
        dtype, B, W, V, _ptr(logits), _ptr(filled), float(lam), float(tau), int(min_fill),
        _ptr(entropy), _ptr(score), _ptr(argmax_tok), _ptr(selected), _stream(stream)))


def wedlm_lm_head_packed_size(dtype, hidden, V):
    return lib().wedlm_lm_head_packed_size(dtype, hidden, V)


def wedlm_lm_head_pack(dtype, hidden, V, w_vocab, w_packed, stream=None):
    _check("wedlm_lm_head_pack", lib().wedlm_lm_head_pack(
        dtype, hidden, V, _ptr(w_vocab), _ptr(w_packed), _stream(stream)))


def wedlm_lm_head_select_workspace_size(dtype, B, W, hidden, V):
    return lib().wedlm_lm_head_select_workspace_size(dtype, B, W, hidden, V)


def wedlm_lm_head_select(dtype, B, W, hidden, V, hidden_states, w_packed, filled, lam, tau, min_fill,
                         entropy, score, argmax_tok, selected, workspace, workspace_bytes,
                         stream=None):
    _check("wedlm_lm_head_select", lib().wedlm_lm_head_select(
        dtype, B, W, hidden, V, _ptr(hidden_states), _ptr(w_packed), _ptr(filled), float(lam),
        float(tau), int(min_fill), _ptr(entropy), _ptr(score), _ptr(argmax_tok), _ptr(selected),
        _ptr(workspace), workspace_bytes, _stream(stream)))


def wedlm_commit_prefix(dtype, n_layers, B, W, Hkv, D, page_size, num_pages, max_pages, run_len,
                        selected, argmax_tok, k_phys, v_phys, block_table, k_cache, v_cache, tokens,
                        filled, prefix_len, commit_len, cache_slot, mask_id, stream=None):
    _check("wedlm_commit_prefix", lib().wedlm_commit_prefix(
        dtype, n_layers, B, W, Hkv, D, page_size, num_pages, max_pages, _ptr(run_len),
        _ptr(selected), _ptr(argmax_tok), _ptr(k_phys), _ptr(v_phys), _ptr(block_table),
        _ptr(k_cache), _ptr(v_cache), _ptr(tokens), _ptr(filled), _ptr(prefix_len),
        _ptr(commit_len), _ptr(cache_slot), int(mask_id), _stream(stream)))


def wedlm_window_attn_rope(dtype, n_layers, B, W, Hq, Hkv, D, page_size, num_pages, max_pages,
                           max_prefix_len, scale, theta, q, k, v, perm, pos, k_cache, v_cache,
                           block_table, prefix_len, commit_run, out_phys, workspace,
                           workspace_bytes, flags=0, stream=None):
    _check("wedlm_window_attn_rope", lib().wedlm_window_attn_rope(
        dtype, n_layers, B, W, Hq, Hkv, D, page_size, num_pages, max_pages, max_prefix_len,
        float(scale), float(theta), _ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(pos),
        _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(prefix_len), _ptr(commit_run),
        _ptr(out_phys), _ptr(workspace), workspace_bytes, flags, _stream(stream)))


def wedlm_commit_prefix_rope(dtype, n_layers, B, W, Hkv, D, page_size, num_pages, max_pages, theta,
                             run_len, selected, argmax_tok, k, v, block_table, k_cache, v_cache,
                             tokens, filled, prefix_len, commit_len, cache_slot, mask_id,
                             stream=None):
    _check("wedlm_commit_prefix_rope", lib().wedlm_commit_prefix_rope(
        dtype, n_layers, B, W, Hkv, D, page_size, num_pages, max_pages, float(theta),
        _ptr(run_len), _ptr(selected), _ptr(argmax_tok), _ptr(k), _ptr(v), _ptr(block_table),
        _ptr(k_cache), _ptr(v_cache), _ptr(tokens), _ptr(filled), _ptr(prefix_len),
        _ptr(commit_len), _ptr(cache_slot), int(mask_id), _stream(stream)))


def wedlm_select_commit_reorder(dtype, B, W, V, logits, lam, tau, min_fill, page_size, num_pages,
                                max_pages, commit_rule, block_table, run_len, tokens, filled,
                                prefix_len, commit_len, cache_slot, mask_id, entropy, score,
                                argmax_tok, selected, perm, inv_perm, pos, n_obs, workspace,
                                workspace_bytes, stream=None):
    _check("wedlm_select_commit_reorder", lib().wedlm_select_commit_reorder(
        dtype, B, W, V, _ptr(logits), float(lam), float(tau), int(min_fill), page_size, num_pages,
        max_pages, int(commit_rule), _ptr(block_table), _ptr(run_len), _ptr(tokens), _ptr(filled),
        _ptr(prefix_len), _ptr(commit_len), _ptr(cache_slot), int(mask_id), _ptr(entropy),
        _ptr(score), _ptr(argmax_tok), _ptr(selected), _ptr(perm), _ptr(inv_perm), _ptr(pos),
        _ptr(n_obs), _ptr(workspace), workspace_bytes, _stream(stream)))


def wedlm_window_attn_rope_entropy(dtype, n_layers, B, W, Hq, Hkv, D, page_size, num_pages,
                                   max_pages, max_prefix_len, scale, theta, q, k, v, perm, pos,
                                   k_cache, v_cache, block_table, prefix_len, commit_run, out_phys,
                                   workspace, workspace_bytes, flags, V, logits, ent_workspace,
                                   ent_workspace_bytes, stream=None):
    _check("wedlm_window_attn_rope_entropy", lib().wedlm_window_attn_rope_entropy(
        dtype, n_layers, B, W, Hq, Hkv, D, page_size, num_pages, max_pages, max_prefix_len,
        float(scale), float(theta), _ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(pos),
        _ptr(k_cache), _ptr(v_cache), _ptr(block_table), _ptr(prefix_len), _ptr(commit_run),
        _ptr(out_phys), _ptr(workspace), workspace_bytes, flags, V, _ptr(logits),
        _ptr(ent_workspace), ent_workspace_bytes, _stream(stream)))


def wedlm_entropy_partials(dtype, B, W, V, logits, workspace, workspace_bytes, stream=None):
    _check("wedlm_entropy_partials", lib().wedlm_entropy_partials(
        dtype, B, W, V, _ptr(logits), _ptr(workspace), workspace_bytes, _stream(stream)))


def wedlm_select_commit_reorder_partials(dtype, B, W, V, lam, tau, min_fill, page_size,
                                         num_pages, max_pages, commit_rule, block_table, run_len,
                                         tokens, filled, prefix_len, commit_len, cache_slot,
                                         mask_id, entropy, score, argmax_tok, selected, perm,
                                         inv_perm, pos, n_obs, workspace, workspace_bytes,
                                         stream=None):
    _check("wedlm_select_commit_reorder_partials", lib().wedlm_select_commit_reorder_partials(
        dtype, B, W, V, float(lam), float(tau), int(min_fill), page_size, num_pages, max_pages,
        int(commit_rule), _ptr(block_table), _ptr(run_len), _ptr(tokens), _ptr(filled),
        _ptr(prefix_len), _ptr(commit_len), _ptr(cache_slot), int(mask_id), _ptr(entropy),
        _ptr(score), _ptr(argmax_tok), _ptr(selected), _ptr(perm), _ptr(inv_perm), _ptr(pos),
        _ptr(n_obs), _ptr(workspace), workspace_bytes, _stream(stream)))


def wedlm_select_commit_reorder_combine(dtype, B, W, V, lam, tau, min_fill, page_size,
                                        num_pages, max_pages, commit_rule, block_table, run_len,
                                        tokens, filled, prefix_len, commit_len, cache_slot,
                                        mask_id, entropy, score, argmax_tok, selected, perm,
                                        inv_perm, pos, n_obs, workspace, workspace_bytes,
                                        attn_n_layers, attn_Hq, attn_Hkv, attn_D,
                                        attn_max_prefix_len, attn_workspace, attn_workspace_bytes,
                                        attn_out, stream=None):
    _check("wedlm_select_commit_reorder_combine", lib().wedlm_select_commit_reorder_combine(
        dtype, B, W, V, float(lam), float(tau), int(min_fill), page_size, num_pages, max_pages,
        int(commit_rule), _ptr(block_table), _ptr(run_len), _ptr(tokens), _ptr(filled),
        _ptr(prefix_len), _ptr(commit_len), _ptr(cache_slot), int(mask_id), _ptr(entropy),
        _ptr(score), _ptr(argmax_tok), _ptr(selected), _ptr(perm), _ptr(inv_perm), _ptr(pos),
        _ptr(n_obs), _ptr(workspace), workspace_bytes, attn_n_layers, attn_Hq, attn_Hkv, attn_D,
        attn_max_prefix_len, _ptr(attn_workspace), attn_workspace_bytes, _ptr(attn_out),
        _stream(stream)))


def wedlm_block_attn_rope(dtype, S, N, W, Hq, Hkv, D, page_size, num_pages, max_pages, scale,
                          theta, q, k, v, perm, pos, k_cache, v_cache, block_table, out,
                          stream=None):
    _check("wedlm_block_attn_rope", lib().wedlm_block_attn_rope(
        dtype, S, N, W, Hq, Hkv, D, page_size, num_pages, max_pages, float(scale), float(theta),
        _ptr(q), _ptr(k), _ptr(v), _ptr(perm), _ptr(pos), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_table), _ptr(out), _stream(stream)))


def wedlm_read_probe(src, nbytes, block_order, n_blocks, sink, grid, stream=None):
    _check("wedlm_read_probe", lib().wedlm_read_probe(
        _ptr(src), nbytes, _ptr(block_order), int(n_blocks), _ptr(sink), int(grid),
        _stream(stream)))
