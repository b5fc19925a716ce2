"""Paged KV-cache layout of the library, built from and read back into logical rows.

Set-up and inspection plumbing (torch indexing on the device), not part of the
window step: it fills the caches a prefill would have left, and reads rows
back for checks. Layouts (``include/wedlm.h``):
  k_cache [n_layers][num_pages][Hkv][D / X][P][X], X = 16 bytes / element size,
  v_cache [n_layers][num_pages][Hkv][D][P],
position t of sequence b at page block_table[b][t // P], offset t % P.
"""

import torch


def vec_elems(dtype):
    return 16 // torch.empty((), dtype=dtype).element_size()


def alloc_caches(n_layers, num_pages, Hkv, D, page_size, dtype, device):
    X = vec_elems(dtype)
    kc = torch.zeros((n_layers, num_pages, Hkv, D // X, page_size, X), dtype=dtype, device=device)
    vc = torch.zeros((n_layers, num_pages, Hkv, D, page_size), dtype=dtype, device=device)
    return kc, vc


def _page_index(block_table_row, positions, page_size):
    pages = block_table_row[positions // page_size].long()
    return pages, (positions % page_size).long()


def write_rows(kc, vc, layer, block_table_row, start, k_rows, v_rows):
    """Store logical rows [n, Hkv, D] at positions start .. start+n-1 of one sequence."""
    n = k_rows.shape[0]
    if n == 0:
        return
    P = kc.shape[4]
    X = kc.shape[5]
    Hkv, D = k_rows.shape[1], k_rows.shape[2]
    dev = kc.device
    pos = torch.arange(start, start + n, device=dev)
    bt = block_table_row.to(dev)
    pages, offs = _page_index(bt, pos, P)
    kr = k_rows.to(device=dev, dtype=kc.dtype).reshape(n, Hkv, D // X, X)
    # kc[layer][page][h][slice][off][x] <- kr[n][h][slice][x]
    kc[layer].permute(0, 3, 1, 2, 4)[pages, offs] = kr
    vr = v_rows.to(device=dev, dtype=vc.dtype)
    # vc[layer][page][h][d][off] <- vr[n][h][d]
    vc[layer].permute(0, 3, 1, 2)[pages, offs] = vr


def read_rows(kc, vc, layer, block_table_row, start, n):
    """Logical rows [n, Hkv, D] (K, V) at positions start .. start+n-1 of one sequence."""
    P = kc.shape[4]
    X = kc.shape[5]
    Hkv = kc.shape[2]
    D = kc.shape[3] * X
    dev = kc.device
    pos = torch.arange(start, start + n, device=dev)
    pages, offs = _page_index(block_table_row.to(dev), pos, P)
    k = kc[layer].permute(0, 3, 1, 2, 4)[pages, offs].reshape(n, Hkv, D)
    v = vc[layer].permute(0, 3, 1, 2)[pages, offs]
    return k, v
