"""Dual-stream masking attention forward on the window-step kernels.

hyper.ai summary of WeDLM, "Method": training pairs a clean memory stream with
a masked prediction stream over the same logical positions; the prediction
stream is cut into blocks that are topologically reordered, and a prediction
token attends to the memory stream's context of the preceding blocks and,
inside its block, causally.

Block j of the prediction stream is exactly a decoding window: W = Bk slots
at logical positions j*Bk .., reordered, attending causally to itself over a
prefix - here the memory stream's first j*Bk positions. So the forward runs
the library's calls with one "sequence" per (sample, block):

  1. wedlm_window_reorder of all-observed flags gives the memory stream's
     identity order and positions; wedlm_commit_prefix_rope writes every
     memory block's rotated keys and values into a paged cache (one 16-token
     page list per sample, shared by all its blocks' block-table rows);
  2. wedlm_window_attn_rope over the memory blocks: causal attention of the
     memory stream (block j over the memory prefix plus itself);
  3. wedlm_window_reorder of the prediction stream's observed flags, then
     wedlm_window_attn_rope over the prediction blocks against the same
     memory prefix.

Argument marshalling and buffer management only: every operation runs in the
library's kernels. Outputs are in physical order per block (as the attention
entry points return them); ``inv_perm`` maps slots to physical rows.
"""

import torch

from . import wedlm as W_

PAGE = 16


class DualStreamAttention:
    """Buffers and launches of one dual-stream attention layer for fixed shapes.

    S samples of N positions, blocks of Bk (N % Bk == 0, N % 16 == 0), bf16
    (D = 128) or f32 projections [S, N, H, D] of both streams.
    """

    def __init__(self, S, N, Bk, Hq, Hkv, D, theta, dtype, device, scale=None):
        if N % Bk or N % PAGE or not (1 <= Bk <= W_.MAX_WINDOW):
            raise ValueError("N must be a multiple of Bk and of 16, and Bk <= 64")
        self.S, self.N, self.Bk, self.Hq, self.Hkv, self.D = S, N, Bk, Hq, Hkv, D
        self.theta = theta
        self.dt = W_.dtype_code(dtype)
        self.scale = D ** -0.5 if scale is None else scale
        self.nb = N // Bk
        self.Bp = S * self.nb                      # one window per (sample, block)
        self.max_pages = N // PAGE
        self.num_pages = S * self.max_pages
        i32 = dict(dtype=torch.int32, device=device)
        j = torch.arange(self.nb, **i32)
        self.prefix_len = (j * Bk).repeat(S).contiguous()
        pages = torch.arange(self.num_pages, **i32).view(S, 1, self.max_pages)
        self.block_table = pages.expand(S, self.nb, self.max_pages).reshape(self.Bp, -1).contiguous()
        X = 16 // torch.tensor([], dtype=dtype).element_size()
        self.k_cache = torch.empty((1, self.num_pages, Hkv, D // X, PAGE, X), dtype=dtype,
                                   device=device)
        self.v_cache = torch.empty((1, self.num_pages, Hkv, D, PAGE), dtype=dtype, device=device)
        self.all_obs = torch.ones((self.Bp, Bk), dtype=torch.uint8, device=device)

        def order():
            return {k: torch.empty(s, **i32) for k, s in (
                ("perm", (self.Bp, Bk)), ("inv", (self.Bp, Bk)), ("pos", (self.Bp, Bk)),
                ("n_obs", (self.Bp,)), ("run", (self.Bp,)))}
        self.mem, self.pred = order(), order()
        # scratch window state for the commit call (its state half is not used)
        self.tokens = torch.empty((self.Bp, Bk), **i32)
        self.filled_scratch = torch.empty((self.Bp, Bk), dtype=torch.uint8, device=device)
        self.len_scratch = torch.empty((self.Bp,), **i32)
        self.commit_len = torch.empty((self.Bp,), **i32)
        self.cache_slot = torch.empty((self.Bp, Bk), **i32)
        self.selected = torch.zeros((self.Bp, Bk), dtype=torch.uint8, device=device)
        self.argmax = torch.zeros((self.Bp, Bk), **i32)
        self.out_mem = torch.empty((1, self.Bp, Bk, Hq, D), dtype=dtype, device=device)
        self.out_pred = torch.empty_like(self.out_mem)
        self.ws_bytes = W_.wedlm_window_attn_workspace_size(self.dt, 1, self.Bp, Bk, Hq, Hkv, D,
                                                            PAGE, N - Bk)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=device)

    def _view(self, x, H):
        return x.reshape(1, self.Bp, self.Bk, H, self.D)

    def _reorder(self, filled, o, stream):
        W_.wedlm_window_reorder(self.Bp, self.Bk, filled, self.prefix_len, o["perm"], o["inv"],
                                o["pos"], o["n_obs"], o["run"], stream)

    def _attend(self, q, k, v, o, out, stream):
        W_.wedlm_window_attn_rope(self.dt, 1, self.Bp, self.Bk, self.Hq, self.Hkv, self.D, PAGE,
                                  self.num_pages, self.max_pages, self.N - self.Bk, self.scale,
                                  self.theta, q, k, v, o["perm"], o["pos"], self.k_cache,
                                  self.v_cache, self.block_table, self.prefix_len, None, out,
                                  self.ws if self.ws_bytes else None, self.ws_bytes,
                                  flags=W_.WEDLM_ATTN_SHARED_PAGES, stream=stream)

    def forward(self, q_mem, k_mem, v_mem, q_pred, k_pred, v_pred, filled, stream=None):
        """q_* [S, N, Hq, D], k_* / v_* [S, N, Hkv, D] (slot order, before RoPE),
        filled [S, N] uint8 (the prediction stream's observed positions).

        Returns (out_mem, out_pred): [1, S * N / Bk, Bk, Hq, D] each, block
        rows in physical order (the memory stream's is its slot order);
        ``self.pred["inv"]`` maps a prediction slot to its physical row.
        """
        qm, km, vm = self._view(q_mem, self.Hq), self._view(k_mem, self.Hkv), self._view(v_mem, self.Hkv)
        qp, kp, vp = self._view(q_pred, self.Hq), self._view(k_pred, self.Hkv), self._view(v_pred, self.Hkv)
        # 1. the memory stream's rotated keys and values into the paged cache
        self._reorder(self.all_obs, self.mem, stream)
        self.filled_scratch.copy_(self.all_obs)
        self.len_scratch.copy_(self.prefix_len)
        W_.wedlm_commit_prefix_rope(self.dt, 1, self.Bp, self.Bk, self.Hkv, self.D, PAGE,
                                    self.num_pages, self.max_pages, self.theta, self.mem["run"],
                                    self.selected, self.argmax, km, vm, self.block_table,
                                    self.k_cache, self.v_cache, self.tokens, self.filled_scratch,
                                    self.len_scratch, self.commit_len, self.cache_slot, -1, stream)
        # 2. memory stream: causal over the memory prefix and its own block
        self._attend(qm, km, vm, self.mem, self.out_mem, stream)
        # 3. prediction stream: reordered blocks over the memory prefix
        self._reorder(filled.reshape(self.Bp, self.Bk), self.pred, stream)
        self._attend(qp, kp, vp, self.pred, self.out_pred, stream)
        return self.out_mem, self.out_pred
