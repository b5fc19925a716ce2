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
  2. the attention of the memory blocks: causal attention of the memory
     stream (block j over the memory prefix plus itself). The memory
     stream's attention is plain causal attention over the whole sequence, so
     its result does not depend on the block size: it runs in windows of its
     own size whatever Bk is (64 keys with the block kernel, whose cache tiles
     then need no mask; 16 with the window kernel, its fastest window shape),
     and its output, in identity order, has the same layout as Bk-key blocks;
  3. wedlm_window_reorder of the prediction stream's observed flags, then
     the attention of the prediction blocks against the same memory prefix.

The attentions run wedlm_block_attn_rope (the windows of a sample end to
end, 256 query rows of consecutive windows per key tile) where it has a
kernel (bf16, D = 128, 256 % (Hq / Hkv) == 0), else wedlm_window_attn_rope
with one block-table row per (sample, block), all rows of a sample sharing
its pages; both compute the same windows.

Argument marshalling and buffer management only: every operation runs in the
library's kernels. Outputs are in physical order per block (as the attention
entry points return them); ``inv_perm`` maps slots to physical rows.
"""

import torch

from . import wedlm as W_

PAGE = 16


class _Blocks:
    """One stream's windows: S samples of N positions in blocks of W, block j
    at logical positions j*W .. over a prefix of the sample's first j*W
    memory positions (one window per (sample, block))."""

    def __init__(self, S, N, W, Hq, Hkv, D, dt, dtype, device, block_pages):
        i32 = dict(dtype=torch.int32, device=device)
        self.W, self.nb = W, N // W
        self.Bp = S * self.nb
        j = torch.arange(self.nb, **i32)
        self.prefix_len = (j * W).repeat(S).contiguous()
        self.block_table = block_pages.expand(S, self.nb, block_pages.shape[-1]).reshape(
            self.Bp, -1).contiguous()
        self.all_obs = torch.ones((self.Bp, W), dtype=torch.uint8, device=device)
        self.order = {k: torch.empty(sh, **i32) for k, sh in (
            ("perm", (self.Bp, W)), ("inv", (self.Bp, W)), ("pos", (self.Bp, W)),
            ("n_obs", (self.Bp,)), ("run", (self.Bp,)))}
        self.out = torch.empty((1, self.Bp, W, Hq, D), dtype=dtype, device=device)
        self.ws_bytes = W_.wedlm_window_attn_workspace_size(dt, 1, self.Bp, W, Hq, Hkv, D, PAGE,
                                                            N - W)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=device)


class DualStreamAttention:
    """Buffers and launches of one dual-stream attention layer for fixed shapes.

    S samples of N positions, blocks of Bk (N % Bk == 0, N % 16 == 0), bf16
    (D = 128) or f32 projections [S, N, H, D] of both streams.
    """

    MEMORY_WINDOW = 16        # memory-stream window of the window kernel
    MEMORY_WINDOW_BLOCK = 64  # and of the block kernel (when N is a multiple of it)

    def __init__(self, S, N, Bk, Hq, Hkv, D, theta, dtype, device, scale=None, kernel=None):
        """kernel: "block" (wedlm_block_attn_rope), "window"
        (wedlm_window_attn_rope) or None for the block kernel where it has
        one."""
        if N % Bk or N % PAGE or not (1 <= Bk <= W_.MAX_WINDOW):
            raise ValueError("N must be a multiple of Bk and of 16, and Bk <= 64")
        has_block = dtype == torch.bfloat16 and D == 128 and 256 % (Hq // Hkv) == 0
        if kernel is None:
            kernel = "block" if has_block else "window"
        if kernel not in ("block", "window") or (kernel == "block" and not has_block):
            raise ValueError(f"no {kernel!r} attention kernel for these shapes")
        self.kernel = kernel
        self.S, self.N, self.Bk, self.Hq, self.Hkv, self.D = S, N, Bk, Hq, Hkv, D
        self.theta = theta
        self.dt = W_.dtype_code(dtype)
        self.scale = D ** -0.5 if scale is None else scale
        self.max_pages = N // PAGE
        self.num_pages = S * self.max_pages
        i32 = dict(dtype=torch.int32, device=device)
        # one page list per sample, shared by the block-table rows of all its blocks
        pages = torch.arange(self.num_pages, **i32).view(S, 1, self.max_pages)
        self.sample_table = pages.view(S, self.max_pages)
        self.memory_window = (self.MEMORY_WINDOW_BLOCK
                              if kernel == "block" and N % self.MEMORY_WINDOW_BLOCK == 0
                              else self.MEMORY_WINDOW)
        self.mem_blocks = _Blocks(S, N, self.memory_window, Hq, Hkv, D, self.dt, dtype, device,
                                  pages)
        self.pred_blocks = _Blocks(S, N, Bk, Hq, Hkv, D, self.dt, dtype, device, pages)
        self.mem, self.pred = self.mem_blocks.order, self.pred_blocks.order
        X = 16 // torch.tensor([], dtype=dtype).element_size()
        self.k_cache = torch.empty((1, self.num_pages, Hkv, D // X, PAGE, X), dtype=dtype,
                                   device=device)
        self.v_cache = torch.empty((1, self.num_pages, Hkv, D, PAGE), dtype=dtype, device=device)
        # scratch window state for the commit call over the memory windows (its
        # state half is not used)
        m = self.mem_blocks
        self.tokens = torch.empty((m.Bp, m.W), **i32)
        self.filled_scratch = torch.empty((m.Bp, m.W), dtype=torch.uint8, device=device)
        self.len_scratch = torch.empty((m.Bp,), **i32)
        self.commit_len = torch.empty((m.Bp,), **i32)
        self.cache_slot = torch.empty((m.Bp, m.W), **i32)
        self.selected = torch.zeros((m.Bp, m.W), dtype=torch.uint8, device=device)
        self.argmax = torch.zeros((m.Bp, m.W), **i32)
        # the memory stream's output in Bk-key blocks: the same memory (identity order)
        self.out_mem = m.out.view(1, S * N // Bk, Bk, Hq, D)
        self.out_pred = self.pred_blocks.out

    def _view(self, x, H, blk):
        return x.reshape(1, blk.Bp, blk.W, H, self.D)

    def _reorder(self, filled, blk, stream):
        o = blk.order
        W_.wedlm_window_reorder(blk.Bp, blk.W, filled, blk.prefix_len, o["perm"], o["inv"],
                                o["pos"], o["n_obs"], o["run"], stream)

    def _attend(self, q, k, v, blk, stream):
        o = blk.order
        if self.kernel == "block":
            W_.wedlm_block_attn_rope(self.dt, self.S, self.N, blk.W, self.Hq, self.Hkv, self.D,
                                     PAGE, self.num_pages, self.max_pages, self.scale, self.theta,
                                     q, k, v, o["perm"], o["pos"], self.k_cache, self.v_cache,
                                     self.sample_table, blk.out, stream)
            return
        W_.wedlm_window_attn_rope(self.dt, 1, blk.Bp, blk.W, self.Hq, self.Hkv, self.D, PAGE,
                                  self.num_pages, self.max_pages, self.N - blk.W, self.scale,
                                  self.theta, q, k, v, o["perm"], o["pos"], self.k_cache,
                                  self.v_cache, blk.block_table, blk.prefix_len, None, blk.out,
                                  blk.ws if blk.ws_bytes else None, blk.ws_bytes,
                                  flags=W_.WEDLM_ATTN_SHARED_PAGES, stream=stream)

    def forward(self, q_mem, k_mem, v_mem, q_pred, k_pred, v_pred, filled, stream=None):
        """q_* [S, N, Hq, D], k_* / v_* [S, N, Hkv, D] (slot order, before RoPE),
        filled [S, N] uint8 (the prediction stream's observed positions).

        Returns (out_mem, out_pred): [1, S * N / Bk, Bk, Hq, D] each, block
        rows in physical order (the memory stream's is its slot order);
        ``self.pred["inv"]`` maps a prediction slot to its physical row.
        """
        m, p = self.mem_blocks, self.pred_blocks
        qm, km, vm = (self._view(q_mem, self.Hq, m), self._view(k_mem, self.Hkv, m),
                      self._view(v_mem, self.Hkv, m))
        qp, kp, vp = (self._view(q_pred, self.Hq, p), self._view(k_pred, self.Hkv, p),
                      self._view(v_pred, self.Hkv, p))
        # 1. the memory stream's rotated keys and values into the paged cache
        self._reorder(m.all_obs, m, stream)
        self.filled_scratch.copy_(m.all_obs)
        self.len_scratch.copy_(m.prefix_len)
        W_.wedlm_commit_prefix_rope(self.dt, 1, m.Bp, m.W, self.Hkv, self.D, PAGE,
                                    self.num_pages, self.max_pages, self.theta, m.order["run"],
                                    self.selected, self.argmax, km, vm, m.block_table,
                                    self.k_cache, self.v_cache, self.tokens, self.filled_scratch,
                                    self.len_scratch, self.commit_len, self.cache_slot, -1, stream)
        # 2. memory stream: causal over the memory prefix and its own window
        self._attend(qm, km, vm, m, stream)
        # 3. prediction stream: reordered blocks over the memory prefix
        self._reorder(filled.reshape(p.Bp, p.W), p, stream)
        self._attend(qp, kp, vp, p, stream)
        return self.out_mem, self.out_pred
