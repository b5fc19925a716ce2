"""Window-step driver: the C entry points in order on one stream.

hyper.ai summary of WeDLM, "Method" (Streaming Parallel Decoding): reorder the
window, run the causal forward over it against the KV cache, select by
distance-penalised entropy, commit the leftmost filled run and refill. Here the
forward's projections and logits are inputs (synthetic), so one step is:
reorder -> RoPE at logical positions -> window attention -> entropy/select ->
commit. With ``fused_rope`` (the default) the RoPE step runs inside the
attention and commit calls (wedlm_window_attn_rope, wedlm_commit_prefix_rope)
instead of as its own pass over the window. With ``fused_tail`` the selection,
the window-state commit and the next step's reorder run as one call
(wedlm_select_commit_reorder), so a chain of steps is one reorder followed by
(attention, tail) pairs; for bf16 the entropy chunk pass then rides in the
attention's launch (wedlm_window_attn_rope_entropy, then
wedlm_select_commit_reorder_partials). Device buffers are allocated once; ``run`` only
enqueues kernels and never synchronises, so steps can be chained or timed back
to back.
"""

from dataclasses import dataclass, field

import torch

from . import wedlm as W_


@dataclass
class StreamState:
    """Device-resident decoding state of a batch of sequences."""
    tokens: torch.Tensor       # [B, W] int32, mask id where not filled
    filled: torch.Tensor       # [B, W] uint8
    prefix_len: torch.Tensor   # [B] int32
    block_table: torch.Tensor  # [B, max_pages] int32
    k_cache: torch.Tensor      # [nl, num_pages, Hkv, D/X, P, X]
    v_cache: torch.Tensor      # [nl, num_pages, Hkv, D, P]
    # the WindowStep whose perm / pos / run_len hold the reorder of this
    # window as it stands (set by the fused tail); code that edits the window
    # by hand sets it to None so that the next step reorders first
    ordered_by: object = field(default=None, compare=False, repr=False)

    def snapshot(self):
        return (self.tokens.clone(), self.filled.clone(), self.prefix_len.clone())

    def restore(self, snap):
        self.tokens.copy_(snap[0])
        self.filled.copy_(snap[1])
        self.prefix_len.copy_(snap[2])
        self.ordered_by = None


class WindowStep:
    """Buffers and launches of one window step for fixed shapes."""

    def __init__(self, n_layers, B, W, Hq, Hkv, D, V, page_size, num_pages, max_pages, dtype,
                 device, max_prefix_len, theta, lam, tau, min_fill=1, mask_id=-1, scale=None,
                 fused_rope=True, commit_rule=W_.COMMIT_STREAM, fused_tail=False):
        self.n_layers, self.B, self.W, self.Hq, self.Hkv, self.D, self.V = (
            n_layers, B, W, Hq, Hkv, D, V)
        self.page_size, self.num_pages, self.max_pages = page_size, num_pages, max_pages
        self.dtype, self.device = dtype, device
        self.dt = W_.dtype_code(dtype)
        self.theta, self.lam, self.tau, self.min_fill, self.mask_id = theta, lam, tau, min_fill, mask_id
        self.scale = scale if scale is not None else D ** -0.5
        self.max_prefix_len = max_prefix_len
        self.fused_rope = fused_rope
        # COMMIT_STREAM: the leading filled run; COMMIT_BLOCK: the whole window once filled
        self.commit_rule = commit_rule
        # fused path: the attention call appends the committed rows (else the
        # commit call writes them itself)
        self.fused_append = True
        # selection + state commit + next reorder in one call (needs fused_rope
        # and fused_append: the rows must be in the cache before the tail)
        self.fused_tail = fused_tail
        i32 = dict(dtype=torch.int32, device=device)
        self.perm = torch.empty((B, W), **i32)
        self.inv = torch.empty((B, W), **i32)
        self.pos = torch.empty((B, W), **i32)
        self.n_obs = torch.empty((B,), **i32)
        self.run_len = torch.empty((B,), **i32)
        fl = dict(dtype=dtype, device=device)
        # physical-order rotated copies: only the unfused path writes them
        self.q_phys = self.k_phys = self.v_phys = None
        if not fused_rope:
            self.q_phys = torch.empty((n_layers, B, W, Hq, D), **fl)
            self.k_phys = torch.empty((n_layers, B, W, Hkv, D), **fl)
            self.v_phys = torch.empty((n_layers, B, W, Hkv, D), **fl)
        self.out_phys = torch.empty((n_layers, B, W, Hq, D), **fl)
        self.entropy = torch.empty((B, W), dtype=torch.float32, device=device)
        self.score = torch.empty((B, W), dtype=torch.float32, device=device)
        self.argmax = torch.empty((B, W), **i32)
        self.selected = torch.empty((B, W), dtype=torch.uint8, device=device)
        self.commit_len = torch.empty((B,), **i32)
        self.cache_slot = torch.empty((B, W), **i32)
        self._size_attn_workspace(max_prefix_len)
        self.ent_ws_bytes = W_.wedlm_entropy_select_workspace_size(self.dt, B, W, V)
        self.ent_ws = torch.empty((max(self.ent_ws_bytes, 1),), dtype=torch.uint8, device=device)
        # optional side stream for the entropy chunk pass (set_overlap)
        self.overlap = None
        # fused tail on bf16: the entropy chunk blocks run in the attention's
        # launch (wedlm_window_attn_rope_entropy); they fill the CUs the
        # attention leaves idle (measured faster on every workload)
        self.fuse_entropy = dtype == torch.bfloat16
        # with the entropy in the attention's launch, the merge of split
        # attention partials runs in the tail's launch
        # (wedlm_select_commit_reorder_combine) instead of a launch of its own
        self.defer_combine = True
        self._ev_in = self._ev_ent = None

    def _size_attn_workspace(self, max_prefix_len):
        self.attn_ws_bytes = W_.wedlm_window_attn_workspace_size(
            self.dt, self.n_layers, self.B, self.W, self.Hq, self.Hkv, self.D, self.page_size,
            max_prefix_len)
        self.attn_ws = torch.empty((max(self.attn_ws_bytes, 1),), dtype=torch.uint8,
                                   device=self.device)

    # -- the five calls -------------------------------------------------------
    def reorder(self, st, stream=None):
        W_.wedlm_window_reorder_rule(self.B, self.W, self.commit_rule, st.filled, st.prefix_len,
                                     self.perm, self.inv, self.pos, self.n_obs, self.run_len,
                                     stream)
        st.ordered_by = self

    def ordered(self, st):
        """Whether perm / pos / run_len already hold the reorder of ``st``."""
        return st.ordered_by is self

    def rope(self, q, k, v, stream=None):
        W_.wedlm_rope_logical(self.dt, self.n_layers, self.B, self.W, self.Hq, self.Hkv, self.D,
                              self.theta, q, k, v, self.perm, self.pos, self.q_phys, self.k_phys,
                              self.v_phys, stream)

    def _attn_mpl(self, max_prefix_len):
        mpl = self.max_prefix_len if max_prefix_len is None else max_prefix_len
        need = W_.wedlm_window_attn_workspace_size(self.dt, self.n_layers, self.B, self.W, self.Hq,
                                                   self.Hkv, self.D, self.page_size, mpl)
        if need > self.attn_ws_bytes:
            self._size_attn_workspace(mpl)
        return mpl

    def attn(self, st, max_prefix_len=None, stream=None):
        mpl = self._attn_mpl(max_prefix_len)
        W_.wedlm_window_attn(self.dt, self.n_layers, self.B, self.W, self.Hq, self.Hkv, self.D,
                             self.page_size, self.num_pages, self.max_pages, mpl, self.scale,
                             self.q_phys, self.k_phys, self.v_phys, st.k_cache, st.v_cache,
                             st.block_table, st.prefix_len, self.out_phys, self.attn_ws,
                             self.attn_ws_bytes, stream=stream)

    def attn_rope(self, st, q, k, v, max_prefix_len=None, stream=None, append=True):
        """Attention with RoPE fused; ``append`` also writes the rows the commit
        will commit (run_len from this step's reorder) into the caches."""
        mpl = self._attn_mpl(max_prefix_len)
        W_.wedlm_window_attn_rope(self.dt, self.n_layers, self.B, self.W, self.Hq, self.Hkv,
                                  self.D, self.page_size, self.num_pages, self.max_pages, mpl,
                                  self.scale, self.theta, q, k, v, self.perm, self.pos,
                                  st.k_cache, st.v_cache, st.block_table, st.prefix_len,
                                  self.run_len if append else None, self.out_phys, self.attn_ws,
                                  self.attn_ws_bytes, stream=stream)

    def entropy_select(self, st, logits, stream=None):
        W_.wedlm_entropy_select(self.dt, self.B, self.W, self.V, logits, st.filled, self.lam,
                                self.tau, self.min_fill, self.entropy, self.score, self.argmax,
                                self.selected, self.ent_ws, self.ent_ws_bytes, stream)

    def commit_rope(self, st, k, v, commit_len=None, stream=None):
        """Fused commit; k = v = None when attn_rope appended the rows already."""
        W_.wedlm_commit_prefix_rope(self.dt, self.n_layers, self.B, self.W, self.Hkv, self.D,
                                    self.page_size, self.num_pages, self.max_pages, self.theta,
                                    self.run_len, self.selected, self.argmax, k, v,
                                    st.block_table, st.k_cache, st.v_cache, st.tokens, st.filled,
                                    st.prefix_len,
                                    self.commit_len if commit_len is None else commit_len,
                                    self.cache_slot, self.mask_id, stream)

    def select_commit_reorder(self, st, logits, commit_len=None, stream=None):
        """Fused tail: selection, window-state commit (rows already appended)
        and the reorder of the refreshed window for the next step."""
        W_.wedlm_select_commit_reorder(
            self.dt, self.B, self.W, self.V, logits, self.lam, self.tau, self.min_fill,
            self.page_size, self.num_pages, self.max_pages, self.commit_rule, st.block_table,
            self.run_len, st.tokens, st.filled, st.prefix_len,
            self.commit_len if commit_len is None else commit_len, self.cache_slot, self.mask_id,
            self.entropy, self.score, self.argmax, self.selected, self.perm, self.inv, self.pos,
            self.n_obs, self.ent_ws, self.ent_ws_bytes, stream)
        st.ordered_by = self

    def commit(self, st, commit_len=None, stream=None):
        W_.wedlm_commit_prefix(self.dt, self.n_layers, self.B, self.W, self.Hkv, self.D,
                               self.page_size, self.num_pages, self.max_pages, self.run_len,
                               self.selected, self.argmax, self.k_phys, self.v_phys,
                               st.block_table, st.k_cache, st.v_cache, st.tokens, st.filled,
                               st.prefix_len, self.commit_len if commit_len is None else commit_len,
                               self.cache_slot, self.mask_id, stream)

    def run(self, st, q, k, v, logits, max_prefix_len=None, commit_len=None, stream=None,
            mark=None):
        """One whole window step.

        ``mark``: optional callable invoked with "attn_start", "attn_end" (also
        the start of entropy/select) and "entropy_end" at those points of the
        launch sequence, e.g. to record timing events on ``stream``. With the
        fused tail "entropy_end" follows the whole tail (selection, state
        commit and the next reorder).

        With the fused tail, perm / inv / pos / n_obs / run_len hold the next
        step's order when ``run`` returns (the order this step used is what
        they held before it, or what its own first reorder wrote).
        """
        tail = self.fused_tail and self.fused_rope and self.fused_append
        if not (tail and self.ordered(st)):
            self.reorder(st, stream)
        if tail and self.overlap is not None:
            self._run_overlapped(st, q, k, v, logits, max_prefix_len, commit_len, stream, mark)
            return
        if tail and self.fuse_entropy:
            # the entropy chunk blocks ride in the attention's launch
            if mark is not None:
                mark("attn_start")
            mpl = self._attn_mpl(max_prefix_len)
            flags = W_.WEDLM_ATTN_DEFER_COMBINE if self.defer_combine else 0
            W_.wedlm_window_attn_rope_entropy(
                self.dt, self.n_layers, self.B, self.W, self.Hq, self.Hkv, self.D,
                self.page_size, self.num_pages, self.max_pages, mpl, self.scale, self.theta, q, k,
                v, self.perm, self.pos, st.k_cache, st.v_cache, st.block_table, st.prefix_len,
                self.run_len, self.out_phys, self.attn_ws, self.attn_ws_bytes, flags, self.V,
                logits, self.ent_ws, self.ent_ws_bytes, stream)
            if mark is not None:
                mark("attn_end")
            if self.defer_combine:
                self._tail_combine(st, commit_len, stream, mpl)
            else:
                self._tail_from_partials(st, commit_len, stream)
            if mark is not None:
                mark("entropy_end")
            return
        if not self.fused_rope:
            self.rope(q, k, v, stream)
        if mark is not None:
            mark("attn_start")
        if self.fused_rope:
            self.attn_rope(st, q, k, v, max_prefix_len, stream, append=self.fused_append)
        else:
            self.attn(st, max_prefix_len, stream)
        if mark is not None:
            mark("attn_end")
        if tail:
            self.select_commit_reorder(st, logits, commit_len, stream)
            if mark is not None:
                mark("entropy_end")
            return
        self.entropy_select(st, logits, stream)
        if mark is not None:
            mark("entropy_end")
        self._commit_after_select(st, k, v, commit_len, stream)

    def _run_overlapped(self, st, q, k, v, logits, max_prefix_len, commit_len, stream, mark):
        """The fused-tail step with the entropy chunk pass on ``self.overlap``.

        The chunk pass reads only the logits, so it runs on the side stream
        while the attention runs on the main one; it starts after everything
        already enqueued on the main stream (the previous step's tail reads
        the same partials), and the tail waits for it.
        """
        main = torch.cuda.current_stream() if stream is None else stream
        side = self.overlap
        self._ev_in.record(main)
        side.wait_event(self._ev_in)
        W_.wedlm_entropy_partials(self.dt, self.B, self.W, self.V, logits, self.ent_ws,
                                  self.ent_ws_bytes, side)
        self._ev_ent.record(side)
        if mark is not None:
            mark("attn_start")
        self.attn_rope(st, q, k, v, max_prefix_len, main, append=True)
        if mark is not None:
            mark("attn_end")
        main.wait_event(self._ev_ent)
        self._tail_from_partials(st, commit_len, main)
        if mark is not None:
            mark("entropy_end")

    def _tail_from_partials(self, st, commit_len, stream):
        """Selection, state commit and next reorder from the chunk partials
        already in the entropy workspace."""
        W_.wedlm_select_commit_reorder_partials(
            self.dt, self.B, self.W, self.V, self.lam, self.tau, self.min_fill, self.page_size,
            self.num_pages, self.max_pages, self.commit_rule, st.block_table, self.run_len,
            st.tokens, st.filled, st.prefix_len,
            self.commit_len if commit_len is None else commit_len, self.cache_slot, self.mask_id,
            self.entropy, self.score, self.argmax, self.selected, self.perm, self.inv, self.pos,
            self.n_obs, self.ent_ws, self.ent_ws_bytes, stream)
        st.ordered_by = self

    def _tail_combine(self, st, commit_len, stream, max_prefix_len):
        """The tail from the chunk partials, with the merge of the attention's
        split partials (deferred by the attention call) in the same launch."""
        W_.wedlm_select_commit_reorder_combine(
            self.dt, self.B, self.W, self.V, self.lam, self.tau, self.min_fill, self.page_size,
            self.num_pages, self.max_pages, self.commit_rule, st.block_table, self.run_len,
            st.tokens, st.filled, st.prefix_len,
            self.commit_len if commit_len is None else commit_len, self.cache_slot, self.mask_id,
            self.entropy, self.score, self.argmax, self.selected, self.perm, self.inv, self.pos,
            self.n_obs, self.ent_ws, self.ent_ws_bytes, self.n_layers, self.Hq, self.Hkv, self.D,
            max_prefix_len, self.attn_ws, self.attn_ws_bytes, self.out_phys, stream)
        st.ordered_by = self

    def set_overlap(self, side_stream):
        """Run the entropy chunk pass on ``side_stream`` (a torch stream of
        default priority) beside the attention, or on the launch stream again
        when None. Only the fused-tail step uses it."""
        self.overlap = side_stream
        if side_stream is not None and self._ev_in is None:
            self._ev_in = torch.cuda.Event()
            self._ev_ent = torch.cuda.Event()

    def capture(self, st, q, k, v, logits, max_prefix_len=None, commit_len=None):
        """A HIP graph of one whole step (``run`` with these arguments), to replay.

        Every launch of the step becomes a kernel node (the step enqueues no
        copy or memset), so a replay costs one graph launch instead of one
        host call per kernel. The graph reads and writes the same device
        buffers at every replay: it runs the step on whatever window state
        ``st`` holds then (restore a snapshot between replays to repeat one
        step). It includes the reorder when ``st`` is not already ordered by
        this step; ``st.ordered_by`` is left as it was, since capturing runs
        nothing.
        """
        self._attn_mpl(max_prefix_len)  # any workspace growth happens before capture
        ordered = st.ordered_by
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            # stream=None: the library launches on the capturing stream
            self.run(st, q, k, v, logits, max_prefix_len=max_prefix_len, commit_len=commit_len)
        st.ordered_by = ordered
        return g

    def _commit_after_select(self, st, k, v, commit_len, stream):
        # the commit below changes the window without reordering it
        st.ordered_by = None
        if self.fused_rope and self.fused_append:
            # the committed rows were appended by attn_rope: window state only
            self.commit_rope(st, None, None, commit_len, stream)
        elif self.fused_rope:
            self.commit_rope(st, k, v, commit_len, stream)
        else:
            self.commit(st, commit_len, stream)


def upload_step_inputs(wl, inp, device):
    """Device state and window inputs from ``synth.make_step_inputs`` output.

    Returns (state, q, k, v, logits, max_prefix_len). Layers whose prefix cache
    was not drawn stay zero.
    """
    from . import layout
    from .synth import torch_dtype

    dt = torch_dtype(wl)
    table = torch.as_tensor(inp["block_table"], dtype=torch.int32)
    kc, vc = layout.alloc_caches(wl.n_layers, inp["num_pages"], wl.Hkv, wl.D, wl.page_size, dt,
                                 device)
    for layer in range(wl.n_layers):
        if inp["k_cache"][layer] is None:
            continue
        for b in range(wl.B):
            layout.write_rows(kc, vc, layer, table[b], 0, torch.from_numpy(inp["k_cache"][layer][b]),
                              torch.from_numpy(inp["v_cache"][layer][b]))
    st = StreamState(
        tokens=torch.as_tensor(inp["tokens"], dtype=torch.int32).to(device),
        filled=torch.as_tensor(inp["filled"], dtype=torch.uint8).to(device),
        prefix_len=torch.as_tensor(inp["prefix_len"], dtype=torch.int32).to(device),
        block_table=table.to(device), k_cache=kc, v_cache=vc)
    q = torch.from_numpy(inp["q"]).to(device=device, dtype=dt)
    k = torch.from_numpy(inp["k"]).to(device=device, dtype=dt)
    v = torch.from_numpy(inp["v"]).to(device=device, dtype=dt)
    logits = torch.from_numpy(inp["logits"]).to(device=device, dtype=dt)
    return st, q, k, v, logits, int(inp["prefix_len"].max())


def make_window_step(wl, inp, device, max_prefix_len, fused_rope=True, commit_rule=None,
                     fused_tail=False):
    """WindowStep sized for a workload and its inputs (streaming commits unless
    ``commit_rule`` says otherwise)."""
    from .synth import torch_dtype

    return WindowStep(wl.n_layers, wl.B, wl.W, wl.Hq, wl.Hkv, wl.D, wl.V, wl.page_size,
                      inp["num_pages"], inp["block_table"].shape[1], torch_dtype(wl), device,
                      max_prefix_len, wl.theta, wl.lam, wl.tau, wl.min_fill, wl.mask_id,
                      fused_rope=fused_rope,
                      commit_rule=W_.COMMIT_STREAM if commit_rule is None else commit_rule,
                      fused_tail=fused_tail)
