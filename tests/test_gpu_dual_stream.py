"""Dual-stream masking attention on the GPU against the oracle.

Every output row of both streams is compared (prediction rows mapped from the
block's physical order back to slot order) with the attention bar
|gpu - ref| <= 2e-3 + 1e-2 |ref|; the oracle rounds the rotated rows to bf16
as the GPU stores them. Cases: block sizes 16, 32 and 64 (M = 256 rows),
GQA 4 and 7 and MHA, random, all-observed and all-masked prediction streams,
several samples, and a 1024-position sequence (64 blocks); each through the
block kernel (wedlm_block_attn_rope, where it has one) and the window kernel
(wedlm_window_attn_rope). Block-kernel shapes: a ragged last workgroup, a
window split across two workgroups (g = 8, 64-key blocks), two own-key tiles
per workgroup (g = 2, MHA), one-slot blocks.
"""

import numpy as np
import pytest
import torch

import oracle
from causal_streaming_decoding_amd.dual_stream import DualStreamAttention
from causal_streaming_decoding_amd.synth import to_f64

from .parity import ATTN_ATOL, ATTN_RTOL, storage_rounding

pytestmark = pytest.mark.gpu


CASES = [
    (2, 256, 16, 8, 2, "random"),
    (1, 256, 32, 28, 4, "random"),     # GQA 7, 224 query rows per block and kv head
    (1, 256, 64, 8, 2, "random"),      # 256 query rows per block and kv head
    (3, 128, 16, 4, 4, "all"),         # MHA; prediction stream fully observed
    (1, 128, 16, 8, 2, "none"),        # prediction stream fully masked
    (1, 1024, 16, 8, 2, "random"),     # 64 blocks: prefixes up to 1008
    (2, 128, 8, 8, 2, "random"),       # blocks smaller than the memory stream's 16-key windows
    (1, 96, 16, 8, 2, "random"),       # block kernel: 64 positions per workgroup, the last ragged
    (1, 256, 64, 16, 2, "random"),     # block kernel only: g = 8, a window across two workgroups
    (1, 512, 32, 4, 2, "random"),      # block kernel: g = 2, two own-key tiles per workgroup
    (1, 384, 16, 4, 4, "random"),      # block kernel: MHA, 256 positions per workgroup, ragged
    (1, 64, 1, 8, 2, "random"),        # one-slot blocks
]


def _params():
    for c in CASES:
        g = c[3] // c[4]
        # the block kernel needs 256 % g == 0; the window kernel W * g <= 256 rows
        kernels = [k for k, ok in (("block", 256 % g == 0), ("window", max(c[2], 16) * g <= 256))
                   if ok]
        for kern in kernels:
            yield pytest.param(*c, kern, id=f"S{c[0]}-N{c[1]}-Bk{c[2]}-{c[3]}x{c[4]}-{c[5]}-{kern}")


@pytest.mark.parametrize("S,N,Bk,Hq,Hkv,fill,kernel", list(_params()))
def test_dual_stream_parity(S, N, Bk, Hq, Hkv, fill, kernel):
    print(f"[dual] S={S} N={N} Bk={Bk} Hq={Hq} Hkv={Hkv} fill={fill} kernel={kernel}", flush=True)
    D, theta = 128, 1e6
    g = torch.Generator(device="cuda").manual_seed(N + Bk + Hq)
    r = lambda h: torch.randn((S, N, h, D), generator=g, device="cuda").to(torch.bfloat16)
    qm, km, vm, qp, kp, vp = r(Hq), r(Hkv), r(Hkv), r(Hq), r(Hkv), r(Hkv)
    if fill == "random":
        filled = (torch.rand((S, N), generator=g, device="cuda") < 0.5).to(torch.uint8)
    else:
        filled = torch.full((S, N), 1 if fill == "all" else 0, dtype=torch.uint8, device="cuda")
    ds = DualStreamAttention(S, N, Bk, Hq, Hkv, D, theta, torch.bfloat16, "cuda", kernel=kernel)
    out_m, out_p = ds.forward(qm, km, vm, qp, kp, vp, filled)
    torch.cuda.synchronize()
    nb = N // Bk
    om = to_f64(out_m).reshape(S, N, Hq, D)
    op_phys = to_f64(out_p).reshape(S, nb, Bk, Hq, D)
    inv = ds.pred["inv"].cpu().numpy().reshape(S, nb, Bk)
    store = storage_rounding("bf16")
    worst = 0.0
    for s in range(S):
        op = np.stack([op_phys[s, j, inv[s, j]] for j in range(nb)]).reshape(N, Hq, D)
        rm, rp = oracle.dual_stream_attention(
            to_f64(qm[s]), to_f64(km[s]), to_f64(vm[s]), to_f64(qp[s]), to_f64(kp[s]),
            to_f64(vp[s]), filled[s].cpu().numpy().astype(bool), Bk, theta, store=store)
        for name, gv, rv in (("memory", om[s], rm), ("prediction", op, rp)):
            err = np.abs(gv - rv)
            ok = err <= ATTN_ATOL + ATTN_RTOL * np.abs(rv)
            assert ok.all(), (name, s, float(err.max()), int((~ok).sum()))
            worst = max(worst, float(err.max()))
    print(f"[dual] max abs err {worst:.2e}", flush=True)
