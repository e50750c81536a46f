"""BF16-KV baseline decode (rq_bf16_decode_attn) against the oracle's FP64
softmax attention over the same BF16 caches, one cache per loop."""
import numpy as np
import pytest
import torch

import synth
from rq_testutil import tol_rel_row
from synth import bf16_bits

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d,n,cap,mask,splits", [(128, 700, 768, 0b1111, 0), (128, 700, 768, 0b0110, 3),
                                                  (128, 700, 768, 0b1001, 2), (64, 129, 129, 0b11, 1),
                                                  (256, 90, 96, 0b101, 2)])
def test_bf16_baseline(oracle, waves, d, n, cap, mask, splits):
    import decode_attention_rq_amd as rq
    L = 4 if d != 64 else 2
    B, H = 2, 3
    g = synth.generator(31)
    ks = [torch.zeros(B, H, cap, d, dtype=torch.bfloat16) for _ in range(L)]
    vs = [torch.zeros(B, H, cap, d, dtype=torch.bfloat16) for _ in range(L)]
    for l in range(L):
        ks[l][:, :, :n] = (torch.randn(B, H, n, d, generator=g) * 1.3).to(torch.bfloat16)
        vs[l][:, :, :n] = torch.randn(B, H, n, d, generator=g).to(torch.bfloat16)
    q = synth.draw_queries(g, L, B, H, d)
    lay = rq.Layout(L, B, H, d, 32, cap, 1, [2] * (L - 1))
    kd = [t.cuda() for t in ks]
    vd = [t.cuda() for t in vs]
    out = torch.full((L, B, H, d), float("nan"), device="cuda")
    ws = rq.workspace_for(lay, n, splits)
    scale = 1 / np.sqrt(d)
    rq.rq_bf16_decode_attn(lay, kd, vd, q.cuda().contiguous(), mask, n, scale, out, ws, splits)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    for l in range(L):
        if not (mask >> l) & 1:
            assert np.isnan(got[l]).all()
            continue
        for b in range(B):
            for h in range(H):
                want = oracle.attention(q[l, b, h].double().numpy(), ks[l][b, h, :n].double().numpy(),
                                        vs[l][b, h, :n].double().numpy(), scale)
                assert tol_rel_row(got[l, b, h], want) <= 2e-3
