"""Helpers shared by the parity tests: build the same seeded inputs for the
oracle (numpy, CPU) and for the HIP library (torch, GPU), and compare.

Nothing here computes any step of the method; the oracle and the library each
do their own arithmetic on the same inputs.
"""
from __future__ import annotations

import numpy as np
import torch

import synth
from synth import bf16_bits


def tol_rel_row(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    """Per row (last axis): max |got - want| / max |want|."""
    return np.abs(got - want).max(-1) / np.maximum(np.abs(want).max(-1), 1e-30)


def oracle_layout(w: synth.Workload, batch: int, cap: int) -> dict:
    return dict(n_loops=w.n_loops, batch=batch, heads=w.heads, d=w.d, g=w.g, cap=cap,
                rotate=w.rotate, bits=list(w.bits), ref_bits=w.ref_bits, ref_group=w.ref_group,
                group_loops=w.group_loops, ref_first=w.ref_first, alpha_mode=w.alpha_mode,
                ref_chain=w.ref_chain)


def gpu_layout(w: synth.Workload, batch: int, cap: int):
    import decode_attention_rq_amd as rq
    return rq.Layout(n_loops=w.n_loops, batch=batch, n_heads=w.heads, head_dim=w.d, group=w.g,
                     capacity=cap, rotate=w.rotate, bits=list(w.bits), ref_bits=w.ref_bits,
                     ref_group=w.ref_group, group_loops=w.group_loops, ref_first=w.ref_first,
                     alpha_mode=w.alpha_mode, ref_chain=w.ref_chain)


def encoder_input(w: synth.Workload, loops: torch.Tensor, ref: torch.Tensor) -> torch.Tensor:
    """rq_encode's input in loop order: with a BF16 reference the other loops;
    with quantized anchors every loop, the drawn reference being the first
    loop (First-loop policy) or the last."""
    if w.ref_bits:
        parts = [ref.unsqueeze(0), loops] if w.ref_first else [loops, ref.unsqueeze(0)]
        return torch.cat(parts)
    return loops


class Case:
    """One layer of workload `w` with `n` tokens in caches of capacity `cap`,
    encoded by the library on the GPU (planes on `device`)."""

    def __init__(self, w: synth.Workload, n: int, cap: int = 0, batch: int = 0, seed=None,
                 device="cuda", gen_device="cpu", t_chunks=None):
        import decode_attention_rq_amd as rq
        self.w, self.n = w, n
        self.B = batch or w.batch
        self.cap = cap or n
        self.data = synth.draw_layer(w, seed=seed, batch=self.B, n=n, device=gen_device)
        self.lay = gpu_layout(w, self.B, self.cap)
        self.k = rq.Cache(self.lay, device)
        self.v = rq.Cache(self.lay, device)
        if not w.ref_bits:
            self.k.ref[:, :, :n] = self.data["k_ref"].to(device)
            self.v.ref[:, :, :n] = self.data["v_ref"].to(device)
        self.q = self.data["q"].to(device).contiguous()
        kin = encoder_input(w, self.data["k_loops"], self.data["k_ref"]).to(device)
        vin = encoder_input(w, self.data["v_loops"], self.data["v_ref"]).to(device)
        chunks = t_chunks or [(0, n)]
        for t0, cnt in chunks:
            rq.rq_encode(self.lay, self.k, self.v, kin[:, :, :, t0:t0 + cnt].contiguous(),
                         vin[:, :, :, t0:t0 + cnt].contiguous(), t0, cnt)
        torch.cuda.synchronize()

    def oracle_planes(self, oracle, bh_list=None):
        """Oracle encode of the same inputs (all (b, h), or a list of them).
        Returns (layout, k_planes, v_planes, q_bits) restricted to the
        selected (b, h) pairs as a batch of len(bh_list) x 1 heads."""
        w, n = self.w, self.n
        if bh_list is None:
            B, H = self.B, w.heads
            sel = lambda t: t
        else:
            B, H = len(bh_list), 1
            dev = self.data["k_ref"].device
            bi = torch.tensor([b for b, _ in bh_list], device=dev)
            hi = torch.tensor([h for _, h in bh_list], device=dev)

            def sel(t, ax=0):
                # t has batch at axis ax and heads at ax+1
                idx = [slice(None)] * t.dim()
                idx[ax] = bi
                idx[ax + 1] = hi
                return t[tuple(idx)].unsqueeze(ax + 1)
        lay = oracle_layout(w, B, n)
        kp = oracle.Planes(w.n_loops, B, H, w.d, w.g, n, w.bits, w.ref_bits, w.ref_group or None,
                           w.group_loops, w.ref_first)
        vp = oracle.Planes(w.n_loops, B, H, w.d, w.g, n, w.bits, w.ref_bits, w.ref_group or None,
                           w.group_loops, w.ref_first)
        if bh_list is None:
            kr, vr, kl, vl, q = (self.data["k_ref"], self.data["v_ref"], self.data["k_loops"],
                                 self.data["v_loops"], self.data["q"])
        else:
            kr, vr = sel(self.data["k_ref"]).cpu(), sel(self.data["v_ref"]).cpu()
            kl, vl = sel(self.data["k_loops"], 1).cpu(), sel(self.data["v_loops"], 1).cpu()
            q = sel(self.data["q"], 1).cpu()
        lay["heads"] = H
        if w.ref_bits:
            oracle.encode(lay, kp, bf16_bits(encoder_input(w, kl, kr)), 0, n)
            oracle.encode(lay, vp, bf16_bits(encoder_input(w, vl, vr)), 0, n)
        else:
            kp.ref[:] = bf16_bits(kr)
            vp.ref[:] = bf16_bits(vr)
            oracle.encode(lay, kp, bf16_bits(kl), 0, n)
            oracle.encode(lay, vp, bf16_bits(vl), 0, n)
        return lay, kp, vp, bf16_bits(q)


def plane_bits(t: torch.Tensor) -> np.ndarray:
    """Device plane -> numpy bytes / uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
