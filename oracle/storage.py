"""Effective KV bit width and storage accounting (test infrastructure).

The ResidualQuant page ("ResidualQuant: KV Cache Quantization for Looped
Transformers with 2-Bit Residuals") prints effective bit widths b_eff
(Table 5, Table 8, Table 10) and an 80.7% storage reduction (Abstract,
Fig. 1).  Table 8's caption says b_eff counts the codes, the scales and
offsets, and the LS coefficients; the appendix that defines it is not on the
pages.  The plainest accounting that reproduces every printed value is

    per stored value:  b + M/g          for a directly quantized loop (or anchor)
                       b + M/g + A/d    for a residual loop (plus its LS coefficient)
                       16               for a BF16 loop

averaged over the loops of the schedule, with M = 16 bits of scale+offset per
group and A = 16 bits of LS coefficient per head_dim vector.  In the layout
this library stores, M = 32 (FP16 scale and FP16 zero) and the reference loop
is BF16; `layout_bits_per_value` reports that.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List


@dataclass(frozen=True)
class Loop:
    kind: str       # "residual", "direct" (also a quantized anchor) or "bf16"
    bits: int = 16
    g: int = 0


def loop_bits(loop: Loop, d: int, meta_bits: int = 16, alpha_bits: int = 16) -> float:
    if loop.kind == "bf16":
        return 16.0
    b = loop.bits + meta_bits / loop.g
    if loop.kind == "residual":
        b += alpha_bits / d
    return b


def effective_bits(schedule: List[Loop], d: int, meta_bits: int = 16,
                   alpha_bits: int = 16) -> float:
    return sum(loop_bits(l, d, meta_bits, alpha_bits) for l in schedule) / len(schedule)


def uniform(bits: int, g: int, n_loops: int = 4, residual: bool = True) -> List[Loop]:
    """Uniform precision: every loop at `bits`.  With residuals, the final
    loop is the (directly quantized) reference and the others are residuals."""
    if not residual:
        return [Loop("direct", bits, g)] * n_loops
    return [Loop("residual", bits, g)] * (n_loops - 1) + [Loop("direct", bits, g)]


def anchored(n_groups: int, n_residual: int, g_res: int, res_bits: int = 2,
             anchor_bits: int = 4, anchor_g: int = 32) -> List[Loop]:
    """n_groups x [res_bits^(x n_residual), anchor_bits]: each group ends with
    one directly quantized anchor (Table 8 caption)."""
    group = [Loop("residual", res_bits, g_res)] * n_residual + [Loop("direct", anchor_bits, anchor_g)]
    return group * n_groups


def storage_reduction(schedule: List[Loop], d: int, **kw) -> float:
    return 1.0 - effective_bits(schedule, d, **kw) / 16.0


def layout_bits_per_value(n_loops: int, bits: List[int], g: int, d: int) -> float:
    """This library's stored layout: BF16 final loop; each earlier loop holds
    `bits[l]`-bit codes, an FP16 scale and an FP16 zero per group and one FP16
    LS coefficient per vector."""
    sched = [Loop("residual", bits[l], g) for l in range(n_loops - 1)] + [Loop("bf16")]
    return effective_bits(sched, d, meta_bits=32, alpha_bits=16)


def layout_bytes_per_token(n_loops: int, bits: List[int], g: int, d: int, ref_bits: int = 0,
                           ref_group: int = 0) -> int:
    """Bytes per (batch, head, token) for K plus V in this library's layout:
    the BF16 reference (ref_bits 0) or a quantized anchor (codes plus FP16
    scale and zero per group of ref_group), plus every residual loop."""
    ga = ref_group or g
    ref = 2 * d if not ref_bits else d * ref_bits // 8 + 4 * (d // ga)
    per_side = ref + sum(d * bits[l] // 8 + 4 * (d // g) + 2 for l in range(n_loops - 1))
    return 2 * per_side


def loop_read_bytes_per_token(bits: int, g: int, d: int, ref_bits: int = 0, ref_group: int = 0) -> int:
    """Bytes per (batch, head, token) that decoding ONE residual loop on its own
    reads (K plus V): the reference or anchor and that loop's planes."""
    ga = ref_group or g
    ref = 2 * d if not ref_bits else d * ref_bits // 8 + 4 * (d // ga)
    return 2 * (ref + d * bits // 8 + 4 * (d // g) + 2)
