"""Algorithmic bytes and FLOPs of MLA / GQLA decode, and the roofline they imply.

Pure arithmetic on shapes, used by the benchmark to price a kernel launch. Units follow
the method's own accounting of decode traffic: every new token rereads the whole cached
history (cours.spawnkit.ai session 18 slides, trainer notes on the MLA slide), and decode
is bound by that cache traffic (GQLA summary, section 1).

Per (query token x visible cached position), absorbed form (GQLA summary, section 2,
"Chemin MQA-Absorbé"):
  * bytes: one latent row (d_c + d_r) * elt, read once per step whatever s_q is;
  * FLOPs: 2*H*(d_c + d_r) for the scores plus 2*H*d_c for the weighted latent sum.
Per (query token x visible cached position), GQA form ("Chemin GQA"):
  * bytes: one expanded row (2*g*d_h + d_r) * elt;
  * FLOPs: 2*H*(d_h + d_r) + 2*H*d_h.
"""
from __future__ import annotations

# MI355X published peaks (dense).
HBM_PEAK_GBS = 8000.0          # GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # TFLOP/s
FP32_VALU_PEAK_TFLOPS = 157.3


def latent_row_bytes(d_c: int, d_r: int, elt: int = 2) -> int:
    return (d_c + d_r) * elt


def gqa_row_bytes(n_groups: int, d_h: int, d_r: int, elt: int = 2) -> int:
    return (2 * n_groups * d_h + d_r) * elt


def absorbed_flops_per_pos(n_heads: int, d_c: int, d_r: int) -> int:
    """FLOPs per (query token, visible position): scores over d_c + d_r, P·C over d_c."""
    return 2 * n_heads * (d_c + d_r) + 2 * n_heads * d_c


def gqa_flops_per_pos(n_heads: int, d_h: int, d_r: int) -> int:
    return 2 * n_heads * (d_h + d_r) + 2 * n_heads * d_h


def absorbed_intensity(n_heads: int, d_c: int, d_r: int, s_q: int = 1, elt: int = 2) -> float:
    """FLOP per cache byte of the absorbed path: s_q query tokens share one read of a row."""
    return s_q * absorbed_flops_per_pos(n_heads, d_c, d_r) / latent_row_bytes(d_c, d_r, elt)


def gqa_intensity(n_heads: int, n_groups: int, d_h: int, d_r: int, s_q: int = 1,
                  elt: int = 2) -> float:
    return s_q * gqa_flops_per_pos(n_heads, d_h, d_r) / gqa_row_bytes(n_groups, d_h, d_r, elt)


def mha_cache_bytes_per_token(layers: int, kv_heads: int, d_head: int, elt: int) -> int:
    """Standard cache: keys and values of every KV head, every layer."""
    return layers * 2 * kv_heads * d_head * elt


def latent_cache_bytes_per_token(layers: int, d_c: int, d_r: int, elt: int) -> int:
    return layers * (d_c + d_r) * elt


def roofline_tokens_per_s(ctx: int, bytes_per_pos: float, flops_per_pos: float,
                          bw_bytes_per_s: float, flops_per_s: float) -> float:
    """Query tokens/s of one layer when each step reads ctx rows: min of the two ceilings."""
    t = max(ctx * bytes_per_pos / bw_bytes_per_s, ctx * flops_per_pos / flops_per_s)
    return 1.0 / t


def fp8_row_bytes(d_c: int, d_r: int) -> int:
    """An e4m3 latent row: one byte per value plus its fp32 scale."""
    return d_c + d_r + 4


def decode_traffic(lens, s_q: int, n_heads: int, d_c: int, d_r: int, d_v: int,
                   n_groups: int, elt: int = 2, row_bytes: int = 0) -> dict:
    """Algorithmic bytes and FLOPs of one absorbed decode call over sequences of lengths lens.

    Split-K core: every cache row once (row_bytes each, default (d_c + d_r) * elt), the
    absorbed queries once. Combine: W_UV once, the outputs once.
    """
    rows = sum(int(L) for L in lens)
    B = len(lens)
    vis = sum(sum(int(L) - s_q + i + 1 for i in range(s_q)) for L in lens)
    rb = row_bytes or latent_row_bytes(d_c, d_r, elt)
    core_bytes = rows * rb + B * s_q * n_heads * (d_c + d_r) * elt
    core_flops = vis * absorbed_flops_per_pos(n_heads, d_c, d_r)
    wuv_bytes = d_c * n_groups * d_v * elt + B * s_q * n_heads * d_v * elt
    wuv_flops = 2 * B * s_q * n_heads * d_c * d_v
    return {"core_bytes": core_bytes, "core_flops": core_flops,
            "combine_bytes": wuv_bytes, "combine_flops": wuv_flops,
            "bytes": core_bytes + wuv_bytes, "flops": core_flops + wuv_flops,
            "cache_bytes": rows * rb}


def gqa_decode_traffic(lens, s_q: int, n_heads: int, n_groups: int, d_h: int, d_r: int,
                       elt: int = 2) -> dict:
    rows = sum(int(L) for L in lens)
    vis = sum(sum(int(L) - s_q + i + 1 for i in range(s_q)) for L in lens)
    B = len(lens)
    b = rows * gqa_row_bytes(n_groups, d_h, d_r, elt) + B * s_q * n_heads * (2 * d_h + d_r) * elt
    return {"bytes": b, "flops": vis * gqa_flops_per_pos(n_heads, d_h, d_r),
            "cache_bytes": rows * gqa_row_bytes(n_groups, d_h, d_r, elt)}


def binding_roofline(nbytes: float, flops: float, ms: float,
                     hbm_gbs: float = HBM_PEAK_GBS,
                     mfma_tflops: float = MFMA_BF16_PEAK_TFLOPS) -> dict:
    """The binding roofline of a launch that moves nbytes and does flops in ms: the larger of
    its HBM time (nbytes at the HBM peak) and its matrix-core time (flops at the bf16 peak),
    and the fraction of that bound achieved, beside both fractions."""
    t_hbm = nbytes / (hbm_gbs * 1e9)
    t_mfma = flops / (mfma_tflops * 1e12)
    t = ms * 1e-3
    return {"bound": "hbm" if t_hbm >= t_mfma else "mfma",
            "frac": max(t_hbm, t_mfma) / t, "frac_hbm": t_hbm / t, "frac_mfma": t_mfma / t,
            "roofline_ms": max(t_hbm, t_mfma) * 1e3}
