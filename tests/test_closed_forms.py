"""Closed forms printed on the pages: cache bytes per token, intensity, projections.

Each expected number is a fixture in tests/golden/closed_forms.json with its citation.
Byte counts are checked both with the accounting formulas and on tensors laid out the way
the library lays out its caches ([num_blocks, block_size, row] for the latent cache,
[num_blocks, block_size, 2*g*d_h + d_r] for the expanded GQA cache).
"""
import json
import os

import pytest
import torch

from mla_latent_kv_21_amd import accounting as A
from mla_latent_kv_21_amd.layout import latent_cache_shape, gqa_cache_shape

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))
MiB = 1 << 20


def test_smallem_cache_sizes():
    g = GOLD
    mha = g["smallem_mha_numbers_per_position"]
    assert 2 * mha["heads"] * mha["d_head"] == mha["value"]
    m = g["smallem_mha_cache_bytes"]
    assert A.mha_cache_bytes_per_token(m["layers"], mha["heads"], mha["d_head"], m["elt"]) * m["ctx"] \
        == m["value"]
    lat = g["smallem_latent_plus_rope_numbers_per_position"]
    # one cache row of the library's layout holds exactly d_c + d_r numbers
    shape = latent_cache_shape(d_c=lat["d_c"], d_r=lat["d_r"], num_blocks=8, block_size=64)
    assert shape[-1] == lat["value"]
    # the whole Smallem context (512 positions) x 8 layers, fp32, in paged tensors
    t = torch.empty(latent_cache_shape(lat["d_c"], lat["d_r"], num_blocks=512 // 64, block_size=64),
                    dtype=torch.float32)
    total = 8 * t.numel() * t.element_size()
    assert total == g["smallem_latent_cache_mib"]["value"] * MiB
    assert m["value"] == g["smallem_latent_cache_mib"]["mha_mib"] * MiB
    assert m["value"] / total == pytest.approx(g["smallem_cache_ratio"]["value"], abs=1e-12)
    assert g["smallem_latent_numbers_per_position"]["value"] == \
        g["smallem_latent_numbers_per_position"]["d_c"]


def test_standard_cache_bytes():
    d = GOLD["dsv1_67b_bytes_per_token"]
    assert A.mha_cache_bytes_per_token(d["layers"], d["kv_heads"], d["d_head"], d["elt"]) == d["value"]
    assert d["value"] == 380 * 1024
    s = GOLD["slides_std_bytes_per_token"]
    per = A.mha_cache_bytes_per_token(s["layers"], s["kv_heads"], s["d_head"], s["elt"])
    assert per == s["value"]
    for k in ("slides_std_bytes_4096", "slides_std_bytes_8192", "slides_std_bytes_131072"):
        assert per * GOLD[k]["tokens"] == GOLD[k]["value"]
    assert A.mha_cache_bytes_per_token(s["layers"], s["kv_heads"], s["d_head"], 1) == \
        GOLD["slides_int8_bytes_per_token"]["value"]
    v = GOLD["slides_variant_dhead_x2"]
    per2 = A.mha_cache_bytes_per_token(s["layers"], s["kv_heads"], 2 * s["d_head"], s["elt"])
    assert per2 == v["bytes_per_token"] and per2 * 131072 == v["bytes_131072"]


def test_latent_cache_bytes():
    m = GOLD["slides_mla_bytes_per_token"]
    per = A.latent_cache_bytes_per_token(m["layers"], m["d_c"], 0, m["elt"])
    assert per == m["value"]
    for k in ("slides_mla_bytes_131072", "slides_mla_bytes_524288", "slides_mla_bytes_4096"):
        assert per * GOLD[k]["tokens"] == GOLD[k]["value"]
    h = GOLD["slides_variant_latent_half"]
    per_h = A.latent_cache_bytes_per_token(m["layers"], m["d_c"] // 2, 0, m["elt"])
    assert per_h == h["bytes_per_token"] and per_h * 131072 == h["bytes_131072"]
    # with the shared rotary key, one bf16 row of the DeepSeek-shaped cache is 1,152 B
    t = torch.empty(latent_cache_shape(512, 64, num_blocks=1, block_size=64), dtype=torch.bfloat16)
    assert t.numel() * t.element_size() // 64 == 1152 == A.latent_row_bytes(512, 64)


def test_gqa_cache_layout_and_fraction():
    f = GOLD["gqla_cache_fraction"]
    gqa_baseline = 2 * f["gqa_kv_heads"] * f["d_h"]
    assert (f["d_c"] + f["d_r"]) / gqa_baseline == f["value"]
    # expanded GQLA row at g = 8, d_h = 128: 2*g*d_h + d_r numbers, 4,224 B in bf16
    shp = gqa_cache_shape(n_groups=8, d_h=128, d_r=64, num_blocks=1, block_size=64)
    assert shp[-1] == 2 * 8 * 128 + 64
    assert A.gqa_row_bytes(8, 128, 64) == 4224


def test_intensity_matches_pages():
    a = GOLD["gqla_absorbed_intensity"]
    x = A.absorbed_intensity(a["h_q"], a["r_kv"], a["d_r"], s_q=1)
    assert round(x) == a["value"]
    r = GOLD["gqla_gqa_ridge_match"]
    for g, s_q in r["cases"]:
        y = A.gqa_intensity(r["h_q"], g, r["d_h"], r["d_r"], s_q=s_q)
        assert abs(y - r["value"]) / r["value"] < 0.05, (g, s_q, y)


def test_projections_reproduce():
    p = GOLD["gqla_projections"]
    L = p["assumed_ctx"]
    b_abs = A.latent_row_bytes(512, 64)
    f_abs = A.absorbed_flops_per_pos(128, 512, 64)
    b_gqa = A.gqa_row_bytes(8, 128, 64)
    f_gqa = 2 * A.gqa_flops_per_pos(128, 128, 64)   # s_q = 2 query tokens per row read
    h100 = A.roofline_tokens_per_s(L, b_abs, f_abs, p["assumed_h100_bw"], 989e12)
    h20_mla = A.roofline_tokens_per_s(L, b_abs, f_abs, p["assumed_h20_bw"], p["assumed_h20_flops"])
    h20_gqa = 2 * A.roofline_tokens_per_s(L, b_gqa, f_gqa, p["assumed_h20_bw"], p["assumed_h20_flops"])
    tol = p["approx_rel"]
    assert abs(h100 / p["h100_absorbed"] - 1) < tol
    assert abs(h20_mla / p["h20_mla"] - 1) < tol
    assert abs(h20_gqa / p["h20_gqa_g8_sq2"] - 1) < tol
