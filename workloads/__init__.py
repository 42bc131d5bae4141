"""Seeded synthetic inputs for MLA / GQLA decode, shared by the tests, the bench and the oracle.

This module only draws numbers and lays them out; it holds none of the method's arithmetic
(no projection, norm, rotation, softmax or attention). Everything it returns is an *input*:
weights, token activations, query vectors, sequence lengths, block tables and, for the
large workloads, the latent-cache rows themselves.

Shapes and value distributions follow the workloads described for this method:

* multi-head latent attention with d_c-wide latents and one shared d_r-wide rotary key per
  position (Smallem article 13, "L'attention latente : compresser le cache", sections
  "L'idée : garder un résumé" and "L'obstacle : RoPE"), DeepSeek-sized latents of 512
  under a 7,168-wide model (same article, "Pourquoi DeepSeek n'observe pas cette perte");
* the GQLA variant whose up-projections are indexed by g groups (gist.science summary of
  arXiv 2605.15250, section 2 "Architecture").

Drawing rules: numpy ``default_rng([seed, stream])`` with one stream per tensor, weights
``N(0, 1/fan_in)``, activations and queries ``N(0, 1)``, RMS gain 1. Floating tensors are
rounded once, here, to the workload's storage dtype with round-to-nearest-even (torch's
float32 -> bfloat16 cast), so the GPU and the oracle receive the very same bits.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

# stream ids of default_rng([seed, stream]); one per tensor kind
S_W_DKV, S_GAMMA, S_W_KR, S_W_UK, S_W_UV, S_X, S_Q_NOPE, S_Q_PE, S_LENS, S_TABLE = range(10)
S_CACHE_C, S_CACHE_KR, S_Q_ABS, S_X_NEW, S_POS_SHIFT = 10, 11, 12, 13, 14
S_W_DQ, S_GAMMA_Q, S_W_UQ, S_W_QR, S_W_O, S_B_O, S_O = 15, 16, 17, 18, 19, 20, 21
S_CACHE_E4M3 = 22


@dataclasses.dataclass(frozen=True)
class Workload:
    """One decode workload: shapes, storage dtype and the sequence-length recipe."""

    name: str
    dtype: str            # "f32" or "bf16": storage type of every float tensor
    batch: int            # B sequences
    s_q: int              # query tokens per sequence in one decode step
    d_model: int          # C
    n_heads: int          # H (= h_q)
    d_nope: int           # D, per-head non-rotary query/key width
    d_v: int              # D_v, per-head value width
    d_c: int              # latent width (r_kv)
    d_r: int              # shared rotary key width (d^R_h)
    n_groups: int         # G; G == H is plain MLA
    block_size: int       # tokens per paged cache block
    ctx: int              # context length (upper bound when ctx_min is set)
    ctx_min: Optional[int] = None   # lengths ~ U[ctx_min, ctx] when set, else all == ctx
    random_table: bool = False      # random physical block ids, else identity layout
    n_split: int = 0                # split-K chunks hint (0: let the library choose)
    spare_blocks: int = 64
    seed: int = 21000

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elt(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def d_q(self) -> int:
        """Width of the query latent: 3 d_c (wider than the key-value latent; 1,536 at
        d_c = 512)."""
        return 3 * self.d_c

    @property
    def row(self) -> int:
        """Elements in one latent-cache row [c || k_r]."""
        return self.d_c + self.d_r

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads of this method by name, each with its own seed.
WORKLOADS = {w.name: w for w in (
    Workload("smallem-fp32", "f32", batch=1, s_q=1, d_model=512, n_heads=8, d_nope=64,
             d_v=64, d_c=128, d_r=32, n_groups=8, block_size=64, ctx=512, seed=21001),
    Workload("mid-bf16", "bf16", batch=16, s_q=1, d_model=4096, n_heads=32, d_nope=128,
             d_v=128, d_c=512, d_r=64, n_groups=32, block_size=64, ctx=4096, seed=21002),
    Workload("dsv3-paged", "bf16", batch=64, s_q=1, d_model=7168, n_heads=128, d_nope=128,
             d_v=128, d_c=512, d_r=64, n_groups=128, block_size=64, ctx=8192,
             ctx_min=1024, random_table=True, seed=21003),
    Workload("long-128k", "bf16", batch=4, s_q=1, d_model=7168, n_heads=128, d_nope=128,
             d_v=128, d_c=512, d_r=64, n_groups=128, block_size=64, ctx=131072,
             n_split=64, seed=21004),
    Workload("gqla-g8", "bf16", batch=32, s_q=1, d_model=7168, n_heads=128, d_nope=128,
             d_v=128, d_c=512, d_r=64, n_groups=8, block_size=64, ctx=32768,
             random_table=True, seed=21005),
    # a prefill: every position of two 4,096-token prompts is a query (s_q = L)
    Workload("prefill-4k", "bf16", batch=2, s_q=4096, d_model=7168, n_heads=128, d_nope=128,
             d_v=128, d_c=512, d_r=64, n_groups=128, block_size=64, ctx=4096,
             random_table=True, seed=21006),
)}


def rng(w: Workload, stream: int, extra: int = 0) -> np.random.Generator:
    return np.random.default_rng([w.seed, stream, extra])


def to_storage(a: np.ndarray, w: Workload) -> torch.Tensor:
    """float32 numpy array -> CPU tensor in the workload's storage dtype (RNE for bf16)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(w.torch_dtype)


def normal(w: Workload, stream: int, shape, std: float = 1.0, extra: int = 0) -> torch.Tensor:
    a = rng(w, stream, extra).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return to_storage(a, w)


# ----------------------------------------------------------------------------- weights
def weights(w: Workload, random_gamma: bool = False) -> dict:
    """W_DKV [C, d_c], gamma [d_c], W_KR [C, d_r], W_UK [d_c, G*D], W_UV [d_c, G*D_v].

    Row-major ``[in, out]``: a row vector times the matrix, as the pages write ``x · W``.
    """
    C, G = w.d_model, w.n_groups
    out = {
        "w_dkv": normal(w, S_W_DKV, (C, w.d_c), std=C ** -0.5),
        "w_kr": normal(w, S_W_KR, (C, w.d_r), std=C ** -0.5),
        "w_uk": normal(w, S_W_UK, (w.d_c, G * w.d_nope), std=w.d_c ** -0.5),
        "w_uv": normal(w, S_W_UV, (w.d_c, G * w.d_v), std=w.d_c ** -0.5),
    }
    if random_gamma:
        g = 1.0 + 0.25 * rng(w, S_GAMMA).standard_normal(size=(w.d_c,), dtype=np.float32)
        out["gamma"] = to_storage(g, w)
    else:
        out["gamma"] = to_storage(np.ones((w.d_c,), np.float32), w)
    return out


def layer_weights(w: Workload) -> dict:
    """The query-side and output weights of the layer: W_DQ [C, d_q], gamma_q [d_q] (random
    around 1), W_UQ [d_q, H*D], W_QR [d_q, H*d_r], W_O [H*D_v, C], b_O [C]."""
    C, H, dq = w.d_model, w.n_heads, w.d_q
    g = 1.0 + 0.25 * rng(w, S_GAMMA_Q).standard_normal(size=(dq,), dtype=np.float32)
    b = 0.1 * rng(w, S_B_O).standard_normal(size=(C,), dtype=np.float32)
    return {
        "w_dq": normal(w, S_W_DQ, (C, dq), std=C ** -0.5),
        "gamma_q": to_storage(g, w),
        "w_uq": normal(w, S_W_UQ, (dq, H * w.d_nope), std=dq ** -0.5),
        "w_qr": normal(w, S_W_QR, (dq, H * w.d_r), std=dq ** -0.5),
        "w_o": normal(w, S_W_O, (H * w.d_v, C), std=(H * w.d_v) ** -0.5),
        "b_o": to_storage(b, w),
    }


def head_outputs(w: Workload, n_tok: int) -> torch.Tensor:
    """[n_tok, H*D_v] ~ N(0, 1): stand-in for the attention outputs fed to the projection."""
    return normal(w, S_O, (n_tok, w.n_heads * w.d_v))


# ----------------------------------------------------------------------------- lengths / paging
def seq_lens(w: Workload) -> np.ndarray:
    """int32 [B]: cache length of each sequence after the step's s_q new tokens."""
    if w.ctx_min is None:
        return np.full((w.batch,), w.ctx, dtype=np.int32)
    r = rng(w, S_LENS)
    return r.integers(w.ctx_min, w.ctx, size=(w.batch,), endpoint=True).astype(np.int32)


def block_table(w: Workload, lens: np.ndarray, max_blocks: Optional[int] = None,
                random: Optional[bool] = None):
    """Paged layout. Returns (table int32 [B, max_blocks], num_blocks).

    Sequence b owns ceil(L_b / bs) blocks; unused table entries hold -1. With a random table
    the physical ids are a seeded permutation of all blocks (plus spare blocks nobody owns),
    otherwise sequence b's blocks are laid out one after the other.
    """
    bs = w.block_size
    need = [(int(L) + bs - 1) // bs for L in lens]
    mb = max(need) if max_blocks is None else max_blocks
    assert mb >= max(need)
    total = sum(need)
    random = w.random_table if random is None else random
    num_blocks = total + (w.spare_blocks if random else 0)
    ids = rng(w, S_TABLE).permutation(num_blocks) if random else np.arange(num_blocks)
    table = np.full((len(lens), mb), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(need):
        table[b, :n] = ids[k:k + n]
        k += n
    return table, num_blocks


# ----------------------------------------------------------------------------- activations
def tokens(w: Workload, n_tok: int, extra: int = 0) -> torch.Tensor:
    """x [n_tok, C] ~ N(0, 1): hidden states of positions entering the cache."""
    return normal(w, S_X, (n_tok, w.d_model), extra=extra)


def queries(w: Workload) -> dict:
    """q_nope [B, s_q, H, D], q_pe [B, s_q, H, d_r] ~ N(0, 1) (not yet rotated)."""
    shp = (w.batch, w.s_q, w.n_heads)
    return {"q_nope": normal(w, S_Q_NOPE, shp + (w.d_nope,)),
            "q_pe": normal(w, S_Q_PE, shp + (w.d_r,))}


def query_positions(w: Workload, lens: np.ndarray) -> np.ndarray:
    """int32 [B, s_q]: position of query i of sequence b is L_b - s_q + i."""
    i = np.arange(w.s_q, dtype=np.int64)
    return (lens.astype(np.int64)[:, None] - w.s_q + i[None, :]).astype(np.int32)


def absorbed_queries(w: Workload) -> torch.Tensor:
    """Directly drawn absorbed query rows [B, s_q, H, d_c + d_r] for decode-only tests.

    Latent part ~ N(0, D/d_c) -- the spread of q_nope (N(0,1), width D) times a W_UK drawn
    N(0, 1/d_c) -- and rotary part ~ N(0, 1), so scores have the spread of real ones.
    """
    shp = (w.batch, w.s_q, w.n_heads)
    lat = rng(w, S_Q_ABS).standard_normal(size=shp + (w.d_c,), dtype=np.float32)
    lat *= np.float32((w.d_nope / w.d_c) ** 0.5)
    rot = rng(w, S_Q_ABS, 1).standard_normal(size=shp + (w.d_r,), dtype=np.float32)
    return to_storage(np.concatenate([lat, rot], axis=-1), w)


def cache_pool(w: Workload, num_blocks: int, extra: int = 0) -> torch.Tensor:
    """A whole paged cache [num_blocks, bs, d_c + d_r] of directly drawn rows ~ N(0, 1).

    Stand-in history for workloads whose full history is too large to push through the
    append step on the host: an RMS-normalised latent with unit gain has unit mean square,
    and x · W_KR with x ~ N(0,1), W_KR ~ N(0, 1/C) is N(0, 1) before rotation (a rotation
    keeps it so), so N(0, 1) rows have the magnitudes of appended rows. Every slot is
    drawn; which rows belong to which sequence is decided by the block table alone.
    """
    a = rng(w, S_CACHE_C, extra).standard_normal(
        size=(num_blocks, w.block_size, w.row), dtype=np.float32)
    return to_storage(a, w)


def cache_pool_device(w: Workload, num_blocks: int, device, extra: int = 0) -> torch.Tensor:
    """Like cache_pool, drawn by torch's seeded generator on the device (for large benchmark
    caches that would take seconds to draw on the host). Seed: seed * 1000 + extra."""
    g = torch.Generator(device=device)
    g.manual_seed(w.seed * 1000 + extra)
    a = torch.randn((num_blocks, w.block_size, w.row), generator=g, device=device,
                    dtype=torch.float32)
    return a.to(w.torch_dtype)


def cache_pool_e4m3(w: Workload, num_blocks: int, extra: int = 0):
    """An e4m3 paged cache drawn directly as bytes: (codes uint8 [num_blocks, bs, d_c + d_r],
    scales float32 [num_blocks, bs]).

    Sign bits uniform; magnitude codes (the low 7 bits, which order E4M3 magnitudes
    log-linearly) ~ round(N(104, 10)) clipped to the finite codes 0 .. 126, i.e. magnitudes
    near 2^6 spread over about three binades; one scale per slot 2^k, k uniform in -8 .. -6.
    The values code x scale then have the spread of the N(0, 1) bf16 rows of cache_pool.
    """
    r = rng(w, S_CACHE_E4M3, extra)
    shp = (num_blocks, w.block_size, w.row)
    mag = np.clip(np.rint(r.normal(104.0, 10.0, size=shp)), 0, 126).astype(np.uint8)
    sign = (r.integers(0, 2, size=shp, dtype=np.uint8) << 7).astype(np.uint8)
    scales = np.exp2(r.integers(-8, -5, size=shp[:2], endpoint=False)).astype(np.float32)
    return torch.from_numpy(mag | sign), torch.from_numpy(scales)
