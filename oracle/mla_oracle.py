"""Plain f64 CPU oracle for MLA decode over a compressed latent cache, and for GQLA.

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the bench's CPU-baseline leg,
never by the product path. It shares no code with the HIP library.

What it computes, and where the pages state it
----------------------------------------------
Sources are the pages this method is described on:

* [Smallem] smallbard.com, Smallem article 13 "L'attention latente : compresser le cache";
* [KV-cache] mkdocs.reaper.mx, DeepSeek-V4.1-Flash "Le cache clé-valeur";
* [Slides] cours.spawnkit.ai session 18 slides "Cache KV, mémoire récurrente, MLA et bas rang";
* [GQLA] gist.science summary of arXiv 2605.15250, "GQLA – Attention Latente par Groupes
  de Requêtes".

The gold answer is the *reconstructed* form, which is the plain definition: keys and values
of every head are rebuilt from the cached latents for every past position ([Smallem] "L'idée
: garder un résumé"; [Slides] "Carte du mécanisme"), each head's key is the concatenation of
its content part and the shared rotary key ([Smallem] "L'obstacle : RoPE"), and textbook
softmax attention follows ([KV-cache] "Le mécanisme d'attention"). The absorbed form
([Smallem] "Ce que DeepSeek fait de plus") and the GQA form ([GQLA] section 2, "Chemin
GQA") are written here as separate functions, so that tests can check that all three agree.

Readings where the pages are silent (each one is also listed in the design notes):

* RoPE: pairs (2j, 2j+1) rotated by pos * base^(-2j/d_r), 0-based absolute positions.
* RMSNorm: y / sqrt(mean(y^2) + eps) * gamma, mean over the d_c latent entries.
* Softmax scale 1/sqrt(D + d_r), D the per-head content width ([Smallem] "L'obstacle : RoPE").
* Head h uses group g(h) = h // (H / G) of the group-indexed up-projections
  ([GQLA] section 2 "Architecture"); G = H is plain MLA.
* Weights are row-major [in, out]: the pages multiply a row vector on the left (x · W).
* Multi-token steps: the s_q new positions are in the cache; query i sees positions
  0 .. L - s_q + i.
* bf16 storage rounds to nearest, ties to even.
* FP8 latent rows (the pages name quantisation as a way to shrink a cache entry, [KV-cache]
  "Les trois dimensions de compression", and one byte per value halves it, [Slides] trainer
  notes on the INT8 check, but fix no format): OCP FP8 E4M3 bytes times one power-of-two
  scale per position, the smallest s with max |row| <= 448 s; bytes rounded to nearest, ties
  to the even code.

Parity pins (what ties this oracle to something other than itself) live in
tests/test_oracle_pins.py. Conventions no page fixes (the RoPE pair layout and frequency
schedule, the RMSNorm epsilon, the bf16 rounding mode) are parity unpinned beyond the
internal consistency checks listed there.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "query_project", "output_project",
    "f64", "round_bf16", "round_storage", "slot", "seq_slots", "gather_rows", "owned_slot_mask",
    "rms_norm", "rope", "latent_rows", "group_of", "softmax_scale",
    "attend", "decode_reconstructed", "absorb_query", "decode_absorbed_latent",
    "project_values", "decode_absorbed", "gqa_expand_rows", "decode_gqa",
    "visible_lengths",
    "e4m3_values", "e4m3_encode", "e4m3_row_scale", "quantize_rows_e4m3", "dequantize_rows_e4m3",
]


def f64(t) -> np.ndarray:
    """Exact f64 copy of a torch tensor (any float dtype) or array."""
    if hasattr(t, "detach"):
        return t.detach().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


# --------------------------------------------------------------------------- rounding
def round_bf16(a) -> np.ndarray:
    """Round f64 values to the nearest bfloat16 value, ties to even, keeping them as f64.

    bfloat16 keeps 8 significant bits and float32's exponent range: a value m * 2**e with
    m in [0.5, 1) is a multiple of 2**(e - 8) while normal (e >= -125); below that the
    spacing stays 2**-133. Magnitudes that round above the largest finite bfloat16
    (2**128 - 2**120) become infinite. np.rint rounds halves to even.
    """
    a = np.asarray(a, dtype=np.float64)
    out = np.array(a, copy=True)
    fin = np.isfinite(a) & (a != 0)
    _, e = np.frexp(a[fin])
    q = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(a[fin] / q) * q
    big = np.abs(r) > (2.0 ** 128 - 2.0 ** 120)
    r[big] = np.copysign(np.inf, r[big])
    out[fin] = r
    return out


def round_storage(a, dtype: str) -> np.ndarray:
    """Round to the storage type of a cache or output tensor ("f32" or "bf16")."""
    if dtype == "bf16":
        return round_bf16(a)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------- paging (integer)
def slot(table: np.ndarray, b: int, p: int, bs: int) -> int:
    """Flat cache slot of position p of sequence b: the position's block, looked up in the
    sequence's row of the block table, times the block size, plus the offset in the block."""
    return int(table[b, p // bs]) * bs + p % bs


def seq_slots(table: np.ndarray, b: int, L: int, bs: int) -> np.ndarray:
    """int64 [L]: slots of positions 0..L-1 of sequence b (the rule of slot())."""
    return np.array([slot(table, b, p, bs) for p in range(L)], dtype=np.int64)


def gather_rows(cache, table: np.ndarray, b: int, L: int) -> np.ndarray:
    """f64 [L, row]: sequence b's first L cache rows read through the block table."""
    nb, bs, row = cache.shape
    flat = cache.reshape(nb * bs, row)
    idx = seq_slots(table, b, L, bs)
    if hasattr(flat, "detach"):
        import torch
        return f64(flat[torch.from_numpy(idx)])
    return f64(flat[idx])


def owned_slot_mask(table: np.ndarray, lens, num_blocks: int, bs: int) -> np.ndarray:
    """bool [num_blocks * bs]: True where some sequence's position lives."""
    m = np.zeros(num_blocks * bs, dtype=bool)
    for b, L in enumerate(lens):
        m[seq_slots(table, b, int(L), bs)] = True
    return m


# --------------------------------------------------------------------------- cache rows (append)
def rms_norm(y: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: y / sqrt(mean(y^2) + eps) * gamma.

    [Smallem] "Le code": the latent goes through an RMS norm before the up-projections,
    because latent and key would otherwise come out several times too small.
    """
    ms = np.mean(y * y, axis=-1, keepdims=True)
    return y / np.sqrt(ms + eps) * gamma


def rope(v: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate the last axis of v by position: pair (2j, 2j+1) turns by pos * base**(-2j/d).

    [Smallem] "L'obstacle : RoPE": rotation encodes the position; it is applied to the
    separate rotary part only, because a rotation does not commute with a matrix. pos may
    be a scalar or broadcast against v[..., 0].
    """
    v = np.asarray(v, dtype=np.float64)
    d = v.shape[-1]
    if d == 0:
        return v.copy()
    j = np.arange(d // 2, dtype=np.float64)
    theta = base ** (-2.0 * j / d)
    phi = np.asarray(pos, dtype=np.float64)[..., None] * theta
    a, b = v[..., 0::2], v[..., 1::2]
    cos, sin = np.cos(phi), np.sin(phi)
    out = np.empty_like(v)
    out[..., 0::2] = a * cos - b * sin
    out[..., 1::2] = a * sin + b * cos
    return out


def latent_rows(x, w_dkv, gamma, w_kr, pos, base: float, eps: float) -> np.ndarray:
    """f64 [n, d_c + d_r]: the cache row [c || k_r] of each position, before storage rounding.

    c = rms(x · W_DKV) * gamma is the latent, the only per-position content kept
    ([Smallem] "L'idée : garder un résumé"; [Slides] "Carte du mécanisme"); k_r =
    rotation(x · W_KR) is one rotary key shared by every head, stored already rotated
    ([Smallem] "L'obstacle : RoPE" and the cache extension in "Le code").
    """
    x, w_dkv, gamma, w_kr = f64(x), f64(w_dkv), f64(gamma), f64(w_kr)
    c = rms_norm(x @ w_dkv, gamma, eps)
    k_r = rope(x @ w_kr, np.asarray(pos), base)
    return np.concatenate([c, k_r], axis=-1)


# --------------------------------------------------------------------------- attention
def group_of(h: int, n_heads: int, n_groups: int) -> int:
    """Group whose up-projection columns head h uses: contiguous runs of H/G heads."""
    return h // (n_heads // n_groups)


def softmax_scale(d_nope: int, d_r: int) -> float:
    """1/sqrt(D + d_r): the width of the concatenated per-head query/key
    ([Smallem] "L'obstacle : RoPE")."""
    return 1.0 / math.sqrt(d_nope + d_r)


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """One query row against keys K [n, d] and values V [n, e]: textbook softmax attention.

    Returns (output [e], lse) with lse = log sum_t exp(scale * q.K_t)
    ([KV-cache] "Le mécanisme d'attention": weights from the scaled comparisons sum to 1
    and average the values).
    """
    z = scale * (K @ q)
    m = np.max(z)
    e = np.exp(z - m)
    s = np.sum(e)
    p = e / s
    return p @ V, m + math.log(s)


def visible_lengths(L: int, s_q: int) -> list:
    """Positions query i of a step sees: 0 .. L - s_q + i, i.e. L - s_q + i + 1 of them."""
    return [L - s_q + i + 1 for i in range(s_q)]


def decode_reconstructed(q_nope, q_pe, q_pos, hist, w_uk, w_uv, n_groups: int, d_c: int,
                         d_v: int, base: float, scale: float | None = None, heads=None):
    """Reconstructed (non-absorbed) decode of one sequence -- the gold answer.

    q_nope [s_q, H, D], q_pe [s_q, H, d_r] (not rotated), q_pos [s_q], hist [L, d_c + d_r]
    cache rows (already including the step's s_q new positions), W_UK [d_c, G*D],
    W_UV [d_c, G*D_v].

    For every head h of group g: K_h = [c · W_UK[:, g] , k_r] and V_h = c · W_UV[:, g] are
    rebuilt for all L positions ([Smallem] "L'idée : garder un résumé"); the query is
    [q_nope_h ; rotation(q_pe_h, pos)] ([Smallem] "L'obstacle : RoPE"); then softmax
    attention over the positions the query may see.
    Returns (out [s_q, H, D_v], lse [s_q, H]); with `heads`, only those heads, in that order.
    """
    q_nope, q_pe, hist, w_uk, w_uv = f64(q_nope), f64(q_pe), f64(hist), f64(w_uk), f64(w_uv)
    s_q, H, D = q_nope.shape
    L = hist.shape[0]
    scale = softmax_scale(D, q_pe.shape[-1]) if scale is None else scale
    c, k_r = hist[:, :d_c], hist[:, d_c:]
    heads = list(range(H)) if heads is None else list(heads)
    out = np.zeros((s_q, len(heads), d_v))
    lse = np.zeros((s_q, len(heads)))
    lim = visible_lengths(L, s_q)
    for j, h in enumerate(heads):
        g = group_of(h, H, n_groups)
        K = np.concatenate([c @ w_uk[:, g * D:(g + 1) * D], k_r], axis=1)
        V = c @ w_uv[:, g * d_v:(g + 1) * d_v]
        for i in range(s_q):
            q = np.concatenate([q_nope[i, h], rope(q_pe[i, h], q_pos[i], base)])
            n = lim[i]
            out[i, j], lse[i, j] = attend(q, K[:n], V[:n], scale)
    return out, lse


# --------------------------------------------------------------------------- absorbed form
def absorb_query(q_nope, q_pe, q_pos, w_uk, n_groups: int, base: float) -> np.ndarray:
    """Absorbed query rows [.., H, d_c + d_r]: [q_nope_h · W_UK[:, g]^T , rotation(q_pe_h)].

    [Smallem] "Ce que DeepSeek fait de plus": q · (c · W) equals (q · W^T) · c, so the
    query can be carried into latent space once and compared with the cached latents.
    [GQLA] section 2: the up-projections are indexed by the head's group.
    """
    q_nope, q_pe, w_uk = f64(q_nope), f64(q_pe), f64(w_uk)
    *lead, H, D = q_nope.shape
    out = []
    for h in range(H):
        g = group_of(h, H, n_groups)
        lat = q_nope[..., h, :] @ w_uk[:, g * D:(g + 1) * D].T
        rot = rope(q_pe[..., h, :], np.asarray(q_pos), base)
        out.append(np.concatenate([lat, rot], axis=-1))
    return np.stack(out, axis=-2)


def decode_absorbed_latent(q_abs, hist, d_c: int, scale: float, heads=None):
    """Latent-space decode of one sequence: the attention of [Smallem] "Ce que DeepSeek fait
    de plus" run on the cached rows themselves.

    q_abs [s_q, H, d_c + d_r], hist [L, d_c + d_r]. Scores are scale * (q_abs . row), i.e.
    the latent part against c plus the rotary part against k_r in one product over the
    concatenation ([Smallem] "Deux produits ou une concaténation ?"); the probabilities
    weight the latents c. Returns (o_lat [s_q, H, d_c], lse [s_q, H]); with `heads`, only
    those heads, in that order.
    """
    q_abs, hist = f64(q_abs), f64(hist)
    s_q, H, _ = q_abs.shape
    L = hist.shape[0]
    heads = list(range(H)) if heads is None else list(heads)
    o = np.zeros((s_q, len(heads), d_c))
    lse = np.zeros((s_q, len(heads)))
    lim = visible_lengths(L, s_q)
    for i in range(s_q):
        n = lim[i]
        for j, h in enumerate(heads):
            o[i, j], lse[i, j] = attend(q_abs[i, h], hist[:n], hist[:n, :d_c], scale)
    return o, lse


def project_values(o_lat, w_uv, n_groups: int, d_v: int, n_heads: int | None = None,
                   heads=None) -> np.ndarray:
    """out_h = o_lat_h · W_UV[:, g(h)]: the weighted latent mapped to the head's values once
    ([Smallem] "Ce que DeepSeek fait de plus"). With `heads`, o_lat holds those heads only
    (in that order) out of n_heads."""
    o_lat, w_uv = f64(o_lat), f64(w_uv)
    *lead, Hs, _ = o_lat.shape
    H = Hs if n_heads is None else n_heads
    heads = list(range(Hs)) if heads is None else list(heads)
    outs = []
    for j, h in enumerate(heads):
        g = group_of(h, H, n_groups)
        outs.append(o_lat[..., j, :] @ w_uv[:, g * d_v:(g + 1) * d_v])
    return np.stack(outs, axis=-2)


def decode_absorbed(q_nope, q_pe, q_pos, hist, w_uk, w_uv, n_groups: int, d_c: int, d_v: int,
                    base: float, scale: float | None = None):
    """Absorbed decode of one sequence end to end (cross-check of the reconstructed form)."""
    D, d_r = np.shape(q_nope)[-1], np.shape(q_pe)[-1]
    scale = softmax_scale(D, d_r) if scale is None else scale
    qa = absorb_query(q_nope, q_pe, q_pos, w_uk, n_groups, base)
    o_lat, lse = decode_absorbed_latent(qa, hist, d_c, scale)
    return project_values(o_lat, w_uv, n_groups, d_v), lse


# --------------------------------------------------------------------------- GQA form
def gqa_expand_rows(hist, w_uk, w_uv, n_groups: int, d_c: int, d_nope: int, d_v: int):
    """Expanded GQA cache rows [L, 2*G*D + d_r] = [K_0 .. K_{G-1} || V_0 .. V_{G-1} || k_r].

    [GQLA] section 2, "Chemin GQA": the latent is expanded once into g key/value groups and
    the cache holds 2*g*d_h numbers plus the shared rotary key per position.
    """
    hist, w_uk, w_uv = f64(hist), f64(w_uk), f64(w_uv)
    c, k_r = hist[:, :d_c], hist[:, d_c:]
    Ks = [c @ w_uk[:, g * d_nope:(g + 1) * d_nope] for g in range(n_groups)]
    Vs = [c @ w_uv[:, g * d_v:(g + 1) * d_v] for g in range(n_groups)]
    return np.concatenate(Ks + Vs + [k_r], axis=1)


def decode_gqa(q_nope, q_pe, q_pos, gqa_rows, n_groups: int, d_v: int, base: float,
               scale: float | None = None, heads=None):
    """Standard grouped-query decode over an expanded cache ([GQLA] "Chemin GQA").

    Head h of group g compares [q_nope_h ; rotation(q_pe_h)] with [K_g ; k_r] and averages
    V_g. Returns (out [s_q, H, D_v], lse [s_q, H]).
    """
    q_nope, q_pe, rows = f64(q_nope), f64(q_pe), f64(gqa_rows)
    s_q, H, D = q_nope.shape
    G = n_groups
    scale = softmax_scale(D, q_pe.shape[-1]) if scale is None else scale
    L = rows.shape[0]
    k_r = rows[:, G * D + G * d_v:]
    heads = list(range(H)) if heads is None else list(heads)
    out = np.zeros((s_q, len(heads), d_v))
    lse = np.zeros((s_q, len(heads)))
    lim = visible_lengths(L, s_q)
    for j, h in enumerate(heads):
        g = group_of(h, H, G)
        K = np.concatenate([rows[:, g * D:(g + 1) * D], k_r], axis=1)
        V = rows[:, G * D + g * d_v:G * D + (g + 1) * d_v]
        for i in range(s_q):
            q = np.concatenate([q_nope[i, h], rope(q_pe[i, h], q_pos[i], base)])
            n = lim[i]
            out[i, j], lse[i, j] = attend(q, K[:n], V[:n], scale)
    return out, lse


# ------------------------------------------------------------------ the layer around the path
def query_project(x, w_dq, gamma_q, w_uq, w_qr, eps: float, round_cq=None):
    """(q_nope [n, H*D], q_pe [n, H*d_r]) of the layer's query side, f64.

    [Smallem] "Le code": query_down (C -> d_q), query_norm, query_up (d_q -> H*D) and
    query_rope (d_q -> H*d_r); "L'obstacle : RoPE": the queries' rotary part is taken from
    their own latent c_q, and rotated by the same rule as the keys (done by absorb_query).
    c_q = RMSNorm(x · W_DQ) * gamma_q; round_cq, when given, is the storage rounding applied to
    c_q between the two products.
    """
    c_q = rms_norm(f64(x) @ f64(w_dq), f64(gamma_q), eps)
    if round_cq is not None:
        c_q = round_cq(c_q)
    return c_q @ f64(w_uq), c_q @ f64(w_qr)


def output_project(o, w_o, b_o=None):
    """y [n, C] = o · W_O + b_O, f64: the layer's proj, a linear layer with bias ([Smallem]
    "Le code"), applied to the heads' outputs o [n, H*D_v] in head order."""
    y = f64(o) @ f64(w_o)
    if b_o is not None:
        y = y + f64(b_o)
    return y


# ------------------------------------------------------------------ FP8 (E4M3) latent rows
def e4m3_values() -> np.ndarray:
    """f64 [256]: the value of every OCP FP8 E4M3 byte, NaN for its two NaN codes.

    Byte s eeee mmm: sign s, exponent field E (bias 7), mantissa field m. E >= 1 is normal,
    (-1)^s 2^(E - 7) (1 + m/8); E = 0 is subnormal, (-1)^s 2^-6 (m/8); E = 15 with m = 7 is
    NaN (the format has no infinities, so E = 15 otherwise stays a normal binade, up to 448).
    """
    out = np.empty(256)
    for b in range(256):
        sign = -1.0 if b & 0x80 else 1.0
        E, m = (b >> 3) & 0xF, b & 0x7
        if E == 15 and m == 7:
            out[b] = np.nan
        elif E == 0:
            out[b] = sign * 2.0 ** -6 * (m / 8.0)
        else:
            out[b] = sign * 2.0 ** (E - 7) * (1.0 + m / 8.0)
    return out


def e4m3_encode(v) -> np.ndarray:
    """uint8 codes of f64 values with |v| <= 448: the nearest E4M3 value, ties to the code with
    an even mantissa (the even code); the sign bit is v's, also for values that round to 0.

    Positive codes 0x00 .. 0x7E are the finite magnitudes in increasing order, so the two
    candidates of |v| are found by a search in that list.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(~np.isfinite(a)) or np.any(a > 448.0):
        raise ValueError("e4m3_encode takes finite values of magnitude at most 448")
    mags = e4m3_values()[:0x7F]
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 0x7E)  # first magnitude >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == mags[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 7)


def e4m3_row_scale(amax: float) -> float:
    """The smallest power of two s with amax <= 448 s (1.0 when amax is 0)."""
    amax = float(amax)
    if amax == 0.0:
        return 1.0
    e = math.ceil(math.log2(amax / 448.0))
    while amax > 448.0 * 2.0 ** e:        # log2 may land one off either way
        e += 1
    while amax <= 448.0 * 2.0 ** (e - 1):
        e -= 1
    return 2.0 ** e


def quantize_rows_e4m3(rows):
    """(codes uint8 [n, w], scales f64 [n]) of rows [n, w]: per row s = e4m3_row_scale(max
    |row|) and codes = e4m3_encode(row / s) (row / s is exact: s is a power of two)."""
    r = f64(rows)
    r = r.reshape(-1, r.shape[-1])
    scales = np.array([e4m3_row_scale(np.max(np.abs(row)) if row.size else 0.0) for row in r])
    codes = e4m3_encode(r / scales[:, None])
    return codes, scales


def dequantize_rows_e4m3(codes, scales) -> np.ndarray:
    """f64 [n, w]: value(code) * scale of each row."""
    c = np.asarray(codes, dtype=np.uint8)
    return e4m3_values()[c] * np.asarray(scales, dtype=np.float64).reshape(-1, *([1] * (c.ndim - 1)))
