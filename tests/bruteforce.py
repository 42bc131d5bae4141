"""Pure-Python loop re-derivation of one MLA/GQLA decode step, for tiny shapes only.

Written the way the Smallem article checks its layer ("Vérifier une couche compliquée"):
no tensors, loops over plain lists, keys really concatenated, softmax summed term by term.
It uses nothing from numpy or from the oracle, so it can pin the oracle.
"""
import math


def _dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def _vec_mat(v, M, col0, ncol):
    """v (len n) times columns col0 .. col0+ncol-1 of M (n rows of lists)."""
    return [sum(v[i] * M[i][col0 + j] for i in range(len(v))) for j in range(ncol)]


def rotate(v, position, base):
    out = list(v)
    d = len(v)
    for j in range(d // 2):
        ang = position * base ** (-2.0 * j / d)
        a, b = v[2 * j], v[2 * j + 1]
        out[2 * j] = a * math.cos(ang) - b * math.sin(ang)
        out[2 * j + 1] = a * math.sin(ang) + b * math.cos(ang)
    return out


def cache_row(x, w_dkv, gamma, w_kr, position, base, eps):
    d_c = len(gamma)
    y = _vec_mat(x, w_dkv, 0, d_c)
    ms = sum(t * t for t in y) / d_c
    c = [y[j] / math.sqrt(ms + eps) * gamma[j] for j in range(d_c)]
    u = _vec_mat(x, w_kr, 0, len(w_kr[0]) if w_kr else 0)
    return c + rotate(u, position, base)


def decode(q_nope, q_pe, q_pos, hist, w_uk, w_uv, n_groups, d_c, d_v, base):
    """q_nope[i][h] (list D), q_pe[i][h] (list d_r), hist[t] (list d_c + d_r).

    Returns out[i][h] (list d_v) and lse[i][h].
    """
    s_q, H = len(q_nope), len(q_nope[0])
    D, d_r = len(q_nope[0][0]), len(q_pe[0][0])
    L = len(hist)
    per = H // n_groups
    out = [[None] * H for _ in range(s_q)]
    lse = [[None] * H for _ in range(s_q)]
    for i in range(s_q):
        n_vis = L - s_q + i + 1
        for h in range(H):
            g = h // per
            query = list(q_nope[i][h]) + rotate(q_pe[i][h], q_pos[i], base)
            scores = []
            values = []
            for t in range(n_vis):
                c = hist[t][:d_c]
                key = _vec_mat(c, w_uk, g * D, D) + list(hist[t][d_c:])
                scores.append(_dot(query, key) / math.sqrt(D + d_r))
                values.append(_vec_mat(c, w_uv, g * d_v, d_v))
            top = max(scores)
            terms = [math.exp(s - top) for s in scores]
            total = 0.0
            for e in terms:
                total += e
            o = [0.0] * d_v
            for t in range(n_vis):
                w = terms[t] / total
                for j in range(d_v):
                    o[j] += w * values[t][j]
            out[i][h] = o
            lse[i][h] = top + math.log(total)
    return out, lse


def query_project(x, w_dq, gamma_q, w_uq, w_qr, eps):
    """Loops for one token: c_q = RMSNorm(x W_DQ) gamma_q, then c_q W_UQ and c_q W_QR."""
    d_q = len(gamma_q)
    y = _vec_mat(x, w_dq, 0, d_q)
    ms = sum(t * t for t in y) / d_q
    c = [y[j] / math.sqrt(ms + eps) * gamma_q[j] for j in range(d_q)]
    q_nope = _vec_mat(c, w_uq, 0, len(w_uq[0]))
    q_pe = _vec_mat(c, w_qr, 0, len(w_qr[0]) if w_qr and w_qr[0] else 0)
    return q_nope, q_pe


def output_project(o, w_o, b_o):
    """Loops for one token: o W_O + b_O."""
    y = _vec_mat(o, w_o, 0, len(w_o[0]))
    return [y[j] + (b_o[j] if b_o is not None else 0.0) for j in range(len(y))]
