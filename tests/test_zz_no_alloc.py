"""mla_decode_noalloc (partials in the library's own device array, no workspace argument)
against mla_decode with a caller workspace, through the C ABI: two calls in a row, the second
with a smaller input, so that the array still holds the first call's larger contents. Both run
the same kernels with the same split plan, so the outputs must be bit-identical; each is also
held to the oracle's bound."""
import pytest
import torch

import workloads as W
from gpu_cases import (TOL, check_lse, check_per_seq, decode_case, dev, note, oracle_decode,
                       run_decode, stream_tag)
from mla_latent_kv_21_amd import binding as M

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def run_noalloc(c, n_split):
    w = c["w"]
    d = M.dims_of(w)
    out = torch.empty(w.batch, w.s_q, w.n_heads, w.d_v, dtype=w.torch_dtype, device="cuda:0")
    lse = torch.empty(w.batch, w.s_q, w.n_heads, dtype=torch.float32, device="cuda:0")
    M.mla_decode_noalloc(d, dev(c["q_abs"]), dev(c["pool"]), dev(c["table"]), dev(c["lens"]),
                         dev(c["w_uv"]), out, lse, n_split=n_split)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


# (workload, lens of the first call, lens of the second, s_q, n_split)
SEQUENCES = [
    ("dsv3-paged", [3000, 200, 777], [150], 1, 0),       # balanced plan, then a smaller one
    ("dsv3-paged", [2600, 1100], [64, 90], 1, 16),       # uniform splits
    ("gqla-g8", [2050, 300], [40], 2, 0),                # grouped, two queries per sequence
    ("smallem-fp32", [512, 300], [77], 1, 3),            # fp32 caches: the portable kernels
]


@pytest.mark.parametrize("wl,lens1,lens2,s_q,n_split", SEQUENCES,
                         ids=[f"{s[0]}-{s[4]}" for s in SEQUENCES])
def test_noalloc_matches_workspace_decode(wl, lens1, lens2, s_q, n_split):
    w = W.WORKLOADS[wl]
    for k, lens in enumerate((lens1, lens2)):
        c = decode_case(w, lens, s_q=s_q, extra=stream_tag(w) + 40 + k)
        note(f"noalloc {wl} call {k} lens={lens} s_q={s_q} n_split={n_split}")
        got, got_lse = run_noalloc(c, n_split)
        ref_out, ref_lse, _ = run_decode(c, n_split=n_split, planned=(n_split == 0))
        assert torch.equal(got, ref_out), "differs from mla_decode with a caller workspace"
        assert torch.equal(got_lse, ref_lse)
        oracle_out, oracle_lse = oracle_decode(c)
        check_per_seq(got, oracle_out, TOL[w.dtype])
        check_lse(got_lse.double().numpy(), oracle_lse, TOL[w.dtype])
