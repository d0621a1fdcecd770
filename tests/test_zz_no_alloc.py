"""The allocation-free decode entry point against the decode with a
caller-provided workspace: same kernels, so the outputs and LSE must be
identical bit for bit, and both within the parity bar of the oracle.  Two
calls in a row, the second with a smaller input (fewer tokens, a narrower
top-k list), so the scratch holds the first call's partials when the second
runs."""
import numpy as np
import pytest
import torch

import gpu_harness as G
import oracle_pins as P
import sparse_mla_attention_gather_amd as dsa
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _noalloc(di, pool_d, wl, out_dtype):
    T, H, K = wl.T, wl.H, wl.K
    out = torch.empty((T, H, 512), dtype=torch.float32 if out_dtype == dsa.DSA_FP32
                      else torch.bfloat16, device=G.DEV)
    lse = torch.empty((T, H), dtype=torch.float32, device=G.DEV)
    err = torch.zeros(1, dtype=torch.int32, device=G.DEV)
    G.check(dsa.dsa_sparse_attn_decode_noalloc(
        di.q, dsa.DSA_BF16, None, T, H, 512, wl.rope_dim, pool_d, pool_d.shape[0],
        wl.layout, dsa.DSA_FP8_E4M3FN, di.topk, K, di.page_table, wl.page_size,
        di.max_pages, di.num_seqs, di.token_seq, di.seq_lens, wl.softmax_scale,
        out, out_dtype, lse, err))
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), G.host(lse), int(err.item())


CASES = [
    (dict(seed=701, T=12, H=16, K=1024, layout=W.RAW, seq_len=1500, page_size=64),
     dict(seed=702, T=5, H=16, K=512, layout=W.RAW, seq_len=900, page_size=64)),
    (dict(seed=703, T=9, H=32, K=896, layout=W.SCALED, seq_len=1200, page_size=32, dup_frac=0.1),
     dict(seed=704, T=3, H=32, K=384, layout=W.SCALED, seq_len=500, page_size=32)),
    (dict(seed=705, T=20, H=64, K=2048, layout=W.RAW, seq_len=2500, page_size=64),
     dict(seed=706, T=2, H=8, K=128, layout=W.RAW, seq_len=200, page_size=16)),
]


@pytest.mark.parametrize("od", [dsa.DSA_FP32, dsa.DSA_BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("first,second", CASES, ids=["raw16", "scaled32", "raw64"])
def test_noalloc_matches_workspace_decode(orc, first, second, od):
    for cfg in (first, second):
        wl = W.small(**cfg)
        print(f"noalloc case {cfg} out {od}", flush=True)
        assert dsa.dsa_attn_workspace_bytes(wl.T, wl.H, wl.K, 0) > 0        # splits
        pool = P.build_pool(orc, wl)
        pool_d = G.dev(pool)
        di = G.DevInputs(wl)
        ref_out, ref_lse, ref_err = G.run_attn(di, pool_d, phase=0, out_dtype=od)
        out, lse, err = _noalloc(di, pool_d, wl, od)
        assert err == ref_err
        assert np.array_equal(out, ref_out)
        assert np.array_equal(lse, ref_lse)
        o_ref, l_ref, e_ref = orc.sparse_attn(wl.q, pool, wl.layout, wl.topk, wl.softmax_scale,
                                              page_table=wl.page_table, page_size=wl.page_size,
                                              token_seq=wl.token_seq, seq_lens=wl.seq_lens)
        assert err == e_ref
        G.assert_attn_close(out, o_ref, od, where=f"noalloc {cfg['seed']}")
        G.assert_lse_close(lse, l_ref, where=f"noalloc {cfg['seed']}")
