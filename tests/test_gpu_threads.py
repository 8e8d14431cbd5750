"""One mask shared by several host threads on the GPU: their first calls race
to build and upload the same device schedules (plain, split and the
transposed mask's), and every thread's forward, split forward and backward
must equal, bit for bit, the results of one thread on a mask of its own."""

import threading

import pytest
import torch

import attention_jvp_causal_attn_amd as aj
from attention_jvp_causal_attn_amd.inputs import make_random
from oracle import tf_allowed

pytestmark = pytest.mark.gpu


def _calls(x, g, mask, ws):
    o, do, lse = aj.attn_jvp_fwd(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], mask)
    o2, do2, lse2 = aj.attn_jvp_fwd(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], mask,
                                    max_splits=3, workspace=ws)
    gq, gk, gv, delta = aj.attn_jvp_bwd(x["q"], x["k"], x["v"], o, g, lse, mask)
    torch.cuda.current_stream().synchronize()
    return [o, do, lse, o2, do2, lse2, gq, gk, gv, delta]


@pytest.mark.parametrize("D", [128, 64])
def test_concurrent_first_calls_on_a_shared_mask(D):
    nf, tpf, fpc, H = 6, 97, 2, 2
    pred = tf_allowed(nf, tpf, fpc)
    x = {k: v.cuda() for k, v in make_random(1, pred.n_q, H, D, dtype="bf16", seed=14100 + D,
                                              tangent_std=0.1).items()}
    g = make_random(1, pred.n_q, H, D, dtype="bf16", seed=14101 + D)["q"].cuda()
    own = aj.attn_jvp_mask_tf(nf, tpf, fpc)
    need = aj.attn_jvp_fwd_split_workspace(x["q"], x["k"], own, 3)
    ref = _calls(x, g, own, torch.empty(max(need, 16), dtype=torch.uint8, device="cuda"))

    shared = aj.attn_jvp_mask_tf(nf, tpf, fpc)      # nothing built or uploaded yet
    n = 4
    start = threading.Barrier(n)
    results, errors = [None] * n, []

    def work(i):
        try:
            ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
            start.wait()
            results[i] = _calls(x, g, shared, ws)
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(n)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for r in results:
        for a, b in zip(r, ref):
            assert torch.equal(a, b)
