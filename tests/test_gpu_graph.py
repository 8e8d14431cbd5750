"""The entry points capture into a HIP graph once their mask's schedules are on
the device (after the first call they only launch kernels): a captured
forward (plain and split) and backward, replayed several times with eager
work and synchronisations in between, reproduce the eager results bit for
bit on every replay."""

import pytest
import torch

import attention_jvp_causal_attn_amd as aj
from attention_jvp_causal_attn_amd.inputs import make_random
from oracle import tf_allowed

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    nf, tpf, fpc, H, D = 6, 70, 2, 2, 128
    pred = tf_allowed(nf, tpf, fpc)
    x = {k: v.cuda() for k, v in make_random(1, pred.n_q, H, D, dtype="bf16", seed=13100,
                                              tangent_std=0.1).items()}
    g = make_random(1, pred.n_q, H, D, dtype="bf16", seed=13101)["q"].cuda()
    mask = aj.attn_jvp_mask_tf(nf, tpf, fpc)
    B, N = 1, pred.n_q
    need = aj.attn_jvp_fwd_split_workspace(x["q"], x["k"], mask, 3)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    outs = {n: torch.empty_like(x["q"]) for n in ("o", "do", "o2", "do2", "gq", "gk", "gv")}
    lse, dlse, lse2, dlse2, delta = (torch.empty(B, H, N, dtype=torch.float32, device="cuda")
                                     for _ in range(5))

    def step(stream):
        aj.attn_jvp_fwd(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], mask, o=outs["o"],
                        d_o=outs["do"], lse=lse, d_lse=dlse, stream=stream)
        aj.attn_jvp_fwd(x["q"], x["k"], x["v"], x["dq"], x["dk"], x["dv"], mask, o=outs["o2"],
                        d_o=outs["do2"], lse=lse2, d_lse=dlse2, max_splits=3, workspace=ws,
                        stream=stream)
        aj.attn_jvp_bwd(x["q"], x["k"], x["v"], outs["o"], g, lse, mask, g_q=outs["gq"],
                        g_k=outs["gk"], g_v=outs["gv"], delta=delta, stream=stream)

    # eager (also uploads every schedule the calls need)
    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [t.clone() for t in list(outs.values()) + [lse, dlse, lse2, dlse2, delta]]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep in range(4):
        for t in list(outs.values()) + [lse, dlse, lse2, dlse2, delta]:
            t.fill_(float("nan"))           # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = list(outs.values()) + [lse, dlse, lse2, dlse2, delta]
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager run"
