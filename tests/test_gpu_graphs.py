"""Entry points captured in a HIP graph: every replay, with eager work and
synchronizations in between, must reproduce the eager results bit for bit (the
kernels are deterministic and every workspace is left all-zero, so replays see
the same state as the eager call)."""
import numpy as np
import pytest
import torch

import quantized_gemv_argmax_amd as qg
import workloads
from tests.gpu_helpers import DEV, case, packed_q4k, packed_q8_0, to_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    torch.cuda.set_device(0)
    ws = qg.Workspace(DEV, 8 << 20)
    # q/k/v stage of a 7B layer (grouped), LM head argmax, LM head top-k with a
    # sampler, small-N verify (N=5 short and long K, N=32, N=2 and 3, the slice form),
    # int8-activation product
    stage = []
    for i, (M, K) in enumerate([(3584, 3584), (512, 3584), (512, 3584)]):
        W = workloads.q4k_blocks(M, K, key=(80, i))
        stage.append((packed_q4k(W, M, K), to_dev(workloads.x_vector(K, key=(80, i))),
                      torch.empty(M, device=DEV), M, K))
    Mh, Kh = 20000, 1024
    wh = packed_q8_0(workloads.q8_0_blocks(Mh, Kh, key=(81,)), Mh, Kh)
    xh = to_dev((workloads.x_vector(Kh, key=(81,)) * 0.05).astype(np.float32))
    oi = torch.empty(1, dtype=torch.int32, device=DEV)
    ov = torch.empty(1, device=DEV)
    u = torch.full((1,), 0.3, device=DEV)
    tk = qg.TopK(20, DEV, True)
    lg = torch.empty(Mh, device=DEV)
    M5, K5 = 3584, 3584
    X5 = to_dev(workloads.x_columns(K5, 5, key=(82,)))
    Y5 = torch.empty((5, M5), device=DEV)
    xq = torch.empty(qg.q8_1_bytes(K5), dtype=torch.uint8, device=DEV)
    y8 = torch.empty(M5, device=DEV)
    # the chunked LDS form of the small-N product: a long-K down projection at N=5
    # and the attention output at N=32
    Md, Kd = 3584, 18944
    wd = packed_q4k(workloads.q4k_blocks(Md, Kd, key=(83,)), Md, Kd)
    Xd = to_dev(workloads.x_columns(Kd, 5, key=(83,)))
    Yd = torch.empty((5, Md), device=DEV)
    X32 = to_dev(workloads.x_columns(K5, 32, key=(84,)))
    Y32 = torch.empty((32, M5), device=DEV)
    # the vector-ALU dot form (N <= 4): one super-block per K-group at N=2, the
    # pipelined walk over the long-K down projection at N=3
    X2 = to_dev(workloads.x_columns(K5, 2, key=(85,)))
    Y2 = torch.empty((2, M5), device=DEV)
    Xd3 = to_dev(workloads.x_columns(Kd, 3, key=(86,)))
    Yd3 = torch.empty((3, Md), device=DEV)
    # the walk forms: K slices with a workspace (down projection, N=32; its arrival
    # counters must come back to zero on every replay) and a many-tile walk (N=32
    # over 18944 rows)
    Xd32 = to_dev(workloads.x_columns(Kd, 32, key=(87,)))
    Yd32 = torch.empty((32, Md), device=DEV)
    Mg, Kg = 18944, 3584
    wg = packed_q4k(workloads.q4k_blocks(Mg, Kg, key=(88,)), Mg, Kg)
    Xg32 = to_dev(workloads.x_columns(Kg, 32, key=(88,)))
    Yg32 = torch.empty((32, Mg), device=DEV)
    wss = qg.Workspace(DEV, qg.qgemm_q4k_smalln_batch_workspace_bytes([(wd, Xd32, Yd32, Md, Kd)]))
    # the slice form: K slices with a workspace (down projection, N=5; its counters
    # too must come back to zero) and, without slices, the grouped q/k/v stage at N=5
    Yd5 = torch.empty((5, Md), device=DEV)
    wss5 = qg.Workspace(DEV, qg.qgemm_q4k_smalln_batch_workspace_bytes([(wd, Xd, Yd5, Md, Kd)]))
    Xqkv = to_dev(workloads.x_columns(K5, 5, key=(89,)))
    Yqkv = [torch.empty((5, p[3]), device=DEV) for p in stage]

    def work():
        qg.qgemv_q4k_batch(stage)
        qg.lmhead_argmax(wh, xh, Mh, Kh, out_index=oi, out_value=ov, ws=ws)
        qg.lmhead_topk(wh, xh, Mh, Kh, 20, logits=lg, sampler=(0.9, 0.95, 0.02, u), ws=ws, out=tk)
        qg.qgemm_q4k_smalln(stage[0][0], X5, M5, K5, Y=Y5)
        qg.qgemm_q4k_smalln(wd, Xd, Md, Kd, Y=Yd)
        qg.qgemm_q4k_smalln(stage[0][0], X32, M5, K5, Y=Y32)
        qg.qgemm_q4k_smalln(stage[0][0], X2, M5, K5, Y=Y2)
        qg.qgemm_q4k_smalln(wd, Xd3, Md, Kd, Y=Yd3)
        qg.quantize_q8_1(stage[0][1], out=xq)
        qg.qgemv_q4k_q8_1(stage[0][0], xq, M5, K5, y=y8)
        qg.qgemm_q4k_smalln_batch_ws([(wd, Xd32, Yd32, Md, Kd)], wss)
        qg.qgemm_q4k_smalln(wg, Xg32, Mg, Kg, Y=Yg32)
        qg.qgemm_q4k_smalln_batch_ws([(wd, Xd, Yd5, Md, Kd)], wss5)
        qg.qgemm_q4k_smalln_batch([(p[0], Xqkv, Y_, p[3], p[4]) for p, Y_ in zip(stage, Yqkv)])

    def snapshot():
        torch.cuda.synchronize()
        outs = [p[2] for p in stage] + [oi, ov, tk.index, tk.logit, tk.logprob, tk.lse, tk.token, lg, Y5, Yd, Y32, xq,
                                        y8, Y2, Yd3, Yd32, Yg32, Yd5] + Yqkv
        return [t.clone() for t in outs]

    case("graph capture: eager reference")
    work()
    ref = snapshot()
    assert int(ws.buf.count_nonzero()) == 0

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        # scribble over the outputs, then replay and compare
        for t in snapshot_targets(stage, oi, ov, tk, lg, Y5, Yd, Y32, xq, y8) + [Y2, Yd3, Yd32, Yg32, Yd5] + Yqkv:
            t.zero_()
        case(f"graph replay {rep}")
        g.replay()
        got = snapshot()
        for k, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a, b), f"replay {rep}: output {k} differs from the eager result"
        assert int(ws.buf.count_nonzero()) == 0
        assert int(wss.buf[:4096].count_nonzero()) == 0, "walk-form arrival counters not back to zero"
        assert int(wss5.buf[:4096].count_nonzero()) == 0, "slice-form arrival counters not back to zero"
        # eager work between replays on the same buffers
        qg.qgemv_q4k(stage[1][0], stage[1][1], stage[1][3], stage[1][4], y=stage[1][2])
        torch.cuda.synchronize()


def snapshot_targets(stage, oi, ov, tk, lg, Y5, Yd, Y32, xq, y8):
    return [p[2] for p in stage] + [oi, ov, tk.index, tk.logit, tk.logprob, tk.lse, tk.token, lg, Y5, Yd, Y32, xq, y8]


def test_lmhead_verify_forms_in_a_graph():
    # both verification forms on fp32 columns (vector-ALU N = 5, matrix-core N = 9)
    # and the int8-column form, captured once and replayed three times with eager
    # work in between; every replay must equal the eager result, and the shared
    # workspace (cleared by the kernels themselves, no memset nodes) stays zero
    import numpy as np
    import workloads
    from tests.gpu_helpers import DEV, case, packed_q8_0
    import quantized_gemv_argmax_amd as qg
    M, K = 5000, 1536
    W = workloads.q8_0_blocks(M, K, key=(70,))
    wp = packed_q8_0(W, M, K)
    X5 = torch.from_numpy(workloads.x_columns(K, 5, key=(70, 5))).to(DEV)
    X9 = torch.from_numpy(workloads.x_columns(K, 9, key=(70, 9))).to(DEV)
    xq = qg.quantize_q8_1_columns(X5)
    ws = qg.Workspace(DEV)
    outs = [(torch.empty(n, dtype=torch.int32, device=DEV), torch.empty(n, device=DEV)) for n in (5, 9, 5)]

    def run():
        qg.lmhead_argmax_verify(wp, X5, M, K, out_index=outs[0][0], out_value=outs[0][1], ws=ws)
        qg.lmhead_argmax_verify(wp, X9, M, K, out_index=outs[1][0], out_value=outs[1][1], ws=ws)
        qg.lmhead_argmax_verify_q8_1(wp, xq, M, K, 5, out_index=outs[2][0], out_value=outs[2][1], ws=ws)

    case("LM-head verification forms in a HIP graph")
    run()
    torch.cuda.synchronize()
    ref = [(i.clone(), v.clone()) for i, v in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for i, v in outs:
            i.fill_(-7)
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (i, v), (ri, rv) in zip(outs, ref):
            assert torch.equal(i, ri) and torch.equal(v, rv), rep
        assert int(ws.buf.count_nonzero()) == 0, rep
        run()  # eager work between replays
        torch.cuda.synchronize()
    assert np.all(ref[0][0].cpu().numpy() >= 0)
