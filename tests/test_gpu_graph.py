"""The whole path (quantize, indexer, sparse attention) captured in a HIP graph.

Every replay must reproduce the eager results bit for bit.  The graph is
replayed several times with eager steps (into other buffers) and
synchronisations in between, and every replay is checked.  The path issues no
memset, allocation or synchronisation, so nothing in it is unsafe to capture.
"""

import numpy as np
import pytest
import torch

import fp8_top_sparse_amd as fts
import workloads as W

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _bf(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _path(wl):
    """Device inputs of a workload and a step(outs) running the path into outs."""
    lib = fts.load()
    if isinstance(wl, W.BlockWorkload):
        Q, IQ = _bf(wl.q_bf16), _bf(wl.idx_q_bf16)
        KC, VC, IK = _dev(wl.k_cache8), _dev(wl.v_cache8), _dev(wl.idx_k8)
        BT, CU, SL = _dev(wl.block_table), _dev(wl.cu_seqlens_q), _dev(wl.seq_lens)
        T, Hq, D = wl.q_bf16.shape
        Hidx, Hkv = wl.idx_q_bf16.shape[1], wl.k_cache8.shape[1]
        mb = wl.block_table.shape[1]
        iws_n = max(1, lib.indexer_topk_workspace_size(T, Hidx, mb))
        aws_n = max(1, lib.sparse_attn_workspace_size(1, wl.block_table.shape[0], T, wl.max_q_len, Hq, Hkv, Hidx,
                                                      D, wl.topk, mb))

        def outs():
            u8, i32, f32 = torch.uint8, torch.int32, torch.float32
            return dict(q8=torch.empty((T, Hq, D), dtype=u8, device="cuda"),
                        iq8=torch.empty((T, Hidx, D), dtype=u8, device="cuda"),
                        ids=torch.empty((Hidx, T, wl.topk), dtype=i32, device="cuda"),
                        out=torch.empty((T, Hq, D), dtype=torch.bfloat16, device="cuda"),
                        ml=torch.empty((T, Hq), dtype=f32, device="cuda"),
                        lse=torch.empty((T, Hq), dtype=f32, device="cuda"),
                        iws=torch.empty(iws_n, dtype=u8, device="cuda"),
                        aws=torch.empty(aws_n, dtype=u8, device="cuda"))

        def step(o):
            fts.fp8_quantize(Q, wl.q_scale, out=o["q8"])
            fts.fp8_quantize(IQ, wl.idx_q_scale, out=o["iq8"])
            fts.indexer_topk(o["iq8"], IK, BT, CU, SL, max_q_len=wl.max_q_len, sm_scale=wl.idx_sm_scale,
                             topk=wl.topk, idx_q_scale=wl.idx_q_scale, idx_k_scale=wl.idx_k_scale, out=o["ids"],
                             workspace=o["iws"])
            fts.sparse_attn_fwd(o["q8"], KC, o["ids"], v=VC, sm_scale=wl.sm_scale, mode="block", block_table=BT,
                                cu_seqlens_q=CU, seq_lens=SL, max_q_len=wl.max_q_len, q_scale=wl.q_scale,
                                k_scale=wl.k_scale, v_scale=wl.v_scale, attn_sink=None if wl.sink is None
                                else SINK, out=o["out"], max_logits=o["ml"], lse=o["lse"], workspace=o["aws"])
        SINK = None if wl.sink is None else _dev(wl.sink)
        return step, outs
    Q, KV, IDX = _bf(wl.q_bf16), _dev(wl.kv8), _dev(wl.indices)
    SINK = None if wl.sink is None else _dev(wl.sink)
    T, Hq, Dqk = wl.q_bf16.shape
    aws_n = max(1, lib.sparse_attn_workspace_size(0, 0, T, 0, Hq, 1, 1, wl.d_v, wl.indices.shape[1], 0))

    def outs():
        return dict(q8=torch.empty((T, Hq, Dqk), dtype=torch.uint8, device="cuda"),
                    out=torch.empty((T, Hq, wl.d_v), dtype=torch.bfloat16, device="cuda"),
                    ml=torch.empty((T, Hq), dtype=torch.float32, device="cuda"),
                    lse=torch.empty((T, Hq), dtype=torch.float32, device="cuda"),
                    aws=torch.empty(aws_n, dtype=torch.uint8, device="cuda"))

    def step(o):
        fts.fp8_quantize(Q, wl.q_scale, out=o["q8"])
        fts.sparse_attn_fwd(o["q8"], KV, IDX, sm_scale=wl.sm_scale, mode="token", d_v=wl.d_v, q_scale=wl.q_scale,
                            k_scale=wl.k_scale, v_scale=wl.v_scale, attn_sink=SINK, out=o["out"],
                            max_logits=o["ml"], lse=o["lse"], workspace=o["aws"])
    return step, outs


def _results(o):
    return {k: v.clone() for k, v in o.items() if k not in ("iws", "aws")}


def _same(a, b, what):
    for k in a:
        x, y = a[k], b[k]
        if x.dtype.is_floating_point:   # bit patterns: NaN-safe, -inf matches -inf
            x, y = x.view(torch.int16 if x.element_size() == 2 else torch.int32), \
                   y.view(torch.int16 if y.element_size() == 2 else torch.int32)
        assert torch.equal(x, y), f"{what}: {k} differs"


def _check_replays(wl):
    step, outs = _path(wl)
    eager = outs()
    step(eager)
    torch.cuda.synchronize()
    ref = _results(eager)

    # warm-up on a side stream, then capture into buffers of the graph's own
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g_out = outs()
    with torch.cuda.stream(side):
        step(g_out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for o in g_out.values():
        o.zero_()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g_out)
    torch.cuda.synchronize()

    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        _same(ref, _results(g_out), f"replay {r}")
        # eager work into other buffers between replays
        other = outs()
        step(other)
        torch.cuda.synchronize()
        _same(ref, _results(other), f"eager step after replay {r}")
        for k in ("out", "ml", "lse"):
            g_out[k].zero_()
        torch.cuda.synchronize()


@pytest.mark.parametrize("n", [3, 5, 1, 4])
def test_graph_replay_is_bitexact(gpu, n):
    """3: GQA prefill with scales and real selection; 5: batched decode with the
    split-K combine; 1: tiny MLA (16-head kernel, list splits); 4: 128-head MLA."""
    _check_replays(W.workload(n, small=True))


def test_graph_replay_is_bitexact_32k_prefill(gpu):
    """The 32768-token GQA prefill at full size, the step bench.py replays: its
    rows see more causal blocks than they select, so the attention runs the
    16-wave configuration, and the indexer scores and selects."""
    _check_replays(W.workload(3))


def test_producers_graph_replay_is_bitexact(gpu):
    """The producers captured together: K/V rows stored by slot, RoPE +
    quantize of MLA queries, qk-norm + RoPE + quantize of index queries (rows)
    and index keys (stored by slot).  Every replay equals the eager result."""
    g = torch.Generator().manual_seed(21)
    k_new = torch.randn(300, 2, 128, generator=g).to(torch.bfloat16).cuda()
    slots = torch.from_numpy(np.random.default_rng(22).permutation(4 * 128)[:300].astype(np.int64)).cuda()
    q = torch.randn(64, 16, 576, generator=g).to(torch.bfloat16).cuda()
    iq = torch.randn(64, 4, 128, generator=g).to(torch.bfloat16).cuda()
    ik = torch.randn(64, 128, generator=g).to(torch.bfloat16).cuda()
    nw = (torch.rand(128, generator=g) + 0.5).cuda()
    ang = np.arange(256)[:, None] * 10000.0 ** (-np.arange(32) / 32.0)[None, :]
    cs = torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], 1).astype(np.float32)).cuda()
    pos = (torch.arange(64, dtype=torch.int64) * 3).cuda()
    islots = (torch.arange(64, dtype=torch.int64) * 2).cuda()

    def outs():
        return dict(kc=torch.zeros((4, 2, 128, 128), dtype=torch.uint8, device="cuda"),
                    q8=torch.empty((64, 16, 576), dtype=torch.uint8, device="cuda"),
                    iq8=torch.empty((64, 4, 128), dtype=torch.uint8, device="cuda"),
                    ikc=torch.zeros((1, 128, 128), dtype=torch.uint8, device="cuda"))

    def step(o):
        fts.fp8_cache_store(k_new, slots, o["kc"], scale=0.75)
        fts.fp8_rope_quantize(q[..., 512:], cs, pos, x_nope=q[..., :512], out=o["q8"], scale=1.5)
        fts.fp8_qknorm_rope_quantize(iq, nw, 1e-6, rope_dim=64, cos_sin_cache=cs, positions=pos, out=o["iq8"])
        fts.fp8_qknorm_rope_quantize(ik, nw, 1e-6, rope_dim=64, cos_sin_cache=cs, positions=pos, write_out=False,
                                     slot_mapping=islots, cache=o["ikc"])

    eager = outs()
    step(eager)
    torch.cuda.synchronize()
    ref = _results(eager)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g_out = outs()
    with torch.cuda.stream(side):
        step(g_out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(g_out)
    torch.cuda.synchronize()
    for r in range(3):
        for o in g_out.values():
            o.zero_()                      # eager fill kernels, outside the graph
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same(ref, _results(g_out), f"producer replay {r}")
        other = outs()
        step(other)
        torch.cuda.synchronize()
        _same(ref, _results(other), f"eager producers after replay {r}")
