"""sparse_attn_fwd_noalloc (the library's per-device scratch instead of a
workspace) against sparse_attn_fwd with a caller workspace: the same kernels,
so the outputs must agree bit for bit.  Two calls in a row share the scratch,
the second with a smaller input (a prefill that fills the scratch with V^T
tiles, then a decode batch that reuses it for split partials), then a token-
mode call with split lists; a call needing more scratch than the library
holds is refused before any launch."""

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import indexer as OI
import workloads as W
from helpers import assert_attention_close, dev, host

pytestmark = pytest.mark.gpu
PAGE = 128


def _block_case(seq_lens, q_lens, seed, topk, Hq=16, Hkv=2, Hidx=4):
    rng = np.random.default_rng(seed)
    B = len(seq_lens)
    nbs = [(s + PAGE - 1) // PAGE for s in seq_lens]
    P = sum(nbs) + 2
    perm = rng.permutation(P).astype(np.int32)
    bt = np.full((B, max(nbs)), -1, np.int32)
    o = 0
    for b, nb in enumerate(nbs):
        bt[b, :nb] = perm[o:o + nb]
        o += nb
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = int(cu[-1])
    codes = lambda shape, std=1.0: W.e4m3_codes((rng.standard_normal(shape) * std).astype(np.float32))
    q8, kc, vc = codes((T, Hq, 128), 1.5), codes((P, Hkv, PAGE, 128)), codes((P, Hkv, PAGE, 128))
    iq, ik = codes((T, Hidx, 128)), codes((P, PAGE, 128))
    sl = np.asarray(seq_lens, np.int32)
    ids = OI.indexer_topk(iq, ik, bt, cu, sl, sm_scale=0.1, topk=topk)
    sink = (rng.standard_normal(Hq) * 4).astype(np.float32)
    return dict(q8=q8, kc=kc, vc=vc, ids=ids, bt=bt, cu=cu, sl=sl, mq=max(q_lens), sink=sink)


def _both(gpu, c, **kw):
    args = (dev(c["q8"]), dev(c["kc"]), dev(c["ids"]))
    common = dict(v=dev(c["vc"]), sm_scale=0.088, mode="block", block_table=dev(c["bt"]),
                  cu_seqlens_q=dev(c["cu"]), seq_lens=dev(c["sl"]), max_q_len=c["mq"], attn_sink=dev(c["sink"]),
                  **kw)
    ref = gpu.sparse_attn_fwd(*args, **common)
    got = gpu.sparse_attn_fwd_noalloc(*args, **common)
    return ref, got


def test_noalloc_matches_workspace_entry_on_consecutive_calls(gpu):
    lib = gpu.load()
    cap = gpu.sparse_attn_noalloc_scratch_bytes()
    assert cap == 32 << 20
    # 1) prefill of 3 sequences: V^T tiles of every block-table slot in the scratch
    c1 = _block_case([3000, 2100, 1500], [3000, 2100, 700], seed=81, topk=8)
    need1 = lib.sparse_attn_workspace_size(1, 3, 5800, 3000, 16, 2, 4, 128, 8, c1["bt"].shape[1])
    assert 0 < need1 <= cap
    ref, got = _both(gpu, c1, q_scale=0.8, k_scale=1.2, v_scale=1.5)
    for x, y in zip(ref, got):
        assert torch.equal(x, y)
    toks = np.arange(0, 5800, 17)
    r = OA.sparse_attn_block(c1["q8"], c1["kc"], c1["vc"], c1["ids"], c1["bt"], c1["cu"], c1["sl"], sm_scale=0.088,
                             q_scale=0.8, k_scale=1.2, v_scale=1.5, attn_sink=c1["sink"], tokens=toks)
    sel = torch.from_numpy(toks).cuda()
    assert_attention_close((got[0][sel], got[1][sel], got[2][sel]), r, "noalloc prefill")
    # 2) a smaller decode batch right after: split partials in the same scratch
    c2 = _block_case([5000, 900, 12000, 129], [1, 1, 1, 1], seed=82, topk=16)
    ref, got = _both(gpu, c2)
    for x, y in zip(ref, got):
        assert torch.equal(x, y)
    r = OA.sparse_attn_block(c2["q8"], c2["kc"], c2["vc"], c2["ids"], c2["bt"], c2["cu"], c2["sl"], sm_scale=0.088,
                             attn_sink=c2["sink"])
    assert_attention_close(got, r, "noalloc decode")


def test_noalloc_token_mode_split_lists(gpu):
    rng = np.random.default_rng(83)
    q8 = W.e4m3_codes((rng.standard_normal((5, 16, 576)) * 2).astype(np.float32))
    kv8 = W.e4m3_codes(rng.standard_normal((3000, 576)).astype(np.float32))
    idx = np.stack([rng.choice(3000, 256, replace=False) for _ in range(5)]).astype(np.int32)
    sk = (rng.standard_normal(16) * 3).astype(np.float32)
    kw = dict(sm_scale=1 / 24, mode="token", q_scale=0.5, k_scale=0.25, v_scale=2.0, attn_sink=dev(sk))
    ref = [host(x) for x in gpu.sparse_attn_fwd(dev(q8), dev(kv8), dev(idx), **kw)]
    got = [host(x) for x in gpu.sparse_attn_fwd_noalloc(dev(q8), dev(kv8), dev(idx), **kw)]
    for x, y in zip(ref, got):
        assert np.array_equal(x, y)


def test_noalloc_refuses_calls_beyond_its_scratch(gpu):
    # 2 sequences over 1024-slot block tables: 2 * 1024 * 2 kv heads * 32 KB of V^T tiles = 128 MiB
    q8 = torch.zeros((2 * 600, 16, 128), dtype=torch.uint8, device="cuda")
    kc = torch.zeros((4, 2, PAGE, 128), dtype=torch.uint8, device="cuda")
    ids = torch.full((4, 1200, 8), -1, dtype=torch.int32, device="cuda")
    bt = torch.full((2, 1024), -1, dtype=torch.int32, device="cuda")
    cu = torch.tensor([0, 600, 1200], dtype=torch.int32, device="cuda")
    sl = torch.tensor([600, 600], dtype=torch.int32, device="cuda")
    lib = gpu.load()
    assert lib.sparse_attn_workspace_size(1, 2, 1200, 600, 16, 2, 4, 128, 8, 1024) > gpu.sparse_attn_noalloc_scratch_bytes()
    with pytest.raises(ValueError, match="scratch"):
        gpu.sparse_attn_fwd_noalloc(q8, kc, ids, v=kc, sm_scale=0.1, mode="block", block_table=bt, cu_seqlens_q=cu,
                                    seq_lens=sl, max_q_len=600)
