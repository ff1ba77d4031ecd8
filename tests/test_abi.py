"""C-ABI checks that need no GPU: exported symbols and host-side validation.

Every call here fails validation (or is an empty no-op) before anything is
launched, so no kernel runs.
"""

import ctypes
import os
import re

import pytest
import torch

import fp8_top_sparse_amd as fts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8ts.h")

EINVAL, EUNSUP = 1, 2


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fts.LIB_PATH):
        pytest.skip("libfp8ts.so not built")
    return fts.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_three_operations():
    names = declared_functions()
    for n in ("fp8_quantize", "fp8_quantize_pair", "indexer_topk", "sparse_attn_fwd", "fp8_cache_store", "fp8_rope_quantize",
              "fp8_qknorm_rope_quantize", "fp8ts_last_error",
              "indexer_topk_workspace_size", "sparse_attn_workspace_size", "fp8ts_abi_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n
        assert n in fts.EXPORTED, n


def test_abi_version(lib):
    assert lib.fp8ts_abi_version() == 1


FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(0x100000)


def last(lib):
    return lib.fp8ts_last_error().decode()


def sc(v):
    return ctypes.byref(ctypes.c_float(v))


# ----------------------------------------------------------- fp8_quantize
def q(lib, **kw):
    a = dict(x=FAKE, dt=0, rows=4, cols=8, xs=8, out=FAKE2, os=8, scale=None)
    a.update(kw)
    return lib.fp8_quantize(a["x"], a["dt"], a["rows"], a["cols"], a["xs"], a["out"], a["os"], a["scale"], None)


def test_quantize_validation(lib):
    assert q(lib, dt=2) == EINVAL and "x_dtype" in last(lib)
    assert q(lib, rows=-1) == EINVAL
    assert q(lib, scale=sc(-1.0)) == EINVAL and "scale" in last(lib)
    assert q(lib, scale=sc(0.0)) == EINVAL
    assert q(lib, scale=sc(float("inf"))) == EINVAL
    assert q(lib, scale=sc(float("nan"))) == EINVAL
    assert q(lib, xs=7) == EINVAL and "x_row_stride" in last(lib)
    assert q(lib, os=4) == EINVAL and "out_row_stride" in last(lib)
    assert q(lib, x=None) == EINVAL
    assert q(lib, out=ctypes.c_void_p(0x1000 + 10)) == EINVAL and "overlap" in last(lib)
    # empty tensors are a no-op that never touches the GPU
    assert q(lib, rows=0) == 0
    assert q(lib, cols=0, x=None, out=None) == 0


# ----------------------------------------------------------- fp8_cache_store
def cs(lib, **kw):
    a = dict(x=FAKE, x2=None, dt=0, n=8, h=2, d=128, d2=0, xts=256, xhs=128, x2ts=0, x2hs=0,
             slots=ctypes.c_void_p(0x20000000), cache=ctypes.c_void_p(0x40000000), pages=4, page=128, scale=None)
    a.update(kw)
    return lib.fp8_cache_store(a["x"], a["x2"], a["dt"], a["n"], a["h"], a["d"], a["d2"], a["xts"], a["xhs"],
                               a["x2ts"], a["x2hs"], a["slots"], a["cache"], a["pages"], a["page"], a["scale"],
                               None)


def qp(lib, **kw):
    a = dict(x0=FAKE, o0=ctypes.c_void_p(0x10000000), n0=1024, s0=None, x1=ctypes.c_void_p(0x20000000),
             o1=ctypes.c_void_p(0x30000000), n1=512, s1=None, dt=0)
    a.update(kw)
    return lib.fp8_quantize_pair(a["x0"], a["o0"], a["n0"], a["s0"], a["x1"], a["o1"], a["n1"], a["s1"], a["dt"],
                                 None)


def test_quantize_pair_validation(lib):
    assert qp(lib, dt=4) == EINVAL and "x_dtype" in last(lib)
    assert qp(lib, n1=-8) == EINVAL
    assert qp(lib, s0=sc(0.0)) == EINVAL and "scale0" in last(lib)
    assert qp(lib, s1=sc(float("inf"))) == EINVAL and "scale1" in last(lib)
    assert qp(lib, x1=None) == EINVAL and "null" in last(lib)
    assert qp(lib, n0=1004) == EUNSUP and "multiples of 8" in last(lib)
    assert qp(lib, x0=ctypes.c_void_p(0x1008)) == EUNSUP and "alignment" in last(lib)
    assert qp(lib, o1=ctypes.c_void_p(0x10000100)) == EINVAL and "overlaps" in last(lib)   # out1 inside out0
    assert qp(lib, o0=ctypes.c_void_p(0x1100)) == EINVAL                                   # out0 inside x0
    assert qp(lib, n0=0, n1=0, x0=None, x1=None, o0=None, o1=None) == 0
    assert qp(lib, n0=0, x0=None, o0=None, s1=sc(-1.0)) == EINVAL                          # scales checked first


def test_cache_store_validation(lib):
    assert cs(lib, dt=3) == EINVAL and "x_dtype" in last(lib)
    assert cs(lib, n=-1) == EINVAL
    assert cs(lib, h=0) == EINVAL
    assert cs(lib, page=0) == EINVAL
    assert cs(lib, d2=64) == EINVAL and "x2" in last(lib)            # dim2 > 0 without x2
    assert cs(lib, x2=FAKE2) == EINVAL and "x2" in last(lib)         # x2 with dim2 == 0
    assert cs(lib, scale=sc(0.0)) == EINVAL and "scale" in last(lib)
    assert cs(lib, scale=sc(float("nan"))) == EINVAL
    assert cs(lib, xhs=64) == EINVAL and "strides" in last(lib)      # heads overlap
    assert cs(lib, xts=200) == EINVAL and "strides" in last(lib)     # tokens overlap
    assert cs(lib, x=None) == EINVAL
    assert cs(lib, pages=0) == EINVAL
    assert cs(lib, cache=ctypes.c_void_p(0x1000 + 64)) == EINVAL and "overlap" in last(lib)
    assert cs(lib, n=1 << 30) == EUNSUP and "2^31" in last(lib)      # 32-bit chunk indexing
    # a head stride is irrelevant with one head; an empty call launches nothing
    assert cs(lib, n=0, x=None, cache=None) == 0


# ----------------------------------------------------------- fp8_rope_quantize
def rq(lib, **kw):
    a = dict(xn=FAKE, xp=ctypes.c_void_p(0x2000), dt=0, n=8, h=16, nope=512, rope=64, nts=16 * 576, nhs=576,
             pts=16 * 576, phs=576, cs=ctypes.c_void_p(0x10000000), maxp=4096, pos=ctypes.c_void_p(0x20000000),
             neox=1, out=ctypes.c_void_p(0x40000000), ots=16 * 576, ohs=576, scale=None)
    a.update(kw)
    return lib.fp8_rope_quantize(a["xn"], a["xp"], a["dt"], a["n"], a["h"], a["nope"], a["rope"], a["nts"],
                                 a["nhs"], a["pts"], a["phs"], a["cs"], a["maxp"], a["pos"], a["neox"], a["out"],
                                 a["ots"], a["ohs"], a["scale"], None)


def test_rope_quantize_validation(lib):
    assert rq(lib, dt=5) == EINVAL and "x_dtype" in last(lib)
    assert rq(lib, rope=63) == EINVAL and "rope_dim" in last(lib)
    assert rq(lib, rope=0) == EINVAL
    assert rq(lib, nope=0) == EINVAL and "x_nope" in last(lib)      # x_nope given without a no-rope part
    assert rq(lib, nope=100) == EUNSUP and "multiple" in last(lib)
    assert rq(lib, rope=24) == EUNSUP
    assert rq(lib, scale=sc(-2.0)) == EINVAL and "scale" in last(lib)
    assert rq(lib, xp=None) == EINVAL
    assert rq(lib, maxp=0) == EINVAL
    assert rq(lib, ohs=500) == EINVAL and "out_head_stride" in last(lib)
    assert rq(lib, ots=576) == EINVAL and "out_token_stride" in last(lib)
    assert rq(lib, xp=ctypes.c_void_p(0x2008)) == EUNSUP and "alignment" in last(lib)
    assert rq(lib, pts=4) == EUNSUP
    assert rq(lib, out=ctypes.c_void_p(0x1000)) == EINVAL and "overlaps" in last(lib)
    assert rq(lib, n=1 << 22) == EUNSUP and "2^31" in last(lib)
    assert rq(lib, n=0, xp=None, out=None) == 0


# ----------------------------------------------------------- fp8_qknorm_rope_quantize
def qn(lib, **kw):
    a = dict(x=FAKE, dt=0, n=8, h=4, d=128, rope=64, xts=512, xhs=128, w=ctypes.c_void_p(0x3000), eps=1e-6,
             cs=ctypes.c_void_p(0x10000000), maxp=4096, pos=ctypes.c_void_p(0x20000000), neox=1,
             out=ctypes.c_void_p(0x40000000), ots=512, ohs=128, slots=None, cache=None, pages=0, page=128,
             scale=None)
    a.update(kw)
    return lib.fp8_qknorm_rope_quantize(a["x"], a["dt"], a["n"], a["h"], a["d"], a["rope"], a["xts"], a["xhs"],
                                        a["w"], a["eps"], a["cs"], a["maxp"], a["pos"], a["neox"], a["out"],
                                        a["ots"], a["ohs"], a["slots"], a["cache"], a["pages"], a["page"],
                                        a["scale"], None)


def test_qknorm_rope_quantize_validation(lib):
    assert qn(lib, dt=2) == EINVAL and "x_dtype" in last(lib)
    assert qn(lib, n=-1) == EINVAL
    assert qn(lib, h=0) == EINVAL
    assert qn(lib, rope=63) == EINVAL and "rope_dim" in last(lib)
    assert qn(lib, rope=256) == EINVAL                                 # rope_dim > head_dim
    assert qn(lib, eps=-1.0) == EINVAL and "eps" in last(lib)
    assert qn(lib, eps=float("inf")) == EINVAL
    assert qn(lib, out=None) == EINVAL and "neither" in last(lib)      # nothing to write
    assert qn(lib, slots=FAKE2, cache=ctypes.c_void_p(0x50000000), pages=4, page=0) == EINVAL
    assert qn(lib, d=100) == EUNSUP and "head_dim" in last(lib)
    assert qn(lib, d=1024, rope=64, xts=4096, xhs=1024, ots=4096, ohs=1024) == EUNSUP
    assert qn(lib, rope=24) == EUNSUP
    assert qn(lib, scale=sc(0.0)) == EINVAL and "scale" in last(lib)
    assert qn(lib, w=None) == EINVAL
    assert qn(lib, pos=None) == EINVAL
    assert qn(lib, slots=FAKE2) == EINVAL and "cache" in last(lib)     # slots without a cache
    assert qn(lib, slots=FAKE2, cache=ctypes.c_void_p(0x50000000), pages=0) == EINVAL
    assert qn(lib, maxp=0) == EINVAL
    assert qn(lib, ohs=100) == EINVAL and "out_head_stride" in last(lib)
    assert qn(lib, ots=128) == EINVAL and "out_token_stride" in last(lib)
    assert qn(lib, x=ctypes.c_void_p(0x1008)) == EUNSUP and "alignment" in last(lib)
    assert qn(lib, w=ctypes.c_void_p(0x3004)) == EUNSUP
    assert qn(lib, out=ctypes.c_void_p(0x1000)) == EINVAL and "out overlaps x" in last(lib)
    assert qn(lib, out=None, slots=FAKE2, cache=ctypes.c_void_p(0x3000), pages=4) == EINVAL and \
        "cache overlaps norm_weight" in last(lib)
    assert qn(lib, n=1 << 22) == EUNSUP and "2^31" in last(lib)
    # rope_dim 0 needs no cos/sin or positions; an empty call launches nothing
    assert qn(lib, n=0, x=None, w=None) == 0


# ----------------------------------------------------------- indexer_topk
def ix(lib, **kw):
    a = dict(q=FAKE, k=FAKE2, pages=16, bt=FAKE, mb=16, cu=FAKE, sl=FAKE, B=1, T=100, mq=100, H=4, D=128,
             page=128, sm=0.1, qs=None, ks=None, topk=8, out=ctypes.c_void_p(0x10000000), ws=FAKE,
             wsz=1 << 30)
    a.update(kw)
    return lib.indexer_topk(a["q"], a["k"], a["pages"], a["bt"], a["mb"], a["cu"], a["sl"], a["B"], a["T"],
                            a["mq"], a["H"], a["D"], a["page"], a["sm"], a["qs"], a["ks"], a["topk"],
                            a["out"], a["ws"], a["wsz"], None)


def test_indexer_validation(lib):
    assert ix(lib, D=64) == EUNSUP and "head_dim" in last(lib)
    assert ix(lib, page=64) == EUNSUP and "page_size" in last(lib)
    assert ix(lib, H=3) == EUNSUP
    assert ix(lib, topk=65) == EUNSUP and "topk" in last(lib)
    assert ix(lib, topk=0) == EUNSUP
    assert ix(lib, mb=5000) == EUNSUP
    assert ix(lib, sm=-1.0) == EINVAL
    assert ix(lib, qs=sc(-2.0)) == EINVAL and "idx_q_scale" in last(lib)
    assert ix(lib, ks=sc(float("nan"))) == EINVAL and "idx_k_scale" in last(lib)
    assert ix(lib, ws=None) == EINVAL and "workspace" in last(lib)
    assert ix(lib, wsz=16) == EINVAL
    assert ix(lib, ws=ctypes.c_void_p(0x1008)) == EINVAL and "aligned" in last(lib)
    assert ix(lib, bt=None) == EINVAL
    assert ix(lib, mq=200) == EINVAL
    assert ix(lib, T=0) == 0          # nothing to do


def test_indexer_workspace_size(lib):
    assert lib.indexer_topk_workspace_size(1000, 4, 256) == 1000 * 4 * 256 * 4
    assert lib.indexer_topk_workspace_size(0, 4, 256) == 0


# ----------------------------------------------------------- sparse_attn_fwd
def at(lib, **kw):
    a = dict(mode=0, q=FAKE, k=FAKE2, v=None, nkv=4096, idx=FAKE, topk=256, tl=None, bt=None, mb=0, cu=None,
             sl=None, B=0, T=64, mq=0, Hq=16, Hkv=1, Hidx=1, Dqk=576, Dv=512, page=0, sm=1 / 24, qs=None,
             ks=None, vs=None, sink=None, out=ctypes.c_void_p(0x10000000), ml=FAKE, lse=FAKE, ws=FAKE,
             wsz=1 << 30)
    a.update(kw)
    return lib.sparse_attn_fwd(a["mode"], a["q"], a["k"], a["v"], a["nkv"], a["idx"], a["topk"], a["tl"], a["bt"],
                               a["mb"], a["cu"], a["sl"], a["B"], a["T"], a["mq"], a["Hq"], a["Hkv"], a["Hidx"],
                               a["Dqk"], a["Dv"], a["page"], a["sm"], a["qs"], a["ks"], a["vs"], a["sink"],
                               a["out"], a["ml"], a["lse"], a["ws"], a["wsz"], None)


BLOCK = dict(mode=1, v=FAKE2, bt=FAKE, mb=64, cu=FAKE, sl=FAKE, B=1, T=8192, mq=8192, Hq=16, Hkv=2, Hidx=4,
             Dqk=128, Dv=128, page=128, topk=64, nkv=64)


def test_attention_token_mode_validation(lib):
    assert at(lib, Dv=256) == EUNSUP and "d_v" in last(lib)
    assert at(lib, Dqk=512) == EUNSUP
    assert at(lib, Hkv=2, Hq=16) == EUNSUP
    assert at(lib, mode=7) == EINVAL
    assert at(lib, sm=float("nan")) == EINVAL
    assert at(lib, qs=sc(0.0)) == EINVAL and "q_scale" in last(lib)
    assert at(lib, ks=sc(-1.0)) == EINVAL and "k_scale" in last(lib)
    assert at(lib, vs=sc(float("inf"))) == EINVAL and "v_scale" in last(lib)
    assert at(lib, idx=None) == EINVAL
    assert at(lib, nkv=0) == EINVAL
    assert at(lib, out=FAKE) == EINVAL and "overlap" in last(lib)
    assert at(lib, T=0) == 0


def test_attention_block_mode_validation(lib):
    assert at(lib, **{**BLOCK, "page": 64}) == EUNSUP and "page_size" in last(lib)
    assert at(lib, **{**BLOCK, "Dv": 64}) == EUNSUP
    assert at(lib, **{**BLOCK, "Hidx": 3}) == EINVAL
    assert at(lib, **{**BLOCK, "Hq": 24, "Hkv": 4, "Hidx": 6}) == EUNSUP    # groups of 6 and 4 do not nest
    assert at(lib, **{**BLOCK, "Hq": 12, "Hkv": 2, "Hidx": 3}) == EUNSUP and "nest" in last(lib)
    assert at(lib, **{**BLOCK, "topk": 65}) == EUNSUP
    assert at(lib, **{**BLOCK, "mb": 5000}) == EUNSUP
    assert at(lib, **{**BLOCK, "v": None}) == EINVAL
    assert at(lib, **{**BLOCK, "bt": None}) == EINVAL
    assert at(lib, **{**BLOCK, "mq": 9000}) == EINVAL
    assert at(lib, **{**BLOCK, "Hq": 15}) == EINVAL


def test_attention_workspace_sizes(lib):
    # block prefill over sequences of several tiles keeps one bf16 V^T tile
    # (128 keys x 128 dims) per (block-table slot, kv head)
    assert lib.sparse_attn_workspace_size(1, 1, 8192, 8192, 16, 2, 4, 128, 64, 64) == 64 * 2 * 128 * 128 * 2
    assert lib.sparse_attn_workspace_size(1, 3, 3 * 4096, 4096, 16, 2, 4, 128, 64, 40) == 3 * 40 * 2 * 128 * 128 * 2
    # short prefill (fewer than 4 tiles per sequence) and large-head token mode need none
    assert lib.sparse_attn_workspace_size(1, 1, 96, 96, 16, 2, 4, 128, 64, 64) == 0
    assert lib.sparse_attn_workspace_size(0, 0, 4096, 0, 128, 1, 1, 512, 2048, 0) == 0
    # decode splits the block union: partial O plus (m, l) per split
    n = lib.sparse_attn_workspace_size(1, 64, 64, 1, 16, 2, 4, 128, 64, 256)
    assert n > 64 * 16 * 128 * 4
    # small token mode splits its index list
    assert lib.sparse_attn_workspace_size(0, 0, 64, 0, 16, 1, 1, 512, 256, 0) > 0


# ----------------------------------------------------------- host logic of the binding
def test_flatten_to_2d():
    x = torch.empty(4, 3, 8)
    assert fts.flatten_to_2d(x) == (12, 8, 8)
    y = torch.empty(4, 3, 16)[..., :8]
    assert fts.flatten_to_2d(y) == (12, 8, 16)
    z = torch.empty(5, 7, 3, 32)[:, :, :, :8]                  # rows of 8 at a 32-element stride
    assert fts.flatten_to_2d(z) == (105, 8, 32)
    assert fts.flatten_to_2d(torch.empty(1, 6, 8)) == (6, 8, 8)
    assert fts.flatten_to_2d(torch.empty(6, 1, 8)[:, :, :]) == (6, 8, 8)
    # a size-1 dim adds no rows, whatever its stride
    w = torch.empty(6, 16).as_strided((6, 1, 8), (16, 999, 1))
    assert fts.flatten_to_2d(w) == (6, 8, 16)
    assert fts.flatten_to_2d(torch.empty(8)) == (1, 8, 8)
    assert fts.flatten_to_2d(torch.empty(0, 4, 8)) == (0, 8, 8)
    with pytest.raises(ValueError):
        fts.flatten_to_2d(torch.empty(8, 4).t())
    with pytest.raises(ValueError):
        fts.flatten_to_2d(torch.empty(4, 6, 8)[:, :3, :])
    with pytest.raises(ValueError):
        fts.flatten_to_2d(torch.empty(3, 4, 8).transpose(0, 1))


# The binding checks what the C ABI cannot see (tensor shapes, dtypes and
# devices) before anything reaches the library; these run on CPU tensors,
# which fail on the shape checks before the device check.
def _block_args(**over):
    T, Hq, Hkv, Hidx, P, D, B, MB, k = 10, 16, 2, 4, 5, 128, 2, 3, 4
    a = dict(q=torch.zeros(T, Hq, D, dtype=torch.uint8), k=torch.zeros(P, Hkv, 128, D, dtype=torch.uint8),
             indices=torch.zeros(Hidx, T, k, dtype=torch.int32), v=torch.zeros(P, Hkv, 128, D, dtype=torch.uint8),
             block_table=torch.zeros(B, MB, dtype=torch.int32), cu_seqlens_q=torch.tensor([0, 4, 10], dtype=torch.int32),
             seq_lens=torch.tensor([4, 6], dtype=torch.int32))
    a.update(over)
    return a


def _run_block(a, **kw):
    return fts.sparse_attn_fwd(a["q"], a["k"], a["indices"], sm_scale=0.1, mode="block", v=a["v"],
                               block_table=a["block_table"], cu_seqlens_q=a["cu_seqlens_q"],
                               seq_lens=a["seq_lens"], max_q_len=6, **kw)


def test_binding_rejects_mismatched_block_tensors(lib):
    with pytest.raises(ValueError, match="k rows hold 64"):
        _run_block(_block_args(k=torch.zeros(5, 2, 128, 64, dtype=torch.uint8)))
    with pytest.raises(ValueError, match="v must be"):
        _run_block(_block_args(v=torch.zeros(4, 2, 128, 128, dtype=torch.uint8)))
    with pytest.raises(ValueError, match="v must be"):
        _run_block(_block_args(v=torch.zeros(5, 1, 128, 128, dtype=torch.uint8)))
    with pytest.raises(ValueError, match="cu_seqlens_q needs"):
        _run_block(_block_args(cu_seqlens_q=torch.tensor([0, 10], dtype=torch.int32)))
    with pytest.raises(ValueError, match="seq_lens"):
        _run_block(_block_args(seq_lens=torch.tensor([4, 6, 1], dtype=torch.int32)))
    with pytest.raises(ValueError, match="out must be"):
        _run_block(_block_args(), out=torch.zeros(10, 16, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must be"):
        _run_block(_block_args(), out=torch.zeros(10, 16, 128, dtype=torch.float32))
    with pytest.raises(ValueError, match="max_logits must be"):
        _run_block(_block_args(), max_logits=torch.zeros(10, 8, dtype=torch.float32))
    with pytest.raises(ValueError, match="lse must be"):
        _run_block(_block_args(), lse=torch.zeros(16, 10, dtype=torch.float32).t())
    # every shape right: the CPU tensors then fail the device check
    with pytest.raises(ValueError, match="must be on"):
        _run_block(_block_args())


def test_binding_rejects_mismatched_token_tensors(lib):
    q = torch.zeros(3, 16, 576, dtype=torch.uint8)
    idx = torch.zeros(3, 8, dtype=torch.int32)
    with pytest.raises(ValueError, match="k rows hold 512"):
        fts.sparse_attn_fwd(q, torch.zeros(100, 512, dtype=torch.uint8), idx, sm_scale=0.1)
    with pytest.raises(ValueError, match="v must be"):
        fts.sparse_attn_fwd(q, torch.zeros(100, 576, dtype=torch.uint8), idx, sm_scale=0.1,
                            v=torch.zeros(99, 512, dtype=torch.uint8))
    with pytest.raises(ValueError, match="topk_length"):
        fts.sparse_attn_fwd(q, torch.zeros(100, 576, dtype=torch.uint8), idx, sm_scale=0.1,
                            topk_length=torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="must be on"):
        fts.sparse_attn_fwd(q, torch.zeros(100, 576, dtype=torch.uint8), idx, sm_scale=0.1)


def test_binding_rejects_mismatched_indexer_tensors(lib):
    iq = torch.zeros(10, 4, 128, dtype=torch.uint8)
    ik = torch.zeros(5, 128, 128, dtype=torch.uint8)
    bt = torch.zeros(2, 3, dtype=torch.int32)
    cu = torch.tensor([0, 4, 10], dtype=torch.int32)
    sl = torch.tensor([4, 6], dtype=torch.int32)
    with pytest.raises(ValueError, match="cu_seqlens_q needs"):
        fts.indexer_topk(iq, ik, bt, cu[:2], sl, max_q_len=6, sm_scale=0.1, topk=4)
    with pytest.raises(ValueError, match="out must be"):
        fts.indexer_topk(iq, ik, bt, cu, sl, max_q_len=6, sm_scale=0.1, topk=4,
                         out=torch.zeros(4, 10, 8, dtype=torch.int32))
    with pytest.raises(ValueError, match="must be on"):
        fts.indexer_topk(iq, ik, bt, cu, sl, max_q_len=6, sm_scale=0.1, topk=4)


def test_binding_maps_status_to_python_errors(lib):
    assert q(lib, dt=9) == EINVAL
    with pytest.raises(ValueError, match="x_dtype"):
        fts._check(EINVAL)
    with pytest.raises(fts.Fp8tsError):
        fts._check(3)


# ----------------------------------------------------------- the header from plain C
C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "fp8ts.h"

int main(void) {
  if (fp8ts_abi_version() != 1) return 10;
  float bad = -1.0f;
  /* every call below fails validation on the host before any launch */
  if (fp8_quantize((const void *)0x1000, 7, 4, 8, 8, (uint8_t *)0x100000, 8, NULL, 0) != FP8TS_EINVAL) return 11;
  if (!strstr(fp8ts_last_error(), "x_dtype")) return 12;
  if (fp8_quantize((const void *)0x1000, FP8TS_BF16, 4, 8, 8, (uint8_t *)0x100000, 8, &bad, 0) != FP8TS_EINVAL)
    return 13;
  if (indexer_topk(NULL, NULL, 1, NULL, 1, NULL, NULL, 1, 1, 1, 4, 64, 128, 0.1f, NULL, NULL, 8, NULL, NULL, 0, 0)
      != FP8TS_EUNSUPPORTED) return 14;
  if (fp8_cache_store((const void *)0x1000, NULL, FP8TS_BF16, 4, 1, 128, 64, 128, 128, 0, 0,
                      (const int64_t *)0x2000, (uint8_t *)0x100000, 4, 128, NULL, 0) != FP8TS_EINVAL) return 15;
  if (fp8_rope_quantize(NULL, (const void *)0x1000, FP8TS_BF16, 4, 1, 0, 63, 0, 0, 64, 64,
                        (const float *)0x2000, 16, (const int64_t *)0x3000, 1, (uint8_t *)0x100000, 64, 64, NULL, 0)
      != FP8TS_EINVAL) return 16;
  if (fp8_qknorm_rope_quantize((const void *)0x1000, FP8TS_BF16, 4, 4, 128, 64, 512, 128, (const float *)0x2000,
                               -1.0f, (const float *)0x3000, 16, (const int64_t *)0x4000, 1, (uint8_t *)0x100000,
                               512, 128, NULL, NULL, 0, 128, NULL, 0) != FP8TS_EINVAL) return 19;
  if (sparse_attn_workspace_size(FP8TS_BLOCK_MODE, 0, 0, 0, 16, 2, 4, 128, 64, 8) != 0) return 17;
  /* empty inputs are no-ops */
  if (fp8_quantize(NULL, FP8TS_FP16, 0, 8, 8, NULL, 8, NULL, 0) != FP8TS_OK) return 18;
  printf("ok\n");
  return 0;
}
"""


def test_header_compiles_as_c_and_links(lib, tmp_path):
    """include/fp8ts.h is a C header: a C program built with gcc links the library
    and gets the documented status codes (host validation only, no GPU)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("gcc or the ROCm headers are missing")
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(fts.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", "/opt/rocm/include", str(src), "-o", str(exe), f"-L{libdir}", "-l:libfp8ts.so",
           f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120,
                       env={**os.environ, "HIP_VISIBLE_DEVICES": ""})
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)
