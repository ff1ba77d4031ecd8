"""Benchmark of the FP8 top-k sparse attention hot path on one MI355X.

One step = the whole path over one batch of synthetic input, inputs resident
in HBM: fp8_quantize of Q and idx_q (one fp8_quantize_pair launch),
indexer_topk, sparse_attn_fwd.  Default workload: the 32768-token causal GQA
block-sparse prefill with U(0.1, 4) per-tensor scales (16 q / 2 kv heads, d
128, page 128, 4 index heads, top-64 of 256 blocks), where all three steps do
real work.  The long-MLA prefill (4096 x 128 heads, top-2048 of 65536 tokens)
and the decode batch (64 x 32k, top-64 blocks) follow under "extra_workloads"
(--workload N times one of them alone).

Prints ONE JSON line.  ``value`` = algorithmic attention TFLOP/s over the whole
step, timed over K replays of the step captured as one HIP graph; ``roofline``
describes the dominant kernel (sparse attention), timed with HIP events on the
stream it runs on over K eager steps, each after a 512 MiB read that evicts
the 256 MB last-level cache; ``cpu_baseline`` times the CPU oracle on a
bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N]
       [--no-extra] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA
PEAK_HBM_GBPS = 8000.0       # MI355X HBM3E
PAGE = 128


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-extra", action="store_true", help="skip the extra workloads (4 and 5)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (HBM counter calibration)")
    return ap.parse_args()


def calibrate_copy(mib: int) -> None:
    """A plain copy of known size, so rocprofv3 FETCH_SIZE / WRITE_SIZE can be scaled."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}))


# Q and idx_q quantized by one fp8_quantize_pair launch (same bytes as two
# fp8_quantize calls); FP8TS_BENCH_SINGLE_QUANTIZE=1 times the two calls instead
PAIR_QUANTIZE = os.environ.get("FP8TS_BENCH_SINGLE_QUANTIZE", "0") != "1"

TRAFFIC_SUMMARY = {2: "profiles/attn_block_prefill__gqa_prefill_8192.md",
                   3: "profiles/attn_block_prefill__gqa_prefill_32768_h16kv2_top64_scaled.md",
                   4: "profiles/attn_token_mla__mla_prefill_4096x128_s65536_top2048.md",
                   5: "profiles/attn_block_decode__gqa_decode_b64_s32768_top64.md"}


# the source file of the attention kernel that dominates each workload's step
KERNEL_SOURCE = {2: "fp8_top_sparse_amd/csrc/attention_block.hip",
                 3: "fp8_top_sparse_amd/csrc/attention_block.hip",
                 4: "fp8_top_sparse_amd/csrc/attention_latent.hip",
                 5: "fp8_top_sparse_amd/csrc/attention_decode.hip"}


def kernel_source_digest(workload: int) -> str:
    """sha256 (first 16 hex) of the workload's attention kernel source and its build flags."""
    import hashlib
    h = hashlib.sha256()
    for f in (KERNEL_SOURCE[workload], "fp8_top_sparse_amd/csrc/attn_common.h",
              "fp8_top_sparse_amd/csrc/device.h", "fp8_top_sparse_amd/build.py"):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(workload: int):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary,
    or None when there is none or the kernel changed since it was taken."""
    path = TRAFFIC_SUMMARY.get(workload)
    if not path or not os.path.exists(os.path.join(ROOT, path)):
        return None
    text = open(os.path.join(ROOT, path)).read()
    import re
    dig = re.search(r"first 16 hex\): `([0-9a-f]{16})`", text)
    val = re.search(r"traffic_bytes_per_launch: (\d+)", text)
    if not dig or not val or dig.group(1) != kernel_source_digest(workload):
        return None
    return int(val.group(1))


def block_attention_flops(ids: np.ndarray, pos: np.ndarray, hq: int, hidx: int, d_qk: int, d_v: int) -> int:
    """Exact algorithmic flops: 2 (d_qk + d_v) per (query head, visible selected key)."""
    valid = ids >= 0
    n = np.clip(pos[None, :, None] + 1 - PAGE * ids.astype(np.int64), 0, PAGE)
    keys = int(np.where(valid, n, 0).sum())
    return keys * (hq // hidx) * 2 * (d_qk + d_v)


def block_prefill_issued_flops(ids: np.ndarray, cu_seqlens_q, pos: np.ndarray, hq: int, hkv: int, hidx: int,
                               d: int, max_blocks: int, rows_per_wg: int = 256):
    """Matrix-core work the block prefill kernel issues for these selections
    (QK + PV, 2 * 2 * d flop per row and key), as against the algorithmic
    count: a workgroup takes rows_per_wg rows of one (sequence, kv head),
    rows ordered token-major (row r: token r // G, head r % G), and visits the
    union of its rows' selected blocks; each 16-row wave computes a block's
    128 keys for all its rows when any of its rows selected the block, and
    skips it otherwise.  None when G does not divide 16 (no such shapes here)."""
    G = hq // hkv
    gqi = hq // hidx
    if 16 % G:
        return None
    tw, tt = 16 // G, rows_per_wg // G           # tokens per wave, per workgroup
    T = ids.shape[1]
    sel = np.zeros((hidx, T, max_blocks), bool)
    for h in range(hidx):
        r = np.repeat(np.arange(T), ids.shape[2])
        v = ids[h].reshape(-1).astype(np.int64)
        ok = (v >= 0) & (v < max_blocks)
        sel[h, r[ok], v[ok]] = True
    sel &= np.arange(max_blocks)[None, None, :] <= (pos // PAGE)[None, :, None]   # blocks with a visible key
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    waves = 0
    for kh in range(hkv):
        lists = sorted({(kh * G + h) // gqi for h in range(G)})
        s_kh = np.logical_or.reduce(sel[lists], axis=0)          # [T, blocks]: any list of the token
        for b in range(len(cu) - 1):
            for t0 in range(int(cu[b]), int(cu[b + 1]), tt):
                tile = s_kh[t0:min(t0 + tt, int(cu[b + 1]))]
                union = tile.any(0)
                pad = np.zeros((tt - tile.shape[0], max_blocks), bool)
                per_wave = np.concatenate([tile, pad]).reshape(tt // tw, tw, max_blocks).any(1)
                waves += int(per_wave[:, union].sum())
    return waves * 16 * PAGE * d * 4


def decode_attention_bytes(ids: np.ndarray, seq: np.ndarray, hq: int, hidx: int, hkv: int, d: int) -> int:
    """Algorithmic HBM bytes of block-mode decode attention: every (sequence, kv
    head) reads the K and V pages of the union of its index heads' selected
    blocks once (2 * PAGE * d bytes each), plus the e4m3 queries and the bf16
    outputs (max_logits / lse: 8 bytes per row)."""
    per_kv = hidx // hkv
    pages = 0
    for b in np.unique(seq):
        rows = np.nonzero(seq == b)[0]
        for kh in range(hkv):
            sel = ids[kh * per_kv:(kh + 1) * per_kv][:, rows].ravel()
            pages += len(np.unique(sel[sel >= 0]))
    rows = len(seq) * hq
    return pages * 2 * PAGE * d + rows * (d + 2 * d + 8)


def token_positions(cu_seqlens_q, seq_lens):
    """(sequence id, absolute position) of every flattened query token."""
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    sl = np.asarray(seq_lens, dtype=np.int64)
    seq = np.repeat(np.arange(len(sl)), np.diff(cu))
    start = cu[:-1][seq]
    return seq, sl[seq] - (cu[1:] - cu[:-1])[seq] + (np.arange(int(cu[-1])) - start)


def timed_copies(pairs, flush, reps: int) -> dict:
    """A reference for small HBM-bound launches: torch device copies dst <- src
    of the same input tensors, one launch each as the producer makes, timed
    the same way (cache-evicting read between repetitions).  Bytes: 2 read +
    2 written per bf16 element."""
    import torch
    nbytes = sum(4 * src.numel() for src, _ in pairs)

    def run():
        for src, dst in pairs:
            dst.copy_(src)

    run()
    times = []
    for _ in range(reps):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = float(np.mean(times))
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"launches": len(pairs), "ms": round(ms, 4), "bytes": int(nbytes), "GBps": round(gbps, 1),
            "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4)}


def measure_cache_store(fts, wl, block: bool, reps: int) -> dict:
    """fp8_cache_store of the workload's new keys into fresh caches, HBM-bound.

    Block workloads store K and V ([T, Hkv, 128] bf16 each, with the
    workload's scales) and index-K ([T, 128]) into paged caches through the
    block table; token workloads pack latent (512) + rope (64) rows into the
    flat [S, 576] array.  Algorithmic bytes: 2 read + 1 written per element,
    plus 8 per slot per call.  A 512 MiB buffer is read between repetitions
    (outside the events) so the inputs come from HBM, not the 256 MB
    last-level cache; reading leaves no dirty lines whose write-back would be
    charged to the store.
    """
    import torch
    g = torch.Generator(device="cuda").manual_seed(77)
    if block:
        T = wl.q_bf16.shape[0]
        P, Hkv = wl.k_cache8.shape[0], wl.k_cache8.shape[1]
        seq, pos = token_positions(wl.cu_seqlens_q, wl.seq_lens)     # this step's new keys
        slots = torch.from_numpy(wl.block_table[seq, pos // PAGE].astype(np.int64) * PAGE + pos % PAGE).cuda()
        jobs = []
        for heads, scale in ((Hkv, wl.k_scale), (Hkv, wl.v_scale), (1, wl.idx_k_scale)):
            x = torch.randn((T, heads, 128), generator=g, device="cuda").to(torch.bfloat16)
            cache = torch.empty((P, heads, PAGE, 128), dtype=torch.uint8, device="cuda")
            jobs.append((x, None, cache, scale))
        n_tok = T
    else:
        S = wl.kv8.shape[0]
        slots = torch.arange(S, dtype=torch.int64, device="cuda")
        kv_a = torch.randn((S, 512), generator=g, device="cuda").to(torch.bfloat16)
        k_pe = torch.randn((S, 64), generator=g, device="cuda").to(torch.bfloat16)
        jobs = [(kv_a, k_pe, torch.empty((S, 576), dtype=torch.uint8, device="cuda"), wl.k_scale)]
        n_tok = S
    elems = sum(x.numel() + (0 if x2 is None else x2.numel()) for x, x2, _, _ in jobs)
    nbytes = 3 * elems + 8 * n_tok * len(jobs)
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")

    def run():
        for x, x2, cache, scale in jobs:
            fts.fp8_cache_store(x, slots, cache, scale=scale, x2=x2)

    run()
    times = []
    for _ in range(reps):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = float(np.mean(times))
    gbps = nbytes / (ms * 1e-3) / 1e9
    copies = [(x, torch.empty_like(x)) for x, _, _, _ in jobs]
    return {"ms": round(ms, 4), "launches": len(jobs), "bytes": int(nbytes), "GBps": round(gbps, 1),
            "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
            "device_copy_same_inputs": timed_copies(copies, flush, reps)}


def measure_rope_quantize(fts, Q, reps: int) -> dict:
    """fp8_rope_quantize of the MLA queries: no-rope part 512 + rope part 64
    (rotate-half, RoFormer angles, positions 0..T-1), HBM-bound.

    Algorithmic bytes: 2 read + 1 written per element, plus 8 per position
    and the fp32 cos/sin rows of the T positions.  The same 512 MiB read
    flush as the cache store runs between repetitions.
    """
    import torch
    T, H, D = Q.shape
    R = D - 512
    i = np.arange(R // 2, dtype=np.float64)
    ang = np.arange(T, dtype=np.float64)[:, None] * 10000.0 ** (-2.0 * i / R)[None, :]
    cache = torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)).cuda()
    pos = torch.arange(T, dtype=torch.int64, device="cuda")
    out = torch.empty((T, H, D), dtype=torch.uint8, device="cuda")
    nbytes = 3 * Q.numel() + 8 * T + 4 * T * R
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")

    def run():
        fts.fp8_rope_quantize(Q[..., 512:], cache, pos, x_nope=Q[..., :512], out=out)

    run()
    times = []
    for _ in range(reps):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = float(np.mean(times))
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "bytes": int(nbytes), "GBps": round(gbps, 1),
            "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4)}


def measure_qknorm_rope_quantize(fts, T: int, hidx: int, reps: int) -> dict:
    """fp8_qknorm_rope_quantize of a step's index rows: the index query
    [T, hidx, 128] into fp8 rows and the T new index keys [T, 128] stored into
    the paged index-K cache, both with the last 64 dims rotated (rotate-half,
    RoFormer angles, positions 0..T-1), seeded N(0, 1) bf16 inputs.

    Algorithmic bytes: 2 read + 1 written per element, plus per token its
    position (8 B, read by both calls), slot (8 B) and the two fp32 cos/sin
    rows (256 B each call).  The same 512 MiB read flush as the other producers
    runs between repetitions.
    """
    import torch
    R, D = 64, 128
    g = torch.Generator(device="cuda").manual_seed(11)
    iq = torch.randn((T, hidx, D), generator=g, device="cuda").to(torch.bfloat16)
    ik = torch.randn((T, D), generator=g, device="cuda").to(torch.bfloat16)
    w = torch.rand(D, generator=g, device="cuda") + 0.5
    i = np.arange(R // 2, dtype=np.float64)
    ang = np.arange(T, dtype=np.float64)[:, None] * 10000.0 ** (-2.0 * i / R)[None, :]
    cache = torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)).cuda()
    pos = torch.arange(T, dtype=torch.int64, device="cuda")
    pages = (T + PAGE - 1) // PAGE
    kc = torch.empty((pages, PAGE, D), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, hidx, D), dtype=torch.uint8, device="cuda")
    nbytes = 3 * (iq.numel() + ik.numel()) + T * (8 + 8 + 8 + 2 * 4 * R)
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")

    def run():
        fts.fp8_qknorm_rope_quantize(iq, w, 1e-6, rope_dim=R, cos_sin_cache=cache, positions=pos, out=out)
        fts.fp8_qknorm_rope_quantize(ik, w, 1e-6, rope_dim=R, cos_sin_cache=cache, positions=pos,
                                     write_out=False, slot_mapping=pos, cache=kc)

    run()
    times = []
    for _ in range(reps):
        flush.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = float(np.mean(times))
    gbps = nbytes / (ms * 1e-3) / 1e9
    copies = [(iq, torch.empty_like(iq)), (ik, torch.empty_like(ik))]
    return {"launches": 2, "ms": round(ms, 4), "bytes": int(nbytes), "GBps": round(gbps, 1),
            "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
            "device_copy_same_inputs": timed_copies(copies, flush, reps)}


def run_workload(n: int, steps: int, warmup: int, producers: bool) -> dict:
    """Times workload n: K graph replays of the whole step (``value``), then K
    eager steps with HIP events around each call (per-kernel times), each
    eager step after a 512 MiB read that evicts the last-level cache."""
    import torch
    import fp8_top_sparse_amd as fts
    import workloads as W

    lib = fts.load()
    wl = W.workload(n)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    block = isinstance(wl, W.BlockWorkload)
    if block:
        Q = bf(wl.q_bf16)
        IQ = bf(wl.idx_q_bf16)
        KC, VC, IK = d(wl.k_cache8), d(wl.v_cache8), d(wl.idx_k8)
        BT, CU, SL = d(wl.block_table), d(wl.cu_seqlens_q), d(wl.seq_lens)
        T, Hq, D = wl.q_bf16.shape
        Hidx = wl.idx_q_bf16.shape[1]
        Hkv = wl.k_cache8.shape[1]
        q8 = torch.empty((T, Hq, D), dtype=torch.uint8, device="cuda")
        iq8 = torch.empty((T, Hidx, D), dtype=torch.uint8, device="cuda")
        ids = torch.empty((Hidx, T, wl.topk), dtype=torch.int32, device="cuda")
        out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device="cuda")
        ml = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
        lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
        iws = torch.empty(max(1, lib.indexer_topk_workspace_size(T, Hidx, wl.block_table.shape[1])),
                          dtype=torch.uint8, device="cuda")
        aws_n = lib.sparse_attn_workspace_size(1, wl.block_table.shape[0], T, wl.max_q_len, Hq, Hkv, Hidx, D,
                                               wl.topk, wl.block_table.shape[1])
        aws = torch.empty(max(1, aws_n), dtype=torch.uint8, device="cuda")
    else:
        Q = bf(wl.q_bf16)
        KV, IDX = d(wl.kv8), d(wl.indices)
        SINK = None if wl.sink is None else d(wl.sink)
        T, Hq, Dqk = wl.q_bf16.shape
        q8 = torch.empty((T, Hq, Dqk), dtype=torch.uint8, device="cuda")
        out = torch.empty((T, Hq, wl.d_v), dtype=torch.bfloat16, device="cuda")
        ml = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
        lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
        aws_n = lib.sparse_attn_workspace_size(0, 0, T, 0, Hq, 1, 1, wl.d_v, wl.indices.shape[1], 0)
        aws = torch.empty(max(1, aws_n), dtype=torch.uint8, device="cuda")

    kinds = ("quant", "index", "attn") if block else ("quant", "attn")

    def new_events():
        return {k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for k in kinds}

    def step(ev=None):
        def rec(k, i):
            if ev is not None:
                ev[k][i].record()
        rec("quant", 0)
        if block and PAIR_QUANTIZE:
            fts.fp8_quantize_pair(Q, wl.q_scale, IQ, wl.idx_q_scale, out0=q8, out1=iq8)
        else:
            fts.fp8_quantize(Q, wl.q_scale, out=q8)
            if block:
                fts.fp8_quantize(IQ, wl.idx_q_scale, out=iq8)
        rec("quant", 1)
        if block:
            rec("index", 0)
            fts.indexer_topk(iq8, IK, BT, CU, SL, max_q_len=wl.max_q_len, sm_scale=wl.idx_sm_scale,
                             topk=wl.topk, idx_q_scale=wl.idx_q_scale, idx_k_scale=wl.idx_k_scale, out=ids,
                             workspace=iws)
            rec("index", 1)
            rec("attn", 0)
            fts.sparse_attn_fwd(q8, KC, ids, v=VC, sm_scale=wl.sm_scale, mode="block", block_table=BT,
                                cu_seqlens_q=CU, seq_lens=SL, max_q_len=wl.max_q_len, q_scale=wl.q_scale,
                                k_scale=wl.k_scale, v_scale=wl.v_scale, out=out, max_logits=ml, lse=lse,
                                workspace=aws)
            rec("attn", 1)
        else:
            rec("attn", 0)
            fts.sparse_attn_fwd(q8, KV, IDX, sm_scale=wl.sm_scale, mode="token", d_v=wl.d_v,
                                q_scale=wl.q_scale, k_scale=wl.k_scale, v_scale=wl.v_scale, attn_sink=SINK,
                                out=out, max_logits=ml, lse=lse, workspace=aws)
            rec("attn", 1)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # algorithmic work, counted from the path's own selections
    index_flops = 0
    index_scored = False
    if block:
        _, pos = token_positions(wl.cu_seqlens_q, wl.seq_lens)
        ids_h = ids.cpu().numpy()
        flops = block_attention_flops(ids_h, pos, Hq, Hidx, D, D)
        quant_bytes = 3 * (wl.q_bf16.size + wl.idx_q_bf16.size)
        # indexer bytes: ids written; when some row needs scoring, also the index
        # query and every index key of the sequence read once.  Indexer flops:
        # 2 * 128 per (index head, visible key) of every row with more blocks than k
        nb = pos // PAGE + 1
        index_bytes = ids_h.size * 4
        index_scored = bool((nb > wl.topk).any())
        if index_scored:
            index_bytes += wl.idx_q_bf16.size + int(wl.seq_lens.sum()) * 128
            index_flops = int((pos[nb > wl.topk] + 1).sum()) * Hidx * 2 * 128
    else:
        idx = wl.indices
        n_valid = int(((idx >= 0) & (idx < wl.kv8.shape[0])).sum())
        flops = n_valid * Hq * 2 * (Dqk + wl.d_v)
        quant_bytes = 3 * wl.q_bf16.size
        index_bytes = 0

    # The step is captured once as a HIP graph (its launches replay with no
    # host work in between; the path issues no allocation, memset or
    # synchronisation) after a warm-up on the capture stream.
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()

    # timed region: exactly K steps (graph replays)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)

    # per-kernel times: K eager steps with HIP events on the launch stream,
    # each after a 512 MiB read (outside the events) that evicts the 256 MB
    # last-level cache, so every input comes from HBM; a read leaves no dirty
    # lines whose write-back would land inside the timed step
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    evs = [new_events() for _ in range(steps)]
    for i in range(steps):
        flush.sum()
        step(evs[i])
    torch.cuda.synchronize()
    ms = {k: float(np.mean([e[k][0].elapsed_time(e[k][1]) for e in evs])) for k in kinds}
    ms.setdefault("index", None)
    del flush

    ms_step = total_ms / steps
    attn_tflops = flops / (ms["attn"] * 1e-3) / 1e12
    value = flops / (ms_step * 1e-3) / 1e12
    res = {
        "value": round(value, 3),
        "ms_per_step": round(ms_step, 4),
        "config": {"workload": wl.name, "tokens": int(T), "q_heads": int(Hq),
                   "attention_gflop_per_step": round(flops / 1e9, 3)},
        "kernels_ms": {k: (round(v, 4) if v is not None else None) for k, v in ms.items()},
        "attention_tflops": round(attn_tflops, 3),
        "attention_frac_fp8_peak": round(attn_tflops / PEAK_FP8_TFLOPS, 4),
        "quantize_GBps": round(quant_bytes / (ms["quant"] * 1e-3) / 1e9, 1),
        "quantize_frac_hbm_peak": round(quant_bytes / (ms["quant"] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 3), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": committed_traffic(n)},
    }
    if block and wl.max_q_len > 1:
        issued = block_prefill_issued_flops(ids_h, wl.cu_seqlens_q, pos, Hq, Hkv, Hidx, D, wl.block_table.shape[1])
        if issued:
            itf = issued / (ms["attn"] * 1e-3) / 1e12
            res["attention_issued"] = {"gflop": round(issued / 1e9, 3), "useful_fraction": round(flops / issued, 4),
                                       "tflops": round(itf, 3), "frac_fp8_peak": round(itf / PEAK_FP8_TFLOPS, 4)}
    if block:
        gbps = index_bytes / (ms["index"] * 1e-3) / 1e9
        res["indexer_topk_GBps"] = round(gbps, 1)
        if index_scored:
            itf = index_flops / (ms["index"] * 1e-3) / 1e12
            res["indexer_scoring"] = {"gflop": round(index_flops / 1e9, 3), "tflops": round(itf, 3),
                                      "frac_fp8_peak": round(itf / PEAK_FP8_TFLOPS, 4), "bytes": int(index_bytes)}
        else:
            # no row sees more than k blocks: the ids are the closed form, written
            # without scoring, so the rate is that of an id write
            res["indexer_topk_note"] = "closed form: no row has more than k blocks, nothing scored"
    if block and wl.max_q_len == 1:
        # decode: one query per sequence, so the attention streams the selected
        # K/V pages and is bound by HBM, not by the matrix cores
        seq, _ = token_positions(wl.cu_seqlens_q, wl.seq_lens)
        dbytes = decode_attention_bytes(ids_h, seq, Hq, Hidx, Hkv, D)
        gbps = dbytes / (ms["attn"] * 1e-3) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                           "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": committed_traffic(n),
                           "algorithmic_bytes": int(dbytes)}
        # the decode indexer reads every index key of the batch once
        res["indexer_topk_frac_hbm_peak"] = round(res["indexer_topk_GBps"] / PEAK_HBM_GBPS, 4)
    if producers:
        res["cache_store"] = measure_cache_store(fts, wl, block, steps)
        if block:
            res["qknorm_rope_quantize"] = measure_qknorm_rope_quantize(fts, int(T), int(Hidx), steps)
        else:
            res["rope_quantize"] = measure_rope_quantize(fts, Q, steps)
    del graph
    torch.cuda.synchronize()
    return res, wl, block


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "this build has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return

    import torch
    import fp8_top_sparse_amd as fts

    fts.load()
    torch.cuda.set_device(0)
    head, wl, block = run_workload(args.workload, args.steps, args.warmup, producers=True)
    result = {
        "metric": "fp8 sparse-attn prefill TFLOP/s (% fp8 MFMA peak); indexer top-k GB/s",
        "value": head.pop("value"),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (QK) / bf16 (PV)",
        "data": "synthetic",
        "launch": "one captured HIP graph per step, replayed K times; kernels_ms from K eager steps, "
                  "each after a 512 MiB cache-evicting read",
    }
    result["config"] = dict(head.pop("config"), parallelism="single GPU")
    result.update(head)
    if not args.no_extra and args.workload == 3:
        # the other two headline shapes: long-MLA token-mode prefill and the decode batch
        extra = {}
        for n in (4, 5):
            torch.cuda.empty_cache()
            r, _, _ = run_workload(n, max(10, args.steps // 2), args.warmup, producers=False)
            extra[r["config"]["workload"]] = r
        result["extra_workloads"] = extra
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, block)
    print(json.dumps(result))


def cpu_baseline(wl, block: bool, min_seconds: float = 10.0, max_tokens: int = 4096) -> dict:
    """The CPU oracle (float64, numpy) on a bounded sample of the same workload:
    batches of randomly chosen query tokens go through quantize, indexer and
    attention until at least `min_seconds` of work is done.  `cores` is the
    number of host cores the process may run on (its CPU affinity), which is
    also the BLAS thread count; `parallelism` is what the oracle achieved
    (process CPU time / wall time), and `blas` names the BLAS library."""
    import workloads as W  # noqa: F401
    from oracle import attention as OA
    from oracle import indexer as OI
    from oracle import quantize as OQ

    rng = np.random.default_rng(0)
    T = wl.q_bf16.shape[0]
    order = rng.permutation(T)[:max_tokens]
    batch = 8 if block else 2
    flops, done = 0, 0
    wall0, cpu0 = time.perf_counter(), time.process_time()
    if block:
        iq8_all = OQ.quantize(wl.idx_q_bf16, OQ.BF16, wl.idx_q_scale)
        _, pos = OI.positions(wl.cu_seqlens_q, wl.seq_lens)
    while done < len(order) and time.perf_counter() - wall0 < min_seconds:
        toks = np.sort(order[done:done + batch])
        done += len(toks)
        q8 = OQ.quantize(wl.q_bf16[toks], OQ.BF16, wl.q_scale)
        full_q8 = np.zeros(wl.q_bf16.shape, np.uint8)
        full_q8[toks] = q8
        if block:
            ids = OI.indexer_topk(iq8_all, wl.idx_k8, wl.block_table, wl.cu_seqlens_q, wl.seq_lens,
                                  sm_scale=wl.idx_sm_scale, idx_q_scale=wl.idx_q_scale,
                                  idx_k_scale=wl.idx_k_scale, topk=wl.topk, tokens=toks)
            full_ids = np.full((ids.shape[0], T, wl.topk), -1, np.int32)
            full_ids[:, toks] = ids
            OA.sparse_attn_block(full_q8, wl.k_cache8, wl.v_cache8, full_ids, wl.block_table, wl.cu_seqlens_q,
                                 wl.seq_lens, sm_scale=wl.sm_scale, q_scale=wl.q_scale, k_scale=wl.k_scale,
                                 v_scale=wl.v_scale, tokens=toks)
            flops += block_attention_flops(ids, pos[toks], wl.q_bf16.shape[1], ids.shape[0], 128, 128)
        else:
            OA.sparse_attn_token(full_q8, wl.kv8, wl.indices, sm_scale=wl.sm_scale, d_v=wl.d_v,
                                 q_scale=wl.q_scale, k_scale=wl.k_scale, v_scale=wl.v_scale,
                                 attn_sink=wl.sink, tokens=toks)
            flops += int((wl.indices[toks] >= 0).sum()) * wl.q_bf16.shape[1] * 2 * (576 + wl.d_v)
    dt = time.perf_counter() - wall0
    achieved = (time.process_time() - cpu0) / dt
    blas = {}
    try:
        import threadpoolctl
        for info in threadpoolctl.threadpool_info():
            if info.get("user_api") == "blas":
                blas = {"library": info.get("internal_api"), "version": info.get("version"),
                        "threads": info.get("num_threads")}
                break
    except ImportError:
        pass
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": len(os.sched_getaffinity(0)),
            "parallelism": round(achieved, 2), "blas": blas, "kind": "oracle",
            "sample": f"{done} query tokens of {wl.name} (random, all heads) through quantize, indexer and "
                      f"attention (float64 numpy, {dt:.1f} s)"}


if __name__ == "__main__":
    main()
