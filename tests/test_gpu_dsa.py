"""GPU parity of the sparse decode (mla_dsa_select, mla_dsa_decode).

Source: "DeepSeek-V3.2-Exp unboxing", 初步研读: an FP8 index kernel scores
the cached tokens (per-head weights on the queries, a per-token scale on the
keys) and the attention then runs over the top-k tokens only.

Checks, on seeded inputs (FP8 codes uniform over the finite E4M3 codes,
weights N(0, 1), key scales U[0.25, 1)):
* index scores: the GPU's fp32 scores are within the fp32 accumulation bound
  of the float64 oracle (|err| <= 256 * 2^-24 * sum of |terms|);
* top-k, exact: the GPU's kept positions equal the oracle's top-k applied to
  the GPU's own scores (the decision taken in the kernel's precision: same
  numbers, same tie rule), with the count min(top_k, len) and -1 padding;
* top-k, valid: against the oracle's float64 scores, no kept position scores
  below, and no dropped position above, the k-th largest score by more than
  the score bound;
* ties: on inputs whose scores are small exact sums (many equal values), the
  GPU's selection equals the oracle's selection on the oracle's scores;
* decode over the kept positions: within the decode bound (max-abs 2e-2,
  relative RMS 5e-3) of the float64 oracle decode over the same positions;
  with top_k >= every length the sparse decode is bit-identical to
  mla_decode (same positions, same order, same split plan).
"""
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import cache_insert as oracle_insert
from oracle import dsa
from oracle.fp8 import e4m3_decode

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
REL_RMS = 5e-3
SCORE_ULPS = 256.0 * 2.0 ** -24


def _torch():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a, torch):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def filled(d):
    """The workload's cache with the new token of every sequence written (the
    oracle's insert): every position below seq_lens is a real entry."""
    return oracle_insert(d["cache"], d["kv_a"], d["rms_w"], d["block_table"], d["seq_lens"],
                         d["q_len"], float(np.float32(wl.EPS)), wl.ROPE_BASE, wl.LATENT)


def score_bound(ix, d, b):
    """fp32 accumulation bound of sequence b's scores: 256 units of 2^-24
    times the sum of the absolute terms (weighted query sum, 128 products)."""
    n = int(d["seq_lens"][b])
    t = np.arange(n)
    blk = d["block_table"][b, t // wl.PAGE].astype(np.int64)
    k = np.abs(e4m3_decode(ix["index_k"][blk, t % wl.PAGE]))
    ks = np.asarray(ix["index_k_scale"], dtype=np.float64)[blk, t % wl.PAGE]
    q = np.abs(e4m3_decode(ix["index_q"][b]))
    w = np.abs(np.asarray(ix["index_w"], dtype=np.float64)[b])
    return SCORE_ULPS * ((w @ q) @ k.T) * ks + 1e-30


def run_select(d, ix, top_k, torch):
    bt = dev(d["block_table"], torch)
    sl = dev(d["seq_lens"], torch)
    from mla_latent_kv_07_amd import dsa_select
    scores, idx, counts = dsa_select(dev(ix["index_q"], torch), dev(ix["index_w"], torch),
                                     dev(ix["index_k"], torch), dev(ix["index_k_scale"], torch),
                                     bt, sl, int(d["seq_lens"].max()), top_k)
    torch.cuda.synchronize()
    return scores.cpu().numpy(), idx.cpu().numpy(), counts.cpu().numpy()


def check_selection(d, ix, top_k, scores, idx, counts, seqs):
    for b in seqs:
        n = int(d["seq_lens"][b])
        kk = min(top_k, n)
        assert counts[b] == kk
        assert np.all(idx[b, kk:] == -1)
        got = idx[b, :kk]
        # exact: the oracle's rule on the GPU's own numbers
        mine = dsa.topk_positions(scores[b, :n].astype(np.float64), top_k)
        assert np.array_equal(got, mine), f"sequence {b}: selection differs from the tie rule"
        # scores and validity against the float64 oracle
        ref = dsa.index_scores(ix["index_q"], ix["index_w"], ix["index_k"], ix["index_k_scale"],
                               d["block_table"], n, b)
        bound = score_bound(ix, d, b)
        err = np.abs(scores[b, :n] - ref)
        assert np.all(err <= bound), f"sequence {b}: score error {float((err / bound).max()):.2f} x bound"
        if kk < n:
            thr = np.sort(ref)[::-1][kk - 1]
            keep = np.zeros(n, dtype=bool)
            keep[got] = True
            assert np.all(ref[keep] >= thr - 2 * bound[keep])
            assert np.all(ref[~keep] <= thr + 2 * bound[~keep])


def run_decode(d, cache, ix, top_k, torch, hint=0):
    from mla_latent_kv_07_amd import dsa_decode
    idx = torch.empty((d["batch"], top_k), dtype=torch.int32, device="cuda")
    out = dsa_decode(dev(d["q"], torch), dev(d["kv_b"], torch), dev(cache, torch),
                     dev(d["block_table"], torch), dev(d["seq_lens"], torch),
                     int(d["seq_lens"].max()), dev(ix["index_q"], torch),
                     dev(ix["index_w"], torch), dev(ix["index_k"], torch),
                     dev(ix["index_k_scale"], torch), top_k, softmax_scale=d["softmax_scale"],
                     indices_out=idx, num_splits_hint=hint)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), idx.cpu().numpy()


def check_decode(d, cache, got, idx, top_k, seqs):
    for b in seqs:
        kk = min(top_k, int(d["seq_lens"][b]))
        sub = {k: d[k][b:b + 1] for k in ("q", "block_table", "seq_lens")}
        ref = dsa.decode_sparse(sub["q"], d["kv_b"], cache, sub["block_table"], sub["seq_lens"],
                                [idx[b, :kk]], softmax_scale=d["softmax_scale"])[0]
        e = got[b] - ref
        mx = float(np.abs(e).max())
        rr = float(np.sqrt(np.mean(e * e)) / np.sqrt(np.mean(ref * ref)))
        assert mx <= MAX_ABS and rr <= REL_RMS, f"sequence {b}: max-abs {mx:.3g} rel-rms {rr:.3g}"


SMALL = [
    # (name, batch, heads, lens, top_k, index_heads)
    ("ragged_k64", 4, 16, [1, 70, 300, 64], 64, 8),
    ("multi_page_k200", 3, 32, [2000, 257, 1500], 200, 64),
    ("keep_all", 3, 16, [5, 130, 190], 256, 4),
    ("k1", 2, 16, [77, 1], 1, 16),
    # longer than the 16384 positions top-k holds in registers: the re-read path
    ("long_reread", 2, 16, [20000, 300], 3000, 8),
    # 128 heads: the kept rows read in place (slot list) ...
    ("h128_in_place", 3, 128, [2500, 40, 700], 1000, 16),
    # ... and gathered when a sequence keeps more than 4096 positions
    ("h128_gather_k4200", 2, 128, [4500, 300], 4200, 8),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_select_small(case):
    torch = _torch()
    name, batch, heads, lens, top_k, hi = case
    say(f"dsa select {name}")
    d = wl.make_inputs(batch, 1, heads, lens, permute=True, seed=71)
    ix = wl.make_index_inputs(d, index_heads=hi, seed=72)
    scores, idx, counts = run_select(d, ix, top_k, torch)
    check_selection(d, ix, top_k, scores, idx, counts, range(batch))


def test_select_ties_exact():
    """Scores that are small exact sums: the query is 1.0 in dimension 0 of
    every head, weights 1 and 0.5, keys drawn from {0.5, 1, 2, 4, -1} in
    dimension 0 and 0 elsewhere, scale 1 or 0.5: every score is exact in fp32
    and float64, with many equal values, so the GPU's selection must equal the
    oracle's on the oracle's scores."""
    torch = _torch()
    say("dsa select ties")
    d = wl.make_inputs(3, 1, 16, [640, 333, 1000], permute=True, seed=73)
    rng = np.random.default_rng(74)
    nb = d["cache"].shape[0]
    q = np.zeros((3, 4, 128), dtype=np.uint8)
    q[:, :, 0] = 0x38                                   # 1.0
    w = np.tile(np.array([1.0, 0.5, 1.0, 0.5], dtype=np.float32), (3, 1))
    k = np.zeros((nb, wl.PAGE, 128), dtype=np.uint8)
    k[:, :, 0] = rng.choice(np.array([0x30, 0x38, 0x40, 0x48, 0xB8], dtype=np.uint8),
                            size=(nb, wl.PAGE))
    ks = rng.choice(np.array([1.0, 0.5], dtype=np.float32), size=(nb, wl.PAGE))
    ks[0, :5] = 0.0                                     # a few exact zeros
    ix = dict(index_q=q, index_w=w, index_k=k, index_k_scale=ks.astype(np.float32))
    for top_k in (1, 37, 300, 700):
        scores, idx, counts = run_select(d, ix, top_k, torch)
        for b in range(3):
            n = int(d["seq_lens"][b])
            ref = dsa.index_scores(q, w, k, ks, d["block_table"], n, b)
            assert np.array_equal(scores[b, :n].astype(np.float64), ref)
            kk = min(top_k, n)
            assert np.array_equal(idx[b, :kk], dsa.topk_positions(ref, top_k))
            assert np.all(idx[b, kk:] == -1)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_dsa_decode_small(case):
    torch = _torch()
    name, batch, heads, lens, top_k, hi = case
    say(f"dsa decode {name}")
    d = wl.make_inputs(batch, 1, heads, lens, permute=True, seed=75)
    ix = wl.make_index_inputs(d, index_heads=hi, seed=76)
    cache = filled(d)
    got, idx = run_decode(d, cache, ix, top_k, torch)
    scores, idx2, counts = run_select(d, ix, top_k, torch)
    assert np.array_equal(idx, idx2)
    check_selection(d, ix, top_k, scores, idx, counts, range(batch))
    check_decode(d, cache, got, idx, top_k, range(batch))


def test_dsa_keep_all_equals_dense_decode():
    torch = _torch()
    say("dsa keep-all vs dense decode")
    from mla_latent_kv_07_amd import decode
    d = wl.make_inputs(5, 1, 128, [1, 64, 65, 1000, 3000], permute=True, seed=77)
    ix = wl.make_index_inputs(d, index_heads=64, seed=78)
    cache = filled(d)
    got, idx = run_decode(d, cache, ix, 4096, torch)
    dense = decode(dev(d["q"], torch), dev(d["kv_b"], torch), dev(cache, torch),
                   dev(d["block_table"], torch), dev(d["seq_lens"], torch),
                   int(d["seq_lens"].max()), softmax_scale=d["softmax_scale"])
    torch.cuda.synchronize()
    assert np.array_equal(got, dense.float().cpu().numpy())
    for b in range(5):
        n = int(d["seq_lens"][b])
        assert np.array_equal(idx[b, :n], np.arange(n))


def test_dsa_v3_b64_l8192_k2048_sampled():
    """The full-size sparse workload (64 sequences of 8192 cached tokens, 128
    heads, 64 index heads, top-2048) in the benchmark's launch configuration
    (kept rows read in place); every sequence's selection and every output
    element against the oracle."""
    torch = _torch()
    say("dsa v3_b64_l8192 top-2048")
    d = wl.make_workload("v3_b64_l8192")
    ix = wl.make_index_inputs(d, index_heads=64, seed=1)
    cache = filled(d)
    got, idx = run_decode(d, cache, ix, 2048, torch)
    scores, idx2, counts = run_select(d, ix, 2048, torch)
    assert np.array_equal(idx, idx2)
    check_selection(d, ix, 2048, scores, idx, counts, range(d["batch"]))
    check_decode(d, cache, got, idx, 2048, range(d["batch"]))
    assert np.all(np.isfinite(got))


def test_dsa_rejects_bad_arguments():
    torch = _torch()
    from mla_latent_kv_07_amd import MLAError, dsa_decode
    d = wl.make_inputs(2, 1, 16, [100, 50], seed=79)
    ix = wl.make_index_inputs(d, index_heads=8, seed=80)
    args = [dev(d["q"], torch), dev(d["kv_b"], torch), dev(filled(d), torch),
            dev(d["block_table"], torch), dev(d["seq_lens"], torch), 100,
            dev(ix["index_q"], torch), dev(ix["index_w"], torch), dev(ix["index_k"], torch),
            dev(ix["index_k_scale"], torch)]
    for bad_k in (0, (1 << 16) + 1):
        with pytest.raises(MLAError):
            dsa_decode(*args, bad_k)
    small_ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(MLAError):
        dsa_decode(*args, 64, workspace=small_ws)


def test_dsa_decode_fp8_cache():
    """mla_dsa_decode_fp8: the same selection (it does not depend on the latent
    cache), the decode over the kept FP8 rows within the decode bound of the
    oracle on the dequantised entries (exact in bf16), and, keeping every
    position, bit-identical to mla_decode_fp8."""
    torch = _torch()
    from oracle import fp8 as ofp8
    from mla_latent_kv_07_amd import decode, dsa_decode
    say("dsa decode fp8 cache")
    d = wl.make_inputs(3, 1, 128, [2000, 300, 4100], permute=True, seed=81)
    ix = wl.make_index_inputs(d, index_heads=64, seed=82)
    cache = filled(d)
    v = (cache.astype(np.uint32) << 16).view(np.float32)
    c8 = ofp8.quantize_cache(np.where(np.isfinite(v), cache, np.uint16(0)).astype(np.uint16))
    deq = ofp8.f64_to_bf16_bits(ofp8.dequantize_cache(c8))
    args = (dev(d["q"], torch), dev(d["kv_b"], torch), dev(c8, torch),
            dev(d["block_table"], torch), dev(d["seq_lens"], torch), int(d["seq_lens"].max()),
            dev(ix["index_q"], torch), dev(ix["index_w"], torch), dev(ix["index_k"], torch),
            dev(ix["index_k_scale"], torch))
    for top_k in (256, 1000):
        idx_t = torch.empty((3, top_k), dtype=torch.int32, device="cuda")
        out = dsa_decode(*args, top_k, softmax_scale=d["softmax_scale"], indices_out=idx_t,
                         fp8=True)
        torch.cuda.synchronize()
        got, idx = out.float().cpu().numpy(), idx_t.cpu().numpy()
        _, idx2, _ = run_select(d, ix, top_k, torch)
        assert np.array_equal(idx, idx2)
        check_decode(d, deq, got, idx, top_k, range(3))
    out = dsa_decode(*args, 8192, softmax_scale=d["softmax_scale"], fp8=True)
    dense = decode(args[0], args[1], args[2], args[3], args[4], args[5],
                   softmax_scale=d["softmax_scale"], fp8=True)
    torch.cuda.synchronize()
    assert torch.equal(out, dense)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_dsa_graph_replay_matches_eager(fp8):
    """The sparse step (insert of the new token, then mla_dsa_decode) captured
    as a HIP graph and replayed, as the benchmark runs it: every replay equals
    the eager result bit for bit, with eager work between replays."""
    torch = _torch()
    import mla_latent_kv_07_amd as mla
    from oracle import fp8 as ofp8
    say(f"dsa graph replay fp8={fp8}")
    d = wl.make_inputs(4, 1, 128, [3000, 700, 64, 5000], permute=True, seed=83)
    ix = wl.make_index_inputs(d, index_heads=64, seed=84)
    cache0 = d["cache"]
    if fp8:
        v = (cache0.astype(np.uint32) << 16).view(np.float32)
        cache0 = ofp8.quantize_cache(np.where(np.isfinite(v), cache0, np.uint16(0)).astype(np.uint16))
    kv_a, rms_w, q, kv_b = (dev(d[k], torch) for k in ("kv_a", "rms_w", "q", "kv_b"))
    bt, sl = dev(d["block_table"], torch), dev(d["seq_lens"], torch)
    iq, iw, ik, iks = (dev(ix[k], torch) for k in ("index_q", "index_w", "index_k",
                                                   "index_k_scale"))
    max_len, top_k = int(d["seq_lens"].max()), 1024
    eps = float(np.float32(wl.EPS))
    ws = torch.empty(mla.dsa_workspace_bytes(128, 4, max_len, top_k), dtype=torch.uint8,
                     device="cuda")

    def step(cache, out):
        mla.cache_insert(kv_a, rms_w, bt, sl, cache, eps=eps, heads=128, fp8=fp8)
        return mla.dsa_decode(q, kv_b, cache, bt, sl, max_len, iq, iw, ik, iks, top_k, out=out,
                              workspace=ws, fp8=fp8)

    cache_e = dev(cache0, torch)
    ref = step(cache_e, None).clone()
    torch.cuda.synchronize()
    cache_g = dev(cache0, torch)
    out_g = torch.empty_like(ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(cache_g, out_g)
    torch.cuda.synchronize()
    for r in range(3):
        out_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), f"replay {r} differs from the eager result"
        other = step(cache_e, None)
        torch.cuda.synchronize()
        assert torch.equal(other, ref)


@pytest.mark.parametrize("hint", [1, 3, 8])
def test_dsa_decode_split_hint(hint):
    """The sparse decode with an explicit split count per sequence (the
    caller's num_splits_hint instead of the planner's choice): the same
    selection, the decode within the bound of the oracle."""
    torch = _torch()
    say(f"dsa decode hint={hint}")
    d = wl.make_inputs(3, 1, 128, [3000, 200, 5000], permute=True, seed=85)
    ix = wl.make_index_inputs(d, index_heads=64, seed=86)
    cache = filled(d)
    got, idx = run_decode(d, cache, ix, 1500, torch, hint=hint)
    _, idx2, _ = run_select(d, ix, 1500, torch)
    assert np.array_equal(idx, idx2)
    check_decode(d, cache, got, idx, 1500, range(3))


def test_dsa_in_place_full_slot_list():
    """Kept rows read in place with one work item per sequence of 4096 kept
    positions (num_splits_hint 1): the largest slot list the decode stages
    (64 pages); the decode within the bound of the oracle."""
    torch = _torch()
    say("dsa in place, 4096 kept positions in one item")
    d = wl.make_inputs(2, 1, 128, [5000, 4100], permute=True, seed=87)
    ix = wl.make_index_inputs(d, index_heads=16, seed=88)
    cache = filled(d)
    got, idx = run_decode(d, cache, ix, 4096, torch, hint=1)
    check_decode(d, cache, got, idx, 4096, range(2))
