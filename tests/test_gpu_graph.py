"""The insert + decode step captured as a HIP graph (torch.cuda.CUDAGraph on
the library's stream argument) and replayed: every replay must reproduce the
eager result bit for bit, with eager work and synchronisations between the
replays.  The library records no memset and allocates nothing, so its calls
are capture-safe."""
import numpy as np
import pytest

import workloads as wl

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_07_amd as mla
    print("[graph] insert + decode, B=4 q_len=2 H=128", flush=True)
    d = wl.make_inputs(4, 2, 128, [70, 1500, 300, 4097], permute=True, seed=51, spare_blocks=2)
    to = lambda a: (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
                    if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a)).cuda())
    cache0 = to(d["cache"])
    kv_a, rms_w, q, kv_b = to(d["kv_a"]), to(d["rms_w"]), to(d["q"]), to(d["kv_b"])
    bt, sl = to(d["block_table"]), to(d["seq_lens"])
    max_len = int(d["seq_lens"].max())
    eps = float(np.float32(wl.EPS))
    ws = torch.empty(mla.decode_workspace_bytes(128, 4, 2, max_len), dtype=torch.uint8, device="cuda")

    # eager reference
    cache_e = cache0.clone()
    mla.cache_insert(kv_a, rms_w, bt, sl, cache_e, eps=eps, heads=128)
    ref = mla.decode(q, kv_b, cache_e, bt, sl, max_len, workspace=ws).clone()
    torch.cuda.synchronize()

    cache_g = cache0.clone()
    out_g = torch.empty_like(ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mla.cache_insert(kv_a, rms_w, bt, sl, cache_g, eps=eps, heads=128)
        mla.decode(q, kv_b, cache_g, bt, sl, max_len, out=out_g, workspace=ws)
    torch.cuda.synchronize()
    for r in range(4):
        out_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), f"replay {r} differs from the eager result"
        # bit patterns: unwritten slots hold NaN sentinels, which never compare equal
        assert torch.equal(cache_g.view(torch.int16), cache_e.view(torch.int16)), \
            f"replay {r}: cache differs"
        # eager work on the same stream between replays
        other = mla.decode(q, kv_b, cache_e, bt, sl, max_len)
        torch.cuda.synchronize()
        assert torch.equal(other, ref)


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_graph_replay_of_fused_step(fp8):
    """mla_decode_step (the benchmark's step) captured and replayed: each
    replay equals the eager step bit for bit (output and cache), with eager
    work between replays."""
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_07_amd as mla
    from oracle import fp8 as ofp8
    print(f"[graph] fused step fp8={fp8}, B=3 q_len=2 H=128", flush=True)
    d = wl.make_inputs(3, 2, 128, [2, 900, 2049], permute=True, seed=52, spare_blocks=1)
    to = lambda a: (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
                    if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a)).cuda())
    c = d["cache"]
    if fp8:
        v = (c.astype(np.uint32) << 16).view(np.float32)
        c = ofp8.quantize_cache(np.where(np.isfinite(v), c, np.uint16(0)).astype(np.uint16))
    cache0 = to(c)
    kv_a, rms_w, q, kv_b = to(d["kv_a"]), to(d["rms_w"]), to(d["q"]), to(d["kv_b"])
    bt, sl = to(d["block_table"]), to(d["seq_lens"])
    max_len = int(d["seq_lens"].max())
    eps = float(np.float32(wl.EPS))
    ws = torch.empty(mla.decode_workspace_bytes(128, 3, 2, max_len), dtype=torch.uint8, device="cuda")
    bits = (lambda t: t) if fp8 else (lambda t: t.view(torch.int16))

    cache_e = cache0.clone()
    ref = mla.decode_step(q, kv_a, rms_w, kv_b, cache_e, bt, sl, max_len, eps=eps, workspace=ws,
                          fp8=fp8).clone()
    torch.cuda.synchronize()
    cache_g = cache0.clone()
    out_g = torch.empty_like(ref)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mla.decode_step(q, kv_a, rms_w, kv_b, cache_g, bt, sl, max_len, eps=eps, out=out_g,
                        workspace=ws, fp8=fp8)
    torch.cuda.synchronize()
    for r in range(4):
        out_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), ref.view(torch.int16)), \
            f"replay {r} differs from the eager step"
        assert torch.equal(bits(cache_g), bits(cache_e)), f"replay {r}: cache differs"
        other = mla.decode_step(q, kv_a, rms_w, kv_b, cache_e, bt, sl, max_len, eps=eps, fp8=fp8)
        torch.cuda.synchronize()
        assert torch.equal(other.view(torch.int16), ref.view(torch.int16))
