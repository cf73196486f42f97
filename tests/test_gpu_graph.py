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
