"""A serving decode step captured in a HIP graph: append one token per sequence (quantizing
the staging tiles that fill) and decode over the cache, replayed step after step. The entry
points allocate nothing, set no memory with memset and never synchronize, so the whole step
captures. Every replay is checked against the same step run eagerly on a copy of the cache,
with eager work and synchronizations between the replays."""
import numpy as np
import pytest
import torch

from tests import kvarn_testlib as T
from tests.test_gpu_parity import _build_cache

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def K():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need an MI355X; torch.cuda.is_available() is False")
    from kv_cache_quantization_tile_amd import kvarn
    return kvarn


def test_decode_step_graph_replays(K):
    lens = [300, 1000, 125]            # the last sequence's staging tile fills at step 3
    hkv, G, steps = 2, 8, 6
    params = K.params_from_dtype("kvarn_k4v2_g128", 8)
    kp, vp, bt, kt, vt, sl, _ = _build_cache(K, params, lens, hkv, seed=300, spare=1,
                                             width=max(L // 128 for L in lens) + 3)
    # the page that each sequence's staging tile fills next
    bt_h = bt.cpu().numpy()
    free = sorted(set(range(kp.shape[0])) - set(int(p) for p in bt_h.ravel() if p >= 0))
    for b, L in enumerate(lens):
        bt_h[b, L // 128] = free[b]
    bt = torch.from_numpy(bt_h).cuda()
    B, hq = len(lens), hkv * G
    mx = max(lens) + steps
    gen = torch.Generator().manual_seed(301)
    news = [(torch.randn((B, hkv, 128), generator=gen).to(torch.float16).cuda(),
             torch.randn((B, hkv, 128), generator=gen).to(torch.float16).cuda(),
             torch.randn((B, hq, 128), generator=gen).to(torch.float16).cuda())
            for _ in range(steps)]
    # eager reference on a copy of the cache
    ref = [t.clone() for t in (kp, vp, kt, vt)]
    sl_ref = sl.clone()
    want = []
    for kn, vn, q in news:
        K.append_tokens(params, kn, vn, sl_ref, ref[2], ref[3], bt, ref[0], ref[1])
        sl_ref += 1
        want.append(K.decode_attention(params, q, ref[0], ref[1], bt, sl_ref, mx, ref[2], ref[3]))
    torch.cuda.synchronize()
    # the captured step: static inputs, lengths advanced in place by the graph itself
    kn_s, vn_s, q_s = (t.clone() for t in news[0])
    sl_g = sl.clone()
    ws = K.new_workspace(params, B, hq, hkv, mx)
    out = torch.empty((B, hq, 128), dtype=torch.float16, device="cuda")
    one = torch.ones_like(sl_g)

    def step():
        K.append_tokens(params, kn_s, vn_s, sl_g, kt, vt, bt, kp, vp)
        sl_g.add_(one)
        K.decode_attention(params, q_s, kp, vp, bt, sl_g, mx, kt, vt, workspace=ws, out=out)

    # warm up the side stream the capture uses (lengths restored afterwards)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kp0, vp0, kt0, vt0, sl0 = (t.clone() for t in (kp, vp, kt, vt, sl_g))
        step()
        for dst, src in ((kp, kp0), (vp, vp0), (kt, kt0), (vt, vt0), (sl_g, sl0)):
            dst.copy_(src)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for i, (kn, vn, q) in enumerate(news):
        kn_s.copy_(kn)
        vn_s.copy_(vn)
        q_s.copy_(q)
        graph.replay()
        torch.cuda.synchronize()
        scratch = torch.randn(1 << 20, device="cuda").sum()    # eager work between replays
        assert torch.equal(out, want[i]), f"replay {i}"
        del scratch
    assert torch.equal(kp, ref[0]) and torch.equal(vp, ref[1])
    assert torch.equal(sl_g, sl_ref)
    err = T.check_decode(news[-1][2], out, kp, vp, bt, sl_g, G, k_tail=kt, v_tail=vt)
    print(f"graph decode step: {steps} replays equal eager, last step max rel err {err:.2e}", flush=True)
