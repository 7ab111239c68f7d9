"""ap_decode_attn captured in a HIP graph (needs an MI355X): the decode path enqueues
only kernels (no memset or copy nodes), so a serving loop may capture a step and replay
it.  Each replay, with eager work on the same device between replays, must reproduce
the eagerly computed output bit for bit."""
import pytest
import torch

from gpu_helpers import make_inputs, upload_decode
from rank_compressed_kv_ap_amd import workloads as wl

pytestmark = pytest.mark.gpu

SHAPES = {
    # rank 64, r_lo 16: the single-kernel decode
    "single_kernel": (wl.LLAVA.replace(cfg_id=131, batch=4, n_q_heads=8, n_kv_heads=8, head_dim=64,
                                       n_tokens=500, n_text=9, rank=64, r_lo=16, top_k=125, grid=None,
                                       inner_dim=256), 0),
    # explicit splits: selection, split-N flash-decode and combine
    "three_kernels": (wl.GQA.replace(cfg_id=132, batch=3, n_q_heads=8, n_kv_heads=2, head_dim=64,
                                     n_tokens=700, rank=48, r_lo=16, top_k=175, inner_dim=128), 3),
}


@pytest.mark.parametrize("name", list(SHAPES))
def test_decode_graph_replays_equal_eager(gpu_lib, name):
    w, splits = SHAPES[name]
    seqs = make_inputs(w, 2)
    cache, q, tk, tv = upload_decode(w, seqs, gpu_lib)
    kw = dict(r_lo=w.r_lo, top_k=w.top_k, scale=w.scale, text_k=tk, text_v=tv, splits=splits)
    ref = gpu_lib.decode(cache, q, **kw)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gpu_lib.decode(cache, q, out=out, **kw)
    torch.cuda.synchronize()
    other = torch.empty_like(q)
    for rep in range(3):
        out.fill_(float("nan"))
        gpu_lib.decode(cache, q * 0.5, out=other, **kw)   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}"
    del graph
    cache.free()
