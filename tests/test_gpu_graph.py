"""The fused encode and decode under HIP graph capture, and on two streams
at once.  The calls allocate nothing and enqueue only kernel launches, so a
serving loop can capture them once and replay.  Every replay is checked
against the eager result, with eager work and synchronizations between
replays, and the input changes between replays (the graph reads it afresh
each time)."""
import sys

import numpy as np
import pytest
import torch

import kv_cache_compression_kvc_amd as kvc
from kv_cache_compression_kvc_amd import inputs, presets

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("bk,bv,G", [(4, 4, 128), (2, 4, 64)])
def test_encode_decode_graph_replays(bk, bv, G):
    p = presets.preset("llama3_8b_4k").with_(name="graph", layers=3, tokens=301, kv_heads=8,
                                             bits_k=bk, bits_v=bv, group=G, seed=9)
    xs = [inputs.make_kv(p, device=DEV), inputs.make_kv(p.with_(seed=9, k_sigma=2.0), device=DEV)]
    refs = []
    for x in xs:
        b = kvc.encode(x, bk, bv, G, seed=p.seed)
        refs.append((b, kvc.decode(b, x.shape, p.dtype, bk, bv, G, seed=p.seed)))
    x_in = xs[0].clone()
    total, _ = kvc.encoded_size(p.layers, p.tokens, p.kv_heads, p.head_dim, bk, bv, G, p.dtype)
    blob = torch.zeros(total, dtype=torch.uint8, device=DEV)
    y = torch.zeros_like(x_in)
    # one eager call first: the library caches the launch shapes outside the capture
    kvc.encode(x_in, bk, bv, G, seed=p.seed, out=blob)
    kvc.decode(blob, x_in.shape, p.dtype, bk, bv, G, seed=p.seed, out=y)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    _say("graph: capture", bk, bv, G)
    with torch.cuda.graph(g, stream=side):
        kvc.encode(x_in, bk, bv, G, seed=p.seed, out=blob)
        kvc.decode(blob, x_in.shape, p.dtype, bk, bv, G, seed=p.seed, out=y)
    for r in range(6):
        k = r % 2
        x_in.copy_(xs[k])
        blob.fill_(0xA5)
        y.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say("  replay", r)
        assert torch.equal(blob, refs[k][0]), "replay %d: blob" % r
        assert torch.equal(y.view(torch.int16), refs[k][1].view(torch.int16)), "replay %d: decode" % r
        # eager work between replays
        z = kvc.decode(refs[1 - k][0], x_in.shape, p.dtype, bk, bv, G, seed=p.seed)
        torch.cuda.synchronize()
        assert torch.equal(z.view(torch.int16), refs[1 - k][1].view(torch.int16))
    del g


@pytest.mark.parametrize("pool_order", [False, True])
def test_paged_graph_replays(pool_order):
    p = presets.preset("qwen7b_paged").with_(name="graph-paged", layers=2, num_requests=5,
                                              len_min=1, len_max=200, seed=4)
    lens = inputs.request_lengths(p)
    table, nb = inputs.block_table(p, lens)
    offs, total = kvc.paged_layout(lens, p.layers, p.kv_heads, p.head_dim, p.bits_k, p.bits_v, p.group, p.dtype)
    bt, sl, of = (torch.from_numpy(a).to(DEV) for a in (table, lens, offs))
    order = None
    if pool_order:
        items = kvc.paged_order(table, lens, offs, p.block_size, nb)
        order = torch.from_numpy(items.view(np.uint8)).to(DEV)
    pools = [inputs.make_pool(p, nb, device=DEV), inputs.make_pool(p.with_(k_sigma=2.0), nb, device=DEV)]
    refs = []
    for pool in pools:
        b = kvc.encode_paged(pool, bt, sl, of, total, p.bits_k, p.bits_v, p.group, seed=p.seed)
        d = torch.full_like(pool, 3.0)
        kvc.decode_paged(b, d, bt, sl, of, p.bits_k, p.bits_v, p.group, seed=p.seed)
        refs.append((b, d))
    pool_in = pools[0].clone()
    blob = torch.zeros(total, dtype=torch.uint8, device=DEV)
    out = torch.full_like(pool_in, 3.0)
    kvc.encode_paged(pool_in, bt, sl, of, total, p.bits_k, p.bits_v, p.group, seed=p.seed, out=blob, order=order)
    kvc.decode_paged(blob, out, bt, sl, of, p.bits_k, p.bits_v, p.group, seed=p.seed, order=order)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    _say("graph: capture paged", "pool order" if pool_order else "request order")
    with torch.cuda.graph(g, stream=side):
        kvc.encode_paged(pool_in, bt, sl, of, total, p.bits_k, p.bits_v, p.group, seed=p.seed, out=blob, order=order)
        kvc.decode_paged(blob, out, bt, sl, of, p.bits_k, p.bits_v, p.group, seed=p.seed, order=order)
    for r in range(6):
        k = r % 2
        pool_in.copy_(pools[k])
        blob.fill_(0xA5)
        out.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say("  replay", r)
        assert torch.equal(blob, refs[k][0]), "replay %d: blob" % r
        assert torch.equal(out.view(torch.int16), refs[k][1].view(torch.int16)), "replay %d: decode" % r
    del g


def test_two_streams_at_once_equal_serial():
    """Encodes and decodes enqueued on two streams at the same time, on
    independent buffers, give the same bits as the same calls run one after
    the other: the kernels share no state, and the launch-shape cache is
    filled on the host under a lock."""
    shapes = [(4, 4, 128, 301), (2, 8, 64, 77), (8, 2, 32, 190)]
    cases = []
    for n, (bk, bv, G, T) in enumerate(shapes):
        p = presets.preset("llama3_8b_4k").with_(name="streams-%d" % n, layers=2, tokens=T, kv_heads=8,
                                                 bits_k=bk, bits_v=bv, group=G, seed=n)
        x = inputs.make_kv(p, device=DEV)
        b = kvc.encode(x, bk, bv, G, seed=n)
        cases.append((p, x, b, kvc.decode(b, x.shape, p.dtype, bk, bv, G, seed=n)))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rep in range(3):
        for k, (p, x, b, y) in enumerate(cases):
            s = streams[(k + rep) % 2]
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                ob = torch.empty_like(b)
                oy = torch.empty_like(y)
                kvc.encode(x, p.bits_k, p.bits_v, p.group, seed=p.seed, out=ob, stream=s)
                kvc.decode(ob, x.shape, p.dtype, p.bits_k, p.bits_v, p.group, seed=p.seed, out=oy, stream=s)
            outs.append((k, ob, oy))
    torch.cuda.synchronize()
    _say("two streams:", len(outs), "calls")
    for k, ob, oy in outs:
        assert torch.equal(ob, cases[k][2])
        assert torch.equal(oy.view(torch.int16), cases[k][3].view(torch.int16))
