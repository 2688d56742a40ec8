"""Graph capture: the prefill step (sep_mask_compact, then sep_attn_prefill),
the prefill backward, and the same prompt streamed into a cache in chunks
(sep_cache_reset, then per chunk sep_attn_prefill_chunk and
sep_cache_update), each captured once as a HIP graph and replayed, on the
8192-token Llama-3 layer workload. Their entry points allocate nothing and
issue no memset, so a caller (a serving loop) may capture them.

Every replay writes into outputs that eager work overwrote first, and must
equal the eager launches: bit for bit, except dk and dv, whose initial and
separator rows are summed with fp32 atomics in a varying order (relative
1e-5). The eager launches themselves are checked against the oracle at this
size in test_gpu_prefill.py (every head, row and log-sum-exp) and, on small
and sampled full-size cases, in test_gpu_prefill_backward.py.
"""
import math

import numpy as np
import pytest
import torch

from inputs import configs, gen
from kv_cache_compression_sep_amd import (chunk_workspace_bytes, sep_attn_prefill, sep_attn_prefill_backward,
                                          sep_attn_prefill_chunk, sep_cache_update, sep_mask_compact)

from .gpu_util import guarded_cache, guarded_empty, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def capture(fn):
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_cap):
        fn()
    torch.cuda.current_stream().wait_stream(s_cap)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s_cap):
        fn()
    torch.cuda.synchronize()
    return g


def replay_and_compare(g, outs, refs, exact, tag):
    for i in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else (255 if o.dtype == torch.uint8 else -1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (o, r) in enumerate(zip(outs, refs)):
            if exact[j]:
                assert torch.equal(o, r), f"{tag}: replay {i}, output {j} differs"
            else:
                assert torch.allclose(o, r, rtol=1e-5, atol=1e-6), f"{tag}: replay {i}, output {j} differs"
        print(f"[{tag}] replay {i} matches the eager launches", flush=True)


@pytest.fixture(scope="module")
def layer():
    cfg = configs.LLAMA3_LAYER_PREFILL
    x = gen.prefill_inputs(cfg)
    return dict(cfg=cfg, ids=to_dev(x["ids"]), q=to_dev(x["q"], "bf16"), k=to_dev(x["k"], "bf16"),
                v=to_dev(x["v"], "bf16"), sep=to_dev(np.asarray(cfg.sep_ids, np.int32)))


def outputs(t):
    """The step's outputs, guarded (the conftest hook checks the guards
    after the test)."""
    cfg = t["cfg"]
    B, Hq, S, D = cfg.B, cfg.Hq, cfg.S, cfg.D
    t["is_sep"] = guarded_empty((B, S), torch.uint8)
    t["rank"] = guarded_empty((B, S + 1), torch.int32)
    t["sep_pos"] = guarded_empty((B, S), torch.int32)
    t["count"] = guarded_empty((B,), torch.int32)
    t["out"] = guarded_empty((B, Hq, S, D), torch.bfloat16)
    t["lse"] = guarded_empty((B, Hq, S), torch.float32)


@pytest.mark.timeout(600)
def test_prefill_step_graph_replays_match_eager(layer):
    t = layer
    outputs(t)
    cfg = t["cfg"]
    scale = 1.0 / math.sqrt(cfg.D)

    def step():
        sep_mask_compact(t["ids"], t["sep"], is_sep=t["is_sep"], rank=t["rank"], sep_pos=t["sep_pos"],
                         count=t["count"])
        sep_attn_prefill(t["q"], t["k"], t["v"], t["is_sep"], t["rank"], t["sep_pos"], cfg.a, cfg.n, scale,
                         return_lse=True, out=t["out"], lse=t["lse"])

    step()
    torch.cuda.synchronize()
    outs = [t[n] for n in ("is_sep", "rank", "sep_pos", "count", "out", "lse")]
    refs = [o.clone() for o in outs]
    g = capture(step)
    replay_and_compare(g, outs, refs, [True] * len(outs), "prefill step")


@pytest.mark.timeout(600)
def test_prefill_backward_graph_replays_match_eager(layer):
    t = layer
    outputs(t)
    cfg = t["cfg"]
    B, Hq, Hkv, S, D = cfg.B, cfg.Hq, cfg.Hkv, cfg.S, cfg.D
    scale = 1.0 / math.sqrt(D)
    sep_mask_compact(t["ids"], t["sep"], is_sep=t["is_sep"], rank=t["rank"], sep_pos=t["sep_pos"], count=t["count"])
    sep_attn_prefill(t["q"], t["k"], t["v"], t["is_sep"], t["rank"], t["sep_pos"], cfg.a, cfg.n, scale,
                     return_lse=True, out=t["out"], lse=t["lse"])
    g_ = torch.Generator(device="cuda").manual_seed(1006)
    dout = torch.randn((B, Hq, S, D), device="cuda", generator=g_).to(torch.bfloat16)
    dq, dk, dv = (guarded_empty((B, Hq, S, D), torch.float32), guarded_empty((B, Hkv, S, D), torch.float32),
                  guarded_empty((B, Hkv, S, D), torch.float32))
    delta = guarded_empty((B, Hq, S), torch.float32)

    def call():
        sep_attn_prefill_backward(t["q"], t["k"], t["v"], t["out"], dout, t["lse"], t["is_sep"], t["rank"],
                                  t["sep_pos"], cfg.a, cfg.n, scale, dq=dq, dk=dk, dv=dv, delta=delta)

    call()
    torch.cuda.synchronize()
    outs = [delta, dq, dk, dv]
    refs = [o.clone() for o in outs]
    g = capture(call)
    replay_and_compare(g, outs, refs, [True, True, False, False], "prefill backward")


@pytest.mark.timeout(600)
def test_chunked_prompt_graph_replays_match_eager(layer):
    """The prompt in 4 chunks of 2048 into the streaming cache (4/64/64/256),
    window 256: every chunk's output and the whole cache (K/V rows, pos,
    tok, state) after a replay equal the eager calls'. Before each replay
    the outputs are poisoned, K/V zeroed and pos/tok/state set to garbage,
    so the replay itself must write them (its reset restores pos/tok/state)."""
    t = layer
    cfg = t["cfg"]
    sc = configs.STREAM_DECODE
    B, Hq, Hkv, S, D = cfg.B, cfg.Hq, cfg.Hkv, cfg.S, cfg.D
    C, n = 2048, cfg.n
    scale = 1.0 / math.sqrt(D)
    spans = [(c0, c0 + C) for c0 in range(0, S, C)]
    qc = [t["q"][:, :, c0:c1].contiguous() for c0, c1 in spans]
    kc = [t["k"][:, :, c0:c1].contiguous() for c0, c1 in spans]
    vc = [t["v"][:, :, c0:c1].contiguous() for c0, c1 in spans]
    ic = [t["ids"][:, c0:c1].contiguous() for c0, c1 in spans]
    cache = guarded_cache(B, Hkv, D, sc.a, sc.s, sc.p, sc.w)
    ws = guarded_empty((chunk_workspace_bytes(cache, C),), torch.uint8)
    outs = [guarded_empty((B, Hq, C, D), torch.bfloat16) for _ in spans]

    def prompt():
        cache.reset()
        for j in range(len(spans)):
            sep_attn_prefill_chunk(qc[j], kc[j], vc[j], ic[j], cache, t["sep"], n, scale, workspace=ws, out=outs[j])
            sep_cache_update(cache, kc[j], vc[j], ic[j], t["sep"])

    def scrub():
        cache.k.zero_()
        cache.v.zero_()
        for m in (cache.pos, cache.tok, cache.state):
            m.fill_(7)

    scrub()
    prompt()
    torch.cuda.synchronize()
    state = [cache.k, cache.v, cache.pos, cache.tok, cache.state]
    refs_o = [o.clone() for o in outs]
    refs_c = [m.clone() for m in state]
    g = capture(prompt)
    for i in range(REPLAYS):
        scrub()
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (o, r) in enumerate(zip(outs, refs_o)):
            assert torch.equal(o, r), f"chunked prompt: replay {i}, chunk {j} output differs"
        for name, m, r in zip(("k", "v", "pos", "tok", "state"), state, refs_c):
            assert torch.equal(m, r), f"chunked prompt: replay {i}, cache {name} differs"
        print(f"[chunked prompt] replay {i} matches the eager calls", flush=True)
