"""Graph capture: the prefill step (sep_mask_compact, then sep_attn_prefill)
and the prefill backward, each captured once as a HIP graph and replayed, on
the 8192-token Llama-3 layer workload. Their entry points allocate nothing
and issue no memset, so a caller (a serving loop) may capture them.

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
from kv_cache_compression_sep_amd import sep_attn_prefill, sep_attn_prefill_backward, sep_mask_compact

from .gpu_util import guarded_empty, to_dev

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
