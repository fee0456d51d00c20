"""The decode calls captured in a HIP graph (torch.cuda.CUDAGraph on ROCm):
every replay, with eager calls and synchronisations between replays, gives
the eager result bit for bit — the whole-row path (its per-call partition), the
per-head path with splits (its arrival counters, left at zero by every call),
the prefill kernel and the MLA decode.  Workspaces and outputs are allocated before capture; the
calls enqueue kernels only.  Every test prints its case first."""
from __future__ import annotations

import pytest
import torch

from fp8_paged_kv_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fp8_paged_kv_amd import binding
    binding.lib()
    return binding


def _check_replays(run_eager, run_into, outs, tag):
    """run_eager(stream) -> list of reference outputs; run_into(stream) enqueues the calls
    writing `outs`.  Capture once, replay four times with eager work in between."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ref = [r.clone() for r in run_eager(s)]
        run_into(s)                                   # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        run_into(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"{tag}: replay {rep}, output {i} differs from the eager call"
        with torch.cuda.stream(s):
            run_eager(s)                              # eager calls between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("num_splits", [0, 3])
def test_gqa_decode_graph_replays(B, num_splits):
    cfg = synth.GqaConfig(name="graph", B=3, s1=1, nq=16, nkv=2, seq_lens=(300, 1100, 2500), s2_tile=256,
                          num_blocks=40, max_blocks_per_seq=20, seed=31)
    sets = [synth.make_gqa_inputs(cfg, device="cuda", seed=31 + i) for i in range(2)]
    print(f"[gpu] graph replays, gqa decode, splits={num_splits}", flush=True)
    need, _ = B.workspace_size(cfg.B, cfg.s1, cfg.nq, cfg.nkv, cfg.D, cfg.block_size, cfg.max_blocks_per_seq,
                               cfg.s2_tile, num_splits)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    shape = (cfg.B * cfg.s1, cfg.nq, cfg.D)
    outs = [torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in sets]
    eager_out = [torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in sets]

    def run_eager(st):
        for inp, o in zip(sets, eager_out):
            B.decode_inputs(inp, num_splits=num_splits, out=o, workspace=ws, stream=st)
        return eager_out

    def run_into(st):
        for inp, o in zip(sets, outs):
            B.decode_inputs(inp, num_splits=num_splits, out=o, workspace=ws, stream=st)

    _check_replays(run_eager, run_into, outs, f"gqa splits={num_splits}")


def test_prefill_kernel_graph_replays(B):
    """A causal prefill chunk on the prefill kernel (1024 query rows per KV head, 64
    workgroups): its in-kernel batch ordering and staging replay bit for bit."""
    cfg = synth.GqaConfig(name="graph-prefill", B=8, s1=64, nq=16, nkv=1,
                          seq_lens=(70, 300, 1100, 2500, 64, 900, 1700, 0), s2_tile=256,
                          num_blocks=8 * 21, max_blocks_per_seq=21, seed=37)
    sets = [dict(synth.make_gqa_inputs(cfg, device="cuda", seed=37 + i), causal=True) for i in range(2)]
    print("[gpu] graph replays, prefill kernel, B=8 s1=64 nq=16 nkv=1 causal", flush=True)
    need, _ = B.workspace_size(cfg.B, cfg.s1, cfg.nq, cfg.nkv, cfg.D, cfg.block_size, cfg.max_blocks_per_seq,
                               cfg.s2_tile, 0)
    ws = torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda")
    shape = (cfg.B * cfg.s1, cfg.nq, cfg.D)
    outs = [torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in sets]
    eager_out = [torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in sets]

    def run_eager(st):
        for inp, o in zip(sets, eager_out):
            B.decode_inputs(inp, num_splits=0, out=o, workspace=ws, stream=st)
        return eager_out

    def run_into(st):
        for inp, o in zip(sets, outs):
            B.decode_inputs(inp, num_splits=0, out=o, workspace=ws, stream=st)

    _check_replays(run_eager, run_into, outs, "prefill kernel")


@pytest.mark.parametrize("nq,s2_tile", [(32, 256), (64, 512)])
def test_mla_decode_graph_replays(B, nq, s2_tile):
    """Captured MLA calls replay the eager result (32- and 64-head query groups)."""
    cfg = synth.MlaConfig("graph-mla", B=2, s1=2, nq=nq, topk=1024, seq_range=(600, 1500), num_blocks=32,
                          max_blocks_per_seq=16, s2_tile=s2_tile, seed=33)
    inp = synth.make_mla_inputs(cfg, device="cuda")
    print(f"[gpu] graph replays, mla decode nq={nq} s2_tile={s2_tile}", flush=True)
    ws = torch.zeros(max(B.mla_workspace_size(cfg.B, cfg.s1, cfg.nq, cfg.topk, cfg.s2_tile), 1),
                     dtype=torch.uint8, device="cuda")
    shape = (cfg.B * cfg.s1 * cfg.nq, 512)
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    eager_out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")

    def run_eager(st):
        B.mla_decode_inputs(inp, out=eager_out, workspace=ws, stream=st)
        return [eager_out]

    def run_into(st):
        B.mla_decode_inputs(inp, out=out, workspace=ws, stream=st)

    _check_replays(run_eager, run_into, [out], "mla")
