"""The chunked prefill captured in a HIP graph (the case the no-allocation
entry point is for: nothing may be allocated while a stream is captured).
kda_chunk_prefill_noalloc and kda_chunk_prefill with a caller workspace are
captured once each on a side stream and replayed three times, with other
eager work and synchronisations between the replays; every replay must
reproduce the eager call bit for bit.  The launches hold no memset nodes: the
chunk map clears the status word with a kernel.  A batch of 256 (sequence,
head) pairs covers the per-head scan the same way."""
import numpy as np
import pytest
import torch

import synth
from kda_cases import dev_inputs, say, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_55_amd as m

    return m


@pytest.mark.parametrize("noalloc,lengths", [
    (True, [700, 0, 333]), (False, [700, 0, 333]),          # 96 pairs: column-block scan
    (True, [100, 64, 0, 90, 1, 120, 77, 65]),               # 256 pairs: per-head scan
])
def test_prefill_graph_replays_match_eager(kda, noalloc, lengths):
    say(f"prefill captured in a graph, noalloc={noalloc}, lengths={lengths}")
    inp = synth.make_inputs(81, lengths, 32, 128, dtype="bf16", h0_std=0.02, chunk=64)
    d = dev_inputs(inp)
    N = len(inp.cu_seqlens) - 1
    o = torch.empty((inp.T, inp.H, inp.dk), dtype=torch.bfloat16, device="cuda")
    ht = torch.empty((N, inp.H, inp.dk, inp.dk), dtype=torch.float32, device="cuda")
    ws = None if noalloc else torch.empty(
        kda.prefill_workspace_bytes(inp.T, inp.H, inp.dk, N, 64), dtype=torch.uint8,
        device="cuda")

    def call():
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                          scale=inp.scale, chunk=64, out=o, ht=ht, workspace=ws,
                          noalloc=noalloc)

    call()  # eager; also takes the static buffer's address on this device before capture
    torch.cuda.synchronize()
    o_ref, s_ref = to_host64(o), to_host64(ht)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            call()
    torch.cuda.synchronize()
    for rep in range(3):
        o.fill_(7.0)
        ht.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host64(o), o_ref), f"o differs on replay {rep}"
        assert np.array_equal(to_host64(ht), s_ref), f"ht differs on replay {rep}"
        # eager work of the program between replays
        torch.mm(torch.ones(256, 256, device="cuda"), torch.ones(256, 256, device="cuda"))
    say("  three replays equal to the eager call bit for bit")
