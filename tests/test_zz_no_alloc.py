"""statekv_prefill_frame_static (the frame step whose working buffers live in
the library's static device scratch, for callers that cannot allocate)
against statekv_prefill_frame on twin states, through the C ABI (needs an
MI355X).

Two workloads of different sizes alternate on the shared static scratch, so
every call follows one with a larger (or smaller) input that left its own
contents behind: outputs, compressed states, detailed caches and scores must
equal those of the allocating entry point bit for bit.
"""
import ctypes

import numpy as np
import pytest
import torch

import kv_cache_compression_statekv_amd as skv
from kv_cache_compression_statekv_amd.workload import CONFIGS, FrameStream, StreamConfig
from gpu_helpers import make_state, to_device

pytestmark = pytest.mark.gpu

SMALL = StreamConfig(name="noalloc_small", config_id=111, dtype="bf16", n_q_heads=8,
                     n_kv_heads=2, head_dim=64, tokens_per_frame=200, budget=700, n_frames=6,
                     n_layers=1, rope_base=1e6, alpha=1.0, n_sinks=4)


def _frame(st, x, n, out, static: bool):
    lib = skv.load_library()
    fn = lib.statekv_prefill_frame_static if static else lib.statekv_prefill_frame
    rc = fn(st._h, x[0].data_ptr(), x[1].data_ptr(), x[2].data_ptr(), n, out.data_ptr())
    assert rc == skv.STATEKV_OK, skv.error_string(rc)


def _state_bits(st):
    k, v, pos = st.compressed_view()
    dk, dv = st.detailed_view()
    sc = st.scores()
    return [k, v, pos, dk, dv] + ([sc["scores"], sc["keep_flag"]] if sc else [])


# Top-B with the scores kept for every frame, and the recency window, whose
# decision and moves run in the launch after pass 1.
@pytest.mark.parametrize("flags", [skv.FLAG_ALWAYS_SCORE, skv.FLAG_RECENT_WINDOW],
                         ids=["topb_scores", "recent_window"])
def test_static_scratch_matches_allocating_entry_point(flags):
    # The larger workload first: the InternVL3-1B-like layer (about 9 MB of
    # working buffers), then the smaller ragged one (about 1.5 MB), alternating.
    big = CONFIGS["ivl3_1b"].replace(n_frames=20)
    work = []
    for wl in (big, SMALL):
        fs = FrameStream(wl)
        frames = [[to_device(a, wl.dtype) for a in fs.frame(n)] for n in range(wl.n_frames)]
        twins = [make_state(wl), make_state(wl)]    # [allocating, static]
        for st in twins:
            st.set_flags(flags)
        shape = (wl.tokens_per_frame, wl.n_q_heads, wl.head_dim)
        outs = [torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in twins]
        work.append((wl, frames, twins, outs))
    for n in range(max(w[0].n_frames for w in work)):
        for wl, frames, twins, outs in work:
            if n >= wl.n_frames:
                continue
            _frame(twins[0], frames[n], n, outs[0], static=False)
            _frame(twins[1], frames[n], n, outs[1], static=True)
            torch.cuda.synchronize()
            assert torch.equal(outs[0], outs[1]), (wl.name, n)
            for a, b in zip(_state_bits(twins[0]), _state_bits(twins[1])):
                assert torch.equal(a, b), (wl.name, n)
    for _, _, twins, _ in work:
        for st in twins:
            st.close()


def test_static_scratch_rejects_oversized_steps():
    """A step whose working buffers exceed the static scratch returns ESCRATCH
    before enqueuing anything; the state stays usable through the allocating
    entry point."""
    wl = StreamConfig(name="noalloc_big", config_id=112, dtype="bf16", n_q_heads=64,
                      n_kv_heads=8, head_dim=128, tokens_per_frame=1024, budget=1024,
                      n_frames=2, n_layers=1, rope_base=1e6, alpha=1.0, n_sinks=0)
    st = make_state(wl)
    x = [to_device(a, wl.dtype) for a in FrameStream(wl).frame(0)]
    out = torch.empty((1024, 64, 128), dtype=torch.bfloat16, device="cuda")
    lib = skv.load_library()
    rc = lib.statekv_prefill_frame_static(st._h, x[0].data_ptr(), x[1].data_ptr(),
                                          x[2].data_ptr(), 0, out.data_ptr())
    assert rc == skv.STATEKV_ESCRATCH
    _frame(st, x, 0, out, static=False)        # frame 0 is still the next frame
    torch.cuda.synchronize()
    _, _, pos = st.compressed_view()
    assert pos.numel() == 1024
    st.close()
