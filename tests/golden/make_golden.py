"""Writes tiny_stream.json: the oracle's selections and scores on the tiny stream.

Calls only the oracle and the seeded workload generator.  The file is a
regression fixture: it records what the pinned oracle computes so that an
accidental change to the oracle's arithmetic shows up as a diff.

Usage: python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from kv_cache_compression_statekv_amd.workload import CONFIGS, FrameStream  # noqa: E402
from oracle import LayerConfig, OracleStream  # noqa: E402


def main():
    wl = CONFIGS["tiny"]
    cfg = LayerConfig(n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                      head_dim=wl.head_dim, tokens_per_frame=wl.tokens_per_frame,
                      budget=wl.budget, dtype=wl.dtype, rope_base=wl.rope_base)
    frames = []
    stream, orc = FrameStream(wl), OracleStream(cfg)
    for n in range(wl.n_frames):
        res = orc.step(*stream.frame(n))
        frames.append({
            "frame": n,
            "pool_pos": [int(p) for p in res.pool_pos],
            "scores32_hex": [float(s).hex() for s in res.scores32],
            "kept_pos": [int(p) for p in orc.state.pos],
            "o_abs_sum": float(abs(res.O_exact).sum()),
        })
    doc = {
        "what": "oracle output on the tiny stream (fp32, Hq=2, Hkv=1, d=64, T=16, B=32, N=8)",
        "source": "paper note 'Linear Scaling Video VLMs for Long Video Understanding', "
                  "section 方法详解 (关键设计 1-3); written by tests/golden/make_golden.py",
        "frames": frames,
    }
    with open(os.path.join(HERE, "tiny_stream.json"), "w") as f:
        json.dump(doc, f, indent=1)


if __name__ == "__main__":
    main()
