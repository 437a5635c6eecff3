"""The oracle against stored values: the 50-digit brute-force case written by
``tests/golden/make_bruteforce_golden.py`` (which calls only ``oracle/``) and
the figures the pages print about chunking (each cited in the fixture)."""
import json
import math
import os

import numpy as np

import oracle.lmhead_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bruteforce_case():
    g = load("bruteforce_h64.json")
    h = np.array(g["hidden_bf16_bits"], dtype=np.uint16)
    W = np.array(g["W_bf16_bits"], dtype=np.uint16)
    t = np.array(g["targets"], dtype=np.int32)
    return g, h, W, t


def test_oracle_matches_bruteforce_golden():
    g, h, W, t = bruteforce_case()
    out = O.forward_backward(h, W, t, g["chunk_size"], np.array(g["g_logp"]), np.array(g["g_ent"]))
    for k in ("logp", "entropy", "lse"):
        ref = np.array([float(x) for x in g[k]])
        assert np.allclose(out[k], ref, rtol=1e-13, atol=1e-14), k
    for k in ("dh", "dW"):
        ref = np.array([[float(x) for x in row] for row in g[k]])
        scale = np.abs(ref).max()
        assert np.allclose(out[k], ref, rtol=1e-10, atol=1e-12 * scale), k
    masked = np.flatnonzero(t < 0)
    assert masked.size == 1
    for k in ("logp", "entropy", "lse"):
        assert float(g[k][masked[0]]) == 0.0


def test_pages_memory_figure_is_one_f32_chunk_of_logits():
    """The chunked head's ~300 MB at chunk 512 is one float32 [chunk, vocab]
    tensor, and 128 chunks cover the batch-16 x 4k tokens; this is the
    transient bound the library's backward workspace is held to."""
    f = load("pages_figures.json")["chunked_lm_head_memory"]
    N = f["batch"] * f["seq_len"]
    per_chunk = f["chunk_size"] * f["vocab"] * 4
    assert abs(per_chunk / 1e6 - f["chunked_MB"]) / f["chunked_MB"] < 0.05
    assert abs(N * f["vocab"] / 1e9 - f["full_logits_GB"]) / f["full_logits_GB"] < 0.01
    assert len(O.chunk_ranges(N, f["chunk_size"])) == 128


def test_pages_chunk_steps():
    """16,384 local tokens in chunks of 4,096 take 4 steps of the chunk loop."""
    f = load("pages_figures.json")["fused_head_steps"]
    assert len(O.chunk_ranges(f["local_tokens"], f["chunk_size"])) == f["steps"]
    assert len(O.chunk_ranges(f["local_tokens"] + 1, f["chunk_size"])) == f["steps"] + 1
    assert O.chunk_ranges(f["local_tokens"] + 1, f["chunk_size"])[-1] == (16384, 16385)


def test_pages_chunk_invariance_figure_is_summation_order_scale():
    """The pages' chunk 4096 vs 1024 differences are at f32 rounding scale;
    the oracle's own chunk dependence is at fp64 rounding scale."""
    f = load("pages_figures.json")["chunk_4096_vs_1024_numerics"]
    assert f["max_abs_diff_grad"] / f["grad_max_abs"] < 1e-6
    assert f["max_abs_diff_logp"] < 1e-5
    g, h, W, t = bruteforce_case()
    a = O.forward_backward(h, W, t, 1, np.array(g["g_logp"]), np.array(g["g_ent"]))
    b = O.forward_backward(h, W, t, 4, np.array(g["g_logp"]), np.array(g["g_ent"]))
    assert np.max(np.abs(a["logp"] - b["logp"])) < 1e-14
    assert np.max(np.abs(a["dW"] - b["dW"])) <= 1e-14 * np.abs(a["dW"]).max()
    assert math.isclose(float(np.abs(a["lse"]).max()), float(np.abs(b["lse"]).max()), rel_tol=1e-15)
