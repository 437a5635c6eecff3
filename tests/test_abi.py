"""The C-ABI library on the host: it loads, exports every function the public
header declares, and rejects bad arguments with the documented codes before
touching the GPU (no compute call runs here). Fake device addresses are
used only on paths that fail validation."""
import json
import os
import re

import pytest

from cross_entropy_amd import _native as nat

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmhead_logps.h")

FAKE = 0x10000        # 64 KiB-aligned non-NULL address; never dereferenced
MIS = FAKE + 2        # misaligned address


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lmhead_logps_\w+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = nat.load()
    names = declared_functions()
    assert set(names) == set(nat.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n
    assert "gfx950" in nat.version()


def test_error_codes_match_header():
    src = open(HEADER).read()
    codes = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define (LMH_ERR_\w+) \((-\d+)\)", src)}
    assert codes == {v: k for k, v in nat.ERROR_NAMES.items()}


def _fwd(**kw):
    a = dict(hidden=FAKE, W=FAKE, targets=FAKE, N=64, H=128, V=300, chunk_size=16, logp=FAKE, entropy=FAKE,
             lse=FAKE, workspace=FAKE, workspace_bytes=0, stream=0)
    a.update(kw)
    return nat.raw_fwd(**a)


def _bwd(**kw):
    a = dict(hidden=FAKE, W=FAKE, targets=FAKE, N=64, H=128, V=300, chunk_size=16, lse=FAKE, entropy=FAKE,
             g_logp=FAKE, g_ent=FAKE, dh=FAKE, dW=FAKE, workspace=FAKE, workspace_bytes=0, stream=0)
    a.update(kw)
    return nat.raw_bwd(**a)


@pytest.mark.parametrize("call", [_fwd, _bwd])
def test_shape_and_chunk_errors(call):
    assert call(N=-1) == -2
    assert call(H=0) == -2
    assert call(V=0) == -2
    assert call(V=1 << 31) == -2
    assert call(N=1 << 31) == -2
    assert call(chunk_size=0) == -3
    assert call(chunk_size=-5) == -3
    assert call(H=96) == -6
    assert "multiple of 64" in nat.load().lmhead_logps_last_error().decode()


def test_forward_null_alignment_and_workspace_errors():
    for k in ("hidden", "W", "targets", "logp", "lse", "workspace"):
        assert _fwd(**{k: 0}) == -1, k
    assert _fwd(hidden=MIS) == -6
    assert _fwd(W=MIS) == -6
    assert _fwd(workspace=MIS) == -6
    need = nat.raw_workspace_bytes(64, 128, 300, 16, False)
    assert _fwd(workspace_bytes=need - 1) == -4
    assert "needed" in nat.load().lmhead_logps_last_error().decode()
    assert _fwd(N=0, hidden=0, W=0, targets=0, logp=0, lse=0, workspace=0) == 0   # N = 0: nothing to do


def test_backward_null_args_alignment_and_workspace_errors():
    assert _bwd(entropy=0) == -5           # g_ent without the forward's entropy
    assert _bwd(dW=0) == -1
    for k in ("hidden", "W", "targets", "lse", "dh", "workspace"):
        assert _bwd(**{k: 0}) == -1, k
    assert _bwd(hidden=MIS) == -6
    assert _bwd(dh=FAKE + 4) == -6         # dh is written 16 bytes at a time
    need = nat.raw_workspace_bytes(64, 128, 300, 16, True)
    assert _bwd(workspace_bytes=need - 1) == -4


def _fwd_t(temperature, **kw):
    a = dict(hidden=FAKE, W=FAKE, targets=FAKE, N=64, H=128, V=300, chunk_size=16, temperature=temperature,
             logp=FAKE, entropy=FAKE, lse=FAKE, workspace=FAKE, workspace_bytes=0, stream=0)
    a.update(kw)
    return nat.raw_fwd_temp(**a)


def _bwd_t(temperature, **kw):
    a = dict(hidden=FAKE, W=FAKE, targets=FAKE, N=64, H=128, V=300, chunk_size=16, temperature=temperature,
             lse=FAKE, entropy=FAKE, g_logp=FAKE, g_ent=FAKE, dh=FAKE, dW=FAKE, workspace=FAKE,
             workspace_bytes=0, stream=0)
    a.update(kw)
    return nat.raw_bwd_temp(**a)


@pytest.mark.parametrize("call", [_fwd_t, _bwd_t])
def test_temperature_errors(call):
    """The tempered calls reject a temperature that is not finite and > 0
    (LMH_ERR_ARGS) and otherwise check arguments like the plain calls."""
    for bad in (0.0, -0.7, float("nan"), float("inf"), -float("inf"), 1e-40):
        assert call(bad) == -5, bad
        assert "temperature" in nat.load().lmhead_logps_last_error().decode()
    assert call(0.7, N=-1) == -2
    assert call(0.7, chunk_size=0) == -3
    assert call(0.7, H=96) == -6
    assert call(0.7, workspace_bytes=0) == -4        # valid temperature: fails on the workspace next


def test_backward_size_limit():
    # 256-row tiles of the transposed operands are addressed with 32-bit byte
    # offsets: the backward (and its workspace query) refuses N or V whose
    # multiple of 256 reaches 2^23
    lim = 1 << 23
    assert _bwd(N=lim - 256, workspace_bytes=0) == -4        # within the limit: only the workspace is short
    assert _bwd(N=lim - 255) == -6
    assert _bwd(V=lim) == -6
    b = nat.raw_workspace_bytes(lim - 256, 128, 300, 16, True)
    assert b > 0
    with pytest.raises(nat.LmheadError):
        nat.raw_workspace_bytes(64, 128, lim - 255, 16, True)
    assert nat.raw_workspace_bytes(64, 128, lim - 255, 16, False) > 0   # the forward has no such limit


def test_backward_ex_flags():
    """lmhead_logps_bwd_ex accepts only its two accumulate bits."""
    a = dict(hidden=FAKE, W=FAKE, targets=FAKE, N=64, H=128, V=300, chunk_size=16, temperature=1.0,
             lse=FAKE, entropy=FAKE, g_logp=FAKE, g_ent=FAKE, dh=FAKE, dW=FAKE, workspace=FAKE,
             workspace_bytes=0, stream=0)
    for bad in (4, 8, 0x80000000):
        assert nat.raw_bwd_ex(flags=bad, **a) == -5, bad
        assert "flags" in nat.load().lmhead_logps_last_error().decode()
    for good in (0, 1, 2, 3):
        assert nat.raw_bwd_ex(flags=good, **a) == -4, good   # valid flags: fails on the workspace next
    assert nat.BWD_ACCUMULATE_DH == 1 and nat.BWD_ACCUMULATE_DW == 2
    src = open(HEADER).read()
    assert "#define LMH_BWD_ACCUMULATE_DH 1u" in src and "#define LMH_BWD_ACCUMULATE_DW 2u" in src


def test_shard_errors():
    """Shard calls reject shards outside [0, V_total) and bad shard counts."""
    fs = dict(hidden=FAKE, W_shard=FAKE, targets=FAKE, N=64, H=128, V_shard=300, vocab_offset=0, V_total=1000,
              chunk_size=16, temperature=1.0, partial=FAKE, workspace=FAKE, workspace_bytes=0, stream=0)
    assert nat.raw_fwd_shard(**dict(fs, vocab_offset=-1)) == -2
    assert nat.raw_fwd_shard(**dict(fs, vocab_offset=701)) == -2          # 701 + 300 > 1000
    assert nat.raw_fwd_shard(**dict(fs, V_total=1 << 31)) == -2
    assert nat.raw_fwd_shard(**dict(fs, partial=0)) == -1
    assert nat.raw_fwd_shard(**dict(fs, partial=MIS)) == -6
    assert nat.raw_fwd_shard(**dict(fs, vocab_offset=700)) == -4          # a valid last shard: workspace next
    ms = dict(partials=FAKE, P=3, targets=FAKE, N=64, V_total=1000, temperature=1.0, logp=FAKE, entropy=FAKE,
              lse=FAKE, stream=0)
    assert nat.raw_merge_shards(**dict(ms, P=0)) == -2
    assert nat.raw_merge_shards(**dict(ms, V_total=0)) == -2
    assert nat.raw_merge_shards(**dict(ms, partials=0)) == -1
    assert nat.raw_merge_shards(**dict(ms, temperature=0.0)) == -5
    assert nat.raw_merge_shards(**dict(ms, N=0)) == 0
    bs = dict(hidden=FAKE, W_shard=FAKE, targets=FAKE, N=64, H=128, V_shard=300, vocab_offset=0, V_total=1000,
              chunk_size=16, temperature=1.0, lse=FAKE, entropy=FAKE, g_logp=FAKE, g_ent=FAKE, dh=FAKE,
              dW_shard=FAKE, flags=0, workspace=FAKE, workspace_bytes=0, stream=0)
    assert nat.raw_bwd_shard(**dict(bs, vocab_offset=900)) == -2
    assert nat.raw_bwd_shard(**dict(bs, flags=4)) == -5
    assert nat.raw_bwd_shard(**bs) == -4


def test_workspace_query_errors():
    import ctypes
    assert nat.load().lmhead_logps_workspace_bytes(1, 64, 10, 4, 0, None) == -1
    with pytest.raises(nat.LmheadError) as e:
        nat.raw_workspace_bytes(1, 65, 10, 4, True)
    assert e.value.code == -6
    assert nat.raw_workspace_bytes(0, 64, 10, 4, True) > 0
    _ = ctypes


SHAPES = [(256, 256, 4096, 128), (4096, 2560, 151936, 512), (65536, 2560, 151936, 512),
          (15237, 4096, 151936, 1024), (15237, 4096, 151936, 4096), (65536, 2560, 151936, 4096),
          (700, 320, 3001, 7), (1, 64, 1, 1)]


def _pad(x, m=256):
    return (x + m - 1) // m * m


def _spread(x):
    """Row stride of the backward's bf16 operands: a multiple of 64 elements
    with an odd quotient (rows strided by a large power of two crowd onto few
    memory channels)."""
    return (((x + 63) // 64) | 1) * 64


def _operand_copies(N, H, V):
    """Input-sized operand copies held by the backward: the bf16 transpose of
    hidden (rows padded to the spread stride) and W's last V % 64 rows padded
    to 64 rows."""
    return 2 * _pad(H) * _spread(_pad(max(N, 1))) + _pad(64 * H * 2)


def _backward_blocks(N, H, V, C):
    """The backward's block shape as the host chooses it: token-block edge
    ct and vocabulary-block edge vb (multiples of 256, the two bf16 cotangent
    buffers within one float32 [C, V] tensor) minimising the float32
    accumulation traffic plus a per-launch cost; blocks evened out."""
    T = 256
    N = max(N, 1)
    budget = max(float(C) * V, float(T * _spread(T)))
    best, best_t = None, 1e300
    for ct in range(T, _pad(N) + 1, T):
        vb = min((int(budget / ct) - 64) // T * T, _pad(V))
        if vb < T:
            break
        n_tb, n_vb = -(-N // ct), -(-V // vb)
        t = (n_tb * n_vb + 1) * 20e-6 + (8.0 * N * H * n_vb + 8.0 * V * H * n_tb) / 5e12
        if t < best_t:
            best_t, best = t, (n_tb, _pad(-(-N // n_tb)), n_vb, _pad(-(-V // n_vb)))
    return best


def test_headline_backward_plan():
    """The headline shape's backward runs 8 token blocks of 8192 x 17
    vocabulary blocks of 8960: the plan that minimises the float32
    accumulation traffic within chunk 512's budget. The library's workspace
    size agrees with that layout to the byte."""
    N, H, V, C = 65536, 2560, 151936, 512
    n_tb, ct, n_vb, vb = _backward_blocks(N, H, V, C)
    assert (n_tb, ct, n_vb, vb) == (8, 8192, 17, 8960)
    dz = _pad(ct * _spread(vb) * 2)
    expect = 2 * dz + _pad(_pad(H) * _spread(_pad(N)) * 2) + _pad(64 * H * 2) + _pad((n_tb * n_vb + 1) * 8 * 4)
    assert nat.raw_workspace_bytes(N, H, V, C, True) == max(expect, nat.raw_workspace_bytes(N, H, V, C, False))


@pytest.mark.parametrize("N,H,V,C", SHAPES)
def test_backward_transient_within_one_f32_chunk_of_logits(N, H, V, C):
    """The backward's [tokens, vocab]-shaped transient (the cotangent block,
    held twice in bf16, its row padding included) stays within one float32
    [chunk_size, V] tensor (at least one 256 x 256 tile with its padded row
    stride); the rest of the workspace is the input-sized transpose of hidden
    and W's padded last rows. The forward's workspace is O(N), independent of
    V."""
    b = nat.raw_workspace_bytes(N, H, V, C, True)
    f = nat.raw_workspace_bytes(N, H, V, C, False)
    assert b <= max(C * V * 4, 256 * _spread(256) * 4) + _operand_copies(N, H, V) + max(f, 1024)
    assert f <= 16 * 128 * max(64, (N + 63) // 64 * 64) + 256


def test_pages_chunk_512_figure():
    """At the pages' headline shape (batch 16 x 4k tokens, 152k vocabulary,
    chunk 512) the backward transient is at most the ~300 MB of one float32
    [512, vocab] chunk of logits (SkyRL "[tx] support long sequence",
    "4. Chunked LM Head")."""
    f = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_figures.json")))["chunked_lm_head_memory"]
    N, H, V = f["batch"] * f["seq_len"], 2560, f["vocab"]
    b = nat.raw_workspace_bytes(N, H, V, f["chunk_size"], True) - _operand_copies(N, H, V)
    assert b <= f["chunk_size"] * V * 4
    assert b / 1e6 < 1.05 * f["chunked_MB"] + 11.2


def test_library_binds_to_one_hip_runtime():
    """The binding imports torch before loading the library, so the process
    holds a single HIP runtime (torch's), whose pointers and streams the
    library is handed."""
    nat.load()
    assert len(nat._hip_runtimes_mapped()) == 1


def test_noalloc_scratch_size_matches_header_and_rejects_large_calls():
    """The fixed scratch of the allocation-free forward: its size in the
    header equals the binding's, and a call that needs more fails with
    LMH_ERR_WORKSPACE on the host, before any device call."""
    src = open(HEADER).read()
    m = re.search(r"#define LMH_NOALLOC_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)", src)
    assert m and int(m.group(1)) << 20 == nat.NOALLOC_SCRATCH_BYTES
    a = dict(hidden=FAKE, W=FAKE, targets=FAKE, N=600_000, H=64, V=151936, chunk_size=512, temperature=1.0,
             logp=FAKE, entropy=FAKE, lse=FAKE, stream=0)
    assert nat.raw_workspace_bytes(600_000, 64, 151936, 512, False) > nat.NOALLOC_SCRATCH_BYTES
    assert nat.raw_fwd_noalloc(**a) == -4
    assert "scratch" in nat.load().lmhead_logps_last_error().decode()
    assert nat.raw_fwd_noalloc(**dict(a, N=-1)) == -2
    assert nat.raw_fwd_noalloc(**dict(a, H=100)) == -6
    assert nat.raw_fwd_noalloc(**dict(a, temperature=0.0)) == -5
    assert nat.raw_fwd_noalloc(**dict(a, N=0)) == 0


def _bwd16(**kw):
    a = dict(hidden=FAKE, W=FAKE, targets=FAKE, N=64, H=128, V=300, chunk_size=16, temperature=1.0, lse=FAKE,
             entropy=FAKE, g_logp=FAKE, g_ent=FAKE, dh=FAKE, dW=FAKE, flags=0, workspace=FAKE, workspace_bytes=0,
             stream=0)
    a.update(kw)
    return nat.raw_bwd_bf16(**a)


def test_bf16_backward_argument_errors():
    """The bf16-gradient backward's host checks: the backward's codes, its
    own workspace size (the float32 backward's plus its accumulators) and
    16-byte aligned bf16 gradients."""
    assert _bwd16(N=-1) == -2
    assert _bwd16(chunk_size=0) == -3
    assert _bwd16(flags=4) == -5
    assert _bwd16(entropy=0) == -5
    assert _bwd16(dW=0) == -1
    assert _bwd16(dW=MIS) == -6
    assert _bwd16(dh=MIS) == -6
    f32 = nat.raw_workspace_bytes(64, 128, 300, 16, nat.WS_BWD)
    b16 = nat.raw_workspace_bytes(64, 128, 300, 16, nat.WS_BWD_BF16)
    assert b16 > f32
    assert _bwd16(workspace_bytes=f32) == -4
    assert "bwd_bf16" in nat.load().lmhead_logps_last_error().decode()
    with pytest.raises(nat.LmheadError):
        nat.raw_workspace_bytes(64, 128, 300, 16, 3)


@pytest.mark.parametrize("N,H,V,C", [(65536, 2560, 151936, 512), (4096, 2560, 151936, 512), (200000, 256, 5000, 64)])
def test_bf16_workspace_holds_the_smaller_gradient_in_float32(N, H, V, C):
    """The bf16 backward's extra workspace: min(N, V) x H float32 (the
    smaller gradient summed over the call) plus one block's rows of the other,
    never a float32 copy of both gradients."""
    f32 = nat.raw_workspace_bytes(N, H, V, C, nat.WS_BWD)
    b16 = nat.raw_workspace_bytes(N, H, V, C, nat.WS_BWD_BF16)
    extra = b16 - f32
    whole = 4 * (-(-min(N, V) // 256) * 256) * H
    # a block edge is at most chunk_size * V / 256 (blocks hold at most chunk_size * V elements, edges >= 256)
    assert whole <= extra <= whole + 4 * H * (C * V // 256 + 256) + 512, (extra, whole)


def test_planner_sweep_sizes():
    """Workspace sizes over a sweep of shapes, chunk sizes and the three
    kinds (run under the host sanitizers by tests/test_sanitize.py, where
    any overflow in the planner's arithmetic aborts): sizes are positive,
    grow with the kind, and the backward's stays below the float32 chunk
    bound plus the input-sized parts."""
    for N in (1, 7, 255, 256, 257, 4096, 65536, 1 << 22, (1 << 23) - 257):
        for H in (64, 2560, 4096):
            for V in (1, 5, 4097, 151936, 248320, (1 << 23) - 257):
                for C in (1, 512, 4096, 1 << 30):
                    f = nat.raw_workspace_bytes(N, H, V, C, nat.WS_FWD)
                    b = nat.raw_workspace_bytes(N, H, V, C, nat.WS_BWD)
                    b16 = nat.raw_workspace_bytes(N, H, V, C, nat.WS_BWD_BF16)
                    assert 0 < f <= b < b16, (N, H, V, C)
                    n_pad, v_pad, h_pad = -(-N // 256) * 256, -(-V // 256) * 256, -(-H // 256) * 256
                    # two bf16 cotangent buffers within max(chunk * V, one tile), hidden^T, W tail, counters
                    dz = 4 * min(max(C * V, 256 * 320), n_pad * (v_pad + 128)) + 4 * 64 * max(n_pad, v_pad)
                    ht = 2 * h_pad * (n_pad + 128)
                    assert b <= max(f, dz + ht + 2 * 64 * H + 8 * 4 * 8192 * 64 + 4096), (N, H, V, C, b)


def test_last_error_is_per_thread():
    """Each thread reads its own call's message (the library keeps the last
    error thread-local): threads failing with different arguments at the same
    time, each checking the message names its own value; a successful call
    clears the calling thread's message only."""
    import ctypes
    import threading
    lib = nat.load()
    errors = []
    start = threading.Barrier(8)

    def worker(k):
        try:
            start.wait()
            out = ctypes.c_size_t(0)
            for it in range(2000):
                bad = -(1000 * k + it + 1)
                rc = lib.lmhead_logps_workspace_bytes(bad, 64, 100, 4, 0, ctypes.byref(out))
                msg = lib.lmhead_logps_last_error().decode()
                if rc != -2 or f"got {bad}" not in msg:
                    errors.append((k, it, rc, msg))
                    return
                if it % 100 == 99:
                    assert lib.lmhead_logps_workspace_bytes(10, 64, 100, 4, 0, ctypes.byref(out)) == 0
                    if lib.lmhead_logps_last_error().decode() != "":
                        errors.append((k, it, "not cleared"))
                        return
        except Exception as e:   # reported below, from the main thread
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]
