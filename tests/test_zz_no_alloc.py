"""int8_gemm_noalloc (the gemm whose split-K workspace is the library's static
device scratch) against int8_gemm_ws (the same gemm with a caller-allocated
workspace): bit-identical outputs on consecutive calls, the second one
smaller, so the scratch holds the first call's partials when the second
starts; shapes that do not split, the same bits as int8_gemm; a call whose
split needs more than the scratch holds is rejected before anything runs.
A few rows of the split result are also checked against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import assert_close, bits_to_dev, dev_to_bits, make_weight, upload
from weight_only_quantized_int8_amd import binding as B
from weight_only_quantized_int8_amd import synth

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _poisoned(m, n):
    return torch.full((m, n), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def _run_ws(W, Xd, m):
    need = B.int8_gemm_workspace_bytes(W.desc, m)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    Y = _poisoned(m, W.out_features)
    rc = B.int8_gemm_ws(W.desc, Xd.data_ptr(), Y.data_ptr(), m, ws.data_ptr(), ws.numel(), _stream())
    assert rc == 0, B.load_library().int8w_last_error()
    return Y


def _run_noalloc(W, Xd, m):
    Y = _poisoned(m, W.out_features)
    rc = B.int8_gemm_noalloc(W.desc, Xd.data_ptr(), Y.data_ptr(), m, _stream())
    assert rc == 0, B.load_library().int8w_last_error()
    return Y


def test_noalloc_split_two_calls_then_smaller():
    N, K, gs = 4096, 14336, 64
    w, rng = make_weight(7_100, N, K, gs)
    W = upload(w)
    for m in (600, 200):  # 60 MiB of partials, then 28 MiB over the first call's
        need = B.int8_gemm_workspace_bytes(W.desc, m)
        log(f"noalloc split m={m} {N}x{K} gs{gs} need={need}")
        assert 0 < need <= B.NOALLOC_SCRATCH_BYTES, "the shape is expected to split within the scratch"
        X = synth.gen_act(rng, (m, K))
        Xd = bits_to_dev(X)
        Y_na = _run_noalloc(W, Xd, m)
        Y_ws = _run_ws(W, Xd, m)
        torch.cuda.synchronize()
        got, exp = dev_to_bits(Y_na), dev_to_bits(Y_ws)
        assert np.array_equal(got, exp), f"m={m}: {np.count_nonzero(got != exp)} outputs differ from int8_gemm_ws"
        rows = np.array([0, 1, m // 2, m - 1])
        Y_ref, A = oracle.gemm(w.packed, w.scales, w.biases, gs, X[rows])
        assert_close(got[rows], Y_ref, A, f"noalloc m={m} sampled rows")


@pytest.mark.parametrize("m,N,K,gs", [(2048, 4096, 4096, 64), (8, 512, 1024, 32), (1, 256, 512, 128)])
def test_noalloc_unsplit_matches_int8_gemm(m, N, K, gs):
    log(f"noalloc unsplit m={m} {N}x{K} gs{gs}")
    w, rng = make_weight(7_200 + m, N, K, gs)
    W = upload(w)
    assert B.int8_gemm_workspace_bytes(W.desc, m) == 0
    Xd = bits_to_dev(synth.gen_act(rng, (m, K)))
    Y_na = _run_noalloc(W, Xd, m)
    Y = _poisoned(m, N)
    assert B.int8_gemm(W.desc, Xd.data_ptr(), Y.data_ptr(), m, _stream()) == 0
    torch.cuda.synchronize()
    assert np.array_equal(dev_to_bits(Y_na), dev_to_bits(Y))


def test_noalloc_rejects_split_beyond_scratch():
    # 4096 x 14336 gs32 at m = 768: 96 tiles split 8 ways, 96 MiB of partials
    N, K, gs, m = 4096, 14336, 32, 768
    packed = torch.empty(N * K // 4, dtype=torch.int32, device="cuda")
    scales = torch.empty(N * (K // gs), dtype=torch.int16, device="cuda")
    biases = torch.empty(N * (K // gs), dtype=torch.int16, device="cuda")
    desc = B.WeightDesc(packed.data_ptr(), scales.data_ptr(), biases.data_ptr(), N, K, gs)
    need = B.int8_gemm_workspace_bytes(desc, m)
    log(f"noalloc reject m={m} {N}x{K} need={need}")
    assert need > B.NOALLOC_SCRATCH_BYTES
    X = torch.zeros((m, K), dtype=torch.bfloat16, device="cuda")
    Y = _poisoned(m, N)
    rc = B.int8_gemm_noalloc(desc, X.data_ptr(), Y.data_ptr(), m, _stream())
    torch.cuda.synchronize()
    assert rc == B.INT8W_ERR_SHAPE
    assert b"scratch" in B.load_library().int8w_last_error()
    assert bool((Y.view(torch.int16) == -1).all()), "a rejected call must enqueue nothing"


def test_noalloc_inside_a_hip_graph():
    """The callers it is for: the call captured in a HIP graph (nothing is
    allocated during capture), replayed three times with new X written
    eagerly between the replays; every replay against int8_gemm_ws on the
    same X, bit for bit."""
    N, K, gs, m = 4096, 14336, 64, 512  # splits K over 4 parts: the scratch is used
    w, rng = make_weight(7_300, N, K, gs)
    W = upload(w)
    assert 0 < B.int8_gemm_workspace_bytes(W.desc, m) <= B.NOALLOC_SCRATCH_BYTES
    Xd = bits_to_dev(synth.gen_act(rng, (m, K)))
    Y = _poisoned(m, N)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # one eager call on the capture stream first
        assert B.int8_gemm_noalloc(W.desc, Xd.data_ptr(), Y.data_ptr(), m, s.cuda_stream) == 0
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rc = B.int8_gemm_noalloc(W.desc, Xd.data_ptr(), Y.data_ptr(), m, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, B.load_library().int8w_last_error()
    for rep in range(3):
        log(f"noalloc graph replay {rep}")
        X = synth.gen_act(rng, (m, K))
        Xd.copy_(bits_to_dev(X))  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = dev_to_bits(Y)
        exp = dev_to_bits(_run_ws(W, Xd, m))
        torch.cuda.synchronize()
        assert np.array_equal(got, exp), f"replay {rep}: {np.count_nonzero(got != exp)} outputs differ"


def test_int8weight_gemm_under_capture_takes_the_static_scratch():
    """Int8Weight.gemm captured with no cached workspace large enough: it does
    not allocate during capture (the static scratch serves the split), and
    every replay equals the eager result."""
    N, K, gs, m = 4096, 14336, 64, 600  # splits K over 5 parts
    w, rng = make_weight(7_400, N, K, gs)
    W = upload(w)
    need = B.int8_gemm_workspace_bytes(W.desc, m)
    assert 0 < need <= B.NOALLOC_SCRATCH_BYTES
    saved = dict(B._workspaces)
    B._workspaces.clear()  # no cached workspace: it would have to grow
    try:
        Xd = bits_to_dev(synth.gen_act(rng, (m, K)))
        Y = _poisoned(m, N)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            torch.empty(1, device="cuda")  # warm the stream's allocator outside capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            W.gemm(Xd, Y)
        assert not B._workspaces, "the workspace grew during capture"
        for rep in range(2):
            log(f"Int8Weight.gemm graph replay {rep}")
            Xd.copy_(bits_to_dev(synth.gen_act(rng, (m, K))))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = dev_to_bits(Y)
            exp = dev_to_bits(_run_ws(W, Xd, m))
            torch.cuda.synchronize()
            assert np.array_equal(got, exp), f"replay {rep}: {np.count_nonzero(got != exp)} outputs differ"
    finally:
        B._workspaces.clear()
        B._workspaces.update(saved)
