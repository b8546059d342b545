"""The calibration streams of include/int8w_measure.h on the GPU: the copy
moves exactly its bytes and the expand widens exactly its bytes to 16 bits
(guard bytes around the destination stay), the read runs over ragged per-wave
ranges and leaves the sink alone for ordinary data."""
import numpy as np
import pytest
import torch

from weight_only_quantized_int8_amd import binding as B

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("nbytes", [1024, 5 * 1024, 1 << 20, 4_194_304 + 3 * 1024, 64 << 20])
def test_stream_copy_is_exact(nbytes):
    log(f"stream copy {nbytes}")
    rng = np.random.default_rng(nbytes)
    src = torch.from_numpy(rng.integers(0, 256, nbytes, dtype=np.uint8)).cuda()
    dst = torch.full((nbytes + 2048,), 0xA5, dtype=torch.uint8, device="cuda")
    rc = B.int8w_stream_copy(src.data_ptr(), dst[1024:].data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream)
    assert rc == B.INT8W_OK
    torch.cuda.synchronize()
    d = dst.cpu().numpy()
    assert np.array_equal(d[1024:1024 + nbytes], src.cpu().numpy())
    assert (d[:1024] == 0xA5).all() and (d[1024 + nbytes:] == 0xA5).all()


@pytest.mark.parametrize("nbytes", [1024, 5 * 1024, 1 << 20, 4_194_304 + 3 * 1024, 64 << 20])
def test_stream_expand_is_exact(nbytes):
    log(f"stream expand {nbytes}")
    rng = np.random.default_rng(nbytes + 1)
    src_h = rng.integers(0, 256, nbytes, dtype=np.uint8)
    src = torch.from_numpy(src_h).cuda()
    dst = torch.full((2 * nbytes + 2048,), 0xA5, dtype=torch.uint8, device="cuda")
    rc = B.int8w_stream_expand(src.data_ptr(), dst[1024:].data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream)
    assert rc == B.INT8W_OK
    torch.cuda.synchronize()
    d = dst.cpu().numpy()
    assert np.array_equal(d[1024:1024 + 2 * nbytes].view("<u2"), src_h.astype(np.uint16))
    assert (d[:1024] == 0xA5).all() and (d[1024 + 2 * nbytes:] == 0xA5).all()


@pytest.mark.parametrize("nbytes", [1024, 7 * 1024, 64 << 20])
def test_stream_read_runs(nbytes):
    log(f"stream read {nbytes}")
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    rc = B.int8w_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == B.INT8W_OK
    torch.cuda.synchronize()
    assert (sink.cpu().numpy() == 7).all()
