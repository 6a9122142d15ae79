"""The plain streaming reads that measure the read ceiling (sd_stream_read,
sd_stream_read_rows): every workgroup's sink word must be the XOR of every
32-bit word of the chunk it was given, so that a read that skipped or
repeated part of its chunk, or read another one, shows. The expected folds
are computed on the host with numpy."""
import numpy as np
import pytest
import torch

import rejection_sampling_verify_softmax_amd as sd

pytestmark = pytest.mark.gpu


def _fold(words):
    return int(np.bitwise_xor.reduce(words)) if words.size else 0


def _data(n_words, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randint(-2**31, 2**31 - 1, (n_words,), generator=g, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("n_words,n_blocks", [(4 * 1024 * 7, 7), (4 * 100003, 13), (4 * 5000, 1)])
def test_stream_read_folds_each_chunk(n_words, n_blocks):
    print(f"stream_read {n_words * 4} bytes over {n_blocks} workgroups", flush=True)
    data = _data(n_words, 21)
    sink = torch.full((n_blocks,), -1, dtype=torch.int32, device="cuda")
    sd.stream_read(data, sink, n_blocks)
    torch.cuda.synchronize()
    host = data.cpu().numpy().view(np.uint32)
    nvec = n_words // 4
    chunk = -(-nvec // n_blocks)
    want = [_fold(host[4 * b * chunk: 4 * min(nvec, (b + 1) * chunk)]) for b in range(n_blocks)]
    assert [int(x) & 0xffffffff for x in sink.cpu().numpy()] == want


@pytest.mark.parametrize("n_rows,row_words,chunk_bytes", [(37, 3004, 4096), (5, 64128, 65536), (3, 12, 1 << 20)])
def test_stream_read_rows_folds_each_row_chunk(n_rows, row_words, chunk_bytes):
    print(f"stream_read_rows {n_rows} rows x {row_words * 4} bytes, chunks of {chunk_bytes}", flush=True)
    data = _data(n_rows * row_words, 22).view(n_rows, row_words)
    chunks = -(-row_words * 4 // chunk_bytes)
    sink = torch.full((n_rows * chunks,), -1, dtype=torch.int32, device="cuda")
    sd.stream_read_rows(data, chunk_bytes, sink)
    torch.cuda.synchronize()
    host = data.cpu().numpy().view(np.uint32)
    cw = chunk_bytes // 4
    want = [_fold(host[r, c * cw: min(row_words, (c + 1) * cw)]) for r in range(n_rows) for c in range(chunks)]
    assert [int(x) & 0xffffffff for x in sink.cpu().numpy()] == want
