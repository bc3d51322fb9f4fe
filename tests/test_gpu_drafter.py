"""GPU parity of ddtree_drafter_topk (through the C ABI) against ``oracle.drafter``.

Bars: token ids bit-exact (the order is decided on the logits themselves,
exactly, on both sides); log-probabilities within 1e-5 absolute of the fp64
oracle (fp32 arithmetic: the row's log-sum-exp is accumulated in fp32 over
up to 163,840 terms, about 1e-6 relative, plus one rounding of the
difference).  Covered: fp32 and bf16 logits, 16-byte and scalar load paths
(vocabulary sizes that are and are not multiples of 4 / 8, and a
misaligned row start), one chunk, many chunks and a ragged last chunk, k from
1 to 32, a vocabulary of one token, rows of many equal logits (ties ordered
by token id), rows with -inf entries, and rows whose last one or two
8192-logit chunks are entirely -inf (a masked vocabulary tail: such a chunk
has no mass and must not poison the row's log-sum-exp); full size: 56 rows (8 requests x 7
depths) of 163,840 logits, the measured configuration.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import drafter
from tree_verify_mla_amd import _lib
from workloads import bf16_bits_to_f32, draw_drafter_logits

pytestmark = pytest.mark.gpu

TOL = 1e-5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _gpu(x_dev, k):
    rows, vocab = x_dev.shape
    vals = torch.empty(rows, k, dtype=torch.float32, device="cuda")
    ids = torch.empty(rows, k, dtype=torch.int32, device="cuda")
    # stale workspace contents must not matter
    ws = torch.full((max(_lib.ddtree_drafter_topk_workspace_size(rows, vocab, k), 1),), 0x5A,
                    dtype=torch.uint8, device="cuda")
    _lib.ddtree_drafter_topk(x_dev, vals, ids, workspace=ws)
    torch.cuda.synchronize()
    return vals.cpu().numpy(), ids.cpu().numpy()


def _check(x_host_f32, x_dev, k):
    vals, ids = _gpu(x_dev, k)
    rv, ri = drafter.batch(x_host_f32, k)
    assert np.array_equal(ids, ri)
    assert np.abs(vals - rv).max() <= TOL


def _dev(x_np, dtype):
    if dtype == "bf16":
        return torch.from_numpy(x_np.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(x_np).cuda()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("vocab,k", [(1, 1), (7, 7), (512, 8), (4097, 16), (8192, 8),
                                     (8193, 32), (32768, 8), (32769, 16), (50001, 4),
                                     (65536, 16), (200003, 32)])
def test_shapes(dtype, vocab, k):
    _say(f"test_shapes {dtype} V={vocab} k={k}")
    rng = np.random.default_rng(vocab * 7 + k)
    x = draw_drafter_logits(rng, 5, vocab, dtype=dtype)
    xf = bf16_bits_to_f32(x) if dtype == "bf16" else x
    _check(xf, _dev(x, dtype), k)


def test_misaligned_rows_take_the_scalar_path():
    _say("test_misaligned_rows_take_the_scalar_path")
    rng = np.random.default_rng(11)
    x = draw_drafter_logits(rng, 3, 8192 * 2 + 1, dtype="f32")
    flat = torch.from_numpy(x.reshape(-1)).cuda()
    buf = torch.empty(flat.numel() + 1, dtype=torch.float32, device="cuda")
    buf[1:] = flat
    view = buf[1:].view(3, -1)                 # starts 4 bytes into the allocation
    assert view.data_ptr() % 16 != 0
    _check(x, view, 8)


def test_ties_and_minus_infinity():
    _say("test_ties_and_minus_infinity")
    rng = np.random.default_rng(12)
    for vocab in (300, 9000, 20000):
        x = rng.integers(-2, 3, size=(4, vocab)).astype(np.float32)   # many equal logits
        x[1, rng.choice(vocab, vocab // 2, replace=False)] = -np.inf
        x[2, :] = 0.0                                                   # a row of equal logits
        _check(x, torch.from_numpy(x).cuda(), 16)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_masked_tail_chunks(dtype):
    _say(f"test_masked_tail_chunks {dtype}")
    rng = np.random.default_rng(14)
    CH = 8192                                      # logits per chunk
    vocab = CH * 4 + 100                           # five chunks, the last one ragged
    x = draw_drafter_logits(rng, 4, vocab, dtype="f32")
    x[0, CH * 4:] = -np.inf                        # the ragged last chunk
    x[1, CH * 3:] = -np.inf                        # the last two chunks
    x[2, :CH] = -np.inf                            # the first chunk
    x[3, CH:CH * 2] = -np.inf                      # a middle chunk
    x[3, CH * 4:] = -np.inf
    if dtype == "bf16":
        from workloads import f32_to_bf16_bits
        xb = f32_to_bf16_bits(x)
        xf = bf16_bits_to_f32(xb)
        _check(xf, _dev(xb, dtype), 16)
    else:
        _check(x, _dev(x, dtype), 16)


def test_full_size_headline_rows():
    _say("test_full_size_headline_rows")
    rng = np.random.default_rng(13)
    for dtype in ("f32", "bf16"):
        x = draw_drafter_logits(rng, 56, 163840, dtype=dtype)
        xf = bf16_bits_to_f32(x) if dtype == "bf16" else x
        _check(xf, _dev(x, dtype), 8)


def test_repeated_calls_on_one_workspace():
    """One workspace serves call after call, with fewer rows too: whatever a
    call leaves in it does not matter to the next."""
    _say("test_repeated_calls_on_one_workspace")
    rng = np.random.default_rng(15)
    V, k = 163840, 8
    ws = torch.empty(_lib.ddtree_drafter_topk_workspace_size(56, V, k), dtype=torch.uint8,
                     device="cuda")
    for rows in (56, 56, 7, 56):
        x = draw_drafter_logits(rng, rows, V, dtype="f32")
        vals = torch.empty(rows, k, dtype=torch.float32, device="cuda")
        ids = torch.empty(rows, k, dtype=torch.int32, device="cuda")
        _lib.ddtree_drafter_topk(torch.from_numpy(x).cuda(), vals, ids, workspace=ws)
        torch.cuda.synchronize()
        rv, ri = drafter.batch(x, k)
        assert np.array_equal(ids.cpu().numpy(), ri)
        assert np.abs(vals.cpu().numpy() - rv).max() <= TOL
