"""GPU parity of the two-tap dynamic convolution (dflash_two_tap_conv) against the
oracle.  Bar: the GPU computes in fp32 and rounds to bf16, so
|y - ref| <= 2^-8 |ref| + 2^-20 (|k0 x_t| + |k1 x_{t-1}|); the identity and shift
kernels are bit-exact.  Inputs are seeded and synthetic."""
import numpy as np
import pytest
import torch

import block_drafting_context_amd as dfl
import oracle
from block_drafting_context_amd import synthetic as syn
from parity_util import cuda, to64


def _run(x, k):
    y = dfl.dflash_two_tap_conv(x.to(cuda()), k.to(cuda()))
    torch.cuda.synchronize()
    return to64(y)


def _check(B, G, D, ng, seed):
    print(f"[conv] B={B} G={G} D={D} groups={ng}", flush=True)
    x = syn.normal((B, G, D), seed, "x", dtype=torch.bfloat16)
    k = syn.normal((B, G, 2, ng), seed, "k")
    got = _run(x, k)
    xs, ks = to64(x), to64(k)
    ref = oracle.two_tap_conv(xs, ks)
    gs = D // ng
    k0 = np.repeat(ks[:, :, 0, :], gs, axis=2)
    k1 = np.repeat(ks[:, :, 1, :], gs, axis=2)
    prev = np.concatenate([np.zeros_like(xs[:, :1]), xs[:, :-1]], axis=1)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -20 * (np.abs(k0 * xs) + np.abs(k1 * prev))
    err = np.abs(got - ref)
    assert (err <= bound).all(), float((err - bound).max())


@pytest.mark.gpu
def test_conv_serving_shape():
    """32 sequences, blocks of 8, width 5120, 80 groups of 64 channels."""
    _check(32, 8, 5120, 80, seed=31)


@pytest.mark.gpu
@pytest.mark.parametrize("B,G,D,ng", [(3, 1, 256, 1), (5, 16, 512, 64), (1, 8, 128, 16), (7, 3, 5120, 1),
                                      (2, 32, 8, 1), (2, 8, 16384, 2048)])
def test_conv_edges(B, G, D, ng):
    """A block of one (the anchor alone), groups of 8 channels, one group, the
    narrowest width (8 channels) over a block of 32, and 2,048 groups of 8."""
    _check(B, G, D, ng, seed=32 + G)


@pytest.mark.gpu
def test_conv_identity_and_shift_are_exact():
    B, G, D, ng = 4, 8, 1024, 16
    x = syn.normal((B, G, D), 33, "x", dtype=torch.bfloat16)
    ident = torch.zeros((B, G, 2, ng))
    ident[:, :, 0] = 1.0
    assert np.array_equal(_run(x, ident), to64(x))
    shift = torch.zeros((B, G, 2, ng))
    shift[:, :, 1] = 1.0
    y = _run(x, shift)
    assert np.array_equal(y[:, 1:], to64(x)[:, :-1])
    assert not y[:, 0].any()
