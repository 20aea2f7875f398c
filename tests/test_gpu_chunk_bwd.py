"""GPU parity of the chunkwise backward pass (lion_attn_chunk_bwd) against the fp64 backward oracle
(marked gpu).

The chunkwise backward computes the same gradients as the full form's backward, so it is held to the
same reference (``oracle.full_bwd``, pinned by finite differences of the forward definition) and the
same condition-aware gate (``tests.test_gpu_bwd.run_case``).  The cases span one chunk, several chunks
with a ragged last one, every supported chunk size and head dimension, the causal variant (no states
entering from the right), signed inputs, one long sequence at the high-resolution length, and 256 (batch, head) pairs.
Chunks of 16 and 32 run on the fp32 matrix-core kernels, chunks of 64 and 128 on the bf16 ones.
"""
from __future__ import annotations

import pytest

from bidirectional_linear_attention_lion_amd import inputs as lin
from tests.test_gpu_bwd import run_case

pytestmark = pytest.mark.gpu

CASES_L = [1, 17, 64, 65, 100, 197, 300]


@pytest.mark.parametrize("kind", [lin.LIT, lin.D, lin.S])
@pytest.mark.parametrize("causal", [False, True])
def test_chunk_bwd_positive(kind, causal):
    for L in CASES_L:
        run_case(1, 2, L, 64, kind, causal=causal, seed=4000 + L, C=64)


@pytest.mark.parametrize("C", [16, 32, 128])
def test_chunk_bwd_chunk_sizes(C):
    for kind in (lin.LIT, lin.D, lin.S):
        run_case(1, 2, 150, 64, kind, seed=4100 + C, C=C)
        run_case(1, 2, 150, 64, kind, causal=True, seed=4150 + C, C=C)


@pytest.mark.parametrize("d,C", [(32, 64), (32, 128), (32, 16), (128, 64), (128, 32), (128, 16)])
def test_chunk_bwd_head_dims(d, C):
    for kind in (lin.LIT, lin.D, lin.S):
        run_case(1, 2, 150, d, kind, seed=4200 + d + C, C=C)


@pytest.mark.parametrize("kind", [lin.LIT, lin.D, lin.S])
def test_chunk_bwd_signed(kind):
    for L in (64, 197, 512):
        run_case(2, 3, L, 64, kind, positive=False, seed=4300 + L, C=64)
    run_case(1, 2, 300, 64, kind, causal=True, positive=False, seed=4399, C=64)


def test_chunk_bwd_long_sequence():
    # 65 chunks of 64 or 33 of 128 (the last one a single token): states carried across the whole length
    run_case(1, 1, 4097, 64, lin.D, positive=False, seed=4400, C=64)
    run_case(1, 1, 4097, 64, lin.S, seed=4401, C=64)
    run_case(1, 1, 4097, 64, lin.D, positive=False, seed=4402, C=128)
    run_case(1, 1, 4097, 64, lin.LIT, causal=True, seed=4403, C=128)


@pytest.mark.parametrize("kind", [lin.LIT, lin.D, lin.S])
@pytest.mark.parametrize("causal", [False, True])
def test_chunk_bwd_chunks_of_128(kind, causal):
    for L in (1, 17, 128, 129, 300, 640):
        run_case(1, 2, L, 64, kind, causal=causal, positive=L % 2 == 0, seed=4600 + L, C=128)


@pytest.mark.parametrize("kind", [lin.LIT, lin.D, lin.S])
def test_chunk_bwd_many_pairs(kind):
    # 256 (batch, head) pairs, 1024 walks and 1280 chunk workgroups in flight at once
    run_case(16, 16, 150, 64, kind, seed=4500, C=32)
    run_case(16, 16, 100, 64, kind, causal=True, positive=False, seed=4501, C=32)
    # the bf16 kernels: 3 and 2 chunks per pair, ragged last chunks
    run_case(16, 16, 150, 64, kind, positive=False, seed=4502, C=64)
    run_case(16, 16, 200, 64, kind, causal=True, seed=4503, C=128)


def test_chunk_bwd_bf16_small_heads_causal():
    # d = 32 on the bf16 kernels, causal, chunks of 64 and 128
    for kind in (lin.LIT, lin.D, lin.S):
        run_case(1, 2, 300, 32, kind, causal=True, positive=False, seed=4700 + kind, C=128)
        run_case(1, 2, 300, 32, kind, causal=True, seed=4710 + kind, C=64)
