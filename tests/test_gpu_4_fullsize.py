"""Parity at the benchmark sizes, in the launch configuration bench.py times.

Every unit's decisions and coreset are checked, and every output row: the
oracle forms a unit's (unmasked) or an Express block's (causal) outputs
together from the replayed coreset.  The approximation error against exact
attention is taken on sampled queries (exact fp64 attention of every row of
the causal prefill would be 8.8 TFLOP), always including the first and last
token of the first and last unit.
"""

import pytest
import torch

from sub_quadratic_attention_amd import inputs
from tests.parity import run_and_compare, sample_queries

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_quadratic_attention_amd import binding
    binding.load_library()


def test_vit_token_mixing_full():
    d = inputs.vit_token_mixing(seed=0)
    qs = sample_queries(64, 3136, 1, 600, seed=1, always=[(0, 0, 0), (63, 3135, 0)])
    s = run_and_compare("vit B=64 S=3136", d, False, 1, 1, 64, 64, block_outputs=True, error_queries=qs)
    assert s["decisions"] == 175616


def test_biggan_self_attention_full():
    d = inputs.biggan_self_attention(seed=0)
    qs = sample_queries(32, 4096, 1, 600, seed=2, always=[(0, 0, 0), (31, 4095, 0)])
    s = run_and_compare("biggan B=32 S=4096", d, False, 1, 1, 64, 256, block_outputs=True, error_queries=qs)
    assert s["decisions"] == 129024


def test_causal_prefill_full():
    d = inputs.causal_prefill(seed=0)
    qs = sample_queries(1, 32768, 32, 800, seed=3, always=[(0, 0, 0), (0, 32767, 31), (0, 1023, 5), (0, 1024, 5)])
    s = run_and_compare("causal prefill H=32 S=32768", d, True, 32, 32, 128, 128, block_outputs=True,
                        error_queries=qs)
    assert s["decisions"] == 131072


def test_unmasked_small_full_config():
    d = inputs.unmasked_small(seed=0)
    s = run_and_compare("unmasked small", d, False, 1, 1, 64, 64)
    assert s["decisions"] == 240


def test_vit_token_mixing_subsampled_full():
    """The ViT layer under the sqrt(S) size rule: base subsampling (one point per 7), then the
    Compress of 448 points per unit, 56 coreset points of weight 56."""
    d = inputs.vit_token_mixing(seed=0)
    qs = sample_queries(64, 3136, 1, 600, seed=4, always=[(0, 0, 0), (63, 3135, 0)])
    s = run_and_compare("vit subsampled B=64 S=3136", d, False, 1, 1, 64, 64, subsample_base=True,
                        block_outputs=True, error_queries=qs)
    assert s["decisions"] == 64 * 392 and s["idx"].shape[1] == 56
