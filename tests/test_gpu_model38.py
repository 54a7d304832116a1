"""Parity of the 38 CSA2 layers of one decode step: the encoder's 18 layers at
compression ratio 2 (three groups of Full + 5 Reuse over L/2 entries) and the
decoder's 20 (Full + 3 Reuse with the hierarchical candidate build, then four
groups of Reindex + 3 Reuse), each over its own caches, in the launch
configuration bench.py times.  Every layer's Top-512, candidate blocks and
output are checked against the oracle (indices bit-exact, outputs within
2e-3) on every row at reduced sizes and on sampled rows at full size."""
import pytest

from fp4_kv_cache_02_amd import synth
from tests.test_gpu_fullsize import run_fullsize

pytestmark = pytest.mark.gpu


def test_model38_reduced_all_rows():
    for w in synth.model_step(reduced=True):
        run_fullsize(w, list(range(w.R)))


def test_model38_fullsize_sampled_rows():
    for w in synth.model_step():
        run_fullsize(w, [0, w.R - 1])
