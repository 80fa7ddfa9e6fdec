"""The measurement probes' C ABI without a GPU: every symbol of include/muonbank_probes.h is exported and
bound, and every argument error returns before a launch."""

import os
import re

import pytest

from newton_schulz_bank_amd import api, probes
from tests.conftest import ROOT

NULL, SHAPE, ALIGN, ALIAS = 1, 2, 4, 6


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(api.LIB_PATH):
        from newton_schulz_bank_amd import build
        build.build()
    return probes._lib()


def test_every_declared_probe_is_exported(L):
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "muonbank_probes.h")).read(), flags=re.S)
    names = set(re.findall(r"^\s*mb_status\s+(\w+)\s*\(", text, flags=re.M))
    assert names == set(probes.EXPORTED)
    for n in names:
        assert hasattr(L, n)


def test_probe_argument_errors(L):
    p = 1 << 36
    assert L.mb_probe_mfma_bf16(16, 4, None, None) == NULL
    assert L.mb_probe_mfma_bf16(0, 4, p, None) == SHAPE
    assert L.mb_probe_mfma_bf16(16, 0, p, None) == SHAPE
    assert L.mb_probe_mfma_bf16(16, 70000, p, None) == SHAPE
    assert L.mb_probe_mfma_bf16(16, 4, p + 4, None) == ALIGN
    assert L.mb_probe_copy(None, p, 1024, None) == NULL
    assert L.mb_probe_copy(p, p + 4096, 0, None) == SHAPE
    assert L.mb_probe_copy(p, p + 4096, 1000, None) == SHAPE
    assert L.mb_probe_copy(p + 8, p + 4096, 1024, None) == ALIGN
    assert L.mb_probe_copy(p, p + 512, 1024, None) == ALIAS


def test_flop_count_of_the_mfma_probe():
    # workgroups x 4 wavefronts x iterations x 4 chains x one 32x32x16 product (2*32*32*16 flops)
    assert probes.mfma_flops(10, 3) == 3 * 4 * 10 * 4 * 32768
