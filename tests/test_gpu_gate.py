"""The support gate on gfx950: 1 for every shape the header lists as
supported, 0 for the rest (the same lists the CPU test checks answer 0
everywhere when no gfx950 is present)."""

from __future__ import annotations

import pytest
import torch

from tests.gpu_util import lib, say
from tests.test_abi import GATE_SUPPORTED, GATE_UNSUPPORTED

pytestmark = pytest.mark.gpu


def test_gate_on_gfx950():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    assert torch.cuda.get_device_properties(0).gcnArchName.startswith("gfx950")
    L = lib()
    say("gate: %d supported, %d unsupported shapes" % (len(GATE_SUPPORTED), len(GATE_UNSUPPORTED)))
    for h, d, bs in GATE_SUPPORTED:
        assert L.mqa_is_supported(h, d, bs) == 1, (h, d, bs)
    for h, d, bs in GATE_UNSUPPORTED:
        assert L.mqa_is_supported(h, d, bs) == 0, (h, d, bs)
