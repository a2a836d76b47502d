"""The device form of the seeded weight generator (synth_inputs/synth_gpu.hip) draws the bytes that
synth.c draws: compared element by element on rows of every workload's matrices (bf16 and fp32,
Gaussian and Student-t, with and without outlier columns), including the first and last rows."""
import numpy as np
import pytest
import torch

from helpers import DEV, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg_i,sel", [(0, 0), (1, 0), (2, 0), (2, 1), (3, 4), (3, 6), (4, 7 * 39 + 6)])
def test_device_draw_equals_host_draw(synth, cfg_i, sel):
    spec = synth.config(cfg_i).matrices[sel]
    log("synth %s %dx%d" % (spec.name, spec.d_out, spec.d_in))
    for row0, n in ((0, 7), (spec.d_out // 2 + 3, 5), (spec.d_out - 6, 6)):
        host = spec.weights(row0, n)
        dev = spec.weights_device(DEV, row0, n)
        torch.cuda.synchronize()
        got = dev.view(torch.int16).cpu().numpy().view(np.uint16) if spec.bf16 else dev.cpu().numpy()
        np.testing.assert_array_equal(got, host)
