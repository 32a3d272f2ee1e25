"""The library's calls are not graph-capture safe, and say so instead of
recording work into a graph: the C ABI returns NVFP4_ERR_CAPTURE for a stream
that is being captured (before it launches anything), and the binding raises
before it allocates a per-call workspace.  Nothing is replayed here."""
import ctypes

import numpy as np
import pytest
import torch

from dit_quantization_amd import nvfp4 as nv
from tests.gpu_helpers import DEV, host

pytestmark = pytest.mark.gpu


def test_calls_refuse_a_capturing_stream():
    codes = torch.zeros((4, 32), dtype=torch.uint8, device=DEV)
    scales = torch.full((4, 4), 0x38, dtype=torch.uint8, device=DEV)
    sg = torch.ones(1, dtype=torch.float32, device=DEV)
    out = torch.full((4, 64), 7.0, dtype=torch.float32, device=DEV)
    marker = torch.zeros(1, dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    statuses = []
    with torch.cuda.graph(g, stream=side):
        marker.add_(1.0)                               # one node, so the graph is not empty
        with pytest.raises(RuntimeError, match="not graph-capture safe"):
            nv.dequant(codes, scales, sg, out=out)
        st = nv.lib().nvfp4_dequant(ctypes.c_void_p(codes.data_ptr()), ctypes.c_void_p(scales.data_ptr()),
                                    ctypes.c_void_p(sg.data_ptr()), 4, 64, ctypes.c_void_p(out.data_ptr()),
                                    nv.F32, ctypes.c_void_p(side.cuda_stream))
        statuses.append(st)
    torch.cuda.synchronize()
    assert statuses == [nv.ERR_CAPTURE]
    assert np.all(host(out) == 7.0)                    # nothing ran
    # the same call outside capture works
    nv.dequant(codes, scales, sg, out=out)
    assert np.all(host(out) == 0.0)
