"""The entry point that allocates nothing: spel_step_static (for callers
that cannot allocate, such as code under HIP graph capture) takes its
workspace from the library's static device array.  It runs the same kernels
as spel_step with a caller workspace, so it must give the same bits; checked
on two calls in a row, the second with a smaller projector (the array keeps
the first call's contents, including the Gram-space iteration's arrival
flags, which the step must clear itself), and against the fp64 oracle of
Section 3.3, Eq. (4)-(7)."""
import numpy as np
import pytest
import torch

import learned_activation_compression_amd as lac
import synth
from oracle import spel
from parity_util import F32_TOL, assert_close, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def step_both(seed, d, r):
    inp = synth.spel_inputs(seed, d, r, 1e-3)
    m0 = torch.from_numpy(synth.gaussian(synth.stream(seed, d, r), (d, r), 1e-4).astype(np.float32))
    g = inp["g"].to(DEV)
    out = []
    for fn in ("spel_step", "spel_step_static"):
        A, m = inp["A"].clone().to(DEV), m0.clone().to(DEV)
        D = torch.empty_like(A)
        st = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        if fn == "spel_step":
            lac.spel_step(A, g, m, 1e-3, 0.9, 8, D_out=D, status=st)
        else:
            lac.spel_step_static(A, g, m, 1e-3, 0.9, 8, D_out=D, status=st)
        out.append((A, m, D, st))
    torch.cuda.synchronize()
    (A1, m1, D1, s1), (A2, m2, D2, s2) = out
    assert int(s1.item()) == 0 and int(s2.item()) == 0
    assert torch.equal(A1, A2) and torch.equal(m1, m2) and torch.equal(D1, D2)
    An, mn, Dn, _ = spel.spel_step(np64(inp["A"]), np64(inp["g"]), np64(m0), 1e-3, 0.9, 8)
    assert_close(np64(A2), An, F32_TOL, "A")
    assert_close(np64(m2), mn, F32_TOL, "m")
    assert_close(np64(D2), Dn, F32_TOL, "D")


def test_static_scratch_matches_the_caller_workspace_on_consecutive_calls():
    step_both(71, 2048, 256)   # the d x r form; 9.75 MiB of the 16 MiB scratch
    step_both(72, 1024, 128)   # smaller, the Gram-space form with its flags in the scratch
    step_both(73, 1024, 128)   # again: the flags left by the previous call are cleared first


def test_static_scratch_rejects_shapes_beyond_its_size():
    d, r = 4096, 256
    assert lac.spel_workspace_bytes(d, r) > (16 << 20)
    A = torch.zeros((d, r), dtype=torch.float32, device=DEV)
    with pytest.raises(lac.MaplError) as e:
        lac.spel_step_static(A, A.clone(), A.clone(), 1e-3, 0.9, 8)
    assert e.value.status == -5
