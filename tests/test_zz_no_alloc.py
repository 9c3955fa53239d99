"""fp4q_quantize_noalloc (the entry point for callers that cannot allocate)
against fp4q_quantize with a caller-allocated workspace, through the C ABI:
byte-identical codes, scales and global scale, on two calls in a row per
rule, the second with a smaller input, so that the second call runs over the
scratch contents the first one left behind."""
import zlib

import numpy as np
import pytest
import torch

from block_scaled_fp4_fp4q_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_scaled_fp4_fp4q_amd import binding
    binding.lib()
    return binding


def to_dev(x):
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(x).to(DEV)


CASES = [
    # (format, rule, objective, rotate, bf16)
    ("nvfp4_sweep_mse_rot16", 0, 1, 0, 16, True),
    ("nvfp4_sweep_wmse", 0, 1, 1, 0, True),
    ("nvfp4_absmax_f32", 0, 0, 0, 0, False),
    ("if4", 2, 0, 0, 0, True),
    ("if4_sweep_rot16", 2, 1, 0, 16, False),
    ("nvfp4_four_over_six", 0, 2, 0, 0, True),
    ("mxfp4_rot32", 1, 0, 0, 32, True),
    ("if6_sweep", 4, 1, 0, 0, True),
    ("if3_wmse", 3, 0, 1, 16, False),
]


@pytest.mark.parametrize("name,fmt,rule,obj,rot,bf16", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_call(B, name, fmt, rule, obj, rot, bf16):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    # the second input is smaller, and its maximum is not the first's, so a
    # stale partial maximum left in the scratch would change the global scale
    for rows, cols, scale in ((3000, 512, 3.0), (257, 256, 0.25)):
        x = (rng.standard_normal((rows, cols)) * scale).astype(np.float32)
        x_h = synth.f32_to_bf16_bits(x) if bf16 else x
        xd = to_dev(x_h)
        imp = to_dev(rng.lognormal(0.0, 1.0, cols).astype(np.float32)) if obj else None
        spec = B.make_spec(fmt, rule, obj, rotate=rot)
        n = rows * cols
        outs = []
        for noalloc in (False, True):
            codes = torch.full((B.code_bytes(fmt, n),), 0xAB, dtype=torch.uint8, device=DEV)
            scales = torch.full((n // spec.block,), 0xCD, dtype=torch.uint8, device=DEV)
            gs = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
            if noalloc:
                B.fp4q_quantize_noalloc(spec, xd, imp, codes, scales, gs)
            else:
                ws = B.alloc_workspace(spec, rows, cols, DEV)
                B.fp4q_quantize(spec, xd, imp, codes, scales, gs, ws)
            torch.cuda.synchronize()
            outs.append((codes.cpu().numpy(), scales.cpu().numpy(), gs.cpu().numpy()))
        (c0, s0, g0), (c1, s1, g1) = outs
        assert np.array_equal(s0, s1), f"{name} {rows}x{cols}: scale bytes differ"
        assert np.array_equal(c0, c1), f"{name} {rows}x{cols}: codes differ"
        if fmt != 1:
            assert g0.view(np.uint32)[0] == g1.view(np.uint32)[0], f"{name}: global scale differs"
