"""flce_forward_backward_static (include/flce.h), the entry point for callers that cannot
allocate, against flce_forward_backward with a caller workspace of the same
FLCE_STATIC_SCRATCH_BYTES: the same schedule and chunking, so the same bits, and the oracle's
tolerances.  Two calls in a row, the second with a smaller input (the array keeps the first
call's contents), with device free memory unchanged across them.  No kernel uses private
(scratch) memory (tests/test_kernel_resources.py), so no dispatch makes the runtime allocate."""
import numpy as np
import pytest
import torch

import oracle
from linear_cross_entropy_lm_amd import inputs as I
from flce_run import compare

pytestmark = pytest.mark.gpu


def _outputs(H, W, dev):
    N, D = H.shape
    V = W.shape[0]
    return dict(loss=torch.empty(1, dtype=torch.float32, device=dev),
                lse=torch.empty(N, dtype=torch.float32, device=dev),
                nv=torch.empty(1, dtype=torch.int32, device=dev),
                st=torch.full((1,), -7, dtype=torch.int32, device=dev),
                dH=torch.full_like(H, float("nan")),
                dW=torch.full((V, D), float("nan"), dtype=torch.float32, device=dev))


def _host(o):
    """Host copies (converted on the host: no device memory is allocated)."""
    return dict(loss=float(o["loss"].item()), lse=o["lse"].cpu().double().numpy(), n_valid=int(o["nv"].item()),
                status=int(o["st"].item()), dH=o["dH"].cpu().float().double().numpy(),
                dW=o["dW"].cpu().double().numpy())


def test_static_scratch_matches_workspace_call():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_cross_entropy_lm_amd import binding as B
    dev = "cuda:0"
    cfgs = [I.case(4500, 512, 20000, "bf16", seed=91),   # recomputing schedule: 2 token x 3 vocabulary chunks
            I.case(700, 256, 3000, "bf16", seed=92)]     # smaller, and the single pass fits the array
    cases = []
    for cfg in cfgs:
        inp = I.generate(cfg)
        H, W, y = inp.device_tensors(dev)
        cases.append((cfg, inp, H, W, y, _outputs(H, W, dev), _outputs(H, W, dev)))
    g = torch.tensor([0.5], dtype=torch.float32, device=dev)
    ws = torch.empty(B.FLCE_STATIC_SCRATCH_BYTES, dtype=torch.uint8, device=dev)
    print("schedules (token chunk, 0 = recomputing):",
          [B.flce_forward_backward_chunk(c.N, c.D, c.V, torch.bfloat16, B.FLCE_STATIC_SCRATCH_BYTES) for c in cfgs],
          flush=True)

    def static(c):
        _, _, H, W, y, a, _ = c
        B.flce_forward_backward_static(H, W, y, g, a["loss"], a["lse"], a["nv"], a["st"], a["dH"], a["dW"])

    def with_ws(c):
        _, _, H, W, y, _, b = c
        B.flce_forward_backward(H, W, y, g, b["loss"], b["lse"], b["nv"], b["st"], b["dH"], b["dW"], ws)

    # warm-up: the first call on the device looks up the array and may load the code object
    static(cases[0])
    with_ws(cases[0])
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info(0)[0]
    for c in cases:  # the larger input, then the smaller one
        cfg, inp = c[0], c[1]
        print("case", cfg.describe(), flush=True)
        static(c)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info(0)[0] == free0, "device memory changed across the static call"
        with_ws(c)
        torch.cuda.synchronize()
        ha, hb = _host(c[5]), _host(c[6])
        assert ha["status"] == 0 and hb["status"] == 0
        for k in ("loss", "lse", "n_valid", "dH", "dW"):
            assert np.array_equal(np.asarray(ha[k]), np.asarray(hb[k])), k
        ref = oracle.forward_backward(inp.h64(), inp.w64(), inp.y64(), g=0.5)
        print("errors", compare(ha, ref, cfg.dtype), flush=True)
    assert torch.cuda.mem_get_info(0)[0] == free0
