"""GPU parity over a seeded sweep of shapes that nobody picked by hand.

Each case draws its sizes (N 1..1400, D a multiple of 8 up to 768, V 1..6000), dtype,
label distribution, ignored fraction, upstream gradient and workspace sizes from one fixed
seed, and checks against one fp64 oracle evaluation:

* the two calls with the default workspace;
* the backward again with a workspace drawn between the least one the backward accepts
  and the default, so the token and vocabulary chunking varies from case to case (dH
  accumulated over vocabulary chunks, dW over token chunks);
* the one-call entry point with a workspace drawn between the recomputing schedule's and
  three times the single pass's, so it runs the single pass with a varying token chunk,
  or falls back to the two calls.

Tolerances are those of the hand-picked parity cases (tests/flce_run.py).
"""
import numpy as np
import pytest
import torch

import oracle
from linear_cross_entropy_lm_amd import inputs as I
from flce_run import compare

pytestmark = pytest.mark.gpu

SWEEP_SEED = 91_357
N_CASES = 18
_TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _draw_cases():
    rng = np.random.default_rng(SWEEP_SEED)
    cases = []
    for i in range(N_CASES):
        dtype = ("bf16", "f16", "f32")[i % 3]
        N = int(rng.integers(1, 1401))
        D = 8 * int(rng.integers(1, 97))
        V = int(rng.integers(1, 6001))
        kw = dict(ignore_frac=float(rng.choice([0.0, 0.05, 0.3])),
                  ignore_layout=str(rng.choice(["random", "tail"])),
                  label_dist=str(rng.choice(["uniform", "zipf"])))
        g = [None, 0.37, 3.0][int(rng.integers(0, 3))]
        u_bwd, u_one = float(rng.random()), float(rng.random())
        cfg = I.case(N, D, V, dtype, seed=5000 + i, **kw)
        cases.append((f"sweep{i:02d}_{dtype}_N{N}_D{D}_V{V}", cfg, g, u_bwd, u_one))
    return cases


CASES = _draw_cases()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_cross_entropy_lm_amd import binding  # noqa: F401  (fails loudly if not built)


def _least_backward_workspace(B, N, D, V, tdt, hi):
    """The smallest workspace flce_backward_chunks accepts (bisection; it accepts every
    size above its least one)."""
    lo = 0
    while hi - lo > 256:
        mid = (lo + hi) // 2
        try:
            B.flce_backward_chunks(N, D, V, tdt, mid)
            hi = mid
        except B.FlceError:
            lo = mid
    return hi


def _forward(B, H, W, y, ws):
    N, dev = H.shape[0], H.device
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    nv = torch.empty(1, dtype=torch.int32, device=dev)
    st = torch.full((1,), -7, dtype=torch.int32, device=dev)
    B.flce_forward(H, W, y, loss, lse, nv, st, ws)
    return loss, lse, nv, st


def _host(loss, lse, nv, st, dH, dW):
    torch.cuda.synchronize()
    return dict(loss=float(loss.item()), lse=lse.cpu().double().numpy(), n_valid=int(nv.item()),
                status=int(st.item()), dH=dH.float().cpu().double().numpy(), dW=dW.cpu().double().numpy())


@pytest.mark.parametrize("name,cfg,g,u_bwd,u_one", CASES, ids=[c[0] for c in CASES])
def test_sweep_parity(name, cfg, g, u_bwd, u_one):
    from linear_cross_entropy_lm_amd import binding as B
    print("case", name, cfg.describe(), "g", g, flush=True)
    inp = I.generate(cfg)
    ref = oracle.forward_backward(inp.h64(), inp.w64(), inp.y64(), g=1.0 if g is None else g)
    H, W, y = inp.device_tensors("cuda:0")
    N, D, V, tdt, dev = cfg.N, cfg.D, cfg.V, _TORCH[cfg.dtype], H.device
    gl = None if g is None else torch.tensor([g], dtype=torch.float32, device=dev)

    # two calls, default workspace; then the backward with a drawn, smaller workspace
    full = B.flce_workspace_bytes(N, D, V, tdt)
    ws_full = torch.empty(full, dtype=torch.uint8, device=dev)
    loss, lse, nv, st = _forward(B, H, W, y, ws_full)
    least = _least_backward_workspace(B, N, D, V, tdt, full)
    ws_bytes = {"default": full, "drawn": least + int(u_bwd * (full - least))}
    for label, nbytes in ws_bytes.items():
        tc, vc = B.flce_backward_chunks(N, D, V, tdt, nbytes)
        print(f"  backward, {label} workspace {nbytes}: chunks {tc} x {vc}", flush=True)
        ws = ws_full if nbytes == full else torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dH = torch.full_like(H, float("nan"))
        dW = torch.full((V, D), float("nan"), dtype=torch.float32, device=dev)
        B.flce_backward(H, W, y, lse, nv, gl, dH, dW, ws)
        got = _host(loss, lse, nv, st, dH, dW)
        assert got["status"] == 0
        print("  errors", compare(got, ref, cfg.dtype), flush=True)

    # one call: single pass with a drawn token chunk, or the fallback below its workspace
    sp = B.flce_forward_backward_workspace_bytes(N, D, V, tdt)
    lo, hi = min(full, sp), 3 * sp
    nbytes = lo + int(u_one * (hi - lo))
    tc = B.flce_forward_backward_chunk(N, D, V, tdt, nbytes)
    print(f"  one call, workspace {nbytes}: token chunk {tc} (0: two calls)", flush=True)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    loss1 = torch.empty(1, dtype=torch.float32, device=dev)
    lse1 = torch.empty(N, dtype=torch.float32, device=dev)
    nv1 = torch.empty(1, dtype=torch.int32, device=dev)
    st1 = torch.full((1,), -7, dtype=torch.int32, device=dev)
    dH = torch.full_like(H, float("nan"))
    dW = torch.full((V, D), float("nan"), dtype=torch.float32, device=dev)
    B.flce_forward_backward(H, W, y, gl, loss1, lse1, nv1, st1, dH, dW, ws)
    got = _host(loss1, lse1, nv1, st1, dH, dW)
    assert got["status"] == 0
    print("  errors", compare(got, ref, cfg.dtype), flush=True)
