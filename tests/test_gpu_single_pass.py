"""GPU parity of flce_forward_backward (include/flce.h), the forward and backward in one
call, against the fp64 oracle: the single-pass schedule (workspace of
flce_forward_backward_workspace_bytes) on small ragged cases, several token chunks with a
short last one, every dtype, an upstream gradient and a custom ignore_index, and the
Llama-3-shaped full size; and the fallback schedule (a smaller workspace), which must
equal separate flce_forward + flce_backward calls bit for bit.

Tolerances are the fused path's (tests/flce_run.py): the single pass rounds p~ = exp(z - m)
to the input type and then rounds dz once more, one extra rounding of the same size as
the slab's own.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from linear_cross_entropy_lm_amd import inputs as I
from flce_run import compare, compare_golden, run_gpu

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_cross_entropy_lm_amd import binding  # noqa: F401  (fails loudly if not built)


def run_fb(inp, g=None, ignore_index=-100, single=True, ws_factor=1.0, device="cuda:0") -> dict:
    from linear_cross_entropy_lm_amd import binding as B
    H, W, y = inp.device_tensors(device)
    N, D = H.shape
    V = W.shape[0]
    sp_bytes = B.flce_forward_backward_workspace_bytes(N, D, V, H.dtype)
    two_bytes = B.flce_workspace_bytes(N, D, V, H.dtype)
    if not single:
        # the fallback needs a workspace that fits the two calls but not the single pass
        assert two_bytes < sp_bytes, (two_bytes, sp_bytes)
    ws = torch.empty(int(sp_bytes * ws_factor) if single else two_bytes, dtype=torch.uint8, device=device)
    loss = torch.empty(1, dtype=torch.float32, device=device)
    lse = torch.empty(N, dtype=torch.float32, device=device)
    nv = torch.empty(1, dtype=torch.int32, device=device)
    st = torch.full((1,), -7, dtype=torch.int32, device=device)
    dH = torch.full_like(H, float("nan"))
    dW = torch.full((V, D), float("nan"), dtype=torch.float32, device=device)
    gl = None if g is None else torch.tensor([g], dtype=torch.float32, device=device)
    B.flce_forward_backward(H, W, y, gl, loss, lse, nv, st, dH, dW, ws, ignore_index)
    torch.cuda.synchronize()
    return dict(loss=float(loss.item()), lse=lse.cpu().double().numpy(), n_valid=int(nv.item()),
                status=int(st.item()), dH=dH.float().cpu().double().numpy(), dW=dW.cpu().double().numpy())


CASES = [
    ("tiny_f32", None),
    ("ragged_bf16", I.case(300, 512, 1031, "bf16", seed=71)),
    ("ragged_f32", I.case(300, 512, 1031, "f32", seed=72)),
    ("ragged_f16", I.case(300, 512, 1031, "f16", seed=73)),
    ("raggedD_bf16", I.case(513, 264, 2500, "bf16", seed=74, ignore_frac=0.2)),
    ("zipf_bf16", I.case(640, 256, 4099, "bf16", seed=75, label_dist="zipf")),
    # two token chunks (4096 + 404 rows: the short one runs with more vocabulary splits)
    ("two_chunks_bf16", I.case(4500, 256, 3000, "bf16", seed=76)),
    ("two_chunks_f16", I.case(4500, 256, 3000, "f16", seed=77)),
    ("V1_f32", I.case(65, 128, 1, "f32", seed=78, ignore_frac=0.0)),
    ("V1_bf16", I.case(65, 128, 1, "bf16", seed=79, ignore_frac=0.0)),
    ("N1_D64_f16", I.case(1, 64, 300, "f16", seed=80, ignore_frac=0.0)),
    ("D8_bf16", I.case(257, 8, 1031, "bf16", seed=84)),
    ("D8200_bf16", I.case(300, 8200, 1031, "bf16", seed=85)),
]


@pytest.mark.parametrize("name,cfg", CASES, ids=[c[0] for c in CASES])
def test_single_pass_parity(name, cfg):
    cfg = cfg or I.CONFIGS[name]
    print("case", cfg.describe(), flush=True)
    inp = I.generate(cfg)
    # fp16 runs with a loss scale, as fp16 training does: at g = 1 and N_valid in the
    # thousands, dH entries fall below fp16's smallest normal
    g = 1024.0 if cfg.dtype == "f16" else None
    got = run_fb(inp, g=g)
    ref = oracle.forward_backward(inp.h64(), inp.w64(), inp.y64(), g=g or 1.0)
    err = compare(got, ref, cfg.dtype)
    assert got["status"] == 0
    print("errors", err, flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_single_pass_one_chunk(dtype):
    """A workspace 1.2x the least: the 4500 rows fit one chunk of 4608 (dW written once,
    never read back)."""
    cfg = I.case(4500, 256, 3000, dtype, seed=83)
    inp = I.generate(cfg)
    g = 1024.0 if dtype == "f16" else None
    got = run_fb(inp, g=g, ws_factor=1.2)
    ref = oracle.forward_backward(inp.h64(), inp.w64(), inp.y64(), g=g or 1.0)
    compare(got, ref, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_pass_grad_and_ignore_index(dtype):
    cfg = I.case(400, 256, 900, dtype, seed=79, ignore_frac=0.0)
    inp = I.generate(cfg)
    y = inp.y.clone()
    y[::6] = 11
    inp = I.Inputs(cfg, inp.H, inp.W, y)
    got = run_fb(inp, g=-2.5, ignore_index=11)
    ref = oracle.forward_backward(inp.h64(), inp.w64(), inp.y64(), ignore_index=11, g=-2.5)
    compare(got, ref, dtype)


def test_single_pass_all_rows_ignored():
    cfg = I.case(300, 256, 1000, "bf16", seed=80)
    inp = I.generate(cfg)
    inp = I.Inputs(cfg, inp.H, inp.W, torch.full((300,), -100, dtype=torch.int64))
    got = run_fb(inp)
    assert got["n_valid"] == 0 and got["loss"] == 0.0
    assert np.all(got["dH"] == 0.0) and np.all(got["dW"] == 0.0)


def test_single_pass_bitwise_deterministic():
    inp = I.generate(I.case(4500, 256, 3000, "bf16", seed=81))
    a, b = run_fb(inp), run_fb(inp)
    for k in ("loss", "lse", "dH", "dW"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fallback_equals_forward_then_backward(dtype):
    """A workspace too small for the single pass runs the two-call schedule: identical bits.
    (V > 8192, so the two-call workspace, with its 8192-wide vocabulary chunks, is the
    smaller one.)"""
    inp = I.generate(I.case(700, 256, 20000, dtype, seed=82))
    a = run_fb(inp, g=0.75, single=False)
    b = run_gpu(inp, g=0.75)
    for k in ("loss", "lse", "dH", "dW"):
        assert np.array_equal(np.asarray(a[k]), np.asarray(b[k])), k


@pytest.mark.parametrize("name,ws_factor", [("llama3", 1.0), ("llama3", 2.0), ("llama3_f16", 1.0)])
def test_single_pass_fullsize_llama3(name, ws_factor):
    """16384 x 4096 x 128256 in one call (four token chunks of 4096, or two of 8192 with
    twice the workspace), bf16 and fp16: loss, every row's lse, dH and dW on the sampled rows
    against the stored oracle run, and the properties that hold at any size on the whole
    output.  fp16 runs with a loss scale of 1024 (dH entries at g = 1 fall below fp16's
    normal range) and divides it out, which is exact."""
    from linear_cross_entropy_lm_amd import binding as B
    cfg = I.CONFIGS[name]
    print("case", cfg.describe(), "workspace factor", ws_factor, flush=True)
    gold = np.load(os.path.join(GOLDEN, f"fullsize_{name}.npz"))
    inp = I.generate(cfg)
    assert inp.digest() == str(gold["digest"]), "seeded inputs differ from the stored oracle run"
    dev = "cuda:0"
    H, W, y = inp.device_tensors(dev)
    N, D, V = cfg.N, cfg.D, cfg.V
    ws = torch.empty(int(B.flce_forward_backward_workspace_bytes(N, D, V, H.dtype) * ws_factor), dtype=torch.uint8,
                     device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    nv = torch.empty(1, dtype=torch.int32, device=dev)
    st = torch.empty(1, dtype=torch.int32, device=dev)
    dH = torch.full_like(H, float("nan"))
    dW = torch.full((V, D), float("nan"), dtype=torch.float32, device=dev)
    scale = 1024.0 if cfg.dtype == "f16" else 1.0
    g = None if scale == 1.0 else torch.tensor([scale], dtype=torch.float32, device=dev)
    B.flce_forward_backward(H, W, y, g, loss, lse, nv, st, dH, dW, ws)
    torch.cuda.synchronize()
    if scale != 1.0:
        dH = dH.float() / scale
        dW = dW / scale
    assert int(st.item()) == 0 and int(nv.item()) == int(gold["n_valid"])
    err = compare_golden(gold, loss, lse, dH, dW, cfg.dtype)
    print(f"loss {loss.item():.6f} (oracle {float(gold['loss']):.6f}); errors {err}", flush=True)
    assert bool(torch.isfinite(dW).all()) and bool(torch.isfinite(dH.float()).all())
    assert bool((dH[y == -100] == 0).all())
    colsum = dW.double().sum(dim=0).norm().item()
    assert colsum <= 1e-2 * dW.double().norm().item()
    lhs = (dW.double() * W.double()).sum().item()
    rhs = (dH.double() * H.double()).sum().item()
    assert abs(lhs - rhs) <= 1e-2 * abs(lhs)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_single_pass_labels_in_the_last_partial_vocab_tile(dtype):
    """As the two-call case: every label in the last seven rows of a 1031-row vocabulary."""
    cfg = I.case(300, 256, 1031, dtype, seed=81, ignore_frac=0.0)
    inp0 = I.generate(cfg)
    y = 1024 + torch.arange(300, dtype=torch.int64) % 7
    y[::11] = -100
    inp = I.with_labels(inp0, y)
    g = 1024.0 if dtype == "f16" else None
    got = run_fb(inp, g=g)
    ref = oracle.forward_backward(inp.h64(), inp.w64(), inp.y64(), g=g or 1.0)
    assert got["status"] == 0
    compare(got, ref, dtype)


def test_single_pass_capped_chunk():
    """16640 rows at the Qwen-2.5 vocabulary (V = 152064, D = 64, bf16) with a workspace
    that holds one chunk of every row: such a chunk's kept slab, read transposed by the dW
    contraction, would span 16640 x 304128 bytes (5.06e9), past the kernels' 32-bit buffer
    offsets.  The call caps the chunk (4096 rows: five chunks, the last of 256) and must
    match the stored oracle run on the loss, every lse, and dH and dW rows at every tile
    edge."""
    from linear_cross_entropy_lm_amd import binding as B
    name = "spcap_bf16"
    cfg = I.GOLDEN_CASES[name]
    print("case", cfg.describe(), flush=True)
    gold = np.load(os.path.join(GOLDEN, f"fullsize_{name}.npz"))
    inp = I.generate(cfg)
    assert inp.digest() == str(gold["digest"]), "seeded inputs differ from the stored oracle run"
    dev = "cuda:0"
    H, W, y = inp.device_tensors(dev)
    N, D, V = cfg.N, cfg.D, cfg.V
    ws_bytes = 6 * 10**9
    assert N * 304128 > 2**32  # one chunk of all rows would have wrapped 32-bit offsets
    assert B.flce_forward_backward_chunk(N, D, V, H.dtype, ws_bytes) == 4096
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    nv = torch.empty(1, dtype=torch.int32, device=dev)
    st = torch.empty(1, dtype=torch.int32, device=dev)
    dH = torch.full_like(H, float("nan"))
    dW = torch.full((V, D), float("nan"), dtype=torch.float32, device=dev)
    B.flce_forward_backward(H, W, y, None, loss, lse, nv, st, dH, dW, ws)
    torch.cuda.synchronize()
    del ws
    assert int(st.item()) == 0 and int(nv.item()) == int(gold["n_valid"])
    err = compare_golden(gold, loss, lse, dH, dW, cfg.dtype)
    print(f"loss {loss.item():.6f} (oracle {float(gold['loss']):.6f}); errors {err}", flush=True)
    assert bool(torch.isfinite(dW).all()) and bool(torch.isfinite(dH.float()).all())
    assert bool((dH[y == -100] == 0).all())
    lhs = (dW.double() * W.double()).sum().item()
    rhs = (dH.double() * H.double()).sum().item()
    assert abs(lhs - rhs) <= 1e-2 * abs(lhs)
    torch.cuda.empty_cache()
