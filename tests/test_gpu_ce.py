"""GPU parity of the cross-entropy over materialised logits (include/flce_ce.h) against the
fp64 oracle (oracle.ce_from_logits), element by element, on seeded logits with ragged
row lengths, padded rows and the edge cases; plus the Llama-3-shaped full size.

Tolerances: loss relative 1e-5 and lse within 1e-5 * max(|lse|, 1) for every dtype (each
row's exponentials sum in fp32; inputs are identical on both sides); dZ Frobenius 1e-5 for fp32 output, 4e-3 for
bf16 (rounding, 2^-9) and 1e-3 for fp16 (2^-11).  fp16 cases run with a loss scale
g = 4096: at g = 1, dZ ~ p / N_valid falls below fp16's smallest normal.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from linear_cross_entropy_lm_amd import inputs as I
from flce_run import rel_fro

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL_GRAD = {"f32": 1e-5, "bf16": 4e-3, "f16": 1e-3}
G_DEFAULT = {"f32": 1.0, "bf16": 1.0, "f16": 4096.0}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_cross_entropy_lm_amd import binding  # noqa: F401  (fails loudly if not built)


def _say(*a):
    print(*a, flush=True)


def _pitch(V: int, dtype: str, extra: int = 0) -> int:
    """Smallest row pitch >= V + extra whose rows start 16-byte aligned."""
    k = 4 if dtype == "f32" else 8
    return -(-(V + extra) // k) * k


def run_ce(inp, g=None, ignore_index=-100, inplace=False, out_pad=False, device="cuda:0") -> dict:
    from linear_cross_entropy_lm_amd import binding as B
    Z, y = inp.device_tensors(device)
    N, V = Z.shape
    ws = torch.empty(B.flce_ce_workspace_bytes(N), dtype=torch.uint8, device=device)
    loss = torch.empty(1, dtype=torch.float32, device=device)
    lse = torch.empty(N, dtype=torch.float32, device=device)
    nv = torch.empty(1, dtype=torch.int32, device=device)
    st = torch.full((1,), -7, dtype=torch.int32, device=device)
    B.flce_ce_forward(Z, y, loss, lse, nv, st, ws, ignore_index)
    if inplace:
        dZbuf, dZ = None, Z
    else:
        P = _pitch(V, inp.cfg.dtype, 1 if out_pad else 0)
        dZbuf = torch.full((N, P), float("nan"), dtype=Z.dtype, device=device)
        dZ = dZbuf[:, :V]
    gl = None if g is None else torch.tensor([g], dtype=torch.float32, device=device)
    B.flce_ce_backward(Z, y, lse, nv, gl, dZ, ignore_index)
    torch.cuda.synchronize()
    out = dict(loss=float(loss.item()), lse=lse.cpu().double().numpy(), n_valid=int(nv.item()),
               status=int(st.item()), dZ=dZ.float().cpu().double().numpy())
    if dZbuf is not None and out_pad:
        out["pad"] = dZbuf[:, V:].float().cpu().numpy()
    return out


def check(got, inp, g, ignore_index=-100):
    ref = oracle.ce_from_logits(inp.z64(), inp.y64(), ignore_index=ignore_index, g=g)
    assert got["n_valid"] == ref["n_valid"]
    if ref["n_valid"]:
        assert abs(got["loss"] - ref["loss"]) <= 1e-5 * abs(ref["loss"])
    else:
        assert got["loss"] == 0.0
    # fp32 rounding of a log-sum-exp scales with its terms, not with lse itself, which can
    # sit near 0 for short rows: error relative to max(|lse|, 1)
    lse_abs = np.abs(got["lse"] - ref["lse"])
    lse_err = float(np.max(lse_abs / np.maximum(np.abs(ref["lse"]), 1.0)))
    assert lse_err <= 1e-5, (lse_err, float(lse_abs.max()))
    err = rel_fro(got["dZ"], ref["dZ"]) if np.linalg.norm(ref["dZ"]) > 0 else float(np.abs(got["dZ"]).max())
    assert err <= TOL_GRAD[inp.cfg.dtype], err
    _say("errors", dict(lse=lse_err, dZ=err))
    return ref


# Rows must start 16-byte aligned: ragged V comes with a padded pitch (pad columns hold
# 1e4, so a read past V would show in lse).
CASES = [
    ("ragged_f32", I.logit_case(300, 1031, "f32", seed=31, ld=1032)),
    ("ragged_bf16", I.logit_case(300, 1031, "bf16", seed=32, ld=1032)),
    ("ragged_f16", I.logit_case(300, 1031, "f16", seed=33, ld=1040)),
    ("contig_bf16", I.logit_case(257, 4096, "bf16", seed=34)),
    ("pitch_f32", I.logit_case(129, 4099, "f32", seed=35, ld=4108)),
    ("pitch_f16", I.logit_case(65, 2051, "f16", seed=36, ld=2056)),
    ("one_col", I.logit_case(7, 1, "bf16", seed=37, ignore_frac=0.0, ld=8)),
    ("short_rows", I.logit_case(64, 7, "f32", seed=38, ld=8)),
    ("zipf_bf16", I.logit_case(512, 32003, "bf16", seed=39, label_dist="zipf", ld=32008)),
    ("wide_spread", I.logit_case(96, 8192, "bf16", seed=40, z_std=30.0)),
]


@pytest.mark.parametrize("name,cfg", CASES, ids=[c[0] for c in CASES])
def test_ce_parity(name, cfg):
    _say("case", cfg.describe())
    inp = I.generate_logits(cfg)
    g = G_DEFAULT[cfg.dtype]
    got = run_ce(inp, g=g, out_pad=True)
    check(got, inp, g)
    assert got["status"] == 0
    assert np.isnan(got["pad"]).all(), "columns past V were written"


def test_ce_inplace_backward():
    cfg = I.logit_case(300, 2500, "bf16", seed=41, ld=2504)
    inp = I.generate_logits(cfg)
    a = run_ce(inp)
    b = run_ce(inp, inplace=True)
    assert np.array_equal(a["dZ"], b["dZ"])
    check(b, inp, 1.0)


def test_ce_custom_ignore_index_negative_grad():
    cfg = I.logit_case(200, 900, "f32", seed=42, ignore_frac=0.0)
    inp = I.generate_logits(cfg)
    y = inp.y.clone()
    y[::5] = 3
    inp = I.LogitInputs(cfg, inp.Z, y)
    got = run_ce(inp, g=-2.5, ignore_index=3)
    check(got, inp, -2.5, ignore_index=3)


def test_ce_all_ignored_and_bad_labels():
    cfg = I.logit_case(100, 500, "bf16", seed=43, ld=504)
    inp = I.generate_logits(cfg)
    ign = I.LogitInputs(cfg, inp.Z, torch.full((100,), -100, dtype=torch.int64))
    got = run_ce(ign)
    assert got["n_valid"] == 0 and got["loss"] == 0.0 and got["status"] == 0
    assert np.all(got["dZ"] == 0.0)
    y = inp.y.clone()
    y[10], y[20] = 500, -3
    bad = I.LogitInputs(cfg, inp.Z, y)
    got = run_ce(bad)
    assert got["status"] == 1
    y_ref = y.numpy().copy()
    y_ref[10], y_ref[20] = -100, -100
    check(got, I.LogitInputs(cfg, inp.Z, torch.from_numpy(y_ref)), 1.0)


def test_ce_rows_beyond_one_launch_grid():
    """1.1M rows: more rows and backward pieces than one launch's 2^20 workgroups, so both
    kernels loop over their work."""
    cfg = I.logit_case(1_100_000, 5, "bf16", seed=45, ld=8)
    _say("case", cfg.describe())
    inp = I.generate_logits(cfg)
    got = run_ce(inp, out_pad=True)
    check(got, inp, 1.0)
    assert got["status"] == 0
    assert np.isnan(got["pad"]).all(), "columns past V were written"


def test_ce_bitwise_deterministic():
    cfg = I.logit_case(333, 5000, "bf16", seed=44)
    inp = I.generate_logits(cfg)
    a, b = run_ce(inp), run_ce(inp)
    assert a["loss"] == b["loss"] and np.array_equal(a["lse"], b["lse"]) and np.array_equal(a["dZ"], b["dZ"])


def test_ce_fullsize_llama3():
    """16384 rows x 128256 bf16 logits (4.2 GB): loss and every row's lse against the stored
    oracle run, dZ on sampled rows; on the whole output, rows of dZ sum to zero and ignored
    rows are exactly zero."""
    cfg = I.LOGIT_CONFIGS["ce_llama3"]
    _say("case", cfg.describe())
    gold = np.load(os.path.join(GOLDEN, "fullsize_ce_llama3.npz"))
    inp = I.generate_logits(cfg)
    assert inp.digest() == str(gold["digest"]), "seeded inputs differ from the stored oracle run"
    from linear_cross_entropy_lm_amd import binding as B
    dev = "cuda:0"
    Z, y = inp.device_tensors(dev)
    N, V = Z.shape
    ws = torch.empty(B.flce_ce_workspace_bytes(N), dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    nv = torch.empty(1, dtype=torch.int32, device=dev)
    st = torch.empty(1, dtype=torch.int32, device=dev)
    B.flce_ce_forward(Z, y, loss, lse, nv, st, ws)
    dZ = torch.empty_like(Z)
    B.flce_ce_backward(Z, y, lse, nv, None, dZ)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(nv.item()) == int(gold["n_valid"])
    loss_err = abs(loss.item() - float(gold["loss"])) / float(gold["loss"])
    lse_err = float(np.max(np.abs(lse.cpu().double().numpy() - gold["lse"]) / np.abs(gold["lse"])))
    rows = torch.from_numpy(gold["dz_rows"]).to(dev)
    dz_err = rel_fro(dZ[rows].float().cpu().numpy(), gold["dz"])
    _say(f"loss {loss.item():.6f} (oracle {float(gold['loss']):.6f}) rel {loss_err:.2e}; lse max rel {lse_err:.2e}; "
         f"dZ rows rel {dz_err:.2e}")
    assert loss_err <= 1e-5 and lse_err <= 1e-5 and dz_err <= TOL_GRAD["bf16"]
    rowsum = dZ.float().sum(dim=1).abs().max().item()
    scale = 1.0 / int(gold["n_valid"])
    assert rowsum <= 1e-2 * scale, rowsum
    assert bool((dZ[y == -100] == 0).all())
