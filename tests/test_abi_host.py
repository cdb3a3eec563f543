"""Host-only checks of the C ABI: the library loads, exports every function include/flce.h
declares, and its synchronous argument checks and workspace arithmetic behave as the
header documents.  Nothing here launches a kernel, so it runs without a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("flce.h", "flce_ce.h", "flce_norm.h")]


@pytest.fixture(scope="module")
def B():
    from linear_cross_entropy_lm_amd import binding
    return binding


def _declared():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(flce_[a-z_]+)\s*\(", text))
    return names


def test_exports_every_declared_symbol(B):
    names = _declared()
    assert names == set(B.SIGNATURES), names ^ set(B.SIGNATURES)
    raw = ctypes.CDLL(B.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings(B):
    for code in range(5):
        s = B.flce_status_string(code)
        assert s.startswith(["FLCE_OK", "FLCE_ERR_INVALID_ARG", "FLCE_ERR_ALIGN", "FLCE_ERR_WORKSPACE",
                             "FLCE_ERR_HIP"][code])
    assert "unknown" in B.flce_status_string(99)


def _r(x, a=256):
    return (x + a - 1) // a * a


def _fwd_bytes(N, V):
    ntn, nvt = -(-N // 256), -(-V // 256)
    splits = min(max(256 // ntn, 1), nvt)
    return _r(splits * N * 8) + _r(N * 4) + _r(ntn * 8) + 2 * _r(ntn * 4)


def _bwd_bytes(N, D, esize, tc, vc, half):
    return 3 * _r(N * 4) + _r(4) + _r(tc * vc * esize) + (_r(tc * D * 4) if half else 0)


@pytest.mark.parametrize("N,D,V,dt", [(64, 256, 1024, 0), (4096, 4096, 32000, 1), (8192, 4096, 32768, 1),
                                      (16384, 4096, 128256, 1), (8192, 3584, 152064, 1), (1, 8, 1, 1),
                                      (700, 384, 3000, 0), (4096, 4096, 32000, 2), (16384, 4096, 128256, 2),
                                      (1, 8, 1, 2)])
def test_workspace_formula(B, N, D, V, dt):
    esize = 4 if dt == 0 else 2
    tc, vc = _r(min(N, 4096)), _r(min(V, 8192))
    while vc > 4096 and _bwd_bytes(N, D, esize, tc, vc, dt != 0) > 0.05 * 2 * N * V:
        vc -= 256
    expect = max(_fwd_bytes(N, V), _bwd_bytes(N, D, esize, tc, vc, dt != 0))
    assert B.flce_workspace_bytes(N, D, V, dt) == expect
    assert B.flce_backward_chunks(N, D, V, dt, expect) == (tc, vc)


def test_llama3_scratch_under_five_percent_of_unfused_logits(B):
    from linear_cross_entropy_lm_amd.scratch import scratch_fraction, unfused_logit_bytes
    ws = B.flce_workspace_bytes(16384, 4096, 128256, 1)
    assert unfused_logit_bytes(16384, 128256) == 4_202_692_608
    assert scratch_fraction(ws, 16384, 128256) <= 0.05


def test_chunk_plan_shrinks_with_workspace(B):
    N, D, V = 700, 384, 3000
    full = B.flce_workspace_bytes(N, D, V, 1)
    plans = []
    for ws in (full, full // 2, full // 4, full // 8):
        try:
            plans.append(B.flce_backward_chunks(N, D, V, 1, ws))
        except B.FlceError as e:
            assert e.code == B.FLCE_ERR_WORKSPACE
            break
    assert plans[0] == (768, 3072)  # V = 3000 fits one vocabulary chunk
    for (t0, v0), (t1, v1) in zip(plans, plans[1:]):
        assert t1 <= t0 and v1 <= v0 and (t1, v1) != (t0, v0)
    for tc, vc in plans:
        assert tc % 256 == 0 and vc % 256 == 0
    with pytest.raises(B.FlceError) as e:
        B.flce_backward_chunks(N, D, V, 1, 1000)
    assert e.value.code == B.FLCE_ERR_WORKSPACE


def test_invalid_sizes(B):
    assert B.flce_workspace_bytes(0, 8, 8, 1) == 0
    assert B.flce_workspace_bytes(8, 8, 8, 7) == 0
    assert B.flce_workspace_bytes(2**31, 8, 8, 1) == 0
    with pytest.raises(B.FlceError) as e:
        B.flce_backward_chunks(8, 0, 8, 1, 10**9)
    assert e.value.code == B.FLCE_ERR_INVALID_ARG


# Synchronous error paths with fake (never dereferenced) pointers: the checks run before
# anything touches the device.
A16 = 0x10000


def _fwd(B, H=A16, W=A16, y=A16, N=8, D=8, V=8, dt=1, loss=A16, lse=A16, nv=A16, st=A16, ws=A16,
         wsb=10**6):
    return B.lib.flce_forward(H, W, y, N, D, V, dt, -100, loss, lse, nv, st, ws, wsb, None)


def _bwd(B, H=A16, W=A16, y=A16, lse=A16, nv=A16, g=None, N=8, D=8, V=8, dt=1, dH=A16, dW=A16, ws=A16,
         wsb=10**6):
    return B.lib.flce_backward(H, W, y, lse, nv, g, N, D, V, dt, -100, dH, dW, ws, wsb, None)


def test_forward_argument_errors(B):
    assert _fwd(B, H=None) == B.FLCE_ERR_INVALID_ARG
    assert _fwd(B, loss=None) == B.FLCE_ERR_INVALID_ARG
    assert _fwd(B, ws=None) == B.FLCE_ERR_INVALID_ARG
    assert _fwd(B, N=0) == B.FLCE_ERR_INVALID_ARG
    assert _fwd(B, dt=3) == B.FLCE_ERR_INVALID_ARG
    assert _fwd(B, H=A16 + 8) == B.FLCE_ERR_ALIGN
    assert _fwd(B, D=12) == B.FLCE_ERR_ALIGN            # bf16 needs D % 8 == 0
    assert _fwd(B, D=12, dt=2) == B.FLCE_ERR_ALIGN      # and so does fp16
    assert _fwd(B, y=A16 + 4) == B.FLCE_ERR_ALIGN
    assert _fwd(B, wsb=16) == B.FLCE_ERR_WORKSPACE


def test_backward_argument_errors(B):
    assert _bwd(B, dW=None) == B.FLCE_ERR_INVALID_ARG
    assert _bwd(B, lse=None) == B.FLCE_ERR_INVALID_ARG
    assert _bwd(B, V=0) == B.FLCE_ERR_INVALID_ARG
    assert _bwd(B, dH=A16 + 2) == B.FLCE_ERR_ALIGN
    assert _bwd(B, dt=0, D=6) == B.FLCE_ERR_ALIGN       # fp32 needs D % 4 == 0
    assert _bwd(B, g=A16 + 1) == B.FLCE_ERR_ALIGN
    assert _bwd(B, wsb=100) == B.FLCE_ERR_WORKSPACE


# --- cross-entropy over materialised logits -------------------------------------------


def test_ce_workspace_formula(B):
    for N in (1, 255, 256, 257, 16384):
        nblk = -(-N // 256)
        assert B.flce_ce_workspace_bytes(N) == _r(N * 8) + _r(N * 4) + _r(nblk * 8) + 2 * _r(nblk * 4)
    assert B.flce_ce_workspace_bytes(0) == 0


def _ce_fwd(B, Z=A16, ld=8, y=A16, N=8, V=8, dt=1, loss=A16, lse=A16, nv=A16, st=A16, ws=A16, wsb=10**6):
    return B.lib.flce_ce_forward(Z, ld, y, N, V, dt, -100, loss, lse, nv, st, ws, wsb, None)


def _ce_bwd(B, Z=A16, ld=8, y=A16, lse=A16, nv=A16, g=None, N=8, V=8, dt=1, dZ=A16, ldo=8):
    return B.lib.flce_ce_backward(Z, ld, y, lse, nv, g, N, V, dt, -100, dZ, ldo, None)


def test_ce_argument_errors(B):
    assert _ce_fwd(B, Z=None) == B.FLCE_ERR_INVALID_ARG
    assert _ce_fwd(B, ld=7) == B.FLCE_ERR_INVALID_ARG          # ld < V
    assert _ce_fwd(B, dt=5) == B.FLCE_ERR_INVALID_ARG
    assert _ce_fwd(B, N=0) == B.FLCE_ERR_INVALID_ARG
    assert _ce_fwd(B, Z=A16 + 2) == B.FLCE_ERR_ALIGN
    assert _ce_fwd(B, ld=12, V=12) == B.FLCE_ERR_ALIGN         # 24-byte rows
    assert _ce_fwd(B, wsb=16) == B.FLCE_ERR_WORKSPACE
    assert _ce_bwd(B, dZ=None) == B.FLCE_ERR_INVALID_ARG
    assert _ce_bwd(B, ldo=4) == B.FLCE_ERR_INVALID_ARG
    assert _ce_bwd(B, dZ=A16 + 8) == B.FLCE_ERR_ALIGN
    assert _ce_bwd(B, dt=0, ld=6, V=6, ldo=8) == B.FLCE_ERR_ALIGN   # 24-byte fp32 rows


# --- RMSNorm of the hidden states ----------------------------------------------------


def test_norm_workspace_formula(B):
    for N, D in [(1, 8), (1000, 4096), (1024, 4096), (16384, 4096), (5000, 12288)]:
        grid = min(N, 512)
        groups = -(-grid // 32)
        assert B.flce_rmsnorm_workspace_bytes(N, D) == _r(grid * D * 4) + _r(groups * D * 4)
    assert B.flce_rmsnorm_workspace_bytes(0, 8) == 0
    assert B.flce_rmsnorm_workspace_bytes(8, 16392) == 0


# Every call below has at least one argument the library rejects before launching.
def _n_fwd(B, X=A16, g=A16, N=8, D=64, dt=1, eps=1e-5, H=A16, r=A16):
    return B.lib.flce_rmsnorm_forward(X, g, N, D, dt, eps, H, r, None)


def _n_bwd(B, X=A16, g=A16, r=A16, dH=A16, N=8, D=64, dt=1, dX=A16, dg=A16, ws=A16, wsb=10**8):
    return B.lib.flce_rmsnorm_backward(X, g, r, dH, N, D, dt, dX, dg, ws, wsb, None)


def test_norm_argument_errors(B):
    assert _n_fwd(B, X=None) == B.FLCE_ERR_INVALID_ARG
    assert _n_fwd(B, N=0) == B.FLCE_ERR_INVALID_ARG
    assert _n_fwd(B, dt=3) == B.FLCE_ERR_INVALID_ARG
    assert _n_fwd(B, eps=-1.0) == B.FLCE_ERR_INVALID_ARG
    assert _n_fwd(B, eps=float("nan")) == B.FLCE_ERR_INVALID_ARG
    assert _n_fwd(B, D=16392) == B.FLCE_ERR_INVALID_ARG      # wider than 16384
    assert _n_fwd(B, dt=0, D=16388) == B.FLCE_ERR_INVALID_ARG
    assert _n_fwd(B, D=12) == B.FLCE_ERR_ALIGN                # 24-byte bf16 rows
    assert _n_fwd(B, H=A16 + 4) == B.FLCE_ERR_ALIGN
    assert _n_fwd(B, r=A16 + 2) == B.FLCE_ERR_ALIGN
    assert _n_bwd(B, dH=None) == B.FLCE_ERR_INVALID_ARG
    assert _n_bwd(B, ws=None) == B.FLCE_ERR_INVALID_ARG
    assert _n_bwd(B, dX=A16 + 8) == B.FLCE_ERR_ALIGN
    assert _n_bwd(B, dt=0, D=6) == B.FLCE_ERR_ALIGN           # 24-byte fp32 rows
    assert _n_bwd(B, wsb=100) == B.FLCE_ERR_WORKSPACE



# --- forward and backward in one call ------------------------------------------------


def test_single_pass_workspace_formula(B):
    for N, D, V, dt, es in [(16384, 4096, 128256, 1, 2), (300, 512, 1031, 0, 4), (4097, 256, 32003, 2, 2)]:
        T = min(-(-N // 256) * 256, 4096)
        ld = -(-V // 256) * 256
        nblk = -(-N // 256)
        expect = (2 * _r(nblk * 4) + _r(4) + _r(max(256 * 256, T) * 8) + _r(T * 4) + _r(nblk * 8) + 2 * _r(nblk * 4)
                  + 3 * _r(T * 4) + _r(4) + _r(T * (ld // 128) * 4) + _r(T * ld * es))
        assert B.flce_forward_backward_workspace_bytes(N, D, V, dt) == expect
    # 25% of the 16-bit logit bytes at the Llama-3 shape: the price of skipping the recompute
    frac = B.flce_forward_backward_workspace_bytes(16384, 4096, 128256, 1) / (16384 * 128256 * 2)
    assert 0.25 < frac < 0.26
    assert B.flce_forward_backward_workspace_bytes(0, 64, 64, 1) == 0


def test_single_pass_chunk_choice(B):
    """The token chunk flce_forward_backward takes: the least workspace buys min(N, 4096)
    rows, more buys multiples of 4096 up to N, within the 32-bit offset cap; below the
    least the call takes the two-call schedule (chunk 0)."""
    N, D, V = 16384, 4096, 128256
    least = B.flce_forward_backward_workspace_bytes(N, D, V, 1)
    assert B.flce_forward_backward_chunk(N, D, V, 1, least) == 4096
    assert B.flce_forward_backward_chunk(N, D, V, 1, 2 * least) == 8192
    # 12288 rows of the kept slab would span 3.2e9 bytes, past the 2^31 offset limit
    assert B.flce_forward_backward_chunk(N, D, V, 1, 10 * least) == 8192
    assert B.flce_forward_backward_chunk(N, D, V, 1, least - 1) == 0
    assert B.flce_forward_backward_chunk(N, D, V, 1, B.flce_workspace_bytes(N, D, V, 1)) == 0
    with pytest.raises(B.FlceError) as e:
        B.flce_forward_backward_chunk(N, D, V, 1, 4096)
    assert e.value.code == B.FLCE_ERR_WORKSPACE
    # the case that wrapped 32-bit offsets (16640 x 304128 bytes = 5.06e9) is capped
    assert B.flce_forward_backward_chunk(16640, 64, 152064, 1, 6 * 10**9) == 4096
    # fp32 at a 152064-row vocabulary: 3328 rows is the widest chunk within the limit
    assert B.flce_forward_backward_chunk(8192, 1024, 152064, 0, 10**12) == 3328


def test_single_pass_unavailable_falls_back(B):
    """Where W is too large for one dH contraction (V D es > 2^31), the single pass does not
    run: the workspace query returns the two-call schedule's need and the call takes it."""
    for N, D, V, dt in [(8192, 4096, 152064, 0), (8192, 8192, 152064, 1)]:
        two = B.flce_workspace_bytes(N, D, V, dt)
        assert B.flce_forward_backward_workspace_bytes(N, D, V, dt) == two
        assert B.flce_forward_backward_chunk(N, D, V, dt, two) == 0
        assert B.flce_forward_backward_chunk(N, D, V, dt, 10**12) == 0


def test_widest_fp32_rows_trim_the_vocab_chunk(B):
    """At D = 65536 fp32 an 8192-row vocabulary chunk of W spans exactly 2^31 bytes: the
    default chunk drops to 7936."""
    ws = B.flce_workspace_bytes(16384, 65536, 128256, 0)
    assert B.flce_backward_chunks(16384, 65536, 128256, 0, ws) == (4096, 7936)


# Every call below has an argument the library rejects before launching anything.
def _fb(B, H=A16, W=A16, y=A16, N=512, D=64, V=1024, dt=1, g=None, loss=A16, lse=A16, nv=A16, st=A16, dH=A16,
        dW=A16, ws=A16, wsb=10**5):
    return B.lib.flce_forward_backward(H, W, y, N, D, V, dt, -100, g, loss, lse, nv, st, dH, dW, ws, wsb, None)


def test_forward_backward_argument_errors(B):
    assert _fb(B, H=None) == B.FLCE_ERR_INVALID_ARG
    assert _fb(B, dW=None) == B.FLCE_ERR_INVALID_ARG
    assert _fb(B, N=0) == B.FLCE_ERR_INVALID_ARG
    assert _fb(B, dt=7) == B.FLCE_ERR_INVALID_ARG
    assert _fb(B, D=12) == B.FLCE_ERR_ALIGN
    assert _fb(B, dH=A16 + 8) == B.FLCE_ERR_ALIGN
    assert _fb(B, g=A16 + 2) == B.FLCE_ERR_ALIGN
    # enough for neither schedule (the forward alone would fit 10**5 bytes only at tiny N)
    assert _fb(B, wsb=1000) == B.FLCE_ERR_WORKSPACE
    # enough for the forward but not the backward: rejected before the forward launches
    fwd_only = B.flce_workspace_bytes(512, 64, 1024, 1) // 16
    assert _fb(B, wsb=fwd_only) == B.FLCE_ERR_WORKSPACE


# --- the entry point that allocates nothing -----------------------------------------


def test_static_scratch_size_matches_header(B):
    text = open(HEADERS[0]).read()
    m = re.search(r"#define FLCE_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and (int(m.group(1)) << int(m.group(2))) == B.FLCE_STATIC_SCRATCH_BYTES
    # the default two-call workspace of every workload fits the array
    for N, D, V, dt in [(16384, 4096, 128256, 1), (8192, 3584, 152064, 1), (4096, 4096, 32000, 1),
                        (8192, 4096, 32768, 1), (16384, 4096, 128256, 2), (64, 256, 1024, 0)]:
        assert B.flce_workspace_bytes(N, D, V, dt) <= B.FLCE_STATIC_SCRATCH_BYTES
        assert B.flce_forward_backward_chunk(N, D, V, dt, B.FLCE_STATIC_SCRATCH_BYTES) >= 0


def _fbs(B, H=A16, W=A16, y=A16, N=512, D=64, V=1024, dt=1, g=None, loss=A16, lse=A16, nv=A16, st=A16, dH=A16,
         dW=A16):
    return B.lib.flce_forward_backward_static(H, W, y, N, D, V, dt, -100, g, loss, lse, nv, st, dH, dW, None)


def test_static_rejects_before_touching_the_device(B):
    """Sizes beyond the array and invalid arguments are reported without a GPU."""
    # a vocabulary too wide for the single pass (256 kept rows of 9e6 columns pass the
    # 32-bit offset limit), and 16M rows whose per-row terms alone (12 bytes a row) exceed
    # 144 MiB for the recomputing schedule
    assert B.flce_forward_backward_chunk(16 << 20, 8, 9_000_000, 1, 10**12) == 0
    assert _fbs(B, N=16 << 20, D=8, V=9_000_000) == B.FLCE_ERR_WORKSPACE
    # the single pass needs only a few bytes per row besides its kept chunk: 16M rows at a
    # small vocabulary fit the array
    assert B.flce_forward_backward_chunk(16 << 20, 8, 8, 1, B.FLCE_STATIC_SCRATCH_BYTES) > 0
    assert _fbs(B, N=0) == B.FLCE_ERR_INVALID_ARG
    assert _fbs(B, dt=9) == B.FLCE_ERR_INVALID_ARG
    assert _fbs(B, H=None) == B.FLCE_ERR_INVALID_ARG
    assert _fbs(B, dW=None) == B.FLCE_ERR_INVALID_ARG


def test_binding_fails_loudly_without_the_library(tmp_path):
    """A copy of the package without libflce.so: importing the binding raises ImportError
    (there is no CPU or torch fallback for any entry point)."""
    import shutil
    import subprocess
    import sys
    src = os.path.join(ROOT, "linear_cross_entropy_lm_amd")
    dst = tmp_path / "linear_cross_entropy_lm_amd"
    dst.mkdir()
    for f in os.listdir(src):
        if f.endswith(".py"):
            shutil.copy(os.path.join(src, f), dst / f)
    assert not (dst / "libflce.so").exists()
    r = subprocess.run([sys.executable, "-c", "import linear_cross_entropy_lm_amd.binding"], cwd=tmp_path,
                       env={**os.environ, "PYTHONPATH": str(tmp_path)}, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libflce.so is missing" in r.stderr
