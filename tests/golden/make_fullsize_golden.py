"""Write tests/golden/fullsize_<workload>.npz: fp64 oracle values for the full-size
workloads (Llama-2, Mistral, Llama-3 and Qwen-2.5 shaped heads in bf16, Llama-2 and
Llama-3 in fp16), for the capped single-pass case (spcap_bf16), for a vocabulary whose W holds
more than 2^31 elements (wide_vocab_bf16), for as many tokens in H (long_tokens_bf16), for the
Llama-3-shaped head with fp32 inputs (llama3_f32), and for the cross-entropy over materialised
Llama-3-shaped logits (ce_llama3).

Only the oracle and the seeded input generator are used.  Stored per workload:
  digest         fingerprint of the exact input bytes (checked before comparing)
  loss, n_valid  the mean loss over labelled rows and their count
  lse            per-row log-sum-exp for every row
  dh_rows, dh    whole dH rows: first, last, an ignored row, the last valid row, random
  dw_rows, dw    whole dW rows: first, last, the most frequent labels (the whole head of a
                 Zipf label distribution: its 16 most frequent labels), random
  dh_edge_rows, dh_edge_cols, dh_edge
                 dH at the first and last row of every 256-row token tile (so at the edges
                 of every token chunk the backward can take), each over a 256-column window
                 that walks across D from one tile to the next
  dw_edge_rows, dw_edge_cols, dw_edge
                 dW likewise at the first and last row of every 256-row vocabulary tile
                 (every vocabulary chunk edge among them), each over a walking window
For ce_llama3 instead of dh/dw:
  dz_rows, dz    dZ for a few rows (first, last, an ignored row, random ones)
For chain_llama3 (the final RMSNorm of norm_llama3 feeding the Llama-3-shaped head: H is the
norm's output stored in bf16, dH the head's gradient stored in bf16, as the kernels hand
them on), instead of dh:
  dx_rows, dx, dx_edge_rows, dx_edge_cols, dx_edge   dX as dh above
  dgamma         the norm weight's gradient over every row

Usage:  python tests/golden/make_fullsize_golden.py [workload ...]
"""
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from linear_cross_entropy_lm_amd import inputs as I  # noqa: E402

WORKLOADS = ["llama2", "mistral", "llama3", "qwen25", "llama2_f16", "llama3_f16", "spcap_bf16", "wide_vocab_bf16",
             "long_tokens_bf16", "llama3_f32", "ce_llama3", "chain_llama3"]
TILE = 256


def pick_rows(y: np.ndarray, rng) -> np.ndarray:
    N = len(y)
    ign = np.nonzero(y == -100)[0]
    val = np.nonzero(y != -100)[0]
    rows = {0, N - 1, int(ign[0]), int(val[-1])}
    while len(rows) < 8:
        rows.add(int(rng.integers(0, N)))
    return np.array(sorted(rows), dtype=np.int64)


def pick_vocab(y: np.ndarray, V: int, rng) -> np.ndarray:
    lab = y[y != -100]
    vals, counts = np.unique(lab, return_counts=True)
    head = vals[np.argsort(-counts, kind="stable")[:16]]
    vs = {0, V - 1, int(lab[0])} | {int(v) for v in head}
    while len(vs) < len(head) + 8:
        vs.add(int(rng.integers(0, V)))
    return np.array(sorted(vs), dtype=np.int64)


def tile_edges(n: int, D: int):
    """The first and last index of every 256-wide tile of n, and for each a window start
    that walks across D (tile t: window t mod ceil(D / 256), clipped to D)."""
    rows, cols = [], []
    n_td = -(-D // TILE)
    for t in range(-(-n // TILE)):
        a, b = t * TILE, min(t * TILE + TILE - 1, n - 1)
        c0 = min((t % n_td) * TILE, max(D - TILE, 0))
        for r in sorted({a, b}):
            rows.append(r)
            cols.append(c0)
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


def windows(full: np.ndarray, cols: np.ndarray, D: int) -> np.ndarray:
    w = min(TILE, D)
    return np.stack([full[i, c:c + w] for i, c in enumerate(cols)]).astype(np.float64)


def logits_golden(name):
    """Loss and every row's lse in 512-row blocks (the fp64 logits of all rows would take
    17 GB), then dZ for the sampled rows with the global N_valid."""
    t0 = time.time()
    cfg = I.LOGIT_CONFIGS[name]
    inp = I.generate_logits(cfg)
    y = inp.y64()
    N = cfg.N
    n_valid = oracle.count_valid(y, cfg.V, oracle.IGNORE_INDEX)
    lse = np.empty(N)
    row_loss = np.empty(N)
    for r0 in range(0, N, 512):
        r1 = min(N, r0 + 512)
        b = oracle.ce_from_logits(inp.z64(np.arange(r0, r1)), y[r0:r1], grads=False)
        lse[r0:r1] = b["lse"]
        row_loss[r0:r1] = b["row_loss"]
    loss = float(row_loss.sum() / n_valid)
    rows = pick_rows(y, np.random.default_rng(cfg.seed))
    dz = oracle.logit_grad(inp.z64(rows), lse[rows], y[rows], 1.0 / n_valid, oracle.IGNORE_INDEX)
    path = os.path.join(HERE, f"fullsize_{name}.npz")
    np.savez_compressed(path, digest=np.array(inp.digest()), loss=np.array(loss), n_valid=np.array(n_valid),
                        lse=lse, dz_rows=rows, dz=dz)
    print(f"{cfg.describe()}: loss {loss:.6f} n_valid {n_valid} -> {os.path.basename(path)} "
          f"({time.time() - t0:.0f} s)", flush=True)


def chain_golden(name):
    """The norm -> head -> loss chain at the Llama-3 shape, in 512-row blocks: per block the
    logits, lse and loss terms, dz (N_valid is known from the labels up front), dH = dz W
    rounded to bf16, and its share of dgamma; dX at the sampled rows; then dW rows."""
    t0 = time.time()
    ncfg, hcfg = I.NORM_CONFIGS["norm_llama3"], I.CONFIGS["llama3"]
    ninp, hinp = I.generate_norm(ncfg), I.generate(hcfg)
    X, gam = ninp.x64(), ninp.gamma64()
    W, y = hinp.w64(), hinp.y64()
    N, D = X.shape
    H = oracle.round_to(oracle.rmsnorm_forward(X, gam, ncfg.eps)["H"], "bf16")
    n_valid = oracle.count_valid(y, hcfg.V)
    rng = np.random.default_rng(hcfg.seed + 17)
    rows = pick_rows(y, rng)
    e_rows, e_cols = tile_edges(N, D)
    want = set(rows.tolist()) | set(e_rows.tolist())
    lse = np.empty(N)
    row_loss = np.zeros(N)
    dgamma = np.zeros(D)
    dx_at = {}
    for r0 in range(0, N, 512):
        r1 = min(N, r0 + 512)
        Z = oracle.logits(H, W, slice(r0, r1))
        L = oracle.logsumexp_rows(Z)
        lse[r0:r1] = L
        yy = y[r0:r1]
        idx = np.nonzero(yy != oracle.IGNORE_INDEX)[0]
        row_loss[r0 + idx] = L[idx] - Z[idx, yy[idx]]
        dH = oracle.round_to(oracle.logit_grad(Z, L, yy, 1.0 / n_valid) @ W, "bf16")
        nb = oracle.rmsnorm_backward(X[r0:r1], gam, dH, ncfg.eps)
        dgamma += nb["dgamma"]
        for r in range(r0, r1):
            if r in want:
                dx_at[r] = nb["dX"][r - r0]
    loss = float(row_loss.sum() / n_valid)
    vrows = pick_vocab(y, hcfg.V, rng)
    ev_rows, ev_cols = tile_edges(hcfg.V, D)
    all_v = np.unique(np.concatenate([vrows, ev_rows]))
    dw_all = oracle.dW_rows(H, W, y, all_v, lse, n_valid)
    atv = {v: i for i, v in enumerate(all_v)}
    dx = np.stack([dx_at[r] for r in rows])
    dx_edge = windows(np.stack([dx_at[r] for r in e_rows]), e_cols, D)
    dw = dw_all[[atv[v] for v in vrows]]
    dw_edge = windows(dw_all[[atv[v] for v in ev_rows]], ev_cols, D)
    path = os.path.join(HERE, f"fullsize_{name}.npz")
    np.savez_compressed(path, digest=np.array(ninp.digest() + hinp.digest()), loss=np.array(loss),
                        n_valid=np.array(n_valid), lse=lse, dx_rows=rows, dx=dx, dx_edge_rows=e_rows,
                        dx_edge_cols=e_cols, dx_edge=dx_edge.astype(np.float32), dgamma=dgamma, dw_rows=vrows, dw=dw,
                        dw_edge_rows=ev_rows, dw_edge_cols=ev_cols, dw_edge=dw_edge.astype(np.float32))
    print(f"{name}: loss {loss:.6f} n_valid {n_valid} -> {os.path.basename(path)} ({time.time() - t0:.0f} s)",
          flush=True)


def config(name):
    return I.CONFIGS[name] if name in I.CONFIGS else I.GOLDEN_CASES[name]


def main(names):
    for name in names:
        if name in I.LOGIT_CONFIGS:
            logits_golden(name)
            continue
        if name == "chain_llama3":
            chain_golden(name)
            continue
        t0 = time.time()
        cfg = config(name)
        inp = I.generate(cfg)
        H, W, y = inp.h64(), inp.w64(), inp.y64()
        st = oracle.forward_stats(H, W, y, row_block=512)
        rng = np.random.default_rng(cfg.seed)
        rows = pick_rows(y, rng)
        vrows = pick_vocab(y, cfg.V, rng)
        e_rows, e_cols = tile_edges(cfg.N, cfg.D)
        ev_rows, ev_cols = tile_edges(cfg.V, cfg.D)
        all_rows = np.unique(np.concatenate([rows, e_rows]))
        all_vrows = np.unique(np.concatenate([vrows, ev_rows]))
        dh_all = oracle.dH_rows(H, W, y, all_rows, st["n_valid"])
        dw_all = oracle.dW_rows(H, W, y, all_vrows, st["lse"], st["n_valid"])
        at = {r: i for i, r in enumerate(all_rows)}
        atv = {v: i for i, v in enumerate(all_vrows)}
        dh = dh_all[[at[r] for r in rows]]
        dw = dw_all[[atv[v] for v in vrows]]
        dh_edge = windows(dh_all[[at[r] for r in e_rows]], e_cols, cfg.D)
        dw_edge = windows(dw_all[[atv[v] for v in ev_rows]], ev_cols, cfg.D)
        path = os.path.join(HERE, f"fullsize_{name}.npz")
        np.savez_compressed(path, digest=np.array(inp.digest()), loss=np.array(st["loss"]),
                            n_valid=np.array(st["n_valid"]), lse=st["lse"], dh_rows=rows, dh=dh,
                            dw_rows=vrows, dw=dw, dh_edge_rows=e_rows, dh_edge_cols=e_cols,
                            dh_edge=dh_edge.astype(np.float32), dw_edge_rows=ev_rows, dw_edge_cols=ev_cols,
                            dw_edge=dw_edge.astype(np.float32))
        print(f"{cfg.describe()}: loss {st['loss']:.6f} n_valid {st['n_valid']} "
              f"-> {os.path.basename(path)} ({time.time() - t0:.0f} s)", flush=True)
        del H, W, inp


if __name__ == "__main__":
    main(sys.argv[1:] or WORKLOADS)
