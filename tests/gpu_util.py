"""Helpers for the GPU parity tests: move seeded problems to the device,
run the HIP path through the C ABI binding, compare with the oracle."""
import sys

import numpy as np
import torch

import oracle as O
from softmax_sink_amd import binding as B


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(p, name):
    x = getattr(p, name)
    if p.dtype in ("bf16", "fp16"):
        dt = torch.bfloat16 if p.dtype == "bf16" else torch.float16
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(dt).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def dev_sinks(p):
    return torch.from_numpy(np.ascontiguousarray(p.sinks)).cuda()


class HipRun:
    """Device copies of a workloads.Problem and the HIP results on them."""

    def __init__(self, p, with_sink=True):
        self.p = p
        self.plan = B.Plan(p.cu_q, p.cu_k, p.num_heads_q, p.num_heads_k, p.head_dim,
                           p.causal, (p.win_left, p.win_right), p.dtype)
        self.q, self.k, self.v = to_dev(p, "q"), to_dev(p, "k"), to_dev(p, "v")
        self.sinks = dev_sinks(p) if with_sink else None
        self.scale = float(p.scale)

    def fwd(self):
        self.out, self.lse = B.forward(self.plan, self.q, self.k, self.v, self.sinks, self.scale)
        torch.cuda.synchronize()
        return self.out.float().cpu().numpy().astype(np.float64), self.lse.cpu().numpy().astype(np.float64)

    def bwd(self):
        self.dout = to_dev(self.p, "dout")
        dq, dk, dv, ds = B.backward(self.plan, self.dout, self.q, self.k, self.v, self.out,
                                    self.lse, self.sinks, self.scale)
        torch.cuda.synchronize()
        self.dq, self.dk, self.dv, self.dsink = dq, dk, dv, ds
        f = lambda t: t.float().cpu().numpy().astype(np.float64)
        return f(dq), f(dk), f(dv), (ds.cpu().numpy().astype(np.float64) if ds is not None else None)


def per_head(fn, heads, workers=8):
    """fn(h) for every head in `heads`, on a thread pool with one BLAS thread
    per call: the oracle's elementwise NumPy work (exp, masks) runs on one
    core per call, so heads side by side use the host's cores. Returns the
    results in the order of `heads`."""
    import concurrent.futures as cf
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1), cf.ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, heads))


def oracle_inputs(p, with_sink=True):
    sinks = p.sinks.astype(np.float64) if with_sink else np.full(p.num_heads_q, -np.inf)
    return (p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), p.cu_q, p.cu_k, sinks,
            float(p.scale), p.causal, p.win_left, p.win_right)


def max_abs(a, b):
    a, b = np.asarray(a), np.asarray(b)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):           # inf - inf where both_inf
        d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.max(d)) if d.size else 0.0


def rel_l2(a, b):
    num = np.linalg.norm((np.asarray(a) - np.asarray(b)).ravel())
    den = np.linalg.norm(np.asarray(b).ravel())
    return float(num / den) if den > 0 else float(num)


# tolerances stated for the method: fp32 out/lse max abs 1e-5; bf16 out max
# abs 1e-2, lse max abs 1e-3, gradients relative L2 2e-2. No bound is stated
# for fp32 gradients: dq, dk, dv are held to relative L2 1e-5, and dsink, a
# sum of signed terms that can cancel, to 1e-5 of the sum of the terms'
# magnitudes (dsink_error below).
TOL = {"fp32": dict(out=1e-5, lse=1e-5, grad=1e-5), "bf16": dict(out=1e-2, lse=1e-3, grad=2e-2)}
# fp16 inputs (finer than bf16) are held to the bf16 bar
TOL["fp16"] = TOL["bf16"]


def dsink_error(ds, rs, ro, rl, dout, sinks):
    """max over heads of |ds_h - rs_h| / sum_i |e^(s_h - lse_hi) D_hi|: the
    error of dsink_h = -sum_i e^(s_h - lse_hi) D_hi, D_hi = dO_hi . out_hi,
    relative to the magnitudes of its terms, as a floating-point sum is
    bounded (its relative L2 error is unbounded when the terms cancel).
    ro [Tq, Hq, D] and rl [Hq, Tq] are the oracle's out and lse, dout
    [Tq, Hq, D], sinks [Hq]."""
    dvec = np.einsum("thd,thd->ht", np.asarray(dout, np.float64), np.asarray(ro, np.float64))
    with np.errstate(invalid="ignore", over="ignore"):
        w = np.exp(np.asarray(sinks, np.float64)[:, None] - np.asarray(rl, np.float64))
    w = np.where(np.isfinite(w), w, 0.0)
    mag = np.abs(w * dvec).sum(axis=1)
    diff = np.abs(np.asarray(ds, np.float64) - np.asarray(rs, np.float64))
    return float(np.max(np.where(mag > 0, diff / np.where(mag > 0, mag, 1.0), diff)))


def sampled_rows_error(p, out, lse, n, seed):
    """Max abs error of out and lse against the oracle on n random (token,
    q-head) rows plus the first and last row of every sequence."""
    rng = np.random.default_rng(seed)
    rows = [(int(rng.integers(0, p.total_q)), int(rng.integers(0, p.num_heads_q)))
            for _ in range(n)]
    for b in range(p.batch):
        if p.cu_q[b + 1] > p.cu_q[b]:
            rows.append((int(p.cu_q[b]), b % p.num_heads_q))
            rows.append((int(p.cu_q[b + 1] - 1), (3 * b) % p.num_heads_q))
    ref = O.sink_attention_rows(p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), p.cu_q, p.cu_k,
                                p.sinks.astype(np.float64), float(p.scale), p.causal,
                                p.win_left, p.win_right, rows)
    e_out = max(max_abs(out[t, h], r["out"]) for (t, h), r in zip(rows, ref))
    e_lse = max(max_abs(lse[h, t], r["lse"]) for (t, h), r in zip(rows, ref))
    return e_out, e_lse
