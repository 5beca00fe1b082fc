"""The named workloads at full size, in the launch configuration bench.py
times, checked against the oracle on outputs it can compute exactly one
slice at a time: whole q-heads (every sequence) for forward and backward,
whole sequences for the split-KV decode, and sampled single rows."""
import numpy as np
import pytest
import torch

import oracle as O
from softmax_sink_amd import workloads as W
from tests.gpu_util import HipRun, TOL, log, max_abs, oracle_inputs, per_head, rel_l2
from tests.gpu_util import sampled_rows_error as _sampled_rows

pytestmark = pytest.mark.gpu


def _fwd_heads(p, g, out, lse, heads):
    ro, rl, _ = O.sink_attention_forward(*oracle_inputs(p), heads=heads)
    return (max(max_abs(out[:, h], ro[:, h]) for h in heads),
            max(max_abs(lse[h], rl[h]) for h in heads))


def test_prefill_varlen_full_size():
    p = W.config("prefill_varlen")
    log(f"prefill_varlen: Tq={p.total_q} lens={np.diff(p.cu_q).tolist()}")
    g = HipRun(p)
    out, lse = g.fwd()
    e_out, e_lse = _fwd_heads(p, g, out, lse, [0, 9, 22, 31])
    s_out, s_lse = _sampled_rows(p, out, lse, 256, 1)
    log(f"  heads 0,9,22,31: max|d out|={e_out:.3e} max|d lse|={e_lse:.3e}; "
        f"sampled rows: {s_out:.3e} {s_lse:.3e}")
    tol = TOL["bf16"]
    assert max(e_out, s_out) <= tol["out"] and max(e_lse, s_lse) <= tol["lse"]


# dq/dk/dv are compared on q-heads spread over the slot classes of the
# head-to-XCD mapping (head_of_slot: XCD x runs q-heads x*Hq/8 .. x*Hq/8 +
# Hq/8 - 1), and dsink as the whole [Hq] vector (relative L2, as the target
# states it; the per-head errors are logged: one head's dsink is a sum of
# random-sign terms that can cancel by two orders of magnitude, and D uses
# the stored bf16 output, as the "slime" page's backward does).
@pytest.mark.parametrize("name,heads", [
    ("train_varlen", [0, 5, 18, 31]),
    ("gqa_window", list(range(0, 8)) + list(range(40, 48))),
    ("train_varlen_d256", [0, 7, 10, 15])])
def test_training_workloads_full_size(name, heads):
    p = W.config(name)
    log(f"{name}: Tq={p.total_q} lens={np.diff(p.cu_q).tolist()} H={p.num_heads_q}/{p.num_heads_k}")
    g = HipRun(p)
    out, lse = g.fwd()
    dq, dk, dv, ds = g.bwd()
    args = oracle_inputs(p)
    dout = p.as_f32("dout")
    G = p.num_heads_q // p.num_heads_k
    kvh = sorted({h // G for h in heads})
    log(f"  GPU done; oracle backward on q-heads {heads} (kv-heads {kvh}), dsink on all heads")
    q, k, v, cu_q, cu_k, sinks = args[:6]

    def one_head(h):
        """The oracle's problem of q-head h alone (its kv-head, its sink)."""
        hk = h // G
        return (q[:, h:h + 1], k[:, hk:hk + 1], v[:, hk:hk + 1], cu_q, cu_k,
                sinks[h:h + 1]) + tuple(args[6:])

    def fwd_head(h):
        o, l, _ = O.sink_attention_forward(*one_head(h))
        return o[:, 0], l[0]

    def bwd_head(h):
        r = O.sink_attention_backward(dout[:, h:h + 1], *one_head(h))
        return r[0][:, 0], r[1][:, 0], r[2][:, 0]

    fwd = per_head(fwd_head, heads)
    bwd = per_head(bwd_head, heads)
    rs = np.array(per_head(lambda h: O.sink_attention_dsink(dout[:, h:h + 1], *one_head(h))[0],
                           list(range(p.num_heads_q))))
    e_out = max(max_abs(out[:, h], f[0]) for h, f in zip(heads, fwd))
    e_lse = max(max_abs(lse[h], f[1]) for h, f in zip(heads, fwd))
    rq = {h: b[0] for h, b in zip(heads, bwd)}
    rk = {hk: sum(b[1] for h, b in zip(heads, bwd) if h // G == hk) for hk in kvh}
    rv = {hk: sum(b[2] for h, b in zip(heads, bwd) if h // G == hk) for hk in kvh}
    # dk / dv of a kv-head sum over its whole group: check the kv-heads whose
    # every q-head was computed
    full_kv = [hk for hk in kvh if all(hk * G + j in heads for j in range(G))]
    assert full_kv, "no complete GQA group among the checked heads"
    errs = dict(dq=rel_l2(np.stack([dq[:, h] for h in heads]), np.stack([rq[h] for h in heads])),
                dk=rel_l2(np.stack([dk[:, hk] for hk in full_kv]), np.stack([rk[hk] for hk in full_kv])),
                dv=rel_l2(np.stack([dv[:, hk] for hk in full_kv]), np.stack([rv[hk] for hk in full_kv])),
                dsink=rel_l2(ds, rs))
    per_dq = {h: round(float(rel_l2(dq[:, h], rq[h])), 5) for h in heads}
    per_ds = [round(float(abs(a - b) / max(abs(b), 1e-30)), 4) for a, b in zip(ds, rs)]
    s_out, s_lse = _sampled_rows(p, out, lse, 128, 2)
    log(f"  max|d out|={max(e_out, s_out):.3e} max|d lse|={max(e_lse, s_lse):.3e} "
        + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    log(f"  dq rel-L2 per head {per_dq}; kv-heads checked for dk/dv {full_kv}")
    log(f"  dsink relative error per head {per_ds}")
    tol = TOL["bf16"]
    assert max(e_out, s_out) <= tol["out"] and max(e_lse, s_lse) <= tol["lse"]
    assert all(v <= tol["grad"] for v in errs.values()), errs
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()
    assert np.isfinite(ds).all()


def test_decode_softmax_n_full_size():
    p = W.config("decode_softmax_n")
    log(f"decode_softmax_n: Tq={p.total_q} Tk={p.total_k}")
    g = HipRun(p)
    assert g.plan.mode == 1
    out, lse = g.fwd()
    lk = np.diff(p.cu_k)
    seqs = sorted({int(np.argmax(lk)), int(np.argmin(lk)), 0, 17, 40, 63})
    sub = p.sub_batch(seqs)
    ro, rl, _ = O.sink_attention_forward(*oracle_inputs(sub))
    rows = np.concatenate([np.arange(p.cu_q[b], p.cu_q[b + 1]) for b in seqs])
    e_out = max_abs(out[rows], ro)
    e_lse = max_abs(lse[:, rows], rl)
    log(f"  sequences {seqs}: max|d out|={e_out:.3e} max|d lse|={e_lse:.3e}")
    tol = TOL["bf16"]
    assert e_out <= tol["out"] and e_lse <= tol["lse"]


def test_gqa_window_bnsd_equals_packed_bitwise():
    """The gqa_window workload handed over in the BNSD layout (as the
    gqa_window_bnsd bench line does) runs the same arithmetic as the packed
    call: every output equals the packed one bit for bit."""
    from softmax_sink_amd import binding as B
    p = W.config("gqa_window_bnsd")
    S = int(np.diff(p.cu_q)[0])
    log(f"gqa_window_bnsd: B={p.batch} S={S} H={p.num_heads_q}/{p.num_heads_k}")
    g = HipRun(p)
    g.fwd()
    g.bwd()
    plan = B.PaddedPlan(p.batch, S, S, None, None, p.num_heads_q, p.num_heads_k, p.head_dim,
                        p.causal, (p.win_left, p.win_right), p.dtype, "BNSD")
    # BNSD views of the packed device tensors: [T, N, D] -> [B, N, S, D]
    bnsd = lambda t: t.view(p.batch, S, t.shape[1], t.shape[2]).transpose(1, 2).contiguous()
    packed = lambda t: t.transpose(1, 2).reshape(p.batch * S, t.shape[1], t.shape[3])
    q, k, v, do = bnsd(g.q), bnsd(g.k), bnsd(g.v), bnsd(g.dout)
    out, lse = B.forward_padded(plan, q, k, v, g.sinks, g.scale)
    dq, dk, dv, ds = B.backward_padded(plan, do, q, k, v, out, lse, g.sinks, g.scale)
    torch.cuda.synchronize()
    same = lambda a, b: torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))
    assert same(packed(out), g.out)
    # lse [B, Hq, S] against the packed [Hq, Tq]
    assert torch.equal(lse.transpose(0, 1).reshape(p.num_heads_q, -1), g.lse)
    assert same(packed(dq), g.dq) and same(packed(dk), g.dk) and same(packed(dv), g.dv)
    assert torch.equal(ds, g.dsink)
    log("  BNSD forward and backward equal the packed results bit for bit")


@pytest.mark.parametrize("name", ["train_varlen", "gqa_window", "train_varlen_d256",
                                  "decode_softmax_n"])
def test_full_size_runs_are_reproducible(name):
    """Every output of a full-size workload is the same bits on a second and
    a third run (no atomics, fixed reduction orders; a race would show here)."""
    p = W.config(name)
    g = HipRun(p)
    train = name != "decode_softmax_n"
    runs = []
    for _ in range(3):
        g.fwd()
        outs = [g.out.clone(), g.lse.clone()]
        if train:
            g.bwd()
            outs += [g.dq.clone(), g.dk.clone(), g.dv.clone(), g.dsink.clone()]
        runs.append(outs)
    bits = lambda t: t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert torch.equal(bits(a), bits(b))
    log(f"{name}: three runs equal bit for bit")
