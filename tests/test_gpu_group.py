"""GPU parity of the grouped forward (qlora_linear_fwd_group): several adapted linears that share x
run as one fused launch where the shapes allow, each output checked against the oracle's linear on
that linear's own dequantised weight ("QLoRA, explained", The algorithm, step by step).

Tolerance as for the single forward (relative Frobenius error <= 5e-3, elementwise <= 1e-2 *
max|ref|) for y and u; with B = 0, one-hot rows of x give rows of each y that equal columns of that
weight's W~ bit for bit, which pins which weight every column tile reads and where it writes.
"""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import (assert_close, bf16_to_dev, bits_from_dev, dev, f64_from_bits, log, oracle_weight,
                         to_dev)

pytestmark = pytest.mark.gpu


def _group(seed, M, Ns, K, r, kind="gauss"):
    g = wl.rng_for("single", 700 + seed, "x")
    x = wl.to_bf16_bits(g.standard_normal((M, K), dtype=np.float32))
    ws, As, Bs = [], [], []
    for i, N in enumerate(Ns):
        ws.append(wl.weight("single", 700 + seed + 10 * i, N, K, kind, 0.02))
        As.append(wl.to_bf16_bits(g.standard_normal((r, K), dtype=np.float32) * np.float32(0.01)))
        Bs.append(wl.to_bf16_bits(g.standard_normal((N, r), dtype=np.float32) * np.float32(0.01)))
    return x, ws, As, Bs


def _run_group(qws, x, As, Bs, s, keep_u=True):
    import torch
    import bit_nf4_quantised_amd as q
    M = x.shape[0]
    r = As[0].shape[0]
    ys = [torch.empty(M, w.N, dtype=torch.int16, device=dev()) for w in qws]
    us = [torch.empty(M, r, dtype=torch.float32, device=dev()) for _ in qws] if keep_u else None
    q.qlora_linear_fwd_group(qws, bf16_to_dev(x), [bf16_to_dev(a) for a in As], [bf16_to_dev(b) for b in Bs], s,
                             ys, us)
    torch.cuda.synchronize()
    return [bits_from_dev(y) for y in ys], ([u.cpu().numpy() for u in us] if keep_u else None)


def _quantize(w, double_quant=True):
    import torch
    import bit_nf4_quantised_amd as q
    qw = q.quantize_weight(to_dev(w.astype(np.float32)), double_quant=double_quant)
    torch.cuda.synchronize()
    if double_quant:
        return qw, oracle_weight(w)
    packed, absmax = oracle.quantize(w)
    return qw, oracle.dequant_blocks(packed, absmax, oracle.codebook(), 64, w.size).reshape(w.shape)


@pytest.mark.parametrize("M,Ns,K,r,s,dq", [
    (600, (8192, 2048, 2048), 2048, 16, 2.0, True),   # one launch; 288 tiles, the 32 past the first
                                                      #   round in four contraction ranges each
    (300, (8208, 4112), 512, 32, 0.5, True),          # one launch, no tail; ragged last tiles in both
    (300, (8192, 2048, 2048), 512, 16, 2.0, False),   # one launch, fp32 block scales
    (100, (400, 128), 960, 16, 2.0, True),            # at most 128 tokens: linear by linear
    (3, (416, 1040, 96), 1088, 64, 0.5, True),        # few tokens: the few-token path, linear by linear
])
def test_group_matches_oracle(M, Ns, K, r, s, dq):
    x, ws, As, Bs = _group(M + K + r, M, Ns, K, r)
    log(f"[group] M={M} N={Ns} K={K} r={r} dq={dq}")
    qw_wt = [_quantize(w, dq) for w in ws]
    ys, us = _run_group([qw for qw, _ in qw_wt], x, As, Bs, s)
    for i, ((_, wt), a, b) in enumerate(zip(qw_wt, As, Bs)):
        yr, ur = oracle.linear_fwd(x, wt, a, b, s)
        assert_close(f"y{i}", f64_from_bits(ys[i]), yr)
        assert_close(f"u{i}", us[i], ur)


def test_group_one_hot_rows_are_exact():
    # B = 0: row i of x one-hot at column c_i gives y_j[i] = column c_i of W~_j, for every weight j of
    # the group (a one-launch shape with a tail)
    M, Ns, K, r = 600, (8192, 2048, 2048), 2048, 16
    x, ws, As, Bs = _group(5, M, Ns, K, r)
    qw_wt = [_quantize(w) for w in ws]
    x = np.zeros((M, K), np.uint16)
    cols = [(7 * i + 3) % K for i in range(M)]
    for i, c in enumerate(cols):
        x[i, c] = 0x3F80
    ys, _ = _run_group([qw for qw, _ in qw_wt], x, As, [np.zeros_like(b) for b in Bs], 2.0, keep_u=False)
    for j, (_, wt) in enumerate(qw_wt):
        assert np.array_equal(ys[j], wt[:, cols].T), j


def test_group_matches_single_forwards():
    # the same linears through qlora_linear_fwd one by one: equal within the forward's tolerance (the
    # contraction may be summed in other ranges), u bit for bit (the same launches form it)
    import torch
    import bit_nf4_quantised_amd as q
    M, Ns, K, r, s = 600, (8192, 2048, 2048), 2048, 16, 2.0
    x, ws, As, Bs = _group(9, M, Ns, K, r)
    qws = [_quantize(w)[0] for w in ws]
    ys, us = _run_group(qws, x, As, Bs, s)
    for i, (qw, a, b) in enumerate(zip(qws, As, Bs)):
        y1 = torch.empty(M, qw.N, dtype=torch.int16, device=dev())
        u1 = torch.empty(M, r, dtype=torch.float32, device=dev())
        q.qlora_linear_fwd(qw, bf16_to_dev(x), bf16_to_dev(a), bf16_to_dev(b), s, y1, u1)
        torch.cuda.synchronize()
        assert np.array_equal(u1.cpu().numpy(), us[i]), i
        assert_close(f"y{i}", f64_from_bits(ys[i]), f64_from_bits(bits_from_dev(y1)))


def test_group_refuses_mixed_weights():
    import torch
    import bit_nf4_quantised_amd as q
    M, K, r = 300, 512, 16
    x, ws, As, Bs = _group(11, M, (2048, 1024), K, r)
    a = _quantize(ws[0])[0]
    b = _quantize(ws[1], double_quant=False)[0]
    ys = [torch.empty(M, w.N, dtype=torch.int16, device=dev()) for w in (a, b)]
    with pytest.raises(q.NF4Error):
        q.qlora_linear_fwd_group([a, b], bf16_to_dev(x), [bf16_to_dev(v) for v in As],
                                 [bf16_to_dev(v) for v in Bs], 2.0, ys)


@pytest.mark.parametrize("M,Ns,K", [(600, (8192, 2048, 2048), 2048), (100, (400, 128), 960), (3, (416, 96), 1088)])
def test_group_recompute_equals_the_forward(M, Ns, K):
    # with the u the forward saved, the grouped recompute gives the same y bit for bit
    import torch
    import bit_nf4_quantised_amd as q
    r, s = 16, 2.0
    x, ws, As, Bs = _group(13, M, Ns, K, r)
    qws = [_quantize(w)[0] for w in ws]
    ys, us = _run_group(qws, x, As, Bs, s)
    y2 = [torch.empty(M, w.N, dtype=torch.int16, device=dev()) for w in qws]
    q.qlora_linear_fwd_recompute_group(qws, bf16_to_dev(x), [bf16_to_dev(a) for a in As], [bf16_to_dev(b) for b in Bs],
                                       s, [to_dev(u) for u in us], y2)
    torch.cuda.synchronize()
    for i in range(len(qws)):
        assert np.array_equal(bits_from_dev(y2[i]), ys[i]), i


def _run_bwd_group(qws, x, dys, As, Bs, s, us, accumulate=False, dA0=None, dB0=None):
    import torch
    import bit_nf4_quantised_amd as q
    M, K = x.shape
    r = As[0].shape[0]
    dxs = [torch.empty(M, K, dtype=torch.int16, device=dev()) for _ in qws]
    dAs = [to_dev(a) if dA0 is not None else torch.empty(r, K, dtype=torch.float32, device=dev())
           for a in (dA0 if dA0 is not None else qws)]
    dBs = [to_dev(b) if dB0 is not None else torch.empty(w.N, r, dtype=torch.float32, device=dev())
           for w, b in zip(qws, dB0 if dB0 is not None else qws)]
    q.qlora_linear_bwd_group(qws, bf16_to_dev(x), [bf16_to_dev(d) for d in dys], [bf16_to_dev(a) for a in As],
                             [bf16_to_dev(b) for b in Bs], s, [to_dev(u) for u in us], dxs, dAs, dBs,
                             accumulate=accumulate)
    torch.cuda.synchronize()
    return [bits_from_dev(d) for d in dxs], [d.cpu().numpy() for d in dAs], [d.cpu().numpy() for d in dBs]


@pytest.mark.parametrize("M,Ns,K,r,s", [
    (300, (2048, 512, 512), 12288, 16, 2.0),   # one dX launch: 3 x 192 tiles (each linear alone: 256-row
                                               #   tiles, no split, so dX bit-equal to the single calls)
    (600, (2064, 1040), 4096, 32, 0.5),        # one dX launch, ragged contractions, 3 row blocks
    (100, (400, 128), 960, 16, 2.0),           # at most 128 tokens: linear by linear
    (200, (512, 256, 384, 128), 1024, 32, 1.0),  # four linears: ranks add up past 64, so one pass over X
                                                 #   per linear, and eight sums in one reduction launch
    (130, (256, 256, 256, 256), 2048, 16, 2.0),  # four linears at rank 16: one pass over X for all
])
def test_bwd_group_matches_oracle_and_single_calls(M, Ns, K, r, s):
    import torch
    import bit_nf4_quantised_amd as q
    x, ws, As, Bs = _group(17 + M, M, Ns, K, r)
    g = wl.rng_for("single", 900 + M, "dy")
    dys = [wl.to_bf16_bits(g.standard_normal((M, N), dtype=np.float32)) for N in Ns]
    log(f"[group] bwd M={M} N={Ns} K={K} r={r}")
    qw_wt = [_quantize(w) for w in ws]
    qws = [qw for qw, _ in qw_wt]
    _, us = _run_group(qws, x, As, Bs, s)
    dxs, dAs, dBs = _run_bwd_group(qws, x, dys, As, Bs, s, us)
    for i, ((qw, wt), a, b, dy) in enumerate(zip(qw_wt, As, Bs, dys)):
        dxr, dar, dbr = oracle.linear_bwd(x, dy, wt, a, b, s)
        assert_close(f"dx{i}", f64_from_bits(dxs[i]), dxr)
        assert_close(f"dA{i}", dAs[i], dar)
        assert_close(f"dB{i}", dBs[i], dbr)
        # the single backward of the same linear: dA, dB bit for bit (same launches); dX bit for bit
        # where its own launch takes the same tiles without a split, else within the tolerance
        dx1 = torch.empty(M, K, dtype=torch.int16, device=dev())
        dA1 = torch.empty(r, K, dtype=torch.float32, device=dev())
        dB1 = torch.empty(qw.N, r, dtype=torch.float32, device=dev())
        q.qlora_linear_bwd(qw, bf16_to_dev(x), bf16_to_dev(dy), bf16_to_dev(a), bf16_to_dev(b), s, to_dev(us[i]), dx1,
                           dA1, dB1)
        torch.cuda.synchronize()
        assert np.array_equal(dA1.cpu().numpy(), dAs[i]), i
        assert np.array_equal(dB1.cpu().numpy(), dBs[i]), i
        if M == 300:
            assert np.array_equal(bits_from_dev(dx1), dxs[i]), i
        else:
            assert_close(f"dx{i} single", f64_from_bits(dxs[i]), f64_from_bits(bits_from_dev(dx1)))


def test_bwd_group_one_hot_rows_are_exact():
    # B = 0: row i of dY_j one-hot at row n_i of W_j gives dX_j[i] = row n_i of W~_j, for every
    # linear j of a one-launch group (which pins the weight, activation and output of every tile)
    M, Ns, K, r = 300, (2048, 512, 512), 12288, 16
    x, ws, As, Bs = _group(21, M, Ns, K, r)
    qw_wt = [_quantize(w) for w in ws]
    qws = [qw for qw, _ in qw_wt]
    dys = []
    rows = []
    for N in Ns:
        d = np.zeros((M, N), np.uint16)
        rr = [(5 * i + 1) % N for i in range(M)]
        for i, n in enumerate(rr):
            d[i, n] = 0x3F80
        dys.append(d)
        rows.append(rr)
    us = [np.zeros((M, r), np.float32) for _ in Ns]
    dxs, _, _ = _run_bwd_group(qws, x, dys, As, [np.zeros_like(b) for b in Bs], 2.0, us)
    for j, (_, wt) in enumerate(qw_wt):
        assert np.array_equal(dxs[j], wt[rows[j]]), j


@pytest.mark.parametrize("Ns,r", [((512, 256, 256), 16), ((256, 384, 128, 256), 32)])
def test_bwd_group_accumulates_like_single_calls(Ns, r):
    # accumulate = 1 adds into dA, dB as the single backward does, bit for bit, in both forms of the
    # passes over X (one launch for the group, one per linear)
    import torch
    import bit_nf4_quantised_amd as q
    M, K, s = 260, 1088, 0.5
    x, ws, As, Bs = _group(29 + r, M, Ns, K, r)
    g = wl.rng_for("single", 950 + r, "dy")
    dys = [wl.to_bf16_bits(g.standard_normal((M, N), dtype=np.float32)) for N in Ns]
    dA0 = [g.standard_normal((r, K), dtype=np.float32) for _ in Ns]
    dB0 = [g.standard_normal((N, r), dtype=np.float32) for N in Ns]
    log(f"[group] bwd accumulate N={Ns} r={r}")
    qw_wt = [_quantize(w) for w in ws]
    qws = [qw for qw, _ in qw_wt]
    _, us = _run_group(qws, x, As, Bs, s)
    _, dAs, dBs = _run_bwd_group(qws, x, dys, As, Bs, s, us, accumulate=True, dA0=dA0, dB0=dB0)
    for i, ((qw, wt), a, b, dy) in enumerate(zip(qw_wt, As, Bs, dys)):
        _, dar, dbr = oracle.linear_bwd(x, dy, wt, a, b, s)
        assert_close(f"dA{i}", dAs[i] - dA0[i].astype(np.float64), dar)
        assert_close(f"dB{i}", dBs[i] - dB0[i].astype(np.float64), dbr)
        dx1 = torch.empty(M, K, dtype=torch.int16, device=dev())
        dA1, dB1 = to_dev(dA0[i]), to_dev(dB0[i])
        q.qlora_linear_bwd(qw, bf16_to_dev(x), bf16_to_dev(dy), bf16_to_dev(a), bf16_to_dev(b), s, to_dev(us[i]), dx1,
                           dA1, dB1, accumulate=True)
        torch.cuda.synchronize()
        assert np.array_equal(dA1.cpu().numpy(), dAs[i]), i
        assert np.array_equal(dB1.cpu().numpy(), dBs[i]), i
