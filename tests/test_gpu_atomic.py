"""Atomic-expert layer on the GPU (OmniMoE page, technical summary 2.1-2.2)
against the fp64 oracle, both schedules: row/column logits within the fp32
dot-product bound, the Cartesian top-k bit-exact with the oracle's selection
on the GPU's own logits (fp32 scores), the own-logit selection equal to the
exact one wherever the k-th/(k+1)-th margin exceeds 1e-3, and the layer
output within the output bar. Plus the two schedules timed on a
million-parameter-per-expert-grid shape."""
import numpy as np
import pytest
import torch

import oracle.atomic as A
from quantized_mixture_experts_qmoe_amd import (QMOE_SCHEDULE_EXPERT_CENTRIC, QMOE_SCHEDULE_TOKEN_CENTRIC,
                                                AtomicLayer)
from quantized_mixture_experts_qmoe_amd.inputs import bf16_bits_to_f32, make_atomic_inputs
from gpu_util import (MARGIN, MAX_ABS_RMS, assert_output_close, bf16_tensor_to_f64, half_ulp_bf16, logit_bound,
                      to_dev_bf16)

pytestmark = pytest.mark.gpu

SCHEDULES = {"expert": QMOE_SCHEDULE_EXPERT_CENTRIC, "token": QMOE_SCHEDULE_TOKEN_CENTRIC}


@pytest.mark.parametrize("schedule", ["expert", "token"])
@pytest.mark.parametrize("T,d,nr,nc,k", [(300, 512, 64, 64, 8), (1, 512, 1, 50, 4), (64, 1024, 17, 130, 8),
                                         (1000, 512, 1024, 2, 3), (257, 512, 8, 8, 1), (40, 2048, 300, 300, 8),
                                         # wider rows: the token kernel without the look-ahead slot (d > 2048),
                                         # the row kernel in batches of eight chunks with a tail (d > 4096)
                                         (50, 3072, 16, 16, 2), (37, 4608, 12, 12, 5), (20, 8192, 3, 40, 8)])
def test_atomic_layer(schedule, T, d, nr, nc, k):
    print(f"[case] atomic {schedule} T={T} d={d} grid={nr}x{nc} k={k}", flush=True)
    inp = make_atomic_inputs(T, d, nr, nc, seed=T + nr + nc)
    layer = AtomicLayer(inp.w_in, inp.w_out, inp.router_rows, inp.router_cols, top_k=k, max_tokens=T)
    route = dict(logits_rows=torch.empty((T, nr), dtype=torch.float32, device="cuda"),
                 logits_cols=torch.empty((T, nc), dtype=torch.float32, device="cuda"),
                 topk_idx=torch.empty((T, k), dtype=torch.int32, device="cuda"),
                 topk_w=torch.empty((T, k), dtype=torch.float32, device="cuda"))
    y = layer.forward(to_dev_bf16(inp.x), schedule=SCHEDULES[schedule], route=route)
    torch.cuda.synchronize()
    lr, lc = route["logits_rows"].cpu().numpy(), route["logits_cols"].cpu().numpy()
    idx, w = route["topk_idx"].cpu().numpy(), route["topk_w"].cpu().numpy()
    layer.close()
    ref = A.layer(inp.x, inp.w_in, inp.w_out, inp.router_rows, inp.router_cols, k)
    # logits within the fp32 dot-product bound
    assert np.all(np.abs(lr - ref["lr"]) <= logit_bound(inp.x, inp.router_rows, False) + 1e-30)
    assert np.all(np.abs(lc - ref["lc"]) <= logit_bound(inp.x, inp.router_cols, False) + 1e-30)
    # on the GPU's own logits the selection is the definition's, bit for bit
    g_idx, g_w, _ = A.topk(A.scores(lr, lc, np.float32), k)
    assert np.array_equal(idx, g_idx)
    assert np.allclose(w, g_w, rtol=0, atol=1e-6)
    # against the exact logits: equal sets wherever the margin exceeds 1e-3
    near = ref["margin"] <= MARGIN
    for t in range(T):
        if set(idx[t].tolist()) != set(ref["idx"][t].tolist()):
            assert near[t], (t, ref["margin"][t])
    print(f"[routing] tokens under margin {MARGIN}: {int(near.sum())}", flush=True)
    y_ref = A.layer(inp.x, inp.w_in, inp.w_out, inp.router_rows, inp.router_cols, k, given=idx)["y"]
    # few rank-one terms per token make heavy-tailed outputs (largest |y| tens
    # of RMS): where half a bf16 ulp of the largest |y_ref| reaches three
    # quarters of the max-abs bar, the bar applies beyond the output's own
    # rounding (half a bf16 ulp of y_ref)
    own = float(half_ulp_bf16(y_ref).max() / np.sqrt(np.mean(y_ref ** 2)))
    print(f"[parity] half a bf16 ulp of the largest |y_ref|: {own:.3e} RMS", flush=True)
    assert_output_close(bf16_tensor_to_f64(y), y_ref, f"atomic {schedule}", own >= 0.75 * MAX_ABS_RMS)


@pytest.mark.parametrize("T,nr,nc,k", [(300, 64, 64, 8), (1000, 1024, 2, 3), (40, 300, 300, 8), (257, 8, 8, 1),
                                       (1, 1, 50, 4)])
def test_atomic_task_list_is_the_stable_sort(oracle_mod, T, nr, nc, k):
    """The expert-centric task list, bit for bit: the stable sort of the
    (token, slot) tasks by expert group (ceil(N/256) consecutive flat indices
    per group), tokens ascending inside a group (OmniMoE page, technical
    summary 2.2: routing decisions flattened and grouped by expert), computed
    by the oracle's dispatch on the GPU's own selection."""
    d = 512
    print(f"[case] atomic task list T={T} grid={nr}x{nc} k={k}", flush=True)
    inp = make_atomic_inputs(T, d, nr, nc, seed=3 * T + nr)
    layer = AtomicLayer(inp.w_in, inp.w_out, inp.router_rows, inp.router_cols, top_k=k, max_tokens=T)
    route = dict(topk_idx=torch.empty((T, k), dtype=torch.int32, device="cuda"),
                 perm=torch.full((T * k,), -1, dtype=torch.int32, device="cuda"))
    layer.forward(to_dev_bf16(inp.x), schedule=QMOE_SCHEDULE_EXPERT_CENTRIC, route=route)
    torch.cuda.synchronize()
    idx, perm = route["topk_idx"].cpu().numpy(), route["perm"].cpu().numpy()
    layer.close()
    N = nr * nc
    B = (N + 255) // 256
    counts, offsets, ref_perm, _ = oracle_mod.dispatch(idx // B, (N + B - 1) // B)
    assert np.array_equal(perm, ref_perm)


@pytest.mark.parametrize("schedule", ["expert", "token"])
def test_cartesian_topk_exact_rounding_ties(schedule):
    """Scores that round to the same fp32 value although their row logits
    differ: the selection must still follow the definition (equal scores go to
    the lower flat index), also where the tied pair lies outside the best k
    rows or columns. Token t routes on one-hot x (position t % 8), so its
    logits are router entries exactly: row logits 1 + j/128 (half of them fall
    on a rounding tie at 2^17, where the fp32 spacing is 1/64) and column
    logits 2^17 + 1024 c. The first token is the smallest case: rows 1.0 and
    1.0078125, one column 2^17, k = 1, both scores 131073: expert 0 wins."""
    d, T = 512, 64
    rng = np.random.default_rng(5)

    def bits(a):
        return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)

    for nr, nc, k in [(2, 1, 1), (40, 24, 8), (64, 64, 8), (13, 100, 5), (100, 3, 7)]:
        rr = np.zeros((nr, d), np.float32)
        rc = np.zeros((nc, d), np.float32)
        for p in range(8):
            rr[:, p] = 1.0 + rng.permutation(128)[:nr] / 128.0 if nr > 2 else [1.0, 1.0078125]
            rc[:, p] = 131072.0 + 1024.0 * rng.integers(0, 4, nc)
        x = np.zeros((T, d), np.float32)
        x[np.arange(T), np.arange(T) % 8] = 1.0
        w_in = make_atomic_inputs(1, d, nr, nc, seed=9).w_in
        w_out = make_atomic_inputs(1, d, nr, nc, seed=10).w_out
        print(f"[case] cartesian ties {schedule} grid={nr}x{nc} k={k}", flush=True)
        layer = AtomicLayer(w_in, w_out, bits(rr), bits(rc), top_k=k, max_tokens=T)
        route = dict(logits_rows=torch.empty((T, nr), dtype=torch.float32, device="cuda"),
                     logits_cols=torch.empty((T, nc), dtype=torch.float32, device="cuda"),
                     topk_idx=torch.empty((T, k), dtype=torch.int32, device="cuda"),
                     topk_w=torch.empty((T, k), dtype=torch.float32, device="cuda"))
        layer.forward(to_dev_bf16(bits(x)), schedule=SCHEDULES[schedule], route=route)
        torch.cuda.synchronize()
        layer.close()
        lr, lc = route["logits_rows"].cpu().numpy(), route["logits_cols"].cpu().numpy()
        assert np.array_equal(lr, rr[:, np.arange(T) % 8].T) and np.array_equal(lc, rc[:, np.arange(T) % 8].T)
        s32 = A.scores(lr, lc, np.float32)
        g_idx, g_w, _ = A.topk(s32, k)
        idx = route["topk_idx"].cpu().numpy()
        assert np.array_equal(idx, g_idx), (nr, nc, k)
        assert np.allclose(route["topk_w"].cpu().numpy(), g_w, rtol=0, atol=1e-6)
        if nr == 2:
            assert np.all(idx[:, 0] == 0)
        # the case exercises ties at the k-th score that cross the best rows
        n_tie = int(sum(np.sum(s32[t] == s32[t, g_idx[t, -1]]) > 1 for t in range(T)))
        print(f"[routing] tokens with a tie at the k-th score: {n_tie} of {T}", flush=True)


@pytest.mark.parametrize("nr,nc", [(256, 256), (64, 64)])
def test_atomic_schedules_timed(nr, nc):
    """Atomic experts of width 2048, top-8, 8192 tokens, on a 256 x 256 grid
    (65536 experts, W and V 512 MB, about one task per expert) and a 64 x 64
    grid (4096 experts, 16 tasks per expert): the two schedules timed with HIP
    events on one stream."""
    T, d, k = 8192, 2048, 8
    inp = make_atomic_inputs(T, d, nr, nc, seed=1)
    layer = AtomicLayer(inp.w_in, inp.w_out, inp.router_rows, inp.router_cols, top_k=k, max_tokens=T)
    x = to_dev_bf16(inp.x)
    y = torch.empty_like(x)
    res = {}
    for name in ("expert", "token", "expert", "token"):
        for _ in range(2):
            layer.forward(x, y=y, schedule=SCHEDULES[name])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            layer.forward(x, y=y, schedule=SCHEDULES[name])
        e1.record()
        e1.synchronize()
        res.setdefault(name, []).append(e0.elapsed_time(e1) / 10 * 1e3)
    # algorithmic bytes of the expert kernels: x, y, and every selected
    # expert's w_in and w_out rows once; the expert-centric kernel also writes
    # the fp32 task rows that the combine reads back
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    layer.forward(x, y=y, schedule=SCHEDULES["token"], route={"topk_idx": idx})
    torch.cuda.synchronize()
    layer.close()
    uniq = int(torch.unique(idx).numel())
    xy, rows_w = 2 * T * d * 2, uniq * 2 * d * 2
    print(f"[atomic] {nr}x{nc} grid: {uniq} distinct experts selected; algorithmic MB: "
          f"token kernel {(xy + rows_w) / 1e6:.1f}, expert-row kernel {(T * d * 2 + rows_w + T * k * d * 4) / 1e6:.1f}, "
          f"combine {(T * k * d * 4 + T * d * 2) / 1e6:.1f}", flush=True)
    for name, v in res.items():
        us = min(v)
        print(f"[atomic] {nr}x{nc} grid, {name}-centric: {us:.1f} us per forward, {T / us:.2f} M tokens/s",
              flush=True)
