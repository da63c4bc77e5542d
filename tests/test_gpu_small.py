"""GPU parity at sizes the oracle finishes in seconds: every stage compared
element by element with the oracle on the same seeded inputs.  Shapes span
several GEMM tiles with ragged row counts per expert, the three score modes,
the selection-only bias and its update step, the shared expert, capacity
dropping, and the degenerate cases (one expert, k = E, one token, E = 256,
k > 64, zero router, empty experts)."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_ffn_08_amd import _lib
from mixture_experts_ffn_08_amd import inputs as minp
from mixture_experts_ffn_08_amd.inputs import SIGMOID_THEN_TOPK as SIG, SOFTMAX_THEN_TOPK as SM_TK, \
    TOPK_THEN_SOFTMAX as TK_SM
from support import TOL, ExpertCache, LayerRun, assert_same_sum, check_dispatch, check_route, check_stats, host, \
    log, max_rel

pytestmark = pytest.mark.gpu

S = minp.LayerShape
SMALL = [
    S("small_renorm", "bf16", 300, 256, 16, 4, 384, 0, SM_TK, True, None, False),
    S("small_shared", "bf16", 257, 384, 8, 2, 256, 512, SM_TK, False, None, False),
    S("small_topk_first", "bf16", 193, 128, 32, 3, 128, 0, TK_SM, False, None, False),
    S("small_capacity", "bf16", 400, 256, 8, 2, 256, 0, TK_SM, False, 0.8, False),
    S("small_zipf", "bf16", 256, 256, 64, 8, 128, 128, SM_TK, True, None, True),
    minp.SHAPES["tiny_f32"],
    S("f32_ragged", "f32", 100, 72, 5, 2, 40, 24, SM_TK, True, 1.0, False),
    S("one_expert", "bf16", 50, 128, 1, 1, 128, 0, SM_TK, False, None, False),
    S("k_equals_E", "bf16", 70, 128, 4, 4, 128, 0, SM_TK, True, None, False),
    S("one_token", "bf16", 1, 256, 16, 4, 256, 256, SM_TK, True, None, False),
    S("E256", "bf16", 130, 128, 256, 8, 128, 0, SM_TK, True, None, True),
    S("E256_few_tokens", "bf16", 50, 256, 256, 8, 128, 0, SIG, False, None, False, select_bias=0.01),
    S("k_over_64", "bf16", 40, 128, 200, 70, 128, 0, TK_SM, False, None, False),
    S("tiny_capacity_f32", "f32", 64, 64, 8, 2, 128, 0, TK_SM, False, 1.25, False),
    # above the router's few-token threshold (E > 64: score blocks of 64 experts, then selection;
    # else scores and selection in one kernel), with d / 128 odd and even
    S("many_tokens", "bf16", 2100, 128, 16, 4, 128, 0, SM_TK, True, None, False),
    S("many_tokens_E128_d640", "bf16", 2200, 640, 128, 8, 128, 0, SM_TK, True, None, False),
    S("many_tokens_E32_d896_topk_first", "bf16", 2111, 896, 32, 4, 128, 0, TK_SM, False, None, False,
      select_bias=0.02),
    S("many_tokens_E256_d384_sigmoid", "bf16", 2500, 384, 256, 8, 128, 0, SIG, False, None, False),
    S("many_tokens_E200_k70", "bf16", 2070, 128, 200, 70, 128, 0, TK_SM, False, None, False),
    # sigmoid scoring and the selection-only bias, in each mode and both router shapes
    S("sigmoid", "bf16", 300, 256, 16, 4, 256, 0, SIG, False, None, False),
    S("sigmoid_biased_shared", "bf16", 257, 256, 32, 6, 128, 256, SIG, False, None, False, select_bias=0.05),
    S("softmax_biased", "bf16", 300, 256, 64, 8, 128, 0, SM_TK, True, None, False, select_bias=0.01),
    S("topk_first_biased_cap", "bf16", 400, 256, 8, 2, 256, 0, TK_SM, False, 1.0, False, select_bias=0.5),
    S("many_tokens_sigmoid_biased", "bf16", 2100, 128, 16, 4, 128, 0, SIG, False, None, True, select_bias=0.05),
    S("many_tokens_softmax_biased", "bf16", 2100, 128, 64, 6, 128, 0, SM_TK, False, None, False,
      select_bias=0.01),
    S("f32_sigmoid_biased", "f32", 100, 72, 5, 2, 40, 0, SIG, False, None, False, select_bias=0.1),
    # 64 < E <= 128 above the few-token threshold: scores as a DMA-fed GEMM with the selection in
    # the same block; each score mode, a selection bias and a logit bias, d / 64 not a multiple of 3
    S("many_tokens_E96_sigmoid_biased", "bf16", 2100, 256, 96, 6, 128, 0, SIG, False, None, False,
      select_bias=0.05),
    S("many_tokens_E128_topk_first_zipf", "bf16", 2300, 384, 128, 8, 128, 0, TK_SM, False, None, True),
    S("many_tokens_E72_softmax_biased", "bf16", 2051, 1152, 72, 8, 128, 0, SM_TK, False, None, False,
      select_bias=0.01),
    # ... and from T = 4096 on, 64-token blocks on 8 waves (ragged last block)
    S("many_tokens_E96_wide_sigmoid_biased", "bf16", 4133, 256, 96, 6, 128, 0, SIG, False, None, False,
      select_bias=0.05),
    S("many_tokens_E128_wide_softmax_renorm", "bf16", 4097, 384, 128, 8, 128, 0, SM_TK, True, None, False),
    # E = 256 with T (E / 64) past the split-score limit: the fused kernel with 256 experts
    S("many_tokens_E256_fused", "bf16", 8300, 128, 256, 8, 128, 0, SM_TK, True, None, True, select_bias=0.002),
]


def full_check(inp, out):
    s = inp.shape
    xs = minp.as_f32(inp.x, s.dtype)
    ex = ExpertCache(inp)
    sh = ex.shared()
    tie = check_route(inp, out)
    counts, offsets, row_of, perm_token = check_dispatch(inp, out)
    check_stats(inp, out)
    tol = TOL[s.dtype]
    # experts on the GPU's own permuted rows
    R = int(offsets[-1])
    b = run_state["bufs"]
    if b.x_perm is not None:
        assert np.array_equal(host(b.x_perm)[:R], xs[perm_token]), "x_perm must be an exact gather"
    x_perm = xs[perm_token]
    a_ref, y_ref = oracle.grouped_swiglu(x_perm, offsets, ex)
    if R:
        a_gpu, y_gpu = host(b.a)[:R], host(b.y_perm)[:R]
        assert max_rel(a_gpu, a_ref) <= tol, max_rel(a_gpu, a_ref)
        assert max_rel(y_gpu, y_ref) <= tol, max_rel(y_gpu, y_ref)
    else:
        y_gpu = np.zeros((0, s.d), np.float32)
    shared_gpu = None
    if sh is not None:
        shared_gpu = host(b.shared_y)
        s_ref = oracle.swiglu(xs, *sh)
        assert max_rel(shared_gpu, s_ref) <= tol
    # combine, stage-isolated: the GPU's own y_perm, weights, rows and shared output
    y_comb = oracle.round_to(oracle.combine(y_gpu, out["row_of"], out["w"], shared_gpu, d=s.d), s.dtype)
    ref64 = np.abs(oracle.combine(y_gpu, out["row_of"], out["w"], shared_gpu, d=s.d))
    bound = (2.0 ** -7 if s.dtype == "bf16" else 2e-6) * ref64 + 1e-6 * max(ref64.max(), 1e-30)
    assert np.all(np.abs(out["y"] - y_comb) <= bound), "combine"
    # end to end against the oracle's whole layer, outside tokens whose routing differs
    full = oracle.layer_forward(xs, minp.as_f32(inp.w_router, s.dtype), inp.bias, ex, sh, k=s.k, mode=s.mode,
                                renorm=s.renorm, phi=s.phi, alpha=s.alpha, dtype=s.dtype,
                                select_bias=inp.select_bias)
    same = ~(out["idx"] != full["idx"]).any(1)
    if s.phi is not None:
        same &= ~tie  # a flipped token shifts later arrivals' ranks; compare routing-identical tokens only
    err = np.abs(out["y"][same] - full["y64"][same]).max() if same.any() else 0.0
    ymax = np.abs(full["y64"]).max()
    log(f"[{s.name}] end-to-end max|dy|/max|y| = {err / max(ymax, 1e-30):.3e} (tol {tol}), "
        f"{int((~same).sum())} tokens excluded")
    assert err <= tol * ymax


run_state = {}


@pytest.mark.parametrize("shape", SMALL, ids=[s.name for s in SMALL])
def test_small_layer_parity(shape):
    inp = minp.LayerInputs(shape, seed=0)
    run = LayerRun(inp)
    out = run.run()
    run_state["bufs"] = run.bufs
    try:
        full_check(inp, out)
    finally:
        run_state.clear()
        run.free()


@pytest.mark.parametrize("idx", [1, 3, 6])
def test_materialized_gather_matches_fused(idx):
    """moe_permute with an x_perm buffer gathers exactly; the gate/up GEMM on that
    copy gives bit-identical results to the GEMM reading x through perm_token."""
    shape = SMALL[idx]
    inp = minp.LayerInputs(shape, seed=2)
    fused = LayerRun(inp).run()
    run = LayerRun(inp, gathered=True)
    out = run.run()
    run_state["bufs"] = run.bufs
    try:
        R = int(out["offsets"][-1])                  # perm_token rows past R are not written
        for key in fused:
            a, b = np.asarray(fused[key]), np.asarray(out[key])
            if key == "perm_token":
                a, b = a[:R], b[:R]
            assert np.array_equal(a, b), key
        full_check(inp, out)
    finally:
        run_state.clear()
        run.free()


SCATTER_CASES = ["small_renorm", "small_shared", "small_capacity", "small_zipf", "tiny_f32", "f32_ragged",
                 "one_token", "E256", "k_over_64", "many_tokens", "many_tokens_E128_d640"]


@pytest.mark.parametrize("name", SCATTER_CASES)
def test_scatter_combine_matches_gather(name):
    """The down GEMM with the weighted sum in its epilogue (float32 atomics into an
    accumulator, then + shared expert, one rounding) against the down GEMM writing
    y_perm and the gather combine: routing, dispatch and statistics bit-identical,
    y one rounding of the same sum apart (tiled, skinny and float32 GEMM kernels,
    the shared expert, dropped slots, k > 64), twice in a row on one workspace;
    and y against the oracle's whole layer."""
    shape = next(s for s in SMALL if s.name == name)
    inp = minp.LayerInputs(shape, seed=5)
    g = LayerRun(inp)
    ref = g.run()
    g.free()
    run = LayerRun(inp, scatter=True)
    try:
        s = shape
        R = int(ref["offsets"][-1])
        for rep in range(2):
            out = run.run()
            for key in ("scores", "idx", "w", "near_tie", "counts", "offsets", "row_of", "f", "P", "l_aux",
                        "max_over_mean"):
                assert np.array_equal(np.asarray(out[key]), np.asarray(ref[key])), key
            assert np.array_equal(out["perm_token"][:R], ref["perm_token"][:R])
            frac = assert_same_sum(out["y"], ref["y"], s.dtype, f"{name} call {rep}")
            log(f"[{name}] scatter combine, call {rep}: {100 * frac:.3f}% of y differs from the gather combine "
                f"(within one rounding)")
        ex = ExpertCache(inp)
        xs = minp.as_f32(inp.x, s.dtype)
        full = oracle.layer_forward(xs, minp.as_f32(inp.w_router, s.dtype), inp.bias, ex, ex.shared(), k=s.k,
                                    mode=s.mode, renorm=s.renorm, phi=s.phi, alpha=s.alpha, dtype=s.dtype,
                                    select_bias=inp.select_bias)
        same = ~(out["idx"] != full["idx"]).any(1) & ~((out["near_tie"] == 1) | (full["near_tie"] == 1))
        if same.any():
            err = np.abs(out["y"][same] - full["y64"][same]).max()
            assert err <= TOL[s.dtype] * np.abs(full["y64"]).max()
    finally:
        run.free()


LAYER_CALL_CASES = [
    # decode batches: the selection, dispatch and statistics as one block (T <= 64, T k <= 512)
    S("decode_E128_k8", "bf16", 64, 256, 128, 8, 128, 0, SM_TK, True, None, True),
    S("decode_capacity", "bf16", 60, 128, 16, 4, 128, 0, TK_SM, False, 0.5, False),
    S("decode_sigmoid_biased_shared", "bf16", 33, 128, 64, 6, 128, 256, SIG, False, None, False, select_bias=0.05),
    S("decode_E256_k2", "bf16", 7, 128, 256, 2, 128, 0, SM_TK, False, None, False),
    next(s for s in SMALL if s.name == "one_token"),
    next(s for s in SMALL if s.name == "E256_few_tokens"),
    # just past the one-block limits, and the other forms
    S("decode_k9", "bf16", 64, 128, 32, 9, 128, 0, SM_TK, True, None, False),
    # 64-token router blocks with k = 8: the router writes the dispatch's histograms (ragged last block)
    S("prefill_E128_k8_router_hist", "bf16", 4133, 128, 128, 8, 128, 0, SM_TK, True, None, False),
    S("prefill_E96_k8_capacity", "bf16", 4100, 128, 96, 8, 128, 0, SIG, False, 0.9, False, select_bias=0.02),
    next(s for s in SMALL if s.name == "small_shared"),
    next(s for s in SMALL if s.name == "tiny_f32"),
    next(s for s in SMALL if s.name == "k_over_64"),
]

_LAYER_OUTPUTS = ("scores", "idx", "w", "near_tie", "counts", "offsets", "row_of", "f", "P", "l_aux",
                  "max_over_mean", "y")


@pytest.mark.parametrize("shape", LAYER_CALL_CASES, ids=lambda s: s.name)
def test_layer_call_matches_separate_calls_bitwise(shape):
    """moe_layer_forward (one call; with T <= 64 and T k <= 512 in bf16 the
    selection, dispatch and statistics run as one block) against the separate
    entry points on fresh buffers: every output and intermediate bit for bit; and
    the layer against the oracle."""
    from mixture_experts_ffn_08_amd.layer import Buffers
    inp = minp.LayerInputs(shape, seed=6)
    run = LayerRun(inp)
    try:
        s = shape
        out = run.run()
        R = int(out["offsets"][-1])
        b, lay = run.bufs, run.layer
        one = {key: np.asarray(out[key]).copy() for key in _LAYER_OUTPUTS}
        one["perm_token"] = out["perm_token"][:R].copy()
        one["a"], one["y_perm"] = host(b.a)[:R], host(b.y_perm)[:R]
        if s.F_shared:
            one["shared_y"] = host(b.shared_y)
        b2 = Buffers(s, s.T, "cuda")
        for t in (b2.logits, b2.topk_w, b2.a, b2.y_perm, b2.y):
            t.fill_(float("nan"))
        st = torch.cuda.current_stream()
        lay.route(run.x, b2, st)
        lay.permute(run.x, b2, st)
        lay.gate_up(run.x, b2, st)
        lay.down(b2, st)
        lay.shared_expert(run.x, b2, st)
        lay.combine(b2, st)
        lay.stats(b2, st)
        torch.cuda.synchronize()
        two = dict(scores=host(b2.logits), idx=host(b2.topk_idx), w=host(b2.topk_w),
                   near_tie=host(b2.near_tie), counts=host(b2.counts), offsets=host(b2.offsets),
                   row_of=host(b2.row_of), f=host(b2.f), P=host(b2.P), l_aux=host(b2.l_aux)[0],
                   max_over_mean=host(b2.max_over_mean)[0], y=host(b2.y), perm_token=host(b2.perm_token)[:R],
                   a=host(b2.a)[:R], y_perm=host(b2.y_perm)[:R])
        if s.F_shared:
            two["shared_y"] = host(b2.shared_y)
        for key in one:
            assert np.array_equal(np.asarray(one[key]), np.asarray(two[key]), equal_nan=False), key
        fused = s.dtype == "bf16" and s.T <= 64 and s.T * s.k <= 512
        log(f"[{s.name}] layer call {'(one-block selection, dispatch and statistics) ' if fused else ''}"
            f"bit-identical to the separate calls")
        run_state["bufs"] = b
        full_check(inp, out)
    finally:
        run_state.clear()
        run.free()


def test_determinism_two_runs_bitwise():
    inp = minp.LayerInputs(SMALL[4], seed=3)
    run = LayerRun(inp)
    a = run.run()
    b = run.run()
    R = int(a["offsets"][-1])
    for key in a:
        u, v = np.asarray(a[key]), np.asarray(b[key])
        if key == "perm_token":
            u, v = u[:R], v[:R]
        assert np.array_equal(u, v), key
    run.free()


def test_zero_router_ties_pick_lowest_experts():
    shape = SMALL[0]
    inp = minp.LayerInputs(shape, seed=1)
    inp.w_router = np.zeros_like(inp.w_router)
    run = LayerRun(inp)
    out = run.run()
    assert (out["idx"] == np.arange(shape.k)).all()
    assert (out["near_tie"] == 1).all()
    np.testing.assert_allclose(out["w"], 1.0 / shape.k, rtol=1e-6)
    assert out["max_over_mean"] == np.float32(shape.E / shape.k)
    check_dispatch(inp, out)
    run.free()


def test_bias_update_matches_oracle_bitwise():
    """moe_bias_update against the oracle's step on the same counts: float32,
    bit-exact; the even share (counts E = T k) leaves the bias unchanged."""
    rng = np.random.default_rng(5)
    for T, k, E in [(64, 8, 128), (100, 2, 8), (7, 3, 5), (300, 4, 256)]:
        counts = rng.multinomial(T * k, np.full(E, 1.0 / E)).astype(np.int32)
        if (T * k) % E == 0:
            counts[0] = T * k // E  # one expert at exactly its share
            counts[1] = T * k - counts[0] - counts[2:].sum()
        b0 = (rng.normal(size=E) * 0.1).astype(np.float32)
        bd = torch.from_numpy(b0.copy()).cuda()
        cd = torch.from_numpy(counts).cuda()
        _lib.moe_bias_update(cd, T, k, E, 0.003, bd)
        torch.cuda.synchronize()
        assert np.array_equal(host(bd), oracle.bias_update(b0, counts, T, k, 0.003)), (T, k, E)


def test_bias_balancing_loop_on_gpu():
    """The router kernels with a selection bias, the dispatch counts and the bias
    step, iterated on the GPU on a router skewed toward low-numbered experts
    ([RS] "Keeping the load even"): each step's bias equals the oracle's step on
    the GPU's counts, and the busiest expert's share falls toward the fair share."""
    shape = S("bias_loop", "bf16", 256, 256, 8, 1, 128, 0, SM_TK, False, None, False)
    inp = minp.LayerInputs(shape, seed=0)
    skew = np.float32(0.3) * np.arange(shape.E, dtype=np.float32)
    run = LayerRun(inp)
    run.weights.bias = torch.from_numpy(-skew).cuda()        # a skewed logit bias
    run.weights.select_bias = torch.zeros(shape.E, dtype=torch.float32, device="cuda")
    b_host = np.zeros(shape.E, np.float32)
    shares = []
    for _ in range(20):
        run.layer.route(run.x, run.bufs)
        run.layer.permute(run.x, run.bufs)
        run.layer.bias_update(run.bufs, 0.02)
        torch.cuda.synchronize()
        counts = host(run.bufs.counts)
        assert counts.sum() == shape.T
        shares.append(counts.max() / shape.T)
        b_host = oracle.bias_update(b_host, counts, shape.T, shape.k, 0.02)
        assert np.array_equal(host(run.weights.select_bias), b_host)
    log(f"[bias_loop] busiest share by step: {' '.join(f'{v:.2f}' for v in shares)}")
    assert shares[0] > 0.3
    assert min(shares[5:]) < 0.125 + 0.05
    run.free()


@pytest.mark.parametrize("T,E,k,phi", [(40, 8, 2, 1.0), (300, 16, 4, 0.8), (700, 8, 3, 1.25)])
def test_padded_dispatch_matches_oracle(T, E, k, phi):
    """Capacity-padded layout, bit-exact: counts, offsets e*C, slots (rank order,
    -1 padding), row_of, and the gathered slot rows with zero padding."""
    shape = S("padded", "bf16", T, 128, E, k, 128, 0, SM_TK, True, phi, False)
    inp = minp.LayerInputs(shape, seed=2)
    run = LayerRun(inp)
    run.layer.route(run.x, run.bufs)
    C = oracle.capacity(T, k, E, phi)
    slot = torch.empty(E * C, dtype=torch.int32, device="cuda")
    xs = torch.empty((E * C, shape.d), dtype=torch.bfloat16, device="cuda")
    b = run.bufs
    _lib.moe_permute_padded(b.topk_idx, T, k, E, C, run.x, shape.d, b.counts, b.offsets, b.row_of, slot, xs,
                            b.ws_permute)
    torch.cuda.synchronize()
    idx = host(b.topk_idx)
    counts, offsets, row_of, slot_token = oracle.dispatch_padded(idx, E, C)
    assert np.array_equal(host(b.counts), counts)
    assert np.array_equal(host(b.offsets), offsets)
    assert np.array_equal(host(b.row_of), row_of)
    assert np.array_equal(host(slot), slot_token)
    x_ref = oracle.gather_slots(minp.as_f32(inp.x, "bf16"), slot_token)
    assert np.array_equal(host(xs), x_ref)
    run.free()


@pytest.mark.parametrize("T,k,E,phi,padded", [
    (20000, 8, 128, None, False),   # 313 dispatch blocks, dropless
    (17000, 8, 256, 1.0, False),    # 266 blocks, capacity
    (40000, 4, 64, 0.9, False),     # 313 blocks, capacity below the even share
    (20000, 8, 128, 1.25, True),    # capacity-padded layout
])
def test_dispatch_beyond_one_rank_launch(T, k, E, phi, padded):
    """More than 256 dispatch blocks (T k > 131072): the histogram, the scan over
    blocks and experts, and the ranks run as three launches.  Counts, offsets,
    row_of and the permutation bit-exact against the oracle, on random distinct
    experts per token with a skewed expert popularity."""
    rng = np.random.default_rng(T + E)
    pop = rng.permutation(E)
    keys = rng.random((T, E)) * (1.0 + pop / E)[None, :]        # some experts chosen more often
    idx = np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    assert (T * k + 511) // 512 > 256
    cap = oracle.capacity(T, k, E, phi)
    d = 128
    dev_idx = torch.from_numpy(idx).cuda()
    x = torch.zeros((T, d), dtype=torch.bfloat16, device="cuda")
    counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    row_of = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(_lib.moe_permute_workspace_bytes(T, k, E), 1), dtype=torch.uint8, device="cuda")
    if padded:
        slot = torch.full((E * cap,), -7, dtype=torch.int32, device="cuda")
        _lib.moe_permute_padded(dev_idx, T, k, E, cap, x, d, counts, offsets, row_of, slot, None, ws)
        torch.cuda.synchronize()
        c_ref, o_ref, r_ref, s_ref = oracle.dispatch_padded(idx, E, cap)
        assert np.array_equal(host(slot), s_ref)
    else:
        perm = torch.full((T * k,), -7, dtype=torch.int32, device="cuda")
        _lib.moe_permute(dev_idx, T, k, E, -1 if cap is None else cap, x, d, counts, offsets, row_of, perm, None, ws)
        torch.cuda.synchronize()
        c_ref, o_ref, r_ref, p_ref = oracle.dispatch(idx, E, cap)
        assert np.array_equal(host(perm)[:len(p_ref)], p_ref)
    assert np.array_equal(host(counts), c_ref)
    assert np.array_equal(host(offsets), o_ref)
    assert np.array_equal(host(row_of), r_ref)
    dropped = int((r_ref < 0).sum())
    if phi is not None and phi < 1.0:
        assert dropped > 0
    log(f"[dispatch T={T} k={k} E={E} phi={phi} padded={padded}] {(T * k + 511) // 512} blocks, "
        f"{dropped} dropped: bit-exact")


@pytest.mark.parametrize("shape", [
    S("padded_layer", "bf16", 600, 256, 8, 2, 256, 0, TK_SM, False, 1.0, False),
    S("padded_layer_shared", "bf16", 500, 256, 16, 4, 384, 256, SM_TK, True, 1.25, False),
], ids=lambda s: s.name)
def test_padded_layout_layer_matches_compact(shape):
    """The layer over the padded layout (grouped GEMMs over all E*C slots, offsets
    e*C, rows gathered through slot_token) gives the same y as the compact layout,
    bit for bit (every row is computed by the same kernel with the same K order),
    and matches the oracle."""
    inp = minp.LayerInputs(shape, seed=4)
    run = LayerRun(inp)
    out = run.run()                                     # the compact layout
    y_compact = out["y"]
    s, b, lay = shape, run.bufs, run.layer
    C = oracle.capacity(s.T, s.k, s.E, s.phi)
    slots = s.E * C
    assert s.T * s.k > 32 * s.E and slots > 32 * s.E   # both layouts take the tile kernel
    slot = torch.empty(slots, dtype=torch.int32, device="cuda")
    a = torch.empty((slots, s.F), dtype=torch.bfloat16, device="cuda")
    yp = torch.empty((slots, s.d), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((s.T, s.d), dtype=torch.bfloat16, device="cuda")
    _lib.moe_permute_padded(b.topk_idx, s.T, s.k, s.E, C, run.x, s.d, b.counts, b.offsets, b.row_of, slot, None,
                            b.ws_permute)
    w = run.weights
    _lib.moe_grouped_gate_up(run.x, slot, s.T, b.offsets, s.E, slots, s.d, s.F, w.gate, w.up, a)
    _lib.moe_grouped_down(a, b.offsets, s.E, slots, s.F, s.d, w.down, yp)
    if s.F_shared:
        lay.shared_expert(run.x, b)
    _lib.moe_combine(yp, b.row_of, b.topk_w, b.shared_y if s.F_shared else None, s.T, s.k, s.d, y, y_rows=slots)
    torch.cuda.synchronize()
    assert np.array_equal(host(y), y_compact)
    # the scatter combine over the padded slots (padding slots hold token -1)
    ws = torch.empty(_lib.moe_down_combine_workspace_bytes(s.T, s.d, slots), dtype=torch.uint8, device="cuda")
    y_sc = torch.empty((s.T, s.d), dtype=torch.bfloat16, device="cuda")
    _lib.moe_grouped_down_combine(a, b.offsets, s.E, slots, s.F, s.d, w.down, slot, b.row_of, b.topk_w, s.T, s.k,
                                  b.shared_y if s.F_shared else None, y_sc, ws)
    torch.cuda.synchronize()
    assert_same_sum(host(y_sc), y_compact, s.dtype, "padded scatter combine")
    ex = ExpertCache(inp)
    full = oracle.layer_forward(minp.as_f32(inp.x, s.dtype), minp.as_f32(inp.w_router, s.dtype), inp.bias, ex,
                                ex.shared(), k=s.k, mode=s.mode, renorm=s.renorm, phi=s.phi, alpha=s.alpha,
                                dtype=s.dtype)
    same = ~(out["idx"] != full["idx"]).any(1) & ~((out["near_tie"] == 1) | (full["near_tie"] == 1))
    err = np.abs(host(y)[same] - full["y64"][same]).max()
    assert err <= TOL[s.dtype] * np.abs(full["y64"]).max()
    run.free()


@pytest.mark.parametrize("name", ["small_zipf", "small_renorm", "small_shared"])
def test_statistics_on_a_side_stream_match_serial(name):
    """forward() given a second stream (the statistics fork before the combine when
    groups are large, stay serial when small) gives bit-identical outputs to the
    serial chain, over repeated steps on the same buffers."""
    shape = next(s for s in SMALL if s.name == name)
    inp = minp.LayerInputs(shape, seed=5)
    run = LayerRun(inp)
    ref = run.run()
    main, side = torch.cuda.Stream(), torch.cuda.Stream()
    for step in range(3):
        run.layer.forward(run.x, run.bufs, main, side_stream=side)
        main.synchronize()
        b = run.bufs
        for key, t in [("y", b.y), ("f", b.f), ("P", b.P), ("counts", b.counts), ("scores", b.logits)]:
            assert np.array_equal(host(t), ref[key]), f"{key} differs at step {step}"
        assert host(b.l_aux)[0] == ref["l_aux"] and host(b.max_over_mean)[0] == ref["max_over_mean"]
    log(f"[{name}] side-stream statistics bit-identical over 3 steps")
    run.free()


def test_zero_tokens_is_a_no_op():
    shape = SMALL[0].with_(T=0)
    inp = minp.LayerInputs(shape, seed=0)
    run = LayerRun(inp)
    run.layer.forward(run.x, run.bufs)
    torch.cuda.synchronize()
    run.free()


@pytest.mark.parametrize("dtype,sizes", [
    ("bf16", [0, 1, 255, 256, 257, 600, 513, 170]),            # 256-row tiles (K = 256 and 384)
    ("bf16", [0, 1, 127, 128, 129, 300]),                      # 192-row tiles
    ("bf16", [0, 1, 63, 64, 65, 127, 128, 129, 3]),            # small groups: 128-row tiles
    ("bf16", [0, 1, 191, 192, 193, 150, 128, 129, 64]),        # mid-size groups: 192-row tiles
    ("f32", [0, 1, 127, 128, 129, 300]),
    # few rows per group on average: groups of up to 16 rows on the skinny kernel, the
    # larger ones (17 .. 64 rows) on 128-row tiles, in one call
    ("bf16", [0, 1, 3, 16, 17, 0, 31, 33, 64, 2, 5, 0, 40, 7] + [0] * 18),
    ("bf16", [0, 1, 3, 16, 2, 0, 5, 16]),                      # skinny only; the tiled launch finds no group
    ("bf16", [0, 1, 3, 5, 2]),                                 # skinny only, no tiled launch (max_rows <= 16)
])
def test_grouped_gemm_hand_made_groups(dtype, sizes):
    """Ragged groups (empty, single row, tile edges), rows left outside every group,
    called directly through the C ABI."""
    rng = np.random.default_rng(4)
    d, F = (256, 384) if dtype == "bf16" else (40, 24)
    G = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    max_rows = int(offsets[-1]) + (37 if max(sizes) > 64 else 3)  # rows beyond the last group
    td = torch.bfloat16 if dtype == "bf16" else torch.float32

    def mk(shape, scale):
        v = (rng.standard_normal(shape) * scale).astype(np.float32)
        return minp.bf16_bits_to_f32(minp.f32_to_bf16_bits(v)) if dtype == "bf16" else v

    xp = mk((max_rows, d), 1.0)
    wg, wu, wd = mk((G, F, d), d ** -0.5), mk((G, F, d), d ** -0.5), mk((G, d, F), F ** -0.5)
    dev = lambda a: torch.from_numpy(a).cuda().to(td)
    a = torch.full((max_rows, F), 7.0, dtype=td, device="cuda")
    y = torch.full((max_rows, d), 7.0, dtype=td, device="cuda")
    off = torch.from_numpy(offsets).cuda()
    _lib.moe_grouped_swiglu(dev(xp), None, 0, off, G, max_rows, d, F, dev(wg), dev(wu), dev(wd), a, y)
    torch.cuda.synchronize()
    a_ref, y_ref = oracle.grouped_swiglu(xp, offsets, lambda e: (wg[e], wu[e], wd[e]))
    R = int(offsets[-1])
    assert max_rel(host(a)[:R], a_ref) <= TOL[dtype]
    assert max_rel(host(y)[:R], y_ref) <= TOL[dtype]
    assert (host(a)[R:] == 7.0).all() and (host(y)[R:] == 7.0).all(), "rows outside every group are untouched"
    # the same rows gathered through a row index from a shuffled source
    perm = rng.permutation(max_rows).astype(np.int32)
    src = np.empty_like(xp)
    src[perm] = xp                                          # xp[r] == src[perm[r]]
    a2 = torch.full_like(a, 7.0)
    y2 = torch.full_like(y, 7.0)
    _lib.moe_grouped_swiglu(dev(src), torch.from_numpy(perm).cuda(), max_rows, off, G, max_rows, d, F, dev(wg),
                            dev(wu), dev(wd), a2, y2)
    torch.cuda.synchronize()
    assert torch.equal(a2, a) and torch.equal(y2, y), "row-index gather must match the materialized rows"


@pytest.mark.parametrize("d,F", [(128, 128), (256, 128), (128, 384), (256, 256), (384, 512)])
def test_grouped_gemm_many_tiles_per_block(d, F):
    """256-row tiles, several per block (more tiles than blocks), with K = 128 (the
    tile's K loop is only its two next-tile steps), 256, 384 and 512 (the step-2
    loads ahead of the output stores; 384 columns also end in a 128-column n-tile):
    each block's tile boundaries, the next tile's operand loads issued in the last
    steps and the row indices fetched a tile ahead.  Against the oracle, and the
    gathered form bit for bit against the materialized one."""
    rng = np.random.default_rng(11)
    G = 64
    sizes = rng.integers(900, 1400, size=G)
    sizes[5] = 0
    sizes[17] = 1
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    max_rows = int(offsets[-1]) + 5

    def mk(shape, scale):
        v = (rng.standard_normal(shape) * scale).astype(np.float32)
        return minp.bf16_bits_to_f32(minp.f32_to_bf16_bits(v))

    xp = mk((max_rows, d), 1.0)
    wg, wu, wd = mk((G, F, d), d ** -0.5), mk((G, F, d), d ** -0.5), mk((G, d, F), F ** -0.5)
    dev = lambda a: torch.from_numpy(a).cuda().to(torch.bfloat16)
    a = torch.full((max_rows, F), 7.0, dtype=torch.bfloat16, device="cuda")
    y = torch.full((max_rows, d), 7.0, dtype=torch.bfloat16, device="cuda")
    off = torch.from_numpy(offsets).cuda()
    log(f"[many_tiles d={d} F={F}] {int(offsets[-1])} rows in {G} groups")
    _lib.moe_grouped_swiglu(dev(xp), None, 0, off, G, max_rows, d, F, dev(wg), dev(wu), dev(wd), a, y)
    torch.cuda.synchronize()
    a_ref, y_ref = oracle.grouped_swiglu(xp, offsets, lambda e: (wg[e], wu[e], wd[e]))
    R = int(offsets[-1])
    assert max_rel(host(a)[:R], a_ref) <= TOL["bf16"]
    assert max_rel(host(y)[:R], y_ref) <= TOL["bf16"]
    assert (host(a)[R:] == 7.0).all() and (host(y)[R:] == 7.0).all(), "rows outside every group are untouched"
    perm = rng.permutation(max_rows).astype(np.int32)
    src = np.empty_like(xp)
    src[perm] = xp
    a2 = torch.full_like(a, 7.0)
    y2 = torch.full_like(y, 7.0)
    _lib.moe_grouped_swiglu(dev(src), torch.from_numpy(perm).cuda(), max_rows, off, G, max_rows, d, F, dev(wg),
                            dev(wu), dev(wd), a2, y2)
    torch.cuda.synchronize()
    assert torch.equal(a2, a) and torch.equal(y2, y), "row-index gather must match the materialized rows"


@pytest.mark.parametrize("dtype,shared", [("bf16", True), ("bf16", False), ("f32", True)])
@pytest.mark.parametrize("k", [2, 3, 8])
def test_combine_with_every_slot_dropped_reads_no_row(dtype, shared, k):
    """y_rows = 0 (an empty y_perm, every slot dropped): the combine reads no row
    of y_perm, which may be absent, and y is the shared expert's output (or 0)."""
    T, d = 37, 256
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator().manual_seed(5)
    sh = torch.randn(T, d, generator=g).to(td).cuda() if shared else None
    row_of = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.rand(T, k, generator=g).cuda()
    y = torch.full((T, d), float("nan"), dtype=td, device="cuda")
    _lib.moe_combine(None, row_of, w, sh, T, k, d, y, y_rows=0)
    torch.cuda.synchronize()
    want = host(sh) if shared else np.zeros((T, d), np.float32)
    assert np.array_equal(host(y), want)
    log(f"[combine empty y_perm {dtype} k={k} shared={shared}] y equals the shared rows exactly")


def test_stats_on_the_worked_example_as_one_token_batch(golden):
    """moe_stats straight against the pages: one token whose router probabilities
    are The Residual Stream's worked example (scores ln p), k = 2 of 4 experts.
    P = the printed probabilities, f = (1/2, 1/2, 0, 0), E sum f P = 1.6."""
    g = golden("balance_pi_rs.txt")
    E, k = int(g["E"]), int(g["k"])
    logits = torch.from_numpy(np.log(np.array([g["probs"]], np.float64)).astype(np.float32)).cuda()
    counts = torch.tensor([1, 1, 0, 0], dtype=torch.int32, device="cuda")
    f, P = torch.empty(E, device="cuda"), torch.empty(E, device="cuda")
    l_aux, mom = torch.empty(1, device="cuda"), torch.empty(1, device="cuda")
    ws = torch.empty(max(_lib.moe_stats_workspace_bytes(1, E), 1), dtype=torch.uint8, device="cuda")
    _lib.moe_stats(counts, logits, 1, k, E, 1.0, f, P, l_aux, mom, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(f), np.array(g["f_expected"], np.float32))
    np.testing.assert_allclose(host(P), g["P_expected"], rtol=1e-6)
    assert host(l_aux)[0] == pytest.approx(g["balance_term_expected"], rel=1e-6)
    assert host(mom)[0] == 2.0
