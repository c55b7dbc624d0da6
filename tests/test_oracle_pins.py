"""Pins for the CPU oracle: each test checks the oracle against something
other than itself -- a hand-worked example, exact rational arithmetic, the
merge-mode identity computed by brute force, closed forms, invariants the
definition implies, and a textbook stable sort.

Pages cited:
  [LoRA-Land]  "LoRA-Land: turning the LLM into an operating system ..."
  [vLLM-ch7]   "Multi-LoRA hot-plug: one model serving many tenants"
  [icman]      field report on Multi-LoRA in managed inference (news 62580)
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import OracleError, Registry
import workloads as wk

HERE = os.path.dirname(os.path.abspath(__file__))


def _bf16(a):
    """Round a float array to bf16 (torch RNE) and return the bf16 tensor."""
    return torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)


def _f(a):
    return oracle.bf16_bits_to_f64(a)


def _random_case(T, d_in, d_out, ranks, alphas, id_lo, seed, n_modules=1):
    """Seeded tiny case: returns registry, X (bf16), W list (bf16), ids, adapters."""
    wl = wk.small_workload(T, d_in, d_out, len(ranks), max(ranks) + 2, ranks,
                           n_modules=n_modules, key=1000 + seed)
    reg = Registry(len(ranks), len(ranks), max(ranks) + 2, [d_in] * n_modules,
                   [d_out] * n_modules, T)
    ads = {}
    for i, (r, al) in enumerate(zip(ranks, alphas)):
        AB = [wk.adapter_weights(wl, i, m, r) for m in range(n_modules)]
        A = [ab[0] for ab in AB]
        B = [ab[1] for ab in AB]
        # scale the adapter up so the LoRA term is comparable to the base term
        A = [_bf16(_f(a) * 20) for a in A]
        B = [_bf16(_f(b) * 20) for b in B]
        reg.load(i, r, al, A, B)
        ads[i] = (r, al, A, B)
    X = [wk.activation(wl, f"x{m}", d_in) for m in range(n_modules)]
    W = [wk.base_weight(wl, m) for m in range(n_modules)]
    ids = wk.uniform_ids(T, id_lo, len(ranks), seed)
    return reg, X, W, ids, ads


# --------------------------------------------------------------------------
# 1. hand-worked example (tests/golden/hand_example.json)
# --------------------------------------------------------------------------
def test_hand_example_values_and_plan():
    with open(os.path.join(HERE, "golden", "hand_example.json")) as f:
        g = json.load(f)
    reg = Registry(2, g["max_ids"], 4, [g["d_in"]], [g["d_out"]], 8)
    for sid, ad in g["adapters"].items():
        reg.load(int(sid), ad["rank"], ad["alpha"], [np.array(ad["A"], float)],
                 [np.array(ad["B"], float)])
    Y = oracle.lora_linear(reg, 0, np.array(g["X"], float), np.array(g["ids"]),
                           np.array(g["W"], float))
    assert np.array_equal(Y, np.array(g["Y"], float))
    perm, inv, seg_id, seg_off = oracle.plan(g["ids"], g["max_ids"])
    assert perm.tolist() == g["perm"]
    assert inv.tolist() == g["inv"]
    assert seg_id.tolist() == g["seg_id"]
    assert seg_off.tolist() == g["seg_off"]


# --------------------------------------------------------------------------
# 2. exact rational arithmetic within the float64 summation error bound
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed,d_in,d_out", [(0, 7, 6), (1, 7, 6), (2, 6, 6), (5, 5, 5)])
def test_exact_rational_within_error_bound(seed, d_in, d_out):
    # square shapes too: there a transposed W or A/B mix-up has the right shape
    T = 5
    ranks, alphas = [1, 3, 4], [3.0, 5.0, 8.0]      # s = 3, 5/3, 2
    reg, X, W, ids, ads = _random_case(T, d_in, d_out, ranks, alphas, -1, seed)
    Y = oracle.lora_linear(reg, 0, X[0], ids, W[0])
    Xq = [[Fraction(float(v)) for v in row] for row in _f(X[0])]
    Wq = [[Fraction(float(v)) for v in row] for row in _f(W[0])]
    u = 2.0 ** -53
    for t in range(T):
        i = int(ids[t])
        for j in range(d_out):
            exact = sum(Xq[t][k] * Wq[j][k] for k in range(d_in))
            mag = sum(abs(float(Xq[t][k] * Wq[j][k])) for k in range(d_in))
            n = d_in
            if i >= 0:
                r, al, A, B = ads[i]
                Aq = [[Fraction(float(v)) for v in row] for row in _f(A[0])]
                Bq = [[Fraction(float(v)) for v in row] for row in _f(B[0])]
                s = Fraction(al) / Fraction(r)
                uq = [sum(Xq[t][k] * Aq[k][q] for k in range(d_in)) for q in range(r)]
                exact += s * sum(uq[q] * Bq[q][j] for q in range(r))
                umag = [sum(abs(float(Xq[t][k] * Aq[k][q])) for k in range(d_in)) for q in range(r)]
                mag += float(abs(s)) * sum(umag[q] * abs(float(Bq[q][j])) for q in range(r))
                n = d_in + r + 2
            bound = 4 * n * u * mag + 1e-300
            assert abs(Y[t, j] - float(exact)) <= bound, (t, j, Y[t, j], float(exact), bound)


# --------------------------------------------------------------------------
# 3. merge mode == dynamic mode ([icman] section 2.1): brute-force merged weight
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", [3, 4])
def test_merged_weight_brute_force(seed):
    T, d_in, d_out = 9, 13, 5          # d_in != d_out: a transposed operand cannot pass
    ranks, alphas = [2, 4, 1], [4.0, 6.0, 1.5]
    reg, X, W, ids, ads = _random_case(T, d_in, d_out, ranks, alphas, -1, seed, n_modules=2)
    for m in range(2):
        Y = oracle.lora_linear(reg, m, X[m], ids, W[m])
        Xf, Wf = _f(X[m]).tolist(), _f(W[m]).tolist()
        for t in range(T):
            i = int(ids[t])
            # merged weight for this token's adapter: W' = W + s (A B)^T  (d_out x d_in)
            Wm = [row[:] for row in Wf]
            if i >= 0:
                r, al, A, B = ads[i]
                Af, Bf = _f(A[m]).tolist(), _f(B[m]).tolist()
                s = al / r
                for j in range(d_out):
                    for k in range(d_in):
                        Wm[j][k] += s * sum(Af[k][q] * Bf[q][j] for q in range(r))
            for j in range(d_out):
                ref = 0.0
                mag = 0.0
                for k in range(d_in):
                    ref += Xf[t][k] * Wm[j][k]
                    mag += abs(Xf[t][k] * Wm[j][k])
                assert abs(Y[t, j] - ref) <= 1e-12 * (mag + 1.0), (m, t, j)


# --------------------------------------------------------------------------
# 4. closed form: a one-hot token row picks one input column
# --------------------------------------------------------------------------
def test_one_hot_rows_closed_form():
    d_in, d_out, r = 6, 4, 3
    rng = np.random.default_rng(7)
    W = _f(_bf16(rng.normal(size=(d_out, d_in))))
    A = _f(_bf16(rng.normal(size=(d_in, r))))
    B = _f(_bf16(rng.normal(size=(r, d_out))))
    reg = Registry(1, 1, 4, [d_in], [d_out], d_in)
    reg.load(0, r, 1.5 * r, [A], [B])               # s = 1.5
    X = np.eye(d_in)                                 # token k is e_k
    Y = oracle.lora_linear(reg, 0, X, np.zeros(d_in, int), W)
    for k in range(d_in):
        for j in range(d_out):
            # e_k W^T = W[j, k];  e_k A = A[k, :];  (A[k,:]) B[:, j]
            want = W[j, k] + 1.5 * sum(A[k, q] * B[q, j] for q in range(r))
            assert Y[k, j] == pytest.approx(want, rel=1e-13, abs=1e-13)


def test_rank_one_outer_product_closed_form():
    # rank-1 adapter: delta = s (X a) b^T, an outer product
    T, d_in, d_out = 4, 5, 3
    a = np.array([1.0, -2.0, 0.5, 0.0, 4.0])
    b = np.array([2.0, -1.0, 0.25])
    X = np.arange(T * d_in, dtype=float).reshape(T, d_in) - 7.0
    W = np.zeros((d_out, d_in))
    reg = Registry(1, 3, 1, [d_in], [d_out], T)
    reg.load(2, 1, 5.0, [a.reshape(d_in, 1)], [b.reshape(1, d_out)])   # s = 5
    Y = oracle.lora_linear(reg, 0, X, np.full(T, 2), W)
    want = 5.0 * np.outer(X @ a, b)
    assert np.array_equal(Y, want)


# --------------------------------------------------------------------------
# 5. id -1 is pure base ([vLLM-ch7] "switching LoRA per request")
# --------------------------------------------------------------------------
def test_base_rows_equal_base_exactly():
    reg, X, W, ids, _ = _random_case(12, 16, 8, [2, 3], [4.0, 6.0], -1, 11)
    ids[::3] = -1
    Y = oracle.lora_linear(reg, 0, X[0], ids, W[0])
    Y0 = oracle.base_linear(X[0], W[0])
    for t in np.where(ids == -1)[0]:
        assert np.array_equal(Y[t], Y0[t])
    Xf, Wf = _f(X[0]), _f(W[0])
    for t in np.where(ids == -1)[0]:       # and equal to a loop-computed X W^T
        for j in range(8):
            assert Y[t, j] == pytest.approx(sum(Xf[t, k] * Wf[j, k] for k in range(16)),
                                            rel=1e-14, abs=1e-14)
    # rows with an adapter differ from base (B is not zero)
    assert not np.allclose(Y[ids >= 0], Y0[ids >= 0])


# --------------------------------------------------------------------------
# 6. per-sample branches ([icman] section 2.1): token permutation invariance
# --------------------------------------------------------------------------
def test_token_permutation_invariance():
    reg, X, W, ids, _ = _random_case(17, 24, 10, [1, 2, 4], [2.0, 4.0, 8.0], -1, 12)
    Y = oracle.lora_linear(reg, 0, X[0], ids, W[0])
    p = np.random.default_rng(5).permutation(17)
    Yp = oracle.lora_linear(reg, 0, X[0][torch.as_tensor(p)], ids[p], W[0])
    assert np.array_equal(Yp, Y[p])


# --------------------------------------------------------------------------
# 7. mixed ranks aligned to a maximum rank ([vLLM-ch7] "performance notes"):
#    zero padding is wasted work, not a different result; scale uses true r
# --------------------------------------------------------------------------
def test_zero_padding_and_true_rank_scale():
    d_in, d_out, r, pad = 8, 6, 2, 5
    rng = np.random.default_rng(9)
    A = rng.normal(size=(d_in, r))
    B = rng.normal(size=(r, d_out))
    X = rng.normal(size=(3, d_in))
    W = rng.normal(size=(d_out, d_in))
    reg = Registry(2, 2, 64, [d_in], [d_out], 3)
    reg.load(0, r, 3.0, [A], [B])                                       # s = 1.5
    Ap = np.concatenate([A, np.zeros((d_in, pad))], axis=1)
    Bp = np.concatenate([B, np.zeros((pad, d_out))], axis=0)
    reg.load(1, r + pad, 1.5 * (r + pad), [Ap], [Bp])                   # same s
    Y0 = oracle.lora_linear(reg, 0, X, np.zeros(3, int), W)
    Y1 = oracle.lora_linear(reg, 0, X, np.ones(3, int), W)
    np.testing.assert_allclose(Y0, Y1, rtol=1e-14, atol=1e-14)
    # the scale is alpha / true rank, not alpha / max_rank (max_rank is 64 here)
    want = X @ W.T + 1.5 * (X @ A) @ B
    np.testing.assert_allclose(Y0, want, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# 8. grouping by LoRA id ([LoRA-Land] section 2) == a textbook stable sort
# --------------------------------------------------------------------------
def _textbook_plan(ids):
    T = len(ids)
    perm = sorted(range(T), key=lambda t: (ids[t], t))
    inv = [0] * T
    for p, t in enumerate(perm):
        inv[t] = p
    seg_id, seg_off = [], []
    for p, t in enumerate(perm):
        if p == 0 or ids[t] != ids[perm[p - 1]]:
            seg_id.append(ids[t])
            seg_off.append(p)
    seg_off.append(T)
    return perm, inv, seg_id, seg_off


PLAN_CASES = {
    "empty": [],
    "single": [5],
    "all_base": [-1] * 70,
    "all_one": [3] * 65,
    "all_distinct": list(range(63, -1, -1)),
    "descending_dups": [9, 9, 8, 8, 7, -1, -1, 7, 0, 0],
    "ragged_base_mix": [(t * 37) % 11 - 1 for t in range(131)],
}


@pytest.mark.parametrize("name", sorted(PLAN_CASES))
def test_plan_adversarial(name):
    ids = PLAN_CASES[name]
    got = oracle.plan(ids, 2000)
    want = _textbook_plan(ids)
    for g, w in zip(got, want):
        assert g.tolist() == list(w)
    # numpy's stable argsort agrees too
    if ids:
        assert got[0].tolist() == np.argsort(np.asarray(ids), kind="stable").tolist()


@pytest.mark.parametrize("key", [1, 2, 3, 4, 5])
def test_plan_on_workload_ids(key):
    wl = wk.WORKLOADS[key]
    for seed in (wl.default_seed, 11):
        ids = wk.adapter_ids(wl, seed)
        got = oracle.plan(ids, wl.n_adapters)
        want = _textbook_plan(ids.tolist())
        for g, w in zip(got, want):
            assert g.tolist() == list(w)


def test_plan_2000_distinct_ids():
    ids = np.random.default_rng(3).permutation(2000).astype(np.int32).tolist()
    got = oracle.plan(ids, 2000)
    assert got[2].tolist() == list(range(2000))
    assert got[3].tolist() == list(range(2001))
    assert [ids[t] for t in got[0]] == list(range(2000))


def test_plan_rejects_out_of_range():
    with pytest.raises(OracleError) as e:
        oracle.plan([0, 2000], 2000)
    assert e.value.status == oracle.ID_RANGE
    with pytest.raises(OracleError) as e:
        oracle.plan([-2], 4)
    assert e.value.status == oracle.ID_RANGE


# --------------------------------------------------------------------------
# 9. registry: strict mode ([icman] section 4.1), rank limit ([vLLM-ch7]
#    --max-lora-rank, [icman] section 3.3), hot-plug ([LoRA-Land] section 3)
# --------------------------------------------------------------------------
def _tiny_adapter(rank, d_in=4, d_out=3, fill=1.0):
    return [np.full((d_in, rank), fill)], [np.full((rank, d_out), fill)]


def test_registry_error_codes():
    reg = Registry(2, 10, 8, [4], [3], 16)
    A, B = _tiny_adapter(8)
    with pytest.raises(OracleError) as e:
        reg.load(0, 9, 18.0, *_tiny_adapter(9))
    assert e.value.status == oracle.RANK
    with pytest.raises(OracleError) as e:
        reg.load(0, 0, 1.0, *_tiny_adapter(1))
    assert e.value.status == oracle.RANK
    with pytest.raises(OracleError) as e:
        reg.load(10, 2, 4.0, *_tiny_adapter(2))
    assert e.value.status == oracle.ID_RANGE
    reg.load(0, 8, 16.0, A, B)
    with pytest.raises(OracleError) as e:
        reg.load(0, 8, 16.0, A, B)
    assert e.value.status == oracle.EXISTS
    reg.load(1, 2, 4.0, *_tiny_adapter(2))
    with pytest.raises(OracleError) as e:
        reg.load(2, 2, 4.0, *_tiny_adapter(2))
    assert e.value.status == oracle.POOL_FULL
    with pytest.raises(OracleError) as e:
        reg.unload(5)
    assert e.value.status == oracle.NOT_LOADED
    reg.unload(1)
    reg.load(2, 2, 4.0, *_tiny_adapter(2))


def test_strict_mode_rejects_unloaded_and_out_of_range_ids():
    reg = Registry(4, 4, 4, [4], [3], 16)
    reg.load(1, 2, 4.0, *_tiny_adapter(2))
    X, W = np.ones((3, 4)), np.ones((3, 4))
    with pytest.raises(OracleError) as e:
        oracle.lora_linear(reg, 0, X, [1, 2, -1], W)     # id 2 not loaded
    assert e.value.status == oracle.NOT_LOADED
    with pytest.raises(OracleError) as e:
        oracle.lora_linear(reg, 0, X, [2, 4, 1], W)      # out of range wins
    assert e.value.status == oracle.ID_RANGE
    with pytest.raises(OracleError) as e:
        oracle.lora_linear(reg, 0, X, [1, -2, 1], W)
    assert e.value.status == oracle.ID_RANGE


def test_hot_plug_round_trip():
    reg, X, W, ids, ads = _random_case(10, 8, 6, [2, 3], [4.0, 6.0], 0, 21)
    Y1 = oracle.lora_linear(reg, 0, X[0], ids, W[0])
    reg.unload(1)
    if (ids == 1).any():
        with pytest.raises(OracleError) as e:
            oracle.lora_linear(reg, 0, X[0], ids, W[0])
        assert e.value.status == oracle.NOT_LOADED
    r, al, A, B = ads[1]
    reg.load(1, r, al, A, B)
    Y2 = oracle.lora_linear(reg, 0, X[0], ids, W[0])
    assert np.array_equal(Y1, Y2)


def test_sampled_matches_full():
    reg, X, W, ids, _ = _random_case(11, 16, 12, [2, 3, 1], [4.0, 3.0, 2.0], -1, 31)
    Y = oracle.lora_linear(reg, 0, X[0], ids, W[0])
    rows = np.array([0, 3, 10])
    cols = np.array([1, 5, 11, 7])
    Ys = oracle.lora_linear_sampled(reg, 0, X[0][torch.as_tensor(rows)], ids[rows],
                                    W[0][torch.as_tensor(cols)], cols)
    np.testing.assert_allclose(Ys, Y[np.ix_(rows, cols)], rtol=1e-13, atol=1e-13)


def test_parity_metrics_detect_a_dropped_delta():
    # the tolerances must be able to see a missing or doubled LoRA term at the
    # workloads' value scales (X ~ N(0,1), W, A, B ~ N(0, 0.02))
    wl = wk.WORKLOADS[1]
    reg = Registry(4, 4, 8, [1024], [1024], 64)
    for i in range(4):
        A, B = wk.adapter_weights(wl, i, 0, 8)
        reg.load(i, 8, 16.0, [A], [B])
    X = wk.activation(wl, "x", 1024)
    W = wk.base_weight(wl, 0)
    ids = wk.adapter_ids(wl)
    Y = oracle.lora_linear(reg, 0, X, ids, W)
    Y0 = oracle.base_linear(X, W)
    good = torch.as_tensor(Y, dtype=torch.float32).to(torch.bfloat16)
    mx, rl1, _ = oracle.parity_metrics(good, Y)
    assert mx <= oracle.MAX_REL_TOL and rl1 <= oracle.RELL1_TOL
    dropped = torch.as_tensor(Y0, dtype=torch.float32).to(torch.bfloat16)
    mx, rl1, _ = oracle.parity_metrics(dropped, Y)
    assert mx > oracle.MAX_REL_TOL or rl1 > oracle.RELL1_TOL
    doubled = torch.as_tensor(2 * Y - Y0, dtype=torch.float32).to(torch.bfloat16)
    mx, rl1, _ = oracle.parity_metrics(doubled, Y)
    assert mx > oracle.MAX_REL_TOL or rl1 > oracle.RELL1_TOL


def test_target_sets_skip_untargeted_modules():
    """An adapter without pages for a module is pure base there ([vLLM-ch7]
    performance notes, skip path): its rows equal X W^T exactly, and on the
    modules it does target it equals the same adapter loaded with every
    module (and the merged weight of the pinned brute force)."""
    g = np.random.default_rng(5)
    d_in, d_out, T = 6, 5, 7
    full = Registry(3, 3, 4, [d_in] * 3, [d_out] * 3, T)
    part = Registry(3, 3, 4, [d_in] * 3, [d_out] * 3, T)
    As = [np.round(g.standard_normal((d_in, 3)) * 8) / 8 for _ in range(3)]
    Bs = [np.round(g.standard_normal((3, d_out)) * 8) / 8 for _ in range(3)]
    full.load(0, 3, 6.0, As, Bs)
    part.load(0, 3, 6.0, [As[0], None, As[2]], [Bs[0], None, Bs[2]])
    X = np.round(g.standard_normal((T, d_in)) * 4) / 4
    W = np.round(g.standard_normal((d_out, d_in)) * 4) / 4
    ids = np.array([0, -1, 0, 0, -1, 0, 0])
    for m in (0, 2):
        np.testing.assert_array_equal(oracle.lora_linear(part, m, X, ids, W),
                                      oracle.lora_linear(full, m, X, ids, W))
    np.testing.assert_array_equal(oracle.lora_linear(part, 1, X, ids, W), X @ W.T)
    # the targeted module against the merged weight W + s (A B)^T, by loops
    Wm = [[W[j][k] + 2.0 * sum(As[0][k][q] * Bs[0][q][j] for q in range(3)) for k in range(d_in)]
          for j in range(d_out)]
    Y = oracle.lora_linear(part, 0, X, ids, W)
    for t in range(T):
        if ids[t] < 0:
            continue
        for j in range(d_out):
            ref = sum(X[t][k] * Wm[j][k] for k in range(d_in))
            assert abs(Y[t, j] - ref) <= 1e-12 * (1 + abs(ref))
    with pytest.raises(OracleError) as e:
        part.load(1, 3, 6.0, [None] * 3, [None] * 3)
    assert e.value.status == oracle.INVALID_ARG
    with pytest.raises(OracleError) as e:
        part.load(1, 3, 6.0, [As[0], None, As[2]], [Bs[0], Bs[1], Bs[2]])
    assert e.value.status == oracle.INVALID_ARG


def test_round_to_bf16_matches_torch_rne():
    """The oracle's bf16 rounding against torch's float32 -> bfloat16 cast (round
    to nearest even), on random values, ties and values near powers of two."""
    g = np.random.default_rng(9)
    v = np.concatenate([g.standard_normal(4000).astype(np.float32) * 3,
                        (np.arange(-300, 300, dtype=np.float32) + 0.5) * 2.0 ** -7,
                        np.float32([1.00390625, 1.01171875, -1.00390625, 255.5, 0.0])])
    ref = torch.as_tensor(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_to_bf16(v.astype(np.float64)), ref)


def test_dequant_q4_against_elementwise_definition():
    """W[n, k] = bf16((q - z) s) per 128-wide group, by plain loops over a
    tiny weight, with groups that differ in zero point and scale."""
    g = np.random.default_rng(4)
    N, K = 3, 256
    q = g.integers(0, 16, size=(N, K))
    z = g.integers(0, 16, size=(N, K // 128))
    s = _bf16(np.abs(g.standard_normal((N, K // 128))) * 0.01)
    W = oracle.dequant_q4(q, z, s)
    sf = _f(s)
    for n in range(N):
        for k in range(K):
            exact = float((int(q[n, k]) - int(z[n, k // 128]))) * float(sf[n, k // 128])
            assert W[n, k] == float(torch.tensor(exact, dtype=torch.float32).to(torch.bfloat16))
    # a zero point equal to q gives exact zeros; scale 1 and z 0 give q itself
    q2 = np.full((1, 128), 9)
    assert not oracle.dequant_q4(q2, np.array([[9]]), _bf16([[0.5]])).any()
    np.testing.assert_array_equal(oracle.dequant_q4(np.arange(128).reshape(1, 128) % 16, np.array([[0]]),
                                                    _bf16([[1.0]]))[0], np.arange(128) % 16)


def test_chain_is_the_sum_of_its_members():
    """A chain ([LoRA-Land] set_adaptive_chain) adds each member's update: its
    term equals the members' terms computed one adapter at a time, the merged
    weight W + sum_c s_c (A_c B_c)^T by loops, and a chain of one adapter
    equals that adapter."""
    g = np.random.default_rng(8)
    d_in, d_out, T = 6, 5, 6
    reg = Registry(8, 8, 48, [d_in], [d_out], T)
    params = {0: (3, 6.0), 1: (5, 7.5), 2: (16, 32.0)}
    mats = {}
    for i, (r, al) in params.items():
        A = np.round(g.standard_normal((d_in, r)) * 8) / 8
        B = np.round(g.standard_normal((r, d_out)) * 8) / 8
        mats[i] = (A, B, al / r)
        reg.load(i, r, al, [A], [B])
    reg.load_chain(5, [0, 1, 2])
    reg.load_chain(6, [2, 0])
    reg.load_chain(7, [1])
    X = np.round(g.standard_normal((T, d_in)) * 4) / 4
    W = np.round(g.standard_normal((d_out, d_in)) * 4) / 4
    Y0 = X @ W.T
    single = {i: oracle.lora_linear(reg, 0, X, np.full(T, i), W) - Y0 for i in params}
    Yc = oracle.lora_linear(reg, 0, X, np.full(T, 5), W)
    np.testing.assert_allclose(Yc - Y0, single[0] + single[1] + single[2], rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.lora_linear(reg, 0, X, np.full(T, 6), W) - Y0,
                               single[2] + single[0], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(oracle.lora_linear(reg, 0, X, np.full(T, 7), W),
                                  oracle.lora_linear(reg, 0, X, np.full(T, 1), W))
    Wm = [[W[j][k] + sum(mats[i][2] * sum(mats[i][0][k][q] * mats[i][1][q][j]
                                           for q in range(params[i][0])) for i in (0, 1, 2))
           for k in range(d_in)] for j in range(d_out)]
    for t in range(T):
        for j in range(d_out):
            ref = sum(X[t][k] * Wm[j][k] for k in range(d_in))
            assert abs(Yc[t, j] - ref) <= 1e-9 * (1 + abs(ref))
    # the chain is a snapshot: unloading a member leaves it intact
    reg.unload(0)
    np.testing.assert_array_equal(oracle.lora_linear(reg, 0, X, np.full(T, 5), W), Yc)
    for members, status in [([1, 1], oracle.INVALID_ARG), ([], oracle.INVALID_ARG),
                            ([0, 1], oracle.NOT_LOADED), ([5, 1], oracle.INVALID_ARG),
                            ([2, 2 + 0], oracle.INVALID_ARG), ([9], oracle.ID_RANGE)]:
        with pytest.raises(OracleError) as e:
            reg.load_chain(3, members)
        assert e.value.status == status, members
    reg.load(3, 16, 32.0, [np.ones((d_in, 16))], [np.ones((16, d_out))])
    reg.load(0, 16, 32.0, [np.ones((d_in, 16))], [np.ones((16, d_out))])
    with pytest.raises(OracleError) as e:
        reg.load_chain(4, [2, 3, 0, 1])                       # 16 + 16 + 16 + 5 = 53 > 48
    assert e.value.status == oracle.RANK
    reg.load_chain(4, [2, 3, 1])                              # 16 + 16 + 5 = 37 fits


def test_chain_rank_is_the_sum_of_member_ranks():
    """A chain is one adapter of rank sum_c r_c, refused only above the pool's
    max rank ([vLLM-ch7] "starting a multi-LoRA service", --max-lora-rank;
    [icman] section 3.3).  Pinned where a block-padded rule would differ:
    three rank-5 adapters (15) fit a max rank of 16, a fourth (20) does not,
    and a sum of exactly the max rank fits; the accepted chain's term is the
    members' terms added."""
    g = np.random.default_rng(21)
    d_in, d_out, T = 7, 4, 5
    reg = Registry(12, 12, 16, [d_in], [d_out], T)
    mats = {}
    for i, r in enumerate([5, 5, 5, 5, 11, 1]):
        A = np.round(g.standard_normal((d_in, r)) * 8) / 8
        B = np.round(g.standard_normal((r, d_out)) * 8) / 8
        mats[i] = (A, B)
        reg.load(i, r, 2.0 * r, [A], [B])
    reg.load_chain(6, [0, 1, 2])                               # 5 + 5 + 5 = 15 <= 16
    reg.load_chain(7, [4, 0])                                  # 11 + 5 = 16 == max rank
    for members in ([0, 1, 2, 3], [4, 0, 5], [4, 1, 2]):       # 20, 17, 21 > 16
        with pytest.raises(OracleError) as e:
            reg.load_chain(8, members)
        assert e.value.status == oracle.RANK, members
    X = np.round(g.standard_normal((T, d_in)) * 4) / 4
    W = np.round(g.standard_normal((d_out, d_in)) * 4) / 4
    ref = X @ W.T + sum(2.0 * (X @ mats[i][0]) @ mats[i][1] for i in (0, 1, 2))
    np.testing.assert_allclose(oracle.lora_linear(reg, 0, X, np.full(T, 6), W), ref, rtol=0, atol=1e-12)
