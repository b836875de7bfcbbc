"""Pins for the float64 CPU oracle (no GPU).

Each test checks the oracle against something other than itself: hand-worked examples,
closed forms that the mathematics fixes, the duality between the recurrent and the
quadratic form, the block decomposition at many chunk lengths, and invariants (split and
resume, packing, linearity, group sharing).  Citations are to the page "Transformers are
SSMs" (paper summary) unless stated otherwise.
"""
import os

import numpy as np
import pytest

import oracle
from workloads import bf16_round, make_inputs, packed_lengths

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ALL_FORMS = ("recurrence", "recurrence_np", "quadratic", "chunked1", "chunked2", "chunked3")


def run_form(form, X, logA, B, C, init=None, seq_offsets=None):
    if form == "recurrence":
        return oracle.recurrence(X, logA, B, C, init, seq_offsets)
    if form == "recurrence_np":
        return oracle.recurrence_np(X, logA, B, C, init, seq_offsets)
    if form == "quadratic":
        return oracle.quadratic(X, logA, B, C, init, seq_offsets)
    if form.startswith("chunked"):
        return oracle.chunked(X, logA, B, C, int(form[len("chunked"):]), init, seq_offsets)
    raise ValueError(form)


def rand_problem(seed, b=2, T=37, H=4, P=6, N=5, G=2, init=True, nseq=None):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((b, T, H, P))
    B = rng.standard_normal((b, T, G, N)) / np.sqrt(N)
    C = rng.standard_normal((b, T, G, N)) / np.sqrt(N)
    logA = -rng.uniform(0.001, 0.5, size=(b, T, H))
    ns = b if nseq is None else nseq
    I = rng.standard_normal((ns, H, P, N)) * 0.3 if init else None
    return X, logA, B, C, I


def rel(a, b):
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


# --------------------------------------------------------------------------- worked examples

def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


@pytest.mark.parametrize("form", ALL_FORMS)
def test_worked_scalar_ssm(form):
    """Section 3.2.2 / appendix B: h_t = a_t h_{t-1} + x_t, hand-computed values."""
    rows = _golden_lines("scalar_ssm_worked.txt")
    init = float(rows[0][1])
    data = np.array([[float(v) for v in r] for r in rows[1:-1]])
    final = float(rows[-1][1])
    T = data.shape[0]
    X = data[:, 2].reshape(1, T, 1, 1)
    logA = np.log(data[:, 1]).reshape(1, T, 1)
    ones = np.ones((1, T, 1, 1))
    Y, F = run_form(form, X, logA, ones, ones, np.full((1, 1, 1, 1), init))
    np.testing.assert_allclose(Y.reshape(-1), data[:, 3], rtol=0, atol=1e-14)
    np.testing.assert_allclose(F.reshape(-1), [final], rtol=0, atol=1e-14)


@pytest.mark.parametrize("form", ALL_FORMS)
def test_worked_p2_n3(form):
    """One head with P=2, N=3: state orientation S[p][n] and the outer product x B^T."""
    g = {r[0]: [float(v) for v in r[1:]] for r in _golden_lines("ssd_p2_n3_worked.txt")}
    X = np.array([g["x0"], g["x1"]]).reshape(1, 2, 1, 2)
    B = np.array([g["B0"], g["B1"]]).reshape(1, 2, 1, 3)
    C = np.array([g["C0"], g["C1"]]).reshape(1, 2, 1, 3)
    logA = np.log(np.array(g["a"])).reshape(1, 2, 1)
    Y, F = run_form(form, X, logA, B, C)
    np.testing.assert_allclose(Y.reshape(2, 2), [g["y0"], g["y1"]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(F.reshape(2, 3), np.array(g["final"]).reshape(2, 3), rtol=0,
                               atol=1e-14)


# --------------------------------------------------------------------------- duality, chunking

@pytest.mark.parametrize("init", [False, True])
def test_duality_recurrence_equals_quadratic(init):
    """Section 5.1 / 5.3: the linear (recurrent) and quadratic (masked attention) forms agree."""
    X, logA, B, C, I = rand_problem(1, init=init)
    Yr, Fr = oracle.recurrence(X, logA, B, C, I)
    Yq, Fq = oracle.quadratic(X, logA, B, C, I)
    assert rel(Yr, Yq) < 1e-12
    assert rel(Fr, Fq) < 1e-12


def test_recurrence_numpy_twin():
    X, logA, B, C, I = rand_problem(2)
    Yr, Fr = oracle.recurrence(X, logA, B, C, I)
    Yn, Fn = oracle.recurrence_np(X, logA, B, C, I)
    assert rel(Yr, Yn) < 1e-13 and rel(Fr, Fn) < 1e-13


@pytest.mark.parametrize("Q", [1, 2, 3, 16, 64, 256])
def test_chunked_equals_recurrence_any_chunk_length(Q):
    """Section 6: the block decomposition is exact for every chunk length, ragged tail too."""
    X, logA, B, C, I = rand_problem(3, b=2, T=300, H=2, P=4, N=3, G=1)
    Yr, Fr = oracle.recurrence(X, logA, B, C, I)
    Yc, Fc = oracle.chunked(X, logA, B, C, Q, I)
    assert rel(Yc, Yr) < 1e-12
    assert rel(Fc, Fr) < 1e-12


def test_chunked_varlen_ragged():
    lens = [5, 0, 70, 1, 33]
    T = sum(lens)
    X, logA, B, C, I = rand_problem(4, b=1, T=T, H=3, P=4, N=6, G=3, nseq=len(lens))
    off = np.concatenate([[0], np.cumsum(lens)])
    Yr, Fr = oracle.recurrence(X, logA, B, C, I, off)
    for Q in (1, 16, 32):
        Yc, Fc = oracle.chunked(X, logA, B, C, Q, I, off)
        assert rel(Yc, Yr) < 1e-12 and rel(Fc, Fr) < 1e-12
    Yq, Fq = oracle.quadratic(X, logA, B, C, I, off)
    assert rel(Yq, Yr) < 1e-12 and rel(Fq, Fr) < 1e-12


# --------------------------------------------------------------------------- closed forms

@pytest.mark.parametrize("form", ALL_FORMS)
def test_closed_form_a_one_is_causal_linear_attention(form):
    """a_t = 1 (logA = 0): the mask is the causal all-ones mask, so the layer is causal linear
    attention, Y = tril(C B^T) X + C init^T (section 4.2 / proposition 4.1; section 5.2)."""
    X, logA, B, C, I = rand_problem(5, b=1, T=20, H=1, P=3, N=4, G=1)
    logA = np.zeros_like(logA)
    Y, F = run_form(form, X, logA, B, C, I)
    c, bb, x, i0 = C[0, :, 0], B[0, :, 0], X[0, :, 0], I[0, 0]
    Yexp = np.tril(c @ bb.T) @ x + c @ i0.T
    Fexp = i0 + x.T @ bb
    assert rel(Y[0, :, 0], Yexp) < 1e-13
    assert rel(F[0, 0], Fexp) < 1e-13


@pytest.mark.parametrize("form", ALL_FORMS)
def test_closed_form_a_zero_is_diagonal(form):
    """a_t = 0 (logA = -inf): the 1-SS matrix is the identity, so y_t = (C_t . B_t) x_t and the
    final state is x_{T-1} B_{T-1}^T (section 3.2.2, degenerate case)."""
    X, logA, B, C, I = rand_problem(6, b=1, T=11, H=2, P=3, N=4, G=1)
    logA = np.full_like(logA, -np.inf)
    Y, F = run_form(form, X, logA, B, C, I)
    cb = np.einsum("tn,tn->t", C[0, :, 0], B[0, :, 0])
    for h in range(2):
        np.testing.assert_allclose(Y[0, :, h], cb[:, None] * X[0, :, h], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(F[0, h], np.outer(X[0, -1, h], B[0, -1, 0]), rtol=1e-13)


@pytest.mark.parametrize("form", ALL_FORMS)
def test_closed_form_zero_input_decays_initial_state(form):
    """x = 0: y_t = exp(sum_{k<=t} logA_k) init C_t and final = exp(sum logA) init (the initial
    state is the state before token 0, decayed by a_0 onwards)."""
    X, logA, B, C, I = rand_problem(7, b=2, T=9, H=2, P=3, N=2, G=2)
    X = np.zeros_like(X)
    Y, F = run_form(form, X, logA, B, C, I)
    for b in range(2):
        for h in range(2):
            dec = np.exp(np.cumsum(logA[b, :, h]))
            Yexp = dec[:, None] * (C[b, :, h] @ I[b, h].T)
            np.testing.assert_allclose(Y[b, :, h], Yexp, rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(F[b, h], dec[-1] * I[b, h], rtol=1e-13)


def test_scalar_ssm_sum_form():
    """P = N = 1, B = C = 1: h_t = sum_u (a_{u+1} ... a_t) x_u (appendix B, cumprodsum)."""
    rng = np.random.default_rng(8)
    T = 50
    x = rng.standard_normal(T)
    a = rng.uniform(0.1, 1.0, T)
    ones = np.ones((1, T, 1, 1))
    Y, F = oracle.recurrence(x.reshape(1, T, 1, 1), np.log(a).reshape(1, T, 1), ones, ones)
    h = np.array([sum(np.prod(a[u + 1:t + 1]) * x[u] for u in range(t + 1)) for t in range(T)])
    np.testing.assert_allclose(Y.reshape(-1), h, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(F.reshape(-1), h[-1:], rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- invariants

@pytest.mark.parametrize("split", [1, 17, 36])
def test_split_resume_equals_full(split):
    """Section 8.2 (context parallel): run a prefix, hand its final state to the rest."""
    X, logA, B, C, I = rand_problem(9)
    Y, F = oracle.recurrence(X, logA, B, C, I)
    Y1, F1 = oracle.recurrence(X[:, :split], logA[:, :split], B[:, :split], C[:, :split], I)
    Y2, F2 = oracle.recurrence(X[:, split:], logA[:, split:], B[:, split:], C[:, split:], F1)
    assert rel(np.concatenate([Y1, Y2], axis=1), Y) < 1e-13
    assert rel(F2, F) < 1e-13


@pytest.mark.parametrize("form", ("recurrence", "quadratic", "chunked3"))
def test_packing_equals_separate_runs(form):
    """Section 8.3: a packed batch with sequence boundaries equals independent per-sequence runs
    (empty and length-1 sequences included; an empty sequence returns its initial state)."""
    lens = [7, 1, 0, 23, 4]
    T = sum(lens)
    X, logA, B, C, I = rand_problem(10, b=1, T=T, H=4, P=3, N=5, G=2, nseq=len(lens))
    off = np.concatenate([[0], np.cumsum(lens)])
    Y, F = run_form(form, X, logA, B, C, I, off)
    for s in range(len(lens)):
        r0, r1 = off[s], off[s + 1]
        if r1 == r0:
            np.testing.assert_allclose(F[s], I[s], rtol=0, atol=0)
            continue
        Ys, Fs = oracle.recurrence_np(X[:, r0:r1], logA[:, r0:r1], B[:, r0:r1], C[:, r0:r1],
                                      I[s:s + 1])
        assert rel(Y[:, r0:r1], Ys) < 1e-13
        assert rel(F[s:s + 1], Fs) < 1e-13


def test_linearity():
    """The SSM is linear in its input and initial state (section 2.1, recurrent view)."""
    X1, logA, B, C, I1 = rand_problem(11)
    X2, _, _, _, I2 = rand_problem(12)
    al, be = 0.7, -1.3
    Y1, F1 = oracle.recurrence(X1, logA, B, C, I1)
    Y2, F2 = oracle.recurrence(X2, logA, B, C, I2)
    Y, F = oracle.recurrence(al * X1 + be * X2, logA, B, C, al * I1 + be * I2)
    assert rel(Y, al * Y1 + be * Y2) < 1e-13
    assert rel(F, al * F1 + be * F2) < 1e-13


@pytest.mark.parametrize("form", ("recurrence", "quadratic", "chunked2"))
def test_group_mapping(form):
    """Section 7.2 grouped heads: head h reads group h // (H/G).  Each head of a G=2, H=4
    problem equals a one-head problem given that group's B and C."""
    X, logA, B, C, I = rand_problem(13, b=1, T=15, H=4, P=3, N=4, G=2)
    Y, F = run_form(form, X, logA, B, C, I)
    for h, g in [(0, 0), (1, 0), (2, 1), (3, 1)]:
        Yh, Fh = oracle.recurrence_np(X[:, :, h:h + 1], logA[:, :, h:h + 1], B[:, :, g:g + 1],
                                      C[:, :, g:g + 1], I[:, h:h + 1])
        assert rel(Y[:, :, h:h + 1], Yh) < 1e-13
        assert rel(F[:, h:h + 1], Fh) < 1e-13


def test_group_broadcast_and_head_permutation():
    """G=1 equals G=H with B, C replicated; permuting heads permutes the outputs."""
    X, logA, B, C, I = rand_problem(14, b=2, T=12, H=3, P=2, N=3, G=1)
    Y1, F1 = oracle.recurrence(X, logA, B, C, I)
    Yh, Fh = oracle.recurrence(X, logA, np.repeat(B, 3, axis=2), np.repeat(C, 3, axis=2), I)
    assert rel(Yh, Y1) < 1e-14 and rel(Fh, F1) < 1e-14
    perm = [2, 0, 1]
    Yp, Fp = oracle.recurrence(X[:, :, perm], logA[:, :, perm], B, C, I[:, perm])
    assert rel(Yp, Y1[:, :, perm]) < 1e-14 and rel(Fp, F1[:, perm]) < 1e-14


# --------------------------------------------------------------------------- input generators

def test_bf16_round_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(15)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -0.0, 0.0, 1e-30, 3e38],
                                 dtype=np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(bf16_round(v), ref)


def test_packed_lengths_procedure():
    rng = np.random.default_rng(16)
    for _ in range(20):
        lens = packed_lengths(rng, 16, 32768, 256, 4096)
        assert sum(lens) == 32768 and min(lens) >= 256 and max(lens) <= 4096 and len(lens) == 16


def test_inputs_reproducible_and_head_subset():
    a = make_inputs(2, 40, 6, 4, 8, 2, "bf16", 99, init_state=True)
    b = make_inputs(2, 40, 6, 4, 8, 2, "bf16", 99, init_state=True, heads=[1, 4])
    np.testing.assert_array_equal(a.X[:, :, [1, 4]], b.X)
    np.testing.assert_array_equal(a.logA[:, :, [1, 4]], b.logA)
    np.testing.assert_array_equal(a.init[:, [1, 4]], b.init)
    np.testing.assert_array_equal(bf16_round(a.X), a.X)
    assert np.all(a.logA < 0) and np.all(np.exp(a.logA) > 0.19)


# --------------------------------------------------------------------------- decode step

def test_decode_step_worked_p2_n3():
    """The hand-worked P=2, N=3 head, stepped one token at a time from a zero state."""
    g = {r[0]: [float(v) for v in r[1:]] for r in _golden_lines("ssd_p2_n3_worked.txt")}
    S = np.zeros((1, 1, 2, 3))
    for t in range(2):
        y, S = oracle.decode_step(S, np.array(g[f"x{t}"]).reshape(1, 1, 2),
                                  np.log(np.array([[g["a"][t]]])),
                                  np.array(g[f"B{t}"]).reshape(1, 1, 3), np.array(g[f"C{t}"]).reshape(1, 1, 3))
        np.testing.assert_allclose(y.reshape(-1), g[f"y{t}"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(S.reshape(-1), g["final"], rtol=0, atol=1e-14)


def test_decode_step_closed_forms():
    """a = 1: S' = S + x B^T; a = 0 (logA = -inf): S' = x B^T, y = (B . C) x."""
    rng = np.random.default_rng(7)
    S0 = rng.standard_normal((2, 3, 4, 5))
    x = rng.standard_normal((2, 3, 4))
    B = rng.standard_normal((2, 1, 5))
    C = rng.standard_normal((2, 1, 5))
    y, S = oracle.decode_step(S0, x, np.zeros((2, 3)), B, C)
    want = S0 + x[..., None] * B[:, :, None, :]
    np.testing.assert_allclose(S, want, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(y, np.einsum("bhpn,bn->bhp", want, C[:, 0]), rtol=1e-13, atol=1e-13)
    y, S = oracle.decode_step(S0, x, np.full((2, 3), -np.inf), B, C)
    np.testing.assert_allclose(S, x[..., None] * B[:, :, None, :], rtol=0, atol=1e-14)
    np.testing.assert_allclose(y, np.sum(B * C, axis=-1)[:, :, None] * x, rtol=1e-13, atol=1e-13)


def test_decode_steps_continue_the_forward_pass():
    """Forward over T tokens, then k decode steps == forward over T + k tokens (the
    recurrent mode resumes exactly where the forward pass's final state stops)."""
    X, logA, B, C, I = rand_problem(31, b=2, T=20, H=4, P=6, N=5, G=2)
    T0 = 14
    Y_all, F_all = oracle.recurrence(X, logA, B, C, I)
    _, S = oracle.recurrence(X[:, :T0], logA[:, :T0], B[:, :T0], C[:, :T0], I)
    for t in range(T0, 20):
        y, S = oracle.decode_step(S, X[:, t], logA[:, t], B[:, t], C[:, t])
        np.testing.assert_allclose(y, Y_all[:, t], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, F_all, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- backward
# The adjoint recurrence is pinned by central finite differences of the forward
# oracle: L = <dY, Y> + <dF, final>, every entry of every input of tiny problems.

def _fd_loss(X, logA, B, C, I, off, dY, dF):
    Y, F = oracle.recurrence(X, logA, B, C, I, off)
    return float(np.sum(dY * Y) + (0.0 if dF is None else np.sum(dF * F)))


def _fd_grad(arr, f, eps=1e-6):
    g = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        v = arr[i]
        arr[i] = v + eps
        lp = f()
        arr[i] = v - eps
        lm = f()
        arr[i] = v
        g[i] = (lp - lm) / (2 * eps)
    return g


@pytest.mark.parametrize("case", ["batch_init_dfinal", "packed_groups_empty", "no_init_no_dfinal"])
def test_backward_matches_finite_differences(case):
    rng = np.random.default_rng(77)
    off = None
    if case == "batch_init_dfinal":
        X, logA, B, C, I = rand_problem(70, b=2, T=5, H=2, P=3, N=2, G=1)
        use_df = True
    elif case == "packed_groups_empty":
        lens = [3, 0, 4, 1]
        off = np.cumsum([0] + lens)
        X, logA, B, C, I = rand_problem(71, b=1, T=8, H=4, P=2, N=3, G=2, nseq=4)
        use_df = True
    else:
        X, logA, B, C, I = rand_problem(72, b=1, T=6, H=2, P=2, N=2, G=2, init=False)
        use_df = False
    nseq = X.shape[0] if off is None else len(off) - 1
    dY = rng.standard_normal(X.shape)
    dF = rng.standard_normal((nseq,) + X.shape[2:] + (B.shape[3],)) if use_df else None
    dX, dlogA, dB, dC, dI = oracle.backward(X, logA, B, C, I, off, dY, dF)
    f = lambda: _fd_loss(X, logA, B, C, I, off, dY, dF)
    for name, arr, got in [("X", X, dX), ("logA", logA, dlogA), ("B", B, dB), ("C", C, dC)] + \
            ([("init", I, dI)] if I is not None else []):
        want = _fd_grad(arr, f)
        np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-8, err_msg=name)
    if I is None:
        assert dI is None


def test_backward_empty_sequence_passes_dfinal_to_dinit():
    X, logA, B, C, I = rand_problem(73, b=1, T=4, H=2, P=2, N=2, G=1, nseq=3)
    off = np.array([0, 4, 4, 4])
    rng = np.random.default_rng(5)
    dY = rng.standard_normal(X.shape)
    dF = rng.standard_normal(I.shape)
    _, _, _, _, dI = oracle.backward(X, logA, B, C, I, off, dY, dF)
    np.testing.assert_array_equal(dI[1:], dF[1:])


def test_backward_long_sequence_crosses_checkpoints():
    """A sequence of 150 tokens (three stretches between stored states), a few
    directional finite differences."""
    X, logA, B, C, I = rand_problem(74, b=1, T=150, H=2, P=3, N=4, G=1)
    rng = np.random.default_rng(6)
    dY = rng.standard_normal(X.shape)
    dF = rng.standard_normal(I.shape)
    grads = oracle.backward(X, logA, B, C, I, None, dY, dF)
    for k, arr in enumerate([X, logA, B, C, I]):
        v = rng.standard_normal(arr.shape)
        eps = 1e-6
        orig = arr.copy()
        arr += eps * v
        lp = _fd_loss(X, logA, B, C, I, None, dY, dF)
        arr[...] = orig - eps * v
        lm = _fd_loss(X, logA, B, C, I, None, dY, dF)
        arr[...] = orig
        want = (lp - lm) / (2 * eps)
        got = float(np.sum(grads[k] * v))
        assert abs(got - want) <= 1e-6 * max(1.0, abs(want)), (k, got, want)
