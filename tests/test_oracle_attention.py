"""Pins for the oracle's forward and backward (CPU only).

Each test compares the oracle with something other than itself:
  * PyTorch's CPU scaled_dot_product_attention in fp64 (forward and autograd backward),
    with the causal flag, with no mask, and with the hand-drawn golden masks as explicit
    boolean masks;
  * closed forms: constant V gives O = V; a single visible key copies that V row (and
    then dQ = dK = 0, dV = sum of dO over the head group); Q = 0 gives O = mean of the
    visible V rows and LSE = ln(number of visible keys);
  * invariants: a document mask equals independent attention per document; GQA equals
    MHA with K/V repeated and dK/dV summed over the group; sum_j dK_j = 0 and
    sum_j dV_j = sum of dO over the group's rows;
  * central finite differences of L = sum(O * dO) in fp64.
"""
import numpy as np
import pytest
import torch

from masked_long_context_tiled_amd.inputs import MaskSpec, block_sparse_keep, document_cu_seqlens
from oracle.attention import attention_backward, attention_forward

from conftest import load_golden_masks

rng0 = np.random.default_rng(1234)


def _rand(*shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


def _small_specs(T):
    """One parameterisation of every mask kind at sequence length T (T multiple of 12)."""
    return [
        (MaskSpec("full"), None),
        (MaskSpec("causal"), None),
        (MaskSpec("full_document", cu_seqlens=(0, T // 3, T // 2, T)), None),
        (MaskSpec("causal_document", cu_seqlens=(0, T // 4, T)), None),
        (MaskSpec("full_sliding_window", window=T // 6), None),
        (MaskSpec("causal_sliding_window", window=T // 4), None),
        (MaskSpec("shared_question", question_len=T // 4, answer_len=T // 4, n_answers=3), None),
        (MaskSpec("prefix_lm_causal", prefix_len=T // 3), None),
        (MaskSpec("causal_blockwise", block_len=T // 6, final_block_len=T // 3), None),
        (MaskSpec("global_sliding", global_len=T // 12, window=T // 6), None),
        (MaskSpec("block_sparse", sparse_block=T // 6), block_sparse_keep(7, 4, 6, 6)),
    ]


def _torch_sdpa(q, k, v, do, allowed=None, is_causal=False):
    """Reference by PyTorch (CPU, fp64). allowed: bool [Hq][T][T] or [T][T] or None."""
    T, Hq, d = q.shape
    G = Hq // k.shape[1]
    Q = torch.tensor(q.transpose(1, 0, 2), requires_grad=True)
    K = torch.tensor(k.transpose(1, 0, 2), requires_grad=True)
    V = torch.tensor(v.transpose(1, 0, 2), requires_grad=True)
    Kr = K.repeat_interleave(G, dim=0)
    Vr = V.repeat_interleave(G, dim=0)
    mask = None if allowed is None else torch.tensor(allowed)
    O = torch.nn.functional.scaled_dot_product_attention(
        Q[None], Kr[None], Vr[None], attn_mask=mask, is_causal=is_causal)[0]
    O.backward(torch.tensor(do.transpose(1, 0, 2)))
    return (O.detach().numpy().transpose(1, 0, 2), Q.grad.numpy().transpose(1, 0, 2),
            K.grad.numpy().transpose(1, 0, 2), V.grad.numpy().transpose(1, 0, 2))


def _check_vs_torch(spec, keep, allowed, is_causal, T, Hq, Hk, d, seed):
    q, k, v, do = (_rand(T, Hq, d, seed=seed), _rand(T, Hk, d, seed=seed + 1),
                   _rand(T, Hk, d, seed=seed + 2), _rand(T, Hq, d, seed=seed + 3))
    r = attention_backward(q, k, v, do, spec, keep=keep)
    O, dQ, dK, dV = _torch_sdpa(q, k, v, do, allowed, is_causal)
    for name, a, b in (("o", r["o"], O), ("dq", r["dq"], dQ), ("dk", r["dk"], dK), ("dv", r["dv"], dV)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11, err_msg=name)
    return q, k, r


def test_vs_torch_full_and_causal_flag():
    _check_vs_torch(MaskSpec("full"), None, None, False, 64, 4, 2, 16, 1)
    _check_vs_torch(MaskSpec("causal"), None, None, True, 64, 4, 2, 16, 5)
    _check_vs_torch(MaskSpec("causal"), None, None, True, 50, 2, 2, 8, 9)   # MHA, ragged T


@pytest.mark.parametrize("case", load_golden_masks(), ids=lambda c: c[0].kind)
def test_vs_torch_golden_masks(case):
    spec, keep, drawn = case
    allowed = drawn.astype(bool)
    if keep is not None:
        keep = np.repeat(keep, 2, axis=0)              # the drawn keep set, for both heads
    _check_vs_torch(spec, keep, allowed, False, 12, 2, 1, 8, 3)


def test_lse_vs_torch_logsumexp():
    T, Hq, Hk, d = 48, 4, 2, 16
    q, k, v = _rand(T, Hq, d, seed=11), _rand(T, Hk, d, seed=12), _rand(T, Hk, d, seed=13)
    spec = MaskSpec("global_sliding", global_len=4, window=7)
    _, lse = attention_forward(q, k, v, spec)
    ii, jj = np.meshgrid(np.arange(T), np.arange(T), indexing="ij")
    allowed = torch.tensor((ii < 4) | (jj < 4) | (np.abs(ii - jj) < 7))
    for h in range(Hq):
        S = torch.tensor(q[:, h]) @ torch.tensor(k[:, h // 2]).T / np.sqrt(d)
        want = torch.logsumexp(S.masked_fill(~allowed, -float("inf")), dim=1).numpy()
        np.testing.assert_allclose(lse[h], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("idx", range(11))
def test_constant_v_gives_v(idx):
    T, Hq, Hk, d = 48, 4, 2, 8
    spec, keep = _small_specs(T)[idx]
    q, k = _rand(T, Hq, d, seed=idx), _rand(T, Hk, d, seed=idx + 50)
    row = _rand(Hk, d, seed=99)
    v = np.broadcast_to(row, (T, Hk, d)).copy()
    O, lse = attention_forward(q, k, v, spec, keep=keep)
    for h in range(Hq):
        np.testing.assert_allclose(O[:, h, :], np.broadcast_to(row[h // 2], (T, d)), rtol=1e-12, atol=1e-12)
    assert np.isfinite(lse).all()


def test_single_visible_key_copies_v_row():
    T, Hq, Hk, d = 40, 4, 2, 8
    q, k, v, do = _rand(T, Hq, d, seed=1), _rand(T, Hk, d, seed=2), _rand(T, Hk, d, seed=3), _rand(T, Hq, d, seed=4)
    # CAUSAL row 0 sees only key 0
    O, _ = attention_forward(q, k, v, MaskSpec("causal"))
    for h in range(Hq):
        np.testing.assert_allclose(O[0, h], v[0, h // 2], rtol=1e-13, atol=1e-13)
    # CAUSAL SLIDING WINDOW w = 1: every row sees only itself
    r = attention_backward(q, k, v, do, MaskSpec("causal_sliding_window", window=1))
    for h in range(Hq):
        np.testing.assert_allclose(r["o"][:, h], v[:, h // 2], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(r["lse"][h], np.einsum("td,td->t", q[:, h], k[:, h // 2]) / np.sqrt(d),
                                   rtol=1e-12, atol=1e-12)
    assert np.abs(r["dq"]).max() < 1e-12 and np.abs(r["dk"]).max() < 1e-12
    for g in range(Hk):
        np.testing.assert_allclose(r["dv"][:, g], do[:, 2 * g] + do[:, 2 * g + 1], rtol=1e-13, atol=1e-13)


def test_zero_q_mean_and_log_count():
    T, Hq, Hk, d = 60, 2, 1, 8
    v = _rand(T, Hk, d, seed=8)
    k = _rand(T, Hk, d, seed=9)
    q = np.zeros((T, Hq, d))
    # CAUSAL: O_i = mean(V_0..V_i), LSE_i = ln(i + 1)
    O, lse = attention_forward(q, k, v, MaskSpec("causal"))
    cm = np.cumsum(v[:, 0], axis=0) / np.arange(1, T + 1)[:, None]
    for h in range(Hq):
        np.testing.assert_allclose(O[:, h], cm, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[h], np.log(np.arange(1, T + 1)), rtol=1e-13, atol=1e-13)
    # FULL SLIDING WINDOW w: LSE_i = ln(min(T, i + w) - max(0, i - w + 1))
    w = 7
    O, lse = attention_forward(q, k, v, MaskSpec("full_sliding_window", window=w))
    i = np.arange(T)
    lo, hi = np.maximum(0, i - w + 1), np.minimum(T, i + w)
    np.testing.assert_allclose(lse[0], np.log(hi - lo), rtol=1e-13, atol=1e-13)
    cs = np.vstack([np.zeros((1, d)), np.cumsum(v[:, 0], axis=0)])
    np.testing.assert_allclose(O[:, 0], (cs[hi] - cs[lo]) / (hi - lo)[:, None], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_document_equals_per_document_attention(causal):
    T, Hq, Hk, d = 96, 4, 2, 8
    cu = document_cu_seqlens(5, T, 10, 40)
    q, k, v, do = _rand(T, Hq, d, seed=21), _rand(T, Hk, d, seed=22), _rand(T, Hk, d, seed=23), _rand(T, Hq, d, seed=24)
    spec = MaskSpec("causal_document" if causal else "full_document", cu_seqlens=cu)
    r = attention_backward(q, k, v, do, spec)
    base = MaskSpec("causal" if causal else "full")
    for a, b in zip(cu[:-1], cu[1:]):
        s = slice(a, b)
        rd = attention_backward(q[s], k[s], v[s], do[s], base)
        for key in ("o", "dq", "dk", "dv"):
            np.testing.assert_allclose(r[key][s], rd[key], rtol=1e-12, atol=1e-12, err_msg=key)
        np.testing.assert_allclose(r["lse"][:, s], rd["lse"], rtol=1e-12, atol=1e-12)


def test_gqa_equals_repeated_mha():
    T, Hq, Hk, d = 36, 6, 2, 8
    spec = MaskSpec("prefix_lm_causal", prefix_len=9)
    q, k, v, do = _rand(T, Hq, d, seed=31), _rand(T, Hk, d, seed=32), _rand(T, Hk, d, seed=33), _rand(T, Hq, d, seed=34)
    r = attention_backward(q, k, v, do, spec)
    kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
    m = attention_backward(q, kr, vr, do, spec)
    for key in ("o", "lse", "dq"):
        np.testing.assert_allclose(r[key], m[key], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dk"], m["dk"].reshape(T, Hk, 3, d).sum(2), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dv"], m["dv"].reshape(T, Hk, 3, d).sum(2), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("idx", range(11))
def test_gradient_sum_identities(idx):
    T, Hq, Hk, d = 48, 4, 2, 8
    spec, keep = _small_specs(T)[idx]
    q, k, v, do = _rand(T, Hq, d, seed=41), _rand(T, Hk, d, seed=42), _rand(T, Hk, d, seed=43), _rand(T, Hq, d, seed=44)
    r = attention_backward(q, k, v, do, spec, keep=keep)
    # rows of dS sum to zero -> sum_j dK_j = 0 per KV head
    np.testing.assert_allclose(r["dk"].sum(0), 0.0, atol=1e-11)
    # P is row-stochastic on rows that see a key -> sum_j dV_j = sum of dO over the group's rows
    has = np.isfinite(r["lse"])                          # [Hq][T]
    for g in range(Hk):
        want = sum((do[:, h] * has[h][:, None]).sum(0) for h in (2 * g, 2 * g + 1))
        np.testing.assert_allclose(r["dv"][:, g].sum(0), want, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("spec_keep", [
    (MaskSpec("causal"), None),
    (MaskSpec("global_sliding", global_len=2, window=5), None),
    (MaskSpec("causal_blockwise", block_len=4, final_block_len=8), None),
    (MaskSpec("block_sparse", sparse_block=6), block_sparse_keep(3, 2, 4, 4)),
], ids=["causal", "global_sliding", "causal_blockwise", "block_sparse"])
def test_finite_differences(spec_keep):
    spec, keep = spec_keep
    T, Hq, Hk, d = 24, 2, 1, 6
    q, k, v, do = _rand(T, Hq, d, seed=51), _rand(T, Hk, d, seed=52), _rand(T, Hk, d, seed=53), _rand(T, Hq, d, seed=54)
    r = attention_backward(q, k, v, do, spec, keep=keep)

    def loss(q_, k_, v_):
        O, _ = attention_forward(q_, k_, v_, spec, keep=keep)
        return float(np.sum(O * do))

    eps = 1e-6
    for name, x, g in (("q", q, r["dq"]), ("k", k, r["dk"]), ("v", v, r["dv"])):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
            ap = [xp if n == name else a for n, a in zip("qkv", args)]
            am = [xm if n == name else a for n, a in zip("qkv", args)]
            num[idx] = (loss(*ap) - loss(*am)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-7, err_msg=name)


def test_fully_masked_row_convention():
    T, Hq, Hk, d, b = 24, 2, 1, 8, 6
    keep = np.ones((Hq, 4, 4), dtype=np.uint8)
    keep[1, 2, :] = 0                                   # head 1, query block 2 sees nothing
    spec = MaskSpec("block_sparse", sparse_block=b)
    q, k, v, do = _rand(T, Hq, d, seed=61), _rand(T, Hk, d, seed=62), _rand(T, Hk, d, seed=63), _rand(T, Hq, d, seed=64)
    r = attention_backward(q, k, v, do, spec, keep=keep)
    rows = slice(2 * b, 3 * b)
    assert np.all(r["o"][rows, 1] == 0) and np.all(r["dq"][rows, 1] == 0)
    assert np.all(np.isneginf(r["lse"][1, rows]))
    for key in ("o", "dq", "dk", "dv"):
        assert np.isfinite(r[key]).all()
    # head 0 is unaffected: equal to FULL attention
    f = attention_backward(q[:, :1], k, v, do[:, :1], MaskSpec("full"))
    np.testing.assert_allclose(r["o"][:, 0], f["o"][:, 0], rtol=1e-12, atol=1e-12)


def test_row_subset_equals_full_rows():
    T, Hq, Hk, d = 64, 4, 1, 8
    spec = MaskSpec("shared_question", question_len=16, answer_len=16, n_answers=3)
    q, k, v, do = _rand(T, Hq, d, seed=71), _rand(T, Hk, d, seed=72), _rand(T, Hk, d, seed=73), _rand(T, Hq, d, seed=74)
    full = attention_backward(q, k, v, do, spec)
    rows = np.array([0, 5, 17, 33, 63])
    part = attention_backward(q, k, v, do, spec, rows=rows, heads=[1, 3], chunk=2)
    np.testing.assert_allclose(part["o"], full["o"][rows][:, [1, 3]], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(part["dq"], full["dq"][rows][:, [1, 3]], rtol=1e-13, atol=1e-13)
    # dK restricted to key columns, accumulated over all rows and heads, equals the full one
    cols = np.array([3, 20, 40])
    kc = attention_backward(q, k, v, do, spec, key_cols=cols, chunk=7)
    np.testing.assert_allclose(kc["dk"], full["dk"][cols], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(kc["dv"], full["dv"][cols], rtol=1e-12, atol=1e-12)
