"""GPU parity: the HIP library against the CPU oracle on seeded inputs.

Top-k indices and accept decisions are compared bit for bit; indexer scores
bit for bit on integer/dyadic inputs (exact in fp32 under any summation
order); attention within max abs error 1e-2 (bf16 inputs, fp32 accumulate).
"""

import math
import sys

import numpy as np
import pytest
import torch

import dsa_inputs as I
from oracle import dsa_oracle as O

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import dsa_sparse_attention_lightning_amd as dsa
    from gpu_util import DEV, DraftDev, to_dev, bits_to_dev

ATTN_TOL = 1e-2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ----------------------------------------------------------------------------
# a1 indexer
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("case", [
    dict(lens=[512], H_I=4, D_I=32, page=64, shuffle=False, R=1),          # tiny shape
    dict(lens=[3001, 1500], H_I=64, D_I=128, page=64, shuffle=True, R=1),  # ragged, paged
    dict(lens=[777], H_I=20, D_I=64, page=16, shuffle=True, R=3),          # odd heads, 3 rows
    dict(lens=[2048], H_I=64, D_I=128, page=64, shuffle=False, R=8),       # verify-pass rows
    dict(lens=[4133, 900], H_I=64, D_I=64, page=16, shuffle=True, R=5),    # 5 rows, ragged, 2 sequences
    dict(lens=[1300], H_I=48, D_I=32, page=64, shuffle=True, R=7),         # 7 rows, partial head block
    dict(lens=[9000], H_I=64, D_I=128, page=64, shuffle=True, R=6),        # 6 rows, several tiles per workgroup
    # long contexts take the Q-in-LDS kernel (5-8 rows, D_I = 128, ld * B >= 2^18)
    dict(lens=[270011], H_I=64, D_I=128, page=64, shuffle=True, R=8),      # 8 rows, ragged tail
    dict(lens=[140000, 131075], H_I=64, D_I=128, page=16, shuffle=True, R=5),   # 2 sequences, 5 rows
    dict(lens=[300000], H_I=48, D_I=128, page=64, shuffle=True, R=7),      # partial head block
])
def test_index_scores_exact(case):
    log("index_scores", case)
    d = I.draft_inputs(7, case["lens"], H_I=case["H_I"], D_I=case["D_I"], H_q=4, H_kv=4, D_qk=64,
                       D_v=64, k=64, R=case["R"], page=case["page"], shuffle_pages=case["shuffle"],
                       integer_indexer=True)
    row_len = d.row_len.copy()
    if case["R"] > 1:   # rows see different prefixes
        for r in range(case["R"]):
            row_len[:, r] = np.maximum(d.lens - 37 * r, 0)
    dd = DraftDev(d)
    rl = to_dev(row_len)
    ld = dd.ld + 5
    out = torch.full((d.B, d.R, ld), -7.0, device=DEV)
    dsa.index_scores(dd.q_index, dd.w, dd.kidx, dd.bt, rl, page=d.page, out=out)
    got = out.cpu().numpy()
    for b in range(d.B):
        ref = O.index_scores(d.q_index[b], d.w[b].astype(np.float64), d.keys[b], row_len[b])
        for r in range(d.R):
            n = row_len[b, r]
            np.testing.assert_array_equal(got[b, r, :n], ref[r, :n].astype(np.float32))
            assert np.all(got[b, r, n:] == -7.0)   # untouched beyond row_len


@pytest.mark.parametrize("seed", range(10))
def test_index_scores_random_shapes(seed):
    """Seeded random indexer shapes on exact integer inputs: 1-4 sequences,
    1-8 rows with different visible prefixes, 1-64 heads, D_I 32/64/128, pages
    of 16 or 64 (shuffled), contexts up to 300,000; every score bit-exact."""
    rng = np.random.default_rng(6000 + seed)
    B = int(rng.integers(1, 5))
    R = int(rng.integers(1, 9))
    H = int(rng.integers(1, 65))
    D = int(rng.choice([32, 64, 128]))
    page = int(rng.choice([16, 64]))
    hi = 300000 if B == 1 else 60000
    lens = [int(x) for x in rng.integers(1, hi, size=B)]
    log("index_scores random", seed, B, R, H, D, page, lens)
    d = I.draft_inputs(7000 + seed, lens, H_I=H, D_I=D, H_q=4, H_kv=4, D_qk=64, D_v=64, k=64, R=R, page=page,
                       shuffle_pages=True, integer_indexer=True)
    row_len = d.row_len.copy()
    for r in range(R):
        row_len[:, r] = np.maximum(d.lens - int(rng.integers(0, 100)) * r, 0)
    dd = DraftDev(d)
    out = torch.full((d.B, d.R, dd.ld), -7.0, device=DEV)
    dsa.index_scores(dd.q_index, dd.w, dd.kidx, dd.bt, to_dev(row_len), page=d.page, out=out)
    got = out.cpu().numpy()
    for b in range(d.B):
        ref = O.index_scores(d.q_index[b], d.w[b].astype(np.float64), d.keys[b], row_len[b])
        for r in range(d.R):
            n = row_len[b, r]
            np.testing.assert_array_equal(got[b, r, :n], ref[r, :n].astype(np.float32))
            assert np.all(got[b, r, n:] == -7.0)


def test_index_scores_chunks_past_every_row():
    """Score rows far longer than every row length (most workgroups see no
    position of any row) and a sequence whose rows are all empty: the
    visible prefixes are bit-exact and nothing past row_len is written, on
    the one-row, 2-4-row and 5-8-row kernels."""
    for R in (1, 3, 8):
        d = I.draft_inputs(71, [3000, 2500], H_I=64, D_I=128, H_q=4, H_kv=4, D_qk=64, D_v=64, k=64, R=R,
                           page=64, shuffle_pages=True, integer_indexer=True)
        row_len = d.row_len.copy()
        for r in range(R):
            row_len[0, r] = 3000 - 37 * r
        row_len[1, :] = 0
        log("index_scores past every row", R, row_len.tolist())
        dd = DraftDev(d)
        ld = 60000
        out = torch.full((d.B, d.R, ld), -7.0, device=DEV)
        dsa.index_scores(dd.q_index, dd.w, dd.kidx, dd.bt, to_dev(row_len), page=d.page, out=out)
        got = out.cpu().numpy()
        for b in range(d.B):
            ref = O.index_scores(d.q_index[b], d.w[b].astype(np.float64), d.keys[b], row_len[b])
            for r in range(d.R):
                n = row_len[b, r]
                np.testing.assert_array_equal(got[b, r, :n], ref[r, :n].astype(np.float32))
                assert np.all(got[b, r, n:] == -7.0)


def test_index_scores_overflow_with_padding_heads():
    """A key row whose dot products overflow fp32 (its scores are +inf in the
    oracle's float64-then-float32 result) with H_I = 20, so every kernel pads
    heads inside its head blocks: the padding heads must add exactly 0, never
    0 * inf = NaN; on the one-row, 2-4-row and 5-8-row kernels."""
    for R in (1, 3, 8):
        d = I.draft_inputs(73, [600], H_I=20, D_I=128, H_q=4, H_kv=4, D_qk=64, D_v=64, k=64, R=R, page=64,
                           shuffle_pages=True, integer_indexer=True)
        log("index_scores overflow", R)
        d.q_index_bits[...] = 0x3F80                   # every query component 1.0
        d.q_index[...] = 1.0
        d.w[...] = np.maximum(d.w, np.float32(1 / 64))   # positive weights
        t = 100
        d.keys[0][t, :] = 2.0 ** 126                    # 128 * 2^126 = 2^133 overflows fp32
        d.kidx_bits[d.block_table[0, t // d.page], t % d.page, :] = 0x7E80
        dd = DraftDev(d)
        out = torch.full((d.B, d.R, dd.ld), -7.0, device=DEV)
        dsa.index_scores(dd.q_index, dd.w, dd.kidx, dd.bt, dd.row_len, page=d.page, out=out)
        got = out.cpu().numpy()
        with np.errstate(over="ignore"):
            ref = O.index_scores(d.q_index[0], d.w[0].astype(np.float64), d.keys[0], d.row_len[0]).astype(np.float32)
        for r in range(d.R):
            n = d.row_len[0, r]
            assert np.isposinf(got[0, r, t]) and np.isposinf(ref[r, t])
            np.testing.assert_array_equal(got[0, r, :n], ref[r, :n])


def test_index_scores_bf16_normal_bound():
    """Continuous N(0,1) bf16 inputs: error within the fp32 accumulation bound."""
    d = I.draft_inputs(8, [4000], H_I=64, D_I=128, H_q=4, H_kv=4, D_qk=64, D_v=64, k=64)
    dd = DraftDev(d)
    got = dsa.index_scores(dd.q_index, dd.w, dd.kidx, dd.bt, dd.row_len, page=d.page).cpu().numpy()
    ref = O.index_scores(d.q_index[0], d.w[0].astype(np.float64), d.keys[0], d.row_len[0])[0]
    bound = 2.0**-16 * (d.w[0, 0].astype(np.float64) @ np.abs(d.q_index[0, 0]) @ np.abs(d.keys[0][:4000]).T)
    err = np.abs(got[0, 0, :4000] - ref[:4000])
    assert np.all(err <= bound + 1e-30), err.max()


# ----------------------------------------------------------------------------
# a2 top-k
# ----------------------------------------------------------------------------
def _topk_case(scores, lens, k):
    B = len(lens)
    ld = scores.shape[1]
    s = to_dev(scores.astype(np.float32).reshape(B, 1, ld))
    rl = to_dev(np.asarray(lens, np.int32).reshape(B, 1))
    got = dsa.topk(s, rl, k).cpu().numpy()[:, 0]
    for b in range(B):
        ref = O.topk(scores[b].astype(np.float32).astype(np.float64), lens[b], k)
        np.testing.assert_array_equal(got[b], ref, err_msg=f"row {b} L={lens[b]} k={k}")


# Row lengths exercising the three top-k paths: keys resident in LDS (ld up to
# 35,840), one workgroup re-reading scores (up to 131,072), multi-workgroup
# histogram pipeline (beyond).
TOPK_LENS = {
    "lds": [20000, 9000, 4097, 2048, 2049, 1, 0, 35000],
    "one": [130000, 36000, 4097, 2049, 0],
    "multi": [300000, 140000, 2049, 5],
}


@pytest.mark.parametrize("path", ["lds", "one", "multi"])
@pytest.mark.parametrize("name", ["normal", "ties", "allequal", "zeros_signed", "negative", "wide_range"])
def test_topk_exact(name, path):
    rng = np.random.default_rng(abs(hash((name, path))) % 2**32)
    k = 2048
    lens = TOPK_LENS[path]
    ld = max(lens) + 3
    shape = (len(lens), ld)
    s = rng.standard_normal(shape).astype(np.float32)
    if name == "ties":
        s = rng.integers(-20, 20, shape).astype(np.float32)
    elif name == "allequal":
        s[:] = 1.5
    elif name == "zeros_signed":
        s = np.where(rng.random(shape) < 0.5, np.float32(0.0), np.float32(-0.0))
        s[:, ::7] = 1.0
    elif name == "negative":
        s = -np.abs(s) - 1.0
    elif name == "wide_range":
        s = (rng.standard_normal(shape) * 10.0 ** rng.integers(-30, 30, shape)).astype(np.float32)
    log("topk", name, path, lens, k)
    _topk_case(s, lens, k)


@pytest.mark.parametrize("pattern", ["ascending", "descending", "blocks", "spikes"])
def test_topk_clustered(pattern):
    """Kept positions packed into whole 64-position runs (one thread of the
    one-workgroup path emits up to 64 of them) or isolated among equal keys."""
    rng = np.random.default_rng(abs(hash(pattern)) % 2**32)
    k, ld = 2048, 32768
    lens = [32768, 32000, 4096 + 37, 20000]
    t = np.arange(ld, dtype=np.float64)
    if pattern == "ascending":          # the top k are the last k positions
        s = np.tile(t, (len(lens), 1))
    elif pattern == "descending":       # the first k positions
        s = np.tile(-t, (len(lens), 1))
    elif pattern == "blocks":           # runs of 64 (and one of 63) high scores, rest low
        s = rng.standard_normal((len(lens), ld)) - 100.0
        for b in range(len(lens)):
            starts = rng.choice(max(1, lens[b] // 64 - 1), size=40, replace=False) * 64
            for i, st in enumerate(starts):
                s[b, st + (i == 0):st + 64] = 50.0 + rng.standard_normal(64 - (i == 0))
    else:                               # a few spikes above a sea of equal keys
        s = np.full((len(lens), ld), 3.0)
        for b in range(len(lens)):
            s[b, rng.choice(lens[b], size=100, replace=False)] = 7.0
    log("topk clustered", pattern, lens, k)
    _topk_case(s.astype(np.float32), lens, k)


@pytest.mark.parametrize("ld", [1000, 30000, 100000, 200000])
def test_topk_small_k_and_k_ge_L(ld):
    rng = np.random.default_rng(ld)
    s = rng.standard_normal((3, ld)).astype(np.float32)
    _topk_case(s, [min(ld, 5), min(ld, 64), min(ld, 100)], 64)     # k >= L rows
    _topk_case(s, [ld, ld - 1, ld // 2], 1)                          # k = 1


def test_topk_workspace_needs_no_initialisation():
    """One workspace, filled with 0xff bytes, serves calls of different
    shapes in turn (more rows, then a longer row, then fewer rows): every
    call clears or writes what it reads, so stale histograms, counts and
    lists of the previous call never reach the result."""
    import torch
    rng = np.random.default_rng(7)
    shapes = [(3, 50000, [50000, 40000, 36001]), (1, 300000, [300000]), (5, 40000, [40000, 39999, 5, 38000, 37000])]
    need = max(dsa.topk_workspace_size(B, 1, ld, 2048) for B, ld, _ in shapes)
    ws = torch.full((need,), 0xff, dtype=torch.uint8, device="cuda:0")
    for B, ld, lens in shapes * 2:
        s = (rng.standard_normal((B, ld)) * 35 + 144).astype(np.float32)
        log("topk reused workspace", B, ld, lens)
        got = dsa.topk(to_dev(s.reshape(B, 1, ld)), to_dev(np.asarray(lens, np.int32).reshape(B, 1)), 2048,
                       workspace=ws).cpu().numpy()[:, 0]
        for b in range(B):
            np.testing.assert_array_equal(got[b], O.topk(s[b].astype(np.float64), lens[b], 2048))


@pytest.mark.parametrize("seed", range(12))
def test_topk_random_shapes(seed):
    """Seeded random shapes over both top-k paths: 1-6 rows, ld from 1,000 to
    300,000, ragged row lengths (some <= k), k from 1 to 8192, and one of five
    score distributions (normal, small-integer ties, indexer-like, uniform,
    a few clustered spikes)."""
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 7))
    ld = int(rng.integers(1000, 300001))
    k = int(rng.choice([1, 7, 64, 257, 2048, 3000, 8192]))
    lens = [int(x) for x in rng.integers(0, ld + 1, size=B)]
    lens[0] = ld
    kind = seed % 5
    if kind == 0:
        s = rng.standard_normal((B, ld))
    elif kind == 1:
        s = rng.integers(-50, 50, (B, ld)).astype(np.float64)
    elif kind == 2:
        s = rng.standard_normal((B, ld)) * 35 + 144
    elif kind == 3:
        s = rng.random((B, ld))
    else:
        s = np.full((B, ld), 1.0)
        for b in range(B):
            s[b, rng.choice(ld, size=min(ld, 3 * k), replace=False)] = rng.integers(2, 6, size=min(ld, 3 * k))
    log("topk random", seed, B, ld, k, kind, lens)
    _topk_case(s.astype(np.float32), lens, k)


def test_topk_rows_longer_than_4096_chunks():
    """A row over 4096 x 4096 positions doubles the chunk size, so every pass
    workgroup loops over several 4096-position blocks (positions, counts and
    list offsets carried across them)."""
    rng = np.random.default_rng(11)
    ld = (1 << 24) + 5000
    s = (rng.standard_normal((1, ld)) * 35 + 144).astype(np.float32)
    for L, k in ((ld, 2048), (ld - 3, 8192), ((1 << 24) + 1, 1)):
        log("topk long row", ld, L, k)
        _topk_case(s, [L], k)


@pytest.mark.parametrize("k", [1, 7, 64, 1500, 2048, 3000, 8192])
@pytest.mark.parametrize("ld", [30000, 50000, 180000])
def test_topk_various_k(k, ld):
    rng = np.random.default_rng(k)
    lens = [ld, 8191, 300]
    s = rng.integers(0, 1000, (3, ld)).astype(np.float32)
    _topk_case(s, lens, k)


# ----------------------------------------------------------------------------
# a3 sparse attention
# ----------------------------------------------------------------------------
def _attn_vs_oracle(d, dd, idx_np, step=0, tol=ATTN_TOL, out_check=True):
    idx = to_dev(idx_np.astype(np.int32))
    out, lse = dsa.sparse_attn(dd.q[step][:, None], dd.k, dd.v, dd.bt, idx, page=d.page,
                               D_v=d.D_v, sm_scale=d.sm_scale)
    out = out.cpu().numpy()[:, 0]
    lse = lse.cpu().numpy()[:, 0]
    err = 0.0
    for b in range(d.B):
        o_ref, lse_ref = O.sparse_attn(d.q[step, b], d.K[b], d.V[b], idx_np[b], d.sm_scale)
        err = max(err, np.abs(out[b] - o_ref).max())
        fin = np.isfinite(lse_ref)
        np.testing.assert_array_equal(np.isfinite(lse[b]), fin)
        if fin.any():
            assert np.abs(lse[b][fin] - lse_ref[fin]).max() < tol
    assert err <= tol, err
    return out, lse, err


@pytest.mark.parametrize("case", [
    dict(lens=[512], H=4, Hkv=4, D=64, k=64, shuffle=False),
    dict(lens=[5000, 3001], H=64, Hkv=64, D=128, k=2048, shuffle=True),
    dict(lens=[900], H=8, Hkv=2, D=128, k=300, shuffle=True),
    dict(lens=[1200, 640], H=16, Hkv=4, D=64, k=1000, shuffle=True),
    dict(lens=[100], H=6, Hkv=3, D=64, k=64, shuffle=False),
    dict(lens=[40000], H=4, Hkv=4, D=128, k=20000, shuffle=True),      # 79 splits (128-way combine)
    dict(lens=[9000], H=32, Hkv=8, D=128, k=6000, shuffle=True),       # GQA 4, 24 splits
    dict(lens=[140000], H=4, Hkv=4, D=64, k=131072, shuffle=True),     # largest k: 1024 tokens per split
])
def test_sparse_attn_matches_oracle(case):
    log("sparse_attn", case)
    d = I.draft_inputs(11, case["lens"], H_I=4, D_I=32, H_q=case["H"], H_kv=case["Hkv"], D_qk=case["D"],
                       D_v=case["D"], k=case["k"], page=64, shuffle_pages=case["shuffle"], G=2)
    dd = DraftDev(d)
    rng = np.random.default_rng(5)
    idx = np.full((d.B, d.k), -1, np.int64)
    for b in range(d.B):
        n = min(d.k, int(d.lens[b]))
        idx[b, :n] = np.sort(rng.choice(int(d.lens[b]), n, replace=False))
    _attn_vs_oracle(d, dd, idx)
    # set semantics: shuffled order and scattered -1 entries give the same result
    idx2 = idx.copy()
    for b in range(d.B):
        rng.shuffle(idx2[b])
    _attn_vs_oracle(d, dd, idx2)


@pytest.mark.parametrize("seed", range(10))
def test_sparse_attn_random_shapes(seed):
    """Seeded random per-head-KV shapes: 1-5 sequences with ragged lengths,
    head dims 64 or 128, GQA groups 1/2/4 (the instantiated set; other
    groups are refused with DSA_ERR_UNSUPPORTED), k from 1 to 12,000 (k > L rows
    included), shuffled or identity pages, and index sets with -1 entries
    scattered through them."""
    rng = np.random.default_rng(2000 + seed)
    B = int(rng.integers(1, 6))
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    H = Hkv * int(rng.choice([1, 2, 4]))
    lens = [int(x) for x in rng.integers(1, 20000, size=B)]
    k = int(rng.choice([1, 17, 256, 2048, 5000, 12000]))
    log("sparse_attn random", seed, B, H, Hkv, D, k, lens)
    d = I.draft_inputs(3000 + seed, lens, H_I=4, D_I=32, H_q=H, H_kv=Hkv, D_qk=D, D_v=D, k=k, page=64,
                       shuffle_pages=bool(seed % 2), G=1)
    dd = DraftDev(d)
    idx = np.full((B, k), -1, np.int64)
    for b in range(B):
        n = min(k, lens[b])
        sel = rng.choice(lens[b], n, replace=False)
        sel[rng.random(n) < 0.05] = -1          # scattered absent entries
        idx[b, :n] = sel
        rng.shuffle(idx[b])
    _attn_vs_oracle(d, dd, idx)


def test_sparse_attn_k_covers_context_equals_dense():
    d = I.draft_inputs(12, [700, 333], H_I=4, D_I=32, H_q=8, H_kv=8, D_qk=128, D_v=128, k=1024, G=1)
    dd = DraftDev(d)
    idx = np.full((d.B, d.k), -1, np.int64)
    for b in range(d.B):
        idx[b, : d.lens[b]] = np.arange(d.lens[b])
    out, lse, _ = _attn_vs_oracle(d, dd, idx)
    for b in range(d.B):
        o_dense, l_dense = O.dense_attn(d.q[0, b], d.K[b], d.V[b], d.lens[b], d.sm_scale)
        assert np.abs(out[b] - o_dense).max() <= ATTN_TOL
        assert np.abs(lse[b] - l_dense).max() <= ATTN_TOL


def test_sparse_attn_empty_and_single():
    d = I.draft_inputs(13, [300], H_I=4, D_I=32, H_q=4, H_kv=4, D_qk=64, D_v=64, k=64, G=1)
    dd = DraftDev(d)
    idx = np.full((1, 64), -1, np.int64)
    out, lse = dsa.sparse_attn(dd.q[0][:, None], dd.k, dd.v, dd.bt, to_dev(idx.astype(np.int32)),
                               page=d.page, sm_scale=d.sm_scale)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    idx[0, 17] = 123
    out, _, _ = _attn_vs_oracle(d, dd, idx)
    np.testing.assert_allclose(out[0], d.V[0][123], atol=1e-6)


# ----------------------------------------------------------------------------
# the draft block: IndexShare + KVShare (the tiny configuration, k > L, latent)
# ----------------------------------------------------------------------------
DRAFT_BLOCK_CASES = {
    # the tiny configuration (MHA 4 x 64, k = 64 of 512)
    "tiny": dict(lens=[512], H_I=4, D_I=32, H_q=4, H_kv=4, D_qk=64, D_v=64, k=64, latent=False, shuffle=False),
    # k > L: -1 padding after the L kept positions, inside the one split
    "mha_k_gt_L": dict(lens=[100, 700], H_I=64, D_I=128, H_q=16, H_kv=8, D_qk=128, D_v=128, k=512,
                       latent=False, shuffle=True),
    # latent MQA, k > L: two 64-token splits, the second part padding
    "latent_k_gt_L": dict(lens=[100], H_I=64, D_I=128, H_q=64, H_kv=1, D_qk=576, D_v=512, k=128,
                          latent=True, shuffle=True),
    # latent MQA, two sequences: the shorter one ends with padding splits and
    # a split that is part padding
    "latent_two_seqs": dict(lens=[3000, 1500], H_I=64, D_I=128, H_q=64, H_kv=1, D_qk=576, D_v=512, k=2048,
                            latent=True, shuffle=True),
}


def _draft_case(case, poison):
    c = DRAFT_BLOCK_CASES[case]
    return I.draft_inputs(0, c["lens"], H_I=c["H_I"], D_I=c["D_I"], H_q=c["H_q"], H_kv=c["H_kv"], D_qk=c["D_qk"],
                          D_v=c["D_v"], k=c["k"], G=7, integer_indexer=True, latent=c["latent"],
                          shuffle_pages=c["shuffle"], poison=poison, spare_page0=True)


@pytest.mark.parametrize("case", list(DRAFT_BLOCK_CASES))
@pytest.mark.parametrize("poison", [False, True])
def test_draft_block(case, poison):
    """Indexer -> top-k -> 7 attention steps reusing the step-1 indices.
    Poisoned runs hold NaN in every row no target wrote: the draft slots, the
    unused page tails and a physical page 0 that no sequence owns (the row an
    absent token's load falls back to).  Outputs must be finite, match the
    oracle, and equal the clean run bit for bit; idx is unchanged by the steps."""
    log("draft block", case, "poison", poison)
    d = _draft_case(case, poison)
    dd = DraftDev(d)
    scores = dsa.index_scores(dd.q_index, dd.w, dd.kidx, dd.bt, dd.row_len, page=d.page, ld=dd.ld)
    idx = dsa.topk(scores, dd.row_len, d.k)[:, 0]
    idx_before = idx.clone()
    outs = []
    for j in range(d.G):
        o, lse = dsa.sparse_attn(dd.q[j][:, None], dd.k, dd.v, dd.bt, idx, page=d.page, D_v=d.D_v,
                                 sm_scale=d.sm_scale)
        outs.append((o.cpu().numpy()[:, 0], lse.cpu().numpy()[:, 0]))
    assert torch.equal(idx, idx_before)      # steps 2..7 reuse the step-1 indices unchanged
    for b in range(d.B):
        L = int(d.lens[b])
        ref_idx, ref_o, ref_lse = O.draft_block(d.q_index[b, 0], d.w[b, 0], d.keys[b], L, d.k,
                                                d.q[:, b], d.K[b], d.V[b], d.sm_scale)
        np.testing.assert_array_equal(idx.cpu().numpy()[b], ref_idx)
        assert np.all(ref_idx < L)
        for j in range(d.G):
            o, lse = outs[j]
            assert np.all(np.isfinite(o[b])), (case, b, j)
            assert np.abs(o[b] - ref_o[j]).max() <= ATTN_TOL
            assert np.abs(lse[b] - ref_lse[j]).max() <= ATTN_TOL
    if poison:
        cd = DraftDev(_draft_case(case, False))
        for j in range(d.G):
            o, lse = dsa.sparse_attn(cd.q[j][:, None], cd.k, cd.v, cd.bt, idx, page=d.page, D_v=d.D_v,
                                     sm_scale=d.sm_scale)
            np.testing.assert_array_equal(o.cpu().numpy()[:, 0], outs[j][0])
            np.testing.assert_array_equal(lse.cpu().numpy()[:, 0], outs[j][1])


def test_latent_poisoned_padding_in_shuffled_splits():
    """Latent MQA with -1 entries scattered through every split and the
    selection in shuffled order, on a poisoned cache (NaN in the physical
    page 0 that absent tokens fall back to): same bits as the clean cache."""
    kw = dict(H_I=4, D_I=32, H_q=64, D_qk=576, D_v=512, k=1000, G=1, latent=True, shuffle_pages=True,
              spare_page0=True)
    d = I.draft_inputs(33, [1500], poison=True, **kw)
    clean = I.draft_inputs(33, [1500], poison=False, **kw)
    rng = np.random.default_rng(9)
    idx = np.full((1, d.k), -1, np.int64)
    idx[0, :700] = rng.choice(1500, 700, replace=False)
    rng.shuffle(idx[0])
    dd, cd = DraftDev(d), DraftDev(clean)
    got, lse, _ = _attn_vs_oracle(d, dd, idx)
    assert np.all(np.isfinite(got))
    o2, l2 = dsa.sparse_attn(cd.q[0][:, None], cd.k, cd.v, cd.bt, to_dev(idx.astype(np.int32)), page=d.page,
                             D_v=d.D_v, sm_scale=d.sm_scale)
    np.testing.assert_array_equal(o2.cpu().numpy()[:, 0], got)
    np.testing.assert_array_equal(l2.cpu().numpy()[:, 0], lse)


# ----------------------------------------------------------------------------
# a4 verification
# ----------------------------------------------------------------------------
def _verify_case(vi, use_philox, tol_margin=1e-5):
    B, G, V = vi.shape
    ua, us = I.verify_uniforms(vi.seed, vi.offset, B, G)
    tl = to_dev(vi.target_logits)
    dl = to_dev(vi.draft_logits)
    dr = to_dev(vi.drafts)
    diag = torch.empty((B, G + 1, 4), device=DEV)
    if use_philox:
        n, em = dsa.spec_verify(tl, dl, dr, seed=vi.seed, offset=vi.offset, diag=diag)
    else:
        uni = np.zeros((B, G + 1, 2), np.float32)
        uni[:, :G, 0] = ua
        uni[:, :, 1] = us
        n, em = dsa.spec_verify(tl, dl, dr, uniforms=to_dev(uni), diag=diag)
    n = n.cpu().numpy()
    em = em.cpu().numpy()
    dg = diag.cpu().numpy()
    ref_n, ref_em, res = O.spec_verify(vi.target_logits, vi.draft_logits, vi.drafts, ua, us)
    near = 0
    for b in range(B):
        r = res[b]
        j = min(n[b], ref_n[b])
        # uniforms actually used match the generator bit for bit
        np.testing.assert_array_equal(dg[b, : j + 1 if j < G else G, 2], ua[b, : j + 1 if j < G else G])
        assert dg[b, n[b], 3] == us[b, n[b]]
        if n[b] != ref_n[b]:
            jj = min(n[b], ref_n[b])
            assert r["accept_margin"][jj] < tol_margin, (b, n[b], ref_n[b], r["accept_margin"][jj])
            near += 1
            continue
        np.testing.assert_array_equal(em[b, : n[b]], vi.drafts[b, : n[b]])
        assert np.all(em[b, n[b] + 1:] == -1)
        if em[b, n[b]] != ref_em[b, n[b]]:
            assert r["sample_margin"] < tol_margin, (b, em[b, n[b]], ref_em[b, n[b]], r["sample_margin"])
            near += 1
        # probabilities of the drafted tokens as the kernel used them
        m = n[b] + (1 if n[b] < G else 0)
        np.testing.assert_allclose(dg[b, :m, 0], r["p_draft"][:m], rtol=2e-5, atol=1e-30)
        np.testing.assert_allclose(dg[b, :m, 1], r["q_draft"][:m], rtol=2e-5, atol=1e-30)
    log(f"verify B={B} G={G} V={V}: mean n={n.mean():.3f}, near-margin cases={near}")
    return n, em, near


@pytest.mark.parametrize("use_philox", [False, True])
def test_spec_verify_tiny(use_philox):
    w = I.WORKLOADS["tiny"]
    vi = I.verify_inputs(w["seed"], 1, w["G"], w["vocab"], w["logit_std"], independent=True)
    n, em, near = _verify_case(vi, use_philox)
    assert near == 0


@pytest.mark.parametrize("std", [0.5, 2.0, 6.0])
def test_spec_verify_many_sequences(std):
    vi = I.verify_inputs(int(std * 10), 64, 7, 5003, std)        # V not a multiple of 4
    _, _, near = _verify_case(vi, True)
    assert near <= 1
    vi = I.verify_inputs(int(std * 10) + 1, 16, 7, 151552, std)
    _, _, near = _verify_case(vi, True)
    assert near <= 1


@pytest.mark.parametrize("B,G,V", [
    (1, 1, 1000),       # one draft
    (3, 32, 4099),      # the largest chain, V not a multiple of 4
    (16, 7, 2048),      # largest batch with the decision inside the mass kernel
    (17, 7, 2048),      # first batch size with the decision in a kernel of its own
    (8, 7, 600000),     # decision inside the mass kernel, logits past the last-level cache (streamed)
])
@pytest.mark.parametrize("schedule", ["onepass", "phased"])
def test_spec_verify_shape_edges(B, G, V, schedule, monkeypatch):
    monkeypatch.setenv("DSA_VERIFY_SCHEDULE", schedule)
    vi = I.verify_inputs(B * 100 + G, B, G, V, 2.0)
    _, _, near = _verify_case(vi, True)
    assert near <= 1


def test_spec_verify_special_cases():
    rng = np.random.default_rng(3)
    B, G, V = 8, 7, 2048
    tl = (rng.standard_normal((B, G + 1, V)) * 2).astype(np.float32)
    # p == q: everything accepted, bonus from p_G
    vi = I.VerifyInputs(tl, tl[:, :G].copy(), rng.integers(0, V, (B, G)).astype(np.int32), 9, 0)
    n, em, _ = _verify_case(vi, True)
    assert np.all(n == G)
    # draft mass only where target is -inf: always rejected at the first position
    tl2 = tl.copy()
    tl2[:, :, V // 2:] = -np.inf
    dl2 = np.full((B, G, V), -np.inf, np.float32)
    dl2[:, :, V // 2:] = 0.0
    dr = rng.integers(V // 2, V, (B, G)).astype(np.int32)
    n, em, _ = _verify_case(I.VerifyInputs(tl2, dl2, dr, 10, 0), True)
    assert np.all(n == 0) and np.all(em[:, 0] < V // 2)


@pytest.mark.parametrize("schedule", ["onepass", "phased"])
@pytest.mark.parametrize("V", [2048, 5003, 151552])
def test_spec_verify_draw_at_the_top_of_the_cdf(V, schedule, monkeypatch):
    """u_smp = 1 - 2^-24 puts u * W within rounding of the total residual
    mass W, where the crossing search may find no crossing and must fall back
    to the last positive entry at every level.  The residual is positive only
    in the last 768 tokens (the tiles before them have zero mass) and the
    last token holds 1/768 of W, so the oracle's draw is the last token.  Both
    schedules."""
    monkeypatch.setenv("DSA_VERIFY_SCHEDULE", schedule)
    B, G = 4, 7
    tl = np.zeros((B, G + 1, V), np.float32)
    tl[..., V - 768:] = 2.0
    dl = np.full((B, G, V), 2.0, np.float32)
    dl[..., V - 768:] = 0.0
    dr = np.full((B, G), 5, np.int32)                 # q(5) > p(5): rejected at j = 0 with u_acc = 0.999
    uni = np.zeros((B, G + 1, 2), np.float32)
    uni[..., 0] = 0.999
    uni[..., 1] = np.float32(1.0 - 2.0**-24)
    uni[1, :, 0] = 0.0                                # sequence 1 accepts everything: bonus draw from p
    dr[1] = V - 1
    n, em = dsa.spec_verify(to_dev(tl), to_dev(dl), to_dev(dr), uniforms=to_dev(uni))
    ref_n, ref_em, _ = O.spec_verify(tl, dl, dr, uni[:, :G, 0], uni[:, :, 1])
    n, em = n.cpu().numpy(), em.cpu().numpy()
    np.testing.assert_array_equal(n, ref_n)
    np.testing.assert_array_equal(em, ref_em)
    assert ref_em[0, 0] == V - 1 and np.all(em[np.arange(B), n] >= 0)


@pytest.mark.parametrize("B,G,V,std", [
    (64, 7, 5003, 2.0),        # V not a multiple of 4 (no 16-byte loads)
    (40, 7, 151552, 0.5),
    (24, 15, 20000, 6.0),      # block-16 chain
    (100, 1, 4096, 2.0),       # one draft: a phase for it and one for the bonus row
    (3, 32, 4099, 2.0),        # the longest chain
    (4, 7, 1 << 20, 2.0),      # the largest vocabulary: 64 chunks per row
])
def test_spec_verify_early_exit(B, G, V, std, monkeypatch):
    """The early-exit schedule (one launch per position; rows past a
    sequence's first rejection are never read), forced at sizes below its
    threshold: decisions, tokens and the diagnostics of the evaluated
    positions equal the oracle's, as for the one-pass schedule."""
    monkeypatch.setenv("DSA_VERIFY_SCHEDULE", "phased")
    log("spec_verify early exit", B, G, V, std)
    vi = I.verify_inputs(B * 1000 + G, B, G, V, std)
    n, _, near = _verify_case(vi, bool(B % 2))
    assert near <= B // 64 + 1
    assert 0 < n.mean() < G   # rejections and accepted positions both occur


def test_spec_verify_early_exit_special_cases(monkeypatch):
    """Early-exit schedule at the extremes: p == q accepts every draft (every
    sequence runs all phases and draws its bonus token from p_G), and draft
    mass only where the target has none rejects every chain at position 0
    (no later phase reads a row)."""
    monkeypatch.setenv("DSA_VERIFY_SCHEDULE", "phased")
    rng = np.random.default_rng(11)
    B, G, V = 16, 3, 30000
    tl = (rng.standard_normal((B, G + 1, V)) * 2).astype(np.float32)
    vi = I.VerifyInputs(tl, tl[:, :G].copy(), rng.integers(0, V, (B, G)).astype(np.int32), 12, 0)
    n, em, _ = _verify_case(vi, True)
    assert np.all(n == G)
    tl[:, :, V // 2:] = -np.inf
    dl = np.full((B, G, V), -np.inf, np.float32)
    dl[:, :, V // 2:] = 0.0
    dr = rng.integers(V // 2, V, (B, G)).astype(np.int32)
    n, em, _ = _verify_case(I.VerifyInputs(tl, dl, dr, 13, 0), False)
    assert np.all(n == 0) and np.all(em[:, 0] < V // 2)


def test_spec_verify_schedules_agree(monkeypatch):
    """Both schedules on the same batch: the same accepted lengths and
    emitted tokens, except where a draw or test lies within the float32
    rounding of its threshold (the schedules fold the softmax statistics in
    different chunks)."""
    vi = I.verify_inputs(77, 48, 7, 50000, 2.0)
    out = {}
    for sched in ("onepass", "phased"):
        monkeypatch.setenv("DSA_VERIFY_SCHEDULE", sched)
        n, em = dsa.spec_verify(to_dev(vi.target_logits), to_dev(vi.draft_logits), to_dev(vi.drafts),
                                seed=vi.seed, offset=vi.offset)
        out[sched] = (n.cpu().numpy(), em.cpu().numpy())
    ua, us = I.verify_uniforms(vi.seed, vi.offset, 48, 7)
    _, _, res = O.spec_verify(vi.target_logits, vi.draft_logits, vi.drafts, ua, us)
    for b in range(48):
        same = out["onepass"][0][b] == out["phased"][0][b] and np.array_equal(out["onepass"][1][b], out["phased"][1][b])
        if not same:
            r = res[b]
            assert min(np.nanmin(r["accept_margin"]), r["sample_margin"]) < 1e-5, b


@pytest.mark.parametrize("seed", range(8))
def test_spec_verify_random_shapes(seed):
    """Seeded random verification shapes: 1-40 sequences, 1-32 drafts,
    vocabularies from 1,000 to 160,000 (odd sizes included), logit scales 0.3 to 8,
    in-kernel Philox or caller-supplied uniforms; decisions and tokens must
    equal the oracle's except near-margin cases (at most one per 64
    sequences, plus one)."""
    rng = np.random.default_rng(4000 + seed)
    B = int(rng.integers(1, 41))
    G = int(rng.integers(1, 33))
    V = int(rng.integers(1000, 160001))
    std = float(rng.choice([0.3, 1.0, 2.0, 4.0, 8.0]))
    log("spec_verify random", seed, B, G, V, std)
    vi = I.verify_inputs(5000 + seed, B, G, V, std)
    _, _, near = _verify_case(vi, bool(seed % 2))
    assert near <= B // 64 + 1


@pytest.mark.parametrize("std", [0.5, 2.0])
def test_spec_verify_block16(std):
    """Block-16 layout: G = 15 drafts plus the bonus position."""
    vi = I.verify_inputs(int(std * 10) + 70, 24, 15, 5003, std)
    _, _, near = _verify_case(vi, True)
    assert near <= 1
    vi = I.verify_inputs(int(std * 10) + 71, 4, 15, 151552, std)
    _, _, near = _verify_case(vi, False)
    assert near <= 1


# ----------------------------------------------------------------------------
# greedy verification (bit-exact: only comparisons)
# ----------------------------------------------------------------------------
def _greedy_inputs(rng, B, G, V, integer):
    if integer:
        tl = rng.integers(-4, 5, size=(B, G + 1, V)).astype(np.float32)      # ties everywhere
    else:
        tl = (rng.standard_normal((B, G + 1, V)) * 2).astype(np.float32)
    best = tl.argmax(axis=-1)
    cut = rng.integers(0, G + 1, size=B)                                     # drafts agree on a prefix
    dr = rng.integers(0, V, size=(B, G)).astype(np.int32)
    for b in range(B):
        dr[b, : cut[b]] = best[b, : cut[b]]
    return tl, dr


@pytest.mark.parametrize("schedule", ["onepass", "phased"])
@pytest.mark.parametrize("G,V,integer", [(7, 1024, True), (7, 1024, False), (15, 1000, True), (15, 5003, False),
                                          (7, 151552, True), (1, 4, False), (32, 3001, True)])
def test_greedy_verify(G, V, integer, schedule, monkeypatch):
    """Both schedules (one pass over every row; early exit, which reads a
    row only while the chain is still accepted), bit-exact with the oracle."""
    monkeypatch.setenv("DSA_VERIFY_SCHEDULE", schedule)
    rng = np.random.default_rng(G * 7 + V + integer)
    B = 6 if V > 100000 else 40
    tl, dr = _greedy_inputs(rng, B, G, V, integer)
    n, em = dsa.spec_verify_greedy(to_dev(tl), to_dev(dr))
    ref_n, ref_em = O.greedy_verify(tl, dr)
    np.testing.assert_array_equal(n.cpu().numpy(), ref_n)
    np.testing.assert_array_equal(em.cpu().numpy(), ref_em)


@pytest.mark.parametrize("schedule", ["onepass", "phased"])
def test_greedy_verify_special_rows(schedule, monkeypatch):
    monkeypatch.setenv("DSA_VERIFY_SCHEDULE", schedule)
    G, V = 3, 4099
    tl = np.zeros((3, G + 1, V), np.float32)
    tl[0] = -np.inf
    tl[0, :, 17] = 1.0                          # one finite entry per row
    tl[1, :, :] = -0.0
    tl[1, :, 5:] = 0.0                          # -0.0 == +0.0: token 0 wins
    tl[2, :, V - 1] = 3.0                       # maximum in the ragged tail
    dr = np.array([[17, 17, 17], [0, 0, 1], [V - 1, 0, 0]], np.int32)
    n, em = dsa.spec_verify_greedy(to_dev(tl), to_dev(dr))
    ref_n, ref_em = O.greedy_verify(tl, dr)
    np.testing.assert_array_equal(n.cpu().numpy(), ref_n)
    np.testing.assert_array_equal(em.cpu().numpy(), ref_em)
    assert list(ref_n) == [3, 2, 1]


# ----------------------------------------------------------------------------
# cross-layer IndexShare and the mixed-KV negative control
# ----------------------------------------------------------------------------
def test_cross_layer_index_share():
    """One indexer + top-k for a block of 4 layers; each layer attends with its
    own queries and paged KV over the shared selection."""
    lens = [3000, 1777]
    layers = [I.draft_inputs(60 + l, lens, H_I=64, D_I=128, H_q=16, H_kv=8, D_qk=128, D_v=128, k=512, G=1,
                             shuffle_pages=True, integer_indexer=True) for l in range(4)]
    d0 = layers[0]
    dd0 = DraftDev(d0)
    scores = dsa.index_scores(dd0.q_index, dd0.w, dd0.kidx, dd0.bt, dd0.row_len, page=d0.page, ld=dd0.ld)
    idx = dsa.topk(scores, dd0.row_len, d0.k)[:, 0]
    for b in range(len(lens)):
        ref_idx, ref_o, ref_lse = O.layer_block(d0.q_index[b, 0], d0.w[b, 0], d0.keys[b], lens[b], d0.k,
                                                [l.q[0, b] for l in layers], [l.K[b] for l in layers],
                                                [l.V[b] for l in layers], d0.sm_scale)
        np.testing.assert_array_equal(idx.cpu().numpy()[b], ref_idx)
        for li, l in enumerate(layers):
            dl = DraftDev(l)
            o, lse = dsa.sparse_attn(dl.q[0][:, None], dl.k, dl.v, dl.bt, idx, page=l.page, sm_scale=l.sm_scale)
            assert np.abs(o.cpu().numpy()[b, 0] - ref_o[li]).max() <= ATTN_TOL
            assert np.abs(lse.cpu().numpy()[b, 0] - ref_lse[li]).max() <= ATTN_TOL


@pytest.mark.parametrize("poison", [False, True])
def test_mixed_kv_negative_control(poison):
    """GLM-5.1 mixed-KV drafting: step j also reads draft-written slots
    L..L+j-1 (per-row index sets, one call with S_q = G).  Clean inputs match
    the oracle; with those slots poisoned (NaN) every step after the first
    turns NaN, while the IndexShare chain over the same cache stays finite."""
    G = 7
    d = I.draft_inputs(31, [2500], H_I=64, D_I=128, H_q=16, H_kv=16, D_qk=128, D_v=128, k=256, G=G,
                       integer_indexer=True, poison=poison)
    dd = DraftDev(d)
    L = int(d.lens[0])
    scores = dsa.index_scores(dd.q_index, dd.w, dd.kidx, dd.bt, dd.row_len, page=d.page, ld=dd.ld)
    idx = dsa.topk(scores, dd.row_len, d.k)[:, 0]
    sets = O.mixed_kv_sets(idx.cpu().numpy()[0], L, G)                   # [G, k + G - 1]
    q = dd.q[:, 0][None].contiguous()                                      # [1, G, H, D]: one row per step
    o, lse = dsa.sparse_attn(q, dd.k, dd.v, dd.bt, to_dev(sets.astype(np.int32))[None], page=d.page,
                             sm_scale=d.sm_scale)
    o = o.cpu().numpy()[0]
    o_share, _ = dsa.sparse_attn(q, dd.k, dd.v, dd.bt, idx, page=d.page, sm_scale=d.sm_scale)
    assert np.all(np.isfinite(o_share.cpu().numpy()))
    if poison:
        assert np.all(np.isfinite(o[0]))
        assert np.all(np.isnan(o[1:]))
    else:
        _, ref_o, ref_lse = O.mixed_kv_draft_block(d.q_index[0, 0], d.w[0, 0], d.keys[0], L, d.k, d.q[:, 0],
                                                   d.K[0], d.V[0], d.sm_scale)
        assert np.abs(o - ref_o).max() <= ATTN_TOL
        assert np.abs(lse.cpu().numpy()[0] - ref_lse).max() <= ATTN_TOL


# ----------------------------------------------------------------------------
# lengths and positions outside the contract are clamped, never read or
# written out of bounds
# ----------------------------------------------------------------------------
def test_out_of_contract_lengths_are_clamped():
    d = I.draft_inputs(71, [3000], H_I=64, D_I=128, H_q=16, H_kv=16, D_qk=128, D_v=128, k=256, G=2,
                       integer_indexer=True)
    dd = DraftDev(d)
    ld = 3002
    cap = min(ld, d.page * d.max_pages)
    ref = dsa.index_scores(dd.q_index, dd.w, dd.kidx, dd.bt, torch.full((1, 1), cap, dtype=torch.int32, device=DEV),
                           page=d.page, ld=ld)
    big = torch.full((1, 1), 1 << 30, dtype=torch.int32, device=DEV)
    got = dsa.index_scores(dd.q_index, dd.w, dd.kidx, dd.bt, big, page=d.page, ld=ld)
    assert torch.equal(got[..., :cap], ref[..., :cap])
    # top-k: a row_len above ld acts as ld (one-workgroup and pipeline paths)
    for L in (3002, 40000):
        sc = torch.randn((1, 1, L), device=DEV)
        a = dsa.topk(sc, torch.full((1, 1), L, dtype=torch.int32, device=DEV), 256)
        b = dsa.topk(sc, torch.full((1, 1), L + 1000, dtype=torch.int32, device=DEV), 256)
        assert torch.equal(a, b)
    # attention: positions past the block table are ignored like -1
    idx = dsa.topk(ref, torch.full((1, 1), 3000, dtype=torch.int32, device=DEV), d.k)[:, 0]
    bad = idx.clone()
    bad[0, :5] = d.page * d.max_pages + torch.arange(5, device=DEV, dtype=torch.int32) * 1000
    neg = idx.clone()
    neg[0, :5] = -1
    o1, l1 = dsa.sparse_attn(dd.q[0][:, None], dd.k, dd.v, dd.bt, bad, page=d.page, sm_scale=d.sm_scale)
    o2, l2 = dsa.sparse_attn(dd.q[0][:, None], dd.k, dd.v, dd.bt, neg, page=d.page, sm_scale=d.sm_scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ----------------------------------------------------------------------------
# HIP graph capture of the draft block: every replay matches the eager result
# ----------------------------------------------------------------------------
def test_draft_block_graph_replays():
    d = I.draft_inputs(21, [3000], H_I=64, D_I=128, H_q=16, H_kv=16, D_qk=128, D_v=128, k=512, G=3)
    dd = DraftDev(d)
    scores = torch.empty((1, 1, dd.ld), device=DEV)
    idx = torch.empty((1, 1, d.k), dtype=torch.int32, device=DEV)
    outs = torch.empty((d.G, 1, 1, d.H_q, d.D_v), device=DEV)
    lses = torch.empty((d.G, 1, 1, d.H_q), device=DEV)
    ws = torch.empty(max(1, dsa.sparse_attn_workspace_size(1, 1, d.H_q, d.H_kv, d.D_qk, d.D_v, d.k)),
                     dtype=torch.uint8, device=DEV)
    vi = I.verify_inputs(22, 4, 7, 3000, 2.0)
    tl, dl, dr = to_dev(vi.target_logits), to_dev(vi.draft_logits), to_dev(vi.drafts)
    n = torch.empty(4, dtype=torch.int32, device=DEV)
    em = torch.empty((4, 8), dtype=torch.int32, device=DEV)
    vws = torch.empty(dsa.spec_verify_workspace_size(4, 7, 3000), dtype=torch.uint8, device=DEV)

    def block():
        dsa.index_scores(dd.q_index, dd.w, dd.kidx, dd.bt, dd.row_len, page=d.page, out=scores)
        dsa.topk(scores, dd.row_len, d.k, out=idx)
        for j in range(d.G):
            dsa.sparse_attn(dd.q[j][:, None], dd.k, dd.v, dd.bt, idx[:, 0], page=d.page, sm_scale=d.sm_scale,
                            out=outs[j], lse=lses[j], workspace=ws)
        dsa.spec_verify(tl, dl, dr, seed=5, offset=1, accepted_len=n, emitted=em, workspace=vws)

    block()
    torch.cuda.synchronize()
    ref = [x.clone() for x in (scores, idx, outs, lses, n, em)]
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        block()
    L = int(d.lens[0])
    for rep in range(4):
        for x in (scores, idx, outs, lses, n, em):
            x.zero_()                    # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(scores[..., :L], ref[0][..., :L]), f"replay {rep}: scores differ"
        for a, b in zip((idx, outs, lses, n, em), ref[1:]):
            assert torch.equal(a, b), f"replay {rep} differs"


@pytest.mark.parametrize("schedule", ["onepass", "phased"])
def test_emitted_tokens_follow_target_distribution(schedule, monkeypatch):
    """The kernel preserves the target distribution (section "Rejection
    sampling and a loss that optimizes acceptance directly"): over 13,000
    independent chains with the same logits, drafts drawn from q and the
    in-kernel Philox uniforms, the first emitted token follows p_1 and the
    second (after an accepted first draft) p_2, by a chi-square test, and the
    first draft's acceptance rate equals sum_x min(p_1, q_1)."""
    from scipy import stats
    monkeypatch.setenv("DSA_VERIFY_SCHEDULE", schedule)
    rng = np.random.default_rng(44)
    V, B, G = 10, 13000, 2
    tl1 = (rng.standard_normal((G + 1, V)) * 1.2).astype(np.float32)
    dl1 = (rng.standard_normal((G, V)) * 1.2).astype(np.float32)
    p = [O.softmax(tl1[j].astype(np.float64)) for j in range(G + 1)]
    q = [O.softmax(dl1[j].astype(np.float64)) for j in range(G)]
    tl = np.ascontiguousarray(np.broadcast_to(tl1, (B, G + 1, V)))
    dl = np.ascontiguousarray(np.broadcast_to(dl1, (B, G, V)))
    dr = np.stack([rng.choice(V, size=B, p=q[j]) for j in range(G)], axis=1).astype(np.int32)
    n, em = dsa.spec_verify(to_dev(tl), to_dev(dl), to_dev(dr), seed=123, offset=0)
    n, em = n.cpu().numpy(), em.cpu().numpy()
    # the first draft is accepted with probability sum_x min(p_1, q_1)
    # (section "Kimi K3"), within five standard errors
    alpha = float(np.minimum(p[0], q[0]).sum())
    assert abs(float((n >= 1).mean()) - alpha) < 5 * math.sqrt(alpha * (1 - alpha) / B)
    first = np.bincount(em[:, 0], minlength=V)
    second = np.bincount(em[n >= 1, 1], minlength=V)
    for counts, pj in ((first, p[0]), (second, p[1])):
        exp = pj * counts.sum()
        assert exp.min() >= 5
        assert stats.chisquare(counts, exp).pvalue > 1e-3


@pytest.mark.parametrize("schedule", ["onepass", "phased"])
def test_verify_graph_replays(schedule, monkeypatch):
    """Rejection-sampling and greedy verification captured in one HIP graph
    (the early-exit schedule is G+3 and 4 dependent launches): every replay,
    with eager work and synchronisation between replays, gives the eager
    call's accepted lengths, tokens and diagnostics."""
    monkeypatch.setenv("DSA_VERIFY_SCHEDULE", schedule)
    B, G, V = 24, 7, 20000
    vi = I.verify_inputs(31, B, G, V, 2.0)
    tl, dl, dr = to_dev(vi.target_logits), to_dev(vi.draft_logits), to_dev(vi.drafts)
    gdr = tl[:, :G].argmax(dim=-1).to(torch.int32)
    gdr[::3, 2] = (gdr[::3, 2] + 1) % V            # some greedy chains stop at position 2
    n = torch.empty(B, dtype=torch.int32, device=DEV)
    em = torch.empty((B, G + 1), dtype=torch.int32, device=DEV)
    dg = torch.empty((B, G + 1, 4), device=DEV)
    gn = torch.empty(B, dtype=torch.int32, device=DEV)
    gem = torch.empty((B, G + 1), dtype=torch.int32, device=DEV)
    vws = torch.empty(dsa.spec_verify_workspace_size(B, G, V), dtype=torch.uint8, device=DEV)
    gws = torch.empty(dsa.spec_verify_greedy_workspace_size(B, G, V), dtype=torch.uint8, device=DEV)

    def call():
        dsa.spec_verify(tl, dl, dr, seed=7, offset=3, accepted_len=n, emitted=em, diag=dg, workspace=vws)
        dsa.spec_verify_greedy(tl, gdr, accepted_len=gn, emitted=gem, workspace=gws)

    call()
    torch.cuda.synchronize()
    outs = (n, em, dg, gn, gem)
    ref = [x.clone() for x in outs]
    assert 0 < float(n.float().mean()) < G and 0 < float(gn.float().mean()) < G
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        call()
    for rep in range(4):
        for x in outs:
            x.zero_()                    # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(a.nan_to_num(-9.0), b.nan_to_num(-9.0)), f"replay {rep} differs"


# ----------------------------------------------------------------------------
# latent MQA attention (one 576-d KV row shared by 64 heads, V = first 512)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("case", [
    dict(lens=[3000, 1500], k=2048, shuffle=True),      # split-k, ragged, one row with -1 padding
    dict(lens=[200], k=64, shuffle=False),              # single split, k < L
    dict(lens=[100], k=128, shuffle=False),             # k > L: padding inside the split
    dict(lens=[1500], k=1000, shuffle=True),            # splits of 63 tokens (a partial chunk)
    dict(lens=[9000], k=8192, shuffle=True),            # several 64-token chunks per split
    dict(lens=[40000], k=32768, shuffle=True),          # the largest k: 32 splits of 1024 tokens
])
def test_latent_attn_matches_oracle(case):
    log("latent", case)
    d = I.draft_inputs(31, case["lens"], H_I=4, D_I=32, H_q=64, D_qk=576, D_v=512, k=case["k"], G=2,
                       latent=True, shuffle_pages=case["shuffle"])
    dd = DraftDev(d)
    rng = np.random.default_rng(7)
    idx = np.full((d.B, d.k), -1, np.int64)
    for b in range(d.B):
        n = min(d.k, int(d.lens[b]))
        idx[b, :n] = np.sort(rng.choice(int(d.lens[b]), n, replace=False))
    _, _, err = _attn_vs_oracle(d, dd, idx)
    log(f"  latent max err {err:.2e}")
    idx2 = idx.copy()
    for b in range(d.B):
        rng.shuffle(idx2[b])
    _attn_vs_oracle(d, dd, idx2)


def test_latent_attn_dense_and_empty():
    d = I.draft_inputs(32, [700], H_I=4, D_I=32, H_q=64, D_qk=576, D_v=512, k=1024, G=1, latent=True)
    dd = DraftDev(d)
    idx = np.full((1, d.k), -1, np.int64)
    idx[0, :700] = np.arange(700)
    out, lse, _ = _attn_vs_oracle(d, dd, idx)
    o_dense, l_dense = O.dense_attn(d.q[0, 0], d.K[0], d.V[0], 700, d.sm_scale)
    assert np.abs(out[0] - o_dense).max() <= ATTN_TOL
    idx[:] = -1
    o, l = dsa.sparse_attn(dd.q[0][:, None], dd.k, dd.v, dd.bt, to_dev(idx.astype(np.int32)), page=d.page,
                           D_v=512, sm_scale=d.sm_scale)
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))


# ----------------------------------------------------------------------------
# verify-pass shape: 8 query rows, row r sees [0, L + r + 1), one index set per row
# ----------------------------------------------------------------------------
def test_verify_pass_rows():
    G = 7
    R = G + 1
    d = I.draft_inputs(41, [5000], H_I=64, D_I=128, H_q=16, H_kv=16, D_qk=128, D_v=128, k=512, G=G + 1,
                       R=R, integer_indexer=True)
    L = int(d.lens[0])
    row_len = np.array([[L + r + 1 for r in range(R)]], np.int32)     # causal rows over the drafted chain
    dd = DraftDev(d)
    rl = to_dev(row_len)
    scores = dsa.index_scores(dd.q_index, dd.w, dd.kidx, dd.bt, rl, page=d.page, ld=L + R + 1)
    idx = dsa.topk(scores, rl, d.k)                                     # [1, R, k]
    ref_s = O.index_scores(d.q_index[0], d.w[0].astype(np.float64), d.keys[0], row_len[0])
    got_s = scores.cpu().numpy()[0]
    for r in range(R):
        np.testing.assert_array_equal(got_s[r, : row_len[0, r]], ref_s[r, : row_len[0, r]].astype(np.float32))
        np.testing.assert_array_equal(idx.cpu().numpy()[0, r], O.topk(ref_s[r], row_len[0, r], d.k))
    # 8 query rows, each with its own index set
    q = torch.stack([dd.q[j][0] for j in range(R)])[None]              # [1, R, H, D]
    out, lse = dsa.sparse_attn(q.contiguous(), dd.k, dd.v, dd.bt, idx, page=d.page, sm_scale=d.sm_scale)
    out = out.cpu().numpy()[0]
    for r in range(R):
        o_ref, _ = O.sparse_attn(d.q[r, 0], d.K[0], d.V[0], idx.cpu().numpy()[0, r], d.sm_scale)
        assert np.abs(out[r] - o_ref).max() <= ATTN_TOL


def test_binding_rejects_bad_outputs():
    """Caller-supplied outputs and workspaces of the wrong shape, dtype or
    device are refused by the binding before any launch."""
    d = I.draft_inputs(0, [300], H_I=4, D_I=32, H_q=4, H_kv=4, D_qk=64, D_v=64, k=64, G=2)
    dd = DraftDev(d)
    # valid inputs throughout (the generator's own cache; k = 512 needs a
    # workspace), so only the binding's checks can fail
    idx = torch.full((1, 512), -1, dtype=torch.int32, device=DEV)
    q = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16, device=DEV)
    kc = dd.k
    assert dsa.sparse_attn_workspace_size(1, 1, 4, 4, 64, 64, 512) > 0
    good = torch.empty((1, 1, 4, 64), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        dsa.sparse_attn(q, kc, kc, dd.bt, idx, page=d.page, out=torch.empty((1, 1, 4, 32), device=DEV))
    with pytest.raises(ValueError):
        dsa.sparse_attn(q, kc, kc, dd.bt, idx, page=d.page, out=good, lse=torch.empty((1, 1, 3), device=DEV))
    with pytest.raises(ValueError):
        dsa.sparse_attn(q, kc, kc, dd.bt.repeat(2, 1), idx, page=d.page, out=good)
    with pytest.raises(ValueError):
        dsa.sparse_attn(q, kc, kc, dd.bt, idx, page=d.page, out=good,
                        workspace=torch.empty(1 << 20, dtype=torch.uint8))          # host workspace
    t = torch.zeros((2, 3, 50), device=DEV)
    dl = torch.zeros((2, 2, 50), device=DEV)
    dr = torch.zeros((2, 2), dtype=torch.int32, device=DEV)
    with pytest.raises(ValueError):
        dsa.spec_verify(t, dl, dr, accepted_len=torch.empty(3, dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError):
        dsa.spec_verify(t, dl, dr, emitted=torch.empty((2, 2), dtype=torch.int32, device=DEV))
    with pytest.raises(ValueError):
        dsa.spec_verify_greedy(t, dr, emitted=torch.empty((2, 3), dtype=torch.int64, device=DEV))
