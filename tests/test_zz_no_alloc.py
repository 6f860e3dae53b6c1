"""The allocation-free attention entry point (dsa_sparse_attn_noalloc)
against dsa_sparse_attn with a caller workspace: the same kernels on the same
inputs, so the outputs must be identical bit for bit.  Two calls in a row,
the second smaller, share the library's per-GPU scratch; a shape whose
partials exceed the scratch is refused before any launch."""

import sys

import numpy as np
import pytest
import torch

import dsa_inputs as I

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import dsa_sparse_attention_lightning_amd as dsa
    from dsa_inputs import device as DI
    from gpu_util import DEV, DraftDev, to_dev


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _both(q, kc, vc, bt, idx, page, D_v, scale):
    ref_o, ref_l = dsa.sparse_attn(q, kc, vc, bt, idx, page=page, D_v=D_v, sm_scale=scale)
    o = torch.full_like(ref_o, 7.0)
    l = torch.full_like(ref_l, 7.0)
    dsa.sparse_attn_noalloc(q, kc, vc, bt, idx, page=page, D_v=D_v, sm_scale=scale, out=o, lse=l)
    torch.cuda.synchronize()
    return (o, l), (ref_o, ref_l)


def _ws(B, S_q, H_q, H_kv, D_qk, D_v, k):
    return dsa.sparse_attn_workspace_size(B, S_q, H_q, H_kv, D_qk, D_v, k)


def test_noalloc_matches_workspace_call_twice_second_smaller():
    # first call: the single-sequence 32K decode shape (8 splits x 16 head groups)
    d = DI.draft_inputs(1, [32768], H_I=64, D_I=128, H_q=64, H_kv=64, D_qk=128, D_v=128, k=2048, G=1)
    sc = dsa.index_scores(d.q_index, d.w, d.kidx, d.block_table, d.row_len, page=d.page, ld=d.ld)
    idx = dsa.topk(sc, d.row_len, d.k)[:, 0]
    big = _ws(1, 1, 64, 64, 128, 128, 2048)
    log("noalloc call 1: decode 32K, partials", big, "bytes")
    assert 0 < big <= dsa.NOALLOC_SCRATCH_BYTES
    (o, l), (ro, rl) = _both(d.q[0][:, None], d.k_cache, d.v_cache, d.block_table, idx, d.page, d.D_v, d.sm_scale)
    assert torch.equal(o, ro) and torch.equal(l, rl)
    assert torch.isfinite(o).all()
    del d, sc, idx
    # second call, smaller: two ragged paged sequences, GQA 2, -1 padding
    h = I.draft_inputs(12, [3000, 700], H_I=4, D_I=32, H_q=16, H_kv=8, D_qk=128, D_v=128, k=1024, G=1,
                       shuffle_pages=True)
    hd = DraftDev(h)
    rng = np.random.default_rng(3)
    idx = np.full((h.B, h.k), -1, np.int32)
    for b in range(h.B):
        n = min(h.k, int(h.lens[b]))
        idx[b, :n] = rng.choice(int(h.lens[b]), n, replace=False)
    small = _ws(2, 1, 16, 8, 128, 128, 1024)
    log("noalloc call 2: 2 sequences GQA 2, partials", small, "bytes")
    assert 0 < small < big
    (o, l), (ro, rl) = _both(hd.q[0][:, None], hd.k, hd.v, hd.bt, to_dev(idx), h.page, h.D_v, h.sm_scale)
    assert torch.equal(o, ro) and torch.equal(l, rl)


def test_noalloc_latent_and_single_split():
    h = I.draft_inputs(13, [1500], H_I=4, D_I=32, H_q=64, D_qk=576, D_v=512, k=1024, G=1, latent=True,
                       shuffle_pages=True)
    hd = DraftDev(h)
    idx = to_dev(np.sort(np.random.default_rng(4).choice(1500, 1024, replace=False)).astype(np.int32)[None])
    (o, l), (ro, rl) = _both(hd.q[0][:, None], hd.k, hd.v, hd.bt, idx, h.page, 512, h.sm_scale)
    assert torch.equal(o, ro) and torch.equal(l, rl)
    # one split (no partials at all): k = 64 of a short context
    h = I.draft_inputs(14, [300], H_I=4, D_I=32, H_q=4, H_kv=4, D_qk=64, D_v=64, k=64, G=1)
    hd = DraftDev(h)
    assert _ws(1, 1, 4, 4, 64, 64, 64) == 0
    idx = to_dev(np.arange(64, dtype=np.int32)[None] * 4)
    (o, l), (ro, rl) = _both(hd.q[0][:, None], hd.k, hd.v, hd.bt, idx, h.page, 64, h.sm_scale)
    assert torch.equal(o, ro) and torch.equal(l, rl)


def test_noalloc_refuses_partials_beyond_scratch():
    # 8 query rows with k = 131072: 128 splits x 512 rows x 128 dims of partials
    B, S_q, H, D, k = 1, 8, 64, 128, 131072
    assert _ws(B, S_q, H, H, D, D, k) > dsa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, S_q, H, D), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((2, 64, H, D), dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros((B, 1), dtype=torch.int32, device=DEV)
    idx = torch.full((B, k), -1, dtype=torch.int32, device=DEV)
    out = torch.full((B, S_q, H, D), 3.0, device=DEV)
    lse = torch.full((B, S_q, H), 3.0, device=DEV)
    with pytest.raises(dsa.DSAError) as e:
        dsa.sparse_attn_noalloc(q, kc, kc, bt, idx, page=64, out=out, lse=lse)
    assert e.value.status == 2 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out == 3.0) and torch.all(lse == 3.0)        # nothing was launched
