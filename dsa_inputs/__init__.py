"""Seeded synthetic inputs for the DSA draft-and-verify path.

This module only *makes inputs*: random draws, bf16 rounding of those draws,
page tables and the paged cache layout.  It holds none of the path's
arithmetic (no scores, selections, attention or verification), so both the
HIP library's tests and the CPU oracle can be fed from it.

Every generator is a pure function of its seed.  bf16 tensors are carried as
uint16 bit patterns (for the device) together with their exact float64 values
(for the oracle).

Counter-based uniforms follow Philox4x64-10 (Salmon, Moraes, Dror, Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC'11), taken from
numpy.random.Philox: key = (seed, 0), counter = (offset, b, j, stream), and a
uniform is the top 24 bits of the block's first 64-bit word scaled by 2^-24.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# ----------------------------------------------------------------------------
# bf16 carried as uint16 bit patterns
# ----------------------------------------------------------------------------
BF16_NAN = np.uint16(0x7FC0)


def bf16_bits(x):
    """Round float values to bf16 (round to nearest, ties to even); uint16 bits."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_value(bits):
    """Exact float64 value of uint16 bf16 bit patterns."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# Philox uniforms
# ----------------------------------------------------------------------------
_M64 = (1 << 64) - 1


def philox_block(seed, counter):
    """Philox4x64-10 block (four uint64 words) at a 256-bit counter.

    numpy's Philox increments its counter before encrypting, so it is started
    one below the wanted counter.
    """
    c = sum((int(counter[i]) & _M64) << (64 * i) for i in range(4))
    c = (c - 1) % (1 << 256)
    words = np.array([(c >> (64 * i)) & _M64 for i in range(4)], dtype=np.uint64)
    key = np.array([int(seed) & _M64, 0], dtype=np.uint64)
    bg = np.random.Philox(counter=words, key=key)
    return bg.random_raw(4)


def philox_uniform(seed, offset, b, j, stream):
    x0 = int(philox_block(seed, (offset, b, j, stream))[0])
    return np.float32((x0 >> 40) * (1.0 / (1 << 24)))


def verify_uniforms(seed, offset, B, G):
    """u_accept [B, G] (stream 0) and u_sample [B, G+1] (stream 1), float32."""
    ua = np.zeros((B, G), np.float32)
    us = np.zeros((B, G + 1), np.float32)
    for b in range(B):
        for j in range(G + 1):
            if j < G:
                ua[b, j] = philox_uniform(seed, offset, b, j, 0)
            us[b, j] = philox_uniform(seed, offset, b, j, 1)
    return ua, us


# ----------------------------------------------------------------------------
# Draft-block inputs (indexer, top-k, sparse attention)
# ----------------------------------------------------------------------------
@dataclass
class DraftInputs:
    """One batch of draft-block inputs.

    Device-layout arrays (numpy, ready to copy):
      q_index_bits [B, R, H_I, D_I] u16     w [B, R, H_I] f32
      kidx_bits    [pages, page, D_I] u16   block_table [B, max_pages] i32
      row_len      [B, R] i32               q_bits [G, B, H_q, D_qk] u16
      k_bits       [pages, page, H_kv, D_qk] u16 (or latent [pages, page, D_qk])
      v_bits       [pages, page, H_kv, D_v]  u16 (None when latent: V aliases K)
    Logical float64 views for the oracle (per sequence, positions [0, cap_b)):
      keys[b] [cap_b, D_I], K[b] [cap_b, H_kv, D_qk], V[b] [cap_b, H_kv, D_v]
    """
    lens: np.ndarray
    R: int
    G: int
    H_I: int
    D_I: int
    H_q: int
    H_kv: int
    D_qk: int
    D_v: int
    k: int
    page: int
    latent: bool
    q_index_bits: np.ndarray
    q_index: np.ndarray
    w: np.ndarray
    kidx_bits: np.ndarray
    block_table: np.ndarray
    row_len: np.ndarray
    q_bits: np.ndarray
    q: np.ndarray
    k_bits: np.ndarray
    v_bits: np.ndarray | None
    keys: list = field(default_factory=list)
    K: list = field(default_factory=list)
    V: list = field(default_factory=list)

    @property
    def B(self):
        return len(self.lens)

    @property
    def max_pages(self):
        return self.block_table.shape[1]

    @property
    def sm_scale(self):
        return 1.0 / np.sqrt(self.D_qk)


def _page_table(rng, caps, page, shuffle, spare_page0=False):
    """Block table over one physical pool of sum_b ceil(cap_b / page) pages,
    optionally shuffled once.  spare_page0: the pool gets one more page, at
    physical index 0, that belongs to no sequence (every table entry shifts up
    by one; the random draws are the same as without it)."""
    n_pages = [(c + page - 1) // page for c in caps]
    total = int(sum(n_pages))
    phys = rng.permutation(total) if shuffle else np.arange(total)
    if spare_page0:
        phys = phys + 1
    max_pages = max(n_pages)
    table = np.full((len(caps), max_pages), -1, np.int32)
    pos = 0
    for b, n in enumerate(n_pages):
        table[b, :n] = phys[pos:pos + n]
        pos += n
    return table, total + int(spare_page0)


def _scatter_pages(logical, table_row, pages_arr, page):
    """Write one sequence's logical rows [cap, ...] into its physical pages."""
    cap = logical.shape[0]
    for i in range((cap + page - 1) // page):
        lo = i * page
        hi = min(cap, lo + page)
        pages_arr[table_row[i], : hi - lo] = logical[lo:hi]


def draft_inputs(seed, lens, *, H_I=64, D_I=128, H_q=64, H_kv=64, D_qk=128,
                 D_v=128, k=2048, G=7, R=1, page=64, shuffle_pages=False,
                 integer_indexer=False, latent=False, poison=False, spare_page0=False):
    """Synthetic draft-block inputs.

    Each sequence b holds L_b = lens[b] target-written positions plus G
    draft-written slots after them (capacity L_b + G).  With poison=True the
    draft-written slots and every unused page row hold bf16 NaN, so any read of
    them shows up in the outputs.  spare_page0=True adds a physical page 0
    that no sequence owns (NaN when poisoned, else zeros): the cache's very
    first row is then never a target-written row.

    integer_indexer: indexer q and keys are integers uniform in [-4, 4] and w
    is m/64 with m uniform in {0..63} (exact in fp32 under any summation
    order); otherwise q, keys ~ N(0, 1) rounded to bf16 and w ~ U(0, 1).
    Attention q, K, V ~ N(0, 1) rounded to bf16.  latent=True stores one
    shared KV row of D_qk dims per position (H_kv = 1); V is its first D_v dims.
    row_len[b, r] = L_b for every row r (all rows see the target-written prefix).
    """
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    B = len(lens)
    caps = [int(L) + G for L in lens]
    if latent:
        H_kv = 1
    table, total_pages = _page_table(rng, caps, page, shuffle_pages, spare_page0)

    # indexer queries and weights
    if integer_indexer:
        qI = rng.integers(-4, 5, size=(B, R, H_I, D_I)).astype(np.float32)
        w = (rng.integers(0, 64, size=(B, R, H_I)) / 64.0).astype(np.float32)
    else:
        qI = rng.standard_normal((B, R, H_I, D_I), dtype=np.float32)
        w = rng.random((B, R, H_I), dtype=np.float32)
    qI_bits = bf16_bits(qI)

    kidx_bits = np.full((total_pages, page, D_I), BF16_NAN if poison else 0, np.uint16)
    if latent:
        k_bits = np.full((total_pages, page, D_qk), BF16_NAN if poison else 0, np.uint16)
        v_bits = None
    else:
        k_bits = np.full((total_pages, page, H_kv, D_qk), BF16_NAN if poison else 0, np.uint16)
        v_bits = np.full((total_pages, page, H_kv, D_v), BF16_NAN if poison else 0, np.uint16)

    keys, Ks, Vs = [], [], []
    for b in range(B):
        L, cap = int(lens[b]), caps[b]
        if integer_indexer:
            kk = rng.integers(-4, 5, size=(cap, D_I)).astype(np.float32)
        else:
            kk = rng.standard_normal((cap, D_I), dtype=np.float32)
        kb = bf16_bits(kk)
        if latent:
            kv = bf16_bits(rng.standard_normal((cap, D_qk), dtype=np.float32))
            vv = None
        else:
            kv = bf16_bits(rng.standard_normal((cap, H_kv, D_qk), dtype=np.float32))
            vv = bf16_bits(rng.standard_normal((cap, H_kv, D_v), dtype=np.float32))
        if poison:
            kb[L:] = BF16_NAN
            kv[L:] = BF16_NAN
            if vv is not None:
                vv[L:] = BF16_NAN
        _scatter_pages(kb, table[b], kidx_bits, page)
        _scatter_pages(kv, table[b], k_bits, page)
        if vv is not None:
            _scatter_pages(vv, table[b], v_bits, page)
        keys.append(bf16_value(kb))
        if latent:
            kf = bf16_value(kv)
            Ks.append(kf[:, None, :])
            Vs.append(kf[:, None, :D_v])
        else:
            Ks.append(bf16_value(kv))
            Vs.append(bf16_value(vv))

    q_bits = bf16_bits(rng.standard_normal((G, B, H_q, D_qk), dtype=np.float32))
    row_len = np.repeat(lens.astype(np.int32)[:, None], R, axis=1)
    return DraftInputs(
        lens=lens, R=R, G=G, H_I=H_I, D_I=D_I, H_q=H_q, H_kv=H_kv, D_qk=D_qk,
        D_v=D_v, k=k, page=page, latent=latent,
        q_index_bits=qI_bits, q_index=bf16_value(qI_bits), w=w,
        kidx_bits=kidx_bits, block_table=table, row_len=row_len,
        q_bits=q_bits, q=bf16_value(q_bits), k_bits=k_bits, v_bits=v_bits,
        keys=keys, K=Ks, V=Vs)


# ----------------------------------------------------------------------------
# Verification inputs
# ----------------------------------------------------------------------------
@dataclass
class VerifyInputs:
    target_logits: np.ndarray   # [B, G+1, V] f32
    draft_logits: np.ndarray    # [B, G, V] f32
    drafts: np.ndarray          # [B, G] i32
    seed: int
    offset: int

    @property
    def shape(self):
        B, G, V = self.draft_logits.shape
        return B, G, V


def gumbel_draw(rng, logits):
    """One draw from softmax(logits) by the Gumbel-max construction
    (argmax of logits plus independent standard Gumbel noise)."""
    g = -np.log(-np.log(rng.random(logits.shape[-1])))
    return int(np.argmax(np.asarray(logits, np.float64) + g))


def verify_inputs(seed, B, G, V, logit_std, *, independent=False, noise_std=1.0,
                  philox_seed=None, offset=0):
    """Target and draft logits with drafts sampled from the draft distribution.

    independent=True: target and draft logits are independent N(0, std^2)
    (the tiny configuration); otherwise draft = target + N(0, noise_std^2).
    """
    rng = np.random.default_rng(seed)
    tl = (rng.standard_normal((B, G + 1, V), dtype=np.float32) * np.float32(logit_std))
    if independent:
        dl = rng.standard_normal((B, G, V), dtype=np.float32) * np.float32(logit_std)
    else:
        dl = tl[:, :G] + rng.standard_normal((B, G, V), dtype=np.float32) * np.float32(noise_std)
    dl = dl.astype(np.float32)
    drafts = np.zeros((B, G), np.int32)
    for b in range(B):
        for j in range(G):
            drafts[b, j] = gumbel_draw(rng, dl[b, j])
    return VerifyInputs(tl, dl, drafts, seed if philox_seed is None else philox_seed, offset)


# ----------------------------------------------------------------------------
# Named workloads (shapes from the problem statement)
# ----------------------------------------------------------------------------
WORKLOADS = {
    "tiny": dict(lens=[512], H_I=4, D_I=32, H_q=4, H_kv=4, D_qk=64, D_v=64,
                 k=64, G=7, vocab=1024, logit_std=2.0, seed=0),
    "decode_32k": dict(lens=[32768], H_I=64, D_I=128, H_q=64, H_kv=64, D_qk=128,
                       D_v=128, k=2048, G=7, vocab=151552, seed=1),
    "batched_16x16k_64k": dict(B=16, len_range=(16384, 65536), H_I=64, D_I=128,
                               H_q=64, H_kv=64, D_qk=128, D_v=128, k=2048, G=7,
                               page=64, shuffle_pages=True, seed=2),
    "long_1m_latent": dict(lens=[1 << 20], H_I=64, D_I=128, H_q=64, D_qk=576,
                           D_v=512, k=2048, G=7, latent=True, seed=3),
    "verify_256x8x151552": dict(B=256, G=7, vocab=151552, logit_stds=(0.5, 2.0, 6.0),
                                seeds=(4, 5, 6)),
}


def batched_lens(seed, B=16, lo=16384, hi=65536):
    """Context lengths uniform over the integers [lo, hi]."""
    return np.random.default_rng(seed + 1000).integers(lo, hi + 1, size=B)
