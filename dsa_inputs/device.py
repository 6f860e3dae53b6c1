"""Seeded synthetic inputs generated directly in device memory (torch).

Same recipes as dsa_inputs (draft_inputs / verify_inputs) at sizes too large
to draw on the host: normal draws are made in fp32 with a seeded
torch.Generator on the device and rounded to bf16.  Like dsa_inputs this
module holds none of the path's arithmetic.  The drafts are drawn from the
draft distribution by the Gumbel-max construction (argmax of logits plus
Gumbel noise), which needs no softmax.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch


@dataclass
class DeviceDraft:
    lens: list
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
    q_index: torch.Tensor      # bf16 [B, R, H_I, D_I]
    w: torch.Tensor            # fp32 [B, R, H_I]
    kidx: torch.Tensor         # bf16 [pages, page, D_I]
    block_table: torch.Tensor  # int32 [B, max_pages]
    row_len: torch.Tensor      # int32 [B, R]
    q: torch.Tensor            # bf16 [G, B, H_q, D_qk]
    k_cache: torch.Tensor      # bf16 [pages, page, H_kv, D_qk] or [pages, page, D_qk]
    v_cache: torch.Tensor      # bf16 [pages, page, H_kv, D_v] or the latent cache itself
    ld: int

    @property
    def B(self):
        return len(self.lens)

    @property
    def sm_scale(self):
        return 1.0 / float(np.sqrt(self.D_qk))


def _randn_bf16(shape, gen, dev, chunk=1 << 26):
    out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    flat = out.view(-1)
    for s in range(0, flat.numel(), chunk):
        e = min(flat.numel(), s + chunk)
        flat[s:e] = torch.randn(e - s, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    return out


def draft_inputs(seed, lens, *, H_I=64, D_I=128, H_q=64, H_kv=64, D_qk=128, D_v=128, k=2048, G=7,
                 R=1, page=64, shuffle_pages=False, latent=False, integer_indexer=False, spare_page0=False,
                 dev="cuda:0"):
    """Device draft-block inputs.  Capacity per sequence is L_b + G (the draft
    slots exist but are never scored or selected).  Page tables follow the
    same construction as dsa_inputs: one physical pool, optionally shuffled
    once (numpy, seeded); spare_page0 adds a physical page 0 that no sequence
    owns (see poison_)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in lens]
    B = len(lens)
    caps = [L + G for L in lens]
    n_pages = [(c + page - 1) // page for c in caps]
    total = int(sum(n_pages))
    phys = rng.permutation(total) if shuffle_pages else np.arange(total)
    if spare_page0:
        phys = phys + 1
        total += 1
    table = np.full((B, max(n_pages)), -1, np.int32)
    pos = 0
    for b, n in enumerate(n_pages):
        table[b, :n] = phys[pos:pos + n]
        pos += n
    if latent:
        H_kv = 1
    if integer_indexer:
        q_index = torch.randint(-4, 5, (B, R, H_I, D_I), generator=gen, device=dev).to(torch.bfloat16)
        w = (torch.randint(0, 64, (B, R, H_I), generator=gen, device=dev).float() / 64.0)
        kidx = torch.randint(-4, 5, (total, page, D_I), generator=gen, device=dev).to(torch.bfloat16)
    else:
        q_index = _randn_bf16((B, R, H_I, D_I), gen, dev)
        w = torch.rand((B, R, H_I), generator=gen, device=dev, dtype=torch.float32)
        kidx = _randn_bf16((total, page, D_I), gen, dev)
    q = _randn_bf16((G, B, H_q, D_qk), gen, dev)
    if latent:
        k_cache = _randn_bf16((total, page, D_qk), gen, dev)
        v_cache = k_cache
    else:
        k_cache = _randn_bf16((total, page, H_kv, D_qk), gen, dev)
        v_cache = _randn_bf16((total, page, H_kv, D_v), gen, dev)
    row_len = torch.tensor(lens, dtype=torch.int32, device=dev)[:, None].repeat(1, R).contiguous()
    return DeviceDraft(lens=lens, G=G, H_I=H_I, D_I=D_I, H_q=H_q, H_kv=H_kv, D_qk=D_qk, D_v=D_v, k=k,
                       page=page, latent=latent, q_index=q_index, w=w, kidx=kidx,
                       block_table=torch.from_numpy(table).to(dev), row_len=row_len, q=q,
                       k_cache=k_cache, v_cache=v_cache, ld=max(caps))


def poison_(d):
    """Writes bf16 NaN, in place, into every cache row that no target wrote:
    the G draft-written slots L_b..L_b+G-1 of each sequence, the unused rows
    of its last page, and every row of a page no sequence owns (physical page
    0 with spare_page0).  Index keys, K and V alike.  A read of any of them
    then shows up as NaN in the outputs."""
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16, device=d.k_cache.device)
    caches = [d.kidx, d.k_cache] + ([] if d.latent else [d.v_cache])
    bt = d.block_table.cpu().numpy()
    owned = np.zeros(d.kidx.shape[0], bool)
    pages, rows = [], []
    for b, L in enumerate(d.lens):
        n_pages = (L + d.G + d.page - 1) // d.page
        owned[bt[b, :n_pages]] = True
        t = np.arange(L, n_pages * d.page)            # draft slots, then the page's unused tail
        pages.append(bt[b, t // d.page])
        rows.append(t % d.page)
    pi = torch.as_tensor(np.concatenate(pages).astype(np.int64), device=d.k_cache.device)
    ri = torch.as_tensor(np.concatenate(rows).astype(np.int64), device=d.k_cache.device)
    spare = torch.as_tensor(np.flatnonzero(~owned).astype(np.int64), device=d.k_cache.device)
    for c in caches:
        c[pi, ri] = nan
        if spare.numel():
            c[spare] = nan


@dataclass
class DeviceVerify:
    target_logits: torch.Tensor   # fp32 [B, G+1, V]
    draft_logits: torch.Tensor    # fp32 [B, G, V]
    drafts: torch.Tensor          # int32 [B, G]
    seed: int
    offset: int


def verify_inputs(seed, B, G, V, logit_std, *, noise_std=1.0, independent=False, dev="cuda:0",
                  philox_seed=None, offset=0):
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    tl = torch.randn((B, G + 1, V), generator=gen, device=dev, dtype=torch.float32) * float(logit_std)
    if independent:
        dl = torch.randn((B, G, V), generator=gen, device=dev, dtype=torch.float32) * float(logit_std)
    else:
        dl = tl[:, :G] + torch.randn((B, G, V), generator=gen, device=dev, dtype=torch.float32) * float(noise_std)
    dl = dl.contiguous()
    drafts = torch.empty((B, G), dtype=torch.int32, device=dev)
    for j in range(G):
        u = torch.rand((B, V), generator=gen, device=dev, dtype=torch.float64).clamp_(min=1e-300)
        gum = -torch.log(-torch.log(u))
        drafts[:, j] = torch.argmax(dl[:, j].double() + gum, dim=-1).to(torch.int32)
    return DeviceVerify(tl, dl, drafts, int(seed if philox_seed is None else philox_seed), int(offset))
