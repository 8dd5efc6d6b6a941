"""Seeded synthetic MLA workloads.

Shapes and distributions follow the workloads of the pages: 12 query heads
per tensor-parallel rank (96 MLA heads under TP8), 576-wide latents stored in
pages of 16 positions, 1 or 3 query tokens per sequence (speculative verify
with st = 2 drafts), bf16 or FP8 E4M3 latents with one per-tensor float32
scale, and a long-context case of 24 MLA layers x 142,000 positions
("Inside Kimi K3 optimization", sections "1. Cache -- DCP" and "4. MLA";
"Kimi K2.6 + DFlash on 8x MI300X", sections "Technical numbers" and
"st=2 vs st=8 & FP8 vs BF16").

Conventions
-----------
* ``N(0, s)``: normal with standard deviation s.
* ``uniform in [a, b]``: integers a..b inclusive, one draw per sequence.
* Seeds: ``numpy.random.SeedSequence(seed).spawn(4)`` gives the streams for
  seq_lens, page table, q and KV (in that order).  The long-context config
  draws page table, q and KV per layer from ``SeedSequence([seed, layer])``.
* Page table: the pool has exactly sum_b ceil(L_b / 16) used blocks (plus
  optional poisoned spare blocks); block ids are a seeded permutation of the
  used blocks, sliced per sequence in order; unused entries are -1.
* FP8: x ~ N(0, 0.5) in float32; kv_scale = float32(max|x| / 448); codes =
  E4M3FN round-to-nearest-even of x / kv_scale, clamped to +-448 (the
  per-tensor "auto-computed" scale).
* Random draws for q and KV use a torch generator on the target device, so
  the same seed gives different (but fixed) values on CPU and GPU; every
  consumer reads the same tensors.
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch

LATENT_DIM = 576
VALUE_DIM = 512
PAGE = 16
SOFTMAX_SCALE = float(np.float32(1.0 / math.sqrt(192.0)))

# name -> workload description
CONFIGS = {
    "c1": dict(seed=1, batch=1, num_q=1, heads=12, kv_dtype="bf16", seq_lo=256, seq_hi=256,
               identity_pages=True,
               desc="tiny decode: B=1, Q=1, H=12, L=256, bf16, identity page table"),
    "c2": dict(seed=2, batch=32, num_q=1, heads=12, kv_dtype="bf16", seq_lo=1024, seq_hi=8192,
               desc="batched decode: B=32, Q=1, H=12, L~U[1024,8192], bf16"),
    "c3": dict(seed=3, batch=32, num_q=3, heads=12, kv_dtype="bf16", seq_lo=4096, seq_hi=32768,
               desc="speculative verify st=2: B=32, Q=3 causal, H=12, L~U[4096,32768], bf16"),
    "c4": dict(seed=4, batch=64, num_q=3, heads=12, kv_dtype="fp8", seq_lo=8192, seq_hi=65536,
               desc="FP8 KV verify: B=64, Q=3 causal, H=12, L~U[8192,65536], fp8 e4m3 + scale"),
    "c5": dict(seed=5, batch=4, num_q=3, heads=12, kv_dtype="fp8", seq_lo=35500, seq_hi=35500,
               layers=24, chunks=8,
               desc="long-context decode: 24 layers x 142,000 fp8 positions (4 x 35,500), "
                    "Q=3, H=12, 8 KV chunks per sequence + LSE merge"),
    "c5b": dict(seed=5, batch=4, num_q=3, heads=12, kv_dtype="fp8", seq_lo=142000, seq_hi=142000,
                layers=24, chunks=8,
                desc="long-context, alternative reading: 24 layers x 4 x 142,000 fp8 positions"),
    # one GPU's share under DCP8: all 96 heads (query all-gathered) over an eighth
    # of the c4 positions of each sequence
    "c6": dict(seed=6, batch=64, num_q=3, heads=96, kv_dtype="fp8", seq_lo=1024, seq_hi=8192,
               desc="DCP8-shaped FP8 verify: B=64, Q=3 causal, H=96, L~U[1024,8192] "
                    "(an eighth of the B=64 FP8 workload's history), fp8 e4m3 + scale"),
}


@dataclass
class MLAInputs:
    q: torch.Tensor            # bf16 [B, Q, H, 576]
    kv: torch.Tensor           # bf16 [NB, 16, 576] or uint8 (FP8 E4M3FN codes) [NB, 16, 576]
    page_table: torch.Tensor   # int32 [B, max_blocks_per_seq]
    seq_lens: torch.Tensor     # int32 [B]
    kv_dtype: str              # "bf16" | "fp8"
    kv_scale: float            # float32 value; 1.0 for bf16
    softmax_scale: float       # float32 value
    meta: dict = field(default_factory=dict)

    @property
    def batch(self):
        return int(self.q.shape[0])

    @property
    def num_q(self):
        return int(self.q.shape[1])

    @property
    def heads(self):
        return int(self.q.shape[2])

    @property
    def num_blocks(self):
        return int(self.kv.shape[0])

    @property
    def max_blocks_per_seq(self):
        return int(self.page_table.shape[1])


def _torch_gen(seedseq, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seedseq.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1)))
    return g


def _page_table(seq_lens, rng, max_blocks, identity):
    pages = [-(-int(L) // PAGE) for L in seq_lens]
    used = int(sum(pages))
    ids = np.arange(used) if identity else rng.permutation(used)
    pt = np.full((len(seq_lens), max_blocks), -1, dtype=np.int32)
    off = 0
    for b, p in enumerate(pages):
        pt[b, :p] = ids[off:off + p]
        off += p
    return pt, used


def _draw_kv(num_blocks, kv_dtype, gen, device, std=0.5):
    x = torch.randn((num_blocks, PAGE, LATENT_DIM), generator=gen, device=device,
                    dtype=torch.float32) * std
    if kv_dtype == "bf16":
        return x.to(torch.bfloat16), 1.0
    amax = float(x.abs().max().item())
    scale = float(np.float32(amax / 448.0)) if amax > 0 else 1.0
    codes = (x / scale).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


def make_inputs(seq_lens, num_q, heads, kv_dtype, seed, device="cpu", identity_pages=False,
                max_blocks_per_seq=None, spare_blocks=0, poison=False, q_std=1.0, kv_std=0.5,
                seed_streams=None):
    """Build one batch.

    seq_lens : iterable of ints (each >= num_q)
    spare_blocks : extra pool blocks never referenced by the page table
    poison   : fill spare blocks and the slots past L in each last page with
               NaN codes, so that a kernel reading them would be visible
    """
    seq_lens = np.asarray(list(seq_lens), dtype=np.int64)
    if seed_streams is None:
        _, s_pt, s_q, s_kv = np.random.SeedSequence(seed).spawn(4)
    else:
        s_pt, s_q, s_kv = seed_streams
    bsz = len(seq_lens)
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(1, int(max(-(-int(L) // PAGE) for L in seq_lens)))
    pt, used = _page_table(seq_lens, np.random.default_rng(s_pt), max_blocks_per_seq,
                           identity_pages)
    nb = used + int(spare_blocks)
    kv, kv_scale = _draw_kv(max(nb, 1), kv_dtype, _torch_gen(s_kv, device), device, kv_std)
    q = (torch.randn((bsz, num_q, heads, LATENT_DIM), generator=_torch_gen(s_q, device),
                     device=device, dtype=torch.float32) * q_std).to(torch.bfloat16)
    if poison:
        raw = kv.view(torch.int16) if kv_dtype == "bf16" else kv
        nan_code = 0x7FC0 if kv_dtype == "bf16" else 0x7F
        if spare_blocks:
            raw[used:] = nan_code
        for b, L in enumerate(seq_lens):
            p = -(-int(L) // PAGE)
            tail = int(L) - (p - 1) * PAGE
            if p > 0 and tail < PAGE:
                raw[int(pt[b, p - 1]), tail:] = nan_code
    return MLAInputs(q=q, kv=kv, page_table=torch.from_numpy(pt).to(device),
                     seq_lens=torch.from_numpy(seq_lens.astype(np.int32)).to(device),
                     kv_dtype=kv_dtype, kv_scale=kv_scale, softmax_scale=SOFTMAX_SCALE,
                     meta=dict(used_blocks=used))


def make_config(name, device="cpu"):
    """Inputs of a named single-layer config (c1..c4)."""
    c = CONFIGS[name]
    ss_len, s_pt, s_q, s_kv = np.random.SeedSequence(c["seed"]).spawn(4)
    rng = np.random.default_rng(ss_len)
    lens = rng.integers(c["seq_lo"], c["seq_hi"] + 1, size=c["batch"])
    mb = -(-c["seq_hi"] // PAGE)
    inp = make_inputs(lens, c["num_q"], c["heads"], c["kv_dtype"], None, device=device,
                      identity_pages=c.get("identity_pages", False), max_blocks_per_seq=mb,
                      seed_streams=(s_pt, s_q, s_kv))
    inp.meta["config"] = name
    return inp


def make_c5_layer(layer, device="cpu", name="c5"):
    """One layer cache of the long-context config (own page table, q, KV, scale)."""
    c = CONFIGS[name]
    s_pt, s_q, s_kv = np.random.SeedSequence([c["seed"], int(layer)]).spawn(3)
    lens = np.full(c["batch"], c["seq_lo"], dtype=np.int64)
    inp = make_inputs(lens, c["num_q"], c["heads"], c["kv_dtype"], None, device=device,
                      max_blocks_per_seq=-(-c["seq_hi"] // PAGE), seed_streams=(s_pt, s_q, s_kv))
    inp.meta["config"] = name
    inp.meta["layer"] = int(layer)
    return inp


def compact_for_oracle(inp, batch_indices=None):
    """Host (numpy) copies for the oracle, restricted to some sequences.

    Only the blocks those sequences reference are copied; the page table is
    renumbered accordingly.  Returns dict(q_bits, kv_raw, page_table,
    seq_lens, kv_dtype, kv_scale, softmax_scale, batch_indices).
    """
    bsz = inp.batch
    idx = list(range(bsz)) if batch_indices is None else [int(b) for b in batch_indices]
    lens = inp.seq_lens.cpu().numpy().astype(np.int64)
    pt = inp.page_table.cpu().numpy()
    blocks = []
    for b in idx:
        blocks.extend(int(x) for x in pt[b, : -(-int(lens[b]) // PAGE)])
    uniq = sorted(set(blocks))
    remap = {old: new for new, old in enumerate(uniq)}
    sel = torch.tensor(uniq if uniq else [0], dtype=torch.long, device=inp.kv.device)
    kv_sub = inp.kv.index_select(0, sel).cpu()
    kv_raw = (kv_sub.view(torch.int16).numpy().view(np.uint16) if inp.kv_dtype == "bf16"
              else kv_sub.numpy().astype(np.uint8))
    new_pt = np.full((len(idx), pt.shape[1]), -1, dtype=np.int64)
    for i, b in enumerate(idx):
        p = -(-int(lens[b]) // PAGE)
        new_pt[i, :p] = [remap[int(x)] for x in pt[b, :p]]
    q_bits = inp.q[idx].cpu().view(torch.int16).numpy().view(np.uint16)
    return dict(q_bits=q_bits, kv_raw=kv_raw, page_table=new_pt, seq_lens=lens[idx],
                kv_dtype=inp.kv_dtype, kv_scale=inp.kv_scale, softmax_scale=inp.softmax_scale,
                batch_indices=idx)


def algorithmic_bytes(seq_lens, num_q, heads, kv_dtype):
    """HBM bytes one layer-step must move at least: visible KV + q + out + lse + page ids."""
    kvb = 2 if kv_dtype == "bf16" else 1
    lens = np.asarray(seq_lens, dtype=np.int64)
    kv = int(lens.sum()) * LATENT_DIM * kvb
    rows = len(lens) * num_q * heads
    return kv + rows * (LATENT_DIM * 2 + VALUE_DIM * 2 + 4) + int((-(-lens // PAGE)).sum()) * 4


def algorithmic_flops(seq_lens, num_q, heads):
    """Useful multiply-add flops (2 per MAC) of QK^T over 576 dims and PV over 512 dims."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    return int(lens.sum()) * num_q * heads * 2 * (LATENT_DIM + VALUE_DIM)
