"""NumPy float64 MLA decode / verify reference (oracle; test infrastructure only).

What is computed, and where it comes from
-----------------------------------------
* Each cached position holds one 576-wide compressed latent, shared by every
  query head of the rank; tensor parallelism splits heads, never the cache
  ("Inside Kimi K3 optimization", section "1. Cache -- DCP").
* The pages never write the attention formula out.  Reading taken (the
  absorbed / MQA form of MLA): every query head dots its 576-wide query with
  the whole 576-wide latent, and the value vector is the first 512 dims of the
  same latent.  The output stays in latent space.
* Positions live in pages of 16 latents addressed through a page table
  ("Kimi K2.6 + DFlash on 8x MI300X", section "Technical numbers": block size
  16 is mandatory for MLA).
* Speculative verify attends Q query tokens per sequence at once ("Inside
  Kimi K3 optimization", section "1. Cache -- DCP": the AITER DCP path was
  extended to multi-token verify).  Reading taken for the causal rule:
  seq_len counts every cached position including the Q new tokens, and query
  token j (0-based) sees positions 0 .. seq_len - Q + j.  Q = 1 is plain
  decode.
* Partial answers carry their normaliser so that shards can be merged with
  the right weights ("Inside Kimi K3 optimization", sections "1. Cache -- DCP"
  and "4. MLA": the history is cut into pieces processed in parallel and the
  pieces are combined).  The normaliser is the natural-log log-sum-exp of the
  scaled scores; a partial's output is normalised by its own sum.
* Padding 12 query heads to 16 leaves the real heads' softmax unchanged
  ("Inside Kimi K3 optimization", section "4. MLA"; "Kimi K3 on AMD MI355X",
  section "What had to be fixed").  The oracle never pads: heads are
  independent, so the unpadded definition is the reference.

Everything is float64, evaluated on the exact stored inputs (bf16 query bits,
bf16 or FP8 KV bytes times the float32 kv_scale, float32 softmax_scale).
Matrix products use numpy (BLAS) as a library step; there is no blocking or
reordering beyond the definition.
"""

import numpy as np

from .formats import bf16_bits_to_f64, decode_kv

LATENT_DIM = 576  # width of one cached latent (512 latent + 64 rope dims)
VALUE_DIM = 512   # the value vector is the first 512 dims of the latent
PAGE = 16         # positions per KV page


def gather_sequence(kv_raw, page_table_row, seq_len, kv_dtype, kv_scale=1.0):
    """Latents of one sequence, in position order: float64 [seq_len, 576].

    Position t lives in page page_table_row[t // 16], slot t % 16.  Only the
    first ceil(seq_len / 16) page-table entries are read, and slots at or past
    seq_len in the last page are dropped.
    """
    n_pages = -(-int(seq_len) // PAGE)
    if n_pages == 0:
        return np.zeros((0, LATENT_DIM), dtype=np.float64)
    blocks = np.asarray(page_table_row[:n_pages], dtype=np.int64)
    raw = np.asarray(kv_raw)[blocks]                      # [n_pages, 16, 576]
    x = decode_kv(raw, kv_dtype, kv_scale).reshape(n_pages * PAGE, LATENT_DIM)
    return x[: int(seq_len)]


def attend(q_rows, latents, softmax_scale):
    """Softmax attention of R query rows over n latents, float64.

    q_rows  : [R, 576];  latents: [n, 576]
    returns : o [R, 512], lse [R]
      s_t = softmax_scale * <q, latent_t>
      lse = log(sum_t exp(s_t))            (computed max-shifted)
      o   = sum_t exp(s_t - lse) * latent_t[:512]
    n = 0 gives o = 0 and lse = -inf.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    latents = np.asarray(latents, dtype=np.float64)
    r = q_rows.shape[0]
    if latents.shape[0] == 0:
        return np.zeros((r, VALUE_DIM)), np.full(r, -np.inf)
    s = np.float64(softmax_scale) * (q_rows @ latents.T)       # [R, n]
    m = s.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    p = np.exp(s - lse[:, None])
    o = p @ latents[:, :VALUE_DIM]
    return o, lse


def _visible(seq_len, num_q, j):
    """Number of positions query token j may see (causal verify rule).

    The rule needs seq_len >= num_q (the Q new tokens are part of the
    sequence); a shorter sequence is rejected here rather than given a
    negative count, which a slice x[:n] would silently wrap around."""
    if int(seq_len) < int(num_q):
        raise ValueError(f"seq_len {int(seq_len)} < num_q {int(num_q)}: outside the causal rule")
    return int(seq_len) - int(num_q) + int(j) + 1


def mla_reference(q_bits, kv_raw, page_table, seq_lens, softmax_scale,
                  kv_dtype="bf16", kv_scale=1.0, batch_indices=None):
    """Unsplit MLA decode (Q = 1) / verify (Q > 1).

    q_bits     : uint16 bf16 bits [B, Q, H, 576]
    kv_raw     : [num_blocks, 16, 576] uint16 bf16 bits or uint8 FP8 codes
    page_table : int [B, max_blocks_per_seq]
    seq_lens   : int [B], each >= Q
    batch_indices : optional subset of sequences to evaluate (others are NaN)

    returns out float64 [B, Q, H, 512], lse float64 [B, Q, H]
    """
    q = bf16_bits_to_f64(q_bits)
    bsz, nq, nh, _ = q.shape
    out = np.full((bsz, nq, nh, VALUE_DIM), np.nan)
    lse = np.full((bsz, nq, nh), np.nan)
    idx = range(bsz) if batch_indices is None else batch_indices
    for b in idx:
        x = gather_sequence(kv_raw, page_table[b], seq_lens[b], kv_dtype, kv_scale)
        for j in range(nq):
            n = _visible(seq_lens[b], nq, j)
            out[b, j], lse[b, j] = attend(q[b, j], x[:n], softmax_scale)
    return out, lse


def mla_partials(q_bits, kv_raw, page_table, seq_lens, softmax_scale, ranges,
                 kv_dtype="bf16", kv_scale=1.0, batch_indices=None):
    """Partial attention over position ranges, each with its normaliser.

    ranges[b] is a list of S half-open position ranges (lo, hi) for sequence b
    (the same S for every sequence).  Partial s of token j covers positions in
    [lo, hi) that token j may see.  An empty partial has o = 0, lse = -inf.

    returns part_out float64 [S, B, Q, H, 512], part_lse float64 [S, B, Q, H]
    """
    q = bf16_bits_to_f64(q_bits)
    bsz, nq, nh, _ = q.shape
    ns = len(ranges[0] if batch_indices is None else ranges[batch_indices[0]])
    part_out = np.full((ns, bsz, nq, nh, VALUE_DIM), np.nan)
    part_lse = np.full((ns, bsz, nq, nh), np.nan)
    idx = range(bsz) if batch_indices is None else batch_indices
    for b in idx:
        x = gather_sequence(kv_raw, page_table[b], seq_lens[b], kv_dtype, kv_scale)
        assert len(ranges[b]) == ns
        for s, (lo, hi) in enumerate(ranges[b]):
            for j in range(nq):
                n = _visible(seq_lens[b], nq, j)
                a, e = int(lo), min(int(hi), n)
                part_out[s, b, j], part_lse[s, b, j] = attend(
                    q[b, j], x[a:max(a, e)], softmax_scale)
    return part_out, part_lse


def merge(part_out, part_lse):
    """Combine S partials (axis 0) by their log-sum-exp normalisers.

      lse = log(sum_s exp(lse_s))            (max-shifted; -inf partials weigh 0)
      out = sum_s exp(lse_s - lse) * o_s
    If every partial is empty: out = 0, lse = -inf.
    """
    part_out = np.asarray(part_out, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    m = part_lse.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(part_lse), np.exp(part_lse - m_safe), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    coef = np.where(finite, w / np.where(finite, tot, 1.0), 0.0)
    out = (coef[..., None] * part_out).sum(axis=0)
    return out, lse


__all__ = ["gather_sequence", "attend", "mla_reference", "mla_partials", "merge",
           "LATENT_DIM", "VALUE_DIM", "PAGE"]
