"""Pure-Python brute-force MLA attention for tiny inputs (oracle; test infrastructure only).

A second, independent statement of the same definition as :mod:`oracle.mla`
(see that module for the readings of the pages), written with explicit loops,
its own bit decoding and ``math.fsum`` so that no BLAS call, array broadcast
or shared helper stands between it and the definition:

  token j of sequence b sees positions t = 0 .. seq_len - Q + j
  latent_t = kv[page_table[b][t // 16]][t % 16]        (576 values)
  s_t  = softmax_scale * sum_d q[b][j][h][d] * latent_t[d]
  lse  = log(sum_t exp(s_t))
  o[c] = sum_t exp(s_t - lse) * latent_t[c],   c < 512

Used on B <= 2, Q <= 3, H <= 4, seq_len <= ~40 to pin the NumPy oracle.
"""

import math
import struct


def _bf16(bits):
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def _e4m3fn(code):
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 15 and man == 7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def brute_force_mla(q_bits, kv_raw, page_table, seq_lens, softmax_scale,
                    kv_dtype="bf16", kv_scale=1.0):
    """Nested lists in, nested lists out: (out[B][Q][H][512], lse[B][Q][H])."""
    scale = float(struct.unpack("<f", struct.pack("<f", float(softmax_scale)))[0])
    kvs = float(struct.unpack("<f", struct.pack("<f", float(kv_scale)))[0])
    bsz = len(q_bits)
    out, lse = [], []
    for b in range(bsz):
        nq = len(q_bits[b])
        L = int(seq_lens[b])
        ob, lb = [], []
        for j in range(nq):
            n_vis = L - nq + j + 1
            latents = []
            for t in range(n_vis):
                blk = int(page_table[b][t // 16])
                raw = kv_raw[blk][t % 16]
                if kv_dtype == "bf16":
                    latents.append([_bf16(v) for v in raw])
                else:
                    latents.append([_e4m3fn(v) * kvs for v in raw])
            oj, lj = [], []
            for h in range(len(q_bits[b][j])):
                q = [_bf16(v) for v in q_bits[b][j][h]]
                scores = [scale * math.fsum(q[d] * lat[d] for d in range(576)) for lat in latents]
                if not scores:
                    oj.append([0.0] * 512)
                    lj.append(-math.inf)
                    continue
                m = max(scores)
                total = math.fsum(math.exp(s - m) for s in scores)
                l_row = m + math.log(total)
                w = [math.exp(s - l_row) for s in scores]
                oj.append([math.fsum(w[t] * latents[t][c] for t in range(len(latents)))
                           for c in range(512)])
                lj.append(l_row)
            ob.append(oj)
            lb.append(lj)
        out.append(ob)
        lse.append(lb)
    return out, lse
