"""Brute-force attention in pure Python, for pinning the oracle on tiny inputs.

Independent of ``oracle/``: scalars and lists only, ``math.fsum`` for every
sum, and the shard of each token found by dealing the request's tokens to the
shards one interleave unit at a time (round-robin), rather than by a formula.
"""

import math


def bf16_to_float(bits):
    import struct
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def fp8_to_float(code):
    """Value of an fp8 E4M3 ("fn") code, by its fields: sign, a 4-bit
    exponent biased by 7 (0 = subnormal), 3 mantissa bits; S.1111.111 is NaN."""
    code = int(code) & 0xFF
    if code & 0x7F == 0x7F:
        return math.nan
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0:
        return sign * math.ldexp(m, -9)
    return sign * math.ldexp(8 + m, e - 10)


def deal_tokens(n, S, I):
    """Deal tokens 0..n-1 to S shards, I consecutive tokens at a time."""
    owner = []
    shard = 0
    while len(owner) < n:
        for _ in range(I):
            if len(owner) == n:
                break
            owner.append(shard)
        shard = (shard + 1) % S
    return owner


def softmax_state(q, keys, scale):
    """(out[512], lse) for one query vector over a list of 576-wide keys."""
    if not keys:
        return [0.0] * 512, -math.inf
    s = [scale * math.fsum(a * b for a, b in zip(q, k)) for k in keys]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = math.fsum(e)
    out = [math.fsum(e[i] * keys[i][d] for i in range(len(keys))) / z for d in range(512)]
    return out, m + math.log(z)


def brute_decode(q_bits, kv_bits, block_table, seq_lens, S, I, scale, causal, kv_scale=None):
    """Nested lists: out[b][r][h], lse[b][r][h], lse_shard[s][b][r][h], out_shard[s][b][r][h].
    With ``kv_scale``, kv_bits holds fp8 codes and row (block, slot) is scaled by kv_scale[block][slot]."""
    B, R, H = len(q_bits), len(q_bits[0]), len(q_bits[0][0])
    bs = len(kv_bits[0])
    out = [[[None] * H for _ in range(R)] for _ in range(B)]
    lse = [[[None] * H for _ in range(R)] for _ in range(B)]
    lse_sh = [[[[None] * H for _ in range(R)] for _ in range(B)] for _ in range(S)]
    out_sh = [[[[None] * H for _ in range(R)] for _ in range(B)] for _ in range(S)]
    for b in range(B):
        L = int(seq_lens[b])
        for r in range(R):
            n = L - (R - 1 - r) if causal else L
            n = max(n, 0)
            keys = []
            for t in range(n):
                blk = int(block_table[b][t // bs])
                if kv_scale is None:
                    keys.append([bf16_to_float(x) for x in kv_bits[blk][t % bs]])
                else:
                    f = float(kv_scale[blk][t % bs])
                    keys.append([fp8_to_float(x) * f for x in kv_bits[blk][t % bs]])
            owner = deal_tokens(n, S, I)
            for h in range(H):
                q = [bf16_to_float(x) for x in q_bits[b][r][h]]
                out[b][r][h], lse[b][r][h] = softmax_state(q, keys, scale)
                for s in range(S):
                    ks = [keys[t] for t in range(n) if owner[t] == s]
                    out_sh[s][b][r][h], lse_sh[s][b][r][h] = softmax_state(q, ks, scale)
    return out, lse, lse_sh, out_sh
