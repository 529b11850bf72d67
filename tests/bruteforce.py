"""Pure-Python brute force for tiny MLA decode cases (test-only, independent of oracle/).

Written from the definition with nothing shared with the oracle: bf16 and
e4m3fn decoding through `struct` and bit arithmetic, a page-by-page walk of
the block table, softmax evaluated directly as exp(z) / sum exp(z) (no max
subtraction), sums with math.fsum. Use only where |z| is small.
"""
import math
import struct


def bf16_bits_to_float(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def e4m3fn_code_to_float(code: int) -> float:
    """OCP E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; S.1111.111 = NaN."""
    code = int(code) & 0xFF
    sign = -1.0 if code >> 7 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * math.ldexp(man, -9)          # (man / 8) * 2^-6
    return sign * math.ldexp(8 + man, exp - 10)     # (1 + man / 8) * 2^(exp - 7)


def fp8_record_to_floats(rec: bytes) -> list:
    assert len(rec) == 656
    scales = struct.unpack("<4f", rec[512:528])
    latent = [e4m3fn_code_to_float(rec[j]) * scales[j // 128] for j in range(512)]
    rope = [bf16_bits_to_float(v) for v in struct.unpack("<64H", rec[528:656])]
    return latent + rope


def brute_force_decode(q_bits, kv, kv_format, block_table, seqlens, *, dv=512, causal=False, scale=None,
                       vcache=None):
    """q_bits: nested lists / array [B][S][H][576] of bf16 bit patterns.
    kv: array [P][64][Hk][576] bf16 bits, or [P][64][Hk][656] uint8 records.
    vcache (optional): array [P][64][Hk][dv] bf16 bits; V of token t is its row there
    (same page and slot as its key) instead of the key's first dv dims.
    Returns (O [B][S][H][dv] lists, LSE [B][H][S] lists)."""
    B, S, H = len(q_bits), len(q_bits[0]), len(q_bits[0][0])
    Hk = len(kv[0][0])
    G = H // Hk
    if scale is None:
        scale = 1.0 / math.sqrt(576.0)

    def row(page, slot, kvh):
        raw = kv[page][slot][kvh]
        if kv_format == "bf16":
            return [bf16_bits_to_float(x) for x in raw]
        return fp8_record_to_floats(bytes(int(x) for x in raw))

    O = [[[None] * H for _ in range(S)] for _ in range(B)]
    LSE = [[[None] * S for _ in range(H)] for _ in range(B)]
    for b in range(B):
        L = int(seqlens[b])
        for kvh in range(Hk):
            keys = []                      # token order, walking the block table page by page
            vals = []
            for i, page in enumerate(block_table[b]):
                for slot in range(64):
                    t = i * 64 + slot
                    if t >= L:
                        break
                    keys.append(row(int(page), slot, kvh))
                    if vcache is not None:
                        vals.append([bf16_bits_to_float(x) for x in vcache[int(page)][slot][kvh]])
                if (i + 1) * 64 >= L:
                    break
            if vcache is None:
                vals = [k[:dv] for k in keys]
            for s in range(S):
                for g in range(G):
                    h = kvh * G + g
                    q = [bf16_bits_to_float(x) for x in q_bits[b][s][h]]
                    allowed = [t for t in range(L) if (not causal) or t <= L - S + s]
                    if not allowed:
                        O[b][s][h] = [0.0] * dv
                        LSE[b][h][s] = -math.inf
                        continue
                    z = [scale * math.fsum(q[d] * keys[t][d] for d in range(576)) for t in allowed]
                    e = [math.exp(v) for v in z]
                    tot = math.fsum(e)
                    O[b][s][h] = [math.fsum(e[i] * vals[t][d] for i, t in enumerate(allowed)) / tot
                                  for d in range(dv)]
                    LSE[b][h][s] = math.log(tot)
    return O, LSE


def brute_force_sparse_decode(q_bits, kv, kv_format, block_table, seqlens, indices, *, dv=512, causal=False,
                              scale=None):
    """Token-level sparse decode by the definition: query token s of sequence b attends to the
    entries of indices[b][s] (a position t names token t of the sequence: page
    block_table[b][t // 64], slot t % 64; -1 names nothing; a repeated position counts again;
    with causal, positions past L_b - S + s are dropped)."""
    B, S, H = len(q_bits), len(q_bits[0]), len(q_bits[0][0])
    Hk = len(kv[0][0])
    G = H // Hk
    if scale is None:
        scale = 1.0 / math.sqrt(576.0)

    def row(page, slot, kvh):
        raw = kv[page][slot][kvh]
        if kv_format == "bf16":
            return [bf16_bits_to_float(x) for x in raw]
        return fp8_record_to_floats(bytes(int(x) for x in raw))

    O = [[[None] * H for _ in range(S)] for _ in range(B)]
    LSE = [[[None] * S for _ in range(H)] for _ in range(B)]
    for b in range(B):
        L = int(seqlens[b])
        for s in range(S):
            sel = [int(t) for t in indices[b][s] if int(t) != -1 and ((not causal) or int(t) <= L - S + s)]
            for kvh in range(Hk):
                keys = [row(int(block_table[b][t // 64]), t % 64, kvh) for t in sel]
                for g in range(G):
                    h = kvh * G + g
                    if not keys:
                        O[b][s][h] = [0.0] * dv
                        LSE[b][h][s] = -math.inf
                        continue
                    q = [bf16_bits_to_float(x) for x in q_bits[b][s][h]]
                    e = [math.exp(scale * math.fsum(q[d] * k[d] for d in range(576))) for k in keys]
                    tot = math.fsum(e)
                    O[b][s][h] = [math.fsum(e[i] * keys[i][d] for i in range(len(keys))) / tot for d in range(dv)]
                    LSE[b][h][s] = math.log(tot)
    return O, LSE


def brute_force_sparse_prefill(q_bits, kv_bits, indices, scale, *, dv=512):
    """Sparse prefill by the definition: query token s, head h attends to the rows
    indices[s][h // G] of kv (its KV head; -1 names nothing; repeats count again)."""
    Sq, H = len(q_bits), len(q_bits[0])
    Hk = len(kv_bits[0])
    G = H // Hk
    O = [[None] * H for _ in range(Sq)]
    LSE = [[None] * H for _ in range(Sq)]
    for s in range(Sq):
        for h in range(H):
            kvh = h // G
            keys = [[bf16_bits_to_float(x) for x in kv_bits[int(t)][kvh]] for t in indices[s][kvh] if int(t) != -1]
            if not keys:
                O[s][h] = [0.0] * dv
                LSE[s][h] = -math.inf
                continue
            q = [bf16_bits_to_float(x) for x in q_bits[s][h]]
            e = [math.exp(scale * math.fsum(q[d] * k[d] for d in range(576))) for k in keys]
            tot = math.fsum(e)
            O[s][h] = [math.fsum(e[i] * keys[i][d] for i in range(len(keys))) / tot for d in range(dv)]
            LSE[s][h] = math.log(tot)
    return O, LSE
