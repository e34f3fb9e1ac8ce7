"""Byte/FLOP ledger of the row operators (pure integer arithmetic).

Counting rule, from "TileLang tutorial, ch. 13: elementwise, normalisation and
RoPE operators", s1.1-s1.2: the bytes of one kernel are every tensor it reads
plus every tensor it writes, each at its own dtype; an intermediate tensor is
paid twice (its producer writes it, its consumer reads it); a fused kernel
reads its inputs once and writes its outputs once.  The result is a lower
bound on traffic, before cache misses, launch, tail and synchronisation.

Each scenario returns ``(unfused_bytes, fused_bytes, flops)``.  The step
lists of the unfused chains follow the pages where they name the steps
(RMSNorm's six calls pow -> mean -> add eps -> rsqrt -> mul -> mul weight,
s3.2.1; the RoPE reference's four products, one subtraction, one addition and
the concatenation, s3.3.2; "three operators written separately" for the fused
op, s3.3.4) and state a reading where the pages do not (LayerNorm's chain,
the scalar operand of scale+add).  Those readings are marked below.

``counted_bytes`` gives the algorithmic minimum of one launch of each
benchmark workload under the same rule (the fused column, with that
workload's own table dtype and layout).
"""
from __future__ import annotations

ELT = {"f16": 2, "bf16": 2, "f32": 4, "fp8": 1}


def _kernel(reads, writes):
    return sum(reads) + sum(writes)


def scale_add(N: int, elt: int = 4):
    """y = x * a + b with a scalar ``a`` and a tensor ``b`` (reading: the pages
    print 20N / 12N, which is what a scalar multiplier and a tensor addend give)."""
    t = N * elt
    unfused = _kernel([t], [t]) + _kernel([t, t], [t])  # mul, then add
    fused = _kernel([t, t], [t])
    return unfused, fused, 2 * N


def rmsnorm(rows: int, n: int, elt: int = 2, stat: int = 4):
    """RMSNorm as the six PyTorch calls; row statistics held in fp32 (``stat``)."""
    E = rows * n * elt
    r = rows * stat
    w = n * elt
    steps = [
        _kernel([E], [E]),          # pow: x -> x^2
        _kernel([E], [r]),          # mean over the row
        _kernel([r], [r]),          # + eps
        _kernel([r], [r]),          # rsqrt
        _kernel([E, r], [E]),       # x * rstd
        _kernel([E, w], [E]),       # * weight
    ]
    fused = _kernel([E, w], [E])
    return sum(steps), fused, 4 * rows * n


def rmsnorm_split(rows: int, n: int, elt: int = 2):
    """The split-K RMSNorm of s3.2.4: x is read twice (sum of squares, then the
    output pass), so the ledger counts one more read of x than the fused kernel."""
    E = rows * n * elt
    return rmsnorm(rows, n, elt)[0], _kernel([E, E, n * elt], [E]), 4 * rows * n


def layernorm(rows: int, n: int, elt: int = 2):
    """LayerNorm.  The pages give only the total (20E + O(rows)); the chain is a
    reading: sum(x), sum(x^2) (statistics stored at the tensor dtype), x - mu,
    * rstd, * gamma, + beta.  Only the printed total (two decimals) is pinned."""
    E = rows * n * elt
    r = rows * elt
    g = n * elt
    steps = [
        _kernel([E], [r]),          # sum(x) -> mu
        _kernel([E], [r]),          # sum(x^2)
        _kernel([E, r], [E]),       # x - mu
        _kernel([E, r], [E]),       # * rstd
        _kernel([E, g], [E]),       # * gamma
        _kernel([E, g], [E]),       # + beta
    ]
    fused = _kernel([E, g, g], [E])
    return sum(steps), fused, 8 * rows * n


def rope(rows: int, rope_dim: int, elt: int = 2, table_rows: int | None = None,
         cs_elt: int | None = None):
    """RoPE (NeoX reference) over ``rows`` rows of ``rope_dim`` channels.  The
    pages' ledger uses one cos/sin row per x row at x's dtype; pass
    ``table_rows``/``cs_elt`` for a per-token table of another dtype."""
    half = rows * (rope_dim // 2) * elt          # one half of x
    trows = rows if table_rows is None else table_rows
    ce = elt if cs_elt is None else cs_elt
    tab = trows * (rope_dim // 2) * ce            # one of cos / sin
    prod = _kernel([half, tab], [half])           # x_half * c  (or * s)
    comb = _kernel([half, half], [half])          # a - b  (or a + b)
    cat = _kernel([half, half], [2 * half])       # concatenate the halves
    unfused = 4 * prod + 2 * comb + cat
    fused = _kernel([2 * half, tab, tab], [2 * half])
    return unfused, fused, 3 * rows * rope_dim


def rmsnorm_rope_fp8(tokens: int, n: int, rope_dim: int, elt: int = 2, cs_elt: int = 2,
                     rope_per_row: int | None = None):
    """RMSNorm -> RoPE -> per-token FP8, as three separately fused kernels vs one.
    FLOPs: 7 per element (norm 4, quantise 3) plus 3 per rotated element; the
    pages' arithmetic-intensity maximum (2.315) is reproduced when the rotation
    covers ``rope_dim`` channels per row (``rope_per_row`` defaults to that)."""
    E = tokens * n * elt
    w = n * elt
    tab = tokens * (rope_dim // 2) * cs_elt
    codes = tokens * n
    scales = tokens * 4
    k_norm = _kernel([E, w], [E])
    k_rope = _kernel([E, tab, tab], [E])
    k_quant = _kernel([E], [codes, scales])
    fused = _kernel([E, w, tab, tab], [codes, scales])
    rot = rope_dim if rope_per_row is None else rope_per_row
    flops = 7 * tokens * n + 3 * tokens * rot
    return k_norm + k_rope + k_quant, fused, flops


def act_quant(rows: int, n: int, group: int, elt: int = 2):
    """Per-group FP8 cast as one kernel: read x, write codes and one fp32 scale
    per group.  FLOPs: |x|, max, scale multiply per element (3)."""
    E = rows * n * elt
    fused = _kernel([E], [rows * n, rows * (n // group) * 4])
    return fused, fused, 3 * rows * n


def qk_norm_rope(tokens: int, q_heads: int, kv_heads: int, head_dim: int, rope_dim: int,
                 elt: int = 2, cs_elt: int = 2):
    """Per-head QK RMSNorm + RoPE in place: q and k columns are read and written
    once, v is not touched; two weight vectors and the cos/sin tables are read.
    Unfused: a per-head RMSNorm kernel then a RoPE kernel on q and k.  FLOPs: 4 per
    q/k value for the weighted RMSNorm and 3 per rotated value (the TileOPs
    formula the page cites in s2.4)."""
    qk = tokens * (q_heads + kv_heads) * head_dim * elt
    w = 2 * head_dim * elt
    tab = tokens * (rope_dim // 2) * cs_elt
    fused = _kernel([qk, w, tab, tab], [qk])
    unfused = _kernel([qk, w], [qk]) + _kernel([qk, tab, tab], [qk])
    flops = 4 * tokens * (q_heads + kv_heads) * head_dim + 3 * tokens * (q_heads + kv_heads) * rope_dim
    return unfused, fused, flops


def qk_norm_rope_fp8_kv(tokens: int, q_heads: int, kv_heads: int, head_dim: int,
                        rope_dim: int, elt: int = 2, cs_elt: int = 2, slot_bytes: int = 8):
    """QK RMSNorm + RoPE with the FP8 KV-cache write, one kernel: the whole q/k/v
    row, the weights, the tables and one slot index per token are read; q is
    written back at its dtype, k and v as one-byte codes plus one fp32 scale per
    (token, kv head).  FLOPs: 7 per q/k value (as above) and 3 per quantised
    k/v value (|x|, max, scale)."""
    qkv = tokens * (q_heads + 2 * kv_heads) * head_dim * elt
    w = 2 * head_dim * elt
    tab = tokens * (rope_dim // 2) * cs_elt
    slots = tokens * slot_bytes
    q = tokens * q_heads * head_dim * elt
    codes = 2 * tokens * kv_heads * head_dim
    scales = 2 * tokens * kv_heads * 4
    fused = _kernel([qkv, w, tab, tab, slots], [q, codes, scales])
    flops = (4 * tokens * (q_heads + kv_heads) * head_dim
             + 3 * tokens * (q_heads + kv_heads) * rope_dim + 3 * codes)
    return fused, fused, flops


def elementwise(n: int, x_elt: int, y_elt: int, has_b: bool):
    """One elementwise kernel over n elements: x (and b, at x's dtype) read once,
    y written once.  FLOPs: one multiply (and one add) per element."""
    fused = _kernel([n * x_elt] + ([n * x_elt] if has_b else []), [n * y_elt])
    return fused, fused, (2 if has_b else 1) * n


def page_scenarios():
    """The five scenarios of the ledger table, with the pages' shapes."""
    return {
        "scale_add": scale_add(1 << 20, 4),
        "rmsnorm": rmsnorm(4096, 4096, 2),
        "layernorm": layernorm(4096, 4096, 2),
        "rope": rope(4096 * 32, 128, 2),
        "rmsnorm_rope_fp8": rmsnorm_rope_fp8(4096, 4096, 128, 2, 2),
    }


def counted_bytes(cfg: dict) -> int:
    """Algorithmic bytes of one launch of a workload (see ``synth.WORKLOADS``)."""
    op = cfg["op"]
    if op == "rmsnorm":
        if cfg.get("x_passes", 1) == 2:
            return rmsnorm_split(cfg["rows"], cfg["n"], ELT[cfg["dtype"]])[1]
        return rmsnorm(cfg["rows"], cfg["n"], ELT[cfg["dtype"]])[1]
    if op == "layernorm":
        return layernorm(cfg["rows"], cfg["n"], ELT[cfg["dtype"]])[1]
    if op == "rope":
        n = cfg["heads"] * cfg["head_dim"]
        e = ELT[cfg["dtype"]]
        T = cfg["tokens"]
        R = cfg["rope_dim"]
        xy = 2 * T * n * e
        tab = 2 * T * (R // 2) * ELT[cfg["cs_dtype"]]
        return xy + tab
    if op == "act_quant":
        return act_quant(cfg["rows"], cfg["n"], cfg.get("group") or cfg["n"],
                         ELT[cfg["dtype"]])[1]
    if op == "qk_norm_rope":
        return qk_norm_rope(cfg["tokens"], cfg["q_heads"], cfg["kv_heads"], cfg["head_dim"],
                            cfg["rope_dim"], ELT[cfg["dtype"]], ELT[cfg["cs_dtype"]])[1]
    if op == "ew":
        return elementwise(cfg["n"], ELT[cfg["dtype"]], ELT[cfg.get("y_dtype", cfg["dtype"])],
                           cfg["kind"] != "scale_cast")[1]
    if op == "qk_kv":
        return qk_norm_rope_fp8_kv(cfg["tokens"], cfg["q_heads"], cfg["kv_heads"],
                                   cfg["head_dim"], cfg["rope_dim"], ELT[cfg["dtype"]],
                                   ELT[cfg["cs_dtype"]])[1]
    if op == "fused":
        n = cfg["heads"] * cfg["head_dim"]
        return rmsnorm_rope_fp8(cfg["tokens"], n, cfg["rope_dim"], ELT[cfg["dtype"]],
                                ELT[cfg["cs_dtype"]])[1]
    raise ValueError(op)
