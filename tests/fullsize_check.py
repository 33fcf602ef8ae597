"""Row checks at full size against the plain definition (fp64 oracle).

At the full sizes the oracle's paged attention over a whole pool would hold
the pool in fp64 several times over, so these checks take each sequence's
logical K/V from the workload (what the pool must hold; the gather through
the tables equals it bit for bit, pinned in tests/test_oracle_attention.py)
and compute attention of the step's rows over it with
`oracle.attention.attention_rows`, one (sequence, KV head) at a time so the
widening to fp64 happens once for the G q heads that share it.
"""
import numpy as np

from oracle import attention as A
from oracle.storage import kv_encode, to_f64


def _kv_of_head(wl, K, V, g):
    sp = wl.spec
    Kg, Vg = K[:, g], V[:, g]
    if sp.kv is not None:  # FP8 pool: the codes of the logical values
        Kg, Vg = kv_encode(Kg, sp.dtype, sp.k_scale), kv_encode(Vg, sp.dtype, sp.v_scale)
    return Kg, Vg


def check_rows(wl, out, tol, rows_of=None, seqs=None):
    """Compare `out` ([sum n][Hq][D], storage representation, batch order)
    with the definition.  rows_of(r, p) -> the rows of batch entry r to
    check (default: every row); seqs: the batch entries to visit (default:
    all).  Every q head of each checked row is compared.  Returns
    (worst |err|, rows checked, |out| at the worst row)."""
    sp = wl.spec
    batch = wl.batch
    G = sp.num_q_heads // sp.num_kv_heads
    starts = np.concatenate([[0], np.cumsum([p.n_new for p in batch])])
    worst, where, count = 0.0, None, 0
    for r in (range(len(batch)) if seqs is None else seqs):
        p = batch[r]
        rows = list(range(p.n_new)) if rows_of is None else list(rows_of(r, p))
        if not rows:
            continue
        K, V = wl.logical_kv(p.seq_id)
        L = p.context_len
        for g in range(sp.num_kv_heads):
            Kg, Vg = _kv_of_head(wl, K, V, g)
            qr = np.concatenate([wl.q[p.seq_id][i, g * G:(g + 1) * G] for i in rows])  # [rows*G][D]
            pos = np.repeat([L - p.n_new + i for i in rows], G)
            ref = A.attention_rows(qr, Kg, Vg, pos, sp.scale, sp.dtype, sp.kv)
            got = to_f64(np.concatenate([out[starts[r] + i, g * G:(g + 1) * G] for i in rows]), sp.dtype)
            err = np.abs(got - ref).max(axis=1)
            j = int(np.argmax(err))
            if err[j] > worst:
                worst, where = float(err[j]), (r, rows[j // G], g * G + j % G, float(np.abs(ref[j]).max()))
            assert err[j] <= tol, (wl.spec.name, r, rows[j // G], g * G + j % G, float(err[j]))
            count += len(rows) * G
    return worst, count, where


def decode_rows(r, p):
    """Every row of a one-token sequence, none of a chunk."""
    return [0] if p.n_new == 1 else []


def chunk_edges(rng, extra=8):
    """First and last row of every chunk plus `extra` random rows of it."""
    def pick(r, p):
        if p.n_new == 1:
            return []
        rows = {0, p.n_new - 1}
        rows.update(int(x) for x in rng.integers(0, p.n_new, size=extra))
        return sorted(rows)
    return pick
