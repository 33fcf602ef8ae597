"""Reference paged attention in fp64.

The pages state the kernel reads a request's scattered blocks through its
block table and stitches them into the logically contiguous K/V sequence
(lshu.cn/news/11644, "方案：页式内存管理", paragraph after the append rule).
So this is the plain definition: gather through the table, then ordinary
scaled dot-product attention over the gathered sequence.

Readings where the pages are silent:
* q head h reads KV head h // (Hq // Hkv) (consecutive q heads share a KV head);
* context_lens include the tokens appended in this step (decode appends the
  current token, then attends: zzmblog.top vLLM guide,
  "Transformer推理与KV缓存");
* the n query rows of a sequence are its last n positions: row i sits at
  position L - n + i and sees keys 0..L - n + i (a chunk of a prompt whose
  earlier part is already cached; lshu.cn/news/11644, "整体架构" scheduler
  loop; 5x10.cn/post/462, "分块预填充"); decode is n = 1;
* a sequence with context length 0 yields zeros (no keys to attend).

`kv` = (kv_dtype, k_scale, v_scale) describes an FP8 pool (the values are
the codes times the scales, storage.kv_values); None: K/V share q's dtype.
"""
import numpy as np

from .storage import kv_values, to_f64


def kv_f64(k, v, dtype, kv=None):
    """Stored K and V -> fp64 values."""
    if kv is not None and kv[0] == "fp8":
        return kv_values(k, kv[1]), kv_values(v, kv[2])
    return to_f64(k, dtype), to_f64(v, dtype)


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    return h // (num_q_heads // num_kv_heads)


def query_positions(context_len: int, n: int):
    """Position of each of the n query rows: the last n of the context."""
    return context_len - n + np.arange(n)


def visible_keys(context_len: int, positions):
    """[n][L] mask: a row at position a sees keys 0..a (inclusive)."""
    return np.arange(context_len)[None, :] <= np.asarray(positions)[:, None]


def gather(pool_k, pool_v, table, context_len, dtype, kv=None):
    """K/V of one sequence in logical order: [L][Hkv][D] each, fp64."""
    bs = pool_k.shape[2]
    nb = pool_k.shape[0]
    j = np.arange(context_len)
    blk = np.asarray(table)[j // bs]
    assert np.all((blk >= 0) & (blk < nb)), "block id out of range"
    off = j % bs
    return kv_f64(pool_k[blk, :, off, :], pool_v[blk, :, off, :], dtype, kv)


def attend(qv, K, V, scale):
    """softmax(scale * K qv) weighted sum of V for one query row.

    Returns (out [D], lse, p [len])."""
    z = scale * (K @ qv)
    m = z.max()
    e = np.exp(z - m)
    l = e.sum()
    p = e / l
    return p @ V, m + np.log(l), p


def attention_rows(q_rows, K, V, positions, scale, dtype, kv=None):
    """Rows of one (sequence, q head) against that head's K/V in logical
    order (K, V [L][D] as stored): row i sees keys 0..positions[i].
    The same definition as `paged_attention`, for a few sampled rows of a
    long sequence.  Returns out [n][D] fp64."""
    q = to_f64(np.asarray(q_rows), dtype)
    Kf, Vf = kv_f64(np.asarray(K), np.asarray(V), dtype, kv)
    out = np.zeros((len(positions), Kf.shape[1]))
    for i, a in enumerate(positions):
        out[i], _, _ = attend(q[i], Kf[: int(a) + 1], Vf[: int(a) + 1], scale)
    return out


def paged_attention(q, pool_k, pool_v, tables, context_lens, q_lens, scale, dtype, kv=None):
    """q: [sum n][Hq][D] storage values, rows in sequence order.

    Returns out [sum n][Hq][D] and lse [sum n][Hq], both fp64.  For each
    sequence and q head the full [n][L] score matrix is formed, keys beyond a
    row's own position are set to -inf, and each row is soft-maxed."""
    q = to_f64(q, dtype)
    T, Hq, D = q.shape
    Hkv = pool_k.shape[1]
    out = np.zeros((T, Hq, D))
    lse = np.full((T, Hq), -np.inf)
    row = 0
    for s in range(len(context_lens)):
        L, n = int(context_lens[s]), int(q_lens[s])
        assert n <= L or L == 0
        if L > 0 and n > 0:
            K, V = gather(pool_k, pool_v, tables[s], L, dtype, kv)
            visible = visible_keys(L, query_positions(L, n))
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hkv)
                z = scale * (q[row:row + n, h, :] @ K[:, g, :].T)
                z = np.where(visible, z, -np.inf)
                m = z.max(axis=1, keepdims=True)
                e = np.exp(z - m)
                lsum = e.sum(axis=1, keepdims=True)
                out[row:row + n, h] = (e / lsum) @ V[:, g, :]
                lse[row:row + n, h] = (m + np.log(lsum))[:, 0]
        row += n
    return out, lse


def split_partials(q, pool_k, pool_v, tables, context_lens, q_lens, scale, dtype, partition):
    """Per-partition softmax state for every (row, head, partition).

    Partition p covers keys [p*partition, (p+1)*partition).  For each it
    returns the running max m_p, the sum l_p of exp(z - m_p) over its visible
    keys and the normalised partial output o_p; a partition with no visible key
    has m = -inf, l = 0, o = 0.  Shapes: m, l [T][Hq][P]; o [T][Hq][P][D]."""
    q = to_f64(q, dtype)
    T, Hq, D = q.shape
    Hkv = pool_k.shape[1]
    P = max(1, -(-int(max(context_lens)) // partition))
    m = np.full((T, Hq, P), -np.inf)
    l = np.zeros((T, Hq, P))
    o = np.zeros((T, Hq, P, D))
    row = 0
    for s in range(len(context_lens)):
        L, n = int(context_lens[s]), int(q_lens[s])
        if L > 0:
            K, V = gather(pool_k, pool_v, tables[s], L, dtype)
            positions = query_positions(L, n)
            for i in range(n):
                last = int(positions[i])
                for h in range(Hq):
                    g = kv_head_of(h, Hq, Hkv)
                    for p in range(P):
                        a, b = p * partition, min((p + 1) * partition, last + 1)
                        if a >= b:
                            continue
                        z = scale * (K[a:b, g] @ q[row + i, h])
                        m[row + i, h, p] = z.max()
                        e = np.exp(z - z.max())
                        l[row + i, h, p] = e.sum()
                        o[row + i, h, p] = (e @ V[a:b, g]) / e.sum()
        row += n
    return m, l, o


def merge_partials(m, l, o):
    """Log-sum-exp merge over the last partition axis.

    M = max_p m_p, w_p = l_p exp(m_p - M), out = sum_p w_p o_p / sum_p w_p,
    lse = M + log(sum_p w_p)."""
    M = m.max(axis=-1)
    safe = np.where(np.isfinite(M), M, 0.0)
    w = np.where(l > 0, l * np.exp(np.where(l > 0, m, 0.0) - safe[..., None]), 0.0)
    W = w.sum(axis=-1)
    out = np.where(W[..., None] > 0, (w[..., None] * o).sum(axis=-2) / np.where(W > 0, W, 1.0)[..., None], 0.0)
    lse = np.where(W > 0, safe + np.log(np.where(W > 0, W, 1.0)), -np.inf)
    return out, lse
