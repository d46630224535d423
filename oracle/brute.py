"""Pure-Python brute force for tiny inputs — an independent second reading
of the oracle's definitions, used only by tests to pin ``bsa_oracle.c``.

TEST INFRASTRUCTURE ONLY.  Nothing here is shared with the C oracle or the
HIP kernels.  Lists and the standard library only (``math.fsum`` for exactly
rounded sums).
"""
import itertools
import math

# axis orders as strings, outermost -> innermost (PAROAttention verdict, key
# machinery: six orders of the F, H, W axes)
ORDER_NAMES = ["FHW", "FWH", "HFW", "HWF", "WFH", "WHF"]


def perm(order: int, F: int, H: int, W: int):
    """Reordered position -> natural index, by enumerating coordinate tuples
    with the outermost axis slowest (itertools.product order)."""
    name = ORDER_NAMES[order]
    ext = {"F": F, "H": H, "W": W}
    out = []
    for tup in itertools.product(*(range(ext[a]) for a in name)):
        c = dict(zip(name, tup))
        out.append((c["F"] * H + c["H"]) * W + c["W"])
    return out


def attention_row(q, keys, vals, scale):
    """Softmax attention of one query over the given (unmasked) keys, with
    exactly rounded sums: returns (o list, lse)."""
    if not keys:
        return [0.0] * len(q), -math.inf
    s = [scale * math.fsum(a * b for a, b in zip(q, k)) for k in keys]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    l = math.fsum(e)
    o = [math.fsum(e[t] * vals[t][c] for t in range(len(vals))) / l for c in range(len(q))]
    return o, m + math.log(l)


def topk_row(keys, k):
    """Indices of the k largest keys, ties by smaller index; ascending."""
    order = sorted(range(len(keys)), key=lambda j: (-keys[j], j))
    return sorted(order[:k])


def window_sets(order, F, H, W, Bq, Bk, T, r0):
    """Temporal window per q-block by direct enumeration of block centres."""
    N = F * H * W
    pm = perm(order, F, H, W)

    def centre(b, B):
        ln = min(B, N - b * B)
        n = pm[b * B + (ln - 1) // 2]
        return n // (H * W), n % (H * W)

    nq, nk = -(-N // Bq), -(-N // Bk)
    out = []
    for i in range(nq):
        fi, oi = centre(i, Bq)
        row = []
        for j in range(nk):
            fj, oj = centre(j, Bk)
            df = abs(fi - fj)
            if df <= T and abs(oi - oj) <= (r0 * W) // (2 ** df):
                row.append(j)
        out.append(row)
    return out


def block_stats(Q, K, B, eps, scale):
    """Dense softmax map of one head (Q, K: lists of rows) cut into B x B
    blocks: returns (cnt, sum, max) as nested lists [nb][nb], with every row
    normalised by an exactly rounded sum."""
    N = len(Q)
    nb = -(-N // B)
    cnt = [[0] * nb for _ in range(nb)]
    sm = [[[] for _ in range(nb)] for _ in range(nb)]
    mx = [[0.0] * nb for _ in range(nb)]
    for r in range(N):
        s = [scale * math.fsum(a * b for a, b in zip(Q[r], K[c])) for c in range(N)]
        top = max(s)
        e = [math.exp(x - top) for x in s]
        tot = math.fsum(e)
        for c in range(N):
            a = e[c] / tot
            i, j = r // B, c // B
            cnt[i][j] += a < eps
            sm[i][j].append(a)
            mx[i][j] = max(mx[i][j], a)
    return cnt, [[math.fsum(v) for v in row] for row in sm], mx
