"""Integer CPU reference of the 64-token chunk table (test side).

For packed sequences with token offsets cu[0..N]: sequence n has
ceil(len_n / 64) chunks; chunk j of sequence n starts at token
cu[n] + 64 j and holds min(64, len_n - 64 j) valid tokens.  Chunks are
numbered sequence by sequence.  Rows past the last chunk (up to the bound
floor((T + 63 N) / 64)) are (-1, 0, 0, 0).
"""
import numpy as np

C = 64


def max_chunks(N: int, T: int) -> int:
    return (T + (C - 1) * N) // C


def chunk_table(cu, N: int, T: int):
    cu = np.array([0, T]) if cu is None else np.asarray(cu, dtype=np.int64)
    mc = max_chunks(N, T)
    rec = np.tile(np.array([-1, 0, 0, 0], dtype=np.int32), (mc, 1))
    seq_off = np.zeros(N + 1, dtype=np.int32)
    c = 0
    for n in range(N):
        seq_off[n] = c
        s0, s1 = int(cu[n]), int(cu[n + 1])
        for j, start in enumerate(range(s0, s1, C)):
            rec[c] = (n, start, min(C, s1 - start), j)
            c += 1
    seq_off[N] = c
    return rec, seq_off, c
