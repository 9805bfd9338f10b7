"""The page's own packed-weight layout, rebuilt from its description (a reading test).

TEST INFRASTRUCTURE ONLY.  Source: "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit
大模型 CUDA GEMV 内核" (blog.gitcode.com), §5.1 (weight permutation) and §5.2
(interleaved packing and decoding), cited as [W2A8].

The product does not use this layout (its tiling is its own, designed for
64-wide wavefronts), but both share the page's 32-bit word format: sixteen
2-bit codes, element e at bit 8*(e%4) + 2*(e//4).  Rebuilding the page's
whole chain and decoding it the way the page decodes is how the tests check
that this reading of the page is self-consistent.

Readings taken here:
  * the 16x32 permutation is applied by gathering: out[i][j] = block[row(i,j)][col(i,j)];
  * inside a compressed byte, the 4 consecutive codes go to bits 0-1, 2-3,
    4-5, 6-7 in order (the page leaves this open; the interleave that follows
    is stated on the 16 codes of a word, so this choice fixes which code is
    "element e" of the word);
  * the page's sentence that byte j ends up holding elements 4j..4j+3
    contradicts its own pattern and shift table; the pattern and the shift
    table are taken as authoritative (they agree with the decode).
"""
import numpy as np

# [W2A8] §5.2: the interleave pattern; field f of the packed word holds element PATTERN[f].
PATTERN = (0, 4, 8, 12, 1, 5, 9, 13, 2, 6, 10, 14, 3, 7, 11, 15)


def _segments():
    """The 32 row segments of a 16x32 block, in the order the page's kernel threads read
    them (one 32-bit word, 16 consecutive K values, per thread): segment t = 16a + 8b + c
    (a, b in {0, 1}, c in 0..7) is row 8a + c, columns 16b .. 16b + 15 -- the first 8
    threads take rows 0-7 of the left half, the next 8 the same rows of the right half,
    then rows 8-15 likewise.  [W2A8] §5.1 (the 16x32 permutation that lays the weights out
    in the threads' reading order)."""
    return [(8 * a + c, 16 * b) for a in range(2) for b in range(2) for c in range(8)]


_SEGMENTS = _segments()


def block_map(i: int, j: int):
    """[W2A8] §5.1: (i, j) of a permuted 16x32 block -> (row, col) it is read from.

    The permuted block holds the segments one after the other, 16 values each: its
    position 32 i + j is value m = (32 i + j) % 16 of segment t = (32 i + j) // 16."""
    t, m = divmod(32 * i + j, 16)
    row, col0 = _SEGMENTS[t]
    return row, col0 + m


def permute(codes: np.ndarray) -> np.ndarray:
    """[W2A8] §5.1: N x K -> (N//16, K//32, 16, 32), each block gathered through block_map."""
    N, K = codes.shape
    assert N % 16 == 0 and K % 32 == 0
    rows = np.empty((16, 32), dtype=np.int64)
    cols = np.empty((16, 32), dtype=np.int64)
    for i in range(16):
        for j in range(32):
            rows[i, j], cols[i, j] = block_map(i, j)
    blocks = codes.reshape(N // 16, 16, K // 32, 32).transpose(0, 2, 1, 3)
    return blocks[:, :, rows, cols]


def compress(codes_flat: np.ndarray) -> np.ndarray:
    """[W2A8] §5.2 step 3: four 2-bit codes per byte (code p of a group at bits 2p)."""
    c = codes_flat.reshape(-1, 4).astype(np.uint8)
    return (c[:, 0] | (c[:, 1] << 2) | (c[:, 2] << 4) | (c[:, 3] << 6)).astype(np.uint8)


def interleave(packed: np.ndarray) -> np.ndarray:
    """[W2A8] §5.2 step 4: inside every 32-bit word, move element e to bit 8*(e%4) + 2*(e//4)."""
    words = packed.view("<u4").astype(np.uint64)
    out = np.zeros_like(words)
    for e in range(16):
        field = (words >> np.uint64(2 * e)) & np.uint64(3)   # element e before the move
        f = PATTERN.index(e)                                 # field that must hold it
        out |= field << np.uint64(2 * f)
    return out.astype("<u4").view(np.uint8)


def pack(w: np.ndarray) -> np.ndarray:
    """[W2A8] §5.2: the page's four-step chain, +2 -> permute -> compress -> interleave."""
    codes = (w.astype(np.int16) + 2).astype(np.uint8)
    perm = permute(codes)
    return interleave(compress(perm.reshape(-1)))


def decode_word(word: int):
    """[W2A8] §5.2: shift by 2i, keep bits 0-1 of every byte, subtract 2 per byte.

    Returns the 16 int8 values, vector i (bytes 0..3) first.
    """
    vals = []
    for i in range(4):
        v = (word >> (2 * i)) & 0x03030303
        for byte in range(4):
            vals.append(((v >> (8 * byte)) & 0xFF) - 2)
    return vals


def unpack(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """Inverse of ``pack``: decode every word with ``decode_word`` and undo the permutation.

    Word index t inside a 16x32 block is "thread" t of the block: row i = t // 2 of
    the permuted block, columns 16*(t % 2) .. +15, which block_map sends to one row
    and 16 consecutive columns of the original block.
    """
    words = packed.view("<u4")
    out = np.zeros((N, K), dtype=np.int8)
    nb, kb = N // 16, K // 32
    idx = 0
    for bn in range(nb):
        for bk in range(kb):
            for t in range(32):
                vals = decode_word(int(words[idx]))
                idx += 1
                i = t // 2
                for jj in range(16):
                    j = 16 * (t % 2) + jj
                    r, c = block_map(i, j)
                    out[16 * bn + r, 32 * bk + c] = vals[jj]
    return out
