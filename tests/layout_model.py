"""A plain numpy statement of the packed-weight byte layout (layout version 2).

Used only to check, byte for byte, what the GPU pack kernel writes.  The layout:
  header            256 bytes
  nibble plane      n_pad * k_pad / 2 bytes, n_pad = ceil(N/128)*128, k_pad = ceil(K/128)*128
                    8x8 micro-blocks: block (row-octet R, k-octet O) at byte 32*(R*(k_pad/8)+O);
                    word i (4 bytes, little endian) of a block = row 8R+i, columns 8O..8O+7;
                    column 8O+j sits in nibble position p(j) = j//2 + 4*(j%2) of the word
  scale plane       at the next 256-byte boundary: g_pad * n_pad scales, g_pad = ceil(k_pad/gs),
                    stored row-octet major: [n_pad/8][g_pad][8] (scale of row n, group g at
                    (n//8)*g_pad*8 + g*8 + n%8)
  padding           code 8 outside [N, K]; scale 0 outside [K/gs, N]
"""
import numpy as np


def rup(v, m):
    return (v + m - 1) // m * m


def layout(N, K, gs, scale_bytes):
    n_pad, k_pad = rup(N, 128), rup(K, 128)
    g_pad = (k_pad + gs - 1) // gs
    nib_off = 256
    nib_bytes = n_pad * k_pad // 2
    scale_off = rup(nib_off + nib_bytes, 256)
    total = rup(scale_off + g_pad * n_pad * scale_bytes, 256)
    return dict(n_pad=n_pad, k_pad=k_pad, g_pad=g_pad, nib_off=nib_off, nib_bytes=nib_bytes,
                scale_off=scale_off, total=total)


def nibble_plane(codes: np.ndarray) -> np.ndarray:
    """Expected nibble plane (uint8) for codes [N, K]."""
    N, K = codes.shape
    n_pad, k_pad = rup(N, 128), rup(K, 128)
    full = np.full((n_pad, k_pad), 8, dtype=np.uint32)
    full[:N, :K] = codes
    # words[n, o] holds row n, k-octet o
    words = np.zeros((n_pad, k_pad // 8), dtype=np.uint32)
    for j in range(8):
        p = j // 2 + 4 * (j % 2)
        words |= full[:, j::8] << np.uint32(4 * p)
    # block (R, O) = 8 consecutive words (rows 8R..8R+7 of k-octet O)
    blocks = words.reshape(n_pad // 8, 8, k_pad // 8).transpose(0, 2, 1)   # [R][O][i]
    return np.ascontiguousarray(blocks).reshape(-1).astype("<u4").view(np.uint8)


def scale_plane(scales: np.ndarray, K: int, gs: int) -> np.ndarray:
    """Expected scale plane bytes for scales [K/gs, N] (fp16 or fp32 numpy array)."""
    G, N = scales.shape
    n_pad, k_pad = rup(N, 128), rup(K, 128)
    g_pad = (k_pad + gs - 1) // gs
    plane = np.zeros((g_pad, n_pad), dtype=scales.dtype)
    plane[:G, :N] = scales
    octet_major = plane.reshape(g_pad, n_pad // 8, 8).transpose(1, 0, 2)    # [n/8][g][n%8]
    return np.ascontiguousarray(octet_major).reshape(-1).view(np.uint8)
