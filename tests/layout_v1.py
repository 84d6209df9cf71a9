"""Independent host-side reading of the packed device layout, version 1.

Written from the layout description in include/dsq.h only (no code shared
with the library): it turns the raw bytes of a packed buffer back into the
oracle's canonical format (codes with k = 2j in the low nibble of byte j for
INT4, fp32 scale and zero point per group), so packed weights can be
compared with the oracle byte for byte.
"""
import numpy as np


def align256(n: int) -> int:
    return (n + 255) // 256 * 256


def geometry(bits, group, K, N):
    rb = K * bits // 8
    ng = K // group
    meta_off = align256(N * rb)
    stride = meta_off + align256(N * ng * (16 if group == 256 else 8))
    return rb, ng, meta_off, stride


def packed_bytes(bits, group, K, N, batch):
    return geometry(bits, group, K, N)[3] * batch


def nibbles_to_canonical(payload: np.ndarray, N: int, K: int) -> np.ndarray:
    """4-bit device words -> canonical bytes (k = 2j low nibble, 2j+1 high)."""
    # device word j: byte i holds k = 8j+i (low nibble) and k = 8j+4+i (high)
    words = payload.reshape(N, K // 8, 4)
    codes = np.empty((N, K // 8, 8), np.uint8)
    codes[:, :, 0:4] = words & 0x0F
    codes[:, :, 4:8] = words >> 4
    codes = codes.reshape(N, K)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def decode_sb_entry(buf: np.ndarray, b: int, K: int, N: int) -> np.ndarray:
    """Super-block format (group 256): the canonical 144-byte blocks
    [N][K/256][144] = 16-byte header, then the 128 canonical code bytes."""
    rb, nb, meta_off, stride = geometry(4, 256, K, N)
    base = b * stride
    canon = nibbles_to_canonical(buf[base:base + N * rb], N, K).reshape(N, nb, 128)
    hdr = buf[base + meta_off:base + meta_off + N * nb * 16].reshape(N, nb, 16)
    return np.concatenate([hdr, canon], axis=-1)


def decode_entry(buf: np.ndarray, b: int, bits: int, group: int, K: int, N: int):
    """Return (canonical q bytes, scale, zp) of batch entry b."""
    rb, ng, meta_off, stride = geometry(bits, group, K, N)
    base = b * stride
    payload = buf[base:base + N * rb].reshape(N, rb)
    meta = buf[base + meta_off:base + meta_off + N * ng * 8].view(np.float32).reshape(N, ng, 2)
    scale = np.ascontiguousarray(meta[:, :, 0])
    zp = np.ascontiguousarray(meta[:, :, 1])
    if bits == 8:
        return np.ascontiguousarray(payload), scale, zp
    return nibbles_to_canonical(payload, N, K), scale, zp


def encode_entry(q_canon: np.ndarray, scale, zp, bits, group, K, N) -> np.ndarray:
    """Inverse of decode_entry (used to test the decoder itself)."""
    rb, ng, meta_off, stride = geometry(bits, group, K, N)
    out = np.zeros(stride, np.uint8)
    if bits == 8:
        out[:N * rb] = q_canon.reshape(-1)
    else:
        codes = np.empty((N, K), np.uint8)
        codes[:, 0::2] = q_canon & 0x0F
        codes[:, 1::2] = q_canon >> 4
        c = codes.reshape(N, K // 8, 8)
        words = (c[:, :, 0:4] | (c[:, :, 4:8] << 4)).astype(np.uint8)
        out[:N * rb] = words.reshape(-1)
    meta = np.stack([scale, zp], axis=-1).astype(np.float32)
    out[meta_off:meta_off + N * ng * 8] = meta.reshape(-1).view(np.uint8)
    return out
