"""CPU-only checks of the C ABI: the library loads, exports every symbol that
include/dsq.h declares, and its host logic (size queries, argument
validation) behaves as documented.  No compute call is made: every call here
returns from the host-side checks before anything would be enqueued."""
import ctypes
import os
import re

import numpy as np
import pytest

import layout_v1
import oracle
from group_quantized_moe_dsq_amd import dsq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsq.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = dsq.lib()
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"libdsq.so does not export {n}"
    assert sorted(dsq.EXPORTS) == names


def test_status_strings():
    for code, name in dsq.STATUS.items():
        assert dsq.status_string(code).startswith(name)
    assert dsq.status_string(12345) == "unknown dsq_status"


@pytest.mark.parametrize("bits,group,K,N,batch", [(8, 64, 4096, 4096, 1), (4, 64, 4096, 2048, 256),
                                                   (8, 128, 2048, 4096, 3), (4, 128, 256, 33, 2),
                                                   (8, 64, 4096, 129280, 1)])
def test_packed_bytes_matches_layout(bits, group, K, N, batch):
    assert dsq.packed_bytes(bits, group, K, N, batch) == layout_v1.packed_bytes(bits, group, K, N,
                                                                                 batch)


def test_packed_bytes_rejects():
    assert dsq.packed_bytes(5, 64, 128, 4, 1) == 0
    assert dsq.packed_bytes(8, 32, 128, 4, 1) == 0
    assert dsq.packed_bytes(8, 64, 100, 4, 1) == 0
    assert dsq.packed_bytes(8, 64, 0, 4, 1) == 0
    assert dsq.packed_bytes(8, 64, 1 << 40, 1 << 40, 1) == 0


def desc(bits=8, group=64, K=128, N=4, batch=1, data=0x10000):
    d = dsq.QWeightDesc()
    rc = dsq.lib().dsq_qweight_init(ctypes.byref(d), bits, group, K, N, batch,
                                    ctypes.c_void_p(data))
    return d, rc


def test_qweight_init_validation():
    d, rc = desc()
    assert rc == 0 and d.layout_version == dsq.LAYOUT_VERSION and d.reserved == 0
    assert desc(data=0x10001)[1] == -3          # not 256-byte aligned
    assert desc(K=100)[1] == -2                 # K % group
    assert desc(bits=3)[1] == -1
    assert desc(data=0)[1] == -1


def test_calls_validate_before_touching_the_device():
    L = dsq.lib()
    d, _ = desc()
    fake = ctypes.c_void_p(0x20000)
    mis = ctypes.c_void_p(0x20004)
    # NULL pointers
    assert L.dsq_gemv(None, 0, fake, fake, None) == -1
    assert L.dsq_gemv(ctypes.byref(d), 0, None, fake, None) == -1
    # expert out of range
    assert L.dsq_gemv(ctypes.byref(d), 1, fake, fake, None) == -1
    # misaligned x
    assert L.dsq_gemv(ctypes.byref(d), 0, mis, fake, None) == -3
    # wrong layout version
    bad = dsq.QWeightDesc.from_buffer_copy(d)
    bad.layout_version = 7
    assert L.dsq_gemv(ctypes.byref(bad), 0, fake, fake, None) == -9
    # gemm: bad math mode, negative M, missing workspace for bf16
    assert L.dsq_gemm(ctypes.byref(d), 0, fake, fake, 4, 9, None, 0, None) == -1
    assert L.dsq_gemm(ctypes.byref(d), 0, fake, fake, -1, 0, None, 0, None) == -2
    assert L.dsq_gemm(ctypes.byref(d), 0, fake, fake, 128, 1, None, 0, None) == -4
    # pack: range of entries
    assert L.dsq_pack_weights(fake, ctypes.byref(d), 0, 2, None, None) == -1
    assert L.dsq_pack_weights(None, ctypes.byref(d), 0, 1, None, None) == -1
    # route: k > E, unsupported sizes
    assert L.dsq_moe_route_topk(fake, None, 4, 8, 9, fake, fake, None) == -2
    assert L.dsq_moe_route_topk(fake, None, 4, 8192, 6, fake, fake, None) == -5
    assert L.dsq_moe_route_topk(None, None, 4, 8, 2, fake, fake, None) == -1


def test_moe_validation_and_workspace_query():
    L = dsq.lib()
    H, I, E = 256, 128, 8
    g, _ = desc(4, 64, H, I, E)
    u, _ = desc(4, 64, H, I, E)
    dn, _ = desc(4, 64, I, H, E)
    fake = ctypes.c_void_p(0x40000)
    need = dsq.moe_workspace_bytes(5, E, 2, H, I, dsq.MATH_FP32)
    assert need > 0
    # workspace too small
    rc = L.dsq_moe_ffn(fake, fake, None, ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), 5, 2,
                       0, fake, fake, need - 1, None, None, None, None, None)
    assert rc == -4
    # mismatched down shape
    dbad, _ = desc(4, 64, H, H, E)
    rc = L.dsq_moe_ffn(fake, fake, None, ctypes.byref(g), ctypes.byref(u), ctypes.byref(dbad), 5,
                       2, 0, fake, fake, need, None, None, None, None, None)
    assert rc == -2
    # mixed bit widths
    u8, _ = desc(8, 64, H, I, E)
    rc = L.dsq_moe_ffn(fake, fake, None, ctypes.byref(g), ctypes.byref(u8), ctypes.byref(dn), 5,
                       2, 0, fake, fake, need, None, None, None, None, None)
    assert rc == -2
    # k > E
    rc = L.dsq_moe_ffn(fake, fake, None, ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), 5,
                       9, 0, fake, fake, need, None, None, None, None, None)
    assert rc == -2
    # the bf16 workspace holds the bf16 copies in addition
    assert dsq.moe_workspace_bytes(256, 256, 6, 4096, 2048, dsq.MATH_BF16_MFMA) > 0
    assert dsq.moe_workspace_bytes(5, E, 9, H, I, 0) == 0


def test_matrix_core_paths_reject_entries_of_2gib():
    """The grouped GEMM and decode kernels address one expert's codes and
    (scale, zp) with 32-bit offsets: an entry of 2 GiB or more is refused up
    front, not computed wrongly."""
    L = dsq.lib()
    fake = ctypes.c_void_p(0x40000)
    # INT8 g64, K = 65536, N = 32768: 2 GiB of codes + 256 MiB of metadata per entry
    H, I, E = 65536, 32768, 2
    assert dsq.packed_bytes(8, 64, H, I, 1) > (1 << 31)
    g, rg = desc(8, 64, H, I, E)
    u, ru = desc(8, 64, H, I, E)
    dn, rd = desc(8, 64, I, H, E)
    assert rg == ru == rd == 0
    rc = L.dsq_moe_ffn(fake, fake, None, ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), 1,
                       2, 0, fake, fake, 1 << 40, None, None, None, None, None)
    assert rc == -5
    # the dense FP32 path with M >= 2 runs the same grouped kernel
    assert L.dsq_gemm(ctypes.byref(g), 0, fake, fake, 2, dsq.MATH_FP32, fake, 1 << 40, None) == -5
    # just below the limit the shape is accepted up to the device check
    g2, _ = desc(8, 64, 4096, 4096, 1)
    assert L.dsq_gemm(ctypes.byref(g2), 0, fake, fake, 2, dsq.MATH_FP32, fake, 1 << 40,
                      None) != -5


def test_superblock_format_shapes_and_limits():
    # group 256 is the 4-bit super-block format: 16-byte block headers
    N, K = 10, 512
    assert dsq.packed_bytes(4, 256, K, N) == layout_v1.packed_bytes(4, 256, K, N, 1)
    assert dsq.packed_bytes(4, 256, K, N) == 2560 + 512   # align256(N*K/2) + align256(N*2*16)
    assert dsq.packed_bytes(8, 256, K, N) == 0            # 8-bit super-blocks: no
    assert dsq.packed_bytes(4, 256, 384, N) == 0          # K % 256 != 0
    L = dsq.lib()
    g, rg = desc(4, 256, 256, 256, 4)
    u, ru = desc(4, 256, 256, 256, 4)
    dn, rd = desc(4, 256, 256, 256, 4)
    assert rg == ru == rd == 0
    fake = ctypes.c_void_p(0x40000)
    # the matrix-core paths do not read it
    assert L.dsq_moe_ffn(fake, fake, None, ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), 5,
                         2, 0, fake, fake, 1 << 30, None, None, None, None, None) == -5
    assert L.dsq_gemm(ctypes.byref(g), 0, fake, fake, 8, 0, fake, 1 << 30, None) == -5


def test_moe_block_validation_and_workspace_query():
    L = dsq.lib()
    H, I, E = 256, 128, 8
    g, _ = desc(4, 64, H, I, E)
    u, _ = desc(4, 64, H, I, E)
    dn, _ = desc(4, 64, I, H, E)
    fake = ctypes.c_void_p(0x40000)
    need = dsq.moe_block_workspace_bytes(5, E, 2, H, I, dsq.MATH_FP32)
    # the normalised rows come first, 256-byte aligned
    assert need == dsq.moe_workspace_bytes(5, E, 2, H, I, dsq.MATH_FP32) + 5 * H * 4

    def call(norm_w, eps, ws_bytes, k=2, xn=None):
        return L.dsq_moe_block(fake, norm_w, eps, fake, None, ctypes.byref(g), ctypes.byref(u),
                               ctypes.byref(dn), 5, k, 0, fake, fake, ws_bytes, xn, None, None,
                               None, None, None)
    assert call(None, 1e-6, need) == -1                      # no norm weight
    for eps in (0.0, -1e-6, float("nan"), float("inf")):
        assert call(fake, eps, need) == -1, eps              # eps not finite and positive
    assert call(fake, 1e-6, need - 1) == -4                  # workspace too small
    assert call(fake, 1e-6, need, k=9) == -2                 # k > E
    assert call(fake, 1e-6, need, xn=ctypes.c_void_p(0x40004)) == -3  # xn_out misaligned
    assert dsq.moe_block_workspace_bytes(5, E, 9, H, I, 0) == 0


def test_empty_token_batches_return_ok_without_a_device():
    # T = 0 is valid for the MoE entry points: nothing is enqueued
    L = dsq.lib()
    H, I, E = 256, 128, 8
    g, _ = desc(4, 64, H, I, E)
    u, _ = desc(4, 64, H, I, E)
    dn, _ = desc(4, 64, I, H, E)
    fake = ctypes.c_void_p(0x40000)
    need = dsq.moe_block_workspace_bytes(0, E, 2, H, I, 0)
    assert need > 0
    assert L.dsq_moe_block(fake, fake, 1e-6, fake, None, ctypes.byref(g), ctypes.byref(u),
                           ctypes.byref(dn), 0, 2, 0, fake, fake, need, None, None, None, None,
                           None, None) == 0
    assert L.dsq_moe_ffn(fake, fake, None, ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), 0,
                         2, 0, fake, fake, dsq.moe_workspace_bytes(0, E, 2, H, I, 0), None, None,
                         None, None, None) == 0
    c = dsq.ExpertCache(4, 64, H, I, 32, 8, device="cpu", pinned=False)
    need = dsq.moe_cached_workspace_bytes(0, 32, 8, 2, H, I, 0)
    assert L.dsq_moe_ffn_cached(fake, fake, None, ctypes.byref(c.desc), 0, 2, 0, fake, fake, need,
                                None, None, None, None, None, None) == 0
    assert c.hits == c.misses == 0 and (c.expert_of == -1).all()


def test_layout_decoder_round_trip():
    """The test-side layout reader inverts its own encoder, and the encoder
    puts INT4 codes where the header says (word j, byte i: k = 8j+i low,
    k = 8j+4+i high)."""
    rng = np.random.default_rng(40)
    w = (rng.standard_normal((5, 256)) * 0.02).astype(np.float32)
    for bits in (8, 4):
        m = oracle.quantize(w, bits, 64)
        raw = layout_v1.encode_entry(m.q, m.scale, m.zp, bits, 64, 256, 5)
        q, s, z = layout_v1.decode_entry(raw, 0, bits, 64, 256, 5)
        np.testing.assert_array_equal(q, m.q)
        np.testing.assert_array_equal(s, m.scale)
        np.testing.assert_array_equal(z, m.zp)
        if bits == 4:
            codes = oracle.unpack_q(m)
            word0 = raw[0:4]
            assert [int(b) & 15 for b in word0] == list(codes[0, 0:4])
            assert [int(b) >> 4 for b in word0] == list(codes[0, 4:8])


def test_topk_validation_and_workspace_query():
    L = dsq.lib()
    fake = ctypes.c_void_p(0x60000)
    mis = ctypes.c_void_p(0x60002)
    N = 129280
    need = dsq.topk_workspace_bytes(N, 50)
    # two ping-pong buffers of the first round's kept keys: k <= 64 keeps 50
    # keys per 4096-value chunk (32 chunks), larger k per 1024-value chunk
    assert need >= 2 * 32 * 50 * 8 and need % 256 == 0
    assert dsq.topk_workspace_bytes(N, 200) >= 2 * 127 * 200 * 8
    assert dsq.topk_workspace_bytes(1000, 5) > 0          # one chunk: no keys kept
    assert dsq.topk_workspace_bytes(N, 0) == 0
    assert dsq.topk_workspace_bytes(10, 11) == 0
    assert dsq.topk_workspace_bytes(N, 257) == 0
    ws = ctypes.c_void_p(0x80000)
    assert L.dsq_topk(None, N, 1, fake, fake, ws, need, None) == -1
    assert L.dsq_topk(fake, N, 0, fake, fake, ws, need, None) == -2
    assert L.dsq_topk(fake, 10, 11, fake, fake, ws, need, None) == -2
    assert L.dsq_topk(fake, N, 257, fake, fake, ws, need, None) == -5
    assert L.dsq_topk(mis, N, 1, fake, fake, ws, need, None) == -3
    assert L.dsq_topk(fake, N, 50, fake, fake, ws, need - 1, None) == -4
    assert L.dsq_topk(fake, N, 50, fake, fake, None, need, None) == -4
    d, _ = desc(8, 64, 256, 100, 1)
    assert L.dsq_gemv_topk(ctypes.byref(d), 0, fake, fake, 101, fake, fake, ws, 1 << 20, None) == -2
    assert L.dsq_gemv_topk(ctypes.byref(d), 1, fake, fake, 1, fake, fake, ws, 1 << 20, None) == -1
    assert L.dsq_gemv_topk(ctypes.byref(d), 0, mis, fake, 1, fake, fake, ws, 1 << 20, None) == -3


def test_moe_group_validation_and_workspace_query():
    L = dsq.lib()
    fake = ctypes.c_void_p(0x50000)
    mis = ctypes.c_void_p(0x50002)
    need = dsq.moe_group_workspace_bytes(100, 256, 6)
    # bitmap (4 words x 256 experts), active list, count
    assert need == 256 * 16 + 256 * 4 + 256
    # many tokens: the per-expert prefixes double the bitmap
    assert dsq.moe_group_workspace_bytes(4096, 256, 6) == 2 * 128 * 256 * 4 + 256 * 4 + 256
    assert dsq.moe_group_workspace_bytes(65537, 256, 6) == 0
    assert dsq.moe_group_workspace_bytes(4, 4097, 6) == 0
    assert dsq.moe_group_workspace_bytes(4, 8, 9) == 0
    grp = L.dsq_moe_group
    assert grp(None, 4, 8, 2, fake, fake, fake, fake, fake, need, None) == -1
    assert grp(fake, 4, 8, 2, None, fake, fake, fake, fake, need, None) == -1
    assert grp(fake, 4, 8, 9, fake, fake, fake, fake, fake, need, None) == -2
    assert grp(fake, -1, 8, 2, fake, fake, fake, fake, fake, need, None) == -2
    assert grp(fake, 4, 5000, 2, fake, fake, fake, fake, fake, need, None) == -5
    assert grp(fake, 4, 8, 40, fake, fake, fake, fake, fake, need, None) == -2
    assert grp(fake, 70000, 8, 2, fake, fake, fake, fake, fake, need, None) == -5
    assert grp(mis, 4, 8, 2, fake, fake, fake, fake, fake, need, None) == -3
    w4 = dsq.moe_group_workspace_bytes(4, 8, 2)
    assert grp(fake, 4, 8, 2, fake, fake, fake, fake, fake, w4 - 1, None) == -4
    assert grp(fake, 4, 8, 2, fake, fake, fake, fake, None, w4, None) == -4
    assert grp(fake, 4, 8, 2, fake, fake, fake, fake, mis, w4, None) == -3
