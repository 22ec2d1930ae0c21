"""GPU checks of q4gsw_pack / q4gsw_unpack: bit-exact bytes and round trips, range checks."""
import numpy as np
import pytest
import torch

from synthetic_inputs import draw_codes, draw_scales
from tests import layout_model
from tests.gpu_helpers import lib

pytestmark = pytest.mark.gpu

SHAPES = [(32, 64, 16), (200, 136, 8), (8192, 2048, 32), (2048, 8192, 128), (130, 96, 12), (7, 44, 4),
          (512, 2048, 32), (1, 8, 8)]


@pytest.mark.parametrize("N,K,gs", SHAPES)
@pytest.mark.parametrize("sdt", ["f16", "f32"])
def test_pack_bytes_and_round_trip(N, K, gs, sdt):
    q = lib()
    g = torch.Generator().manual_seed(N * 31 + K)
    codes = draw_codes(g, N, K)
    scales = draw_scales(g, K // gs, N, sdt, 0.002, 0.02)
    pw = q.pack(codes.cuda(), scales.cuda(), gs)
    L = layout_model.layout(N, K, gs, 2 if sdt == "f16" else 4)
    assert pw.desc.bytes == L["total"] and pw.desc.n_pad == L["n_pad"] and pw.desc.k_pad == L["k_pad"]
    buf = pw.buffer.cpu().numpy()
    want_nib = layout_model.nibble_plane(codes.numpy())
    got_nib = buf[L["nib_off"]:L["nib_off"] + L["nib_bytes"]]
    assert np.array_equal(got_nib, want_nib), "nibble plane differs from the layout statement"
    want_sc = layout_model.scale_plane(scales.numpy(), K, gs)
    got_sc = buf[L["scale_off"]:L["scale_off"] + want_sc.size]
    assert np.array_equal(got_sc, want_sc), "scale plane differs from the layout statement"
    c2, s2 = q.unpack(pw)
    assert torch.equal(c2.cpu(), codes)
    assert torch.equal(s2.cpu().view(torch.int16 if sdt == "f16" else torch.int32),
                       scales.view(torch.int16 if sdt == "f16" else torch.int32))


def test_round_trip_patterns_and_special_scales():
    q = lib()
    N, K, gs = 96, 160, 32
    n = torch.arange(N).view(-1, 1)
    k = torch.arange(K).view(1, -1)
    codes = ((n * 7 + k * 3) % 16).to(torch.uint8)
    # every fp16 bit class: zero, subnormals, normals, large, negative
    bits = torch.tensor([0x0000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x6FFF, 0x7000, 0x7BFF, 0x8001, 0xBC00],
                        dtype=torch.int32)
    sc = bits.repeat((K // gs) * N // len(bits) + 1)[: (K // gs) * N].to(torch.int16).view(torch.float16)
    scales = sc.view(K // gs, N).contiguous()
    pw = q.pack(codes.cuda(), scales.cuda(), gs)
    assert not pw.foldable           # subnormal and too-large scales forbid folding into fp16
    c2, s2 = q.unpack(pw)
    assert torch.equal(c2.cpu(), codes)
    assert torch.equal(s2.cpu().view(torch.int16), scales.view(torch.int16))


def test_fold_flag():
    q = lib()
    codes = torch.full((64, 64), 3, dtype=torch.uint8)
    ok = torch.full((2, 64), 0.01, dtype=torch.float16)
    assert q.pack(codes.cuda(), ok.cuda(), 32).foldable
    edge = ok.clone()
    edge[0, 0] = 8188.0
    edge[1, 5] = 2.0 ** -14
    edge[1, 6] = 0.0
    assert q.pack(codes.cuda(), edge.cuda(), 32).foldable
    big = ok.clone()
    big[1, 63] = 8192.0
    assert not q.pack(codes.cuda(), big.cuda(), 32).foldable
    sub = ok.clone()
    sub[0, 1] = 2.0 ** -15
    assert not q.pack(codes.cuda(), sub.cuda(), 32).foldable
    f32 = torch.full((2, 64), 0.01, dtype=torch.float32)
    assert not q.pack(codes.cuda(), f32.cuda(), 32).foldable


def test_code_out_of_range_rejected():
    q = lib()
    codes = torch.randint(0, 16, (40, 64), dtype=torch.uint8)
    codes[17, 33] = 16
    scales = torch.full((2, 40), 0.01, dtype=torch.float16)
    with pytest.raises(q.Q4gswError) as e:
        q.pack(codes.cuda(), scales.cuda(), 32)
    assert e.value.status == 6
