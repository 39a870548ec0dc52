"""GPU: dequantisation exports and the NF4 packer, bit for bit against the oracle."""
import numpy as np
import pytest

import oracle
from oracle import pack as P
from gpu_util import log, up, bits16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def geg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_expert_gemm_amd as g
    g.lib()
    return g


def test_nf4_export_every_byte_bit_exact(geg):
    log("case: gnf4_dequant, every code byte x 48 absmax values")
    rng = np.random.default_rng(0)
    absv = np.concatenate([
        [0.0, 1.0, 0.5, 2.0 ** -126, 1e-40, 3e-45, 65504.0, 7e4, 1e30, -0.02],
        (rng.standard_normal(38) * 0.05).astype(np.float32)]).astype(np.float32)
    N, K = absv.size, 512
    codes = np.tile(np.arange(256, dtype=np.uint8), (N, 1))          # every byte in every row
    absmax = np.repeat(absv[:, None], K // 64, axis=1).astype(np.float32)
    absmax[:, 1::2] = absmax[:, 1::2][::-1]                           # mix values across blocks
    f32, bf, h = geg.gnf4_dequant(up(codes[None]), up(absmax[None]))
    w32 = oracle.nf4_w32(codes, absmax)
    got = f32[0].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), w32.view(np.uint32))
    assert np.array_equal(bits16(bf[0]), P.bf16_rne_bits(w32))
    gh, rh = bits16(h[0]), P.fp16_rne_bits(w32)
    bad = np.argwhere(gh != rh)
    for n, k in bad[:12]:
        log(f"  fp16 mismatch absmax={absmax[n, k // 64]!r} code={oracle.unpack_nf4_codes(codes)[n, k]} "
            f"w32={w32[n, k]!r} got=0x{gh[n, k]:04x} want=0x{rh[n, k]:04x}")
    assert len(bad) == 0


def test_mxfp4_export_every_byte_and_scale(geg):
    log("case: gmxfp4_dequant, 256 code bytes x 256 scale bytes")
    N, K = 256, 512
    codes = np.tile(np.arange(256, dtype=np.uint8), (N, 1))
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], K // 32, axis=1)
    f32, bf, h = geg.gmxfp4_dequant(up(codes[None]), up(scales[None]))
    w32 = oracle.mxfp4_w32(codes, scales)
    got = f32[0].cpu().numpy()
    nan_ref, nan_got = np.isnan(w32), np.isnan(got)
    assert np.array_equal(nan_ref, nan_got)
    assert np.array_equal(got[~nan_got].view(np.uint32), w32[~nan_ref].view(np.uint32))
    assert np.array_equal(bits16(h[0])[~nan_ref], P.fp16_rne_bits(w32)[~nan_ref])
    # bf16 comes from the gfx950 scaled fp4 -> bf16 conversion the GEMMs use to
    # decode; it must equal RNE(fp32) for every (code, scale) pair, subnormal,
    # overflowing and NaN scales included
    gb = bits16(bf[0])
    rb = P.bf16_rne_bits(w32)
    bnan = ((gb & 0x7F80) == 0x7F80) & ((gb & 0x7F) != 0)
    assert np.array_equal(bnan, nan_ref)
    bad = np.argwhere((gb != rb) & ~nan_ref)
    log(f"  bf16 export mismatches: {len(bad)} at (scale byte, k) {bad[:6].tolist()}")
    assert len(bad) == 0


def test_nf4_packer_matches_oracle(geg):
    log("case: gnf4_quantize vs oracle quantiser")
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((96, 1024)) * 0.02).astype(np.float32)
    w[3, 64:128] = 0.0                                  # all-zero block
    w[5, :64] = np.float32(1e-39)                       # subnormal absmax
    w[7, 128:192] *= 1e6
    q, s = geg.gnf4_quantize(up(w))
    qo, so = oracle.quantize_pack_nf4(w)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), so.view(np.uint32))
