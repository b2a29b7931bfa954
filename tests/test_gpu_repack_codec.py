"""GPU parity of the offline repacks and the FP8 encoder at full size.

* q4_0 repack of a grid whose trained steps are not bf16 values (fp32 steps,
  the case behind the E2B article's "90.0 % of values bit-identical", key
  conclusions): codes, steps and the counted groups bit-exact against the
  oracle, and the share of unpacked values equal to the stored ones (from the
  GPU's own unpack) equal to the oracle's statistic.
* E4M3FNUZ -> OCP E4M3 conversion of the full K=5120, N=25600 layer (E2B
  article, "Tip: E4M3 or E4M3FNUZ"): the GPU's FNUZ repack, the converted
  codes, the scales and the inexact count against the oracle's, and fp32
  value equality dec_ocp(b') * s' == dec_fnuz(b) * s for every element.
* The fp32 -> FP8 encoder on every fp32 bit pattern that is not a NaN (NaN
  inputs are outside the quantisers' contract), OCP and FNUZ, in chunks.
"""

import numpy as np
import pytest
import torch

import gen
from helpers import dev, host

pytestmark = pytest.mark.gpu

OCP, FNUZ = 0, 1


@pytest.fixture(scope="module")
def q():
    import quantized_linear_layers_amd as qlin

    assert torch.cuda.is_available()
    return qlin


def test_repack_q4_0_unrounded_steps(q, oracle):
    d = gen.linear_config(2, bf16_steps=False)
    w = d["w_bf16"]
    pc, sc, ac = oracle.repack_q4_0(w)
    frac = oracle.frac_bit_identical(pc, sc, w)
    wd = dev(w)
    codes, steps, amb = q.repack_q4_0(wd)
    back = q.dequant_q4_bf16(codes, steps)
    share = float((back.view(torch.int16) == wd.view(torch.int16)).double().mean())
    torch.cuda.synchronize()
    assert np.array_equal(host(codes), pc)
    assert np.array_equal(host(steps), sc)
    assert int(host(amb)[0]) == ac > 0
    assert share == frac, (share, frac)


@pytest.fixture(scope="module")
def c3_fnuz(oracle):
    d = gen.linear_config(3)
    p, s, amb = oracle.repack_q4_0(d["w_bf16"])
    assert amb == 0
    wf, sf = oracle.repack_fp8(p, s, d["K"], FNUZ)
    wo, so, bad = oracle.fnuz_to_ocp(wf, sf)
    return dict(w_bf16=d["w_bf16"], wf=wf, sf=sf, wo=wo, so=so, bad=bad)


def test_fnuz_to_ocp_c3_full(q, oracle, c3_fnuz):
    c = c3_fnuz
    codes, steps, _ = q.repack_q4_0(dev(c["w_bf16"]))
    wf, sf = q.repack_fp8(codes, steps, "e4m3fnuz")
    del codes, steps
    assert torch.equal(wf.cpu(), torch.from_numpy(c["wf"]))
    assert np.array_equal(host(sf), c["sf"])
    wo, so, bad = q.fp8_fnuz_to_ocp(wf, sf)
    torch.cuda.synchronize()
    assert int(host(bad)[0]) == c["bad"] == 0
    assert np.array_equal(host(so), c["so"])
    assert torch.equal(wo.cpu(), torch.from_numpy(c["wo"]))
    # value preserved for every element: decode both sides exactly (fp64)
    tf = torch.from_numpy(oracle.fp8_decode_table(FNUZ)).cuda()
    to = torch.from_numpy(oracle.fp8_decode_table(OCP)).cuda()
    for n0 in range(0, wf.shape[0], 4096):
        a = tf[wf[n0:n0 + 4096].long()] * sf[n0:n0 + 4096, None].double()
        b = to[wo[n0:n0 + 4096].long()] * so[n0:n0 + 4096, None].double()
        assert torch.equal(a, b), f"value changed in rows {n0}..{n0 + 4095}"


CHUNK = 1 << 28


@pytest.mark.parametrize("chunk", range((1 << 32) // CHUNK))
@pytest.mark.parametrize("fmt", [OCP, FNUZ], ids=["ocp", "fnuz"])
def test_fp8_encoder_exhaustive(q, oracle, fmt, chunk):
    """fp32 bit patterns [chunk * 2^28, (chunk + 1) * 2^28): the GPU encoder
    equals the oracle's nearest-even saturating encoder on every one that is
    not a NaN."""
    bits = np.arange(chunk * CHUNK, (chunk + 1) * CHUNK, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    want = oracle.fp8_encode_array(x, fmt)
    got = host(q.fp8_encode_f32(dev(x), "e4m3" if fmt == OCP else "e4m3fnuz"))
    bad = (got != want) & ~np.isnan(x)
    if bad.any():
        i = np.flatnonzero(bad)[:4]
        raise AssertionError(f"{int(bad.sum())} mismatches, e.g. bits {[hex(int(b)) for b in bits[i]]} "
                             f"gpu {got[i].tolist()} oracle {want[i].tolist()}")
