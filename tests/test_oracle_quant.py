"""Pins of the oracle's quantized-weight formats (CPU).

A draft head may be post-training quantized to FP8 or NVFP4 (ModelOpt:
export and PTQ section; MAX-walkthrough section 5: a quantized draft carries
weight_scale tensors).  The element encodings are the OCP 8-bit E4M3 and
4-bit E2M1 definitions; the scale layout is this project's reading (one fp32
scale per output row; NVFP4 adds an E4M3 scale per 16 inputs of a row).

Pins: the E4M3 decoder against PyTorch's float8_e4m3fn conversion (a library
routine) on all 256 codes; the E2M1 decoder against the OCP table of
magnitudes; the nibble order and block indexing on hand-built bytes; and a
whole step of a quantized head against the step of a bf16-format head given
the same matrices dequantized by an independent route (torch's float8 cast
and a table lookup), so a transposed scale, a swapped nibble or a shifted
block fails.
"""
import pytest
import torch

import oracle
import workloads as W

F64 = torch.float64
# OCP FP4 E2M1 magnitudes for codes 0..7 (sign is the top bit of the nibble)
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e4m3_matches_torch_float8():
    c = torch.arange(256, dtype=torch.int64)
    a = oracle.decode_e4m3(c)
    b = c.to(torch.uint8).view(torch.float8_e4m3fn).to(F64)
    assert torch.equal(a.isnan(), b.isnan()) and int(a.isnan().sum()) == 2
    ok = ~a.isnan()
    assert torch.equal(a[ok], b[ok])
    assert float(a[0x7E]) == 448.0 and float(a[0x01]) == 2.0 ** -9 and float(a[0x38]) == 1.0


def test_e2m1_table():
    v = oracle.decode_e2m1(torch.arange(16))
    assert v[:8].tolist() == E2M1_TABLE
    assert v[8:].tolist() == [-x for x in E2M1_TABLE]


def test_nvfp4_nibble_order_and_blocks():
    # one row of 32 elements: byte i holds elements 2i (low nibble) and 2i+1
    codes = torch.zeros(1, 16, dtype=torch.uint8)
    codes[0, 0] = 0x21          # element 0 = 0.5, element 1 = 1.0
    codes[0, 8] = 0xA7          # element 16 = 6.0, element 17 = -1.0
    blocks = torch.tensor([[0x38, 0x40]], dtype=torch.uint8)     # E4M3 1.0 and 2.0
    q = oracle.QuantWeight("nvfp4", codes, torch.tensor([0.5]), blocks)
    w = q.dense()
    assert q.shape == (1, 32)
    assert w[0, 0] == 0.25 and w[0, 1] == 0.5
    assert w[0, 16] == 6.0 and w[0, 17] == -1.0
    assert int((w != 0).sum()) == 4


def _dequant_independent(fmt, Wt, name):
    codes, rs = Wt[name], Wt[name + ".row_scale"].to(F64)
    if fmt == "fp8":
        w = codes.view(torch.float8_e4m3fn).to(F64)
    else:
        lut = torch.tensor(E2M1_TABLE + [-x for x in E2M1_TABLE], dtype=F64)
        c = codes.to(torch.int64)
        el = torch.empty(c.shape[0], c.shape[1] * 2, dtype=torch.int64)
        el[:, 0::2], el[:, 1::2] = c & 15, c >> 4
        bs = Wt[name + ".block_scale"].view(torch.float8_e4m3fn).to(F64)
        w = lut[el] * torch.kron(bs, torch.ones(1, 16, dtype=F64))
    return w * rs[:, None]


@pytest.mark.parametrize("name", ["mha_small_fp8", "mla_small_fp8", "mha_small_nvfp4", "mla_small_b48_nvfp4"])
def test_quantized_step_equals_dequantized_bf16_format_step(name):
    cfg = W.get_config(name)
    Wt = W.make_weights(cfg)
    st = W.make_inputs(cfg)
    Wd = {k: v for k, v in Wt.items() if "." not in k}
    for n in oracle.eagle3_oracle.GEMM_WEIGHTS:
        if n in Wt:
            Wd[n] = _dequant_independent(cfg.weight_format, Wt, n)
    rq = oracle.draft_step(cfg, Wt, {k: v.clone() for k, v in st.items()}, 0)
    rd = oracle.draft_step(cfg.replace(weight_format="bf16"), Wd, {k: v.clone() for k, v in st.items()}, 0)
    for k in ("hidden_out", "logits"):
        assert torch.allclose(rq[k], rd[k], rtol=0, atol=1e-12), (name, k)
    assert torch.equal(rq["token_out"], rd["token_out"])
