"""GPU parity of the output RoPE epilogue (rope_output) against the oracle's output_rope."""
import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa_amd as ck
import seedgen
from cases import attention_error, bf16_bits, make_csa_case
from gpu_helpers import Guarded, run_csa, to_dev
from oracle import formats as F, rope as R

pytestmark = pytest.mark.gpu


def _bf16_ulp(x):
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


@pytest.mark.parametrize("base", [10000.0, 1.0e6])
def test_rope_output_parity(base):
    print(f"case: rope_output base={base}", flush=True)
    B, H = 4, 64
    bits = bf16_bits(seedgen.kv_rows_bf16(81, seedgen.tid(seedgen.TID.Q, 9), (B, H, 512)))
    pos = np.array([0, 5, (1 << 20) + 3, 123456789], dtype=np.int64)
    ref = R.output_rope(F.bf16_bits_to_f64(bits), pos[:, None], base)
    ref_bf16 = F.bf16_bits_to_f64(F.f64_to_bf16_bits(ref))
    out = Guarded((B, H, 512), torch.int16)
    out.t.copy_(torch.from_numpy(bits.view(np.int16)))
    ck.rope_output(out.t, B, H, to_dev(pos), base)
    torch.cuda.synchronize()
    assert out.intact()
    got_bits = out.t.cpu().numpy().view(np.uint16)
    assert np.array_equal(got_bits[..., :448], bits[..., :448])          # no-RoPE dims untouched
    assert np.array_equal(got_bits[0], bits[0])                          # position 0: identity
    got = F.bf16_bits_to_f64(got_bits)
    err = np.abs(got - ref_bf16)[..., 448:]
    assert (err <= _bf16_ulp(ref[..., 448:])).all(), float(err.max())    # at most one bf16 ulp


def test_decode_then_rope_matches_oracle():
    """csa_decode followed by rope_output equals the oracle's decode with R(-i) applied."""
    print("case: csa_decode + rope_output", flush=True)
    case = make_csa_case(82, 3, 3000, 128, 64, 64, 512, "mixed", "fp4")
    topk, out = run_csa(case)
    pos = np.array([4 * 3000 + 127, 77, 1 << 20], dtype=np.int64)
    o = to_dev(F.f64_to_bf16_bits(out).view(np.int16))
    ck.rope_output(o, case.B, case.hq, to_dev(pos), 10000.0)
    torch.cuda.synchronize()
    got = F.bf16_bits_to_f64(o.cpu().numpy().view(np.uint16))
    ref = R.output_rope(case.expect_out, pos[:, None], 10000.0)
    err, ok = attention_error(got, ref)
    print(f"decode + rope: max |out - oracle| = {err:.3e}", flush=True)
    assert ok, err
