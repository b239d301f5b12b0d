"""The online softmax's rescale of non-zero accumulators, against the oracle.

The attention keeps a running reference maximum per head and rescales its output
accumulators only when a later 32-row step raises that maximum by more than a factor 2^8.
With N(0,1) rows and queries at scale 1/sqrt(512) that never happens after the first
step, so these inputs are built to take that branch often, in every storage format, for
CSA (REUSE mode, whose row order the caller controls) and HCA:

* rows are e_r = 0.5 z_r + c_r * 1 (z_r ~ N(0,1), 1 the all-ones vector) and queries
  q_h = a_h * 1 + 0.3 z'_h with a per-head slope a_h in [0.25, 0.75];
* along the row list, c follows a ladder of 320-row blocks (ten 32-row steps): nine
  steps at level k, then a step whose first row is a spike at level k + 1 while its other
  31 rows stay at level k; the next block sits at level k + 1, and every list ends with a
  spike step, so the rows before the last spike still carry about half of the output;
* a level is worth a_h * 32.6 * dc base-2 units of logit (dc = 0.52), so heads with
  a_h above about 0.47 see each spike exceed the running maximum by more than 2^8 (their
  accumulators, holding the plateau's rows, are rescaled), the others do not, within the
  same step.

The row values stay below 22.5 in magnitude, the bound of the other workloads' rows.
The batch sizes are chosen so that each query's rows span several 32-row steps in one
workgroup (B = 16 for the 640-row CSA lists, B = 4 for the 2240-row ones, B = 8 for 960
and 2240 HCA rows), with spikes inside those runs of steps; the longer lists run on the
64-head workgroups, the shorter ones on the 16-head ones.  The test first
checks those properties on the oracle's logits, then compares the GPU output with the
oracle (max-abs 1e-2; bf16's half-ulp added where |o| >= 4).
"""
import math

import numpy as np
import pytest
import torch

import compressed_sparse_kv_csa_amd as ck
import seedgen
from cases import KV_FMTS, attention_error, encode_kv, oracle_hca
from gpu_helpers import Guarded, run_hca, to_dev, upload_kv, workspace
from oracle import decode as OD, formats as OF

pytestmark = pytest.mark.gpu
T = seedgen.TID
D = 512
DC = 0.52
LOG2E = 1.4426950408889634


def _ladder(n):
    """Level of each list position: nine steps at level k, then a step whose first row is
    a spike at level k + 1 (the other 31 at k); n is a multiple of 320."""
    assert n % 320 == 0
    p = np.arange(n)
    k = p // 320
    spike = (p % 320) == 288
    return (k + spike) * DC - 2.5


def _queries(seed, B, hq):
    z = seedgen.normal(seed, seedgen.tid(T.Q, 7), (B, hq, D)).double().numpy()
    a = 0.25 + 0.5 * (np.arange(hq) % 16) / 15.0                     # per-head slope
    q = a[None, :, None] + 0.3 * z
    return OF.f64_to_bf16_bits(q)


def _rows(seed, B, n, level):
    """[B][n][512] bf16 rows 0.5 z + level * 1 (level per row)."""
    z = seedgen.normal(seed, seedgen.tid(T.KV, 7), (B, n, D)).double().numpy()
    return OF.f64_to_bf16_bits(0.5 * z + level[..., None])


def _assert_branch_taken(qv, rows, scale):
    """Inputs check: per head, the running maximum over whole 32-row steps rises by more than
    2^8 at some step after the first for some heads, and for other heads never."""
    l2 = scale * LOG2E * (qv @ rows.T)                                   # [H][R] base-2 logits
    n_steps = l2.shape[1] // 32
    steps = l2[:, :n_steps * 32].reshape(l2.shape[0], n_steps, 32).max(axis=2)
    run = np.maximum.accumulate(steps, axis=1)
    rise = steps[:, 1:] - run[:, :-1]
    grows = (rise > 8.0).any(axis=1)
    assert grows.any() and (~grows).any(), "inputs do not split the heads over the branch"
    assert np.abs(rows).max() <= 22.5
    return grows


# (B, W, N_c, k): a 640-row list (16-head workgroups) and a 2240-row one (64-head ones)
LISTS = [(16, 128, 1500, 512), (4, 192, 3000, 2048)]


@pytest.mark.parametrize("B,W,n_c,k", LISTS)
@pytest.mark.parametrize("kv_fmt", ["bf16", "mixed", "fp4"])
def test_csa_reuse_rescale(kv_fmt, B, W, n_c, k):
    seed, hq = 801, 64
    print(f"case: csa REUSE rescale kv={kv_fmt} B={B} W={W} Nc={n_c} Hq={hq} k={k}", flush=True)
    n_list = W + k
    # each query's selection: k distinct compressed rows in a seeded order
    sel = np.stack([seedgen.distinct_indices(seed, seedgen.tid(T.POOL, b), n_c, k) for b in range(B)])
    # the level of every cache row follows its position in the list (other rows level -2.5)
    level = np.full((B, W + n_c), -2.5)
    ladder = _ladder(n_list)
    level[:, :W] = ladder[:W]
    for b in range(B):
        level[b, W + sel[b]] = ladder[W:]
    q_bits = _queries(seed, B, hq)
    kv = encode_kv(_rows(seed, B, W + n_c, level), kv_fmt)
    scale = 1.0 / math.sqrt(D)
    qv = OF.bf16_bits_to_f64(q_bits)
    for b in (0, B - 1):
        _assert_branch_taken(qv[b], OD.csa_rows(kv.values[b], W, sel[b]), scale)
    p = ck.CsaParams(B, hq, 0, k, W, ck.MODE_REUSE, scale, 0)
    kvc, keep = upload_kv(kv, stride_pad=2)
    topk = to_dev(sel.astype(np.int32))
    out = Guarded((B, hq, D), torch.int16)
    ck.csa_decode(p, kvc, None, to_dev(q_bits.view(np.int16)), None, None, topk, out.t,
                  workspace(ck.csa_decode_workspace_bytes(p, n_c)))
    torch.cuda.synchronize()
    assert out.intact()
    got = out.t.cpu().view(torch.bfloat16).double().numpy()
    ref = np.stack([OD.csa_reuse_one(qv[b], kv.values[b], W, sel[b], scale) for b in range(B)])
    err, ok = attention_error(got, ref)
    print(f"max |out - oracle| = {err:.3e}  max |oracle| = {np.abs(ref).max():.3f}", flush=True)
    assert ok, err


@pytest.mark.parametrize("rows", [960, 2240])
@pytest.mark.parametrize("kv_fmt", ["bf16", "mixed", "fp4"])
def test_hca_rescale(kv_fmt, rows):
    seed, B, hq = 802, 8, 64
    print(f"case: hca rescale kv={kv_fmt} B={B} rows={rows} Hq={hq}", flush=True)
    q_bits = _queries(seed, B, hq)
    level = np.broadcast_to(_ladder(rows), (B, rows))
    kv = encode_kv(_rows(seed, B, rows, level), kv_fmt)
    scale = 1.0 / math.sqrt(D)
    qv = OF.bf16_bits_to_f64(q_bits)
    _assert_branch_taken(qv[0], kv.values[0], scale)
    ref = oracle_hca(q_bits, kv, scale)
    got = run_hca(q_bits, kv, scale, stride_pad=3)
    err, ok = attention_error(got, ref)
    print(f"max |out - oracle| = {err:.3e}  max |oracle| = {np.abs(ref).max():.3f}", flush=True)
    assert ok, err


def test_rescale_inputs_detect_a_wrong_alpha():
    """The inputs have power: weighting each row as if every rescale of the heads that take
    the branch had used twice the right factor (the earlier rows' weights doubled at each
    later spike) moves the oracle's output of those heads by more than twice the tolerance."""
    seed, rows, hq = 803, 640, 64
    q_bits = _queries(seed, 1, hq)
    kv = encode_kv(_rows(seed, 1, rows, _ladder(rows)[None]), "bf16")
    qv, e = OF.bf16_bits_to_f64(q_bits)[0], kv.values[0]
    scale = 1.0 / math.sqrt(D)
    grows = _assert_branch_taken(qv, e, scale)
    l = scale * (qv @ e.T)
    good = OD.attention(qv, e, scale)
    spikes_after = (rows - 1 - np.arange(rows) + 32) // 320              # later spikes per row
    w = np.exp(l - l.max(axis=1, keepdims=True)) * 2.0 ** spikes_after[None]
    bad = (w / w.sum(axis=1, keepdims=True)) @ e
    assert np.abs(bad - good)[grows].max() > 2 * 1e-2
