"""Parity of packed forward scans over many short segments: the shapes a multi-segment form of
the fast chunk kernel was written for (several consecutive segments carried through one
workgroup's pipeline, segment starts and ends inside its sequence of chunks, padding rows holding
the next segment's tokens with zeroed gates). Every case is compared with the fp64 oracle on
every output and every final state, with the bf16 checks per 64-token block and on chunk-last
rows as well as over the whole tensor.

The cases use the segment layout of packed training inputs (`segment_layout` on the
"tiny_gdn/fugue.py" page): empty segments, one-token segments, segments of one and of several
chunks, and a short segment right at the end of the packed input after a ragged one.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_70_amd import inputs
from tests._parity import check, check_bf16_detailed, check_states, gpu_np, segments

# A form of the fast kernel that carried several consecutive short segments through one
# workgroup's pipeline was built for these shapes; one build of it made a GPU memory fault on the
# first case here, and no cause was found in its source or its generated code. That form was
# removed; the cases stay, skipped, until a form whose safety can be shown is run on them.
pytestmark = [pytest.mark.gpu, pytest.mark.skip(reason="the multi-segment form of the fast kernel "
                                                         "these cases were written for faulted the GPU once "
                                                         "with no cause found; that form is removed")]


@pytest.fixture(scope="module")
def gdr():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gated_delta_rule_70_amd import binding
    binding.lib()  # raises if the library is missing: there is no fallback
    return binding


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _lengths(n, lo, hi, seed, tail=(30, 5)):
    """n segment lengths in [lo, hi] (a fifth of them empty), then `tail`."""
    g = torch.Generator().manual_seed(seed)
    ls = torch.randint(lo, hi + 1, (n,), generator=g)
    ls[torch.rand(n, generator=g) < 0.2] = 0
    return ls.tolist() + list(tail)


def _run(gdr, case, read="post", out=None, accumulate=False, hT=None):
    d = lambda t: None if t is None else t.cuda()
    o, h = gdr.chunk_fwd(d(case.q), d(case.k), d(case.v), d(case.log_alpha), d(case.beta), hT if hT is not None
                         else d(case.h0), d(case.cu_seqlens), chunk=64, read=read, out=out, accumulate=accumulate,
                         hT=hT)
    torch.cuda.synchronize()
    return o, h


CASES = {
    # name: (segments, lo, hi, Hk, Hv, dv, seed); that form would have put 9, 5, 48 and 6
    # segments in one workgroup
    "600seg-0..150-gqa1x2-dv128": (600, 0, 150, 1, 2, 128, 51),
    "3000seg-0..40-dv32": (3000, 0, 40, 1, 1, 32, 52),
    "2048seg-16..48-H4-dv128": (2048, 16, 48, 4, 4, 128, 53),
    "400seg-1..300-gqa2x4-dv64": (400, 1, 300, 2, 4, 64, 54),
}


@pytest.mark.parametrize("read", ["post", "pre"])
@pytest.mark.parametrize("name", list(CASES))
def test_many_short_segments(gdr, name, read):
    nseg, lo, hi, Hk, Hv, dv, seed = CASES[name]
    lengths = _lengths(nseg, lo, hi, seed)
    case = inputs.chunk_case(Hk=Hk, Hv=Hv, dk=128, dv=dv, dtype=torch.bfloat16, seed=seed, h0_std=0.1,
                             regime="slow", lengths=lengths)
    _say("short segments %s read=%s: %d segments, T=%d" % (name, read, len(lengths), case.q.shape[2]))
    o, h = _run(gdr, case, read)
    ro, rh = oracle.scan(case.q, case.k, case.v, case.log_alpha, case.beta, case.h0, case.cu_seqlens, read=read)
    segs = segments(tuple(o.shape), case.cu_seqlens)
    eo = check_bf16_detailed(gpu_np(o), ro, segs, "o")
    eh = check_states(gpu_np(h), rh, "hT")
    _say("  o: whole %.2e, worst block %.2e, chunk-last rows %.2e; hT: whole %.2e, worst unit %.2e" % (eo + eh))


def test_short_segments_zero_h0_accumulate_inplace(gdr):
    """No initial state (zeros); then out += o with the final state written over h0 in place."""
    lengths = _lengths(700, 0, 90, 55)
    case = inputs.chunk_case(Hk=1, Hv=2, dk=128, dv=128, dtype=torch.bfloat16, seed=55, h0_std=0.1,
                             regime="p5", lengths=lengths)
    h0 = case.h0
    case.h0 = None
    o, h = _run(gdr, case)
    ro, rh = oracle.scan(case.q, case.k, case.v, case.log_alpha, case.beta, None, case.cu_seqlens)
    check(gpu_np(o), ro, torch.bfloat16, "zero h0 o")
    check_states(gpu_np(h), rh, "zero h0 hT")
    # accumulate into a base tensor, final state in place over h0
    case.h0 = h0
    base = torch.randn(tuple(case.v.shape), generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    out = base.cuda()
    state = h0.cuda()
    o2, h2 = _run(gdr, case, out=out, accumulate=True, hT=state)
    ro2, rh2 = oracle.scan(case.q, case.k, case.v, case.log_alpha, case.beta, h0, case.cu_seqlens)
    check(gpu_np(o2), ro2 + base.double().numpy(), torch.bfloat16, "accumulate o")
    check_states(gpu_np(h2), rh2, "in-place hT")
    assert h2.data_ptr() == state.data_ptr()


def test_short_segments_all_empty_tail_group(gdr):
    """The last workgroup's segments are all empty: their final states are their initial
    states, and no chunk runs there."""
    lengths = _lengths(800, 1, 60, 56, tail=()) + [0] * 60
    case = inputs.chunk_case(Hk=1, Hv=2, dk=128, dv=64, dtype=torch.bfloat16, seed=56, h0_std=0.1,
                             regime="slow", lengths=lengths)
    o, h = _run(gdr, case)
    ro, rh = oracle.scan(case.q, case.k, case.v, case.log_alpha, case.beta, case.h0, case.cu_seqlens)
    check(gpu_np(o), ro, torch.bfloat16, "o")
    check_states(gpu_np(h), rh, "hT")
    assert np.array_equal(gpu_np(h)[-60:], case.h0.double().numpy()[-60:])
