"""The oracle's validator against the refusals the pages list (CPU only)."""
import pytest

import oracle as O
from validator_cases import CASES


def to_oracle(members):
    out = []
    for m in members:
        w = m["weight"]
        si, s = m["scale_inv"], m["scale"]
        out.append(O.MemberDesc(O.TensorDesc(w["dtype"], w["shape"], w["addr"]),
                                None if si is None else O.TensorDesc(si["dtype"], si["shape"], si["addr"]),
                                None if s is None else O.TensorDesc(s["dtype"], s["shape"], s["addr"])))
    return out


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_validate(case):
    _, qm, block, members, want = case
    assert O.validate(qm, block, to_oracle(members)) == want


def test_every_refusal_name_is_reachable():
    names = {c[4] for c in CASES}
    listed = {v for k, v in vars(O.Status).items() if not k.startswith("_")}
    assert listed - {"INVALID_ARG"} <= names
