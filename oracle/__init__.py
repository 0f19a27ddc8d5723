"""CPU float64 oracle of the OneLA large-beam GDN decode step.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's CPU
baseline leg may import or call anything in this package; the product path
(the HIP library and its binding) never does, and shares no code with it.

It is the plain definition of what the step computes, written out slowly in
float64 numpy: every beam keeps a full d_v x d_k state and follows its parent
pointers directly. The method's projection replay is written out separately
(`replay_episode`) so that tests can pin it against that definition.

Pins (tests/test_oracle_pins.py): a hand-worked scalar example, the identity
and pure-decay closed forms along parent paths, the delta-rule product form,
the write-back property, exact associative recall with orthonormal keys,
affinity in S0, beam-relabelling equivariance, replay == full state, a
brute-force ancestry walk, and closed forms of the input-side gates and
normalisation (`fused_inputs`, `unit_rows`). No function here is "parity
unpinned".
"""
from .gdn import (  # noqa: F401
    ancestry_walk,
    full_state_episode,
    fused_inputs,
    prompt_state,
    replay_episode,
    unit_rows,
)
