"""CPU fp64 oracle of the decoder-block training step.

TEST INFRASTRUCTURE ONLY.  Only `tests/`, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` may import this package.  It shares no code
with the HIP path (`gpt_decoder_block_amd`), and neither imports the other;
the seeded draws in `seeded_inputs` are the only common module.

Every function is the plain definition written out in numpy float64, forward
plus a hand-written backward by the chain rule; see `oracle.reference` for the
passages each one follows and for the pins that tie it to something other than
itself (the tests under `tests/test_oracle_*.py`).
"""
from .reference import *  # noqa: F401,F403
from .optim import *  # noqa: F401,F403
