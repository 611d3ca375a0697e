"""fp64 CPU oracle of the large-chunk TTT layer. Test infrastructure only (tests, the
smoke check and the benchmark's CPU-baseline leg); the HIP library never imports it."""
from .ttt_oracle import *  # noqa: F401,F403
from .ttt_oracle import (MUON_COEFFS, NS_EPS, apply_vjp, chunk_gradient, chunk_loss, forward_all,  # noqa: F401
                         fw_apply, newton_schulz5, renorm_rows, sequence_forward,
                         sequence_forward_bruteforce, update_state)
