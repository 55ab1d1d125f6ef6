"""CPU oracle for KDA: test infrastructure, never part of the product path.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import anything under this directory.
"""
from .kda_oracle import (kda_recurrence, kda_decode_step, gdn_recurrence,  # noqa: F401
                         gdn_decode_step, as_f64)
from .kda_prologue import (QK_AS_GIVEN, QK_L2, QK_SILU_L2, kda_prologue,  # noqa: F401
                           kda_recurrence_logits, kda_decode_step_logits)
from .kda_backward import (gdn_decode_step_backward, gdn_prefill_backward,  # noqa: F401
                           kda_decode_step_backward,
                           kda_prefill_backward, kda_prefill_backward_logits,
                           kda_prologue_backward)
