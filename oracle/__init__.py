"""CPU oracle (test infrastructure only; see disco_oracle)."""
from .disco_oracle import *  # noqa: F401,F403
from .disco_oracle import Desc, PsiCSR, psi, psi_row, contract, einsum, forward  # noqa: F401
