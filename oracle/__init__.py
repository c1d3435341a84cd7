"""CPU oracle of the DFlash draft round (test infrastructure only; see dflash_oracle)."""
from . import dflash_oracle  # noqa: F401
