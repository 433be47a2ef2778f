"""CPU oracle for the Sign-Muon step (test infrastructure, NumPy only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package; the HIP library never does.
"""
from .signmuon_oracle import *  # noqa: F401,F403
from .signmuon_oracle import (CUBIC, SCALE_FRO, SCALE_SPECTRAL,  # noqa: F401
                              apply_update, bf16_round_nearest_even,
                              frobenius_scale, majority_from_sums,
                              momentum_update, newton_schulz, normalized_sign, pack_signs,
                              polar_ns, polar_svd, prescale, sign_ternary,
                              spectral_scale, step, unpack_signs,
                              vote_sums_from_bits, vote_sums_from_signs,
                              vote_sums_int8_wrapping, weight_decayed_gradient,
                              worker_direction)
