"""Dynamic loss scaler (oracle).

Test infrastructure only (see ``oracle/__init__``).

Page "혼합 정밀도 학습" (itwiki), section "손실 스케일링", and page "Mixed
Precision Training/es" (marovi), section "Escalado dinámico de pérdida": start
at a large scale (2^16); every step check the gradients for inf/NaN; on
overflow skip the weight update and halve the scale; after a fixed number of
clean steps (2000) double it.  GradScaler defaults quoted on the itwiki page:
init 65536, growth 2, backoff 0.5, interval 2000.

Readings: there is no floor or ceiling on the scale (marovi "Limitaciones y
modos de fallo" describes collapse to one as a symptom, not a clamp); the
growth counter restarts at 0 after an overflow and after each growth.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import formats as F


@dataclass
class ScalerState:
    scale: float = 65536.0
    growth_tracker: int = 0


def update(st: ScalerState, found_inf: bool, growth_factor: float = 2.0,
           backoff_factor: float = 0.5, growth_interval: int = 2000) -> ScalerState:
    if found_inf:
        st.scale = float(F.f32(st.scale * float(F.f32(backoff_factor))))
        st.growth_tracker = 0
    else:
        st.growth_tracker += 1
        if st.growth_tracker == growth_interval:
            st.scale = float(F.f32(st.scale * float(F.f32(growth_factor))))
            st.growth_tracker = 0
    return st
