"""Decode workload definitions.

Each workload fixes the per-step shapes (B sequences, H heads, d_v x d_k state
per head), the horizon T, the delta switch of the general recurrence, the decay
and write-gate distributions, the input dtype and the per-head precision tiers.
The recurrence and its constraints (unit-norm q and k, beta in (0, 2), decay in
(0, 1], delta in {0, 1}) are those of "Quantizing Recurrent Language Models Is
Easier Than You Think", Introduction, general recurrence form.

Precision codes match the C ABI: 0 = fp32, 1 = bf16, 2 = int8, 3 = int4, 4 = int6.
Tiers are listed slowest-decaying first, as (fraction of heads, precision).
"""
from dataclasses import dataclass, field

PREC_FP32, PREC_BF16, PREC_INT8, PREC_INT4, PREC_INT6 = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    key: str
    name: str
    B: int
    H: int
    dk: int
    dv: int
    T: int
    delta: int
    decay: str            # "softplus_step" | "uniform_head" | "ssd" | "kda_channel"
    in_bf16: bool = False
    alpha_lo: float = 0.0
    alpha_hi: float = 1.0
    tiers: tuple = ((1.0, PREC_INT8),)
    seeds: tuple = (0,)

    @property
    def per_channel(self) -> bool:
        return self.decay == "kda_channel"

    def scaled(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    # Tiny gated delta rule, small enough for the oracle to run every step.
    "C1": Workload("C1", "gdn-tiny-int8", B=1, H=2, dk=64, dv=64, T=128, delta=1,
                   decay="softplus_step"),
    # Gated-DeltaNet decode shape of a 9B-class hybrid layer; bf16 activations.
    "C2": Workload("C2", "gdn-b64-h32-d128-int8", B=64, H=32, dk=128, dv=128, T=1024,
                   delta=1, decay="uniform_head", in_bf16=True, alpha_lo=0.85, alpha_hi=1.0),
    # Mamba-2 / SSD decode: no delta correction, decay exp(-dt*A), write gate dt.
    "C3": Workload("C3", "ssd-b256-h128-dv64-dk128-int8", B=256, H=128, dk=128, dv=64,
                   T=512, delta=0, decay="ssd"),
    # KDA-style per-channel (key-axis) decay; slowest 25% of heads kept in bf16.
    "C4": Workload("C4", "kda-b128-h32-d128-bf16+int8", B=128, H=32, dk=128, dv=128,
                   T=1024, delta=1, decay="kda_channel",
                   tiers=((0.25, PREC_BF16), (0.75, PREC_INT8))),
    # Large-batch mixed low-bit sweep: fastest-decaying half of the heads in int4.
    "C5": Workload("C5", "gdn-b2048-h32-d128-int8+int4", B=2048, H=32, dk=128, dv=128,
                   T=64, delta=1, decay="uniform_head", alpha_lo=0.7, alpha_hi=1.0,
                   tiers=((0.5, PREC_INT8), (0.5, PREC_INT4)), seeds=tuple(range(8))),
    # The same shape with the slowest-decaying half in int6 instead of int8:
    # the int4 / int6 mix, 5.25 bits per element with the row scales.
    "C5i6": Workload("C5i6", "gdn-b2048-h32-d128-int6+int4", B=2048, H=32, dk=128, dv=128,
                     T=64, delta=1, decay="uniform_head", alpha_lo=0.7, alpha_hi=1.0,
                     tiers=((0.5, PREC_INT6), (0.5, PREC_INT4))),
}


def get_workload(key: str) -> Workload:
    return WORKLOADS[key]
