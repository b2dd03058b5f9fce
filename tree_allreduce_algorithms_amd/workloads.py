"""Seeded synthetic inputs for the collectives: the workloads and their recipe.

This module only draws random numbers.  It holds none of the collectives'
arithmetic, imports neither the HIP binding nor the CPU checker, and is the one
piece of code that the tests, the bench and the checker all share.

Workloads (N logical ranks, T elements per rank; every rank draws from its own
stream):

* ``small_int32``: N=4, T=1024 int32, uniform integers in [-100, 100].
* ``ddp_bucket``: N=8, T=6,553,600 float32 (a 25 MB bucket), Normal(0, 1e-3).
* ``large_grad_fp32``: N=8, T=300,000,000 float32 (1.2 GB per rank), Normal(0, 1e-3).
* ``large_grad_bf16``: the same draw rounded to bfloat16 (nearest-even).
* ``sweep_<T>``: N=4 float32 uniform in [-1, 1), T in {256, 262144, 4194304, 67108864}.
* ``zero_n64``: N=64, T=16,777,217 float32 Normal(0, 1) (N does not divide T).
* ``moe_alltoall``: N=8, T=33,554,432 float32 Normal(0, 1): the AllToAll of an
  expert-parallel token exchange, 8 blocks of 16 MiB per rank.

Host draws use ``numpy.random.default_rng([seed, rank])``.  Device draws (for
the sizes where a host draw plus upload would dominate a run) use a
``torch.Generator`` on the device seeded with ``seed * 1_000_003 + rank``;
they are a different stream of the same distribution.  "1e-3" is the standard
deviation; the integer range includes both ends; the uniform range is
half-open.
"""

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    nranks: int
    count: int
    dtype: str            # "int32" | "float32" | "bfloat16"
    dist: str             # "int_uniform" | "normal" | "uniform_pm1"
    seed: int
    params: dict = field(default_factory=dict)

    @property
    def itemsize(self):
        return 2 if self.dtype == "bfloat16" else 4

    @property
    def rank_bytes(self):
        return self.count * self.itemsize


SWEEP_COUNTS = (256, 262_144, 4_194_304, 67_108_864)

WORKLOADS = {
    "small_int32": Workload("small_int32", 4, 1024, "int32", "int_uniform", 1,
                            {"lo": -100, "hi": 100}),
    "ddp_bucket": Workload("ddp_bucket", 8, 6_553_600, "float32", "normal", 2, {"std": 1e-3}),
    "large_grad_fp32": Workload("large_grad_fp32", 8, 300_000_000, "float32", "normal", 3,
                                {"std": 1e-3}),
    "large_grad_bf16": Workload("large_grad_bf16", 8, 300_000_000, "bfloat16", "normal", 3,
                                {"std": 1e-3}),
    "zero_n64": Workload("zero_n64", 64, 16_777_217, "float32", "normal", 5, {"std": 1.0}),
    "moe_alltoall": Workload("moe_alltoall", 8, 33_554_432, "float32", "normal", 6, {"std": 1.0}),
}
for _t in SWEEP_COUNTS:
    WORKLOADS[f"sweep_{_t}"] = Workload(f"sweep_{_t}", 4, _t, "float32", "uniform_pm1", 4)


def _bf16_bits_from_f32(x):
    """float32 -> bfloat16 bit patterns via torch's CPU conversion (nearest-even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def host_rank(dist, dtype, count, seed, rank, params=None):
    """One rank's input as a NumPy array (bfloat16 as uint16 bit patterns)."""
    params = params or {}
    rng = np.random.default_rng([seed, rank])
    if dist == "int_uniform":
        if dtype != "int32":
            raise ValueError("int_uniform draws int32")
        return rng.integers(params.get("lo", -100), params.get("hi", 100), size=count,
                            endpoint=True, dtype=np.int32)
    if dist == "normal":
        x = rng.standard_normal(count, dtype=np.float32) * np.float32(params.get("std", 1.0))
    elif dist == "uniform_pm1":
        x = rng.random(count, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    if dtype == "float32":
        return x
    if dtype == "bfloat16":
        return _bf16_bits_from_f32(x)
    raise ValueError(f"{dist} cannot draw {dtype}")


def host_inputs(nranks, count, dtype, dist, seed, params=None):
    """N independent rank inputs drawn on the host."""
    return [host_rank(dist, dtype, count, seed, r, params) for r in range(nranks)]


def workload_host_inputs(w: Workload, count=None):
    return host_inputs(w.nranks, w.count if count is None else count, w.dtype, w.dist,
                       w.seed, w.params)


def device_rank(dist, dtype, count, seed, rank, device, params=None, out=None):
    """One rank's input drawn on the device with torch's generator.

    Returns a torch tensor of the storage dtype (torch.bfloat16 for bfloat16).
    ``out`` may be a preallocated tensor of that dtype and size to fill.
    """
    import torch
    params = params or {}
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 1_000_003 + rank)
    tdt = {"int32": torch.int32, "float32": torch.float32, "bfloat16": torch.bfloat16}[dtype]
    if dist == "int_uniform":
        x = torch.randint(params.get("lo", -100), params.get("hi", 100) + 1, (count,),
                          generator=gen, device=device, dtype=torch.int32)
    elif dist == "normal":
        x = torch.randn(count, generator=gen, device=device, dtype=torch.float32)
        x.mul_(params.get("std", 1.0))
    elif dist == "uniform_pm1":
        x = torch.rand(count, generator=gen, device=device, dtype=torch.float32)
        x.mul_(2.0).sub_(1.0)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    if x.dtype != tdt:
        x = x.to(tdt)
    if out is not None:
        out.copy_(x)
        return out
    return x


def device_inputs(nranks, count, dtype, dist, seed, device, params=None):
    return [device_rank(dist, dtype, count, seed, r, device, params) for r in range(nranks)]
