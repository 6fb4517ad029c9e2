"""The five synthetic workloads (shapes, seeds and the sink/scale/order cases).

Q, K and V are i.i.d. N(0,1) rounded to bf16; the bias puts ``delta`` on keys
0..3.  Seeds are fixed per workload so every run sees the same bytes.
The Sweep workload stands in for the P-cast paper's "kernel-faithful"
simulation at N = 4096 (results section), whose head count, head size and
seeds the summaries do not state.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    seed: int
    # (delta, S, order) cases; order 0 = forward, 1 = reverse; S = 0 is the bf16 path
    cases: tuple = field(default_factory=tuple)

    @property
    def pairs(self) -> int:
        """Unmasked (query, key) pairs over all heads."""
        per_head = self.N * (self.N + 1) // 2 if self.causal else self.N * self.N
        return self.B * self.Hq * per_head

    @property
    def flops(self) -> float:
        """Algorithmic flops, FlashAttention convention: 4*B*H*N^2*d, halved when causal."""
        f = 4.0 * self.B * self.Hq * self.N * self.N * self.d
        return f / 2 if self.causal else f


_SWEEP_S = tuple(float(2 ** k) for k in range(10)) + (448.0,)

WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 1024, 64, False, 1,
                     tuple((7.0, s, 0) for s in (1.0, 256.0, 448.0, 0.0))),
    "sweep": Workload("sweep", 1, 8, 8, 4096, 128, True, 2,
                      tuple((float(dl), s, o) for dl in range(11) for s in _SWEEP_S for o in (0, 1))),
    "throughput": Workload("throughput", 4, 32, 32, 8192, 128, True, 3,
                           ((7.0, 256.0, 1), (7.0, 1.0, 0), (7.0, 0.0, 0))),
    "gqa": Workload("gqa", 1, 32, 8, 65536, 128, True, 4,
                    ((7.0, 256.0, 1), (7.0, 448.0, 0))),
    "long": Workload("long", 1, 16, 4, 131072, 128, True, 5,
                     tuple((dl, 256.0, o) for dl in (5.0, 7.0, 9.0) for o in (0, 1))),
}


@dataclass(frozen=True)
class DecodeWorkload:
    """Decode with split KV: Nq new query rows per sequence against Nk cached keys,
    the keys cut into ranges of split_keys."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    split_keys: int
    seed: int
    cases: tuple = field(default_factory=tuple)

    @property
    def flops(self) -> float:
        """4 * d flops per visible (query, key) pair (rows at the last Nq positions)."""
        pairs = self.Nq * self.Nk - self.Nq * (self.Nq - 1) // 2
        return 4.0 * self.B * self.Hq * pairs * self.d

    @property
    def bytes(self) -> int:
        """Compulsory HBM bytes of one call: Q and K (bf16) and the E4M3 V copy read
        once, out (fp32) written once."""
        return self.B * (self.Hq * self.Nq * self.d * (2 + 4) + self.Hkv * self.Nk * self.d * (2 + 1))

    @property
    def bytes_qk8(self) -> int:
        """The same with FP8 logits: K read as E4M3 codes (1 byte) plus one exponent
        (4 bytes) per 64-key block."""
        return self.B * (self.Hq * self.Nq * self.d * (2 + 4) + self.Hkv * self.Nk * self.d * (1 + 1)
                         + self.Hkv * (self.Nk // 64) * 4)


DECODE_WORKLOADS = {
    # one new token for each of 16 sequences of 16k cached keys, GQA 32 / 8; ranges of
    # 2048 keys make 16 * 8 * 8 = 1024 split workgroups, one wave for each SIMD of 256 CUs
    "decode": DecodeWorkload("decode", 16, 32, 8, 1, 16384, 128, 2048, 6,
                             ((7.0, 256.0, 1), (7.0, 1.0, 0))),
    # four new tokens of one 128k-key sequence
    "decode_long": DecodeWorkload("decode_long", 1, 32, 8, 4, 131072, 128, 4096, 7,
                                  ((7.0, 256.0, 1),)),
}
