"""The five synthetic workloads, by shape.

1  tiny causal MHA, fp32, one unpadded segment (small enough for the oracle
   to finish in a fraction of a second);
2  packed THD with padding and GQA: B=2, T=4096, 4 slots of 1024 tokens
   (768 valid, 256 padding), 16 query / 2 K/V heads, D=128, bf16, causal;
3  workload 2 split by the dual-chunk causal load-balancing reorder into
   4 sequence shards, each shard attending to the 4 K/V chunks in ring order
   and merging the partial results;
4  causal sliding-window GQA: B=1, T=32768, one segment, 64 query / 8 K/V
   heads, D=128, bf16, window (4096, 0);
5  one device's share of the tutorial's long-context case: B=2, T=65536 per
   row as 4 slots of 16384 (12288 valid + 4096 padding), 128 query / 8 K/V
   heads, D=128, bf16, causal with window (8192, 0), dual-chunk reorder for
   4 shards, each shard computed as 4 ring steps with merges.

Workload 5 is the tutorial's long-context case (TransformerEngine JAX
"Context-Parallel Attention" tutorial, sections 1 and 3: batch 2, seq 65536,
128/8 heads, head_dim 128, window (8192, 0), padding+causal mask).
"""

from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    batch: int
    seq_len: int            # tokens per batch row, before any sharding
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str              # "bf16" or "f32" for Q, K, V
    causal: bool
    window: tuple           # (left, right); -1 means unbounded
    slots: int              # segment slots per row
    valid_per_slot: int     # valid tokens at the start of each slot
    cp_size: int = 1        # sequence shards (1 = unsplit)
    reorder: str = "none"   # "none" | "dual_chunk" | "striped"
    stripe: int = 1
    seed: int = field(default=0)
    v_head_dim: int = 0     # head dim of V and O; 0 = head_dim

    @property
    def slot_len(self) -> int:
        return self.seq_len // self.slots

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return self.head_dim ** -0.5

    @property
    def dv(self) -> int:
        return self.v_head_dim or self.head_dim

    def describe(self) -> str:
        w = self.window
        dims = f"D{self.head_dim}" + (f"/Dv{self.dv}" if self.dv != self.head_dim else "")
        s = (f"B{self.batch} T{self.seq_len} Hq{self.num_q_heads}/Hkv{self.num_kv_heads} "
             f"{dims} {self.dtype} {'causal' if self.causal else 'full'} "
             f"window({w[0]},{w[1]}) {self.slots}x({self.valid_per_slot} valid + "
             f"{self.slot_len - self.valid_per_slot} pad)")
        if self.cp_size > 1:
            s += f" {self.reorder} reorder, {self.cp_size} shards x {self.cp_size} ring steps"
        return s


CONFIGS = {
    1: Workload(1, "tiny_causal_mha_f32", 1, 256, 4, 4, 64, "f32", True, (-1, -1),
                1, 256, seed=2027),
    2: Workload(2, "packed_thd_gqa_bf16", 2, 4096, 16, 2, 128, "bf16", True, (-1, -1),
                4, 768, seed=2028),
    3: Workload(3, "ring4_packed_thd_gqa_bf16", 2, 4096, 16, 2, 128, "bf16", True, (-1, -1),
                4, 768, cp_size=4, reorder="dual_chunk", seed=2028),
    4: Workload(4, "causal_swa4096_gqa_bf16", 1, 32768, 64, 8, 128, "bf16", True, (4096, 0),
                1, 32768, seed=2030),
    5: Workload(5, "ring4_longctx_swa8192_gqa_bf16", 2, 65536, 128, 8, 128, "bf16", True,
                (8192, 0), 4, 12288, cp_size=4, reorder="dual_chunk", seed=2031),
    # DeepSeek-style MLA head dimensions (query/key 192 = 128 + 64 rotary, value
    # 128), named by the tutorial's "Next steps" for single-GPU attention; the
    # sizes are this suite's choice: one causal 8192-token segment per row,
    # 128 heads with their own K/V (the decompressed form of MLA).
    6: Workload(6, "mla_causal_bf16", 2, 8192, 128, 128, 192, "bf16", True, (-1, -1),
                1, 8192, seed=2032, v_head_dim=128),
}


def get(cfg: int) -> Workload:
    return CONFIGS[int(cfg)]
