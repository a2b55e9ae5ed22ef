"""The five workload shapes of the TP-shard MLP and their value distributions.

Each config names the full FFN (hidden h, FFN width F), the TP degree P and
the number of tokens T = micro-batch x sequence length. One TP rank owns the
column block A_i = A[:, i*f:(i+1)*f], the bias block b1_i and the row block
B_i = B[i*f:(i+1)*f, :], with f = F / P (the tensor-parallel split of the
FFN's two linears: column split for the first, row split for the second, as
in "Understanding the Megatron-LM architecture: how 3D parallelism assigns
roles", section 1).

Where the pages leave a size open, the reading is:
  * FFN width F = 4h for every config.
  * "tiny": h=128, T=2x32 tokens, TP 2, fp32; both shards are emulated.
  * "gpt2_small": h=768 (GPT-2 117M, "Training GPT-2 with Megatron-LM",
    section 4.2 table), context 1024 (section 6.1), TP 1, fp16.
  * "gpt_2p4b": hidden 2560, seq 2048, micro-batch 4 (section 4.1), one
    shard of TP 4, bf16.
  * "gpt_7b": h=4096 (the 4096-dim FFN of section 1), TP 4 (section 5.1),
    seq 2048, micro-batch 4, fp16.
  * "gpt_h10240": hidden 10240, TP 4, micro-batch 8 (tbr8.org practical
    example), seq 2048, bf16.
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class Config:
    name: str
    dtype: str          # storage dtype: "f32", "f16" or "bf16"
    micro_batch: int
    seq_len: int
    hidden: int
    ffn: int            # full FFN width F (all TP ranks together)
    tp: int             # TP degree P
    sigma_x: float
    sigma_w: float
    sigma_b: float
    sigma_dy: float
    seed: int = 0
    all_shards: bool = False  # draw full A, b1, B and emulate every shard

    @property
    def tokens(self) -> int:
        return self.micro_batch * self.seq_len

    @property
    def ffn_shard(self) -> int:
        return shard_width(self.ffn, self.tp)


def shard_width(ffn: int, tp: int) -> int:
    if ffn % tp:
        raise ValueError(f"FFN width {ffn} is not divisible by TP degree {tp}")
    return ffn // tp


CONFIGS = {
    c.name: c
    for c in [
        Config("tiny", "f32", 2, 32, 128, 512, 2, 1.0, 0.02, 0.01, 1.0, all_shards=True),
        Config("gpt2_small", "f16", 4, 1024, 768, 3072, 1, 1.0, 0.02, 0.01, 0.01),
        Config("gpt_2p4b", "bf16", 4, 2048, 2560, 10240, 4, 1.0, 0.02, 0.01, 0.01),
        Config("gpt_7b", "f16", 4, 2048, 4096, 16384, 4, 1.0, 0.02, 0.01, 0.01),
        Config("gpt_h10240", "bf16", 8, 2048, 10240, 40960, 4, 1.0, 0.02, 0.01, 0.01),
    ]
}


def get_config(name: str) -> Config:
    return CONFIGS[name]


@dataclass(frozen=True)
class AttnConfig:
    """Self-attention workload: n heads of width d = hidden / n over
    micro-batch x seq tokens; one TP rank owns n / P heads."""
    name: str
    dtype: str
    micro_batch: int
    seq_len: int
    hidden: int
    heads: int          # all heads (all TP ranks together)
    tp: int
    causal: bool = True
    sigma_x: float = 1.0
    sigma_w: float = 0.02
    sigma_b: float = 0.01
    sigma_dy: float = 0.01
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.micro_batch * self.seq_len

    @property
    def head_dim(self) -> int:
        return self.hidden // self.heads

    @property
    def heads_shard(self) -> int:
        if self.heads % self.tp:
            raise ValueError(f"{self.heads} heads are not divisible by TP degree {self.tp}")
        return self.heads // self.tp


# The 2.4B run prints hidden 2560, 32 attention heads, seq 2048 and
# micro-batch 4 ("Training GPT-2 with Megatron-LM", section 4.1); one rank
# of TP 4 (as for its MLP) owns 8 heads of width 80. The small case keeps the
# same structure at sizes the oracle finishes in milliseconds.
ATTN_CONFIGS = {
    c.name: c
    for c in [
        AttnConfig("attn_small", "f16", 2, 64, 128, 4, 2, sigma_dy=1.0),
        AttnConfig("attn_2p4b", "bf16", 4, 2048, 2560, 32, 4),
    ]
}


def get_attn_config(name: str) -> AttnConfig:
    return ATTN_CONFIGS[name]
