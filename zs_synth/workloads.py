"""The five synthetic workloads of the per-shard step, as plain data.

Sizes and distributions are the pages' sizing case (7.5B parameters on 64
GPUs) plus model-shaped parameter lists; the values are synthetic.  Only
shapes and generator recipes live here: shard bounds come from the caller.
"""

from __future__ import annotations

from dataclasses import dataclass, field


def gpt2_small_tensors() -> list[tuple[str, int]]:
    """GPT-2-small parameter list, flattened in this order: wte, wpe, then per
    layer c_attn.w, c_proj.w, fc.w, proj.w, their four biases, ln1 gamma/beta,
    ln2 gamma/beta; then the final LayerNorm.  148 tensors, 124,439,808 values."""
    d, ff, vocab, ctx = 768, 3072, 50257, 1024
    out = [("wte", vocab * d), ("wpe", ctx * d)]
    for i in range(12):
        p = f"h.{i}."
        out += [
            (p + "attn.c_attn.w", d * 3 * d),
            (p + "attn.c_proj.w", d * d),
            (p + "mlp.c_fc.w", d * ff),
            (p + "mlp.c_proj.w", ff * d),
            (p + "attn.c_attn.b", 3 * d),
            (p + "attn.c_proj.b", d),
            (p + "mlp.c_fc.b", ff),
            (p + "mlp.c_proj.b", d),
            (p + "ln_1.g", d),
            (p + "ln_1.b", d),
            (p + "ln_2.g", d),
            (p + "ln_2.b", d),
        ]
    out += [("ln_f.g", d), ("ln_f.b", d)]
    return out


def llama3_8b_tensors() -> list[tuple[str, int]]:
    """Llama-3-8B parameter list: embed, 32 x [q, k, v, o, gate, up, down,
    attn_norm, ffn_norm], final norm, untied lm_head.  291 tensors,
    8,030,261,248 values."""
    d, kv, ff, vocab = 4096, 1024, 14336, 128256
    out = [("embed", vocab * d)]
    for i in range(32):
        p = f"layers.{i}."
        out += [
            (p + "q", d * d),
            (p + "k", d * kv),
            (p + "v", d * kv),
            (p + "o", d * d),
            (p + "gate", d * ff),
            (p + "up", d * ff),
            (p + "down", ff * d),
            (p + "attn_norm", d),
            (p + "ffn_norm", d),
        ]
    out += [("norm", d), ("lm_head", vocab * d)]
    return out


@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    n: int                      # parameters in the flattened model, N
    p: int                      # data-parallel ranks, P
    shards: tuple               # ranks k whose step is run
    grad_dtype: str             # "f16" or "bf16" (rank-local gradients)
    param_dtype: str            # "f16" or "bf16" (working copy)
    steps: int
    form: str                   # "standard" or "page1_literal"
    grad_kind: str              # "normal" or "edge"
    grad_std: float             # standard deviation for grad_kind "normal"
    grad_layout: str            # "full": P buffers of N; "slice": P buffers of the shard only
    param_layout: str           # "full": one buffer of N; "tensors": one buffer per tensor
    w_std: float = 0.02
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    tensors: tuple = field(default=(), repr=False)   # ((name, numel), ...) or ()
    # edge workload only
    zero_frac: float = 0.0
    const_block: int = 0
    edge_lo: float = 0.0
    edge_hi: float = 0.0


def _const_value(k: int) -> float:
    """Constant gradient of shard k's constant block: (-1)^k * 10^((k mod 11) - 8),
    spanning 1e-8 .. 1e2 (rounded to the gradient dtype by the caller)."""
    return (-1.0) ** k * 10.0 ** ((k % 11) - 8)


WORKLOADS = {
    "tiny_p4": Workload(
        name="tiny_p4",
        description="N=1,000,003 fp32 params, P=4 (last shard short), fp16 grads ~N(0,1e-2), "
                    "all 4 shards, 3 steps, standard Adam",
        n=1_000_003, p=4, shards=(0, 1, 2, 3), grad_dtype="f16", param_dtype="f16", steps=3,
        form="standard", grad_kind="normal", grad_std=1e-2, grad_layout="full",
        param_layout="full"),
    "gpt2_small_p8": Workload(
        name="gpt2_small_p8",
        description="GPT-2-small parameter list (124,439,808 values, 148 tensors), P=8, shard 0 "
                    "via the chunk table, bf16 grads ~N(0,1e-3), 10 steps",
        n=124_439_808, p=8, shards=(0,), grad_dtype="bf16", param_dtype="bf16", steps=10,
        form="standard", grad_kind="normal", grad_std=1e-3, grad_layout="slice",
        param_layout="tensors", tensors=tuple(gpt2_small_tensors())),
    "zero_7p5b_p64": Workload(
        name="zero_7p5b_p64",
        description="7.5B-parameter model at P=64: one shard of M=117,187,500 (rank 63), "
                    "64 fp16 grad slices ~N(0,1e-3), fp16 param buffer of all 7.5e9, 5 steps",
        n=7_500_000_000, p=64, shards=(63,), grad_dtype="f16", param_dtype="f16", steps=5,
        form="standard", grad_kind="normal", grad_std=1e-3, grad_layout="slice",
        param_layout="full"),
    "llama3_8b_p8": Workload(
        name="llama3_8b_p8",
        description="Llama-3-8B parameter list (8,030,261,248 values, 291 tensors), P=8, shard 3 "
                    "(1,003,782,656 values, 42 tensor pieces), bf16 grads ~N(0,1e-3), 5 steps",
        n=8_030_261_248, p=8, shards=(3,), grad_dtype="bf16", param_dtype="bf16", steps=5,
        form="standard", grad_kind="normal", grad_std=1e-3, grad_layout="slice",
        param_layout="tensors", tensors=tuple(llama3_8b_tensors())),
    "edge_p16_literal": Workload(
        name="edge_p16_literal",
        description="N=100,000,007, P=16, all shards, bf16 grads |g|=10^U(-8,2) with random sign, "
                    "5% shared exact zeros, constant block of 65,536 per shard, page-1 literal "
                    "Adam, 20 steps",
        n=100_000_007, p=16, shards=tuple(range(16)), grad_dtype="bf16", param_dtype="bf16",
        steps=20, form="page1_literal", grad_kind="edge", grad_std=0.0, grad_layout="full",
        param_layout="full", zero_frac=0.05, const_block=65_536, edge_lo=1e-8, edge_hi=1e2),
}


const_value = _const_value
