"""Synthetic paged-decode workloads described as data.

A workload is a model shape plus an ordered list of block-manager operations:

* ``("add", seq)``                       register an empty sequence;
* ``("append", seq_ids, counts)``        append ``counts[i]`` tokens to
                                         ``seq_ids[i]`` (one all-or-nothing batch,
                                         sequence-major, in the given order); every
                                         appended token gets K/V rows in every layer;
* ``("fork", parent, child)``            the child shares the parent's blocks;
* ``("decode", seq_ids)``                one query per listed sequence per layer;
* ``("prefill", seq_ids, counts)``       append ``counts[i]`` tokens to ``seq_ids[i]``
                                         exactly as ``append`` does, then attend one
                                         query per appended token (chunked prefill
                                         or verification of draft positions).

The K/V rows of a token are a function of (layer, writing sequence, position)
only, drawn by :func:`synth.draws.token_rows`; queries of the ``i``-th decode
op in layer ``l`` are ``normal_bits(seed, TAG_Q, (i, l), (S, Hq, d))``; queries of
the ``i``-th prefill op are ``normal_bits(seed, TAG_QCHUNK, (i, l), (sum(counts),
Hq, d))``, sequence-major.

The shapes follow the pages' workloads: the Qwen3-8B geometry (36 layers,
8 KV heads of dim 128, 32 query heads), the 70B GQA geometry (64 query heads,
8 KV heads), the 2303/8447-token request lengths and the shared 6144-token
prefix of the inference-optimization chapter, and the 131,072-token agentic
context of the KV-cache-management chapter.  Pool sizes are chosen here; see
the module constants.
"""

from __future__ import annotations

from dataclasses import dataclass, field

from .draws import BF16, F32


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    ops: list = field(default_factory=list)
    partition_tokens: int = 0  # 0: let the library choose
    description: str = ""
    kv_format: str = ""  # "", "q8_0" or "q4_0": the pool stores the rows quantised

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2

    def final_lengths(self) -> dict:
        """Context length of every sequence after all ops (no allocator needed)."""
        lens: dict = {}
        for op in self.ops:
            if op[0] == "add":
                lens[op[1]] = 0
            elif op[0] == "fork":
                lens[op[2]] = lens[op[1]]
            elif op[0] in ("append", "prefill"):
                for s, c in zip(op[1], op[2]):
                    lens[s] += c
        return lens


def _round_robin(targets):
    """Append ops growing the sequences one token per round, in index order."""
    ops = []
    lens = [0] * len(targets)
    while any(l < t for l, t in zip(lens, targets)):
        seqs = tuple(i for i, (l, t) in enumerate(zip(lens, targets)) if l < t)
        ops.append(("append", seqs, tuple(1 for _ in seqs)))
        for i in seqs:
            lens[i] += 1
    return ops


def tiny_fp32() -> Workload:
    """Three fp32 sequences of lengths 5, 7, 9 grown token by token, B = 4."""
    ops = [("add", s) for s in range(3)]
    ops += _round_robin([5, 7, 9])
    ops.append(("decode", (0, 1, 2)))
    return Workload("tiny_fp32", 1, F32, 1, 4, 1, 64, 4, 16, ops,
                    description="fp32 Hq=4 Hkv=1 d=64 B=4, lengths 5/7/9, pool 16")


# Pool of the Qwen3-8B-shaped workloads (37 x 2304 and 16 x 8448 tokens):
# floor(12 GiB / 36 layers / 64 KiB per block-layer).
POOL_QWEN = 5461
# Pool of the 70B-GQA workload: 12 sequences x 8192 blocks, the 60 GiB B=16
# pool of the 70B example.
POOL_70B = 98304
# Pool of the agentic fork workload: 10,304 blocks needed at the end plus ~16 %
# headroom.
POOL_FORK = 12288


def qwen_independent() -> Workload:
    seqs = tuple(range(37))
    ops = [("add", s) for s in seqs]
    ops.append(("append", seqs, tuple(2303 for _ in seqs)))
    ops.append(("append", seqs, tuple(1 for _ in seqs)))
    ops.append(("decode", seqs))
    return Workload("qwen3_8b_37x2304", 2, BF16, 1, 32, 8, 128, 16, POOL_QWEN, ops,
                    description="bf16 Hq=32 Hkv=8 d=128 B=16, 37 sequences x 2304 tokens")


def shared_prefix() -> Workload:
    seqs = tuple(range(16))
    ops = [("add", 0), ("append", (0,), (6144,))]
    ops += [("fork", 0, c) for c in seqs[1:]]
    ops.append(("append", seqs, tuple(2303 for _ in seqs)))
    ops.append(("append", seqs, tuple(1 for _ in seqs)))
    ops.append(("decode", seqs))
    return Workload("shared_prefix_16x8448", 3, BF16, 1, 32, 8, 128, 16, POOL_QWEN, ops,
                    description="bf16 Hq=32 Hkv=8 d=128 B=16, 16 x 8448 tokens sharing 6144")


def gqa70b_128k() -> Workload:
    seqs = tuple(range(12))
    ops = [("add", s) for s in seqs]
    ops.append(("append", seqs, tuple(131072 for _ in seqs)))
    ops.append(("decode", seqs))
    return Workload("gqa70b_12x131072", 4, BF16, 1, 64, 8, 128, 16, POOL_70B, ops,
                    partition_tokens=512,
                    description="bf16 Hq=64 Hkv=8 d=128 B=16, 12 x 131072 tokens, split-K 512")


def agentic_fork(steps: int = 512, layers: int = 36) -> Workload:
    """4 roots of 32769 tokens, each forked 16 ways, then ``steps`` decode steps."""
    ops = []
    roots = tuple(r * 16 for r in range(4))
    for r in roots:
        ops.append(("add", r))
    ops.append(("append", roots, tuple(32769 for _ in roots)))
    for r in roots:
        ops += [("fork", r, r + c) for c in range(1, 16)]
    seqs = tuple(range(64))
    for _ in range(steps):
        ops.append(("append", seqs, tuple(1 for _ in seqs)))
        ops.append(("decode", seqs))
    return Workload("agentic_fork_64x33281", 5, BF16, layers, 32, 8, 128, 16, POOL_FORK, ops,
                    description=f"bf16 Hq=32 Hkv=8 d=128 B=16, {layers} layers, 4 roots x 16 forks,"
                                f" {steps} steps")


def chunked_prompt(prompts=(2048,), chunk=512, layers=1, seed=6) -> Workload:
    """Prompts prefilled chunk by chunk over their own paged history.

    With the defaults this is [KVM] Figure 8: one 2048-token prompt, chunks of
    512 tokens, so iteration k = 3 covers tokens 1024..1535 and attends the
    1536 tokens of chunks 1..3.  Several prompts advance together, one chunk
    each per iteration, until the longest is done.
    """
    seqs = tuple(range(len(prompts)))
    ops = [("add", s) for s in seqs]
    done = [0] * len(prompts)
    while any(d < p for d, p in zip(done, prompts)):
        ids = tuple(s for s in seqs if done[s] < prompts[s])
        counts = tuple(min(chunk, prompts[s] - done[s]) for s in ids)
        ops.append(("prefill", ids, counts))
        for s, c in zip(ids, counts):
            done[s] += c
    blocks = sum(-(-p // 16) for p in prompts)
    return Workload(f"chunked_prompt_{'_'.join(map(str, prompts))}_c{chunk}", seed, BF16, layers, 32, 8, 128, 16,
                    blocks + 16, ops,
                    description=f"bf16 Hq=32 Hkv=8 d=128 B=16, prompts {list(prompts)} in chunks of {chunk}")


# Pool of the chunk workloads: 16 sequences x 8192 tokens = 8192 blocks, plus slack.
POOL_CHUNK = 8208


def prefill_last_chunk() -> Workload:
    """The last 512-token chunk of 16 8K-token prompts ([INF] section 8.2.3: 7680
    cached tokens, 4,063,488 query-key pairs per head; batch 16 as in the
    chapter's 8K-input experiment)."""
    seqs = tuple(range(16))
    ops = [("add", s) for s in seqs]
    ops.append(("append", seqs, tuple(7680 for _ in seqs)))
    ops.append(("prefill", seqs, tuple(512 for _ in seqs)))
    return Workload("prefill_16x512_after_7680", 7, BF16, 1, 32, 8, 128, 16, POOL_CHUNK, ops,
                    description="bf16 Hq=32 Hkv=8 d=128 B=16, 16 x (7680 cached + 512-token chunk)")


def verify_drafts(positions=8) -> Workload:
    """Verification of ``positions`` draft tokens for 16 requests with 8K contexts
    ([INF] section 8.6.3 plan D: 16 requests, 8 positions each)."""
    seqs = tuple(range(16))
    ops = [("add", s) for s in seqs]
    ops.append(("append", seqs, tuple(8192 - positions for _ in seqs)))
    ops.append(("prefill", seqs, tuple(positions for _ in seqs)))
    return Workload(f"verify_16x{positions}_after_{8192 - positions}", 8, BF16, 1, 32, 8, 128, 16, POOL_CHUNK, ops,
                    description=f"bf16 Hq=32 Hkv=8 d=128 B=16, 16 x ({8192 - positions} cached + {positions} drafts)")


def tool_pause(layers: int = 2, seed: int = 8, frames: str = "shuffled") -> Workload:
    """Trajectories paused for a tool call are swapped to host frames and back.

    Eight sequences of mixed lengths (two of them forks of a third, so some of
    their blocks are shared and stay in HBM); sequences 0 and 3 are swapped out,
    the others keep decoding and reuse the freed blocks, then 0 and 3 are
    swapped back in (into other blocks) and everyone decodes.  Hq=32, Hkv=8,
    d=128, B=16, bf16.
    """
    lens = (2304, 37, 16, 1000, 513, 0, 64, 300)
    seqs = tuple(range(len(lens)))
    # "sequential": the host free list starts 0, 1, 2, ... (frames of a swap are consecutive)
    ops = [("host", 256) if frames == "shuffled" else ("host", 256, "sequential")]
    ops += [("add", s) for s in seqs if s not in (6, 7)]
    ops.append(("append", tuple(s for s in seqs if s not in (6, 7)), tuple(lens[s] for s in seqs if s not in (6, 7))))
    ops += [("fork", 3, 6), ("fork", 3, 7)]
    ops.append(("append", (6, 7), (64 - 0, 300 - 0)))
    ops.append(("decode", seqs))
    ops += [("swap_out", 0), ("swap_out", 3)]
    others = tuple(s for s in seqs if s not in (0, 3))
    for _ in range(3):
        ops.append(("append", others, tuple(40 for _ in others)))
        ops.append(("decode", others))
    ops += [("swap_in", 3), ("swap_in", 0)]
    ops.append(("append", seqs, tuple(1 for _ in seqs)))
    ops.append(("decode", seqs))
    blocks = sum(-(-(n + 130) // 16) for n in lens) + 100
    return Workload("tool_pause_8", seed, BF16, layers, 32, 8, 128, 16, blocks, ops,
                    description="bf16 Hq=32 Hkv=8 d=128 B=16, 8 sequences, 2 swapped out and back in")


# The decode workloads by name (the name each builds).
WORKLOADS = {
    "tiny_fp32": tiny_fp32,
    "qwen3_8b_37x2304": qwen_independent,
    "shared_prefix_16x8448": shared_prefix,
    "gqa70b_12x131072": gqa70b_128k,
    "agentic_fork_64x33281": agentic_fork,
}


def get_workload(name: str, **kw) -> Workload:
    return WORKLOADS[name](**kw)
