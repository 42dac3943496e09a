"""The five step workloads, as plain data.

Each entry fixes the shapes and value distributions of one synthetic
block-diffusion step.  The geometries follow the Qwen2.5-VL-3B / 7B
attention shapes that the Fast-dVLM write-up builds on (itsolotime.com
"Fast-dVLM" page, introduction: a Qwen2.5-VL-3B base) and the block sizes
8 / 16 / 32 that both pages discuss (Fast-dVLM page, sections 4.2 and 5.3,
Fig. 6; DiffusionVL notes, "cached block decoding", default training block
D = 8).

Distribution strings read as variance: ``sigma2 = 4`` means standard
deviation 2.  Nothing here computes any part of the method.
"""

F32 = 0
BF16 = 1
FP8KV = 2   # bf16 queries, OCP E4M3 keys and values with one fp32 scale per (item, KV head)

BIDIR = 0   # denoise step: the whole current block is visible to each slot
CAUSAL = 1  # verify step: slot i sees the block only up to itself
QUAD = 2    # quadratic self-speculative step: B drafts (causal) + B groups of mask tokens

CONFIGS = {
    1: dict(
        name="tiny: 1 item, 2q/1kv heads, d64, fp32, prefix 64, D=8 (4 masked), V=1000",
        n_items=1, n_req=1, Hq=2, Hkv=1, d=64, dtype=F32, mode=BIDIR,
        prefix=("fixed", 64), D=8, n_masked=4, V=1000, logit_sigma2=3.0,
        plant=None, S=8, tau=0.9,
    ),
    2: dict(
        name="3B single layer: 16q/2kv, d128, bf16, prefix 1024 (768 vision + 256 text), "
             "D=8 all masked, V=151936 with a +8 planted peak",
        n_items=1, n_req=1, Hq=16, Hkv=2, d=128, dtype=BF16, mode=BIDIR,
        prefix=("fixed", 1024), D=8, n_masked=8, V=151936, logit_sigma2=4.0,
        plant="peak8", S=8, tau=0.9,
    ),
    3: dict(
        name="3B long-reasoning step: 36 layers x (16q/2kv, d128, bf16, prefix 4096), "
             "D=16 with 8 committed, V=151936, S=16, tau=0.9",
        n_items=36, n_req=1, Hq=16, Hkv=2, d=128, dtype=BF16, mode=BIDIR,
        prefix=("fixed", 4096), D=16, n_masked=8, V=151936, logit_sigma2=4.0,
        plant=None, S=16, tau=0.9,
    ),
    4: dict(
        name="3B self-speculative verify: 16q/2kv, d128, bf16, prefix 2048, D=16 draft, "
             "causal, V=151936, geometric(0.3) accepted prefix, then append",
        n_items=1, n_req=1, Hq=16, Hkv=2, d=128, dtype=BF16, mode=CAUSAL,
        prefix=("fixed", 2048), D=16, n_masked=16, V=151936, logit_sigma2=4.0,
        plant="geom0.3", S=16, tau=0.9,
    ),
    5: dict(
        name="7B batched step: 8 requests, prefixes U{2048..8192}, 28q/4kv, d128, bf16, "
             "D=32 all masked, V=152064, S=8, tau=0.8",
        n_items=8, n_req=8, Hq=28, Hkv=4, d=128, dtype=BF16, mode=BIDIR,
        prefix=("uniform", 2048, 8192), D=32, n_masked=32, V=152064, logit_sigma2=4.0,
        plant=None, S=8, tau=0.8,
    ),
}


def seed_of(cfg_id: int) -> int:
    return 1000 + int(cfg_id)


# LM head with a fused confidence epilogue (a step after the attention layers:
# the block's final hidden states times the vocabulary projection give the
# logits that the confidence / commit rule reads).  Shapes of the Qwen2.5-VL-3B
# language model (hidden 2048, vocabulary 151936) at block D = 16.  Hidden
# states ~ N(0, 1); weights ~ N(0, 4 / H), so a logit has variance 4 like the
# logits configs above; ``plants`` masked rows get one token whose weight row
# is a scaled copy of that row's hidden state (a logit near ``gain``).
LMHEAD_CONFIGS = {
    1: dict(name="3B LM head: H=2048, V=151936, D=16 with 8 masked, S=16, tau=0.9",
            n_req=1, D=16, n_masked=8, V=151936, H=2048, S=16, tau=0.9, plants=3, gain=17.0),
    2: dict(name="small LM head: H=256, V=5003, 2 requests x D=8 (5 masked), S=4, tau=0.5",
            n_req=2, D=8, n_masked=5, V=5003, H=256, S=4, tau=0.5, plants=2, gain=17.0),
}


def lmhead_seed_of(cfg_id: int) -> int:
    return 2000 + int(cfg_id)


# Quadratic self-speculative step (Fast-dVLM write-up, section 5.3, the quadratic
# variant; Fig. 6 sweeps block sizes 4..32): the 3B long-reasoning shape of config 3
# with a draft block of B = 16, i.e. B (B + 3) / 2 = 152 block slots per layer
# (16 drafts, then 16 + 15 + ... + 1 mask tokens of the 16 acceptance hypotheses).
QUAD_CONFIGS = {
    1: dict(name="3B quadratic speculative step: 36 layers x (16q/2kv, d128, bf16, prefix 4096), B=16 (152 slots)",
            n_items=36, Hq=16, Hkv=2, d=128, dtype=BF16, prefix=("fixed", 4096), B=16),
    2: dict(name="small quadratic step: 3 items, 8q/2kv, d128, bf16, prefixes 0/77/300, B=5 (20 slots)",
            n_items=3, Hq=8, Hkv=2, d=128, dtype=BF16, prefix=("list", [0, 77, 300]), B=5),
}


def quad_seed_of(cfg_id: int) -> int:
    return 3000 + int(cfg_id)


# Two-stream training attention (Fast-dVLM write-up, sections 4.1-4.4; summary
# page Fig. 3): [clean stream ; noisy stream].  The clean stream is vision tokens
# followed by (prompt, response) turns; the noisy stream holds the responses'
# tokens only.  ``turns`` lists (prompt length, response length) pairs, either one
# list for every sequence or one list per sequence.  Config 1 is the 3B training
# shape at the 2048-token context the write-up's memory figure uses (section 4.4)
# with the target block size 32 (section 4.2); responses are not multiples of 32,
# so the last block of each is truncated.
TWO_STREAM_CONFIGS = {
    1: dict(name="3B two-stream training attention: 8 sequences, 16q/2kv, d128, bf16, clean 2048 "
                 "(1024 vision + 2 turns), noisy 832, D=32",
            n_seq=8, vision=1024, turns=[(128, 638), (64, 194)], D=32, Hq=16, Hkv=2, d=128, dtype=BF16),
    2: dict(name="small two-stream: 2 sequences, 4q/2kv, d64, bf16, ragged turns, D=8",
            n_seq=2, vision=40, turns=[[(8, 37), (5, 20)], [(3, 16), (9, 9), (2, 1)]], D=8, Hq=4, Hkv=2, d=64,
            dtype=BF16),
}


def two_stream_seed_of(cfg_id: int) -> int:
    return 4000 + int(cfg_id)
