"""Which parameters go to Muon and which to AdamW.

Muon is for hidden 2D weight matrices; embeddings, the output head, routers,
norms, biases and other vectors or scalars stay on AdamW ("About Muon: Why
Not Adam", section "How Do We Turn It Into a Real Optimizer?", "Which
parameters"; "Why Muon Works", section 7.1: the rule is dim() == 2 and not
an embedding or output parameter, refined by name and module type).
Convolution kernels must be flattened to 2D by the caller first.
"""


def _is_special(name):
    low = name.lower()
    parts = low.replace("/", ".").split(".")
    for p in parts:
        if p in ("lm_head", "head", "output", "router", "embed", "embedding", "embeddings",
                 "wte", "wpe", "tok_emb", "bias"):
            return True
        if "norm" in p or p.startswith("ln"):
            return True
        if p.startswith("embed"):
            return True
    return False


def route_parameters(named_params, exclude=()):
    """Split ``(name, tensor)`` pairs into ``(muon, adamw)`` lists of pairs.

    A parameter goes to Muon iff it is 2D and its name marks it as neither
    an embedding, an output/LM head, a router, a norm nor a bias.  Names in
    ``exclude`` always go to AdamW.
    """
    muon, adamw = [], []
    exclude = set(exclude)
    for name, p in named_params:
        if p.dim() == 2 and name not in exclude and not _is_special(name):
            muon.append((name, p))
        else:
            adamw.append((name, p))
    return muon, adamw
