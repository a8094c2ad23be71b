"""Oracle for GLM-5.2 IndexShare: source-layer resolution and the layer stack.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: page "GLM5 TensorCast 适配设计" (GLM5 TensorCast adaptation design),
section "GLM-5.2 IndexShare":
  * indexer_types holds one of "full" / "shared" per decoder layer;
  * a full layer is a source layer: it runs the indexer and produces
    topk_indices;
  * a shared layer runs no indexer and reuses the top-k of the nearest
    preceding full layer; a chain full -> shared -> shared forwards the
    same top-k unchanged;
  * a list shorter than the layer count, an unknown type, or a shared layer
    with no preceding full layer is rejected with ValueError.
Section "KV cache dtype and parallel-linear boundary fix": only full source
layers own an indexer cache; shared layers neither own nor alias one.
Section "Configuration constraints", item 6 restates the validation rule.
"""

FULL, SHARED = "full", "shared"


def resolve_sources(indexer_types, n_layers):
    """Per-layer source layer index, or ValueError."""
    types = list(indexer_types)
    if len(types) < n_layers:
        raise ValueError("indexer_types has %d entries for %d layers"
                         % (len(types), n_layers))
    for t in types:
        if t not in (FULL, SHARED):
            raise ValueError("unknown indexer type %r" % (t,))
    src = []
    last_full = None
    for i in range(n_layers):
        if types[i] == FULL:
            last_full = i
            src.append(i)
        else:
            if last_full is None:
                raise ValueError("shared layer %d has no preceding full layer"
                                 % i)
            src.append(last_full)
    return src


def forward(indexer_types, layers, run_indexer, run_attention):
    """Run the stack layer by layer.

    layers        list of per-layer input objects
    run_indexer   f(layer) -> top-k indices (called on full layers only)
    run_attention f(layer, topk) -> attention result
    Returns (per-layer results, per-layer active top-k, indexer call count).
    """
    src = resolve_sources(indexer_types, len(layers))
    active = None
    results, actives, calls = [], [], 0
    for i, layer in enumerate(layers):
        if src[i] == i:
            active = run_indexer(layer)
            calls += 1
        # a shared layer keeps `active`, which came from layer src[i]
        actives.append(active)
        results.append(run_attention(layer, active))
    return results, actives, calls
