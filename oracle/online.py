"""Online TBPTT training segment oracle: numpy f64.

TEST INFRASTRUCTURE ONLY (see the package header).

Follows online_train_segment_tbptt and apply_full_gradients of "infotheory
.../rwkvzip/rwkv7/model.rs".  One segment, for B streams of S (input,
target) steps starting from the streams' live decode state:
  1. gradients of the mean next-token cross-entropy over the segment with
     backpropagation through time truncated at the segment start (the page
     replays its checkpointed chunks in reverse carrying the recurrent
     gradient; the chunking only bounds memory, so the gradient is exact
     BPTT within the segment);
  2. one optimiser update of every parameter (SGD, or Adam with b1 = 0.9,
     b2 = 0.999, eps = 1e-8 and bias corrections 1 - b^t, t counting updates);
  3. the live state: the segment replayed from the start state with the
     updated weights.
Readings where the page leaves a step open:
  - the loss is the plain softmax cross-entropy (the page's probability
    floor and output bias are not shown) and gradients are descent
    directions (the page ascends on target - p with += lr g);
  - clip > 0 clamps every gradient element to [-clip, clip] before the
    update (the page passes clip to its per-tensor update helpers, whose
    bodies are not shown); clip = 0 leaves gradients as they are;
  - Adam: m = b1 m + (1 - b1) g, v = b2 v + (1 - b2) g^2,
    p -= lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).
"""
import numpy as np

from . import stack

B1, B2, ADAM_EPS = 0.9, 0.999, 1e-8


def _leaves(tree, path=()):
    """(path, array) for every parameter array of a model / gradient dict."""
    for k, v in tree.items():
        if k == "blocks":
            for i, b in enumerate(v):
                yield from _leaves(b, path + ("blocks", i))
        elif k == "tm":
            yield from _leaves(v, path + ("tm",))
        elif v is not None:
            yield path + (k,), v


def _get(tree, path):
    for p in path:
        tree = tree[p]
    return tree


def _set(tree, path, value):
    for p in path[:-1]:
        tree = tree[p]
    tree[path[-1]] = value


def clip_grad(g, clip):
    return np.clip(g, -clip, clip) if clip > 0 else g


def sgd_update(p, g, lr, clip):
    return p - lr * clip_grad(g, clip)


def adam_update(p, g, m, v, t, lr, clip):
    """One Adam update at step t (t >= 1); returns (p, m, v)."""
    g = clip_grad(g, clip)
    m = B1 * m + (1.0 - B1) * g
    v = B2 * v + (1.0 - B2) * g * g
    mh = m / (1.0 - B1 ** t)
    vh = v / (1.0 - B2 ** t)
    return p - lr * mh / (np.sqrt(vh) + ADAM_EPS), m, v


def zeros_like_model(model):
    """A model-shaped dict of zero arrays (Adam moments)."""
    z = stack._f64(model)
    for path, v in _leaves(z):
        _set(z, path, np.zeros_like(v))
    return z


def train_segment(model, cfg, tokens, targets, state, optimizer="adam", lr=1e-3, clip=0.0,
                  adam=None, t=1):
    """One online training segment.

    Returns (loss, new_model, new_state, grads, new_adam): loss and grads
    from the weights before the update; new_model after it; new_state the
    live state after replaying the segment with new_model from `state`;
    new_adam the moment estimates (Adam), with `adam` the previous ones (None:
    zeros) and t the index of this update (1 for the first).
    """
    m = stack._f64(model)
    loss, G = stack.train_step(m, cfg, tokens, targets, state=state)
    new = stack._f64(model)
    new_adam = None
    if optimizer == "sgd":
        for path, p in _leaves(m):
            _set(new, path, sgd_update(p, _get(G, path), lr, clip))
    elif optimizer == "adam":
        prev = adam if adam is not None else dict(m=zeros_like_model(m), v=zeros_like_model(m))
        new_adam = dict(m=zeros_like_model(m), v=zeros_like_model(m))
        for path, p in _leaves(m):
            pn, mn, vn = adam_update(p, _get(G, path), _get(prev["m"], path), _get(prev["v"], path),
                                     t, lr, clip)
            _set(new, path, pn)
            _set(new_adam["m"], path, mn)
            _set(new_adam["v"], path, vn)
    else:
        raise ValueError(f"optimizer must be 'sgd' or 'adam', not {optimizer!r}")
    _, new_state = stack.forward(new, cfg, tokens, state)
    return loss, new, new_state, G, new_adam
