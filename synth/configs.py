"""Shapes of the five FedAvg aggregation workloads.

The workloads and their sizes:

* dense, K=3 clients, one flat fp32 vector of 1,000,000 parameters;
* adapter-only, K=8 clients, LoRA rank-16 A/B pairs on q,k,v,o of 32 layers at
  hidden 4096 (16,777,216 bf16 parameters), each client sending a random subset
  of the 128 module adapters;
* dense full model, K=16 clients, a transformer-shaped 2.0B-parameter tensor
  list (24 layers, hidden 2048, FFN 8192, tied embedding 151936x2048), bf16;
* streaming, K=32 clients arriving one after another in 64 MiB chunks of an
  8B-parameter bf16 model (32 layers, hidden 4096, grouped K/V of width 1024,
  FFN 14336, untied vocab 128256);
* sparse partial sharing, 10^9 fp32 parameters, K=20 clients each sending the
  top 10% of its |delta| as sorted (index, value) lists.

Only shapes live here; no arithmetic of the method.
"""

# SeedSequence roles
ROLE_COUNTS = 0    # n_k
ROLE_BASE = 1      # global model / base values
ROLE_VALUES = 2    # client values or deltas
ROLE_SUPPORT = 3   # masks / index lists

# config ids used as the second SeedSequence word
CFG_DENSE_SMALL = 1
CFG_ADAPTER = 2
CFG_DENSE_2B = 3
CFG_STREAM_8B = 4
CFG_SPARSE_1B = 5

CHUNK_BYTES_8B = 64 << 20


def numel_of(shapes):
    total = 0
    for s in shapes:
        p = 1
        for d in s:
            p *= d
        total += p
    return total


def dense_2b_tensor_shapes(layers=24, hidden=2048, ffn=8192, vocab=151936):
    """Tensor list of the 2.0B dense model: per layer q,k,v,o (h x h), gated
    FFN gate/up (f x h) and down (h x f), two norms; a tied embedding and a
    final norm.  1,921,878,016 parameters in 218 tensors at the defaults."""
    shapes = [(vocab, hidden)]
    for _ in range(layers):
        shapes += [(hidden,), (hidden, hidden), (hidden, hidden), (hidden, hidden),
                   (hidden, hidden), (hidden,), (ffn, hidden), (ffn, hidden), (hidden, ffn)]
    shapes.append((hidden,))
    return shapes


def stream_8b_tensor_shapes(layers=32, hidden=4096, kv=1024, ffn=14336, vocab=128256):
    """Tensor list of the 8B streamed model: per layer q,o (h x h), grouped k,v
    (kv x h), gated FFN, two norms; untied embedding and head, final norm.
    8,030,261,248 parameters at the defaults."""
    shapes = [(vocab, hidden)]
    for _ in range(layers):
        shapes += [(hidden,), (hidden, hidden), (kv, hidden), (kv, hidden),
                   (hidden, hidden), (hidden,), (ffn, hidden), (ffn, hidden), (hidden, ffn)]
    shapes += [(hidden,), (vocab, hidden)]
    return shapes


def adapter_segments(layers=32, hidden=4096, rank=16, modules=("q", "k", "v", "o")):
    """Flat layout of the LoRA adapter set: for each layer and module an A
    matrix (rank x hidden) then a B matrix (hidden x rank).  Returns
    (segment_bounds, module_of_segment): bounds has T+1 entries starting at 0,
    and module_of_segment maps each of the T segments to its module number,
    since A and B of one adapter always travel together."""
    bounds = [0]
    module_of = []
    m = 0
    for _ in range(layers):
        for _ in modules:
            for _ab in range(2):
                bounds.append(bounds[-1] + rank * hidden)
                module_of.append(m)
            m += 1
    return bounds, module_of
