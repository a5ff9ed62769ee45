"""Base Batch Shuffling: the batch former ahead of the jagged attention path.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[GEM-MFU, Key points: BBS bullet] and [GEM-MFU, Detailed notes: Base Batch
Shuffling item]: base sub-batches of 128 samples are sorted by sequence
length, and the heaviest and the lightest are merged in turn, which evens out
the sequence-length load of the batches different GPUs (or steps) get,
without any exchange between ranks.

Readings of what the pages leave open (stated where used):
  * a base batch is a run of `base_batch` consecutive samples of the input,
    in input order (the last one may be shorter);
  * its load is the sum over its samples of the cost of a sample: the
    sequence length (cost "tokens", the pages' "sorted by sequence length"),
    or its square (cost "pairs": the visible (query, key) pairs of causal
    self attention grow with L^2);
  * "sort by length" is descending load, ties by base-batch index ascending;
  * "merge the heaviest with the lightest in turn" pairs the k-th heaviest
    with the k-th lightest; pair k becomes merged batch k (the heaviest
    base batch's samples first, then the lightest's, each in input order);
    with an odd number of base batches the median one is a merged batch of
    its own, last.
"""

COSTS = ("tokens", "pairs")


def sample_cost(length, cost):
    if cost == "tokens":
        return int(length)
    if cost == "pairs":
        return int(length) * int(length)
    raise ValueError("cost must be one of %r" % (COSTS,))


def base_batches(n_samples, base_batch):
    """[start, end) of every base batch: consecutive runs of base_batch samples."""
    if base_batch < 1:
        raise ValueError("base_batch must be >= 1")
    return [(s, min(s + base_batch, n_samples)) for s in range(0, n_samples, base_batch)]


def bbs_plan(lengths, base_batch=128, cost="tokens"):
    """Returns (perm, batch_start): the samples of merged batch i are
    perm[batch_start[i] : batch_start[i+1]] (indices into `lengths`)."""
    lengths = [int(x) for x in lengths]
    if any(x < 0 for x in lengths):
        raise ValueError("lengths must be >= 0")
    bases = base_batches(len(lengths), base_batch)
    loads = [sum(sample_cost(lengths[i], cost) for i in range(s, e)) for s, e in bases]
    order = sorted(range(len(bases)), key=lambda k: (-loads[k], k))   # heaviest first
    n = len(order)
    groups = [[order[i], order[n - 1 - i]] for i in range(n // 2)]
    if n % 2:
        groups.append([order[n // 2]])
    perm, batch_start = [], [0]
    for grp in groups:
        for k in grp:
            s, e = bases[k]
            perm.extend(range(s, e))
        batch_start.append(len(perm))
    return perm, batch_start


def merged_loads(lengths, perm, batch_start, cost="tokens"):
    """Load of every merged batch."""
    return [sum(sample_cost(lengths[perm[p]], cost) for p in range(batch_start[i], batch_start[i + 1]))
            for i in range(len(batch_start) - 1)]
