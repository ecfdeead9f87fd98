"""Split-KV work plan, written from its definition -- TEST INFRASTRUCTURE ONLY.

The pages say only that the kernel is tuned for batches of variable-length
sequences (launch announcement quoted on the 8bitnewsroom FlashMLA page; the
aivengo.media feature list says the same).  The plan below is the plain
reading used throughout this repository: cut the batch's work into
``num_parts`` contiguous, equal-cost pieces.

Definition
----------
* Request ``b`` with ``L_b`` cached tokens has ``n_b = ceil(L_b / 64)`` pages.
* Lay the requests with ``n_b > 0`` end to end on a cost line.  Request ``b``
  takes ``c`` units of overhead followed by one unit per page, so page ``j`` of
  request ``b`` sits at position ``x = C_b + c + j`` where ``C_b`` is the total
  cost of the requests before it.  ``T`` is the total cost.
* ``P = min(num_parts, T)``.  The page at position ``x`` belongs to part
  ``floor(x * P / T)``.  Each part therefore owns a contiguous run of the
  batch's pages, possibly spanning several requests.
* ``c = 1 + (s_q * h_q) // 64`` (one unit per page; the overhead stands for a
  request segment's query load and partial-output traffic).

Outputs
-------
* ``meta[p] = [b_first, j_first, b_last, j_last, split_first, 0, 0, 0]`` for a
  part with pages, where the part runs from page ``j_first`` of ``b_first`` to
  page ``j_last`` of ``b_last`` inclusive and ``split_first`` is the part's rank
  among the parts touching ``b_first``.  A part with no pages has
  ``b_first = -1`` and zeros elsewhere.
* ``split_base[b]`` (length ``batch + 1``): prefix sum of the number of parts
  touching each request; request ``b`` owns split slots
  ``split_base[b] .. split_base[b + 1] - 1``.
"""

PAGE = 64
META_INTS = 8


def overhead(s_q, h_q):
    """Cost units charged per request segment."""
    return 1 + (s_q * h_q) // 64


def plan(seqlens, num_parts, c):
    """Return (meta, split_base) as lists of Python ints."""
    batch = len(seqlens)
    pages = [(int(L) + PAGE - 1) // PAGE if int(L) > 0 else 0 for L in seqlens]
    total = sum(c + n for n in pages if n > 0)
    meta = [[-1, 0, 0, 0, 0, 0, 0, 0] for _ in range(num_parts)]
    counts = [0] * batch
    if total > 0:
        parts = min(num_parts, total)
        first_part = {}
        x = 0
        for b, n in enumerate(pages):
            if n == 0:
                continue
            x += c
            for j in range(n):
                p = (x * parts) // total
                if meta[p][0] == -1:
                    meta[p][0] = b
                    meta[p][1] = j
                meta[p][2] = b
                meta[p][3] = j
                if b not in first_part:
                    first_part[b] = p
                counts[b] = p - first_part[b] + 1
                x += 1
        for p in range(num_parts):
            if meta[p][0] != -1:
                meta[p][4] = p - first_part[meta[p][0]]
    split_base = [0]
    for b in range(batch):
        split_base.append(split_base[-1] + counts[b])
    return meta, split_base
