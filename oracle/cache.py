"""HBM hot-row cache over a host-resident table — oracle (TEST INFRASTRUCTURE ONLY).

The CTR article (section 二) keeps the hot embeddings in GPU HBM (its L0) and
the rest in host DRAM (its L1): a lookup tries HBM first and falls back to host
memory on a miss, each tier replaces its least recently used entries, and the
hit and miss rates are monitored.  The article fixes neither the cache's
organisation nor when a missed row enters it.  Reading (the plainest one a GPU
serves batch by batch, deterministic so that it can be checked exactly):

* Organisation: ``sets`` x ``ways`` entries; row r belongs to set
  ``fmix32(r) mod sets``, where fmix32 is the 32-bit finaliser of MurmurHash3
  (Appleby), so clustered row ids still spread over the sets.
* Time is counted in batches: batch t (t = 1, 2, ...) stamps every way it hits
  with t.  All lookups of a batch see the cache as it was when the batch began.
* Each lookup of a valid row is a hit (the row is in its set) or a miss (the
  row is read from host memory).  Pooling reads the same fp32 row either way.
* After the lookups, every set that missed admits one row: the row of its
  earliest missed lookup in batch order (position in the batch's id array).
  It replaces the set's least recently used way — an empty way first, then the
  smallest stamp, ties to the lowest way — and is stamped t.  One admission per
  set per batch bounds the host traffic a batch can cause and keeps a batch
  from evicting rows it has just read (the thrashing the article warns of).
* Counters since the cache was attached: lookups, hits, misses, admissions,
  evictions (admissions that replaced a valid row).  Ids outside the table are
  an input error: they are neither looked up nor counted.
"""
import numpy as np

MASK32 = 0xFFFFFFFF
COUNTERS = ("lookups", "hits", "misses", "admissions", "evictions")


def fmix32(h):
    """The 32-bit finaliser of MurmurHash3 (scalar int in, int out)."""
    h &= MASK32
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & MASK32
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & MASK32
    h ^= h >> 16
    return h


class HotRowCache:
    """Directory of one table's cache: which row each way holds and when it was last used."""

    def __init__(self, sets, ways):
        assert sets >= 1 and ways >= 1
        self.sets, self.ways = int(sets), int(ways)
        self.tags = np.full((self.sets, self.ways), -1, dtype=np.int64)    # row held, -1 empty
        self.stamps = np.zeros((self.sets, self.ways), dtype=np.int64)     # batch of last use
        self.epoch = 0
        self.counters = dict.fromkeys(COUNTERS, 0)

    def set_of(self, row):
        return fmix32(int(row)) % self.sets

    def contains(self, row):
        return int(row) in self.tags[self.set_of(row)]

    def batch(self, lookups, rows=None):
        """One batch.  ``lookups``: (position, row) pairs in batch order, position being the
        lookup's index in the batch's id array.  Rows outside ``[0, rows)`` are skipped.
        Returns a bool array: which lookups hit."""
        self.epoch += 1
        t = self.epoch
        hit = np.zeros(len(lookups), dtype=bool)
        first_miss = {}
        for i, (pos, row) in enumerate(lookups):
            row = int(row)
            if row < 0 or (rows is not None and row >= rows):
                continue
            s = self.set_of(row)
            self.counters["lookups"] += 1
            ways = np.nonzero(self.tags[s] == row)[0]
            if ways.size:
                hit[i] = True
                self.stamps[s, ways[0]] = t
                self.counters["hits"] += 1
            else:
                self.counters["misses"] += 1
                if s not in first_miss or pos < first_miss[s][0]:
                    first_miss[s] = (int(pos), row)
        for s, (_, row) in first_miss.items():
            # least recently used way: empty ways first, then the smallest stamp, then the lowest way
            keys = [(0 if self.tags[s, w] < 0 else 1, self.stamps[s, w], w) for w in range(self.ways)]
            w = min(keys)[2]
            if self.tags[s, w] >= 0:
                self.counters["evictions"] += 1
            self.tags[s, w] = row
            self.stamps[s, w] = t
            self.counters["admissions"] += 1
        return hit


def table_lookups(spec, batch, table):
    """(position, row) of every id the batch looks up in ``table``, in batch order (the
    features that read the table, in spec order; ids in bag order)."""
    from .common import expand
    ex = expand(spec, batch)
    off = ex["bag_offsets"]
    out = []
    for fi, f in enumerate(spec["features"]):
        if f["table"] != table:
            continue
        g0 = ex["bag_base"][fi]
        g1 = g0 + ex["nbags"][fi]
        for pos in range(int(off[g0]), int(off[g1])):
            out.append((pos, int(ex["ids"][pos])))
    return out
