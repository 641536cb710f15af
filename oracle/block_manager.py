"""Reference model of the KV block manager (oracle, test infrastructure only).

What it follows (page "KV cache & continuous batching", section "Visual: the
lifecycle of a request in continuous batching": 16-token blocks, a finished
request frees its blocks at once, a 50-token response uses 4 blocks and a
5000-token one 313; section "2. PagedAttention (vLLM)": blocks allocated on
demand per request; section "4. Prefix caching / prompt caching": prefix
blocks reused across requests sharing the prefix; page "LLM Serving - KV
Cache, Batching, Speculative Decoding", section "KV memory, paging and
prefix identity": shared blocks, exact token prefix, tenant salt), with the
readings the library states: only full blocks are reused; a new request
reuses its longest run of leading full blocks whose exact (salt, token
prefix) is held by a block not yet handed out again, but computes its last
prompt token; freed blocks are handed out least recently freed first (a
sequence releases its blocks last-to-first); an append into a partial block
held by another sequence goes to a private copy.

Written plainly: a block's identity is the tuple (salt, every token id of
the prefix through that block) — no hashing.  Physical block numbers are an
implementation choice, so the tests compare what is unique (cached token
counts, free counts, which (sequence, logical block) pairs share storage)
and check the rest for validity.
"""

from collections import OrderedDict

BLOCK = 16


def blocks_for(tokens):
    """ceil(tokens / 16): whole 16-token blocks (page "KV cache & continuous
    batching", section "Visual: the lifecycle of a request in continuous
    batching", counts 4 blocks for 50 tokens and 313 for 5000)."""
    return -(-tokens // BLOCK)


class BlockManagerModel:
    def __init__(self, num_blocks):
        self.num_blocks = num_blocks
        self.free = OrderedDict((b, None) for b in range(num_blocks))   # first = least recently freed
        self.refs = [0] * num_blocks
        self.ident = [None] * num_blocks          # (salt, prefix tuple) of a registered full block
        self.by_ident = {}
        self.seqs = {}                            # id -> dict(blocks, tokens, salt)

    def _alloc(self):
        b, _ = self.free.popitem(last=False)
        if self.ident[b] is not None:
            del self.by_ident[self.ident[b]]
            self.ident[b] = None
        self.refs[b] = 1
        return b

    def _release(self, b):
        self.refs[b] -= 1
        if self.refs[b] == 0:
            self.free[b] = None

    def _register(self, b, ident):
        if ident not in self.by_ident:
            self.by_ident[ident] = b
            self.ident[b] = ident

    def add(self, sid, tokens, salt=0):
        """Returns the cached token count, or None when blocks run out (state unchanged)."""
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        hits = []
        for i in range((n - 1) // BLOCK):
            b = self.by_ident.get((salt, tuple(tokens[:BLOCK * (i + 1)])))
            if b is None:
                break
            hits.append(b)
        need = blocks_for(n) - len(hits) + sum(1 for b in hits if b in self.free)
        if need > len(self.free):
            return None
        blocks = []
        for b in hits:
            if b in self.free:
                del self.free[b]
                self.refs[b] = 1
            else:
                self.refs[b] += 1
            blocks.append(b)
        while len(blocks) < blocks_for(n):
            blocks.append(self._alloc())
        for i in range(len(hits), n // BLOCK):
            self._register(blocks[i], (salt, tuple(tokens[:BLOCK * (i + 1)])))
        self.seqs[sid] = {"blocks": blocks, "tokens": tokens, "salt": salt}
        return BLOCK * len(hits)

    def append(self, sid, tokens):
        """Returns the number of block copies made, or None when blocks run out."""
        s = self.seqs[sid]
        n = len(s["tokens"])
        need = blocks_for(n + len(tokens)) - blocks_for(n)
        if n % BLOCK and self.refs[s["blocks"][-1]] > 1:
            need += 1
        if need > len(self.free):
            return None
        copies = 0
        for t in tokens:
            if len(s["tokens"]) % BLOCK == 0:
                s["blocks"].append(self._alloc())
            elif self.refs[s["blocks"][-1]] > 1:
                src = s["blocks"][-1]
                s["blocks"][-1] = self._alloc()
                self._release(src)
                copies += 1
            s["tokens"].append(int(t))
            m = len(s["tokens"])
            if m % BLOCK == 0:
                self._register(s["blocks"][-1], (s["salt"], tuple(s["tokens"])))
        return copies

    def fork(self, parent, child):
        p = self.seqs[parent]
        for b in p["blocks"]:
            self.refs[b] += 1
        self.seqs[child] = {"blocks": list(p["blocks"]), "tokens": list(p["tokens"]), "salt": p["salt"]}

    def release(self, sid):
        for b in reversed(self.seqs.pop(sid)["blocks"]):
            self._release(b)

    def sharing(self):
        """Partition of (sequence, logical block) pairs by the storage they use."""
        groups = {}
        for sid, s in self.seqs.items():
            for j, b in enumerate(s["blocks"]):
                groups.setdefault(b, []).append((sid, j))
        return sorted(sorted(g) for g in groups.values())
