"""Cross-request prefix reuse over full pages: a radix tree keyed on token ids.

("NVIDIA TensorRT-LLM详解：架构、KV Cache、调度与部署实践", §10, cross-request KV reuse:
filled KV blocks go into a radix search tree, a new request reuses the blocks of its
longest matching prefix, blocks are evicted by priority (0..100, lowest first) and
then least recent use, and only requests with the same cache salt share blocks; §11:
a block that matches only its first tokens is partly reused by copying those tokens
into a new block, and only leaf blocks are evicted.)

Every node stands for one full page: its key is the page's token ids, its page the
physical page holding their K/V (layer-independent here: one pool).  Host-side
bookkeeping only; the device side of a reuse is the block table (shared pages) and
kv_copy_pages (the partly matched page).
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(eq=False)
class _Node:
    key: tuple
    page: int
    parent: "_Node | None"
    children: dict = field(default_factory=dict)
    refs: int = 0            # requests holding the page now
    priority: int = 35
    tick: int = 0            # last use


@dataclass
class Match:
    pages: list                # physical pages of the matched full pages, in order
    partial_page: int = -1     # a cached page whose first tokens match the next ones
    partial_tokens: int = 0    # how many (copy-on-partial-reuse copies that page)



class PrefixIndex:
    def __init__(self, page_size: int):
        assert page_size >= 1
        self.P = page_size
        self._roots: dict = {}           # salt -> root node
        self._tick = 0
        self._by_page: dict = {}         # page -> node

    # ---- lookup -------------------------------------------------------------------
    def match(self, tokens, salt=0, acquire=True) -> Match:
        """Longest run of full pages of `tokens` in the tree of `salt`, and the best
        partial match for the page after it.  With acquire, every matched node gains a
        reference (release() drops it) and counts as just used."""
        P, node = self.P, self._roots.get(salt)
        m = Match(pages=[])
        if node is None:
            return m
        self._tick += 1
        i = 0
        while (i + 1) * P <= len(tokens):
            child = node.children.get(tuple(tokens[i * P:(i + 1) * P]))
            if child is None:
                break
            node = child
            m.pages.append(child.page)
            if acquire:
                child.refs += 1
                child.tick = self._tick
            i += 1
        rest = tuple(tokens[i * P:(i + 1) * P])
        for key, child in node.children.items():
            n = 0
            while n < min(len(key), len(rest)) and key[n] == rest[n]:
                n += 1
            if n > m.partial_tokens and n < P:
                m.partial_page, m.partial_tokens = child.page, n
        return m

    # ---- insertion and release --------------------------------------------------------
    def insert(self, tokens, pages, salt=0, priority=35):
        """Record the full pages of a sequence (tokens, and the physical page of each of
        its len(tokens) // P full pages).  Pages already in the tree (same prefix) keep
        the tree's page; returns the pages of `pages` the tree did not adopt."""
        P = self.P
        node = self._roots.setdefault(salt, _Node(key=(), page=-1, parent=None))
        self._tick += 1
        unused = []
        for i in range(len(tokens) // P):
            key = tuple(tokens[i * P:(i + 1) * P])
            child = node.children.get(key)
            if child is None:
                child = _Node(key=key, page=int(pages[i]), parent=node, priority=priority, tick=self._tick)
                node.children[key] = child
                self._by_page[child.page] = child
            else:
                if int(pages[i]) != child.page:
                    unused.append(int(pages[i]))
                child.priority = max(child.priority, priority)
                child.tick = self._tick
            node = child
        return unused

    def release(self, pages):
        """Drop one reference from each of these tree pages (a request finished)."""
        for p in pages:
            node = self._by_page.get(int(p))
            if node is not None and node.refs > 0:
                node.refs -= 1

    # ---- eviction -------------------------------------------------------------------
    def evict(self, count: int):
        """Remove up to `count` leaves that no request holds -- lowest priority first,
        then least recently used -- and return their pages (free for reuse).  A parent
        becomes a leaf, and so a candidate, once its children are gone."""
        freed = []
        while len(freed) < count:
            leaves = [n for n in self._by_page.values() if not n.children and n.refs == 0]
            if not leaves:
                break
            victim = min(leaves, key=lambda n: (n.priority, n.tick))
            del victim.parent.children[victim.key]
            del self._by_page[victim.page]
            freed.append(victim.page)
        return freed

    def __len__(self):
        return len(self._by_page)
