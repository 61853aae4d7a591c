"""Cross-request prefix reuse over full pages: a radix tree keyed on token ids.

("NVIDIA TensorRT-LLM详解：架构、KV Cache、调度与部署实践", §10, cross-request KV reuse:
filled KV blocks go into a radix search tree and a new request reuses the blocks of its
longest matching prefix; §11: a block that matches only its first tokens is partly
reused by copying those tokens into a new block of the new request.)

Every node stands for one full page: its key is the page's token ids, its page the
physical page holding their K/V (one pool).  This is the lookup the kernels' block
tables need, nothing more: the serving policy around it (eviction order, reference
counting, tenant isolation) belongs to a scheduler and is not built here.  The device
side of a reuse is the block table (shared pages) and kv_copy_pages (the partly
matched page).
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(eq=False)
class _Node:
    key: tuple
    page: int
    children: dict = field(default_factory=dict)


@dataclass
class Match:
    pages: list                # physical pages of the matched full pages, in order
    partial_page: int = -1     # a cached page whose first tokens match the next ones
    partial_tokens: int = 0    # how many (copy-on-partial-reuse copies that page)


class PrefixIndex:
    def __init__(self, page_size: int):
        assert page_size >= 1
        self.P = page_size
        self._root = _Node(key=(), page=-1)
        self._count = 0

    def match(self, tokens) -> Match:
        """Longest run of full pages of `tokens` in the tree, and the best partial
        match (fewer than page_size tokens) for the page after it."""
        P, node = self.P, self._root
        m = Match(pages=[])
        i = 0
        while (i + 1) * P <= len(tokens):
            child = node.children.get(tuple(tokens[i * P:(i + 1) * P]))
            if child is None:
                break
            node = child
            m.pages.append(child.page)
            i += 1
        rest = tuple(tokens[i * P:(i + 1) * P])
        for key, child in node.children.items():
            n = 0
            while n < min(len(key), len(rest)) and key[n] == rest[n]:
                n += 1
            if n > m.partial_tokens and n < P:
                m.partial_page, m.partial_tokens = child.page, n
        return m

    def insert(self, tokens, pages):
        """Record the full pages of a sequence (tokens, and the physical page of each of
        its len(tokens) // P full pages).  Pages already in the tree (same prefix) keep
        the tree's page; returns the pages of `pages` the tree did not adopt."""
        P, node = self.P, self._root
        unused = []
        for i in range(len(tokens) // P):
            key = tuple(tokens[i * P:(i + 1) * P])
            child = node.children.get(key)
            if child is None:
                child = _Node(key=key, page=int(pages[i]))
                node.children[key] = child
                self._count += 1
            elif int(pages[i]) != child.page:
                unused.append(int(pages[i]))
            node = child
        return unused

    def __len__(self):
        return self._count
