"""Host logic of the radix-tree prefix index (no GPU)."""
from paged_kv_cache_413_amd.prefix_index import PrefixIndex

P = 4
SYS = [1, 2, 3, 4, 5, 6, 7, 8]          # a two-page shared prefix (system prompt, tool schema)


def test_second_request_reuses_the_shared_full_pages():
    idx = PrefixIndex(P)
    a = SYS + [9, 10, 11, 12, 13]
    assert idx.insert(a, [40, 41, 42]) == []
    m = idx.match(SYS + [20, 21, 22, 23, 24])
    assert m.pages == [40, 41] and m.partial_tokens == 0


def test_partial_match_of_the_next_page_is_reported_for_copying():
    idx = PrefixIndex(P)
    idx.insert(SYS + [9, 10, 11, 12], [40, 41, 42])
    m = idx.match(SYS + [9, 10, 99, 98, 97])           # [A, B, C, D] vs [A, B, X, Y]
    assert m.pages == [40, 41] and (m.partial_page, m.partial_tokens) == (42, 2)


def test_salt_isolates_tenants():
    idx = PrefixIndex(P)
    idx.insert(SYS, [40, 41], salt="tenant-a")
    assert idx.match(SYS, salt="tenant-b").pages == []
    assert idx.match(SYS, salt="tenant-a").pages == [40, 41]


def test_duplicate_insert_keeps_the_tree_page():
    idx = PrefixIndex(P)
    idx.insert(SYS, [40, 41])
    assert idx.insert(SYS + [1, 1, 1, 1], [50, 51, 52]) == [50, 51]
    assert idx.match(SYS + [1, 1, 1, 1]).pages == [40, 41, 52]


def test_eviction_takes_free_leaves_by_priority_then_age():
    idx = PrefixIndex(P)
    idx.insert(SYS + [9, 9, 9, 9], [40, 41, 42], priority=35)
    idx.insert(SYS + [7, 7, 7, 7], [40, 41, 43], priority=80)     # shares 40, 41
    idx.insert([5, 5, 5, 5], [44], priority=35)
    m = idx.match(SYS + [9, 9, 9, 9])                              # a request holds 40, 41, 42
    # free leaves: 43 (priority 80), 44 (priority 35, newer than 42 but 42 is held)
    assert idx.evict(1) == [44]
    assert idx.evict(5) == [43]                 # 42 held; 40, 41 are not leaves while 42 stays
    idx.release(m.pages)
    assert idx.evict(5) == [42, 41, 40]         # the chain unwinds leaf by leaf
    assert len(idx) == 0
