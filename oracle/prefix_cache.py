"""Radix-tree prefix cache over the block manager (test infrastructure; see oracle/__init__).

[KVM] cross-turn prefix caching (Table 2, Definition 0.2, Figure 6):

* every node binds a run of prompt tokens (``tokens``) to the ordered physical
  blocks that hold their K/V (``blocks``), keeps its ``children``, its
  ``parent``, a ``ref_count`` of the live requests using it and a
  ``last_access`` time;
* longest prefix match walks from the root along the prompt; only completely
  filled blocks are shared, so the usable hit is rounded down to a block
  boundary, S_usable = floor(S_match / B) * B, and the S_match mod B tail
  tokens are recomputed (block-aligned truncation);
* when a request ends its blocks are not freed: the tree keeps them (here: one
  reference per block in the block manager) and the node becomes dormant once
  its ref_count is 0;
* eviction, leaf first: dormant leaves are taken oldest last_access first; a
  taken leaf gives its blocks back and leaves its parent's children; a parent
  left childless and dormant becomes a candidate in turn; this repeats until
  enough blocks are free or no candidate is left.

Readings (the pages leave these open; the plainest that fits the rest):

* since only full blocks are shared, every edge holds whole blocks, and a
  child is keyed by the tokens of its first block (two children may start with
  the same token and differ later in that block);
* S_match counts tokens: full blocks matched along the tree plus the longest
  common run of tokens with the next block of any child;
* ``last_access`` is a counter advanced by every lookup, attach and insert,
  given to every node the operation walks; ties between candidates go to the
  node created first;
* a request attaches to its matched path (``attach``: its table starts with
  those blocks, the path's nodes gain a ref_count) or inserts its own prefix
  after computing it (``insert``: missing nodes adopt the request's blocks,
  the request's path gains a ref_count); releasing the request removes its
  ref_counts;
* an inserted run that ends inside an existing edge splits nothing; a run that
  diverges inside an edge splits it at the block boundary before the
  divergence.
"""

from __future__ import annotations


class Node:
    __slots__ = ("tokens", "blocks", "children", "parent", "ref_count", "last_access", "order")

    def __init__(self, tokens, blocks, parent, order):
        self.tokens = list(tokens)
        self.blocks = list(blocks)
        self.children = {}
        self.parent = parent
        self.ref_count = 0
        self.last_access = 0
        self.order = order


class PrefixCache:
    def __init__(self, bm):
        self.bm = bm
        self.B = bm.block_size
        self.root = Node([], [], None, 0)
        self.clock = 0
        self.created = 0
        self.pins = {}  # request -> nodes whose ref_count it holds

    # -- helpers -------------------------------------------------------------
    def _key(self, tokens, at):
        return tuple(tokens[at:at + self.B])

    def _tick(self):
        self.clock += 1
        return self.clock

    def _walk(self, tokens, limit):
        """Nodes whose whole edges match tokens[:limit] block by block, the blocks
        they give, and (node, edge blocks matched) where the walk stopped."""
        B = self.B
        node, at, path, blocks = self.root, 0, [], []
        while at + B <= limit:
            child = node.children.get(self._key(tokens, at))
            if child is None:
                break
            e = 0
            while e < len(child.blocks) and at + B <= limit and \
                    child.tokens[e * B:(e + 1) * B] == list(tokens[at:at + B]):
                e += 1
                at += B
            blocks += child.blocks[:e]
            if e < len(child.blocks):
                return path, blocks, (child, e)
            path.append(child)
            node = child
        return path, blocks, (node, None)

    # -- lookup ----------------------------------------------------------------
    def match(self, tokens):
        """(S_match, S_usable, blocks) of the longest cached prefix of ``tokens``."""
        tokens = list(tokens)
        path, blocks, (node, e) = self._walk(tokens, len(tokens))
        full = len(blocks) * self.B
        # tokens matched inside the next block, which is not shared
        if e is not None:
            candidates = [node.tokens[e * self.B:(e + 1) * self.B]]
        else:
            candidates = [c.tokens[:self.B] for c in node.children.values()]
        extra = 0
        for cand in candidates:
            k = 0
            while k < len(cand) and full + k < len(tokens) and cand[k] == tokens[full + k]:
                k += 1
            extra = max(extra, k)
        t = self._tick()
        for n in path + ([node] if e is not None else []):
            n.last_access = t
        return full + extra, full, blocks

    # -- requests --------------------------------------------------------------
    def attach(self, seq, tokens):
        """New request ``seq`` whose table starts with the cached blocks of the longest
        block-aligned prefix of ``tokens``; returns the number of cached tokens."""
        tokens = list(tokens)
        path, blocks, (node, e) = self._walk(tokens, len(tokens))
        self.bm.add_with_blocks(seq, blocks)
        pinned = path + ([node] if e is not None else [])
        t = self._tick()
        for n in pinned:
            n.ref_count += 1
            n.last_access = t
        self.pins[seq] = pinned
        return len(blocks) * self.B

    def insert(self, seq, tokens):
        """Cache the full blocks of tokens[:len(tokens)], which ``seq`` holds as the first
        len(tokens) tokens of its table.  Missing nodes adopt the request's blocks."""
        tokens = list(tokens)
        B = self.B
        table = self.bm.table(seq)
        if len(tokens) > self.bm.length(seq):
            raise ValueError("more tokens than the sequence holds")
        n_blocks = len(tokens) // B
        node, at, path = self.root, 0, []
        while at < n_blocks * B:
            child = node.children.get(self._key(tokens, at))
            if child is None:
                self.created += 1
                leaf = Node(tokens[at:n_blocks * B], table[at // B:n_blocks], node, self.created)
                self.bm.retain(leaf.blocks)
                node.children[self._key(tokens, at)] = leaf
                path.append(leaf)
                break
            e = 0
            while e < len(child.blocks) and at + B <= n_blocks * B and \
                    child.tokens[e * B:(e + 1) * B] == tokens[at:at + B]:
                e += 1
                at += B
            if e < len(child.blocks) and at < n_blocks * B:
                # diverges inside the edge: split at the block boundary
                self.created += 1
                upper = Node(child.tokens[:e * B], child.blocks[:e], node, self.created)
                upper.ref_count = child.ref_count
                upper.last_access = child.last_access
                for req, nodes in self.pins.items():
                    if child in nodes:
                        nodes.append(upper)
                node.children[self._key(child.tokens, 0)] = upper
                child.tokens = child.tokens[e * B:]
                child.blocks = child.blocks[e:]
                child.parent = upper
                upper.children[self._key(child.tokens, 0)] = child
                path.append(upper)
                node = upper
                continue
            path.append(child)
            node = child
        t = self._tick()
        pinned = self.pins.setdefault(seq, [])
        for n in path:
            n.last_access = t
            if n not in pinned:
                n.ref_count += 1
                pinned.append(n)
        return n_blocks * B

    def release(self, seq):
        """The request ends: its nodes lose its ref_count; its table is released."""
        for n in self.pins.pop(seq, []):
            n.ref_count -= 1
        return self.bm.release(seq)

    # -- eviction ----------------------------------------------------------------
    def _dormant_leaves(self):
        out, stack = [], [self.root]
        while stack:
            n = stack.pop()
            stack.extend(n.children.values())
            if n is not self.root and not n.children and n.ref_count == 0:
                out.append(n)
        return out

    def evict(self, target_free):
        """Leaf-first LRU eviction until the free list holds target_free blocks or no
        dormant leaf is left.  Returns the evicted nodes' blocks, in eviction order."""
        freed_blocks = []
        queue = self._dormant_leaves()
        while self.bm.n_free() < target_free and queue:
            leaf = min(queue, key=lambda n: (n.last_access, n.order))
            queue.remove(leaf)
            self.bm.drop(leaf.blocks)
            freed_blocks += leaf.blocks
            parent = leaf.parent
            del parent.children[self._key(leaf.tokens, 0)]
            if parent is not self.root and not parent.children and parent.ref_count == 0:
                queue.append(parent)
        return freed_blocks

    # -- introspection -------------------------------------------------------------
    def nodes(self):
        out, stack = [], list(self.root.children.values())
        while stack:
            n = stack.pop()
            out.append(n)
            stack.extend(n.children.values())
        return out

    def cached_blocks(self):
        return sum(len(n.blocks) for n in self.nodes())


def prefill_flops(n_params, prefix_tokens, n_layers, d_model):
    """Work a cached prefix saves ([KVM] estimate 0.4): 2 N S for the linear layers plus
    4 L d_model S^2 for self-attention over the prefix."""
    return 2 * n_params * prefix_tokens + 4 * n_layers * d_model * prefix_tokens ** 2
