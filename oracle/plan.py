"""Oracle planner: which rows a link recomputes and where every token sits.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this module;
it exists so that tests, the smoke check and the CPU baseline of the benchmark
can check the product planner against an independent statement of the rules.

Rules, each from the pages:

* A prompt is linked from segments: an optional cached prefix, the linked
  chunks in prompt order, and the request's new suffix. Chunks were compiled on
  their own starting at position 0 and are placed at their running offset in
  the prompt (EPIC, atlas.scime.ai summary, "Approach").
* LegoLink-k recomputes the first k tokens of every chunk (k <= 32 in the
  paper; any k >= 0 is accepted here, k = 0 being the link half of
  LegoLink-0) (EPIC summary, "Approach" and the ablation table).
* Block-level recompute refreshes the whole first page of each chunk, which is
  the only request-specific page of the chunk (MEPIC, searcharxiv.org
  abstract).
* Chunk KV is page aligned: every segment starts on a fresh page and its last
  page is padded (MEPIC abstract). Pages that hold no recomputed row are shared
  with the store; the others are private to the request.
* The suffix is new text: all its rows are computed.
* The prefix is cached and not recomputed (reading of the pages, which never
  refresh a prefix); ``recompute_all`` selects every row of every segment and
  is the full-recompute comparator.
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class Segment:
    kind: str               # "prefix" | "chunk" | "suffix"
    chunk_id: int | None    # store id of a cached segment, None for the suffix
    length: int
    start: int              # absolute position of the segment's first token
    recompute: int          # leading rows of the segment that are recomputed


@dataclass(frozen=True)
class LogicalPage:
    segment: int            # index into the request's segment list
    index: int              # page number inside its segment
    pos0: int               # absolute position of slot 0
    valid: int              # slots holding tokens; the rest are padding
    private: bool           # request-private (holds recomputed rows) or shared
    n_new: int              # leading slots written with recomputed rows
    cow: bool               # private page that also keeps cached rows
    source: tuple | None    # (chunk id, page number) of the stored page read or copied


def link_segments(*, chunk_ids, chunk_lens, suffix_len, k, block_level, page_size,
                  prefix_id=None, prefix_len=0, pos_offset=0, recompute_all=False):
    """Segments of one request with their absolute starts and recompute counts."""
    if k < 0:
        raise ValueError("k must be >= 0")
    segs = []
    pos = pos_offset
    if prefix_id is not None:
        r = prefix_len if recompute_all else 0
        segs.append(Segment("prefix", prefix_id, prefix_len, pos, r))
        pos += prefix_len
    for cid, length in zip(chunk_ids, chunk_lens):
        if recompute_all:
            r = length
        elif block_level:
            r = min(page_size, length)
        else:
            r = min(k, length)
        segs.append(Segment("chunk", cid, length, pos, r))
        pos += length
    if suffix_len > 0:
        segs.append(Segment("suffix", None, suffix_len, pos, suffix_len))
    return segs


def total_tokens(segs) -> int:
    return sum(s.length for s in segs)


def selected_positions(segs) -> list[int]:
    """Absolute positions of the recomputed rows, in prompt order."""
    return [s.start + j for s in segs for j in range(s.recompute)]


def token_positions(segs) -> list[int]:
    """Absolute position of every token of the request, in prompt order."""
    return [s.start + j for s in segs for j in range(s.length)]


def logical_pages(segs, page_size: int) -> list[LogicalPage]:
    pages = []
    for si, s in enumerate(segs):
        n_pages = -(-s.length // page_size)
        for q in range(n_pages):
            valid = min(page_size, s.length - q * page_size)
            n_new = max(0, min(s.recompute - q * page_size, valid))
            if s.kind == "suffix":
                pages.append(LogicalPage(si, q, s.start + q * page_size, valid, True, valid, False, None))
            elif n_new > 0:
                cow = n_new < valid
                pages.append(LogicalPage(si, q, s.start + q * page_size, valid, True, n_new, cow,
                                         (s.chunk_id, q) if cow else None))
            else:
                pages.append(LogicalPage(si, q, s.start + q * page_size, valid, False, 0, False,
                                         (s.chunk_id, q)))
    return pages


def position_map(pages, page_size: int) -> list[int]:
    """Absolute position held by each logical slot, -1 for padding."""
    out = []
    for p in pages:
        for s in range(page_size):
            out.append(p.pos0 + s if s < p.valid else -1)
    return out


def row_slots(segs, page_size: int) -> list[tuple[int, int]]:
    """(logical page, slot) where each recomputed row is written, in row order."""
    first_page = []
    n = 0
    for s in segs:
        first_page.append(n)
        n += -(-s.length // page_size)
    out = []
    for si, s in enumerate(segs):
        for j in range(s.recompute):
            out.append((first_page[si] + j // page_size, j % page_size))
    return out
