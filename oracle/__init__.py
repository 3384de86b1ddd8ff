"""Plain CPU oracle for decode attention over a block-table (paged) KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``block_table_attention_amd`` and its HIP library) never imports,
calls or links it, and this package imports nothing from the product path.

What it computes, and where the pages define it:

* ``allocator`` -- a free-FIFO block pool with reference counts, fork, the three
  append paths (new block / write in place / copy-on-write) and release; it
  emits the physical operation trace (slot writes, block copies).
  "M5.3 - KV Memory Layout and Exact Reuse", sections 0x04A-0x04E, 0x05, 0x0AC;
  "Cache Concepts: Prefix Matching vs. Storage" (free FIFO of empty blocks).
* ``layout`` -- axis order -> row-major strides -> element/byte offsets, and the
  checked token -> (logical block, offset) -> slot -> address translator with
  its rejection order.  "M5.3", sections 0x03C-0x03I.
* ``pool`` -- the K/V pool as raw scalar bits; appends and block copies are bit
  copies.  Bit layout of the pool matches the library's documented layout.
* ``attention`` -- binary64 softmax attention of each decode query row over the
  request's contiguous logical K/V history (the plain definition that paging
  must reproduce exactly), plus the partition states (valid, m, l, u) and their
  log-sum-exp merge.  "M5.3", sections 0x0A and 0x0BA.
* ``ledgers`` -- block counts, tails, table cells, copy-on-write costs and the
  other byte/row ledgers the pages print.  "M5.3", sections 0x02, 0x05A, 0x09,
  0x0AB, 0x0BE, 0x0BI, 0x0D; "7. Memory Management and Local Model State".
* ``shared`` -- shared-prefix execution reuse over a chunk tree: the
  monolithic, Hydragen and ChunkAttention schedules and their row ledgers.
  "M5.3", sections 0x0BA-0x0BE.
* ``views`` -- kernel views of allocator blocks (P_a = q P_k) and compact
  (ragged) block tables.  "M5.3", sections 0x0AB-0x0AC.
* ``bundles`` -- cache groups with a layer axis in a declared axis order,
  whole-bundle appends and copies, and the all-or-nothing multi-group
  allocator with rollback.  "M5.3", sections 0x03B-0x03F, 0x04E-0x04F,
  0x05B-0x05C.
* ``vattention`` -- contiguous virtual K/V: the reservation, page and slot
  address algebra, the four ledgers, the slot/page lifecycle with retention
  and reclamation, and decode by request-slot index with no block table.
  "M5.3", sections 0x06A-0x06F, 0x0BJ.

Every function is pinned by ``tests/test_oracle_*.py`` against values the pages
print, closed forms, invariants, an independent library routine or brute force.
"""
