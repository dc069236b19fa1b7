"""Model of the capacity/active-shape UserBuffer manager (test infrastructure only).

Follows [TE#3564] "Proposed API" and "Implementation approach in the prototype":

* the buffer is registered once at its maximum token capacity, ``[max_tokens, hidden]``,
  and never reallocated, freed or re-registered afterwards;
* each communicator keeps that capacity shape and, separately, an active shape;
* setting the active shape changes only the logical shape and the views over the buffer;
  the active ``[T, hidden]`` data is a contiguous prefix of the allocation;
* the active shape must be 2-D, nonzero, fit within the capacity, keep the hidden size,
  and have a first dimension divisible by the tensor-parallel size;
* only unquantized 2-byte bf16 buffers are in scope; quantized ones keep their capacity
  shape.

Readings (the pages leave these open):

* checks run in the order the constraints are listed, the first failure is reported,
  and a rejected call leaves the state unchanged;
* a dimension <= 0 fails the "nonzero" check; "fits within the capacity" means
  T <= capacity rows;
* the initial active shape is the capacity shape (quantized buffers are "left at their
  capacity shape"), so capacity itself must be divisible by tp;
* the reduce-scatter side holds its extra per-rank partial chunks inside the same
  capacity-sized allocation rather than a new one (same page and section): a workspace
  of tp partial slots sized by capacity, whose active part is the packed prefix of
  tp * T rows.
"""

import numpy as np

# Status names.  The C library has its own enumeration; tests compare by name.
OK = "OK"
INVALID_ARG = "INVALID_ARG"
NDIM = "NDIM"
ZERO_DIM = "ZERO_DIM"
CAPACITY = "CAPACITY"
HIDDEN_MISMATCH = "HIDDEN_MISMATCH"
TP_DIVISIBILITY = "TP_DIVISIBILITY"
DTYPE = "DTYPE"
UNSUPPORTED = "UNSUPPORTED"
BUFFER_TOO_SMALL = "BUFFER_TOO_SMALL"

ELEM_BYTES = 2  # bf16
CANARY = 0x7FA5  # a NaN pattern that no computation here produces


class ModelError(Exception):
    def __init__(self, status, msg=""):
        super().__init__(f"{status}: {msg}")
        self.status = status


def check_registration(capacity, hidden, tp_size, dtype="bf16"):
    """Status of registering a ``[capacity, hidden]`` buffer for tp_size ranks."""
    if dtype not in ("bf16", "fp8_e4m3"):
        return DTYPE
    if capacity <= 0 or hidden <= 0 or tp_size < 1:
        return INVALID_ARG
    if capacity % tp_size != 0:
        return TP_DIVISIBILITY
    return OK


def check_active_shape(shape, capacity, hidden, tp_size):
    """Status of an active-shape request, checks in the order the pages list them."""
    shape = tuple(int(d) for d in shape)
    if len(shape) != 2:
        return NDIM
    if shape[0] <= 0 or shape[1] <= 0:
        return ZERO_DIM
    if shape[0] > capacity:
        return CAPACITY
    if shape[1] != hidden:
        return HIDDEN_MISMATCH
    if shape[0] % tp_size != 0:
        return TP_DIVISIBILITY
    return OK


class UserBufferModel:
    """Host model of one registered UserBuffer plus its reduce-scatter workspace.

    ``ub`` holds ``capacity * hidden`` bf16 patterns, ``ws`` holds ``tp * capacity *
    hidden``; both start filled with ``CANARY`` so that any read or write outside an
    active region is visible.
    """

    def __init__(self, capacity, hidden, tp_size, dtype="bf16", canary=CANARY):
        st = check_registration(capacity, hidden, tp_size, dtype)
        if st != OK:
            raise ModelError(st, f"capacity={capacity} hidden={hidden} tp={tp_size} {dtype}")
        self.capacity = int(capacity)
        self.hidden = int(hidden)
        self.tp = int(tp_size)
        self.canary = canary
        self.ub = np.full(self.capacity * self.hidden, canary, dtype=np.uint16)
        self.ws = np.full(self.tp * self.capacity * self.hidden, canary, dtype=np.uint16)
        self.T = self.capacity  # initial active shape = capacity shape

    # -- shapes ------------------------------------------------------------------
    @property
    def capacity_shape(self):
        return (self.capacity, self.hidden)

    @property
    def active_shape(self):
        return (self.T, self.hidden)

    def set_active_shape(self, shape):
        st = check_active_shape(shape, self.capacity, self.hidden, self.tp)
        if st == OK:
            self.T = int(shape[0])  # nothing else changes: no allocation, no copy
        return st

    # -- views and offsets (all from the ACTIVE first dimension) ------------------
    @property
    def active_elems(self):
        return self.T * self.hidden

    @property
    def shard_rows(self):
        return self.T // self.tp

    def row_offset_elems(self, row0):
        """Element offset of active row ``row0`` in the UserBuffer (prefix layout)."""
        return row0 * self.hidden

    def shard_offset_elems(self, r):
        """Element offset of rank r's ``[T/tp, hidden]`` shard."""
        return r * self.shard_rows * self.hidden

    def partial_offset_elems(self, s, row0):
        """Element offset of row ``row0`` of partial slot s in the packed workspace."""
        return (s * self.T + row0) * self.hidden

    def active_view(self):
        return self.ub[: self.active_elems].reshape(self.T, self.hidden)

    def fill_active(self, bits):
        """Write ``[T, hidden]`` patterns into the active prefix (the gathered input)."""
        bits = np.asarray(bits, dtype=np.uint16).reshape(self.T, self.hidden)
        self.ub[: self.active_elems] = bits.ravel()

    def copy_in(self, src_bits, rows, row_offset):
        """Copy ``[rows, hidden]`` into active rows [row_offset, row_offset + rows).

        The copy-size check is against the active T ([TE#3564]: copy-size checks use the
        active element count), not the capacity.
        """
        if rows < 0 or row_offset < 0 or row_offset + rows > self.T:
            return INVALID_ARG
        o = self.row_offset_elems(row_offset)
        self.ub[o: o + rows * self.hidden] = np.asarray(src_bits, np.uint16).ravel()
        return OK
