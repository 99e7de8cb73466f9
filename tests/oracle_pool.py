"""The oracle's RFQ encoding of a whole configuration's X, computed in row
chunks on a pool of CPU processes (the oracle quantizes about 1.4 M elements
per second per core; the 32768 x 13824 activation has 453 M).

Workers are started with "spawn" and import only NumPy, the oracle and the
seeded generators: they never touch the GPU. Each regenerates its own rows
from the configuration's seeds (bit for bit the rows the GPU was fed) and
returns the oracle's packed codes and scales for them."""
import multiprocessing
import os

import numpy as np

import oracle
import workloads

CHUNK_ROWS = 512


def _rfq_rows(args):
    name, r0, r1 = args
    cfg = workloads.CONFIGS[name]
    qx, sx, qr, sr = oracle.residual_quantize(oracle.bf16_bits_to_f64(workloads.x_bf16(cfg, r0, r1)))
    return r0, oracle.pack_codes(qx), sx, oracle.pack_codes(qr), sr


def workers():
    return max(1, min(12, os.cpu_count() or 1))


class RfqCodesFull:
    """The oracle's (qx, sx, qr, sr) for all M rows of cfg's X (packed codes
    uint8 [M, K/2], scales uint8 [M, K/32]), started on the pool at
    construction so that the caller can run the GPU meanwhile; result()
    waits for it."""

    def __init__(self, cfg, nproc=None):
        self.cfg = cfg
        jobs = [(cfg.name, r0, min(r0 + CHUNK_ROWS, cfg.M)) for r0 in range(0, cfg.M, CHUNK_ROWS)]
        self.pool = multiprocessing.get_context("spawn").Pool(nproc or workers())
        self.pending = self.pool.map_async(_rfq_rows, jobs, chunksize=1)

    def result(self, timeout=None):
        M, K = self.cfg.M, self.cfg.K
        qx = np.empty((M, K // 2), np.uint8)
        qr = np.empty((M, K // 2), np.uint8)
        sx = np.empty((M, K // 32), np.uint8)
        sr = np.empty((M, K // 32), np.uint8)
        try:
            for r0, a, b, c, d in self.pending.get(timeout):
                r1 = r0 + a.shape[0]
                qx[r0:r1], sx[r0:r1], qr[r0:r1], sr[r0:r1] = a, b, c, d
        finally:
            self.close()
        return qx, sx, qr, sr

    def close(self):
        if self.pool is not None:
            self.pool.terminate()
            self.pool.join()
            self.pool = None
