"""Writes tests/golden/oracle_small.json from oracle/ only.

The pages print no worked example (no tensors, no formulas), so the stored
values are the oracle's own output on one fixed small input; they freeze the
oracle against unintended change. The input is drawn by gdn_inputs with a
fixed seed. Run from the repo root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

import gdn_inputs  # noqa: E402
from oracle import FMT_E4M3, FMT_INT8, FMT_OFF, chunked_bwd, chunked_fwd  # noqa: E402
from oracle.qdq import qdq32  # noqa: E402

SPEC = dict(gdn_inputs.spec('varlen_int8_gqa4x16_d128'), lengths=[70, 3], Hqk=1, Hv=2,
            Dk=8, Dv=8, dtype='f32')
SEED = 7


def compute():
    x = gdn_inputs.make_inputs(SPEC, SEED, bwd=True)
    args = [x[n].double() for n in ('q', 'k', 'v', 'g', 'beta')]
    out = {}
    for tag, sf, wf in (('e4m3', FMT_E4M3, FMT_E4M3), ('int8', FMT_INT8, FMT_OFF)):
        o, ht = chunked_fwd(*args, 0.25, x['h0'].double(), x['cu_list'], state_fmt=sf,
                            w_fmt=wf, block_v=4)
        gr = chunked_bwd(*args, 0.25, x['do'].double(), x['dht'].double(), x['h0'].double(),
                         x['cu_list'], state_fmt=sf, w_fmt=wf, block_v=4)
        out[tag] = dict(o_sum=float(o.sum()), o_sq=float((o * o).sum()),
                        o_first=o[0, :4, 0, :4].reshape(-1).tolist(),
                        ht_sum=float(ht.sum()), ht_sq=float((ht * ht).sum()),
                        **{f'{k}_sq': float((v * v).sum()) for k, v in gr.items()})
    # one QDQ tile worked by hand: a = 3, d = fl32(3/448), r = fl32(1/d);
    # y = x r = [448, -224, 14.93.., 0]; E4M3 codes [448, -224, 15, 0]
    t = np.array([[3.0, -1.5, 0.1, 0.0]], np.float32)
    o8, c8, d8 = qdq32(t, FMT_E4M3, (1,))
    out['qdq_tile'] = dict(x=t.tolist(), codes=c8.tolist(), d=float(d8[0, 0]),
                           out=o8.astype(np.float64).tolist())
    return out


if __name__ == '__main__':
    with open(os.path.join(HERE, 'oracle_small.json'), 'w') as f:
        json.dump(compute(), f, indent=1)
    print('wrote oracle_small.json')
