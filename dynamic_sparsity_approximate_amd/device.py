"""A prepared matrix resident in HBM with its own workspace (torch owns the memory)."""
from __future__ import annotations

import numpy as np

from . import binding as B


class EffortMatrix:
    """Layout of one fp16 matrix W[in][out] on a device, ready for effort_matvec.

    The host converter runs once; the blob is copied to device memory once; each
    call then reads only the device copy.  `batch` sizes the workspace.
    """

    def __init__(self, w_fp16, P: int = 16, groups: int = 0, device="cuda", batch: int = 1,
                 entry_format: int = B.EFFORT_ENTRY_U32, crop: int = 0):
        import torch

        self.desc, blob = B.effort_prepare_host(w_fp16, P, groups, entry_format, crop)
        self.in_dim = int(self.desc.in_dim)
        self.out_dim = int(self.desc.out_dim)
        self.P = int(self.desc.probes_per_row)
        self.groups = int(self.desc.groups)
        self.layout_bytes = int(self.desc.total_bytes)
        self.layout = torch.from_numpy(blob).to(device)
        self.batch = batch
        self.ws_bytes = B.effort_workspace_bytes(self.desc, batch)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=device)

    @classmethod
    def from_blob(cls, desc, layout_dev, batch: int = 1):
        """Wrap an existing device copy of a prepared blob (shares `layout_dev`)."""
        import torch

        self = cls.__new__(cls)
        self.desc = desc
        self.in_dim, self.out_dim = int(desc.in_dim), int(desc.out_dim)
        self.P, self.groups = int(desc.probes_per_row), int(desc.groups)
        self.layout_bytes = int(desc.total_bytes)
        self.layout = layout_dev
        self.batch = batch
        self.ws_bytes = B.effort_workspace_bytes(desc, batch)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=layout_dev.device)
        return self

    def matvec(self, v, effort: float, y=None, stream=None, record=None):
        """y = approximate v . W.  `record` = (Recorder, key): the same call with
        its parity outputs recorded under `key`."""
        import torch

        if y is None:
            y = torch.empty(self.out_dim, dtype=torch.float32, device=v.device)
        if record is None:
            B.effort_matvec(self.desc, self.layout, v, effort, y, self.ws, self.ws_bytes, stream)
        else:
            rec, key = record
            cutoff, K, rk, fp = rec.single(key, self.in_dim)
            B.effort_matvec_debug(self.desc, self.layout, v, effort, y, self.ws, self.ws_bytes, cutoff,
                                  K, rk, fp, None, None, stream)
        return y

    def matvec_batched(self, v, effort: float, y=None, stream=None):
        import torch

        b = v.shape[0]
        if y is None:
            y = torch.empty((b, self.out_dim), dtype=torch.float32, device=v.device)
        B.effort_matvec_batched(self.desc, self.layout, v, b, effort, y, self.ws, self.ws_bytes, stream)
        return y

    def matvec_batched_debug(self, v, effort: float, with_mask: bool = False, stream=None) -> list:
        """matvec_batched with every vector's parity outputs (the same route
        and kernels, recording on); one dict per vector."""
        import torch

        dev = v.device
        b = v.shape[0]
        y = torch.empty((b, self.out_dim), dtype=torch.float32, device=dev)
        cutoff = torch.empty(b, dtype=torch.float32, device=dev)
        K = torch.empty(2 * b, dtype=torch.int64, device=dev)
        row_kept = torch.empty((b, self.in_dim), dtype=torch.int32, device=dev)
        fp = torch.empty(b, dtype=torch.int64, device=dev)
        mask = (torch.empty((b, self.in_dim, self.out_dim), dtype=torch.uint8, device=dev)
                if with_mask else None)
        B.effort_matvec_batched_debug(self.desc, self.layout, v, b, effort, y, self.ws, self.ws_bytes,
                                      cutoff, K, row_kept, fp, mask, stream)
        torch.cuda.synchronize(dev)
        yh, ch, Kh = y.cpu().numpy(), cutoff.cpu().numpy(), K.cpu().numpy()
        rk, fph = row_kept.cpu().numpy().astype(np.int64), fp.cpu().numpy().view(np.uint64)
        mk = mask.cpu().numpy() if mask is not None else None
        return [{"y": yh[k], "cutoff": ch[k], "K": int(Kh[2 * k]), "Kprime": int(Kh[2 * k + 1]),
                 "row_kept": rk[k], "fingerprint": int(fph[k]), "total_kept": int(rk[k].sum()),
                 "mask": mk[k] if mk is not None else None} for k in range(b)]

    def matvec_debug(self, v, effort: float, with_mask: bool = True, stream=None) -> dict:
        import torch

        dev = v.device
        y = torch.empty(self.out_dim, dtype=torch.float32, device=dev)
        cutoff = torch.empty(1, dtype=torch.float32, device=dev)
        K = torch.empty(2, dtype=torch.int64, device=dev)
        row_kept = torch.empty(self.in_dim, dtype=torch.int32, device=dev)
        fp = torch.empty(1, dtype=torch.int64, device=dev)
        mask = (torch.empty((self.in_dim, self.out_dim), dtype=torch.uint8, device=dev)
                if with_mask else None)
        status = torch.empty(1, dtype=torch.int32, device=dev)
        B.effort_matvec_debug(self.desc, self.layout, v, effort, y, self.ws, self.ws_bytes, cutoff, K,
                              row_kept, fp, mask, status, stream)
        torch.cuda.synchronize(dev)
        out = {
            "y": y.cpu().numpy(),
            "cutoff": cutoff.cpu().numpy()[0],
            "K": int(K[0].item()),
            "Kprime": int(K[1].item()),
            "row_kept": row_kept.cpu().numpy().astype(np.int64),
            "fingerprint": int(fp.cpu().numpy().view(np.uint64)[0]),
            "mask": mask.cpu().numpy() if mask is not None else None,
            "v_nonfinite": bool(int(status.item()) & 1),
            "crop_reached": bool(int(status.item()) & 2),
        }
        out["total_kept"] = int(out["row_kept"].sum())
        return out


class Recorder:
    """Device buffers for the parity outputs of many calls (a decode step, an
    expert block): each call site records under a key, and `results()` returns
    key -> {cutoff, K, Kprime, row_kept, fingerprint} after a synchronize.
    The calls run the same kernels as unrecorded ones with recording on."""

    def __init__(self, device):
        self.device = device
        self._slots = {}  # key -> (cutoff, K, row_kept, fingerprint, index)

    def single(self, key, in_dim):
        import torch

        d = self.device
        bufs = (torch.empty(1, dtype=torch.float32, device=d), torch.empty(2, dtype=torch.int64, device=d),
                torch.empty(in_dim, dtype=torch.int32, device=d), torch.empty(1, dtype=torch.int64, device=d))
        self._slots[key] = bufs + (0,)
        return bufs

    def multi(self, keys, in_dims):
        import torch

        d, c = self.device, len(keys)
        cutoff = torch.empty(c, dtype=torch.float32, device=d)
        K = torch.empty(2 * c, dtype=torch.int64, device=d)
        fp = torch.empty(c, dtype=torch.int64, device=d)
        rks = [torch.empty(m, dtype=torch.int32, device=d) for m in in_dims]
        for j, k in enumerate(keys):
            self._slots[k] = (cutoff, K, rks[j], fp, j)
        return cutoff, K, rks, fp

    def keys(self):
        return list(self._slots)

    def results(self) -> dict:
        import torch

        torch.cuda.synchronize(self.device)
        out = {}
        for k, (cutoff, K, rk, fp, j) in self._slots.items():
            Kh = K.cpu().numpy()
            out[k] = {"cutoff": cutoff.cpu().numpy()[j], "K": int(Kh[2 * j]), "Kprime": int(Kh[2 * j + 1]),
                      "row_kept": rk.cpu().numpy().astype(np.int64),
                      "fingerprint": int(fp.cpu().numpy().view(np.uint64)[j])}
        return out


class EffortGroup:
    """Independent (matrix, vector) pairs multiplied by one call: one launch of
    each kernel for all of them.  Holds its own workspace; the matrices'
    layouts are shared, not copied."""

    def __init__(self, mats):
        import torch

        mats = list(mats)
        if not mats:
            raise ValueError("an EffortGroup needs at least one matrix")
        self.mats = mats
        self.descs = [m.desc for m in mats]
        self.layouts = [m.layout for m in mats]
        self.ws_bytes = B.effort_workspace_bytes_multi(self.descs)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=mats[0].layout.device)

    def matvec(self, vs, efforts, ys=None, stream=None, record=None):
        """ys[j] = approximate vs[j] . W_j at efforts[j]; `vs` may be one vector
        shared by all matrices, `efforts` one float.  `record` = (Recorder,
        keys): the same call with each pair's parity outputs recorded under
        keys[j]."""
        import torch

        if ys is None:
            dev = (vs[0] if isinstance(vs, (list, tuple)) else vs).device
            ys = [torch.empty(m.out_dim, dtype=torch.float32, device=dev) for m in self.mats]
        if record is None:
            B.effort_matvec_multi(self.descs, self.layouts, vs, efforts, ys, self.ws, self.ws_bytes,
                                  stream)
        else:
            rec, keys = record
            cutoff, K, rks, fp = rec.multi(keys, [m.in_dim for m in self.mats])
            B.effort_matvec_multi_debug(self.descs, self.layouts, vs, efforts, ys, self.ws,
                                        self.ws_bytes, cutoff, K, rks, fp, stream)
        return ys
