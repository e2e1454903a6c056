"""Shared helpers of the GPU parity tests: seeded inputs from p3d_synth, the
two independent camera constructions, host<->device transfers and the
tolerance checks. Each side computes from the same drawn inputs; nothing the
GPU produces is ever fed to the oracle."""
import numpy as np
import torch

import p3d_synth as synth


def to_dev(a, bf16=False):
    """numpy -> cuda tensor; uint16 arrays holding bf16 bits -> bfloat16."""
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if bf16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.cuda()


def to_host(t):
    """cuda tensor -> numpy (bfloat16 -> uint16 bits)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(
        np.float32).astype(np.float64)


def distances_spec(w):
    return [w.distance] * w.batch


def product_cameras(p3d, fovs, dists, image_size):
    cams = []
    for a, d in zip(fovs, dists):
        if d is None:
            d = p3d.p3d_distance_from_fov(a, image_size, 0)
        cams.append(p3d.p3d_make_camera(a, d))
    return cams


def oracle_cameras(o, fovs, dists, image_size):
    fs, ds = [], []
    for a, d in zip(fovs, dists):
        if d is None:
            d = o.distance_from_fov(a, image_size, 0)
        f, dd = o.camera(a, d)
        fs.append(f)
        ds.append(dd)
    return np.array(fs, np.float32), np.array(ds, np.float32)


class Inputs:
    """Seeded inputs of one workload (numpy, host)."""

    def __init__(self, w):
        self.w = w
        self.coords = synth.coords(w)
        self.n = w.n_tokens
        self.n_null = w.n_null
        self.feat = synth.feature_map(w)
        self.weight = synth.weight(w)
        self.bias = synth.bias(w)
        self.fovs = synth.fovs(w)
        self.dists = distances_spec(w)
        self.bf16 = w.dtype == "bf16"


def check_fp32_linear(Y_gpu, Y_orc, absmag, tol=1e-5):
    """|Y_gpu - Y| <= tol * (sum_c |W||S| + |b|) per element."""
    err = np.abs(Y_gpu.astype(np.float64) - Y_orc)
    bad = err > tol * absmag + 1e-30
    assert not bad.any(), "fp32 proj_linear: %d elements off, worst %.3e (bound %.3e)" % (
        bad.sum(), (err / (absmag + 1e-30)).max(), tol)


def check_bf16_linear(Y_gpu_bits, Y_orc, tol=2e-2):
    """bf16 proj_linear output: per element |Y_gpu - Y| <= tol (|Y| + rms of
    its row), and max |diff| / max |Y| <= tol over the whole output."""
    Yg = bf16_to_f64(Y_gpu_bits)
    err = np.abs(Yg - Y_orc)
    rms = np.sqrt(np.mean(Y_orc ** 2, axis=1, keepdims=True))
    bad = err > tol * (np.abs(Y_orc) + rms)
    assert not bad.any(), "bf16 proj_linear: %d elements off, worst rel %.3e" % (
        bad.sum(), (err / (np.abs(Y_orc) + rms + 1e-30)).max())
    scale = np.abs(Y_orc).max()
    assert err.max() <= tol * scale, "bf16 proj_linear: max|diff| %.3e vs max|Y| %.3e" % (
        err.max(), scale)
    return err.max() / max(scale, 1e-30), np.corrcoef(Yg.ravel(), Y_orc.ravel())[0, 1]
