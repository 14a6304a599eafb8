"""Shared parity gate of the GPU tests: relative Frobenius error against the
oracle over the whole compared tensor AND over every (b, h) slice of it, both
held to the same tolerance, so that one wrong head (or one wrong row of a short
sequence) cannot hide inside an otherwise accurate tensor."""
import numpy as np

import oracle


def check(tag, got, ref, tol, lead=2):
    """Assert rel_frobenius(got, ref) <= tol over the whole tensor and for each
    slice over the first `lead` axes (none when the tensor has fewer than
    lead + 1 axes); the outputs must be finite."""
    got = np.asarray(got)
    whole = oracle.rel_frobenius(got, ref)
    msg = f"[parity] {tag}: rel_fro={whole:.3e}"
    worst = None
    if got.ndim > lead and got.size:
        per = oracle.rel_frobenius_per_slice(got, ref, lead)
        worst = float(per.max())
        msg += f" worst (b,h) {worst:.3e} at {np.unravel_index(int(per.argmax()), per.shape)}"
    print(msg + f" (tol {tol:.0e})", flush=True)
    assert np.all(np.isfinite(got)), f"{tag}: non-finite outputs"
    assert whole <= tol, f"{tag}: relative Frobenius error {whole:.3e} > {tol:.0e}"
    assert worst is None or worst <= tol, f"{tag}: worst (b, h) relative Frobenius error {worst:.3e} > {tol:.0e}"
    return whole


class HeadGroups:
    """Accumulates a full-size comparison made one head group at a time: the
    whole-tensor error from the groups' norm parts, and the per-(b, h) errors."""

    def __init__(self, tag, tol):
        self.tag, self.tol, self.parts, self.worst = tag, tol, [], (0.0, None)

    def add(self, got, ref, h0):
        self.parts.append(oracle.frobenius_parts(got, ref))
        per = oracle.rel_frobenius_per_slice(got, ref, 2)
        i = np.unravel_index(int(per.argmax()), per.shape)
        assert np.all(np.isfinite(np.asarray(got))), f"{self.tag}: non-finite outputs"
        if per[i] >= self.worst[0]:
            self.worst = (float(per[i]), (int(i[0]), h0 + int(i[1])))
        return per

    def finish(self):
        whole = oracle.combine_rel_frobenius(self.parts)
        print(f"[parity] {self.tag}: whole tensor rel_fro={whole:.3e}, worst (b,h) {self.worst[0]:.3e} at "
              f"{self.worst[1]} (tol {self.tol:.0e})", flush=True)
        assert whole <= self.tol, f"{self.tag}: relative Frobenius error {whole:.3e} > {self.tol:.0e}"
        assert self.worst[0] <= self.tol, f"{self.tag}: worst (b, h) error {self.worst[0]:.3e} > {self.tol:.0e}"
        return whole
