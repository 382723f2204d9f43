"""Symbolic tensor linking and the single-launch mixed-precision trainer.

[LS2] sec. 2.3 (and [L10] technique 3, slide 29): at initialisation the
trainer allocates one contiguous workspace, copies every fp16 parameter (and
gradient) into it in order, and re-points each parameter at its slice.  From
then on one kernel launch updates the whole model; no fp32 master copy of the
parameters exists -- only the Adam moments are fp32.

Each parameter's slice starts at a multiple of 8 elements (16 bytes) so the
kernel's 16-byte accesses stay aligned; the padding elements are zero and stay
zero (p = 0, g = 0 gives m = v = 0 and p unchanged).
"""

import torch

from . import ops

ALIGN = 8


class Workspace:
    """One flat fp16 parameter buffer, one flat fp16 gradient buffer, fp32 moments."""

    def __init__(self, params, device=None):
        self.params = [p for p in params]
        if not self.params:
            raise ValueError("no parameters to link")
        device = device or self.params[0].device
        self.offsets = []
        total = 0
        for p in self.params:
            if p.dtype != torch.float16:
                raise TypeError("the workspace holds fp16 parameters only")
            self.offsets.append(total)
            total += (p.numel() + ALIGN - 1) // ALIGN * ALIGN
        self.numel = total
        self.param = torch.zeros(total, dtype=torch.float16, device=device)
        self.grad = torch.zeros(total, dtype=torch.float16, device=device)
        self.exp_avg = torch.zeros(total, dtype=torch.float32, device=device)
        self.exp_avg_sq = torch.zeros(total, dtype=torch.float32, device=device)
        self.step_count = 0
        with torch.no_grad():
            for p, off in zip(self.params, self.offsets):
                n = p.numel()
                self.param[off:off + n].copy_(p.detach().reshape(-1))
                if p.grad is not None:
                    self.grad[off:off + n].copy_(p.grad.detach().reshape(-1))
                # Re-point the parameter and its gradient at their slices.
                p.data = self.param[off:off + n].view(p.shape)
                p.grad = self.grad[off:off + n].view(p.shape)

    def zero_grad(self):
        self.grad.zero_()

    def step(self, lr, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0, grad_scale=1.0,
             decoupled_wd=True):
        """One Adam step over the whole workspace: exactly one kernel launch."""
        self.step_count += 1
        ops.adam_workspace_step(self.param, self.grad, self.exp_avg, self.exp_avg_sq, lr,
                                betas[0], betas[1], eps, weight_decay, self.step_count,
                                grad_scale, decoupled_wd)

    def state_dict(self):
        """Everything a resume needs: parameters, moments and the step count."""
        return {"param": self.param.detach().clone(), "exp_avg": self.exp_avg.detach().clone(),
                "exp_avg_sq": self.exp_avg_sq.detach().clone(), "step": self.step_count}

    def load_state_dict(self, state):
        with torch.no_grad():
            self.param.copy_(state["param"])
            self.exp_avg.copy_(state["exp_avg"])
            self.exp_avg_sq.copy_(state["exp_avg_sq"])
        self.step_count = int(state["step"])


def link(params, device=None):
    """Link ``params`` into one workspace and return it."""
    return Workspace(params, device)
