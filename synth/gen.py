"""Seeded random tensors (no method arithmetic; see the package docstring)."""
import torch

FP8_MAX = 448.0


def gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal(shape, seed, device="cpu", std=1.0):
    x = torch.randn(*shape, generator=gen(seed, device), device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def bf16_normal(shape, seed, device="cpu"):
    return normal(shape, seed, device).to(torch.bfloat16)


def fp8_per_token(x: torch.Tensor):
    """x [n, ...] float32 -> (codes uint8 [n, ...], scale float32 [n]).

    One scale per token (leading dim) = amax / 448 (1 for an all-zero token);
    codes are torch's float8_e4m3fn cast of x / scale, viewed as bytes."""
    n = x.shape[0]
    amax = x.reshape(n, -1).abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    y = x / scale.reshape((n,) + (1,) * (x.dim() - 1))
    y = y.clamp_(-FP8_MAX, FP8_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.to(torch.float32)


def randperm(n, seed, device="cpu"):
    return torch.randperm(n, generator=gen(seed, device), device=device)


# exact-arithmetic regime E1 ---------------------------------------------
# E4M3 codes of the integers 0..4 (OCP E4M3: 1 = 0x38, 2 = 0x40, 3 = 0x44, 4 = 0x48)
_E1_CODES = torch.tensor([0x00, 0x38, 0x40, 0x44, 0x48], dtype=torch.uint8)


def e1_codes(shape, seed):
    """Codes of integers drawn uniformly from {-4..4}."""
    g = gen(seed)
    mag = torch.randint(0, 5, shape, generator=g)
    neg = torch.randint(0, 2, shape, generator=g).bool() & (mag > 0)
    codes = _E1_CODES[mag]
    codes = torch.where(neg, codes | 0x80, codes)
    return codes.to(torch.uint8)


def e1_pow2_scales(n, seed, lo=-3, hi=3):
    g = gen(seed)
    e = torch.randint(lo, hi + 1, (n,), generator=g).to(torch.float32)
    return torch.pow(2.0, e)


def e1_weights(shape, seed):
    """Multiples of 1/16 in [-1, 1]."""
    g = gen(seed)
    return torch.randint(-16, 17, shape, generator=g).to(torch.float32) / 16.0


# byte views --------------------------------------------------------------
def bf16_bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bits (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")


def fp8_bits(t: torch.Tensor):
    return t.detach().contiguous().cpu().numpy().view("uint8")
