"""Sequential quantization of one decoder block's linear layers (test harness).

The sub-layers are quantized in order, each from the Hessian of its own input; once a
sub-layer is quantized, its dequantized weights carry the calibration tokens to the
next input with a plain product (fp32 accumulation, rounded to bf16).  Reading of the
GPTQ tutorial page's remark that the calibration data are fed through the
already-quantized part of the block before the next part is quantized, reduced to
products only (no attention mixing, norms, residuals or activations):
  q/k/v in   = the calibration tokens X0 (one shared Hessian);
  o_proj in  = v_proj's output with its 8 heads of 128 channels each repeated 4 times
               (the 32 query heads' view of the 8 key/value heads);
  gate/up in = o_proj's output (one shared Hessian);
  down in    = up_proj's output.
The propagation is harness work on the GPU with PyTorch; every quantization step
runs through the library.  Each input's first tokens are kept on the host so that
the oracle can rebuild that sub-layer's problem.
"""
import qz_synth


def dequant(codes, scales, zeros, group):
    """W = s (c - z) per (row, group), fp32 on the device."""
    s = scales.repeat_interleave(group, dim=1)
    z = zeros.float().repeat_interleave(group, dim=1)
    return s * (codes.float() - z)


def propagate(X, Wq, chunk=16384):
    """bf16(X @ Wq^T) with fp32 accumulation, over token chunks."""
    import torch
    Y = torch.empty((X.shape[0], Wq.shape[0]), dtype=torch.bfloat16, device=X.device)
    WqT = Wq.t().contiguous()
    for a in range(0, X.shape[0], chunk):
        Y[a:a + chunk] = (X[a:a + chunk].float() @ WqT).to(torch.bfloat16)
    return Y


def repeat_kv(Xv, kv_heads, head_dim, rep):
    """[n, kv_heads * head_dim] -> [n, kv_heads * rep * head_dim]: each head repeated
    `rep` times in place."""
    n = Xv.shape[0]
    return (Xv.view(n, kv_heads, 1, head_dim).expand(n, kv_heads, rep, head_dim)
            .reshape(n, kv_heads * rep * head_dim).contiguous())


def sublayer_names():
    return [s[0] for s in qz_synth.BLOCK_8B["sublayers"]]


def run_block(q, bits, method, n_keep, n_tokens=None):
    """Quantize the block with `method` ("gptq" or "admm") at `bits` bits, propagating
    that method's result.  Returns {sub-layer: dict(d_i, d_o, input, X_head, W, codes)}
    with X_head the first n_keep tokens of the sub-layer's input (host, bf16 bits), W
    its weights (host, bf16 bits) and the codes the method produced (host)."""
    import torch
    from gpu_util import to_host
    B = qz_synth.BLOCK_8B
    n = B["n"] if n_tokens is None else n_tokens
    group = B["group"]
    inputs = {"x0": qz_synth.calib_bf16_torch(B["calib_seed"], n, B["d_model"], B["p_out"],
                                              B["f_out"])}
    hess = {}
    result = {}
    for idx, (name, src, d_i, d_o, seed) in enumerate(B["sublayers"]):
        X = inputs[src]
        assert X.shape == (n, d_i), (name, X.shape)
        if src not in hess:
            hess[src] = q.qz_build_hessian(X, damp=B["damp"])["H"]
        H = hess[src]
        W = qz_synth.weights_bf16_torch(seed, d_o, d_i)
        if method == "gptq":
            codes, scales, zeros = q.qz_gptq(H, W, bits, group, B["B"])
        else:
            V, lam, sig = q.qz_admmq_prepare(H)
            o = q.qz_admmq(V, lam, sig, W, bits, group, B["iters"], B["rho0"], B["gamma"],
                           B["refresh"], want_U=False)
            codes, scales, zeros = o["codes"], o["scales"], o["zeros"]
            del V, lam, sig, o
        result[name] = dict(d_i=d_i, d_o=d_o, input=src, X_head=to_host(X[:n_keep]),
                            W=to_host(W), codes=to_host(codes))
        if name in ("v_proj", "o_proj", "up_proj"):
            Y = propagate(X, dequant(codes, scales, zeros, group))
            if name == "v_proj":
                rep = B["q_heads"] // B["kv_heads"]
                inputs["x_attn"] = repeat_kv(Y, B["kv_heads"], B["head_dim"], rep)
            elif name == "o_proj":
                inputs["x_mlp"] = Y
            else:
                inputs["x_down"] = Y
            del Y
        del X, H, W, codes, scales, zeros
        # inputs and Hessians that no later sub-layer reads are released
        later = {s[1] for s in B["sublayers"][idx + 1:]}
        for k in [k for k in inputs if k not in later]:
            del inputs[k]
            hess.pop(k, None)
        torch.cuda.empty_cache()
    return result
