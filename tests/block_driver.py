"""Sequential quantization of one decoder block's linear layers (test harness).

The sub-layers are quantized in order, each from the Hessian of its own input; once a
sub-layer is quantized, its dequantized weights carry the calibration tokens through
the block to the next input (GPTQ tutorial page, section 3, the remark after
Algorithm 1: the calibration data pass through the already-quantized part of the block
before the next part is quantized).  The block is a pre-norm, Llama-style decoder
layer, evaluated in fp32 with the sub-layer inputs rounded to bf16:
  x          the block's input hidden states (the synthetic calibration tokens)
  q/k/v in   = RMSNorm(x)                                           (one shared Hessian)
  o_proj in  = causal softmax attention of each 2048-token sequence, 32 query heads of
               128 channels over 8 key/value heads (each shared by 4 query heads),
               scores scaled by 1/sqrt(128), with the quantized q/k/v
  h          = x + o_proj(attention)                                (residual add)
  gate/up in = RMSNorm(h)                                           (one shared Hessian)
  down in    = silu(gate(.)) * up(.)                                (SwiGLU)
RMSNorm gains are 1 (the usual initialisation), eps 1e-6; no rotary embedding (the pages
give none, and it does not change which channels the products mix).  The propagation
is harness work on the GPU with PyTorch in fp32 (attention scores through explicit
products of contiguous operands); every quantization step runs through the library.
Each input's first tokens are kept on the host so that the oracle can rebuild that
sub-layer's problem.
"""
import qz_synth


def dequant(codes, scales, zeros, group):
    """W = s (c - z) per (row, group), fp32 on the device."""
    s = scales.repeat_interleave(group, dim=1)
    z = zeros.float().repeat_interleave(group, dim=1)
    return s * (codes.float() - z)


def rmsnorm(x, eps=1e-6):
    """x / sqrt(mean(x^2) + eps) per token (gain 1), fp32."""
    import torch
    return x * torch.rsqrt((x * x).mean(dim=-1, keepdim=True) + eps)


def causal_attention(xs, Wq, Wk, Wv, q_heads, kv_heads, head_dim):
    """Causal softmax attention of one sequence xs [S x d] (fp32) with projection weights
    Wq [q_heads*hd x d], Wk/Wv [kv_heads*hd x d]; returns [S x q_heads*hd] fp32."""
    import torch
    S = xs.shape[0]
    rep = q_heads // kv_heads
    Q = (xs @ Wq.t()).view(S, q_heads, head_dim).transpose(0, 1).contiguous()
    K = (xs @ Wk.t()).view(S, kv_heads, head_dim).transpose(0, 1).repeat_interleave(rep, dim=0)
    V = (xs @ Wv.t()).view(S, kv_heads, head_dim).transpose(0, 1).repeat_interleave(rep, dim=0)
    Kt = K.transpose(1, 2).contiguous()
    scores = torch.matmul(Q, Kt) * (head_dim ** -0.5)
    mask = torch.ones((S, S), dtype=torch.bool, device=xs.device).triu(1)
    scores.masked_fill_(mask, float("-inf"))
    P = torch.softmax(scores, dim=-1)
    O = torch.matmul(P, V.contiguous())                    # [heads, S, hd]
    return O.transpose(0, 1).reshape(S, q_heads * head_dim)


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
    seq = B["seq_len"]
    assert n % seq == 0
    group, chunk = B["group"], 16384
    x = qz_synth.calib_bf16_torch(B["calib_seed"], n, B["d_model"], B["p_out"], B["f_out"])
    inputs = {"x_qkv": torch.empty_like(x)}
    for a in range(0, n, chunk):
        inputs["x_qkv"][a:a + chunk] = rmsnorm(x[a:a + chunk].float()).to(torch.bfloat16)
    hess, wq, result = {}, {}, {}
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
        wq[name] = dequant(codes, scales, zeros, group)
        del X, H, W, codes, scales, zeros
        if name == "v_proj":      # q, k, v quantized: the attention output feeds o_proj
            xq = inputs["x_qkv"]
            att = torch.empty((n, B["q_heads"] * B["head_dim"]), dtype=torch.bfloat16, device=xq.device)
            for a in range(0, n, seq):
                att[a:a + seq] = causal_attention(xq[a:a + seq].float(), wq["q_proj"], wq["k_proj"],
                                                  wq["v_proj"], B["q_heads"], B["kv_heads"],
                                                  B["head_dim"]).to(torch.bfloat16)
            inputs["x_attn"] = att
        elif name == "o_proj":    # residual add, then the MLP's norm
            xm = torch.empty_like(x)
            WoT = wq["o_proj"].t().contiguous()
            for a in range(0, n, chunk):
                h = x[a:a + chunk].float() + inputs["x_attn"][a:a + chunk].float() @ WoT
                xm[a:a + chunk] = rmsnorm(h).to(torch.bfloat16)
            inputs["x_mlp"] = xm
            del WoT
        elif name == "up_proj":   # SwiGLU: silu(gate) * up feeds down_proj
            xm = inputs["x_mlp"]
            xd = torch.empty((n, B["d_ff"]), dtype=torch.bfloat16, device=xm.device)
            WgT = wq["gate_proj"].t().contiguous()
            WuT = wq["up_proj"].t().contiguous()
            for a in range(0, n, chunk):
                xs = xm[a:a + chunk].float()
                xd[a:a + chunk] = (torch.nn.functional.silu(xs @ WgT) * (xs @ WuT)).to(torch.bfloat16)
            inputs["x_down"] = xd
            del WgT, WuT
        # inputs, Hessians and weights that no later step reads are released
        later = {s[1] for s in B["sublayers"][idx + 1:]}
        for k in [k for k in inputs if k not in later]:
            del inputs[k]
            hess.pop(k, None)
        for k in [k for k in wq if k in ("o_proj", "down_proj") or
                  (k in ("q_proj", "k_proj", "v_proj") and "x_attn" in inputs) or
                  (k in ("gate_proj", "up_proj") and "x_down" in inputs)]:
            del wq[k]
        torch.cuda.empty_cache()
    del x
    return result
