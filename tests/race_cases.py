"""Fused calls whose outputs the race-guard build (libgemm_epi_debug.so, compiled
with -DGE_DEBUG_SYNC: a full wait and workgroup barrier at every pipeline stage
of the tile kernels, device-scope fences around the cross-workgroup handoffs,
and a device synchronisation after every call) must reproduce bit for bit.
Used in-process with the normal library and in a child process with the debug
library; the inputs are seeded, so both see the same bytes."""
import workloads


def run_cases(ge, torch):
    from gpu_helpers import to_dev
    dev = "cuda"

    def gemm(name, M, N, K, seed, **kw):
        w = workloads.WORKLOADS["square_bf16"].with_shape(M=M, N=N, K=K)
        inp = workloads.make_inputs(w, seed=seed)
        B = to_dev(inp["B"])
        if kw.pop("prepack", False):
            B = ge.b_prepack(B)
            kw["prepacked"] = True
        return ge.gemm_epilogue(to_dev(inp["A"]), B, bias=to_dev(inp["bias"]), R=to_dev(inp["R"]),
                                act="gelu_tanh", **kw)

    def w4(M, N, K, seed, prepacked=True):
        w = workloads.WORKLOADS["w4a16_m16"].with_shape(M=M, N=N, K=K)
        inp = workloads.make_inputs(w, seed=seed)
        Wq = torch.from_numpy(inp["Wq"]).to(dev)
        return ge.w4_gemm(to_dev(inp["X"]), ge.w4_prepack(Wq) if prepacked else Wq, to_dev(inp["scales"]),
                          bias=to_dev(inp["bias"]), prepacked=prepacked)

    def w8(fmt, M, N, K, seed):
        base = workloads.WORKLOADS[f"w8a16_{fmt}_m16"]
        w = base.with_shape(M=M, N=N, K=K)
        inp = workloads.make_inputs(w, seed=seed)
        return ge.w4_gemm(to_dev(inp["X"]), torch.from_numpy(inp["Wq"]).to(dev), to_dev(inp["scales"]),
                          bias=to_dev(inp["bias"]), zero_point=inp["zero_point"], fmt=fmt)

    def swiglu(M, N, K, seed, prepacked=False):
        w = workloads.WORKLOADS["swiglu_8b"].with_shape(M=M, N=N, K=K)
        inp = workloads.make_inputs(w, seed=seed)
        Wg, Wu = to_dev(inp["Wg"]), to_dev(inp["Wu"])
        if prepacked:
            Wg, Wu = ge.swiglu_prepack(Wg, Wu)
        return ge.swiglu(to_dev(inp["X"]), Wg, Wu, prepacked=prepacked)

    out = {
        "tile_128": gemm("tile_128", 512, 768, 1024, 1),
        "tile_256": gemm("tile_256", 2048, 2048, 1024, 2),
        "swiglu": swiglu(512, 1024, 512, 3),
        "decode_streamk": gemm("decode_streamk", 16, 4096, 8192, 4),
        "decode_prepacked": gemm("decode_prepacked", 16, 4096, 2048, 5, prepack=True),
        "w4_decode_split": w4(16, 8192, 2048, 6),
        "w4_tile": w4(96, 1024, 1024, 7),  # split over K (4 slices)
        "w4_tile_8wave": w4(100, 32768, 256, 11),  # enough 64 x 256 tiles for every CU: no split
        "w8_u8_split": w8("u8", 16, 4096, 4096, 8),
        "w8_u8_tile": w8("u8", 128, 1024, 1024, 9),
        "w8_fp8_tile": w8("fp8", 128, 1024, 1024, 10),
        "swiglu_prepacked_pairs": swiglu(16, 14336, 512, 12, prepacked=True),  # gate / up block pairs
        "swiglu_raw_pairs": swiglu(16, 14336, 512, 13),
    }
    torch.cuda.synchronize()
    return {k: v.view(torch.int16).cpu().numpy() for k, v in out.items()}
