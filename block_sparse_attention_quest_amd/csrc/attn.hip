// attn.hip - speculative block-sparse decode attention and incremental repair kernels (gfx950).
// The device code, its design notes and citations are in attn_core.hpp.

#include "attn_core.hpp"

namespace prr {
namespace {

// bf16 speculation is held to 256 registers so two waves share each SIMD (in the fused launch the second
// belongs to selection), with two tiles in flight per wave.  Repair runs alone with the same budget: two
// workgroups per CU, so a set at full capacity gets a workgroup per chunk.  The fp32 variants
// (exact-input checks) may use more registers.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_spec_bf16(AttnParams p) {
    attn_body<kKtBf16, D, false, 2>(p, blockIdx.x, gridDim.x);
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_repair_bf16(AttnParams p) {
    attn_body<kKtBf16, D, true, 2>(p, blockIdx.x, gridDim.x);
}

// fp8 tiles take half the registers of bf16 ones: twice as many in flight for the same bytes.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_spec_fp8(AttnParams p) {
    attn_body<kKtFp8, D, false, 2>(p, blockIdx.x, gridDim.x);
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_repair_fp8(AttnParams p) {
    attn_body<kKtFp8, D, true, 2>(p, blockIdx.x, gridDim.x);
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_spec_f32(AttnParams p) {
    attn_body<kKtF32, D, false>(p, blockIdx.x, gridDim.x);
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_repair_f32(AttnParams p) {
    attn_body<kKtF32, D, true>(p, blockIdx.x, gridDim.x);
}

__global__ void clear_kernel(uint32_t *w, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        w[i] = 0u;
}

}  // namespace

size_t attn_workspace_bytes(int batch, int hq, int hkv, int d, int block, int cap) {
    const int units = batch * hkv;
    const int G = hkv > 0 ? hq / hkv : 0;
    return counters_bytes(units) + max_chunks(units, block, cap) * G * (d + 2) * sizeof(float);
}

hipError_t launch_attn(const KvDesc &kv, const void *q, int hq, int block, const int32_t *idx,
                       const int32_t *count, int cap, float scale, float *acc, float *l, float *m,
                       float *out, bool repair, void *ws, hipStream_t stream) {
    AttnParams p;
    const int grid = attn_setup(p, kv, q, hq, block, idx, count, cap, scale, acc, l, m, out, repair, ws);
    void (*k)(AttnParams);
    const bool d128 = kv.d == 128;
    if (kv.fp8) {
        if (repair) k = d128 ? attn_repair_fp8<128> : attn_repair_fp8<64>;
        else k = d128 ? attn_spec_fp8<128> : attn_spec_fp8<64>;
    } else if (kv.bf16) {
        if (repair) k = d128 ? attn_repair_bf16<128> : attn_repair_bf16<64>;
        else k = d128 ? attn_spec_bf16<128> : attn_spec_bf16<64>;
    } else {
        if (repair) k = d128 ? attn_repair_f32<128> : attn_repair_f32<64>;
        else k = d128 ? attn_spec_f32<128> : attn_spec_f32<64>;
    }
    return launch(k, dim3(grid), dim3(kThreads), stream, p);
}

hipError_t launch_clear(void *ws, size_t bytes, hipStream_t stream) {
    const size_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    const int blocks = (int)std::min<size_t>(1024, (n + 255) / 256);
    return launch(clear_kernel, dim3(blocks), dim3(256), stream, (uint32_t *)ws, n);
}

}  // namespace prr
