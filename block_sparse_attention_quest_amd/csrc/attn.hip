// attn.hip - speculative block-sparse decode attention and incremental repair kernels (gfx950).
// The device code, its design notes and citations are in attn_core.hpp.

#include "attn_core.hpp"

#include <mutex>

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

// The buffer of prr_spec_attn_noalloc: the speculative pass's workspace (arrival counters, partial
// states) for callers that cannot allocate.  Each GPU the library runs on holds its own copy until the
// process ends; host code reaches it only through the per-device address below, never by this name.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device of `stream` (the current device for the null stream),
// looked up once per device with that device current.
hipError_t scratch_address(hipStream_t stream, void **out) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    int dev = cur;
    if (stream) {
        hipDevice_t d = 0;
        e = hipStreamGetDevice(stream, &d);
        if (e != hipSuccess) return e;
        dev = d;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *ptr = nullptr;
        e = hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

size_t attn_workspace_bytes(int batch, int hq, int hkv, int d, int block, int cap) {
    const int units = batch * hkv;
    const int G = hkv > 0 ? hq / hkv : 0;
    return counters_bytes(units) + max_chunks(units, block, cap) * G * (d + 2) * sizeof(float);
}

hipError_t launch_attn(const KvDesc &kv, const void *q, int hq, int block, const int32_t *idx,
                       const int32_t *count, const int32_t *pages, int cap, float scale, float *acc, float *l,
                       float *m, float *out, bool repair, void *ws, hipStream_t stream) {
    AttnParams p{};
    const int grid = attn_setup(p, kv, q, hq, block, idx, count, pages, cap, scale, acc, l, m, out, repair, ws);
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

hipError_t launch_spec_noalloc(const KvDesc &kv, const void *q, int hq, int block, const int32_t *idx,
                               const int32_t *count, const int32_t *pages, int cap, float scale, float *acc,
                               float *l, float *m, hipStream_t stream) {
    void *ws = nullptr;
    hipError_t e = scratch_address(stream, &ws);
    if (e != hipSuccess) return e;
    // the arrival counters must start at zero (a fill kernel: no memset node); the partial states are
    // written before they are read
    e = launch_clear(ws, counters_bytes(kv.batch * kv.hkv), stream);
    if (e != hipSuccess) return e;
    return launch_attn(kv, q, hq, block, idx, count, pages, cap, scale, acc, l, m, nullptr, false, ws, stream);
}

hipError_t launch_clear(void *ws, size_t bytes, hipStream_t stream) {
    const size_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    const int blocks = (int)std::min<size_t>(1024, (n + 255) / 256);
    return launch(clear_kernel, dim3(blocks), dim3(256), stream, (uint32_t *)ws, n);
}

}  // namespace prr
