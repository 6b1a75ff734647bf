// append.hip - one decode step's new token into the paged cache and its block's metadata (gfx950).
//
// Citations:
//   [paper] "Predict, Reuse, and Repair: Accelerating Dynamic Sparse Attention for Long-Context LLM
//           Decoding" (full paper text)
//
// Decoding appends one token per sequence and step.  Its key and value go to the page that holds
// position t = seq_len[b] (slot t mod 16); the block metadata of the block that holds t (the channel-wise
// min and max keys of [paper] A.1) absorbs the new key: a block's first token sets both rows, later ones
// take the running min / max, in token order, exactly as a rebuild over the block's valid tokens does.
// Blocks born this way take part in selection at once; the predictor starts their state at the next
// call ([paper] §4.1, state initialisation).  seq_len[b] then advances by one.
//
// Mean-pooled metadata (the fp32 channel-wise block means) is recomputed for the block after the token
// is written: float64 sum over the block's valid tokens in token order, divided by their count, rounded
// once to float32, as a rebuild does.
//
// One workgroup per sequence: its threads cover (kv head, channel); the length is read before and
// written after a workgroup barrier.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kv_types.hpp"
#include "prr_internal.hpp"

namespace prr {
namespace {

struct AppendParams {
    void *k;
    void *v;
    const int32_t *page_table;
    int32_t *seq_len;
    const void *k_new;
    const void *v_new;
    void *meta;
    int hkv, max_pages, num_pages, block, stride;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Element i of a cache-typed array, exactly as a float.
template <int KT>
__device__ __forceinline__ float elem_f32(const void *a, size_t i) {
    if constexpr (KT == kKtF32) return ((const float *)a)[i];
    else if constexpr (KT == kKtBf16) return bf16_bits_to_f32(((const uint16_t *)a)[i]);
    else return fp8_to_f32(((const uint8_t *)a)[i]);
}

// dst[di] = src[si] for cache-typed arrays (a plain copy of the element's bytes).
template <int KT>
__device__ __forceinline__ void copy_elem(void *dst, size_t di, const void *src, size_t si) {
    if constexpr (KT == kKtF32) ((float *)dst)[di] = ((const float *)src)[si];
    else if constexpr (KT == kKtBf16) ((uint16_t *)dst)[di] = ((const uint16_t *)src)[si];
    else ((uint8_t *)dst)[di] = ((const uint8_t *)src)[si];
}

__device__ __forceinline__ double dadd_exact(double a, double b) {
#pragma clang fp contract(off)
    return a + b;
}

template <int KT, int D, bool MEAN>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
    __shared__ int s_t;
    const int b = blockIdx.x;
    if (threadIdx.x == 0) s_t = p.seq_len[b];
    __syncthreads();
    const int t = s_t;
    // a full cache (or a negative length) is the caller's contract; nothing is written then
    if (t < 0 || t >= p.max_pages * kPage) return;
    // the page-table entry only decides where the token goes: the metadata and token loads below do not
    // wait for it (stores are skipped for an out-of-range entry)
    const int ph = p.page_table[(size_t)b * p.max_pages + t / kPage];
    const int slot = t % kPage;
    const int blk = t / p.block;
    const bool first = (t % p.block) == 0;
    const bool ok = ph >= 0 && ph < p.num_pages;
#pragma unroll 4
    for (int idx = threadIdx.x; idx < p.hkv * D; idx += blockDim.x) {
        const int h = idx / D, i = idx - h * D;
        const size_t src = ((size_t)b * p.hkv + h) * D + i;
        const size_t kdst = (((size_t)ph * p.hkv + h) * kPage + slot) * D + i;      // [page][Hkv][16][d]
        const size_t vdst = (((size_t)ph * p.hkv + h) * D + i) * kPage + slot;      // [page][Hkv][d][16]
        const size_t row = (((size_t)b * p.hkv + h) * D + i) * 2 * p.stride;        // [B][Hkv][d][2][stride]
        if constexpr (MEAN) {
            if (ok) {
                copy_elem<KT>(p.k, kdst, p.k_new, src);
                copy_elem<KT>(p.v, vdst, p.v_new, src);
            }
        } else if constexpr (KT != kKtF32) {
            // bf16 metadata (an fp8 key is a bf16 value, so min and max stay exact)
            const float x = elem_f32<KT>(p.k_new, src);
            uint16_t *m16 = (uint16_t *)p.meta;
            const uint16_t mn0 = m16[row + blk], mx0 = m16[row + p.stride + blk];
            const float mn = first ? x : fminf(bf16_bits_to_f32(mn0), x);
            const float mx = first ? x : fmaxf(bf16_bits_to_f32(mx0), x);
            if (ok) {
                copy_elem<KT>(p.k, kdst, p.k_new, src);
                copy_elem<KT>(p.v, vdst, p.v_new, src);
                m16[row + blk] = (uint16_t)(__float_as_uint(mn) >> 16);
                m16[row + p.stride + blk] = (uint16_t)(__float_as_uint(mx) >> 16);
            }
        } else {
            const float x = ((const float *)p.k_new)[src];
            const float vx = ((const float *)p.v_new)[src];
            float *m32 = (float *)p.meta;
            const float mn0 = m32[row + blk], mx0 = m32[row + p.stride + blk];
            if (ok) {
                ((float *)p.k)[kdst] = x;
                ((float *)p.v)[vdst] = vx;
                m32[row + blk] = first ? x : fminf(mn0, x);
                m32[row + p.stride + blk] = first ? x : fmaxf(mx0, x);
            }
        }
    }
    if constexpr (MEAN) {
        __syncthreads();   // the new key is in the cache for every thread of the workgroup
        if (ok) {
            const int t0 = blk * p.block;
            for (int idx = threadIdx.x; idx < p.hkv * D; idx += blockDim.x) {
                const int h = idx / D, i = idx - h * D;
                double acc = 0.0;
                for (int tt = t0; tt <= t; ++tt) {
                    int pg = p.page_table[(size_t)b * p.max_pages + tt / kPage];
                    pg = min(max(pg, 0), p.num_pages - 1);
                    const size_t off = (((size_t)pg * p.hkv + h) * kPage + (tt % kPage)) * D + i;
                    acc = dadd_exact(acc, (double)elem_f32<KT>(p.k, off));
                }
                ((float *)p.meta)[(((size_t)b * p.hkv + h) * D + i) * p.stride + blk] = (float)(acc / (double)(t - t0 + 1));
            }
        }
    }
    __syncthreads();
    if (threadIdx.x == 0 && ok) p.seq_len[b] = t + 1;
}

}  // namespace

hipError_t launch_append(const KvDesc &kv, void *k, void *v, int32_t *seq_len, const void *k_new,
                         const void *v_new, int block, int stride, void *meta, bool mean, hipStream_t stream) {
    AppendParams p;
    p.k = k;
    p.v = v;
    p.page_table = kv.page_table;
    p.seq_len = seq_len;
    p.k_new = k_new;
    p.v_new = v_new;
    p.meta = meta;
    p.hkv = kv.hkv;
    p.max_pages = kv.max_pages;
    p.num_pages = kv.num_pages;
    p.block = block;
    p.stride = stride;
    const int kt = kv.fp8 ? kKtFp8 : kv.bf16 ? kKtBf16 : kKtF32;
#define PRR_AP(KT, DD, MN) \
    if (kt == KT && kv.d == DD && mean == MN) PRR_LAUNCH(append_kernel<KT, DD, MN>, dim3(kv.batch), dim3(256), stream, p); else
#define PRR_AP_T(KT) PRR_AP(KT, 128, false) PRR_AP(KT, 64, false) PRR_AP(KT, 128, true) PRR_AP(KT, 64, true)
    PRR_AP_T(kKtF32) PRR_AP_T(kKtBf16) PRR_AP_T(kKtFp8)
    { return hipErrorInvalidValue; }
#undef PRR_AP_T
#undef PRR_AP
    return hipGetLastError();
}

}  // namespace prr
