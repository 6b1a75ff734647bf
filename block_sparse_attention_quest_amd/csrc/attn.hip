// attn.hip - speculative block-sparse decode attention and incremental repair (gfx950).
//
// Citations:
//   [paper] "Predict, Reuse, and Repair: Accelerating Dynamic Sparse Attention for Long-Context LLM
//           Decoding" (full paper text)
//   [blog]  "PRR: Predict, Reuse, and Repair - Accelerating Dynamic Sparse Attention for Long-Context
//           LLM Decoding" (xllm-io paper review)
//
// What is computed.  For every (sequence b, kv head) unit and each of its G query heads: the attention
// state (acc, l, m) of the query over the tokens of the unit's block set ([paper] §4.3: the speculative
// pass stores the softmax denominator and running maximum next to the output).  In repair mode the new
// tokens' state is folded into the existing state with the online-softmax recurrence ([paper] §4.3,
// [blog] Eq. (6)); work and traffic scale with the number of missed blocks only.
//
// How it maps to CDNA4.
//   * Work list: a unit's set expands to count * (block / 16) pages.  Each wave takes PPW consecutive
//     pages, a workgroup takes 4 waves, and the grid is sized from the set capacity (counts live on
//     the device); waves past the end mask everything.
//   * Loads go straight from HBM into MFMA operand registers with 16-byte loads: K page tiles are
//     token-major ([16][d]) so a lane reads 8 channels of one token; V page tiles are channel-major
//     ([d][16]) so a lane reads 8 tokens of one channel.  No LDS staging of K/V is needed.
//   * bf16: S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16.  Query heads are MFMA columns
//     (G of 16 used), so one K/V tile read serves the whole GQA group.  The QK output rows are assigned
//     to tokens so that each lane ends up holding exactly the 8 consecutive tokens that the PV
//     B-operand needs: no shuffle between the two products.  P enters PV as a bf16 hi + lo pair
//     (two MFMAs), which keeps the product at ~2^-17 relative error while V stays exact.
//   * fp32: the same structure on v_mfma_f32_16x16x4_f32.
//   * Softmax: a wave computes all its scores first, takes one max (two cross-lane steps), then PV
//     with a fixed max - no rescaling inside a wave.  Waves merge in LDS, workgroups merge through a
//     small workspace: the last workgroup of a unit to finish (device-scope counter) folds the
//     partials in fixed order, so results are deterministic run to run.
//   * Exponentials use the hardware base-2 exponential on log2(e)-prescaled scores; m is stored in
//     natural-log units.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "prr_internal.hpp"

namespace prr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

constexpr int pages_per_wave(bool bf16, int d) { return bf16 ? 4 : (d == 128 ? 2 : 4); }

struct AttnParams {
    const void *q;
    const void *k;
    const void *v;
    const int32_t *page_table;
    const int32_t *seq_len;
    const int32_t *idx;
    const int32_t *count;
    float *acc;
    float *l;
    float *m;
    float *out;
    uint32_t *counters;
    float *partials;
    int hq, hkv, G, cap, ppb, max_pages, num_pages, wg_per_unit;
    float c2;  // softmax scale * log2(e)
    int repair;
};

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Device-scope (all XCDs) coherent store and load of one float.
__device__ __forceinline__ void st_dev(float *ptr, float v) {
    __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *ptr) {
    return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Lane-dependent choice between two wave-uniform values, kept as a register select (never an
// indexed private-array access).
__device__ __forceinline__ int pick(int second, int a, int b) {
    int r;
    asm volatile("" : "=v"(r) : "0"(second ? b : a));
    return r;
}

__device__ __forceinline__ float rescale(float mpart, float mtot) {
    return mpart == -INFINITY ? 0.0f : fexp2(mpart - mtot);
}

// Physical pages and valid-token counts of entries page0 .. page0+N-1 of the unit's expanded page
// list.  Branch-free with clamped indices so the N set lookups, then the N page-table lookups, issue
// back to back (two dependent memory rounds instead of 2N).  Out-of-range entries get vt = 0.
template <int N>
__device__ __forceinline__ void page_info(const AttnParams &p, int b, int u, int page0, int total_pages,
                                          int slen, int (&phys)[N], int (&vt)[N]) {
    int sub[N], blk[N];
    bool inr[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const int gp = page0 + i;
        inr[i] = gp < total_pages;
        const int gpc = inr[i] ? gp : 0;
        const int li = gpc / p.ppb;
        sub[i] = gpc - li * p.ppb;
        blk[i] = p.idx[(size_t)u * p.cap + li];
    }
    long lpc[N];
    bool ok[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const long lp = (long)blk[i] * p.ppb + sub[i];
        ok[i] = inr[i] && blk[i] >= 0 && lp < p.max_pages;
        lpc[i] = ok[i] ? lp : 0;
    }
    int ph[N];
#pragma unroll
    for (int i = 0; i < N; ++i) ph[i] = p.page_table[(size_t)b * p.max_pages + lpc[i]];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        vt[i] = ok[i] ? (int)min(max((long)slen - lpc[i] * kPage, 0L), (long)kPage) : 0;
        phys[i] = min(max(ph[i], 0), p.num_pages - 1);
    }
}

// Final write of one (query j, channel c) item: state in natural-log units, optional normalised out.
__device__ __forceinline__ void write_item(const AttnParams &p, size_t head, int c, int D, float a,
                                           float lsum, float m2, bool keep_m, float m_old) {
    p.acc[head * D + c] = a;
    if (c == 0) {
        p.l[head] = lsum;
        p.m[head] = keep_m ? m_old : (m2 == -INFINITY ? -INFINITY : m2 * kLn2);
    }
    if (p.out) p.out[head * D + c] = lsum > 0.0f ? a / lsum : 0.0f;
}

// The last workgroup of a unit folds the unit's nwg partial states (and, in repair mode, the incoming
// state) into the final one.  A thread owns VW consecutive channels of one query head.  Partials are
// visited in index order, MB at a time: every device-scope load of a batch is issued before any is
// used, so a batch costs one memory round trip; batches combine with the same online-softmax step
// (running maximum, rescaled sums), which keeps the result independent of arrival order.
template <int VW, int D>
__device__ __forceinline__ void merge_partials(const AttnParams &p, const float *base, int nwg, size_t head0,
                                               const float *s_mo, const float *s_lo) {
    constexpr int MB = 16;
    constexpr int CPH = D / VW;   // channel groups per head
    const int G = p.G;
    for (int it = threadIdx.x; it < G * CPH; it += kThreads) {
        const int jj = it / CPH, c0 = (it - jj * CPH) * VW;
        const size_t head = head0 + jj;
        float mt = -INFINITY, ls = 0.0f, a[VW];
        float mo = 0.0f, mo2 = -INFINITY;
#pragma unroll
        for (int v = 0; v < VW; ++v) a[v] = 0.0f;
        if (p.repair) {
            mo = s_mo[jj];
            mo2 = mo == -INFINITY ? -INFINITY : mo * kLog2e;
            mt = mo2;
            ls = s_lo[jj];
#pragma unroll
            for (int v = 0; v < VW; ++v) a[v] = p.acc[head * D + c0 + v];
        }
        for (int w0 = 0; w0 < nwg; w0 += MB) {
            float pm[MB], pl[MB], pa[MB][VW];
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const int w = min(w0 + i, nwg - 1);   // clamped: a valid partial, weighted 0 below
                const float *pw = base + ((size_t)w * G + jj) * (D + 2);
                pm[i] = ld_dev(&pw[D + 1]);
                pl[i] = ld_dev(&pw[D]);
#pragma unroll
                for (int v = 0; v < VW; ++v) pa[i][v] = ld_dev(&pw[c0 + v]);
            }
            float mb = mt;
#pragma unroll
            for (int i = 0; i < MB; ++i)
                if (w0 + i < nwg) mb = fmaxf(mb, pm[i]);
            const float fr = rescale(mt, mb);
            ls *= fr;
#pragma unroll
            for (int v = 0; v < VW; ++v) a[v] *= fr;
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const float f = w0 + i < nwg ? rescale(pm[i], mb) : 0.0f;
                ls += f * pl[i];
#pragma unroll
                for (int v = 0; v < VW; ++v) a[v] += f * pa[i][v];
            }
            mt = mb;
        }
#pragma unroll
        for (int v = 0; v < VW; ++v) write_item(p, head, c0 + v, D, a[v], ls, mt, p.repair && mt == mo2, mo);
    }
}

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnParams p) {
    constexpr int PPW = pages_per_wave(BF16, D);
    constexpr int DP = D + 4;  // padded LDS row
    __shared__ float sm_acc[kWaves][16 * DP];
    __shared__ float sm_m[kWaves][16];
    __shared__ float sm_l[kWaves][16];
    __shared__ float s_mo[16], s_lo[16];   // repair: the incoming state's m and l per query head
    __shared__ int s_last;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j = lane & 15;   // query column / operand row
    const int g = lane >> 4;   // lane group (k slice)
    const int u = blockIdx.y;
    const int b = u / p.hkv;
    const int kvh = u - b * p.hkv;
    const int G = p.G;
    const int cnt = min(max(p.count[u], 0), p.cap);
    const int total_pages = cnt * p.ppb;
    const int nwg = (total_pages + kWaves * PPW - 1) / (kWaves * PPW);
    const int wg = blockIdx.x;
    const size_t head0 = (size_t)b * p.hq + (size_t)kvh * G;

    if (total_pages == 0) {
        // empty set: speculation writes the empty state; repair leaves the state untouched
        if (wg != 0) return;
        for (int it = threadIdx.x; it < G * D; it += kThreads) {
            const int jj = it / D, c = it - jj * D;
            const size_t head = head0 + jj;
            if (!p.repair) {
                write_item(p, head, c, D, 0.0f, 0.0f, -INFINITY, false, 0.0f);
            } else if (p.out) {
                const float lo = p.l[head];
                p.out[head * D + c] = lo > 0.0f ? p.acc[head * D + c] / lo : 0.0f;
            }
        }
        return;
    }
    if (wg >= nwg) return;

    const int slen = p.seq_len[b];
    // page0 is uniform per wave; readfirstlane keeps the page lookups in scalar registers
    const int page0 = (wg * kWaves + __builtin_amdgcn_readfirstlane(wave)) * PPW;
    int phys[PPW], vt[PPW];
    page_info<PPW>(p, b, u, page0, total_pages, slen, phys, vt);
#pragma unroll
    for (int i = 0; i < PPW; ++i) {
        phys[i] = __builtin_amdgcn_readfirstlane(phys[i]);
        vt[i] = __builtin_amdgcn_readfirstlane(vt[i]);
    }
    bool partial = false;   // any page of this wave with fewer than 16 valid tokens
#pragma unroll
    for (int i = 0; i < PPW; ++i) partial |= vt[i] < kPage;

    const size_t tile_stride = (size_t)p.hkv * kPage * D;   // elements per physical page
    const size_t tile_off = (size_t)kvh * kPage * D;
    const int jq = j < G ? j : 0;

    float sc[PPW * 4];     // scores: lane holds 4 per page (bf16 pairs: 8 per two pages)
    f32x4 o[D / 16];
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m2, lsum = 0.0f;

    if constexpr (BF16) {
        constexpr int T = PPW / 2;     // 32-token tiles
        constexpr int KS = D / 32;     // k-steps of 32 channels
        const __bf16 *qb = (const __bf16 *)p.q + (head0 + jq) * D;
        const __bf16 *kb = (const __bf16 *)p.k + tile_off;
        const __bf16 *vb = (const __bf16 *)p.v + tile_off;
        bf16x8 qop[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qop[s] = *(const bf16x8 *)(qb + 32 * s + 8 * g);
            if (j >= G) qop[s] = bf16x8{};
        }
        // K operands: tile t, half h: row r -> token 8(r>>2) + 4h + (r&3) of the tile
        bf16x8 kop[T][2][KS];
        bf16x8 vop[T][D / 16];
        const int r = j;
#pragma unroll
        for (int t = 0; t < T; ++t) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int tt = 8 * (r >> 2) + 4 * h + (r & 3);
                const int ph = pick(tt >> 4, phys[2 * t], phys[2 * t + 1]);
                const __bf16 *kp = kb + (size_t)ph * tile_stride + (tt & 15) * D + 8 * g;
#pragma unroll
                for (int s = 0; s < KS; ++s) kop[t][h][s] = *(const bf16x8 *)(kp + 32 * s);
            }
            const int pv = pick(g >> 1, phys[2 * t], phys[2 * t + 1]);
            const int off = 8 * (g & 1);
#pragma unroll
            for (int cb = 0; cb < D / 16; ++cb) {
                vop[t][cb] = *(const bf16x8 *)(vb + (size_t)pv * tile_stride +
                                               (size_t)(16 * cb + r) * kPage + off);
            }
        }
        // S^T tiles
        float mloc = -INFINITY;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int vvt = pick(g >> 1, vt[2 * t], vt[2 * t + 1]);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    acc4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[t][h][s], qop[s], acc4, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int off = 8 * (g & 1) + 4 * h + i;
                    const float x = off < vvt ? acc4[i] * p.c2 : -INFINITY;
                    sc[8 * t + 4 * h + i] = x;
                    mloc = fmaxf(mloc, x);
                }
            }
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        m2 = mloc;
        const float msafe = m2 == -INFINITY ? 0.0f : m2;
        if (partial) {
            // tokens past the sequence end: zero V so stale cache contents cannot reach the output
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int nv = pick(g >> 1, vt[2 * t], vt[2 * t + 1]) - 8 * (g & 1);
#pragma unroll
                for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (e >= nv) vop[t][cb][e] = (__bf16)0.0f;
            }
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            bf16x8 phi, plo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pe = fexp2(sc[8 * t + e] - msafe);
                lsum += pe;
                const __bf16 hi = (__bf16)pe;
                phi[e] = hi;
                plo[e] = (__bf16)(pe - (float)hi);
            }
#pragma unroll
            for (int cb = 0; cb < D / 16; ++cb) {
                o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[t][cb], phi, o[cb], 0, 0, 0);
                o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[t][cb], plo, o[cb], 0, 0, 0);
            }
        }
    } else {
        constexpr int KS = D / 16;     // float4 slices of a row
        const float *qf = (const float *)p.q + (head0 + jq) * D;
        const float *kf = (const float *)p.k + tile_off;
        const float *vf = (const float *)p.v + tile_off;
        f32x4 qop[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            qop[s] = *(const f32x4 *)(qf + 16 * s + 4 * g);
            if (j >= G) qop[s] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        f32x4 kop[PPW][KS];
        f32x4 vop[PPW][D / 16];
#pragma unroll
        for (int pg = 0; pg < PPW; ++pg) {
            const float *kp = kf + (size_t)phys[pg] * tile_stride + j * D + 4 * g;
#pragma unroll
            for (int s = 0; s < KS; ++s) kop[pg][s] = *(const f32x4 *)(kp + 16 * s);
#pragma unroll
            for (int cb = 0; cb < D / 16; ++cb)
                vop[pg][cb] = *(const f32x4 *)(vf + (size_t)phys[pg] * tile_stride +
                                               (size_t)(16 * cb + j) * kPage + 4 * g);
        }
        float mloc = -INFINITY;
#pragma unroll
        for (int pg = 0; pg < PPW; ++pg) {
            f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc4 = __builtin_amdgcn_mfma_f32_16x16x4f32(kop[pg][s][e], qop[s][e], acc4, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = (4 * g + i) < vt[pg] ? acc4[i] * p.c2 : -INFINITY;
                sc[4 * pg + i] = x;
                mloc = fmaxf(mloc, x);
            }
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        m2 = mloc;
        const float msafe = m2 == -INFINITY ? 0.0f : m2;
        if (partial) {
#pragma unroll
            for (int pg = 0; pg < PPW; ++pg) {
                const int nv = vt[pg] - 4 * g;
#pragma unroll
                for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (e >= nv) vop[pg][cb][e] = 0.0f;
            }
        }
#pragma unroll
        for (int pg = 0; pg < PPW; ++pg) {
            float pe[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pe[i] = fexp2(sc[4 * pg + i] - msafe);
                lsum += pe[i];
            }
#pragma unroll
            for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(vop[pg][cb][e], pe[e], o[cb], 0, 0, 0);
        }
    }

    // repair reads the incoming m and l once, before any thread overwrites them
    if (p.repair && threadIdx.x < G) {
        s_mo[threadIdx.x] = p.m[head0 + threadIdx.x];
        s_lo[threadIdx.x] = p.l[head0 + threadIdx.x];
    }
    // wave state -> LDS (lane (j, g) holds channels 16 cb + 4 g + i of query j)
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (j < G) {
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb)
            *(f32x4 *)&sm_acc[wave][j * DP + 16 * cb + 4 * g] = o[cb];
        if (g == 0) {
            sm_m[wave][j] = m2;
            sm_l[wave][j] = lsum;
        }
    }
    __syncthreads();

    const bool single = (nwg == 1);
    float *part = p.partials + ((size_t)u * p.wg_per_unit + wg) * (size_t)G * (D + 2);
    for (int it = threadIdx.x; it < G * D; it += kThreads) {
        const int jj = it / D, c = it - jj * D;
        float mx = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm_m[w][jj]);
        float a = 0.0f, ls = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = rescale(sm_m[w][jj], mx);
            a += f * sm_acc[w][jj * DP + c];
            ls += f * sm_l[w][jj];
        }
        if (single) {
            const size_t head = head0 + jj;
            if (p.repair) {
                const float mo = s_mo[jj];
                const float mo2 = mo == -INFINITY ? -INFINITY : mo * kLog2e;
                const float mt = fmaxf(mx, mo2);
                const float fo = rescale(mo2, mt), fn = rescale(mx, mt);
                write_item(p, head, c, D, fo * p.acc[head * D + c] + fn * a, fo * s_lo[jj] + fn * ls,
                           mt, mt == mo2, mo);
            } else {
                write_item(p, head, c, D, a, ls, mx, false, 0.0f);
            }
        } else {
            st_dev(&part[jj * (D + 2) + c], a);
            if (c == 0) {
                st_dev(&part[jj * (D + 2) + D], ls);
                st_dev(&part[jj * (D + 2) + D + 1], mx);
            }
        }
    }
    if (single) return;

    // Cross-workgroup merge: the last workgroup of the unit folds every partial in index order.
    // Partials are written and read with device-scope (sc1) accesses, which are coherent across the
    // XCDs' L2s by themselves; waiting for this thread's stores to complete before the barrier, and the
    // barrier before the counter increment, orders them ahead of it.  This avoids a device-scope
    // release fence, which would write back every dirty line of the L2.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&p.counters[u], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (uint32_t)(nwg - 1));
    }
    __syncthreads();
    if (!s_last) return;

    const float *base = p.partials + (size_t)u * p.wg_per_unit * (size_t)G * (D + 2);
    if (G * D <= 2 * kThreads) merge_partials<2, D>(p, base, nwg, head0, s_mo, s_lo);
    else merge_partials<4, D>(p, base, nwg, head0, s_mo, s_lo);
    if (threadIdx.x == 0) __hip_atomic_store(&p.counters[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void clear_kernel(uint32_t *w, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        w[i] = 0u;
}

}  // namespace

int attn_wg_per_unit(int block, int cap, bool bf16, int d) {
    const int per_wg = kWaves * pages_per_wave(bf16, d);
    const long pages = (long)cap * (block / kPage);
    return (int)std::max<long>(1, (pages + per_wg - 1) / per_wg);
}

static size_t counters_bytes(int units) { return ((size_t)units * 4 + 255) / 256 * 256; }

size_t attn_workspace_bytes(int batch, int hq, int hkv, int d, int block, int cap) {
    const int units = batch * hkv;
    const int G = hkv > 0 ? hq / hkv : 0;
    // the larger of the bf16 and fp32 layouts, so one query serves both dtypes
    const int wgu = std::max(attn_wg_per_unit(block, cap, true, d), attn_wg_per_unit(block, cap, false, d));
    return counters_bytes(units) + (size_t)units * wgu * G * (d + 2) * sizeof(float);
}

hipError_t launch_attn(const KvDesc &kv, const void *q, int hq, int block, const int32_t *idx,
                       const int32_t *count, int cap, float scale, float *acc, float *l, float *m,
                       float *out, bool repair, void *ws, hipStream_t stream) {
    AttnParams p;
    p.q = q;
    p.k = kv.k;
    p.v = kv.v;
    p.page_table = kv.page_table;
    p.seq_len = kv.seq_len;
    p.idx = idx;
    p.count = count;
    p.acc = acc;
    p.l = l;
    p.m = m;
    p.out = out;
    const int units = kv.batch * kv.hkv;
    p.counters = (uint32_t *)ws;
    p.partials = (float *)((char *)ws + counters_bytes(units));
    p.hq = hq;
    p.hkv = kv.hkv;
    p.G = hq / kv.hkv;
    p.cap = cap;
    p.ppb = block / kPage;
    p.max_pages = kv.max_pages;
    p.num_pages = kv.num_pages;
    p.wg_per_unit = attn_wg_per_unit(block, cap, kv.bf16, kv.d);
    p.c2 = scale * kLog2e;
    p.repair = repair ? 1 : 0;
    const dim3 grid(p.wg_per_unit, units);
    const dim3 blk(kThreads);
    if (kv.bf16) {
        if (kv.d == 128) attn_kernel<true, 128><<<grid, blk, 0, stream>>>(p);
        else attn_kernel<true, 64><<<grid, blk, 0, stream>>>(p);
    } else {
        if (kv.d == 128) attn_kernel<false, 128><<<grid, blk, 0, stream>>>(p);
        else attn_kernel<false, 64><<<grid, blk, 0, stream>>>(p);
    }
    return hipGetLastError();
}

hipError_t launch_clear(void *ws, size_t bytes, hipStream_t stream) {
    const size_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    const int blocks = (int)std::min<size_t>(1024, (n + 255) / 256);
    clear_kernel<<<blocks, 256, 0, stream>>>((uint32_t *)ws, n);
    return hipGetLastError();
}

}  // namespace prr
