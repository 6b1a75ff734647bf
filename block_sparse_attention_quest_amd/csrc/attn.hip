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
//   * Work list.  A unit's set expands to count * (block / 16) pages, cut into chunks of cp pages
//     (8..32, a multiple of 8, chosen at launch so that sets at full capacity spread over one
//     workgroup per CU for the speculative pass, which shares the chip with selection, and two per CU
//     for repair, with half the chunk size since repair sets are the missed part of a selection).  Chunk
//     c belongs to unit c mod units, so a unit's chunks are dispatched to the same XCD and every XCD
//     gets the same number of units.  Workgroup i takes chunks i, i + grid, ...; a chunk past its
//     unit's set size is skipped after one load.  The set size, set entries and page-table entries are
//     looked up with addresses that do not depend on each other where possible: two memory rounds
//     before the first K/V load.
//   * Streaming.  Each of the 4 waves of a workgroup owns a quarter of the chunk and walks it in tiles
//     (bf16: 32 tokens = 2 pages; fp32: 16 tokens = 1 page) with two tiles in flight: the next tile's
//     K and V are loaded into registers while the current one is multiplied.  Loads go straight from
//     HBM into MFMA operand registers as 16-byte loads: K page tiles are token-major ([16][d]) so a lane
//     reads 8 channels of one token; V page tiles are channel-major ([d][16]) so a lane reads 8 tokens
//     of one channel.
//   * bf16: S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16.  Query heads are MFMA columns
//     (G of 16 used), so one K/V tile read serves the whole GQA group.  The QK output rows are assigned
//     to tokens so that each lane ends up holding exactly the 8 consecutive tokens that the PV
//     B-operand needs: no shuffle between the two products.  P enters PV as a bf16 hi + lo pair
//     (two MFMAs), which keeps the product at ~2^-17 relative error while V stays exact.
//   * fp32: the same structure on v_mfma_f32_16x16x4_f32.
//   * Softmax: online across tiles (running maximum per query, rescaled sums); waves merge in LDS;
//     chunks of one unit merge through a small workspace: the last chunk of a unit to finish
//     (device-scope counter) folds the partials in chunk order, so results are deterministic.
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
constexpr int kChunkMin = 8;    // pages per chunk: a multiple of 8 (2 pages per wave) ...
constexpr int kChunkMax = 32;   // ... up to 8 pages per wave (bf16: 4 tiles of 2 pages)
constexpr int kChunkMaxF32 = 16;   // fp32 tiles are 1 page: at most 4 per wave
constexpr int kMaxPagesPerWave = kChunkMax / kWaves;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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
    int units, hq, hkv, G, cap, ppb, max_pages, num_pages;
    int cp, kmax;  // pages per chunk, chunks per unit at full capacity
    float c2;  // softmax scale * log2(e)
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

__device__ __forceinline__ int unit_pages(const AttnParams &p, int u) {
    return min(max(p.count[u], 0), p.cap) * p.ppb;
}

// Page lookups of the wave's pages wbeg .. wbeg + N - 1 of the unit's expanded page list.  Lane
// i < N looks up page wbeg + i with vector loads: the set entry, then the page-table entry (two
// dependent memory rounds, through the vector memory path, which keeps many more requests in flight
// than the scalar cache).  The addresses do not depend on the set size, so these loads are issued
// together with the load of the set size; finish() masks entries at or past wend and broadcasts
// physical page and valid-token count to scalar registers.
struct PageLookup {
    int ph;     // physical page (raw)
    int lp;     // logical page (0 when the set entry is out of range)
    bool lp_ok; // set entry in range
};

__device__ __forceinline__ PageLookup page_lookup(const AttnParams &p, int b, int u, int wbeg) {
    const int i = min(threadIdx.x & 63, kMaxPagesPerWave - 1);
    const int gpc = min(wbeg + i, p.cap * p.ppb - 1);
    const int li = gpc / p.ppb;
    const int sub = gpc - li * p.ppb;
    const int blk = p.idx[(size_t)u * p.cap + li];
    const long lp = (long)blk * p.ppb + sub;
    PageLookup r;
    r.lp_ok = blk >= 0 && lp < p.max_pages;
    r.lp = r.lp_ok ? (int)lp : 0;
    r.ph = p.page_table[(size_t)b * p.max_pages + r.lp];
    return r;
}

template <int N>
__device__ __forceinline__ void page_finish(const AttnParams &p, const PageLookup &r, int wbeg, int wend,
                                            int slen, int (&phys)[N], int (&vt)[N]) {
    const int i = threadIdx.x & 63;
    const bool ok = i < N && wbeg + i < wend && r.lp_ok;
    const int my_vt = ok ? min(max(slen - r.lp * kPage, 0), kPage) : 0;
    const int my_ph = min(max(r.ph, 0), p.num_pages - 1);
#pragma unroll
    for (int k = 0; k < N; ++k) {
        vt[k] = __builtin_amdgcn_readlane(my_vt, k);
        phys[k] = __builtin_amdgcn_readlane(my_ph, k);
    }
}

// Per-wave running state: lane (j, g) holds channels 16 cb + 4 g + i of query column j, the running
// maximum of column j (log2 units) and the lane's share of the denominator.
template <int D>
struct WaveState {
    f32x4 o[D / 16];
    float m;
    float l;
};

// ---- bf16 tiles: 32 tokens (2 pages) ----

template <int D>
struct TileB {
    bf16x8 k[2][D / 32];   // half h, k-step s: row r of S^T -> token 8(r>>2) + 4h + (r&3)
    bf16x8 v[D / 16];      // channel block cb: channel 16 cb + r, tokens 8(g&1) .. +8 of page g>>1
};

template <int D>
__device__ __forceinline__ void load_tile(TileB<D> &t, const __bf16 *kb, const __bf16 *vb, size_t stride,
                                          int pa, int pb, int r, int g) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int tt = 8 * (r >> 2) + 4 * h + (r & 3);
        const int ph = pick(tt >> 4, pa, pb);
        const __bf16 *kp = kb + (size_t)ph * stride + (tt & 15) * D + 8 * g;
#pragma unroll
        for (int s = 0; s < D / 32; ++s) t.k[h][s] = *(const bf16x8 *)(kp + 32 * s);
    }
    const int pv = pick(g >> 1, pa, pb);
    const __bf16 *vp = vb + (size_t)pv * stride + (size_t)r * kPage + 8 * (g & 1);
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) t.v[cb] = *(const bf16x8 *)(vp + (size_t)cb * 16 * kPage);
}

template <int D>
__device__ __forceinline__ void compute_tile(TileB<D> &t, const bf16x8 (&qop)[D / 32], WaveState<D> &st,
                                             int vta, int vtb, float c2, int g) {
    const int vvt = pick(g >> 1, vta, vtb);
    float sc[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
            acc4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.k[h][s], qop[s], acc4, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x = 8 * (g & 1) + 4 * h + i < vvt ? acc4[i] * c2 : -INFINITY;
            sc[4 * h + i] = x;
            tmax = fmaxf(tmax, x);
        }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mnew = fmaxf(st.m, tmax);
    const float alpha = rescale(st.m, mnew);
    const float msafe = mnew == -INFINITY ? 0.0f : mnew;
    st.m = mnew;
    st.l *= alpha;
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) st.o[cb] *= alpha;
    if (vta < kPage || vtb < kPage) {
        // tokens past the sequence end: zero V so stale cache contents cannot reach the output
        const int nv = vvt - 8 * (g & 1);
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (e >= nv) t.v[cb][e] = (__bf16)0.0f;
    }
    bf16x8 phi, plo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float pe = fexp2(sc[e] - msafe);
        st.l += pe;
        const __bf16 hi = (__bf16)pe;
        phi[e] = hi;
        plo[e] = (__bf16)(pe - (float)hi);
    }
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) {
        st.o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.v[cb], phi, st.o[cb], 0, 0, 0);
        st.o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.v[cb], plo, st.o[cb], 0, 0, 0);
    }
}

// Walk NT bf16 tiles (pages phys[0 .. 2 NT)) with the next tile's loads in flight.
template <int D, int NT>
__device__ __forceinline__ void wave_pass_bf16(const AttnParams &p, size_t head0, int kvh, int j, int g,
                                               const int (&phys)[kMaxPagesPerWave],
                                               const int (&vt)[kMaxPagesPerWave], WaveState<D> &st) {
    const size_t stride = (size_t)p.hkv * kPage * D;   // elements per physical page
    const __bf16 *kb = (const __bf16 *)p.k + (size_t)kvh * kPage * D;
    const __bf16 *vb = (const __bf16 *)p.v + (size_t)kvh * kPage * D;
    TileB<D> buf[2];
    load_tile<D>(buf[0], kb, vb, stride, phys[0], phys[1], j, g);
    if constexpr (NT > 1) load_tile<D>(buf[1], kb, vb, stride, phys[2], phys[3], j, g);
    bf16x8 qop[D / 32];
    const __bf16 *qb = (const __bf16 *)p.q + (head0 + (j < p.G ? j : 0)) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
        qop[s] = *(const bf16x8 *)(qb + 32 * s + 8 * g);
        if (j >= p.G) qop[s] = bf16x8{};
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        compute_tile<D>(buf[t & 1], qop, st, vt[2 * t], vt[2 * t + 1], p.c2, g);
        if (t + 2 < NT)
            load_tile<D>(buf[t & 1], kb, vb, stride, phys[2 * t + 4], phys[2 * t + 5], j, g);
    }
}

// ---- fp32 tiles: 16 tokens (1 page) ----

template <int D>
struct TileF {
    f32x4 k[D / 16];   // token j, channels 16 s + 4 g .. +4
    f32x4 v[D / 16];   // channel 16 cb + j, tokens 4 g .. +4
};

template <int D>
__device__ __forceinline__ void load_tile(TileF<D> &t, const float *kf, const float *vf, size_t stride, int ph,
                                          int j, int g) {
    const float *kp = kf + (size_t)ph * stride + j * D + 4 * g;
    const float *vp = vf + (size_t)ph * stride + (size_t)j * kPage + 4 * g;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) t.k[s] = *(const f32x4 *)(kp + 16 * s);
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) t.v[cb] = *(const f32x4 *)(vp + (size_t)cb * 16 * kPage);
}

template <int D>
__device__ __forceinline__ void compute_tile(TileF<D> &t, const f32x4 (&qop)[D / 16], WaveState<D> &st, int vtp,
                                             float c2, int g) {
    f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc4 = __builtin_amdgcn_mfma_f32_16x16x4f32(t.k[s][e], qop[s][e], acc4, 0, 0, 0);
    float sc[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sc[i] = 4 * g + i < vtp ? acc4[i] * c2 : -INFINITY;
        tmax = fmaxf(tmax, sc[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mnew = fmaxf(st.m, tmax);
    const float alpha = rescale(st.m, mnew);
    const float msafe = mnew == -INFINITY ? 0.0f : mnew;
    st.m = mnew;
    st.l *= alpha;
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) st.o[cb] *= alpha;
    if (vtp < kPage) {
        const int nv = vtp - 4 * g;
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (e >= nv) t.v[cb][e] = 0.0f;
    }
    float pe[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        pe[i] = fexp2(sc[i] - msafe);
        st.l += pe[i];
    }
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            st.o[cb] = __builtin_amdgcn_mfma_f32_16x16x4f32(t.v[cb][e], pe[e], st.o[cb], 0, 0, 0);
}

template <int D, int NT>
__device__ __forceinline__ void wave_pass_f32(const AttnParams &p, size_t head0, int kvh, int j, int g,
                                              const int (&phys)[kMaxPagesPerWave],
                                              const int (&vt)[kMaxPagesPerWave], WaveState<D> &st) {
    const size_t stride = (size_t)p.hkv * kPage * D;
    const float *kf = (const float *)p.k + (size_t)kvh * kPage * D;
    const float *vf = (const float *)p.v + (size_t)kvh * kPage * D;
    TileF<D> buf[2];
    load_tile<D>(buf[0], kf, vf, stride, phys[0], j, g);
    if constexpr (NT > 1) load_tile<D>(buf[1], kf, vf, stride, phys[1], j, g);
    f32x4 qop[D / 16];
    const float *qf = (const float *)p.q + (head0 + (j < p.G ? j : 0)) * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        qop[s] = *(const f32x4 *)(qf + 16 * s + 4 * g);
        if (j >= p.G) qop[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        compute_tile<D>(buf[t & 1], qop, st, vt[t], p.c2, g);
        if (t + 2 < NT) load_tile<D>(buf[t & 1], kf, vf, stride, phys[t + 2], j, g);
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

// The last chunk of a unit folds the unit's nch partial states (and, in repair mode, the incoming
// state) into the final one.  A thread owns VW consecutive channels of one query head.  Partials are
// visited in chunk order, MB at a time: every device-scope load of a batch is issued before any is
// used, so a batch costs one memory round trip; batches combine with the same online-softmax step
// (running maximum, rescaled sums), which keeps the result independent of arrival order.
template <int VW, int D, bool REPAIR>
__device__ __forceinline__ void merge_partials(const AttnParams &p, const float *base, int nch, size_t head0,
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
        if (REPAIR) {
            mo = s_mo[jj];
            mo2 = mo == -INFINITY ? -INFINITY : mo * kLog2e;
            mt = mo2;
            ls = s_lo[jj];
#pragma unroll
            for (int v = 0; v < VW; ++v) a[v] = p.acc[head * D + c0 + v];
        }
        for (int w0 = 0; w0 < nch; w0 += MB) {
            float pm[MB], pl[MB], pa[MB][VW];
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const int w = min(w0 + i, nch - 1);   // clamped: a valid partial, weighted 0 below
                const float *pw = base + ((size_t)w * G + jj) * (D + 2);
                pm[i] = ld_dev(&pw[D + 1]);
                pl[i] = ld_dev(&pw[D]);
#pragma unroll
                for (int v = 0; v < VW; ++v) pa[i][v] = ld_dev(&pw[c0 + v]);
            }
            float mb = mt;
#pragma unroll
            for (int i = 0; i < MB; ++i)
                if (w0 + i < nch) mb = fmaxf(mb, pm[i]);
            const float fr = rescale(mt, mb);
            ls *= fr;
#pragma unroll
            for (int v = 0; v < VW; ++v) a[v] *= fr;
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const float f = w0 + i < nch ? rescale(pm[i], mb) : 0.0f;
                ls += f * pl[i];
#pragma unroll
                for (int v = 0; v < VW; ++v) a[v] += f * pa[i][v];
            }
            mt = mb;
        }
#pragma unroll
        for (int v = 0; v < VW; ++v) write_item(p, head, c0 + v, D, a[v], ls, mt, REPAIR && mt == mo2, mo);
    }
}

template <bool BF16, int D, bool REPAIR>
__device__ __forceinline__ void attn_body(const AttnParams &p) {
    constexpr int DP = D + 4;  // padded LDS row
    __shared__ float sm_acc[kWaves][16 * DP];
    __shared__ float sm_m[kWaves][16];
    __shared__ float sm_l[kWaves][16];
    __shared__ float s_mo[16], s_lo[16];   // repair: the incoming state's m and l per query head
    __shared__ int s_last;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15;   // query column / operand row
    const int g = lane >> 4;   // lane group (k slice)
    const int G = p.G;
    const int cp = p.cp;
    const int pw = cp / kWaves;   // pages per wave: 2, 4, 6 or 8 (fp32: 2 or 4)
    const int total = p.units * p.kmax;

    // Chunk c covers pages [k cp, (k + 1) cp) of unit u = c mod units, k = c / units.  Chunks past a
    // unit's set size are skipped; chunk 0 of a unit with an empty set still writes its output.
    for (int c = blockIdx.x; c < total; c += gridDim.x) {
        const int u = c % p.units, k = c / p.units;
        const int b = u / p.hkv, kvh = u - b * p.hkv;
        const int wbeg = k * cp + wave * pw;
        const PageLookup look = page_lookup(p, b, u, wbeg);
        const int npages = unit_pages(p, u);
        const int nch = max(1, (npages + cp - 1) / cp);
        if (k >= nch) continue;
        const int slen = p.seq_len[b];
        const size_t head0 = (size_t)b * p.hq + (size_t)kvh * G;
        if (REPAIR && threadIdx.x < G) {
            s_mo[threadIdx.x] = p.m[head0 + threadIdx.x];
            s_lo[threadIdx.x] = p.l[head0 + threadIdx.x];
        }
        if (REPAIR && npages == 0) {
            // nothing missed: the state stays bit-for-bit as it is; only the normalised output
            if (p.out) {
                for (int it = threadIdx.x; it < G * D; it += kThreads) {
                    const int jj = it / D, cc = it - jj * D;
                    const size_t head = head0 + jj;
                    const float lo_ = p.l[head];
                    p.out[head * D + cc] = lo_ > 0.0f ? p.acc[head * D + cc] / lo_ : 0.0f;
                }
            }
            __syncthreads();
            continue;
        }

        const int cend = min(npages, k * cp + cp);
        const int wend = min(cend, wbeg + pw);

        WaveState<D> st;
#pragma unroll
        for (int cb = 0; cb < D / 16; ++cb) st.o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        st.m = -INFINITY;
        st.l = 0.0f;
        if (wbeg < wend) {
            int phys[kMaxPagesPerWave], vt[kMaxPagesPerWave];
            page_finish<kMaxPagesPerWave>(p, look, wbeg, wend, slen, phys, vt);
            if constexpr (BF16) {
                switch (pw) {
                    case 2: wave_pass_bf16<D, 1>(p, head0, kvh, j, g, phys, vt, st); break;
                    case 4: wave_pass_bf16<D, 2>(p, head0, kvh, j, g, phys, vt, st); break;
                    case 6: wave_pass_bf16<D, 3>(p, head0, kvh, j, g, phys, vt, st); break;
                    default: wave_pass_bf16<D, 4>(p, head0, kvh, j, g, phys, vt, st); break;
                }
            } else {
                if (pw == 2) wave_pass_f32<D, 2>(p, head0, kvh, j, g, phys, vt, st);
                else wave_pass_f32<D, 4>(p, head0, kvh, j, g, phys, vt, st);
            }
        }
        // wave state -> LDS (lane (j, g) holds channels 16 cb + 4 g + i of query j)
        float lsum = st.l;
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        if (j < G) {
#pragma unroll
            for (int cb = 0; cb < D / 16; ++cb) *(f32x4 *)&sm_acc[wave][j * DP + 16 * cb + 4 * g] = st.o[cb];
            if (g == 0) {
                sm_m[wave][j] = st.m;
                sm_l[wave][j] = lsum;
            }
        }
        __syncthreads();

        const bool single = (nch == 1);
        float *part = p.partials + ((size_t)u * p.kmax + k) * G * (D + 2);
        for (int it = threadIdx.x; it < G * D; it += kThreads) {
            const int jj = it / D, cc = it - jj * D;
            float mx = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm_m[w][jj]);
            float a = 0.0f, ls = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float f = rescale(sm_m[w][jj], mx);
                a += f * sm_acc[w][jj * DP + cc];
                ls += f * sm_l[w][jj];
            }
            if (single) {
                const size_t head = head0 + jj;
                if (REPAIR) {
                    const float mo = s_mo[jj];
                    const float mo2 = mo == -INFINITY ? -INFINITY : mo * kLog2e;
                    const float mt = fmaxf(mx, mo2);
                    const float fo = rescale(mo2, mt), fn = rescale(mx, mt);
                    write_item(p, head, cc, D, fo * p.acc[head * D + cc] + fn * a, fo * s_lo[jj] + fn * ls,
                               mt, mt == mo2, mo);
                } else {
                    write_item(p, head, cc, D, a, ls, mx, false, 0.0f);
                }
            } else {
                st_dev(&part[jj * (D + 2) + cc], a);
                if (cc == 0) {
                    st_dev(&part[jj * (D + 2) + D], ls);
                    st_dev(&part[jj * (D + 2) + D + 1], mx);
                }
            }
        }
        if (single) {
            __syncthreads();   // LDS is reused by the next chunk
            continue;
        }

        // Cross-chunk merge: the last chunk of the unit to finish folds every partial in chunk order.
        // Partials are written and read with device-scope (sc1) accesses, which are coherent across
        // the XCDs' L2s by themselves; waiting for this thread's stores to complete before the barrier,
        // and the barrier before the counter increment, orders them ahead of it.  This avoids a
        // device-scope release fence, which would write back every dirty line of the L2.
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) {
            const uint32_t prev = __hip_atomic_fetch_add(&p.counters[u], 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            s_last = (prev == (uint32_t)(nch - 1));
        }
        __syncthreads();
        if (s_last) {
            const float *base = p.partials + (size_t)u * p.kmax * G * (D + 2);
            if (G * D <= 2 * kThreads) merge_partials<2, D, REPAIR>(p, base, nch, head0, s_mo, s_lo);
            else merge_partials<4, D, REPAIR>(p, base, nch, head0, s_mo, s_lo);
            if (threadIdx.x == 0)
                __hip_atomic_store(&p.counters[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
    }
}

// bf16 (the streaming path) is held to 256 registers so two waves share each SIMD; the fp32 variant
// (exact-input checks) may use more.
template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_spec_bf16(AttnParams p) {
    attn_body<true, D, false>(p);
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attn_repair_bf16(AttnParams p) {
    attn_body<true, D, true>(p);
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_spec_f32(AttnParams p) {
    attn_body<false, D, false>(p);
}

template <int D>
__global__ __launch_bounds__(kThreads) void attn_repair_f32(AttnParams p) {
    attn_body<false, D, true>(p);
}

__global__ void clear_kernel(uint32_t *w, size_t n) {
    for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        w[i] = 0u;
}

size_t counters_bytes(int units) { return ((size_t)units * 4 + 255) / 256 * 256; }

// Partials kept per launch: every chunk of every unit at the smallest chunk size.
size_t max_chunks(int units, int block, int cap) {
    const long pages = (long)cap * (block / kPage);
    return (size_t)units * (size_t)std::max<long>(1, (pages + kChunkMin - 1) / kChunkMin);
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
    p.units = units;
    p.hq = hq;
    p.hkv = kv.hkv;
    p.G = hq / kv.hkv;
    p.cap = cap;
    p.ppb = block / kPage;
    p.max_pages = kv.max_pages;
    p.num_pages = kv.num_pages;
    p.c2 = scale * kLog2e;
    // Workgroups in flight.  The speculative pass runs next to selection, so it keeps one workgroup per
    // CU (half of every SIMD's registers) and leaves the other half to the selection kernels; a
    // workgroup then walks several chunks in turn.  Repair runs alone on the critical path and takes two
    // workgroups per CU.  The chunk size spreads a full set (count = cap) over the target; repair sets
    // are usually a fraction of the capacity (the missed part of the selection), so repair uses half
    // of that chunk size to keep the chip busy.
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) cus = n;
    }
    const long target = repair ? 2L * cus : (long)cus;
    const long cap_pages = (long)cap * p.ppb;
    const long full = (long)units * cap_pages;
    const int cmax = kv.bf16 ? kChunkMax : kChunkMaxF32;
    auto round8 = [](long x) { return (x + kChunkMin - 1) / kChunkMin * kChunkMin; };
    long cp = std::min<long>(std::max<long>(round8((full + target - 1) / target), kChunkMin), cmax);
    if (repair) cp = std::max<long>(kChunkMin, round8(cp / 2));
    p.cp = (int)cp;
    p.kmax = (int)std::max<long>(1, (cap_pages + cp - 1) / cp);
    const int grid = (int)std::min<long>((long)units * p.kmax, target);
    const dim3 blk(kThreads);
    if (kv.bf16) {
        if (repair) {
            if (kv.d == 128) attn_repair_bf16<128><<<grid, blk, 0, stream>>>(p);
            else attn_repair_bf16<64><<<grid, blk, 0, stream>>>(p);
        } else {
            if (kv.d == 128) attn_spec_bf16<128><<<grid, blk, 0, stream>>>(p);
            else attn_spec_bf16<64><<<grid, blk, 0, stream>>>(p);
        }
    } else {
        if (repair) {
            if (kv.d == 128) attn_repair_f32<128><<<grid, blk, 0, stream>>>(p);
            else attn_repair_f32<64><<<grid, blk, 0, stream>>>(p);
        } else {
            if (kv.d == 128) attn_spec_f32<128><<<grid, blk, 0, stream>>>(p);
            else attn_spec_f32<64><<<grid, blk, 0, stream>>>(p);
        }
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
