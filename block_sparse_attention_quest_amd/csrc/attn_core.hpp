// attn_core.hpp - device code of the speculative block-sparse decode attention and incremental
// repair (gfx950), shared by the attention kernels and the fused selection + speculation launch.
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
//     (8..256, a multiple of 8, chosen at launch so that sets at full capacity spread over about one
//     workgroup per CU; half that chunk size for repair, whose sets are the missed part of a
//     selection).  Chunk
//     c belongs to unit c mod units, so a unit's chunks are dispatched to the same XCD and every XCD
//     gets the same number of units.  Workgroup i takes chunks i, i + grid, ...; a chunk past its
//     unit's set size is skipped after one load.  The set size, set entries and page-table entries are
//     looked up with addresses that do not depend on each other where possible: two memory rounds
//     before the first K/V load.
//   * Streaming.  Each of the 4 waves of a workgroup owns a quarter of the chunk (up to 64 pages, one
//     page-table lookup per lane, broadcast with readlane as the wave walks) and walks it in tiles
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
//   * fp8 (E4M3 codes, bf16 queries): the bf16 structure on half the bytes.  A lane loads 16 channels of
//     a K token (the channels of two k-steps; the query operand takes the same channel order) and 8
//     tokens of a V channel, and converts them to bf16 in registers, exactly; the products are the bf16
//     ones.
//   * fp32: the same structure on v_mfma_f32_16x16x4_f32.
//   * Softmax: online across tiles (running maximum per query, rescaled sums); waves merge in LDS;
//     chunks of one unit merge through a small workspace: the last chunk of a unit to finish
//     (device-scope counter) folds the partials in chunk order, so results are deterministic.
//   * Exponentials use the hardware base-2 exponential on log2(e)-prescaled scores; m is stored in
//     natural-log units.

#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "kv_types.hpp"
#include "prr_internal.hpp"

namespace prr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kChunkStep = 8;    // pages per chunk: a multiple of 8 (2 pages per wave), ...
constexpr int kChunkMin = 16;    // ... at least 16 (both tiles of a wave's pair in flight at once) ...
constexpr int kChunkMax = 256;   // ... up to 64 pages per wave: one page-table lookup per lane
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
    const int32_t *pages;   // the set's page work list (may be null): [units][cap ppb] physical pages or -1
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

// A K/V tile load: plain, or non-temporal (NT: the line is streamed through without being kept in the
// caches).  Every tile is read once.  V tiles always use NT loads; K tiles use them in the speculative
// pass only.  Measured at 128K context, batch 8: NT loads took the speculative pass from 30.6 to 29.2 us;
// in repair, whose tiles arrive in one burst, NT on V alone saved 0.5 us, while NT on K cost 1.1 us.
template <bool NT, typename T>
__device__ __forceinline__ T ld_tile(const void *ptr) {
    if constexpr (NT) return __builtin_nontemporal_load((const T *)ptr);
    else return *(const T *)ptr;
}

// Device-scope (all XCDs) coherent store and load of two adjacent floats (8-byte aligned), x in the
// low word.
__device__ __forceinline__ void st_dev2(float *ptr, float x, float y) {
    const uint64_t w = (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
    __hip_atomic_store((uint64_t *)ptr, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev2(const float *ptr) {
    return __hip_atomic_load((const uint64_t *)ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float lo_f(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ float hi_f(uint64_t w) { return __uint_as_float((uint32_t)(w >> 32)); }

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

// Set entries and sizes written earlier in the same launch by a workgroup of another XCD are read with
// device-scope loads (COHERENT); a set from an earlier launch with plain ones.
template <bool COHERENT = false>
__device__ __forceinline__ int ld_set(const int32_t *ptr) {
    if constexpr (COHERENT) return __hip_atomic_load(ptr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *ptr;
}

template <bool COHERENT = false>
__device__ __forceinline__ int unit_pages(const AttnParams &p, int u) {
    return min(max(ld_set<COHERENT>(&p.count[u]), 0), p.cap) * p.ppb;
}

// Page lookups of the wave's pages wbeg .. wbeg + N - 1 of the unit's expanded page list.  Lane
// i < N looks up page wbeg + i with vector loads: the set entry, then the page-table entry (two
// dependent memory rounds, through the vector memory path, which keeps many more requests in flight
// than the scalar cache).  With a page work list (p.pages) the physical page comes with the set entry,
// in the same round: only a list slot of -1 whose page holds tokens by now (slen: the sequence length)
// is looked up in the page table; a -1 page without tokens is masked whatever its address.  The addresses
// do not depend on the set size, so these loads are issued together with the load of the set size;
// finish() masks entries at or past wend and broadcasts physical page and valid-token count to scalar
// registers.
struct PageLookup {
    int ph;     // physical page (raw)
    int lp;     // logical page (0 when the set entry is out of range)
    bool lp_ok; // set entry in range
};

template <bool COHERENT = false>
__device__ __forceinline__ PageLookup page_lookup(const AttnParams &p, int b, int u, int wbeg, int pw, int slen) {
    const int i = threadIdx.x & 63;
    PageLookup r;
    r.ph = 0;
    r.lp = 0;
    r.lp_ok = false;
    if (i < pw) {
        const int gpc = min(wbeg + i, p.cap * p.ppb - 1);
        const int li = gpc / p.ppb;
        const int sub = gpc - li * p.ppb;
        const int blk = ld_set<COHERENT>(&p.idx[(size_t)u * p.cap + li]);
        const int listed = p.pages ? ld_set<COHERENT>(&p.pages[((size_t)u * p.cap) * p.ppb + gpc]) : -1;
        const long lp = (long)blk * p.ppb + sub;
        r.lp_ok = blk >= 0 && lp < p.max_pages;
        r.lp = r.lp_ok ? (int)lp : 0;
        if (!p.pages || (listed < 0 && r.lp_ok && (long)r.lp * kPage < slen))
            r.ph = p.page_table[(size_t)b * p.max_pages + r.lp];
        else
            r.ph = listed;
    }
    return r;
}

// Lane i's page of the wave list: physical page (clamped into the cache) and valid-token count.
// Entries at or past wend are padding: valid-token count 0 (the tile computation masks them out) and
// the wave's last real page as the address, which was just read and is served from cache.
struct LanePage {
    int ph;
    int vt;
};

__device__ __forceinline__ LanePage page_finish(const AttnParams &p, const PageLookup &r, int wbeg, int wend,
                                                int slen) {
    const int i = threadIdx.x & 63;
    const bool in = wbeg + i < wend;
    const int ph = min(max(r.ph, 0), p.num_pages - 1);
    const int last = __builtin_amdgcn_readlane(ph, wend - wbeg - 1);
    LanePage lp;
    lp.vt = in && r.lp_ok ? min(max(slen - r.lp * kPage, 0), kPage) : 0;
    lp.ph = in ? ph : last;
    return lp;
}

// Page i of the wave list, broadcast from lane i (i is wave-uniform).
__device__ __forceinline__ int lane_val(int v, int i) { return __builtin_amdgcn_readlane(v, i); }

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

template <int D, bool NT>
__device__ __forceinline__ void load_tile(TileB<D> &t, const __bf16 *kb, const __bf16 *vb, size_t stride,
                                          int pa, int pb, int r, int g) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int tt = 8 * (r >> 2) + 4 * h + (r & 3);
        const int ph = pick(tt >> 4, pa, pb);
        const __bf16 *kp = kb + (size_t)ph * stride + (tt & 15) * D + 8 * g;
#pragma unroll
        for (int s = 0; s < D / 32; ++s) t.k[h][s] = ld_tile<NT, bf16x8>(kp + 32 * s);
    }
    const int pv = pick(g >> 1, pa, pb);
    const __bf16 *vp = vb + (size_t)pv * stride + (size_t)r * kPage + 8 * (g & 1);
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) t.v[cb] = ld_tile<true, bf16x8>(vp + (size_t)cb * 16 * kPage);
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

// Walk nt bf16 tiles (tile t = pages 2t and 2t + 1 of the wave list, held by lanes 2t and 2t + 1 of
// pg) with NBUF tiles in flight: while one is multiplied, the next NBUF - 1 are loading.  The tile count
// is padded to a multiple of NBUF (padding pages are masked and re-read cached addresses), so the
// steady-state loop issues all of its loads unconditionally: every path into the loop header then has
// the same loads outstanding and the compiler's wait counts keep the other tiles in flight while one is
// multiplied.  The loop is not unrolled, so register use does not depend on the tile count.  q is loaded
// first so that the first tile waits for q and its own loads only.
template <int D, int NBUF, bool NT>
__device__ __forceinline__ void wave_pass_bf16(const AttnParams &p, size_t head0, int kvh, int j, int g,
                                               LanePage pg, int nt, WaveState<D> &st) {
    const size_t stride = (size_t)p.hkv * kPage * D;   // elements per physical page
    const __bf16 *kb = (const __bf16 *)p.k + (size_t)kvh * kPage * D;
    const __bf16 *vb = (const __bf16 *)p.v + (size_t)kvh * kPage * D;
    bf16x8 qop[D / 32];
    const __bf16 *qb = (const __bf16 *)p.q + (head0 + (j < p.G ? j : 0)) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qop[s] = *(const bf16x8 *)(qb + 32 * s + 8 * g);
    auto load = [&](TileB<D> &tb, int t) {
        load_tile<D, NT>(tb, kb, vb, stride, lane_val(pg.ph, 2 * t), lane_val(pg.ph, 2 * t + 1), j, g);
    };
    auto comp = [&](TileB<D> &tb, int t) {
        compute_tile<D>(tb, qop, st, lane_val(pg.vt, 2 * t), lane_val(pg.vt, 2 * t + 1), p.c2, g);
    };
    const int nte = (nt + NBUF - 1) / NBUF * NBUF;   // <= 32: pages 2t, 2t + 1 stay below lane 64
    TileB<D> buf[NBUF];
#pragma unroll
    for (int b = 0; b < NBUF; ++b) load(buf[b], b);
    if (j >= p.G) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) qop[s] = bf16x8{};
    }
    int t = 0;
#pragma unroll 1
    for (; t + NBUF < nte; t += NBUF) {
#pragma unroll
        for (int b = 0; b < NBUF; ++b) {
            comp(buf[b], t + b);
            load(buf[b], t + NBUF + b);
        }
    }
#pragma unroll
    for (int b = 0; b < NBUF; ++b) comp(buf[b], t + b);
}

// ---- fp8 tiles: 32 tokens (2 pages) of E4M3 codes ----

template <int D>
struct TileE {
    u32x4 k[2][D / 64];   // half h, m: row r of S^T -> token 8(r>>2) + 4h + (r&3), channels 64 m + 16 g .. +16
    u32x2 v[D / 16];      // channel block cb: channel 16 cb + r, tokens 8(g&1) .. +8 of page g>>1
};

template <int D, bool NT>
__device__ __forceinline__ void load_tile(TileE<D> &t, const uint8_t *kb, const uint8_t *vb, size_t stride,
                                          int pa, int pb, int r, int g) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int tt = 8 * (r >> 2) + 4 * h + (r & 3);
        const int ph = pick(tt >> 4, pa, pb);
        const uint8_t *kp = kb + (size_t)ph * stride + (tt & 15) * D + 16 * g;
#pragma unroll
        for (int m = 0; m < D / 64; ++m) t.k[h][m] = ld_tile<NT, u32x4>(kp + 64 * m);
    }
    const int pv = pick(g >> 1, pa, pb);
    const uint8_t *vp = vb + (size_t)pv * stride + (size_t)r * kPage + 8 * (g & 1);
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) t.v[cb] = ld_tile<true, u32x2>(vp + (size_t)cb * 16 * kPage);
}

// Eight E4M3 codes (bytes of lo, then of hi) as eight bf16 values, exactly.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
    const bf16x2v a = fp8x2_to_bf16<false>(lo), b = fp8x2_to_bf16<true>(lo);
    const bf16x2v c = fp8x2_to_bf16<false>(hi), d = fp8x2_to_bf16<true>(hi);
    bf16x8 r;
    r[0] = a[0];
    r[1] = a[1];
    r[2] = b[0];
    r[3] = b[1];
    r[4] = c[0];
    r[5] = c[1];
    r[6] = d[0];
    r[7] = d[1];
    return r;
}

// The tile in bf16 (k-step 2 m + e takes channels 64 m + 16 g + 8 e .. +8), then the bf16 products.
template <int D>
__device__ __forceinline__ void compute_tile(const TileE<D> &t, const bf16x8 (&qop)[D / 32], WaveState<D> &st,
                                             int vta, int vtb, float c2, int g) {
    TileB<D> tb;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int m = 0; m < D / 64; ++m) {
            tb.k[h][2 * m] = fp8x8_to_bf16(t.k[h][m].x, t.k[h][m].y);
            tb.k[h][2 * m + 1] = fp8x8_to_bf16(t.k[h][m].z, t.k[h][m].w);
        }
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) tb.v[cb] = fp8x8_to_bf16(t.v[cb].x, t.v[cb].y);
    compute_tile<D>(tb, qop, st, vta, vtb, c2, g);
}

// Walk nt fp8 tiles, structured like the bf16 walk; the query operand takes the fp8 tiles' channel
// order.
template <int D, int NBUF, bool NT>
__device__ __forceinline__ void wave_pass_fp8(const AttnParams &p, size_t head0, int kvh, int j, int g,
                                              LanePage pg, int nt, WaveState<D> &st) {
    const size_t stride = (size_t)p.hkv * kPage * D;   // bytes per physical page
    const uint8_t *kb = (const uint8_t *)p.k + (size_t)kvh * kPage * D;
    const uint8_t *vb = (const uint8_t *)p.v + (size_t)kvh * kPage * D;
    bf16x8 qop[D / 32];
    const __bf16 *qb = (const __bf16 *)p.q + (head0 + (j < p.G ? j : 0)) * D;
#pragma unroll
    for (int m = 0; m < D / 64; ++m)
#pragma unroll
        for (int e = 0; e < 2; ++e) qop[2 * m + e] = *(const bf16x8 *)(qb + 64 * m + 16 * g + 8 * e);
    auto load = [&](TileE<D> &tb, int t) {
        load_tile<D, NT>(tb, kb, vb, stride, lane_val(pg.ph, 2 * t), lane_val(pg.ph, 2 * t + 1), j, g);
    };
    auto comp = [&](TileE<D> &tb, int t) {
        compute_tile<D>(tb, qop, st, lane_val(pg.vt, 2 * t), lane_val(pg.vt, 2 * t + 1), p.c2, g);
    };
    const int nte = (nt + NBUF - 1) / NBUF * NBUF;   // <= 32: pages 2t, 2t + 1 stay below lane 64
    TileE<D> buf[NBUF];
#pragma unroll
    for (int b = 0; b < NBUF; ++b) load(buf[b], b);
    if (j >= p.G) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) qop[s] = bf16x8{};
    }
    int t = 0;
#pragma unroll 1
    for (; t + NBUF < nte; t += NBUF) {
#pragma unroll
        for (int b = 0; b < NBUF; ++b) {
            comp(buf[b], t + b);
            load(buf[b], t + NBUF + b);
        }
    }
#pragma unroll
    for (int b = 0; b < NBUF; ++b) comp(buf[b], t + b);
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

// Walk nt fp32 tiles (tile t = page t of the wave list), structured like the bf16 walk.
template <int D>
__device__ __forceinline__ void wave_pass_f32(const AttnParams &p, size_t head0, int kvh, int j, int g,
                                              LanePage pg, int nt, WaveState<D> &st) {
    const size_t stride = (size_t)p.hkv * kPage * D;
    const float *kf = (const float *)p.k + (size_t)kvh * kPage * D;
    const float *vf = (const float *)p.v + (size_t)kvh * kPage * D;
    f32x4 qop[D / 16];
    const float *qf = (const float *)p.q + (head0 + (j < p.G ? j : 0)) * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qop[s] = *(const f32x4 *)(qf + 16 * s + 4 * g);
    auto load = [&](TileF<D> &tf, int t) { load_tile<D>(tf, kf, vf, stride, lane_val(pg.ph, t), j, g); };
    auto comp = [&](TileF<D> &tf, int t) { compute_tile<D>(tf, qop, st, lane_val(pg.vt, t), p.c2, g); };
    const int nte = (nt + 1) & ~1;
    TileF<D> buf[2];
    load(buf[0], 0);
    load(buf[1], 1);
    if (j >= p.G) {
#pragma unroll
        for (int s = 0; s < D / 16; ++s) qop[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    int t = 0;
#pragma unroll 1
    for (; t + 2 < nte; t += 2) {
        comp(buf[0], t);
        load(buf[0], t + 2);
        comp(buf[1], t + 1);
        load(buf[1], t + 3);
    }
    comp(buf[0], t);
    comp(buf[1], t + 1);
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
// visited in chunk order, MB at a time: every device-scope load of a batch (8 bytes each: l and m, then
// channel pairs) is issued before any is used, so a batch costs one memory round trip; slots past nch
// are the empty state (l = 0, m = -inf, acc = 0), which the merge step leaves without effect.  Batches
// combine with the same online-softmax step (running maximum, rescaled sums), which keeps the result
// independent of arrival order.
template <int VW, int D, bool REPAIR>
__device__ __forceinline__ void merge_partials(const AttnParams &p, const float *base, int nch, size_t head0,
                                               const float *s_mo, const float *s_lo, int tid,
                                               const float *base2 = nullptr, int n2 = 0) {
    constexpr int MB = 8;
    constexpr int CPH = D / VW;   // channel groups per head
    const int G = p.G;
    for (int it = tid; it < G * CPH; it += kThreads) {
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
        // slots [0, nch) at base, then [nch, nch + n2) at base2
        const int ntot = nch + n2;
        for (int w0 = 0; w0 < ntot; w0 += MB) {
            uint64_t lm[MB], pa[MB][VW / 2];
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                lm[i] = (uint64_t)__float_as_uint(-INFINITY) << 32;
#pragma unroll
                for (int v = 0; v < VW / 2; ++v) pa[i][v] = 0;
                if (w0 + i < ntot) {
                    const int w = w0 + i;
                    const float *pw = (w < nch ? base + (size_t)w * G * (D + 2) : base2 + (size_t)(w - nch) * G * (D + 2)) +
                                      (size_t)jj * (D + 2);
                    lm[i] = ld_dev2(&pw[D]);
#pragma unroll
                    for (int v = 0; v < VW / 2; ++v) pa[i][v] = ld_dev2(&pw[c0 + 2 * v]);
                }
            }
            float mb = mt;
#pragma unroll
            for (int i = 0; i < MB; ++i) mb = fmaxf(mb, hi_f(lm[i]));
            const float fr = rescale(mt, mb);
            ls *= fr;
#pragma unroll
            for (int v = 0; v < VW; ++v) a[v] *= fr;
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const float f = rescale(hi_f(lm[i]), mb);
                ls += f * lo_f(lm[i]);
#pragma unroll
                for (int v = 0; v < VW / 2; ++v) {
                    a[2 * v] += f * lo_f(pa[i][v]);
                    a[2 * v + 1] += f * hi_f(pa[i][v]);
                }
            }
            mt = mb;
        }
#pragma unroll
        for (int v = 0; v < VW; ++v) write_item(p, head, c0 + v, D, a[v], ls, mt, REPAIR && mt == mo2, mo);
    }
}

// LDS of the attention chunk walk: the waves' partial states, the incoming state's m and l (repair),
// the last-arriver flag.  A kernel with several roles declares it once and hands it to each.
template <int D>
struct AttnSmem {
    float acc[kWaves][16 * (D + 4)];   // padded rows
    float m[kWaves][16];
    float l[kWaves][16];
    float mo[16], lo[16];
    int last;
};

// The layer step as one launch (selection, the speculative pass and repair in one grid): the speculative
// chunks of a unit and its repair slots (the missed set M cut into chunks of cp_rep pages, kmax_rep slots
// per unit at full capacity) all write partial states; every speculative chunk and every repair slot
// arrives on the unit's counter, nch_spec + kmax_rep in all, and the last one merges the speculative
// partials and then the repair partials (slot order: deterministic) into the final state over P u M.  A
// repair slot first waits for the unit's M (the flag its top-K sets after storing M with device-scope
// stores); slots past M's chunks arrive without a partial.  The merge resets the counter and the flag for
// the next launch.
// Unit u's M flag is word u * kReadyStride of the flag array: one flag per 256 bytes, so that the repair
// slots polling different units' flags do not all poll the same few cache lines (measured at 128K, batch
// 8: 50.9 us for the layer step with the flags packed, 50.1 us spaced).
constexpr int kReadyStride = 64;

struct FusedParams {
    AttnParams pm;          // M's set: chunks of cp_rep pages, kmax_rep slots per unit, partials [units][kmax_rep][G][D + 2]
    uint32_t *ready;        // [units] M of the unit stored (set by its top-K, reset by its merge)
    uint32_t *status;       // set when a repair slot gave up waiting for M (see wait_ready)
};

template <int KT, int D, bool REPAIR, int NBUF, bool FUSED>
__device__ __forceinline__ void attn_chunks(const AttnParams &p, const FusedParams &fp, int wg, int nwg,
                                            AttnSmem<D> &sm);

template <int KT, int D, bool REPAIR, int NBUF = 2>
__device__ __forceinline__ void attn_body(const AttnParams &p, int wg, int nwg) {
    __shared__ AttnSmem<D> sm;
    attn_chunks<KT, D, REPAIR, NBUF, false>(p, FusedParams{}, wg, nwg, sm);
}

// The final merge of a unit of the fused launch: its speculative partials (P's chunks), then the partials
// of M's chunks; resets the unit's counter and M flag.  pm: M's set (for its chunk count).
template <int D>
__device__ __forceinline__ void fused_merge(const AttnParams &p, const AttnParams &pm, const FusedParams &fp, int u,
                                            size_t head0, int nch_spec, int tid) {
    const int nrep = (unit_pages<true>(pm, u) + pm.cp - 1) / pm.cp;
    const int G = p.G;
    const float *base = p.partials + (size_t)u * p.kmax * G * (D + 2);
    const float *base2 = pm.partials + (size_t)u * pm.kmax * G * (D + 2);
    if (G * D <= 2 * kThreads) merge_partials<2, D, false>(p, base, nch_spec, head0, nullptr, nullptr, tid, base2, nrep);
    else merge_partials<4, D, false>(p, base, nch_spec, head0, nullptr, nullptr, tid, base2, nrep);
    if (tid == 0) {
        __hip_atomic_store(&p.counters[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&fp.ready[u * kReadyStride], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <int KT, int D, bool REPAIR, int NBUF, bool FUSED>
__device__ __forceinline__ void attn_chunks(const AttnParams &p, const FusedParams &fp, int wg, int nwg,
                                            AttnSmem<D> &sm) {
    constexpr int DP = D + 4;  // padded LDS row
    auto &sm_acc = sm.acc;
    auto &sm_m = sm.m;
    auto &sm_l = sm.l;
    float *s_mo = sm.mo;   // repair: the incoming state's m and l per query head
    float *s_lo = sm.lo;
    int &s_last = sm.last;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15;   // query column / operand row
    const int g = lane >> 4;   // lane group (k slice)
    const int G = p.G;
    const int cp = p.cp;
    const int pw = cp / kWaves;   // pages per wave: an even number from 4 to 64
    const int total = p.units * p.kmax;

    // Chunk c covers pages [k cp, (k + 1) cp) of unit u = c mod units, k = c / units.  Chunks past a
    // unit's set size are skipped; chunk 0 of a unit with an empty set still writes its output.
    for (int c = wg; c < total; c += nwg) {
        const int u = c % p.units, k = c / p.units;
        const int b = u / p.hkv, kvh = u - b * p.hkv;
        const int wbeg = k * cp + wave * pw;
        const int slen = p.seq_len[b];
        const PageLookup look = page_lookup(p, b, u, wbeg, pw, slen);
        // In repair mode the incoming m and l go out with the set lookups and reach LDS only after the
        // tile walk, so no tile load waits for them.
        float mo_in = 0.0f, lo_in = 0.0f;
        if (REPAIR && threadIdx.x < G) {
            const size_t h = (size_t)b * p.hq + (size_t)kvh * G + threadIdx.x;
            mo_in = p.m[h];
            lo_in = p.l[h];
        }
        const int npages = unit_pages(p, u);
        const int nch = max(1, (npages + cp - 1) / cp);
        if (k >= nch) continue;
        const size_t head0 = (size_t)b * p.hq + (size_t)kvh * G;
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
            const LanePage pg = page_finish(p, look, wbeg, wend, slen);
            const int nw = wend - wbeg;   // pages of this wave, 1 .. pw
            if constexpr (KT == kKtBf16)
                wave_pass_bf16<D, NBUF, !REPAIR>(p, head0, kvh, j, g, pg, (nw + 1) / 2, st);
            else if constexpr (KT == kKtFp8)
                wave_pass_fp8<D, NBUF, !REPAIR>(p, head0, kvh, j, g, pg, (nw + 1) / 2, st);
            else wave_pass_f32<D>(p, head0, kvh, j, g, pg, nw, st);
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
        if (REPAIR && threadIdx.x < G) {
            s_mo[threadIdx.x] = mo_in;
            s_lo[threadIdx.x] = lo_in;
        }
        __syncthreads();

        const bool single = !FUSED && nch == 1;   // the fused launch merges every unit with its repair
        float *part = p.partials + ((size_t)u * p.kmax + k) * G * (D + 2);
        // The thread index as an opaque value: the per-thread offsets below are then computed here,
        // after the tile walk, instead of being hoisted to the kernel start and kept live through it.
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        for (int it = tid; it < G * D / 2; it += kThreads) {
            const int jj = it / (D / 2), cc = (it - jj * (D / 2)) * 2;   // channels cc, cc + 1
            float mx = -INFINITY;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm_m[w][jj]);
            float a0 = 0.0f, a1 = 0.0f, ls = 0.0f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float f = rescale(sm_m[w][jj], mx);
                const float2 x = *(const float2 *)&sm_acc[w][jj * DP + cc];
                a0 += f * x.x;
                a1 += f * x.y;
                ls += f * sm_l[w][jj];
            }
            if (single) {
                const size_t head = head0 + jj;
                if (REPAIR) {
                    const float mo = s_mo[jj];
                    const float mo2 = mo == -INFINITY ? -INFINITY : mo * kLog2e;
                    const float mt = fmaxf(mx, mo2);
                    const float fo = rescale(mo2, mt), fn = rescale(mx, mt);
                    const float lt = fo * s_lo[jj] + fn * ls;
                    write_item(p, head, cc, D, fo * p.acc[head * D + cc] + fn * a0, lt, mt, mt == mo2, mo);
                    write_item(p, head, cc + 1, D, fo * p.acc[head * D + cc + 1] + fn * a1, lt, mt, mt == mo2, mo);
                } else {
                    write_item(p, head, cc, D, a0, ls, mx, false, 0.0f);
                    write_item(p, head, cc + 1, D, a1, ls, mx, false, 0.0f);
                }
            } else {
                st_dev2(&part[jj * (D + 2) + cc], a0, a1);
                if (cc == 0) st_dev2(&part[jj * (D + 2) + D], ls, mx);
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
            s_last = FUSED ? prev == (uint32_t)(nch + fp.pm.kmax - 1) : prev == (uint32_t)(nch - 1);
        }
        __syncthreads();
        if (s_last) {
            if constexpr (FUSED) {
                fused_merge<D>(p, fp.pm, fp, u, head0, nch, tid);
            } else {
                const float *base = p.partials + (size_t)u * p.kmax * G * (D + 2);
                if (G * D <= 2 * kThreads) merge_partials<2, D, REPAIR>(p, base, nch, head0, s_mo, s_lo, tid);
                else merge_partials<4, D, REPAIR>(p, base, nch, head0, s_mo, s_lo, tid);
                if (threadIdx.x == 0)
                    __hip_atomic_store(&p.counters[u], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __syncthreads();
    }
}

// Thread 0 of a repair slot waits for the unit's M (set by the unit's top-K in the same launch).  The
// top-K runs in a scoring workgroup, and workgroups are dispatched in index order, scoring first, so the
// workgroup a slot waits for is running or done by the time the slot runs.  The wait is bounded all the
// same, so that no wave can spin forever: after about a second the slot sets *status and goes on (the
// state then lacks the unit's M).
__device__ __forceinline__ void wait_ready(const FusedParams &fp, int u) {
    uint32_t n = 0;
    while (__hip_atomic_load(&fp.ready[u * kReadyStride], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
        __builtin_amdgcn_s_sleep(8);
        if (++n >= (1u << 22)) {
            __hip_atomic_store(fp.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
    }
}

// The repair slots of the fused launch: slot c covers pages [k cp_rep, (k + 1) cp_rep) of unit u's M
// (u = c mod units, k = c / units, so the first chunks of every unit come first).  After M is stored, the
// slot walks its pages like a chunk of prr_repair without an incoming state, stores its partial and
// arrives; slots past M's pages arrive without one.  ps: P's set (the unit's speculative chunk count and
// the final outputs).
template <int KT, int D, int NBUF>
__device__ __forceinline__ void fused_repair_slots(const AttnParams &ps, const FusedParams &fp, int wg, int nwg,
                                                   AttnSmem<D> &sm) {
    constexpr int DP = D + 4;
    const AttnParams &pm = fp.pm;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int j = lane & 15;
    const int g = lane >> 4;
    const int G = pm.G;
    const int cp = pm.cp;
    const int pw = cp / kWaves;
    const int total = pm.units * pm.kmax;
    for (int c = wg; c < total; c += nwg) {
        const int u = c % pm.units, k = c / pm.units;
        const int b = u / pm.hkv, kvh = u - b * pm.hkv;
        const int nsp = unit_pages(ps, u);   // P is an input of the launch: plain loads
        const int slen = pm.seq_len[b];
        if (threadIdx.x == 0) wait_ready(fp, u);
        __syncthreads();
        const int wbeg = k * cp + wave * pw;
        const PageLookup look = page_lookup<true>(pm, b, u, wbeg, pw, slen);
        const int npages = unit_pages<true>(pm, u);
        const int nch_spec = max(1, (nsp + ps.cp - 1) / ps.cp);
        const size_t head0 = (size_t)b * pm.hq + (size_t)kvh * G;
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        if (k * cp < npages) {
            const int cend = min(npages, k * cp + cp);
            const int wend = min(cend, wbeg + pw);
            WaveState<D> st;
#pragma unroll
            for (int cb = 0; cb < D / 16; ++cb) st.o[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
            st.m = -INFINITY;
            st.l = 0.0f;
            if (wbeg < wend) {
                const LanePage pg = page_finish(pm, look, wbeg, wend, slen);
                const int nw = wend - wbeg;
                if constexpr (KT == kKtBf16)
                    wave_pass_bf16<D, NBUF, false>(pm, head0, kvh, j, g, pg, (nw + 1) / 2, st);
                else if constexpr (KT == kKtFp8)
                    wave_pass_fp8<D, NBUF, false>(pm, head0, kvh, j, g, pg, (nw + 1) / 2, st);
                else wave_pass_f32<D>(pm, head0, kvh, j, g, pg, nw, st);
            }
            float lsum = st.l;
            lsum += __shfl_xor(lsum, 16);
            lsum += __shfl_xor(lsum, 32);
            if (j < G) {
#pragma unroll
                for (int cb = 0; cb < D / 16; ++cb) *(f32x4 *)&sm.acc[wave][j * DP + 16 * cb + 4 * g] = st.o[cb];
                if (g == 0) {
                    sm.m[wave][j] = st.m;
                    sm.l[wave][j] = lsum;
                }
            }
            __syncthreads();
            float *part = pm.partials + ((size_t)u * pm.kmax + k) * G * (D + 2);
            for (int it = tid; it < G * D / 2; it += kThreads) {
                const int jj = it / (D / 2), cc = (it - jj * (D / 2)) * 2;
                float mx = -INFINITY;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm.m[w][jj]);
                float a0 = 0.0f, a1 = 0.0f, ls = 0.0f;
#pragma unroll
                for (int w = 0; w < kWaves; ++w) {
                    const float f = rescale(sm.m[w][jj], mx);
                    const float2 x = *(const float2 *)&sm.acc[w][jj * DP + cc];
                    a0 += f * x.x;
                    a1 += f * x.y;
                    ls += f * sm.l[w][jj];
                }
                st_dev2(&part[jj * (D + 2) + cc], a0, a1);
                if (cc == 0) st_dev2(&part[jj * (D + 2) + D], ls, mx);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) {
            const uint32_t prev = __hip_atomic_fetch_add(&ps.counters[u], 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            sm.last = prev == (uint32_t)(nch_spec + pm.kmax - 1);
        }
        __syncthreads();
        if (sm.last) { fused_merge<D>(ps, pm, fp, u, head0, nch_spec, tid); }
        __syncthreads();
    }
}

// Workspace counters: one chunk-arrival counter per unit (attention), then one scoring-arrival counter
// per unit (the fused selection + speculation launch), padded to 256 bytes.
size_t counters_bytes(int units) { return ((size_t)units * 8 + 255) / 256 * 256; }

// Partials kept per launch: every chunk of every unit at kChunkStep pages (no chunk is smaller).
size_t max_chunks(int units, int block, int cap) {
    const long pages = (long)cap * (block / kPage);
    return (size_t)units * (size_t)std::max<long>(1, (pages + kChunkStep - 1) / kChunkStep);
}

// Fills the kernel parameters of one speculative (repair = false) or repair launch and returns its
// grid size (workgroups).  target_wgs: workgroups to spread a full set over (default: one per CU).
int attn_setup(AttnParams &p, const KvDesc &kv, const void *q, int hq, int block, const int32_t *idx,
               const int32_t *count, const int32_t *pages, int cap, float scale, float *acc, float *l, float *m,
               float *out, bool repair, void *ws, int target_wgs = 0) {
    p.q = q;
    p.k = kv.k;
    p.v = kv.v;
    p.page_table = kv.page_table;
    p.seq_len = kv.seq_len;
    p.idx = idx;
    p.count = count;
    p.pages = pages;
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
    // Workgroups in flight: about one per CU, i.e. one wave on every SIMD, which leaves the other half of
    // each SIMD's registers to the selection kernels that run beside the speculative pass.  A full set
    // (count = cap) is spread over that many chunks, each as large as the work allows (fewer chunks
    // mean fewer partial states to merge); repair sets are usually a fraction of the capacity (the
    // missed part of a selection), so repair uses half that chunk size to keep the chip busy, and up
    // to two workgroups per CU (it runs alone, two waves per SIMD), so that every chunk of a set at full
    // capacity has a workgroup of its own instead of waiting for another chunk of the same workgroup.
    // Small sets do not fill the chip either way; there a chunk keeps at least kChunkMin pages, so that
    // each wave has both tiles of its pair in flight (8-page chunks gave a wave one tile and twice the
    // partial states to merge: at 32K, batch 1, the speculative pass took 12.9 us and repair 12.6 us
    // against 12.2 and 11.9 us with 16 pages, and at 512K paged 17.7 and 16.6 against 14.7 and 13.4 us).
    const int cus = device_cu_count();
    const long target = target_wgs > 0 ? target_wgs : cus;
    const long cap_pages = (long)cap * p.ppb;
    const long full = (long)units * cap_pages;
    auto round8 = [](long x) { return (x + kChunkStep - 1) / kChunkStep * kChunkStep; };
    long cp = std::min<long>(std::max<long>(round8((full + target - 1) / target), kChunkMin), kChunkMax);
    if (repair) cp = std::max<long>(kChunkMin, round8(cp / 2));
    p.cp = (int)cp;
    p.kmax = (int)std::max<long>(1, (cap_pages + cp - 1) / cp);
    return (int)std::min<long>((long)units * p.kmax, repair ? 2 * target : target);
}

}  // namespace
}  // namespace prr
