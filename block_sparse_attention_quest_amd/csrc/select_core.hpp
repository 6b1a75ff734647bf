// select_core.hpp - device code of GQA Quest scoring, top-K selection with M = A \ P, and the fused
// EMA level/trend predictor (gfx950), shared by the selection kernels and the fused selection +
// speculation launch.  Floating-point contraction is off for all of it: every float64 multiply and add
// below is a separately rounded IEEE operation, in the order the comments state, so scores and
// predictions are bit-identical to a plain float64 evaluation of the same formulas.
//
// Citations:
//   [paper] "Predict, Reuse, and Repair: Accelerating Dynamic Sparse Attention for Long-Context LLM
//           Decoding" (full paper text)
//   [blog]  "PRR: Predict, Reuse, and Repair - Accelerating Dynamic Sparse Attention for Long-Context
//           LLM Decoding" (xllm-io paper review)
//
// Scoring ([paper] A.1): s_p = sum_i max(qbar_i mn_{p,i}, qbar_i mx_{p,i}).  Because rounding is
// monotone, max(round(qbar mn), round(qbar mx)) = round(qbar mx) when qbar >= 0 and round(qbar mn)
// otherwise, so the kernel reads only the metadata row the sign of qbar_i selects: half the bytes of
// reading both, with identical bits.  Metadata is channel-major ([d][2][N]): a lane owns one block,
// issues one load per channel for all d channels before using any (a wave's load covers 64 consecutive
// blocks), then accumulates in channel order.
//
// Mean-pooled scoring ([paper] §2.1: selection compresses each block, e.g. by its mean): s_p = sum_i
// qbar_i mean_{p,i} over the fp32 block means ([d][N] per unit), in channel order, one block per lane.
//
// Top-K ([paper] §1, §2.1; ties to the smaller block index): one workgroup per (sequence, kv head) keeps
// all N keys in registers (order-preserving 64-bit images of the fp64 scores; 256 threads with up to 8
// contiguous keys each up to 2048 keys) and runs an MSD radix select with 8-bit digits: per pass the
// candidates' digits are counted in an LDS histogram, one barrier completes it, and every wave finds the
// boundary digit from the 256 counts with a DPP prefix sum over its lanes and one ballot.  Leading bits
// shared by every key are skipped, and the search stops as soon as the boundary digit's bucket is taken
// whole.  Ties on the full key go to the smaller index through a prefix sum over the threads'
// contiguous index ranges, which also yields the ascending output positions directly.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "prr_internal.hpp"

#pragma clang fp contract(off)

namespace prr {
namespace {

constexpr int kTopkKeysPerThread = 32;   // upper bound on keys held per thread by the top-K kernels

__device__ __forceinline__ double dadd(double a, double b) {
#pragma clang fp contract(off)
    return a + b;
}
__device__ __forceinline__ double dmul(double a, double b) {
#pragma clang fp contract(off)
    return a * b;
}
__device__ __forceinline__ double dsub(double a, double b) {
#pragma clang fp contract(off)
    return a - b;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Order-preserving image of a double (larger double -> larger key); -0.0 maps with +0.0.
__device__ __forceinline__ uint64_t order_key(double x) {
    uint64_t b = (uint64_t)__double_as_longlong(x);
    if (b == 0x8000000000000000ull) b = 0;
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int o) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o);
    return ((uint64_t)hi << 32) | lo;
}

template <int W>
struct __align__(16) TopkSmem {
    uint32_t hist[3][256];       // digit counts of three consecutive passes (each cleared a pass ahead)
    uint64_t andor[W][2];
    uint32_t scan[2][W];
};

// Reductions over the 64 lanes of a wave with DPP row operations (quad swaps, half-row and row
// mirrors, then the row-15 and row-31 broadcasts); the result is complete in lane 63 only.
__device__ __forceinline__ uint32_t dpp_sum63(uint32_t x) {
    x += __builtin_amdgcn_update_dpp(0u, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    x += __builtin_amdgcn_update_dpp(0u, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    x += __builtin_amdgcn_update_dpp(0u, x, 0x141, 0xF, 0xF, false);  // row_half_mirror
    x += __builtin_amdgcn_update_dpp(0u, x, 0x140, 0xF, 0xF, false);  // row_mirror
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);  // row_bcast15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);  // row_bcast31 into rows 2, 3
    return x;
}
__device__ __forceinline__ uint32_t dpp_and63(uint32_t x) {
    x &= __builtin_amdgcn_update_dpp(~0u, x, 0xB1, 0xF, 0xF, false);
    x &= __builtin_amdgcn_update_dpp(~0u, x, 0x4E, 0xF, 0xF, false);
    x &= __builtin_amdgcn_update_dpp(~0u, x, 0x141, 0xF, 0xF, false);
    x &= __builtin_amdgcn_update_dpp(~0u, x, 0x140, 0xF, 0xF, false);
    x &= __builtin_amdgcn_update_dpp(~0u, x, 0x142, 0xA, 0xF, false);
    x &= __builtin_amdgcn_update_dpp(~0u, x, 0x143, 0xC, 0xF, false);
    return x;
}
__device__ __forceinline__ uint32_t dpp_or63(uint32_t x) {
    x |= __builtin_amdgcn_update_dpp(0u, x, 0xB1, 0xF, 0xF, false);
    x |= __builtin_amdgcn_update_dpp(0u, x, 0x4E, 0xF, 0xF, false);
    x |= __builtin_amdgcn_update_dpp(0u, x, 0x141, 0xF, 0xF, false);
    x |= __builtin_amdgcn_update_dpp(0u, x, 0x140, 0xF, 0xF, false);
    x |= __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);
    x |= __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);
    return x;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: row shifts by 1, 2, 4 and 8 scan each
// 16-lane row, then the row-15 broadcast adds row 0's total to row 1 and row 2's to row 3, and the row-31
// broadcast adds the total of rows 0 and 1 to rows 2 and 3.
__device__ __forceinline__ uint32_t dpp_incl_scan(uint32_t x) {
    x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xA, 0xF, false);  // row_bcast15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xC, 0xF, false);  // row_bcast31 into rows 2, 3
    return x;
}

// Exclusive prefix sum over the workgroup (W waves) in thread order; `total` gets the sum.  `buf` selects
// one of two LDS slots so back-to-back scans need a single barrier each.  A one-wave workgroup scans in
// registers only.
template <int W>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, TopkSmem<W> &sm, int buf, uint32_t &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t v = dpp_incl_scan(x);
    if constexpr (W == 1) {
        total = __builtin_amdgcn_readlane(v, 63);
        return v - x;
    } else {
        if (lane == 63) sm.scan[buf][wave] = v;
        __syncthreads();
        uint32_t before = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const uint32_t sw = sm.scan[buf][w];
            tot += sw;
            before += w < wave ? sw : 0u;
        }
        total = tot;
        return before + v - x;
    }
}

__device__ __forceinline__ uint64_t mask_from(int shift) {   // bits >= shift
    return shift >= 64 ? 0ull : ~((1ull << shift) - 1ull);
}

// Select the k largest keys (key descending, index ascending) among the n valid ones.  Thread t owns
// indices [t*KPT, t*KPT + KPT).  Returns a bitmask over the thread's KPT keys.
//
// A radix select over 8-bit digits, from the highest bit in which the valid keys differ: each pass
// counts the candidates' digits in an LDS histogram (LDS atomics), every wave finds the boundary digit
// from the 256 counts (a lane per 4 digits, a prefix sum over the lanes), and the candidates narrow to
// that digit; it stops once the boundary digit's keys are all taken.  Three histograms rotate, so that
// the one a pass fills was cleared during the pass before and a pass needs one barrier.  Keys equal to
// the boundary on all 64 bits are taken in index order.  (Against 4-bit digits counted in registers:
// 2-3 passes instead of 4-5; one workgroup: 1.8 against 4.3 us for 512 keys, 3.0 against 5.7 us for
// 2048, 8.4 against 13.6 us for 8192.)
template <int KPT, int W>
__device__ uint32_t block_topk(const uint64_t (&key)[KPT], int n, int k, TopkSmem<W> &sm) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int base = threadIdx.x * KPT;
    uint32_t valid = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        if (base + j < n) valid |= 1u << j;
    if (k <= 0) return 0u;
    if (k >= n) return valid;
    for (int i = threadIdx.x; i < 256; i += 64 * W) {
        sm.hist[0][i] = 0u;
        sm.hist[1][i] = 0u;
    }

    // common leading bits of all valid keys
    uint64_t a = ~0ull, o = 0ull;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        if (valid >> j & 1u) {
            a &= key[j];
            o |= key[j];
        }
    {
        const uint32_t alo = __builtin_amdgcn_readlane(dpp_and63((uint32_t)a), 63);
        const uint32_t ahi = __builtin_amdgcn_readlane(dpp_and63((uint32_t)(a >> 32)), 63);
        const uint32_t olo = __builtin_amdgcn_readlane(dpp_or63((uint32_t)o), 63);
        const uint32_t ohi = __builtin_amdgcn_readlane(dpp_or63((uint32_t)(o >> 32)), 63);
        a = ((uint64_t)ahi << 32) | alo;
        o = ((uint64_t)ohi << 32) | olo;
    }
    if constexpr (W > 1) {
        if (lane == 0) {
            sm.andor[wave][0] = a;
            sm.andor[wave][1] = o;
        }
        __syncthreads();   // also orders the histogram clears before the first pass
        a = ~0ull;
        o = 0ull;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            a &= sm.andor[w][0];
            o |= sm.andor[w][1];
        }
    } else {
        __builtin_amdgcn_wave_barrier();
    }
    const uint64_t diff = a ^ o;

    uint64_t prefix, mask;
    int remaining = k;
    bool take_all = false;
    if (diff == 0) {
        prefix = a;          // every key equal: pure tie break by index
        mask = ~0ull;
    } else {
        const int top = 63 - __clzll((long long)diff);
        int shift = (top / 8) * 8;
        mask = mask_from(shift + 8);
        prefix = a & mask;
        for (int pass = 0; shift >= 0; shift -= 8, ++pass) {
            const int buf = pass % 3;
#pragma unroll
            for (int j = 0; j < KPT; ++j)
                if ((valid >> j & 1u) && (key[j] & mask) == prefix)
                    __hip_atomic_fetch_add(&sm.hist[buf][(uint32_t)(key[j] >> shift) & 255u], 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
            // the histogram of the next pass: its last reader was the pass before this one
            for (int i = threadIdx.x; i < 256; i += 64 * W) sm.hist[(pass + 1) % 3][i] = 0u;
            if constexpr (W > 1) __syncthreads();
            else __builtin_amdgcn_wave_barrier();
            // lane l: digits 4l .. 4l + 3 and S = the count of digits >= 4l; the boundary digit is the
            // largest d whose suffix count reaches `remaining` (the suffix counts fall as d grows)
            const uint4 c = *(const uint4 *)&sm.hist[buf][4 * lane];
            const uint32_t s4 = c.x + c.y + c.z + c.w;
            const uint32_t incl = dpp_incl_scan(s4);
            const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
            const uint32_t S0 = total - (incl - s4);
            const uint32_t S3 = S0 - c.x - c.y - c.z, S2 = S3 + c.z, S1 = S2 + c.y;
            const uint32_t rem = (uint32_t)remaining;
            const uint64_t ge = __ballot(S0 >= rem);
            const int L = 63 - __clzll((long long)ge);
            const int i = S3 >= rem ? 3 : S2 >= rem ? 2 : S1 >= rem ? 1 : 0;
            const uint32_t ci = i == 3 ? c.w : i == 2 ? c.z : i == 1 ? c.y : c.x;
            const uint32_t si = i == 3 ? S3 : i == 2 ? S2 : i == 1 ? S1 : S0;
            const int dsel = 4 * L + __builtin_amdgcn_readlane(i, L);
            const uint32_t csel = (uint32_t)__builtin_amdgcn_readlane((int)ci, L);
            const uint32_t cum = (uint32_t)__builtin_amdgcn_readlane((int)si, L) - csel;
            remaining -= (int)cum;
            prefix |= (uint64_t)dsel << shift;
            mask |= 255ull << shift;
            if (csel == (uint32_t)remaining) {
                take_all = true;
                break;
            }
        }
    }

    uint32_t sel = 0, tie = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        if (!(valid >> j & 1u)) continue;
        const uint64_t mk = key[j] & mask;
        if (mk > prefix) sel |= 1u << j;
        else if (mk == prefix) tie |= 1u << j;
    }
    if (take_all) return sel | tie;
    // ties on the full key: the `remaining` smallest indices win
    uint32_t total;
    const uint32_t before = block_excl_scan(__popc(tie), sm, 0, total);
    uint32_t r = before;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        if (tie >> j & 1u) {
            if (r < (uint32_t)remaining) sel |= 1u << j;
            ++r;
        }
    return sel;
}

// ------------------------------------------------------------------------------------------------
// Scoring
// ------------------------------------------------------------------------------------------------

struct ScoreParams {
    const void *q;
    const void *meta;
    const int32_t *seq_len;
    double *scores;
    int hq, hkv, G, block, stride, nmax;
};

// Blocks per lane of the scoring workgroups: two for bf16 min/max metadata (one 4-byte load per channel
// covers both) and for the fp32 block means of mean-pooled scoring (one 8-byte load per channel, in two
// halves of the channels), one for fp32 min/max.  prr_select's score kernel, which has the chip to
// itself, takes one bf16 min/max block per lane (a 2-byte load per channel) for twice the waves.
template <bool BF16, bool MEAN = false>
constexpr int kScoreBPL = (BF16 || MEAN) ? 2 : 1;

// Rows of at least this many blocks (512K tokens at block 16) score bf16 min/max metadata four blocks per
// lane (one 8-byte load per channel) when their top-K takes three stages either way: half as many
// scoring workgroups, so that the scoring grid of a long row leaves room for the rest of a fused launch
// (or is resident at all).  Rows that fill the chip at two blocks per lane lose by it (fewer workgroups
// for the same bytes), so shorter rows keep two.
constexpr int kWideScoreBlocks = 32768;
constexpr int kWideScoreBPL = 4;
// ... and so do rows whose 512-block parts would number more than this over all units (one per CU of
// the MI355X) in a fused launch, where the scoring grid would otherwise take the speculative pass's slots.
constexpr long kWideScoreParts = 256;

// Blocks per scoring workgroup (256 lanes of kScoreBPL blocks, or kWideScoreBPL), on the host.
constexpr int score_bpw(bool bq, bool mean, bool wide = false) {
    return 256 * (wide ? kWideScoreBPL : (bq || mean) ? 2 : 1);
}

// Scores blocks [256 BPL bx, 256 BPL (bx + 1)) of unit u (BPL consecutive blocks per lane).  COHERENT:
// the scores are stored with device-scope stores, for a reader on another XCD within the same launch.
// BPL: kScoreBPL, or kWideScoreBPL for bf16 min/max metadata.
template <bool BF16, int D, bool COHERENT = false, bool MEAN = false, int BPL = kScoreBPL<BF16, MEAN>>
__device__ __forceinline__ void score_body(const ScoreParams &p, int bx, int u, double (&kept)[BPL]) {
    static_assert(BPL == kScoreBPL<BF16, MEAN> || (BF16 && !MEAN && (BPL == kWideScoreBPL || BPL == 1)),
                  "one or four blocks per lane: bf16 min/max metadata only");
    __shared__ double s_qbar[D];
    __shared__ int s_row[D];             // metadata row of channel i: 1 (max) when qbar_i >= 0, else 0 (min)
    const int b = u / p.hkv, kvh = u - b * p.hkv;
    const int slen_raw = p.seq_len[b];   // in flight with the query loads
    if (threadIdx.x < D) {
        // qbar_i = (sum_{g=0}^{G-1} q_{kvh G + g, i}) / G, summed in order from +0.0
        double acc = 0.0;
        for (int gq = 0; gq < p.G; ++gq) {
            const size_t off = ((size_t)b * p.hq + (size_t)kvh * p.G + gq) * D + threadIdx.x;
            const double x = BF16 ? (double)bf16_to_f32(((const uint16_t *)p.q)[off])
                                  : (double)((const float *)p.q)[off];
            acc = dadd(acc, x);
        }
        const double qb = acc / (double)p.G;
        s_qbar[threadIdx.x] = qb;
        s_row[threadIdx.x] = qb >= 0.0 ? 1 : 0;
    }
    __syncthreads();
    const int slen = max(slen_raw, 0);
    const int nb = min((slen + p.block - 1) / p.block, p.nmax);
    const int p0 = (bx * 256 + threadIdx.x) * BPL;
    if (p0 >= nb) return;
    // every channel's load is issued before the first is used: one memory round trip per thread.  The
    // row (min or max) depends on the sign of qbar_i only, so the row address is wave-uniform (scalar)
    // and each lane adds its own block offset.
    // Buffer loads: the unit's metadata is one buffer resource (scalar base), the row offset a scalar
    // and the lane's block offset the only vector operand, shared by all d loads.
    // Mean-pooled scoring: one fp32 row (the block means) per channel, [d][stride].
    constexpr int ES = (BF16 && !MEAN) ? 2 : 4;   // element size
    constexpr int ROWS = MEAN ? 1 : 2;            // rows per channel
    const char *ubase = (const char *)p.meta + (size_t)u * D * ROWS * p.stride * ES;
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void *)ubase, (short)0, D * ROWS * p.stride * ES, 0x00020000);
    const int voff = p0 * ES;
    double acc[BPL];
#pragma unroll
    for (int e = 0; e < BPL; ++e) acc[e] = 0.0;
    if constexpr (MEAN) {
        // blocks p0 and p0 + 1 of one channel are adjacent fp32 values (8-byte aligned: p0 and the row
        // stride are even).  Channels are taken in two halves, each loaded before it is used, so that the
        // loaded pairs take D registers like the other layouts.
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            uint32_t lo[D / 2], hi[D / 2];
#pragma unroll
            for (int j = 0; j < D / 2; ++j) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff, (half * D / 2 + j) * p.stride * ES, 0);
                lo[j] = v[0];
                hi[j] = v[1];
            }
#pragma unroll
            for (int j = 0; j < D / 2; ++j) {
                const double qb = s_qbar[half * D / 2 + j];
                acc[0] = dadd(acc[0], dmul(qb, (double)__uint_as_float(lo[j])));
                acc[1] = dadd(acc[1], dmul(qb, (double)__uint_as_float(hi[j])));
                asm volatile("" : "+v"(acc[0]), "+v"(acc[1]));
                if (j % 16 == 15) __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else if constexpr (BPL == kWideScoreBPL) {
        // bf16 min/max, four blocks per lane: blocks p0 .. p0 + 3 of one row are 8 adjacent bytes (8-byte
        // aligned: p0 is a multiple of 4 and the row stride of 8).  Channels in two halves, each loaded
        // before it is used, so that the loaded words take D registers as in the other layouts.
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            uint32_t lo[D / 2], hi[D / 2];
#pragma unroll
            for (int j = 0; j < D / 2; ++j) {
                const int i = half * D / 2 + j;
                const int sgn = __builtin_amdgcn_readfirstlane(s_row[i]);
                const auto v = __builtin_amdgcn_raw_buffer_load_b64(rsrc, voff, (2 * i + sgn) * p.stride * ES, 0);
                lo[j] = v[0];
                hi[j] = v[1];
            }
#pragma unroll
            for (int j = 0; j < D / 2; ++j) {
                const double qb = s_qbar[half * D / 2 + j];
#pragma unroll
                for (int e = 0; e < BPL; ++e) {
                    const uint32_t w = e < 2 ? lo[j] : hi[j];
                    acc[e] = dadd(acc[e], dmul(qb, (double)bf16_to_f32((uint16_t)(w >> (16 * (e & 1))))));
                }
                asm volatile("" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
                if (j % 16 == 15) __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else {
        uint32_t raw[D];
#pragma unroll
        for (int i = 0; i < D; ++i) {
            // qbar >= 0: the max term is qbar * mx (row 1); otherwise qbar * mn (row 0).  bf16: the 4 bytes
            // hold blocks p0 and p0 + 1; fp32: block p0.
            const int sgn = __builtin_amdgcn_readfirstlane(s_row[i]);
            if constexpr (BF16 && BPL == 1)   // one bf16 block per lane: a 2-byte load
                raw[i] = (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rsrc, voff, (2 * i + sgn) * p.stride * ES, 0);
            else
                raw[i] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsrc, voff, (2 * i + sgn) * p.stride * ES, 0);
        }
#pragma unroll
        for (int i = 0; i < D; ++i) {
            // the accumulation is a sequential chain; a scheduling barrier every 16 channels lets the qbar
            // reads run at most 16 channels ahead (hoisting all of them would hold 2 D doubles in registers)
            const uint32_t r = raw[i];
            const double qb = s_qbar[i];
#pragma unroll
            for (int e = 0; e < BPL; ++e) {
                const double x = BF16 ? (double)bf16_to_f32((uint16_t)(r >> (16 * e))) : (double)__uint_as_float(r);
                acc[e] = dadd(acc[e], dmul(qb, x));
            }
            // the chains of a lane's blocks advance together, channel by channel (otherwise the compiler
            // runs one chain to the end first and parks the other's operands in spare registers)
            if constexpr (BPL == 2) asm volatile("" : "+v"(acc[0]), "+v"(acc[1]));
            if (i % 16 == 15) __builtin_amdgcn_sched_barrier(0);
        }
    }
    double *out = p.scores + (size_t)u * p.nmax;
#pragma unroll
    for (int e = 0; e < BPL; ++e) kept[e] = acc[e];
#pragma unroll
    for (int e = 0; e < BPL; ++e)
        if (p0 + e < nb) {
            if constexpr (COHERENT)
                __hip_atomic_store(&out[p0 + e], acc[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                out[p0 + e] = acc[e];
        }
}

// The same without handing the scores back.
template <bool BF16, int D, bool COHERENT = false, bool MEAN = false>
__device__ __forceinline__ void score_body(const ScoreParams &p, int bx, int u) {
    double kept[kScoreBPL<BF16, MEAN>];
    score_body<BF16, D, COHERENT, MEAN>(p, bx, u, kept);
}

// ------------------------------------------------------------------------------------------------
// Top-K + set difference
// ------------------------------------------------------------------------------------------------

__device__ __forceinline__ void st_dev_u64(uint64_t *ptr, uint64_t v) {
    __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev_i32(int32_t *ptr, int32_t v) {
    __hip_atomic_store(ptr, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct TopkParams {
    const double *scores;
    const int32_t *seq_len;
    const int32_t *p_idx;
    const int32_t *p_cnt;
    int32_t *a_idx;
    int32_t *a_cnt;
    int32_t *m_idx;
    int32_t *m_cnt;
    int hkv, block, nmax, topk, p_cap, a_cap, m_cap;
    // page work lists of A and M (each may be null): [units][cap ppb] physical page ids (set_pages)
    int32_t *a_pages;
    int32_t *m_pages;
    const int32_t *page_table;   // [batch][max_pages]
    int max_pages;
};

// M's entries and count: device-scope stores when a workgroup of the same launch reads them (COH_M).
template <bool COH_M>
__device__ __forceinline__ void st_m(int32_t *ptr, int32_t v) {
    if constexpr (COH_M) st_dev_i32(ptr, v);
    else *ptr = v;
}

// Page work lists (the physical pages of a set, for the attention passes that read the set): slot
// e ppb + s of unit u's list holds the physical page of page s of the set's entry e (logical page
// idx[e] ppb + s), or -1 where that page holds no token yet.  A page is mapped once a token is written to
// it and keeps its mapping, so a list written for a sequence stays valid while the sequence grows; the
// readers look up -1 slots whose page has tokens by then.  The entries go through LDS in stages of
// kPageStage, and the workgroup's threads then fill the slots together, four page-table loads per thread
// in flight: one memory round trip per 4 TPB slots.
constexpr int kPageStage = 1024;

// Written by the workgroup that ranked the set: thread t's selected candidates (bits over its KPT
// candidates, block ids blk) take output positions pos0, pos0 + 1, ... in candidate order; count = the
// set size (workgroup-uniform).  COH: device-scope stores (a reader in the same launch).
template <int KPT, int TPB, bool COH>
__device__ __forceinline__ void write_set_pages(int32_t *list, const int32_t *page_table, int max_pages, int ppb,
                                                int b, int slen, uint32_t bits, uint32_t pos0,
                                                const int (&blk)[KPT], int count, int32_t *s_ent) {
    for (int c0 = 0; c0 < count; c0 += kPageStage) {
        __syncthreads();   // the stage is free
        uint32_t pos = pos0;
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            if (bits >> j & 1u) {
                const int r = (int)pos - c0;
                if (r >= 0 && r < kPageStage) s_ent[r] = blk[j];
                ++pos;
            }
        __syncthreads();
        const int n = min(count - c0, kPageStage) * ppb;
        for (int i0 = threadIdx.x; i0 < n; i0 += 4 * TPB) {
            int32_t ph[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = i0 + r * TPB;
                ph[r] = -1;
                if (i < n) {
                    const int e = i / ppb;
                    const long lp = (long)s_ent[e] * ppb + (i - e * ppb);
                    if (lp < max_pages && lp * kPage < slen) ph[r] = page_table[(size_t)b * max_pages + lp];
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = i0 + r * TPB;
                if (i < n) st_m<COH>(&list[(size_t)c0 * ppb + i], ph[r]);
            }
        }
    }
}

// Top-K of unit u's scores and M = A \ P, by a workgroup of TPB threads holding KPT keys each.
// COHERENT: the scores are read with device-scope loads (written by other workgroups of the same launch).
// COH_M: M is stored with device-scope stores (read by other workgroups of the same launch).
template <int KPT, int TPB, bool COHERENT = false, bool COH_M = false>
__device__ __forceinline__ void topk_body(const TopkParams &p, int u) {
    constexpr int W = TPB / 64;
    __shared__ TopkSmem<W> sm;
    __shared__ uint32_t s_pbits[TPB * KPT / 32];
    const int b = u / p.hkv;
    const bool want_m = p.m_idx != nullptr;
    // Every load goes out at once (one memory round trip): the length, P's count, the whole score row
    // and P's first TPB entries, none waiting for another; the row past the unit's block count and P
    // past its count are masked afterwards.
    const int slen = p.seq_len[b];
    const int pcnt = want_m ? p.p_cnt[u] : 0;
    uint64_t key[KPT];
    const int base = threadIdx.x * KPT;
    const double *row = p.scores + (size_t)u * p.nmax;
    double sv[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        if constexpr (COHERENT)
            sv[j] = base + j < p.nmax ? __hip_atomic_load(&row[base + j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                      : 0.0;
        else
            sv[j] = base + j < p.nmax ? row[base + j] : 0.0;
    }
    const int x0 = want_m && (int)threadIdx.x < p.p_cap ? p.p_idx[(size_t)u * p.p_cap + threadIdx.x] : -1;
    const int nb = min((slen + p.block - 1) / p.block, p.nmax);
    if (want_m) {
        for (int i = threadIdx.x; i < TPB * KPT / 32; i += TPB) s_pbits[i] = 0u;
        __syncthreads();
        const int pc = min(max(pcnt, 0), p.p_cap);
        if ((int)threadIdx.x < pc && x0 >= 0 && x0 < nb) atomicOr(&s_pbits[x0 >> 5], 1u << (x0 & 31));
        for (int i = threadIdx.x + TPB; i < pc; i += TPB) {
            const int x = p.p_idx[(size_t)u * p.p_cap + i];
            if (x >= 0 && x < nb) atomicOr(&s_pbits[x >> 5], 1u << (x & 31));
        }
    }
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = base + j < nb ? order_key(sv[j]) : 0ull;
    const uint32_t sel = block_topk<KPT, W>(key, nb, p.topk, sm);
    __syncthreads();   // P bitmap complete (and top-K scratch released)
    uint32_t inm = 0;
    if (want_m) {
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            if ((sel >> j & 1u) && !(s_pbits[(base + j) >> 5] >> ((base + j) & 31) & 1u)) inm |= 1u << j;
    }
    uint32_t total;
    const uint32_t off = block_excl_scan((uint32_t)__popc(sel) | ((uint32_t)__popc(inm) << 16), sm, 1, total);
    uint32_t oa = off & 0xffffu, om = off >> 16;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        if (sel >> j & 1u) p.a_idx[(size_t)u * p.a_cap + oa++] = base + j;
        if (inm >> j & 1u) st_m<COH_M>(&p.m_idx[(size_t)u * p.m_cap + om++], base + j);
    }
    if (threadIdx.x == 0) {
        p.a_cnt[u] = (int32_t)(total & 0xffffu);
        if (want_m) st_m<COH_M>(&p.m_cnt[u], (int32_t)(total >> 16));
    }
    if (p.a_pages || (want_m && p.m_pages)) {
        __shared__ int32_t s_ent[kPageStage];
        int blk[KPT];
#pragma unroll
        for (int j = 0; j < KPT; ++j) blk[j] = base + j;
        const int ppb = p.block / kPage;
        if (p.a_pages)
            write_set_pages<KPT, TPB, false>(p.a_pages + (size_t)u * p.a_cap * ppb, p.page_table, p.max_pages, ppb, b,
                                             slen, sel, off & 0xffffu, blk, (int)(total & 0xffffu), s_ent);
        if (want_m && p.m_pages)
            write_set_pages<KPT, TPB, COH_M>(p.m_pages + (size_t)u * p.m_cap * ppb, p.page_table, p.max_pages, ppb,
                                             b, slen, inm, off >> 16, blk, (int)(total >> 16), s_ent);
    }
}

// ---- two-stage top-K for long rows ----
//
// The K largest keys of a row are among the union of the K largest of every part of it (a key beaten by
// fewer than K keys of the whole row is beaten by fewer than K of its part), so a row too long for one
// workgroup's registers is ranked in two stages: each scoring workgroup keeps the local top-kl (kl =
// min(K, its block count)) of its own blocks as candidates (order key, block index), in ascending block
// order; the unit's last workgroup ranks the candidates of all parts.  Candidate positions then follow
// the block order, so ties still go to the smaller block index.

constexpr int kMaxTwoStageBlocks = 32768;   // P bitmap of the final candidate ranking (LDS)

// Candidate slots of a two-stage top-K: [units][parts][kl] order keys and block indices, [units][parts]
// counts (device memory of the caller's workspace).
struct CandParams {
    uint64_t *key;
    int32_t *idx;
    int32_t *cnt;
    int kl;
};

// The middle and final stages of a three-stage top-K inside a fused launch: the group candidates (c2:
// [units][ng][kl2]), one part-arrival counter per (unit, group) and one group-arrival counter per unit
// (zero at rest; the last arriver resets its counter), groups of gp parts.
struct GroupParams {
    CandParams c2;
    uint32_t *part_arr;    // [units][ng]
    uint32_t *group_arr;   // [units]
    int gp, ng;
};

// Stage 1: the local top-kl of the workgroup's blocks [first_block, first_block + 256 BPL) (lane t holds
// blocks first_block + BPL t + e with scores kept[e]); n_local of them exist.  Writes the candidates and
// their count with device-scope stores.
template <int BPL>
__device__ __forceinline__ void local_candidates(const double (&kept)[BPL], int n_local, int kl, int first_block,
                                                 uint64_t *ckey, int32_t *cidx, int32_t *ccnt, TopkSmem<4> &sm) {
    uint64_t key[BPL];
    const int base = threadIdx.x * BPL;
#pragma unroll
    for (int e = 0; e < BPL; ++e) key[e] = base + e < n_local ? order_key(kept[e]) : 0ull;
    const uint32_t sel = block_topk<BPL, 4>(key, n_local, kl, sm);
    __syncthreads();   // top-K scratch released
    uint32_t total;
    uint32_t off = block_excl_scan((uint32_t)__popc(sel), sm, 1, total);
#pragma unroll
    for (int e = 0; e < BPL; ++e)
        if (sel >> e & 1u) {
            st_dev_u64(&ckey[off], key[e]);
            st_dev_i32(&cidx[off], first_block + base + e);
            ++off;
        }
    if (threadIdx.x == 0) st_dev_i32(ccnt, (int32_t)total);
}

// Middle stage of a three-stage top-K (rows with more candidate slots than one ranking holds): the top
// kout of the candidate slots of gparts consecutive parts (part c holds ccnt[c] of its kl slots), 256
// threads with KPT slots each (256 KPT >= gparts kl), written as the candidates of one group in slot
// order, with device-scope stores.  Slot order is block order, so ties still go to the smaller index,
// and the selection stays exact: a block beaten by fewer than K blocks of the row is beaten by fewer
// than K of its group's candidates.
template <int KPT>
__device__ __forceinline__ void group_candidates(const uint64_t *ckey, const int32_t *cidx, const int32_t *ccnt,
                                                 int gparts, int kl, int kout, uint64_t *okey, int32_t *oidx,
                                                 int32_t *ocnt) {
    constexpr int TPB = 256, W = 4;
    __shared__ TopkSmem<W> sm;
    __shared__ int s_cnt[TPB];
    __shared__ int s_total;
    const int my_cnt = (int)threadIdx.x < gparts
                           ? __hip_atomic_load(&ccnt[threadIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
    const int base = threadIdx.x * KPT;
    const int nslots = gparts * kl;
    uint64_t key[KPT];
    int32_t idx[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int pos = base + j;
        key[j] = pos < nslots ? __hip_atomic_load(&ckey[pos], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
        idx[j] = pos < nslots ? __hip_atomic_load(&cidx[pos], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
    }
    if ((int)threadIdx.x < gparts) s_cnt[threadIdx.x] = my_cnt;
    __syncthreads();
    if (threadIdx.x == 0) {
        int t = 0;
        for (int c = 0; c < gparts; ++c) t += s_cnt[c];
        s_total = t;
    }
    uint32_t valid = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int pos = base + j;
        const int c = pos / kl, slot = pos - c * kl;
        if (c < gparts && slot < s_cnt[min(c, gparts - 1)]) valid |= 1u << j;
        else key[j] = 0ull;
    }
    __syncthreads();   // s_total
    // valid candidate keys are images of finite scores, all above the padding key 0
    const uint32_t sel = s_total <= kout ? valid : block_topk<KPT, W>(key, nslots, kout, sm) & valid;
    __syncthreads();
    uint32_t total;
    uint32_t off = block_excl_scan((uint32_t)__popc(sel), sm, 1, total);
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        if (sel >> j & 1u) {
            st_dev_u64(&okey[off], key[j]);
            st_dev_i32(&oidx[off], idx[j]);
            ++off;
        }
    if (threadIdx.x == 0) st_dev_i32(ocnt, (int32_t)total);
}

// Stage 2: the top-K of unit u over its nparts x kl candidate slots (part c holds ccnt[c] candidates)
// and M = A \ P, written like topk_body.  256 threads with KPT slots each (256 KPT >= nparts kl).
// NBITS: the longest row (in blocks) whose P bitmap the workgroup holds in LDS.
template <int KPT, bool COH_M = false, int NBITS = kMaxTwoStageBlocks>
__device__ __forceinline__ void topk_candidates_body(const TopkParams &p, int u, const uint64_t *ckey,
                                                     const int32_t *cidx, const int32_t *ccnt, int nparts,
                                                     int kl) {
    constexpr int TPB = 256, W = 4;
    __shared__ TopkSmem<W> sm;
    __shared__ uint32_t s_pbits[NBITS / 32];
    __shared__ int s_cnt[TPB];
    __shared__ int s_total;
    const int b = u / p.hkv;
    const bool want_m = p.m_idx != nullptr;
    // Every load goes out at once, as in topk_body: the length, P's count, the part counts, every
    // candidate slot and P's first TPB entries; slots past their part's count are masked afterwards.
    const int slen = p.seq_len[b];
    const int pcnt = want_m ? p.p_cnt[u] : 0;
    const int my_cnt = (int)threadIdx.x < nparts
                           ? __hip_atomic_load(&ccnt[threadIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
    const int base = threadIdx.x * KPT;
    const int nslots = nparts * kl;
    uint64_t key[KPT];
    int32_t idx[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int pos = base + j;
        key[j] = pos < nslots ? __hip_atomic_load(&ckey[pos], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0ull;
        idx[j] = pos < nslots ? __hip_atomic_load(&cidx[pos], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
    }
    const int x0 = want_m && (int)threadIdx.x < p.p_cap ? p.p_idx[(size_t)u * p.p_cap + threadIdx.x] : -1;
    const int nb = min((slen + p.block - 1) / p.block, p.nmax);
    if ((int)threadIdx.x < nparts) s_cnt[threadIdx.x] = my_cnt;
    if (want_m)
        for (int i = threadIdx.x; i < (nb + 31) / 32; i += TPB) s_pbits[i] = 0u;
    __syncthreads();
    if (threadIdx.x == 0) {
        int t = 0;
        for (int c = 0; c < nparts; ++c) t += s_cnt[c];
        s_total = t;
    }
    uint32_t valid = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int pos = base + j;
        const int c = pos / kl, slot = pos - c * kl;
        if (c < nparts && slot < s_cnt[min(c, nparts - 1)]) valid |= 1u << j;
        else key[j] = 0ull;
    }
    if (want_m) {
        const int pc = min(max(pcnt, 0), p.p_cap);
        if ((int)threadIdx.x < pc && x0 >= 0 && x0 < nb) atomicOr(&s_pbits[x0 >> 5], 1u << (x0 & 31));
        for (int i = threadIdx.x + TPB; i < pc; i += TPB) {
            const int x = p.p_idx[(size_t)u * p.p_cap + i];
            if (x >= 0 && x < nb) atomicOr(&s_pbits[x >> 5], 1u << (x & 31));
        }
    }
    __syncthreads();   // counts total, P bitmap complete
    // valid candidate keys are images of finite scores, all above the padding key 0
    const uint32_t sel = s_total <= p.topk ? valid : block_topk<KPT, W>(key, nparts * kl, p.topk, sm) & valid;
    __syncthreads();
    uint32_t inm = 0;
    if (want_m) {
#pragma unroll
        for (int j = 0; j < KPT; ++j)
            if ((sel >> j & 1u) && !(s_pbits[idx[j] >> 5] >> (idx[j] & 31) & 1u)) inm |= 1u << j;
    }
    uint32_t total;
    const uint32_t off = block_excl_scan((uint32_t)__popc(sel) | ((uint32_t)__popc(inm) << 16), sm, 1, total);
    uint32_t oa = off & 0xffffu, om = off >> 16;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        if (sel >> j & 1u) p.a_idx[(size_t)u * p.a_cap + oa++] = idx[j];
        if (inm >> j & 1u) st_m<COH_M>(&p.m_idx[(size_t)u * p.m_cap + om++], idx[j]);
    }
    if (threadIdx.x == 0) {
        p.a_cnt[u] = (int32_t)(total & 0xffffu);
        if (want_m) st_m<COH_M>(&p.m_cnt[u], (int32_t)(total >> 16));
    }
    if (p.a_pages || (want_m && p.m_pages)) {
        __shared__ int32_t s_ent[kPageStage];
        const int ppb = p.block / kPage;
        if (p.a_pages)
            write_set_pages<KPT, TPB, false>(p.a_pages + (size_t)u * p.a_cap * ppb, p.page_table, p.max_pages, ppb, b,
                                             slen, sel, off & 0xffffu, idx, (int)(total & 0xffffu), s_ent);
        if (want_m && p.m_pages)
            write_set_pages<KPT, TPB, COH_M>(p.m_pages + (size_t)u * p.m_cap * ppb, p.page_table, p.max_pages, ppb,
                                             b, slen, inm, off >> 16, idx, (int)(total >> 16), s_ent);
    }
}

// ------------------------------------------------------------------------------------------------
// EMA update + prediction + top-|P|
// ------------------------------------------------------------------------------------------------

struct PredictParams {
    const double *scores;
    const int32_t *seq_len;
    double *level;
    double *trend;
    int32_t *live;
    int32_t *p_idx;
    int32_t *p_cnt;
    int hkv, block, nmax, budget, p_cap;
    double alpha, beta, gamma;
    int32_t *p_pages;            // P's page work list (may be null), as TopkParams' lists
    const int32_t *page_table;
    int max_pages;
};

// EMA update, prediction and top-|P| of unit u, by a workgroup of TPB threads holding KPT keys each.
template <int KPT, int TPB>
__device__ __forceinline__ void predict_body(const PredictParams &p, int u) {
    constexpr int W = TPB / 64;
    __shared__ TopkSmem<W> sm;
    const int b = u / p.hkv;
    // Up to 16 keys per thread every load goes out at once (one memory round trip): the length, the live
    // count and the row's scores and state over all max_blocks columns; columns past the unit's block
    // count are not used.  With 32 keys per thread the state would not fit in registers: the loads then
    // wait for the length and cover the unit's blocks only.
    constexpr bool PREFETCH = KPT <= 16;
    const int slen = p.seq_len[b];
    const int live_raw = p.live[u];
    const size_t ro = (size_t)u * p.nmax;
    const int base = threadIdx.x * KPT;
    double is_v[PREFETCH ? KPT : 1], l0_v[PREFETCH ? KPT : 1], t0_v[PREFETCH ? KPT : 1];
    if constexpr (PREFETCH) {
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            const int i = base + j;
            const bool in = i < p.nmax;
            is_v[j] = in ? p.scores[ro + i] : 0.0;
            l0_v[j] = in ? p.level[ro + i] : 0.0;
            t0_v[j] = in ? p.trend[ro + i] : 0.0;
        }
    }
    const int nb = min((slen + p.block - 1) / p.block, p.nmax);
    const int live = min(max(live_raw, 0), nb);
    const double one_a = dsub(1.0, p.alpha);
    const double one_b = dsub(1.0, p.beta);
    uint64_t key[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const int i = base + j;
        key[j] = 0ull;
        if (i < nb) {
            const double is = PREFETCH ? is_v[PREFETCH ? j : 0] : p.scores[ro + i];
            const double l0 = PREFETCH ? l0_v[PREFETCH ? j : 0] : p.level[ro + i];
            const double t0 = PREFETCH ? t0_v[PREFETCH ? j : 0] : p.trend[ro + i];
            double lv, tr;
            if (i < live) {
                // trend = beta (IS - level_old) + (1 - beta) trend_old;  level = alpha IS + (1 - alpha) level_old
                tr = dadd(dmul(p.beta, dsub(is, l0)), dmul(one_b, t0));
                lv = dadd(dmul(p.alpha, is), dmul(one_a, l0));
            } else {
                lv = is;      // a block seen for the first time starts at its score with no trend
                tr = 0.0;
            }
            p.level[ro + i] = lv;
            p.trend[ro + i] = tr;
            key[j] = order_key(dadd(lv, dmul(p.gamma, tr)));   // prediction level + gamma trend
        }
    }
    const uint32_t sel = block_topk<KPT, W>(key, nb, p.budget, sm);
    uint32_t total;
    const uint32_t off = block_excl_scan((uint32_t)__popc(sel), sm, 1, total);
    uint32_t o = off;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
        if (sel >> j & 1u) p.p_idx[(size_t)u * p.p_cap + o++] = base + j;
    if (threadIdx.x == 0) {
        p.p_cnt[u] = (int32_t)total;
        p.live[u] = nb;
    }
    if (p.p_pages) {
        __shared__ int32_t s_ent[kPageStage];
        int blk[KPT];
#pragma unroll
        for (int j = 0; j < KPT; ++j) blk[j] = base + j;
        const int ppb = p.block / kPage;
        write_set_pages<KPT, TPB, false>(p.p_pages + (size_t)u * p.p_cap * ppb, p.page_table, p.max_pages, ppb, b,
                                         slen, sel, off, blk, (int)total, s_ent);
    }
}

// Long rows in parts (the predictor's counterpart of the two-stage top-K): workgroup `part` of unit u
// updates the EMA state of blocks [512 part, +512) (two per thread, the arithmetic of predict_body) and
// keeps the local top-min(budget, 512) of their predictions as candidates; the unit's last part to
// finish ranks the candidates of all parts (topk_candidates_body) into P_next and sets live.
__device__ __forceinline__ void predict_part_body(const PredictParams &p, int u, int part, uint64_t *ckey,
                                                  int32_t *cidx, int32_t *ccnt, int kl, TopkSmem<4> &sm) {
    constexpr int BPL = 2, BPW = 256 * BPL;
    const int b = u / p.hkv;
    const int slen = p.seq_len[b];
    const int live_raw = p.live[u];
    const size_t ro = (size_t)u * p.nmax;
    const int first = part * BPW;
    const int base = first + (int)threadIdx.x * BPL;
    double is_v[BPL], l0_v[BPL], t0_v[BPL];
#pragma unroll
    for (int e = 0; e < BPL; ++e) {
        const int i = base + e;
        const bool in = i < p.nmax;
        is_v[e] = in ? p.scores[ro + i] : 0.0;
        l0_v[e] = in ? p.level[ro + i] : 0.0;
        t0_v[e] = in ? p.trend[ro + i] : 0.0;
    }
    const int nb = min((slen + p.block - 1) / p.block, p.nmax);
    const int live = min(max(live_raw, 0), nb);
    const double one_a = dsub(1.0, p.alpha);
    const double one_b = dsub(1.0, p.beta);
    double pred[BPL];
#pragma unroll
    for (int e = 0; e < BPL; ++e) {
        const int i = base + e;
        pred[e] = 0.0;
        if (i < nb) {
            double lv, tr;
            if (i < live) {
                tr = dadd(dmul(p.beta, dsub(is_v[e], l0_v[e])), dmul(one_b, t0_v[e]));
                lv = dadd(dmul(p.alpha, is_v[e]), dmul(one_a, l0_v[e]));
            } else {
                lv = is_v[e];
                tr = 0.0;
            }
            p.level[ro + i] = lv;
            p.trend[ro + i] = tr;
            pred[e] = dadd(lv, dmul(p.gamma, tr));
        }
    }
    const int n_local = min(max(nb - first, 0), BPW);
    local_candidates<BPL>(pred, n_local, kl, first, ckey, cidx, ccnt, sm);
}

// Workgroup shape of the top-K kernels for rows of up to nmax keys: one wave per SIMD (256 threads) with
// up to 4 keys each up to 1024 keys; 1024 threads with 2 to 32 keys beyond that. With 8-bit digits a
// pass costs few barriers, so at 2048 keys spreading the per-key work (the predictor's EMA update and
// the digit histogram) over 16 waves beats 4 waves with 8 keys each.
void topk_shape(int nmax, int &tpb, int &kpt) {
    tpb = nmax <= 128 ? 64 : nmax <= 1024 ? 256 : 1024;
    kpt = 1;
    while (kpt * tpb < nmax) kpt *= 2;
}

}  // namespace
}  // namespace prr

// back to the default (contraction allowed) for code that follows the include
#pragma clang fp contract(fast)
