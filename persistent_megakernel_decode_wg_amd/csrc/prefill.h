// prefill.h -- multi-token prefill (gfx950): the decoder over P prompt positions at once, writing the same
// KV cache the decode step reads and the logits / greedy argmax of the last position.
//
// At batch P the projections are dense contractions [P x K] x [K x N], so they run on the matrix cores:
// v_mfma_f32_16x16x32_bf16 takes, in every lane, 8 consecutive bf16 inputs of one row of each operand, which
// is exactly one 16-byte group of the packed weight layout, so the GEMMs read the decode step's packed blob
// in place.  Activations enter as hi/lo bf16 pairs (hi = bf16(x), lo = bf16(x - hi), two products per
// tile), as in the decode step's dot products, so inputs carry ~16 significant bits and the products with
// bf16 weights are exact in fp32.  Per layer: RMSNorm -> hi/lo; Q/K/V GEMM with bias, RoPE, the KV-cache
// append of every position and the rotated queries; causal attention over the cache (fp32, online
// softmax); output projection + residual; RMSNorm; gate/up GEMM with SiLU * up; down projection +
// residual.  Then the final norm and the tied vocabulary projection of the last position, and its argmax.
// (MegaBake third-party article, "Where it breaks today": prefill through the megakernel's decode-shaped
// bodies is slow above ~64 tokens; project site, "Next": fast long-prompt prefill.)
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace mbk {

typedef __bf16 pf_bf16x8 __attribute__((ext_vector_type(8)));
typedef float pf_f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int pf_u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPfTileP = 64;    // prompt positions are padded to a multiple of this

// Device buffers and shape of one prefill call (kernel argument, by value).
struct PfParams {
    const uint8_t *blob;     // packed weights (+ RoPE table)
    uint16_t *kv;            // [NL][2][nkv][S][hd] bf16
    const int32_t *tok;      // [P] token ids
    float *x;                // [Pp][H] residual stream
    float *q;                // [Pp][nq * hd] rotated queries
    uint16_t *inh[2], *inl[2];  // GEMM inputs as hi/lo bf16 [Pp][ks] (two buffers, used in turn)
    float *part;             // [4][Pp][rows] quarter sums of a k-split projection (rows: hidden or Q/K/V rows)
    float *logits;           // [V]
    int32_t *argmax_out;     // device int32
    uint32_t *prev_token;    // the decode workspace's previous-argmax word, or null
    MatGeom embed;
    uint64_t rope;           // byte offset of the fp32 RoPE table [S][hd/2][2] in blob
    int32_t P, Pp, ks, pos0;
    int32_t H, nq, nkv, hd, I, V, S, gqa, hd_shift;
    float eps, scale;
};

__device__ __forceinline__ float pf_bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t pf_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// dst[i] <- hi/lo of v[i] for the row's K entries; entries [K, ks) cleared (the GEMM's k tail reads them).
__device__ __forceinline__ void pf_store_split(uint16_t *dh, uint16_t *dl, int i, float v) {
    const uint16_t h = pf_to_bf16(v);
    dh[i] = h;
    dl[i] = pf_to_bf16(v - pf_bf16f(h));
}

// RMSNorm of x row r (or of the embedding row of its token when from_embed, which also sets x) times the
// bf16 weight at norm_off, split into hi/lo row `dst_row` of input buffer `dst`, two entries per 32-bit store;
// entries [H, H rounded up to 32) are cleared (the GEMMs read a row's inputs in k steps of 32 and nothing past
// them).  One workgroup of 256 threads per row.
__global__ __launch_bounds__(256) void k_pf_norm(PfParams p, uint64_t norm_off, int dst, int from_embed, int last_only) {
    __shared__ float red[8];
    const int r = last_only ? p.P - 1 : (int)blockIdx.x;
    const int dst_row = last_only ? 0 : r;
    const int h32 = (p.H + 31) & ~31;
    float *xr = p.x + (size_t)r * p.H;
    uint16_t *dh = p.inh[dst] + (size_t)dst_row * p.ks, *dl = p.inl[dst] + (size_t)dst_row * p.ks;
    if (r >= p.P) {  // padding rows of the position tiles: zero inputs
        for (int i = 2 * (int)threadIdx.x; i < h32; i += 512) *(uint32_t *)(dh + i) = *(uint32_t *)(dl + i) = 0u;
        return;
    }
    if (from_embed) {
        const int t = p.tok[r];
        for (int i = threadIdx.x; i < p.H; i += 256) {
            const uint16_t *e = (const uint16_t *)(p.blob + row_group_offset(p.embed, t, i >> 3));
            xr[i] = pf_bf16f(e[i & 7]);
        }
        __syncthreads();
    }
    float ss = 0.f;
    for (int i = threadIdx.x; i < p.H; i += 256) ss += xr[i] * xr[i];
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float rn = rsqrtf(tot / (float)p.H + p.eps);
    const uint16_t *w = (const uint16_t *)(p.blob + norm_off);
    for (int i = 2 * (int)threadIdx.x; i < h32; i += 512) {
        uint32_t hh = 0u, ll = 0u;
        if (i < p.H) {  // H is a multiple of 8: i + 1 < H too
            const float v0 = xr[i] * rn * pf_bf16f(w[i]), v1 = xr[i + 1] * rn * pf_bf16f(w[i + 1]);
            const uint16_t h0 = pf_to_bf16(v0), h1 = pf_to_bf16(v1);
            hh = (uint32_t)h0 | ((uint32_t)h1 << 16);
            ll = (uint32_t)pf_to_bf16(v0 - pf_bf16f(h0)) | ((uint32_t)pf_to_bf16(v1 - pf_bf16f(h1)) << 16);
        }
        *(uint32_t *)(dh + i) = hh;
        *(uint32_t *)(dl + i) = ll;
    }
    if (last_only) {
        // rows 1 .. 15 of the vocabulary projection's position block
        for (int rr = 1; rr < 16; ++rr)
            for (int i = 2 * (int)threadIdx.x; i < h32; i += 512)
                *(uint32_t *)(p.inh[dst] + (size_t)rr * p.ks + i) = *(uint32_t *)(p.inl[dst] + (size_t)rr * p.ks + i) = 0u;
    }
}

// C[pos][n] = sum_k in[pos][k] W[n][k] for the packed matrix g.  A workgroup takes packed rows
// [16 RB bx, 16 RB (bx + 1)) (RB row blocks of 16) and positions [16 NPB by, 16 NPB (by + 1)) (NPB position
// blocks of 16) of input buffer `src` (np_rows rows in all, a multiple of 16), so every activation load feeds
// RB matrix products and every weight load NPB.  RB = 4, NPB = 2 where that still leaves enough workgroups to
// fill the device, else RB = 2 or 1 and NPB = 1 or 2 by the matrix's size.  The k steps are split over KS waves (contiguous ranges; the partial
// tiles are added through LDS in wave order by wave 0, so the result depends neither on timing nor on RB or
// NPB), which multiplies the loads in flight and shortens each wave's chain.  Lane l feeds row l % 16
// of each operand with input group 4 s + l / 16 of k step s (32 inputs); the k steps go in batches (8 with
// one row block, 4 with two or four) whose loads are all issued before the batch's products.  After the k loop lane
// l holds C[16 NPB by + 16 j + 4 (l / 16) + r][16 RB bx + 16 rb + l % 16] in acc[rb][j][r].  Epilogue by op.
constexpr int kPfPos = 32;
template <int OP, bool FP8 = false>
__device__ __forceinline__ void pf_epilogue(const PfParams &p, const MatGeom &g, int layer, int dst, uint64_t bias_off,
                                            int n, int pos, float y) {
    const int hd = p.hd, half = hd >> 1, Q = p.nq * hd, KVr = p.nkv * hd;
    const bool nrow = n < g.rows;
    // fp8 rows: the products were formed with the codes' values; the row's power-of-two scale comes here
    if (FP8 && nrow) y *= *(const float *)(p.blob + row_scale_offset(g, n));
    if (OP == OP_QKV) {
        // packed rows 2m, 2m+1 of a query or key head are its dims m, m + hd/2 (adjacent lanes)
        const int which = n >= Q + KVr ? 2 : (n >= Q ? 1 : 0);
        const int base = n - (which == 0 ? 0 : (which == 1 ? Q : Q + KVr));
        const int i = base & (hd - 1);
        const int srow = which == 2 ? base : (base & ~(hd - 1)) + ((i & 1) ? (i >> 1) + half : (i >> 1));
        if (bias_off != ~(uint64_t)0 && nrow)
            y += pf_bf16f(((const uint16_t *)(p.blob + bias_off))[(which == 0 ? 0 : (which == 1 ? Q : Q + KVr)) + srow]);
        const float partner = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(y), 0xB1, 0xf, 0xf, false));
        if (!nrow || pos >= p.P) return;
        const int slot = p.pos0 + pos;
        if (which == 2) {
            const int jh = srow >> p.hd_shift, d = srow & (hd - 1);
            p.kv[((((size_t)layer * 2 + 1) * p.nkv + jh) * p.S + slot) * hd + d] = pf_to_bf16(y);
            return;
        }
        if (i & 1) return;  // the odd row is the partner of this pair
        const int h = srow >> p.hd_shift, m = srow & (hd - 1);
        const float2 cs = ((const float2 *)(p.blob + p.rope))[(size_t)slot * half + m];
        const float r0 = y * cs.x - partner * cs.y, r1 = partner * cs.x + y * cs.y;
        if (which == 0) {
            p.q[(size_t)pos * Q + h * hd + m] = r0;
            p.q[(size_t)pos * Q + h * hd + m + half] = r1;
        } else {
            uint16_t *kc = p.kv + ((((size_t)layer * 2 + 0) * p.nkv + h) * p.S + slot) * hd;
            kc[m] = pf_to_bf16(r0);
            kc[m + half] = pf_to_bf16(r1);
        }
    } else if (OP == OP_O || OP == OP_DOWN) {
        if (nrow && pos < p.P) p.x[(size_t)pos * p.H + n] += y;
    } else if (OP == OP_GATEUP) {
        // packed row 2i is gate row i, 2i + 1 up row i (adjacent lanes)
        const float up = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(y), 0xB1, 0xf, 0xf, false));
        if (!nrow || pos >= p.P || (n & 1)) return;
        pf_store_split(p.inh[dst] + (size_t)pos * p.ks, p.inl[dst] + (size_t)pos * p.ks, n >> 1, y / (1.f + __expf(-y)) * up);
    } else {  // vocabulary projection of the last position (row 0 of the block)
        if (nrow && pos == 0) p.logits[n] = y;
    }
}

// Eight E4M3 codes (k order, byte j = code j) as the eight bf16 inputs of a matrix-instruction lane: each code
// is widened to fp32 by the hardware conversion (OCP E4M3 on gfx950) and its top half taken -- exact, since
// a code's value has at most four significant bits.
__device__ __forceinline__ pf_u32x4 pf_fp8x8_to_bf16(uint2 c) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.x, true);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, false), e = __builtin_amdgcn_cvt_pk_f32_fp8((int)c.y, true);
    pf_u32x4 r;
    r.x = (__float_as_uint(a[0]) >> 16) | (__float_as_uint(a[1]) & 0xffff0000u);
    r.y = (__float_as_uint(b[0]) >> 16) | (__float_as_uint(b[1]) & 0xffff0000u);
    r.z = (__float_as_uint(d[0]) >> 16) | (__float_as_uint(d[1]) & 0xffff0000u);
    r.w = (__float_as_uint(e[0]) >> 16) | (__float_as_uint(e[1]) & 0xffff0000u);
    return r;
}

template <int OP, int kPfRB, int KS, bool FP8, int NPB>
__global__ __launch_bounds__(64 * KS) void k_pf_gemm(PfParams p, MatGeom g, int layer, int src, int dst, int np_rows,
                                                     uint64_t bias_off) {
    constexpr int kPfBatch = kPfRB == 1 ? 8 : 4;
    const int l = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 16 * kPfRB + (l & 15);  // this lane's row in row block 0 (+16 rb)
    const int pb = blockIdx.y * 16 * NPB;
    const int nb = min(16 * NPB, np_rows - pb) >> 4;    // position blocks of 16: 1 .. NPB
    const int kq = l >> 4, ngrp = g.K >> 3, nall = (ngrp + 3) >> 2;
    // this wave's k steps [sb, sb + nsteps)
    const int sb = nall * wv / KS, nsteps = nall * (wv + 1) / KS - sb;
    const uint16_t *ah = p.inh[src], *al = p.inl[src];
    const size_t arow0 = (size_t)(pb + (l & 15)) * p.ks;
    pf_f32x4 acc[kPfRB][NPB];
#pragma unroll
    for (int rb = 0; rb < kPfRB; ++rb)
#pragma unroll
        for (int j = 0; j < NPB; ++j) acc[rb][j] = (pf_f32x4){0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nsteps; s0 += kPfBatch) {
        pf_u32x4 bw[kPfRB][kPfBatch], xh[NPB][kPfBatch], xl[NPB][kPfBatch];
#pragma unroll
        for (int i = 0; i < kPfBatch; ++i) {
            const int kg = 4 * (sb + s0 + i) + kq;
            const bool step = s0 + i < nsteps;
#pragma unroll
            for (int rb = 0; rb < kPfRB; ++rb) {
                const int n = n0 + 16 * rb;
                bw[rb][i] = (pf_u32x4){0u, 0u, 0u, 0u};
                if (step && n < g.rows && kg < ngrp) {
                    // fp8: the 8 inputs kg are half kg & 1 of 16-code group kg / 2
                    if (FP8)
                        bw[rb][i] = pf_fp8x8_to_bf16(*(const uint2 *)(p.blob + row_group_offset(g, n, kg >> 1) + 8 * (kg & 1)));
                    else
                        bw[rb][i] = *(const pf_u32x4 *)(p.blob + row_group_offset(g, n, kg));
                }
            }
#pragma unroll
            for (int j = 0; j < NPB; ++j) {
                xh[j][i] = xl[j][i] = (pf_u32x4){0u, 0u, 0u, 0u};
                if (step && j < nb) {
                    const size_t at = arow0 + (size_t)16 * j * p.ks + 8 * kg;
                    xh[j][i] = *(const pf_u32x4 *)(ah + at);
                    xl[j][i] = *(const pf_u32x4 *)(al + at);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kPfBatch; ++i) {
#pragma unroll
            for (int rb = 0; rb < kPfRB; ++rb) {
                const pf_bf16x8 b = __builtin_bit_cast(pf_bf16x8, bw[rb][i]);
#pragma unroll
                for (int j = 0; j < NPB; ++j) {
                    acc[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(pf_bf16x8, xh[j][i]), b,
                                                                         acc[rb][j], 0, 0, 0);
                    acc[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(pf_bf16x8, xl[j][i]), b,
                                                                         acc[rb][j], 0, 0, 0);
                }
            }
        }
    }
    if (KS > 1) {
        // partial tiles of the waves, added in wave order
        __shared__ pf_f32x4 part[KS > 1 ? KS - 1 : 1][kPfRB][NPB][64];
        if (wv > 0)
#pragma unroll
            for (int rb = 0; rb < kPfRB; ++rb)
#pragma unroll
                for (int j = 0; j < NPB; ++j) part[wv - 1][rb][j][l] = acc[rb][j];
        __syncthreads();
        if (wv > 0) return;
#pragma unroll
        for (int w = 0; w < KS - 1; ++w)
#pragma unroll
            for (int rb = 0; rb < kPfRB; ++rb)
#pragma unroll
                for (int j = 0; j < NPB; ++j) acc[rb][j] += part[w][rb][j][l];
    }
    // epilogue: lane l holds C[pb + 16 j + 4 kq + r][n0 + 16 rb]
#pragma unroll
    for (int rb = 0; rb < kPfRB; ++rb)
#pragma unroll
        for (int j = 0; j < NPB; ++j) {
            if (j >= nb) break;
#pragma unroll
            for (int r = 0; r < 4; ++r) pf_epilogue<OP, FP8>(p, g, layer, dst, bias_off, n0 + 16 * rb, pb + 16 * j + 4 * kq + r, acc[rb][j][r]);
        }
}

// The same products for long prompts, with operand tiles shared by the workgroup's four waves: a workgroup
// takes 32 WRB packed rows x 64 positions; wave (wr, wc) = (w / 2, w % 2) computes rows 16 WRB wr .. (WRB row
// blocks) x positions 32 wc .. + 31 (two position blocks).  Every 16 x 32 operand tile of a k step (the 16
// rows' input groups 4 s .. 4 s + 3, one 16-byte group per lane exactly as the matrix instruction takes it)
// is loaded once for the workgroup straight into LDS (global_load_lds, 1 KiB per wave-wide load), so each
// weight tile feeds two waves and each activation tile two; the loads run kPfLAhead stages (of kPfLStep k
// steps) ahead of the products.  Each row's products are formed in the order of k_pf_gemm<., ., 4>: the k
// steps in four contiguous quarters, each quarter's chain from zero (hi then lo input per step), and the
// quarter sums added in order -- so the result equals that kernel's bit for bit (weight groups past the
// matrix's K and rows past its end are read clamped: they meet zero inputs or feed no output).
constexpr int kPfLStep = 1;                              // k steps per stage
constexpr int kPfLAhead = 2;                             // stages in flight ahead of the one computed
template <int WRB> struct PfLGeom {
    static constexpr int kTiles = (8 + 2 * WRB) * kPfLStep;  // 1 KiB tiles per stage: 8 activation + 2 WRB weight
    static constexpr int kStageBytes = kTiles * 1024;
    static constexpr int kLds = (kPfLAhead + 1) * kStageBytes;
    static_assert(kTiles % 4 == 0, "every wave issues the same number of loads per stage");
};
typedef __attribute__((address_space(3))) void pf_lds_void_t;
typedef __attribute__((address_space(1))) void pf_glb_void_t;

template <int OP, int WRB, bool SPLIT>
__global__ __launch_bounds__(256) void k_pf_gemm_lds(PfParams p, MatGeom g, int layer, int src, int dst, int np_rows,
                                                     uint64_t bias_off) {
    typedef PfLGeom<WRB> Gm;
    constexpr int kPerStep = 8 + 2 * WRB;                 // tiles of one k step
    extern __shared__ __attribute__((aligned(16))) uint8_t pf_ring[];
    const int l = threadIdx.x & 63, wv = threadIdx.x >> 6, wr = wv >> 1, wc = wv & 1;
    const int rbase = blockIdx.x * 32 * WRB, pbase = blockIdx.y * 64;
    const int ngrp = g.K >> 3, nall = (ngrp + 3) >> 2;
    // SPLIT: this workgroup forms only quarter blockIdx.z of the k steps and stores its chain to p.part
    const int s_lo = SPLIT ? nall * (int)blockIdx.z / 4 : 0, s_hi = SPLIT ? nall * ((int)blockIdx.z + 1) / 4 : nall;
    const int nst = (s_hi - s_lo + kPfLStep - 1) / kPfLStep;
    const uint16_t *ah = p.inh[src], *al = p.inl[src];
    // the loads of stage st: wave w issues tiles w, w + 4, ... of the stage; tile u of a k step is
    // activation block u / 2 (hi for even u, lo for odd) for u < 8, weight row block u - 8 after
    auto issue = [&](int st) {
        uint8_t *buf = pf_ring + (st % (kPfLAhead + 1)) * Gm::kStageBytes;
#pragma unroll
        for (int t = wv; t < Gm::kTiles; t += 4) {
            const int i = t / kPerStep, u = t - i * kPerStep, s = s_lo + st * kPfLStep + i;
            if (s >= s_hi) continue;
            const int kg = 4 * s + (l >> 4);
            const uint8_t *a;
            if (u < 8) {
                const size_t row = (size_t)(pbase + 16 * (u >> 1) + (l & 15));
                a = (const uint8_t *)((u & 1 ? al : ah) + row * p.ks + 8 * kg);
            } else {
                const int n = min(rbase + 16 * (u - 8) + (l & 15), g.rows - 1);
                a = p.blob + row_group_offset(g, n, min(kg, ngrp - 1));
            }
            __builtin_amdgcn_global_load_lds((pf_glb_void_t *)a, (pf_lds_void_t *)(buf + t * 1024), 16, 0, 0);
        }
    };
    pf_f32x4 acc[WRB][2], tot[WRB][2];
#pragma unroll
    for (int rb = 0; rb < WRB; ++rb)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[rb][j] = tot[rb][j] = (pf_f32x4){0.f, 0.f, 0.f, 0.f};
    int q = 0, qend = nall / 4;  // current quarter and its end (quarter q is [nall q / 4, nall (q + 1) / 4))
    auto close_quarter = [&]() {
#pragma unroll
        for (int rb = 0; rb < WRB; ++rb)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                tot[rb][j] = q == 0 ? acc[rb][j] : tot[rb][j] + acc[rb][j];
                acc[rb][j] = (pf_f32x4){0.f, 0.f, 0.f, 0.f};
            }
        ++q;
        qend = nall * (q + 1) / 4;
    };
    for (int st = 0; st < kPfLAhead && st < nst; ++st) issue(st);
    for (int st = 0; st < nst; ++st) {
        // this wave's loads of stage st are complete once at most those of the later stages in flight remain
        // (the last stage may hold fewer, so near the end nothing may remain), and its reads of stage st - 1
        // are complete before another wave's loads may overwrite that stage
        constexpr int kLater = Gm::kTiles / 4 * (kPfLAhead - 1);  // this wave's loads of kPfLAhead - 1 full stages
        static_assert(kLater < 64, "vmcnt range");
        if (st + kPfLAhead < nst) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kLater) : "memory");
        else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        // every wave's loads of stage st are in LDS and every wave is done with stage st - 1 (the barrier alone:
        // the loads of the later stages stay in flight); no LDS access moves across it
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (st + kPfLAhead < nst) issue(st + kPfLAhead);
        const uint8_t *buf = pf_ring + (st % (kPfLAhead + 1)) * Gm::kStageBytes;
#pragma unroll
        for (int i = 0; i < kPfLStep; ++i) {
            const int s = s_lo + st * kPfLStep + i;
            if (s >= s_hi) break;
            if (!SPLIT)
                while (q < 3 && s >= qend) close_quarter();
            const uint8_t *tb = buf + i * kPerStep * 1024 + l * 16;
            pf_u32x4 xa[2][2], wb[WRB];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                xa[j][0] = *(const pf_u32x4 *)(tb + (2 * (2 * wc + j) + 0) * 1024);
                xa[j][1] = *(const pf_u32x4 *)(tb + (2 * (2 * wc + j) + 1) * 1024);
            }
#pragma unroll
            for (int rb = 0; rb < WRB; ++rb) wb[rb] = *(const pf_u32x4 *)(tb + (8 + WRB * wr + rb) * 1024);
#pragma unroll
            for (int rb = 0; rb < WRB; ++rb) {
                const pf_bf16x8 b = __builtin_bit_cast(pf_bf16x8, wb[rb]);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    acc[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(pf_bf16x8, xa[j][0]), b,
                                                                         acc[rb][j], 0, 0, 0);
                    acc[rb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(pf_bf16x8, xa[j][1]), b,
                                                                         acc[rb][j], 0, 0, 0);
                }
            }
        }
    }
    const int kq = l >> 4;
    if (SPLIT) {
#pragma unroll
        for (int rb = 0; rb < WRB; ++rb) {
            const int n = rbase + 16 * WRB * wr + 16 * rb + (l & 15);
            if (n >= g.rows) continue;
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int pos = pbase + 32 * wc + 16 * j + 4 * kq + r;
                    p.part[((size_t)blockIdx.z * np_rows + pos) * g.rows + n] = acc[rb][j][r];
                }
        }
        return;
    }
    while (q < 4) close_quarter();  // the remaining quarters (possibly empty) in order
#pragma unroll
    for (int rb = 0; rb < WRB; ++rb)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                pf_epilogue<OP>(p, g, layer, dst, bias_off, rbase + 16 * WRB * wr + 16 * rb + (l & 15),
                                pbase + 32 * wc + 16 * j + 4 * kq + r, tot[rb][j][r]);
}

// A k-split shared-tile GEMM's outputs: the four quarter chains added in order, as the unsplit kernels add
// them, then the epilogue (one thread per output; adjacent rows in adjacent lanes, as the Q/K/V epilogue's
// lane pairs need).
template <int OP>
__global__ __launch_bounds__(256) void k_pf_split_sum(PfParams p, MatGeom g, int layer, int dst, int np_rows,
                                                      uint64_t bias_off) {
    const int n = (int)(blockIdx.x * 256 + threadIdx.x), pos = (int)blockIdx.y;
    if (n >= g.rows) return;
    const size_t q = (size_t)np_rows * g.rows, at = (size_t)pos * g.rows + n;
    const float t = ((p.part[at] + p.part[at + q]) + p.part[at + 2 * q]) + p.part[at + 3 * q];
    pf_epilogue<OP>(p, g, layer, dst, bias_off, n, pos, t);
}

// Columns [K, K rounded up to 32) of the rows written by the attention or the gate/up epilogue (the next
// GEMM reads a row in k steps of 32).
__global__ __launch_bounds__(256) void k_pf_clear_tail(PfParams p, int buf, int K) {
    const int r = blockIdx.x;
    for (int i = K + (int)threadIdx.x; i < ((K + 31) & ~31); i += 256) {
        p.inh[buf][(size_t)r * p.ks + i] = 0;
        p.inl[buf][(size_t)r * p.ks + i] = 0;
    }
}

// Causal attention of prompt positions pos0 + 16 bx .. pos0 + 16 bx + 15, query head h, each over cache
// positions 0 .. its own (the current one included, rounded to bf16 as the cache holds it).  Four waves,
// four queries each; keys in blocks of 64 aligned at cache position 0, shared by the 16 queries: a block's
// keys and values are staged in LDS with one batch of 16-byte loads (the key rows' 16-byte chunks rotated
// by row so that lanes reading chunk c of different rows hit different banks).  Lane t of a wave scores key
// t of the block for the wave's four queries (full dot product over the head dims); per query a running
// maximum, sum and output (online softmax; a block wholly past a query's position leaves its state exactly
// unchanged, so the result does not depend on how the prompt is split into calls); the weighted values
// with lanes over the head dims, from LDS.  Output hi/lo into input buffer dst.
constexpr int kPfAttnQ = 16, kPfAttnQW = 4;
__global__ __launch_bounds__(256) void k_pf_attn(PfParams p, int layer, int dst) {
    __shared__ float qs[kPfAttnQ * 128];
    __shared__ float ps[kPfAttnQ * 64];
    __shared__ pf_u32x4 kb[64 * 16], vb[64 * 16];   // up to 64 keys x 128 dims of bf16 each
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, hd = p.hd, c16 = hd >> 3;
    const int h = blockIdx.y, j = h / p.gqa, q0 = blockIdx.x * kPfAttnQ;
    const int nqb = min(kPfAttnQ, p.P - q0);
    for (int i = tid; i < kPfAttnQ * hd; i += 256) {
        const int qr = i >> p.hd_shift, d = i & (hd - 1);
        qs[i] = qr < nqb ? p.q[(size_t)(q0 + qr) * p.nq * hd + h * hd + d] * p.scale : 0.f;
    }
    const uint16_t *K = p.kv + (((size_t)layer * 2 + 0) * p.nkv + j) * p.S * hd;
    const uint16_t *V = p.kv + (((size_t)layer * 2 + 1) * p.nkv + j) * p.S * hd;
    const int Lmax = p.pos0 + q0 + nqb;           // keys the block's last query sees
    int lim[kPfAttnQW];                            // keys 0 .. lim - 1 for this wave's queries
    float M[kPfAttnQW], Ls[kPfAttnQW], o0[kPfAttnQW], o1[kPfAttnQW];
#pragma unroll
    for (int u = 0; u < kPfAttnQW; ++u) {
        const int qr = w * kPfAttnQW + u;
        lim[u] = p.pos0 + q0 + min(qr, nqb - 1) + 1;
        M[u] = -INFINITY;
        Ls[u] = o0[u] = o1[u] = 0.f;
    }
    for (int t0 = 0; t0 < Lmax; t0 += 64) {
        const int nk = min(64, Lmax - t0);
        {
            pf_u32x4 kw[4], vw[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = tid + 256 * u, r = i / c16, c = i & (c16 - 1);
                if (i < 64 * c16 && r < nk) {
                    kw[u] = ((const pf_u32x4 *)(K + (size_t)(t0 + r) * hd))[c];
                    vw[u] = ((const pf_u32x4 *)(V + (size_t)(t0 + r) * hd))[c];
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = tid + 256 * u, r = i / c16, c = i & (c16 - 1);
                if (i < 64 * c16 && r < nk) {
                    kb[r * c16 + (c ^ (r & (c16 - 1)))] = kw[u];
                    vb[i] = vw[u];
                }
            }
        }
        __syncthreads();
        const int t = t0 + l;
        float s[kPfAttnQW];
#pragma unroll
        for (int u = 0; u < kPfAttnQW; ++u) s[u] = 0.f;
        if (l < nk) {
            for (int c = 0; c < c16; ++c) {
                const pf_u32x4 kw = kb[l * c16 + (c ^ (l & (c16 - 1)))];
                float kf[8];
                kf[0] = __uint_as_float(kw.x << 16); kf[1] = __uint_as_float(kw.x & 0xffff0000u);
                kf[2] = __uint_as_float(kw.y << 16); kf[3] = __uint_as_float(kw.y & 0xffff0000u);
                kf[4] = __uint_as_float(kw.z << 16); kf[5] = __uint_as_float(kw.z & 0xffff0000u);
                kf[6] = __uint_as_float(kw.w << 16); kf[7] = __uint_as_float(kw.w & 0xffff0000u);
#pragma unroll
                for (int u = 0; u < kPfAttnQW; ++u) {
                    const float *qd = qs + (w * kPfAttnQW + u) * hd + 8 * c;
#pragma unroll
                    for (int e = 0; e < 8; ++e) s[u] = fmaf(qd[e], kf[e], s[u]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kPfAttnQW; ++u) {
            const float sv = t < lim[u] ? s[u] : -INFINITY;
            float mp = sv;
            for (int o = 32; o > 0; o >>= 1) mp = fmaxf(mp, __shfl_xor(mp, o));
            const float mn = fmaxf(M[u], mp);
            const float cf = M[u] == -INFINITY ? 0.f : __expf(M[u] - mn);
            const float pw = t < lim[u] ? __expf(sv - mn) : 0.f;
            float sp = pw;
            for (int o = 32; o > 0; o >>= 1) sp += __shfl_xor(sp, o);
            Ls[u] = Ls[u] * cf + sp;
            o0[u] *= cf;
            o1[u] *= cf;
            M[u] = mn;
            ps[(w * kPfAttnQW + u) * 64 + l] = pw;
        }
        __syncthreads();
        const uint16_t *vs = (const uint16_t *)vb;
        const float *pw4 = ps + w * kPfAttnQW * 64;
        for (int k = 0; k < nk; ++k) {
            const float v0 = l < hd ? pf_bf16f(vs[k * hd + l]) : 0.f;
            const float v1 = l + 64 < hd ? pf_bf16f(vs[k * hd + l + 64]) : 0.f;
#pragma unroll
            for (int u = 0; u < kPfAttnQW; ++u) {
                const float pk = pw4[u * 64 + k];
                o0[u] = fmaf(pk, v0, o0[u]);
                o1[u] = fmaf(pk, v1, o1[u]);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < kPfAttnQW; ++u) {
        const int qr = w * kPfAttnQW + u;
        if (qr >= nqb) break;
        const float inv = 1.f / Ls[u];
        uint16_t *dh = p.inh[dst] + (size_t)(q0 + qr) * p.ks + h * hd, *dl = p.inl[dst] + (size_t)(q0 + qr) * p.ks + h * hd;
        if (l < hd) pf_store_split(dh, dl, l, o0[u] * inv);
        if (l + 64 < hd) pf_store_split(dh, dl, l + 64, o1[u] * inv);
    }
}

// Causal attention on the matrix cores, head size HD (a multiple of 32): one wave per workgroup takes
// queries q0 .. q0 + 15 (prompt positions pos0 + q0 ..) of head h; keys in blocks of 32 aligned at cache
// position 0.  Scores as S^T = K Q^T: operand A is 16 cached keys x 32 head dims (16 contiguous bytes of
// a key row per lane, read straight from the cache), operand B the 16 queries' 32 dims as hi/lo bf16 pairs
// (held in registers, pre-scaled); lane (g = l / 16, c = l % 16) gets keys 4 g + r of each 16-key tile for
// query c.  Online softmax per query over the lane's 8 keys and the 4 lane groups of its column (a block
// wholly past a query's position leaves its state exactly unchanged).  Weighted values as O^T = V^T P^T:
// operand B is exactly those 8 probabilities per lane (hi/lo pairs; the order of the 32 keys in the
// contraction is the lanes' own: tile 0 keys 4 g .. 4 g + 3, then tile 1's), operand A the values of the
// same keys at 16 head dims, read from the block's values staged transposed in LDS.  Lane (g, c), register
// r of output tile dt holds query c, dim 16 dt + 4 g + r.  The W waves of a workgroup take the key blocks in
// turn (wave w blocks w, w + W, ...), each with its own running state and its own staging area, so the
// longest chain of blocks (the last queries of a long prompt) is W times shorter; at the end the waves'
// states meet in LDS and wave 0 combines them in wave order with the log-sum-exp rule (a wave whose blocks
// all lie past a query's position adds exactly nothing).  Output hi/lo into input buffer dst.
template <int HD, int W>
__global__ __launch_bounds__(64 * W) void k_pf_attn_mma(PfParams p, int layer, int dst) {
    constexpr int KS = HD / 32, DT = HD / 16, VR = 32 + 4;   // score k steps, output tiles, V^T row (bf16)
    constexpr int NS = 2 + 4 * DT;                           // floats of one lane's state: max, sum, outputs
    static_assert((W - 1) * 64 * NS * 4 <= W * HD * VR * 2, "the waves' states fit the staging areas");
    __shared__ __attribute__((aligned(16))) uint16_t vts[W * HD * VR];
    const int l = threadIdx.x & 63, wv = threadIdx.x >> 6, g = l >> 4, c = l & 15;
    uint16_t *vt = vts + wv * HD * VR;
    const int h = blockIdx.y, j = h / p.gqa, q0 = blockIdx.x * 16;
    const int nqb = min(16, p.P - q0);
    const int qc = min(c, nqb - 1);                 // padding columns repeat the last query (never stored)
    const int qpos = p.pos0 + q0 + qc;              // keys 0 .. qpos for this lane's query
    const int Lmax = p.pos0 + q0 + nqb;             // keys the block's last query sees
    pf_bf16x8 qh[KS], ql[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const float *qr = p.q + (size_t)(q0 + qc) * p.nq * HD + h * HD + 32 * s + 8 * g;
        uint16_t hb[8], lb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = qr[e] * p.scale;
            hb[e] = pf_to_bf16(v);
            lb[e] = pf_to_bf16(v - pf_bf16f(hb[e]));
        }
        qh[s] = __builtin_bit_cast(pf_bf16x8, hb);
        ql[s] = __builtin_bit_cast(pf_bf16x8, lb);
    }
    const uint16_t *K = p.kv + (((size_t)layer * 2 + 0) * p.nkv + j) * p.S * HD;
    const uint16_t *V = p.kv + (((size_t)layer * 2 + 1) * p.nkv + j) * p.S * HD;
    float M = -INFINITY, Ls = 0.f;
    pf_f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = (pf_f32x4){0.f, 0.f, 0.f, 0.f};
    // a block's keys (operand A tiles) and values (the lane's 16-byte chunks), loaded one block ahead
    constexpr int VC = HD / 16;                     // value chunks per lane and block
    pf_u32x4 kw[2][KS], vw[VC];
    auto load_block = [&](int t0) {
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            const int key = t0 + 16 * tau + c;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                kw[tau][s] = (pf_u32x4){0u, 0u, 0u, 0u};
                if (key < Lmax) kw[tau][s] = *(const pf_u32x4 *)(K + (size_t)key * HD + 32 * s + 8 * g);
            }
        }
#pragma unroll
        for (int u = 0; u < VC; ++u) {
            const int ci = l + 64 * u, key = ci / (HD / 8), dc = ci % (HD / 8);
            vw[u] = (pf_u32x4){0u, 0u, 0u, 0u};
            if (t0 + key < Lmax) vw[u] = *(const pf_u32x4 *)(V + (size_t)(t0 + key) * HD + 8 * dc);
        }
    };
    if (32 * wv < Lmax) load_block(32 * wv);
    for (int t0 = 32 * wv; t0 < Lmax; t0 += 32 * W) {
        // this block's values, transposed: vt[d][key] (keys past the last query's position are zero)
#pragma unroll
        for (int u = 0; u < VC; ++u) {
            const int ci = l + 64 * u, key = ci / (HD / 8), dc = ci % (HD / 8);
            const uint32_t ww[4] = {vw[u].x, vw[u].y, vw[u].z, vw[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vt[(8 * dc + 2 * e) * VR + key] = (uint16_t)(ww[e] & 0xffffu);
                vt[(8 * dc + 2 * e + 1) * VR + key] = (uint16_t)(ww[e] >> 16);
            }
        }
        // scores of keys t0 + 16 tau + 4 g + r for query c
        float sc[2][4];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
            pf_f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const pf_bf16x8 a = __builtin_bit_cast(pf_bf16x8, kw[tau][s]);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[s], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[s], acc, 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[tau][r] = t0 + 16 * tau + 4 * g + r <= qpos ? acc[r] : -INFINITY;
        }
        if (t0 + 32 * W < Lmax) load_block(t0 + 32 * W);   // the next block's loads overlap this block's math
        float mb = sc[0][0];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int r = 0; r < 4; ++r) mb = fmaxf(mb, sc[tau][r]);
        mb = fmaxf(mb, __shfl_xor(mb, 16));
        mb = fmaxf(mb, __shfl_xor(mb, 32));
        const float mn = fmaxf(M, mb);
        const float cf = M == -INFINITY ? 0.f : __expf(M - mn);
        float pw[8], sb = 0.f;
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = sc[tau][r] == -INFINITY ? 0.f : __expf(sc[tau][r] - mn);
                pw[4 * tau + r] = v;
                sb += v;
            }
        sb += __shfl_xor(sb, 16);
        sb += __shfl_xor(sb, 32);
        Ls = Ls * cf + sb;
        M = mn;
        uint16_t ph[8], pl[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ph[e] = pf_to_bf16(pw[e]);
            pl[e] = pf_to_bf16(pw[e] - pf_bf16f(ph[e]));
        }
        const pf_bf16x8 bh = __builtin_bit_cast(pf_bf16x8, ph), bl = __builtin_bit_cast(pf_bf16x8, pl);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the wave's staged values are in LDS
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const uint16_t *row = vt + (16 * dt + c) * VR;
            const uint2 v0 = *(const uint2 *)(row + 4 * g), v1 = *(const uint2 *)(row + 16 + 4 * g);
            const pf_u32x4 vw = {v0.x, v0.y, v1.x, v1.y};
            const pf_bf16x8 a = __builtin_bit_cast(pf_bf16x8, vw);
#pragma unroll
            for (int r = 0; r < 4; ++r) o[dt][r] *= cf;
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, o[dt], 0, 0, 0);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // read before the next block is staged
    }
    if (W > 1) {
        // the waves' states, then wave 0 combines them in wave order
        float *st = (float *)vts;
        __syncthreads();   // every wave is past its last block (the states reuse the staging areas)
        if (wv > 0) {
            float *d = st + ((wv - 1) * 64 + l) * NS;
            d[0] = M;
            d[1] = Ls;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) d[2 + 4 * dt + r] = o[dt][r];
        }
        __syncthreads();
        if (wv > 0) return;
        float mm = M;
#pragma unroll
        for (int w = 1; w < W; ++w) mm = fmaxf(mm, st[((w - 1) * 64 + l) * NS]);
        const float f0 = M == -INFINITY ? 0.f : __expf(M - mm);
        Ls *= f0;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[dt][r] *= f0;
#pragma unroll
        for (int w = 1; w < W; ++w) {
            const float *d = st + ((w - 1) * 64 + l) * NS;
            const float f = d[0] == -INFINITY ? 0.f : __expf(d[0] - mm);
            Ls = fmaf(d[1], f, Ls);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) o[dt][r] = fmaf(d[2 + 4 * dt + r], f, o[dt][r]);
        }
    }
    if (c >= nqb) return;
    const float inv = 1.f / Ls;
    uint16_t *dh = p.inh[dst] + (size_t)(q0 + c) * p.ks + h * HD, *dl = p.inl[dst] + (size_t)(q0 + c) * p.ks + h * HD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) pf_store_split(dh, dl, 16 * dt + 4 * g + r, o[dt][r] * inv);
}

// Greedy argmax of the V logits (lowest index among equal maxima); also the decode step's previous token.
// The rule picks the largest value, then the lowest index, so any scan order gives the same index: each thread
// takes every 1024th group of four logits (one 16-byte load, four loads in flight) where V is a multiple of 4.
__device__ __forceinline__ void pf_amax_take(float v, int i, float &best, int &idx) {
    if (v > best || (v == best && i < idx)) { best = v; idx = i; }
}
__global__ __launch_bounds__(1024) void k_pf_argmax(PfParams p) {
    __shared__ float bv[1024];
    __shared__ int bi[1024];
    float best = -INFINITY;
    int idx = 0x7fffffff;
    if ((p.V & 3) == 0 && ((uintptr_t)p.logits & 15) == 0) {
        const float4 *l4 = (const float4 *)p.logits;
        const int n4 = p.V >> 2;
        int i = threadIdx.x;
        for (; i + 3 * 1024 < n4; i += 4 * 1024) {
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = l4[i + u * 1024];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int b = 4 * (i + u * 1024);
                pf_amax_take(v[u].x, b, best, idx);
                pf_amax_take(v[u].y, b + 1, best, idx);
                pf_amax_take(v[u].z, b + 2, best, idx);
                pf_amax_take(v[u].w, b + 3, best, idx);
            }
        }
        for (; i < n4; i += 1024) {
            const float4 v = l4[i];
            pf_amax_take(v.x, 4 * i, best, idx);
            pf_amax_take(v.y, 4 * i + 1, best, idx);
            pf_amax_take(v.z, 4 * i + 2, best, idx);
            pf_amax_take(v.w, 4 * i + 3, best, idx);
        }
    } else {
        for (int i = threadIdx.x; i < p.V; i += 1024) pf_amax_take(p.logits[i], i, best, idx);
    }
    bv[threadIdx.x] = best;
    bi[threadIdx.x] = idx;
    __syncthreads();
    for (int s = 512; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) {
            const float v = bv[threadIdx.x + s];
            const int i = bi[threadIdx.x + s];
            if (v > bv[threadIdx.x] || (v == bv[threadIdx.x] && i < bi[threadIdx.x])) {
                bv[threadIdx.x] = v;
                bi[threadIdx.x] = i;
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        p.argmax_out[0] = bi[0];
        if (p.prev_token) *p.prev_token = (uint32_t)bi[0];
    }
}

}  // namespace mbk
