// bodies.h -- device bodies of the decode step (gfx950, wave64).
//
// Every body is a __device__ function run by one workgroup; the persistent
// kernel calls them in task-list order with a grid barrier between intervals,
// the ablation kernel calls one interval per launch.  Both therefore produce
// bitwise identical results.
//
// Memory model.  Each XCD of the chip has its own L2 and the L2s are not kept
// coherent with each other, so data handed from one workgroup to another
// (activations, attention partials, counters, the freshly appended KV slot)
// is written and read with device-scope (sc1) accesses, which go to the
// memory side.  Weights and the RoPE table never change while a kernel runs
// and are read with streaming (nt) loads.  A workgroup waits for its own
// stores (s_waitcnt) before announcing completion.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace mbk {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Per-launch parameters (kernel argument, passed by value).
struct Params {
    const uint8_t *blob;      // packed weights + RoPE table + interval table
    const Interval *iv;       // interval table (inside blob)
    uint16_t *kv;             // [NL][2][nkv][S][hd] bf16
    uint8_t *ws;              // workspace
    WsLayout wl;
    float *logits;            // [V] or null
    int32_t *argmax_out;      // device int32
    const float *rope;        // [S][hd/2][2] (cos, sin)
    MatGeom embed;            // packed tied embedding / LM head
    uint64_t final_norm_off;
    int32_t n_wg, n_intervals;
    int32_t H, nq, nkv, hd, I, V, S, NL;
    int32_t max_splits, gqa;
    float eps, scale;         // RMSNorm eps, 1/sqrt(head_dim)
    int32_t token, pos;       // token < 0: previous device argmax
    int32_t step_from_ws;     // 1: read token/pos from the workspace (graph replay)
    uint32_t epoch_base;      // grid barriers completed on this workspace before the call
    int32_t spin_limit, skip_wg, skip_interval;
    int32_t first_iv, last_iv;
};

#define MBK_DEV __device__ __forceinline__

// ---- access helpers ------------------------------------------------------------------------------

MBK_DEV float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
MBK_DEV float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
MBK_DEV float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN).
MBK_DEV uint16_t to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu)) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

MBK_DEV u32x4 ld_stream(const uint8_t *p) { return __builtin_nontemporal_load((const u32x4 *)p); }

MBK_DEV float ldc(const float *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MBK_DEV void stc(float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MBK_DEV uint32_t ldc_u(const uint32_t *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MBK_DEV void stc_u(uint32_t *p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MBK_DEV uint32_t atom_add(uint32_t *p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

MBK_DEV auto rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
}
// 16-byte device-coherent load (sc1) at byte offset off from base.
MBK_DEV u32x4 ldc16(const void *base, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(rsrc(base), off, 0, 16);
}
MBK_DEV void stc16(void *base, uint32_t off, u32x4 v) { __builtin_amdgcn_raw_buffer_store_b128(v, rsrc(base), off, 0, 16); }
MBK_DEV void stc_b16(void *base, uint32_t off, uint16_t v) {
    __builtin_amdgcn_raw_buffer_store_b16((short)v, rsrc(base), off, 0, 16);
}

template <class T> MBK_DEV T *ws_ptr(const Params &p, uint64_t off) { return (T *)(p.ws + off); }

MBK_DEV uint32_t ord_key(float f) {
    uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// ---- grid barrier ---------------------------------------------------------------------------------
// Counting barrier with a monotonically growing arrival count (the pages'
// counting_grid_barrier: one add per block, then wait until the count
// reaches (ordinal + 1) * workers), arranged in two levels so the adds are
// spread over 8 counters: workgroup w adds to the counter of group w % 8; the
// last arrival of a group adds to the global counter, waits for all groups
// and then publishes the epoch on its group's release word, which the other
// members poll.  Every wait is bounded; on expiry the error word is set and
// the caller stops.

MBK_DEV bool spin_until(const uint32_t *p, uint32_t target, int limit) {
    for (int it = 0; (int32_t)(ldc_u(p) - target) < 0; ++it)
        if (it >= limit) return false;
    return true;
}

MBK_DEV bool grid_barrier(const Params &p, uint32_t epoch, int ivi) {
    __shared__ int ok_s;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's stores are complete
    __syncthreads();
    if (threadIdx.x == 0) {
        const int w = blockIdx.x, grp = w % kGroups;
        const int ngroups = p.n_wg < kGroups ? p.n_wg : kGroups;
        const uint32_t members = (uint32_t)((p.n_wg - grp + kGroups - 1) / kGroups);
        uint32_t *cnt = ws_ptr<uint32_t>(p, p.wl.bar_group + 256u * grp);
        uint32_t *rel = ws_ptr<uint32_t>(p, p.wl.bar_rel + 256u * grp);
        uint32_t *glob = ws_ptr<uint32_t>(p, p.wl.bar_global);
        bool ok;
        if (w == p.skip_wg && ivi == p.skip_interval) {
            ok = spin_until(rel, epoch, p.spin_limit);  // never arrives: the group waits in vain
        } else {
            uint32_t old = atom_add(cnt, 1u);
            if (old == epoch * members - 1u) {
                atom_add(glob, 1u);
                ok = spin_until(glob, epoch * (uint32_t)ngroups, p.spin_limit);
                if (ok) stc_u(rel, epoch);
            } else {
                ok = spin_until(rel, epoch, p.spin_limit);
            }
        }
        if (!ok) stc_u(ws_ptr<uint32_t>(p, p.wl.ctrl), 1u);
        ok_s = ok;
    }
    __syncthreads();
    return ok_s != 0;
}

// ---- reductions ----------------------------------------------------------------------------------

MBK_DEV float wave_sum(float v) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) v += __shfl_xor(v, m);
    return v;
}

// Sum over the workgroup in a fixed order; every thread gets the result.
MBK_DEV float block_sum(float v, float *red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) s += red[i];
    return s;
}

// ---- input vectors ---------------------------------------------------------------------------------

MBK_DEV int step_token(const Params &p) {
    int t = p.step_from_ws ? (int)ldc_u(ws_ptr<uint32_t>(p, p.wl.ctrl) + 3) : p.token;
    if (t < 0) t = (int)ldc_u(ws_ptr<uint32_t>(p, p.wl.ctrl) + 1);
    return t;
}
MBK_DEV int step_pos(const Params &p) {
    return p.step_from_ws ? (int)ldc_u(ws_ptr<uint32_t>(p, p.wl.ctrl) + 4) : p.pos;
}

// Element r of the embedding row of `token` (bf16 -> fp32), read from the packed LM head.
MBK_DEV float embed_elem(const Params &p, int token, int r) {
    const uint8_t *c = p.blob + row_group_offset(p.embed, token, r >> 3);
    return bf16f(((const uint16_t *)c)[r & 7]);
}

// xs[0..K) <- residual stream (embedding row of `token` for layer 0), optionally
// RMS-normalised with the bf16 weight at blob offset norm_off.
MBK_DEV void load_residual(const Params &p, float *xs, float *red, bool from_embed, int token, uint64_t norm_off) {
    const int K = p.H;
    float ss = 0.f;
    if (from_embed) {
        for (int g = threadIdx.x; g < K / 8; g += kThreads) {
            u32x4 w = *(const u32x4 *)(p.blob + row_group_offset(p.embed, token, g));
            float v[8] = {bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y), bf_lo(w.z), bf_hi(w.z), bf_lo(w.w), bf_hi(w.w)};
#pragma unroll
            for (int e = 0; e < 8; ++e) { xs[g * 8 + e] = v[e]; ss += v[e] * v[e]; }
        }
    } else {
        for (int g = threadIdx.x; g < K / 4; g += kThreads) {
            u32x4 w = ldc16(p.ws, (uint32_t)(p.wl.x + 16u * g));
            float v[4] = {__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w)};
#pragma unroll
            for (int e = 0; e < 4; ++e) { xs[g * 4 + e] = v[e]; ss += v[e] * v[e]; }
        }
    }
    if (norm_off != ~(uint64_t)0) {
        float tot = block_sum(ss, red);  // contains the barrier that makes xs visible
        float r = rsqrtf(tot / (float)K + p.eps);
        const uint16_t *nw = (const uint16_t *)(p.blob + norm_off);
        for (int k = threadIdx.x; k < K; k += kThreads) xs[k] = xs[k] * r * bf16f(nw[k]);
    }
    __syncthreads();
}

// xs[0..K) <- fp32 workspace vector at byte offset off.
MBK_DEV void load_vec(const Params &p, float *xs, uint64_t off, int K) {
    for (int g = threadIdx.x; g < K / 4; g += kThreads) {
        u32x4 w = ldc16(p.ws, (uint32_t)(off + 16u * g));
        *(u32x4 *)(xs + 4 * g) = w;
    }
    __syncthreads();
}

// ---- GEMV ------------------------------------------------------------------------------------------
// Dot products of the RT rows of packed tile t with xs (fp32 in LDS).  Lane l
// covers row l / L and input groups (l % L) + it * L; the row sum is reduced
// over its L lanes, so every lane of the row ends up holding it.
MBK_DEV float gemv_tile(const uint8_t *blob, const MatGeom &g, int64_t t, const float *xs, int lane) {
    const int L = g.L, IT = g.IT, kl = lane & (L - 1);
    const uint8_t *base = blob + chunk_offset(g, t, 0, lane);
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    for (int it0 = 0; it0 < IT; it0 += 8) {
        u32x4 w[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (it0 + u < IT) w[u] = ld_stream(base + (size_t)(it0 + u) * 1024u);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (it0 + u < IT) {
                const float *xv = xs + (kl + (it0 + u) * L) * 8;
                const float4 xa = *(const float4 *)xv, xb = *(const float4 *)(xv + 4);
                a0 = fmaf(bf_lo(w[u].x), xa.x, a0);
                a1 = fmaf(bf_hi(w[u].x), xa.y, a1);
                a2 = fmaf(bf_lo(w[u].y), xa.z, a2);
                a3 = fmaf(bf_hi(w[u].y), xa.w, a3);
                a0 = fmaf(bf_lo(w[u].z), xb.x, a0);
                a1 = fmaf(bf_hi(w[u].z), xb.y, a1);
                a2 = fmaf(bf_lo(w[u].w), xb.z, a2);
                a3 = fmaf(bf_hi(w[u].w), xb.w, a3);
            }
        }
    }
    float acc = (a0 + a1) + (a2 + a3);
    for (int m = 1; m < L; m <<= 1) acc += __shfl_xor(acc, m);
    return acc;
}

// Runs fn(tile, row_sum, lane) for every tile of the interval owned by this
// workgroup: item i goes to workgroup (i + rot) % n_wg, and the workgroup's
// items are dealt to its waves in turn.
template <class Fn>
MBK_DEV void for_my_tiles(const Params &p, const Interval &iv, const float *xs, Fn &&fn) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwg = p.n_wg;
    const int first = (int)((blockIdx.x + (uint32_t)nwg - (uint32_t)(iv.rot % nwg)) % (uint32_t)nwg);
    for (int64_t t = first + (int64_t)wave * nwg; t < iv.n_items; t += (int64_t)kWaves * nwg) {
        float y = gemv_tile(p.blob, iv.mat, t, xs, lane);
        fn(t, y, lane);
    }
}

// ---- operators -------------------------------------------------------------------------------------

// Q/K/V projection (+bias), RoPE on query/key pairs, KV append.
MBK_DEV void op_qkv(const Params &p, const Interval &iv, float *xs, float *red) {
    const int token = iv.layer == 0 ? step_token(p) : 0, pos = step_pos(p);
    load_residual(p, xs, red, iv.layer == 0, token, iv.norm_off);
    const int hd = p.hd, Q = p.nq * hd, KVr = p.nkv * hd, half = hd / 2;
    const MatGeom &g = iv.mat;
    const uint16_t *bias = iv.bias_off != ~(uint64_t)0 ? (const uint16_t *)(p.blob + iv.bias_off) : nullptr;
    const float2 *rope = (const float2 *)p.rope + (size_t)pos * half;
    float *q = ws_ptr<float>(p, p.wl.q);
    uint16_t *kc = p.kv + ((size_t)iv.layer * 2 + 0) * p.nkv * p.S * hd;
    uint16_t *vc = p.kv + ((size_t)iv.layer * 2 + 1) * p.nkv * p.S * hd;
    for_my_tiles(p, iv, xs, [&](int64_t t, float y, int lane) {
        const float partner = __shfl_xor(y, g.L);
        if ((lane & (g.L - 1)) != 0) return;
        const int rr = lane / g.L, prow = (int)(t * g.RT) + rr;
        if (prow >= g.rows) return;
        RowSrc s = packed_row_source(MAT_QKV, prow, hd, Q, KVr);
        if (s.which == 2) {  // value row: its own epilogue
            float v = y + (bias ? bf16f(bias[Q + KVr + s.row]) : 0.f);
            const int j = s.row / hd, d = s.row % hd;
            stc_b16(vc, (uint32_t)((((size_t)j * p.S + pos) * hd + d) * 2u), to_bf16(v));
            return;
        }
        if (rr & 1) return;  // odd rows are the partner of the pair handled below
        const int boff = s.which == 0 ? 0 : Q;
        const int h = s.row / hd, m = s.row % hd;  // m < hd/2
        float u = y, w = partner;
        if (bias) { u += bf16f(bias[boff + s.row]); w += bf16f(bias[boff + s.row + half]); }
        const float2 cs = rope[m];
        const float r0 = u * cs.x - w * cs.y, r1 = w * cs.x + u * cs.y;
        if (s.which == 0) {
            stc(q + h * hd + m, r0);
            stc(q + h * hd + m + half, r1);
        } else {
            const size_t base = ((size_t)h * p.S + pos) * hd;
            stc_b16(kc, (uint32_t)((base + m) * 2u), to_bf16(r0));
            stc_b16(kc, (uint32_t)((base + m + half) * 2u), to_bf16(r1));
        }
    });
}

// x += W_o o (residual add in the epilogue).
MBK_DEV void op_o(const Params &p, const Interval &iv, float *xs) {
    load_vec(p, xs, p.wl.o, p.nq * p.hd);
    const int token = iv.layer == 0 ? step_token(p) : 0;
    float *x = ws_ptr<float>(p, p.wl.x);
    const MatGeom &g = iv.mat;
    const bool first = iv.layer == 0;
    for_my_tiles(p, iv, xs, [&](int64_t t, float y, int lane) {
        if ((lane & (g.L - 1)) != 0) return;
        const int r = (int)(t * g.RT) + lane / g.L;
        if (r >= g.rows) return;
        const float xin = first ? embed_elem(p, token, r) : ldc(x + r);
        stc(x + r, xin + y);
    });
}

// a = silu(W_gate xn) * (W_up xn), xn = RMSNorm(x).
MBK_DEV void op_gateup(const Params &p, const Interval &iv, float *xs, float *red) {
    load_residual(p, xs, red, false, 0, iv.norm_off);
    float *a = ws_ptr<float>(p, p.wl.a);
    const MatGeom &g = iv.mat;
    for_my_tiles(p, iv, xs, [&](int64_t t, float y, int lane) {
        const float up = __shfl_xor(y, g.L);
        if ((lane & (g.L - 1)) != 0) return;
        const int rr = lane / g.L, prow = (int)(t * g.RT) + rr;
        if ((rr & 1) || prow >= g.rows) return;
        const float gt = y;
        stc(a + (prow >> 1), gt / (1.f + __expf(-gt)) * up);
    });
}

// x += W_down a.
MBK_DEV void op_down(const Params &p, const Interval &iv, float *xs) {
    load_vec(p, xs, p.wl.a, p.I);
    float *x = ws_ptr<float>(p, p.wl.x);
    const MatGeom &g = iv.mat;
    for_my_tiles(p, iv, xs, [&](int64_t t, float y, int lane) {
        if ((lane & (g.L - 1)) != 0) return;
        const int r = (int)(t * g.RT) + lane / g.L;
        if (r >= g.rows) return;
        stc(x + r, ldc(x + r) + y);
    });
}

// logits = E RMSNorm(x); greedy argmax through one 64-bit atomic max per
// workgroup; the last workgroup to finish publishes the index.
MBK_DEV void op_lmhead(const Params &p, const Interval &iv, float *xs, float *red) {
    load_residual(p, xs, red, false, 0, iv.norm_off);
    const MatGeom &g = iv.mat;
    uint64_t best = 0;
    for_my_tiles(p, iv, xs, [&](int64_t t, float y, int lane) {
        if ((lane & (g.L - 1)) != 0) return;
        const int r = (int)(t * g.RT) + lane / g.L;
        if (r >= g.rows) return;
        if (p.logits) p.logits[r] = y;
        const uint64_t key = ((uint64_t)ord_key(y) << 32) | (uint64_t)(0xffffffffu - (uint32_t)r);
        best = key > best ? key : best;
    });
    // workgroup max
    for (int m = 1; m < 64; m <<= 1) {
        uint64_t o = ((uint64_t)__shfl_xor((uint32_t)(best >> 32), m) << 32) | __shfl_xor((uint32_t)best, m);
        best = o > best ? o : best;
    }
    __shared__ uint64_t wbest[kWaves];
    if ((threadIdx.x & 63) == 0) wbest[threadIdx.x >> 6] = best;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 0; i < kWaves; ++i) best = wbest[i] > best ? wbest[i] : best;
        uint64_t *key = ws_ptr<uint64_t>(p, p.wl.argkey);
        if (best) __hip_atomic_fetch_max(key, best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        uint32_t *ctrl = ws_ptr<uint32_t>(p, p.wl.ctrl);
        if (atom_add(ctrl + 2, 1u) == (uint32_t)p.n_wg - 1u) {
            const uint64_t k = __hip_atomic_load(key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const int32_t idx = (int32_t)(0xffffffffu - (uint32_t)k);
            p.argmax_out[0] = idx;
            stc_u(ctrl + 1, (uint32_t)idx);
            stc_u(ctrl + 2, 0u);
        }
    }
}

// ---- attention ---------------------------------------------------------------------------------------
// Decode attention for KV head j over cached positions [t0, t1), the G query
// heads of the group packed together so each key and value is read once
// (README mirror, "Current status": flash decoding, query heads sharing a KV
// head packed at long context).  LP = hd/8 lanes share one position; a wave
// covers 64/LP positions per step.  Online softmax per lane group, then a
// log-sum-exp merge across lane groups (shuffles) and across waves (LDS).
// Result: per head (m, l, acc[hd]) in LDS `out` ([G][hd + 4] floats).

MBK_DEV void lse_merge(float &m, float &l, float *acc, float m2, float l2, const float *acc2, int n) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;
    const float c1 = __expf(m - mn), c2 = __expf(m2 - mn);
    l = l * c1 + l2 * c2;
    for (int e = 0; e < n; ++e) acc[e] = acc[e] * c1 + acc2[e] * c2;
    m = mn;
}

template <int G>
MBK_DEV void attend_range(const Params &p, int layer, int j, int t0, int t1, float *out) {
    const int hd = p.hd, LP = hd / 8, PPW = 64 / LP;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int slot = lane / LP, dl = lane % LP;
    const float *q = ws_ptr<float>(p, p.wl.q);
    float qf[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        u32x4 a = ldc16(p.ws, (uint32_t)(p.wl.q + ((size_t)(j * G + h) * hd + dl * 8) * 4u));
        u32x4 b = ldc16(p.ws, (uint32_t)(p.wl.q + ((size_t)(j * G + h) * hd + dl * 8 + 4) * 4u));
        qf[h][0] = __uint_as_float(a.x) * p.scale; qf[h][1] = __uint_as_float(a.y) * p.scale;
        qf[h][2] = __uint_as_float(a.z) * p.scale; qf[h][3] = __uint_as_float(a.w) * p.scale;
        qf[h][4] = __uint_as_float(b.x) * p.scale; qf[h][5] = __uint_as_float(b.y) * p.scale;
        qf[h][6] = __uint_as_float(b.z) * p.scale; qf[h][7] = __uint_as_float(b.w) * p.scale;
    }
    (void)q;
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY; l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }
    const uint16_t *Kb = p.kv + (((size_t)layer * 2 + 0) * p.nkv + j) * p.S * hd;
    const uint16_t *Vb = p.kv + (((size_t)layer * 2 + 1) * p.nkv + j) * p.S * hd;
    for (int base = t0 + wave * PPW; base < t1; base += kWaves * PPW) {
        const int t = base + slot;
        const bool valid = t < t1;
        u32x4 kw = {0, 0, 0, 0}, vw = {0, 0, 0, 0};
        if (valid) {
            kw = ldc16(Kb, (uint32_t)(((size_t)t * hd + dl * 8) * 2u));
            vw = ldc16(Vb, (uint32_t)(((size_t)t * hd + dl * 8) * 2u));
        }
        const float kf[8] = {bf_lo(kw.x), bf_hi(kw.x), bf_lo(kw.y), bf_hi(kw.y), bf_lo(kw.z), bf_hi(kw.z), bf_lo(kw.w), bf_hi(kw.w)};
        const float vf[8] = {bf_lo(vw.x), bf_hi(vw.x), bf_lo(vw.y), bf_hi(vw.y), bf_lo(vw.z), bf_hi(vw.z), bf_lo(vw.w), bf_hi(vw.w)};
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float d = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) d = fmaf(qf[h][e], kf[e], d);
            for (int msk = 1; msk < LP; msk <<= 1) d += __shfl_xor(d, msk);
            if (valid) {
                const float mn = fmaxf(m[h], d);
                const float c = __expf(m[h] - mn), pw = __expf(d - mn);
                l[h] = l[h] * c + pw;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pw, vf[e], acc[h][e] * c);
                m[h] = mn;
            }
        }
    }
    // merge the position slots of this wave
    for (int msk = LP; msk < 64; msk <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float a2[8];
            const float m2 = __shfl_xor(m[h], msk), l2 = __shfl_xor(l[h], msk);
#pragma unroll
            for (int e = 0; e < 8; ++e) a2[e] = __shfl_xor(acc[h][e], msk);
            lse_merge(m[h], l[h], acc[h], m2, l2, a2, 8);
        }
    }
    // merge the waves through LDS: scratch [wave][G][hd + 4]
    float *scr = out + G * (hd + 4);
    const int stride = hd + 4;
    if (slot == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float *r = scr + ((size_t)wave * G + h) * stride;
            if (dl == 0) { r[0] = m[h]; r[1] = l[h]; }
#pragma unroll
            for (int e = 0; e < 8; ++e) r[4 + dl * 8 + e] = acc[h][e];
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * hd; idx += kThreads) {
        const int h = idx / hd, e = idx % hd;
        float mm = -INFINITY, ll = 0.f, aa = 0.f;
        for (int w = 0; w < kWaves; ++w) {
            const float *r = scr + ((size_t)w * G + h) * stride;
            lse_merge(mm, ll, &aa, r[0], r[1], &r[4 + e], 1);
        }
        float *o = out + (size_t)h * stride;
        if (e == 0) { o[0] = mm; o[1] = ll; }
        o[4 + e] = aa;
    }
    __syncthreads();
}

// One attention item: KV head j, split s of the cached context.  A single
// split writes o directly; with several, each split stores its partial and
// the last split to arrive (one atomic per split) merges all partials in
// split order, so the result does not depend on arrival order.
template <int G>
MBK_DEV void attention_item(const Params &p, int layer, int j, int s, float *lds) {
    const int pos = step_pos(p), Lc = pos + 1, hd = p.hd, stride = hd + 4;
    int chunk = (Lc + p.max_splits - 1) / p.max_splits;
    if (chunk < kAttnMinChunk) chunk = kAttnMinChunk;
    const int nsplit = (Lc + chunk - 1) / chunk;
    if (s >= nsplit) return;
    const int t0 = s * chunk, t1 = min(Lc, t0 + chunk);
    float *res = lds;  // [G][stride]
    attend_range<G>(p, layer, j, t0, t1, res);
    float *o = ws_ptr<float>(p, p.wl.o);
    if (nsplit == 1) {
        for (int idx = threadIdx.x; idx < G * hd; idx += kThreads) {
            const int h = idx / hd, e = idx % hd;
            const float *r = res + (size_t)h * stride;
            stc(o + (size_t)(j * G + h) * hd + e, r[4 + e] / r[1]);
        }
        return;
    }
    // store this split's partial: part[j][s][h][stride]
    const uint64_t pbase = p.wl.part + ((uint64_t)(j * p.max_splits + s) * G) * stride * 4u;
    for (int idx = threadIdx.x; idx < G * stride / 4; idx += kThreads)
        stc16(p.ws, (uint32_t)(pbase + 16u * idx), *(const u32x4 *)(res + 4 * idx));
    __shared__ int last_s;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t *cnt = ws_ptr<uint32_t>(p, p.wl.merge_cnt + 256u * j);
        const bool last = atom_add(cnt, 1u) == (uint32_t)nsplit - 1u;
        if (last) stc_u(cnt, 0u);
        last_s = last;
    }
    __syncthreads();
    if (!last_s) return;
    // load every partial of head group j into LDS, then merge in split order
    float *all = lds;  // [nsplit][G][stride]
    const uint64_t gbase = p.wl.part + ((uint64_t)(j * p.max_splits) * G) * stride * 4u;
    const int n16 = nsplit * G * stride / 4;
    for (int idx = threadIdx.x; idx < n16; idx += kThreads)
        *(u32x4 *)(all + 4 * idx) = ldc16(p.ws, (uint32_t)(gbase + 16u * idx));
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * hd; idx += kThreads) {
        const int h = idx / hd, e = idx % hd;
        float mm = -INFINITY, ll = 0.f, aa = 0.f;
        for (int q = 0; q < nsplit; ++q) {
            const float *r = all + ((size_t)q * G + h) * stride;
            lse_merge(mm, ll, &aa, r[0], r[1], &r[4 + e], 1);
        }
        stc(o + (size_t)(j * G + h) * hd + e, aa / ll);
    }
}

MBK_DEV void op_attention(const Params &p, const Interval &iv, float *lds) {
    const int nwg = p.n_wg;
    const int first = (int)((blockIdx.x + (uint32_t)nwg - (uint32_t)(iv.rot % nwg)) % (uint32_t)nwg);
    for (int i = first; i < iv.n_items; i += nwg) {
        const int j = i / p.max_splits, s = i % p.max_splits;
        switch (p.gqa) {
            case 1: attention_item<1>(p, iv.layer, j, s, lds); break;
            case 2: attention_item<2>(p, iv.layer, j, s, lds); break;
            case 3: attention_item<3>(p, iv.layer, j, s, lds); break;
            case 4: attention_item<4>(p, iv.layer, j, s, lds); break;
            case 5: attention_item<5>(p, iv.layer, j, s, lds); break;
            case 6: attention_item<6>(p, iv.layer, j, s, lds); break;
            case 7: attention_item<7>(p, iv.layer, j, s, lds); break;
            default: attention_item<8>(p, iv.layer, j, s, lds); break;
        }
        __syncthreads();
    }
}

// ---- interval dispatch -------------------------------------------------------------------------------

MBK_DEV void run_interval(const Params &p, int ivi, float *lds, float *red) {
    const Interval iv = p.iv[ivi];
    if (ivi == 0 && blockIdx.x == 0 && threadIdx.x == 0) {
        __hip_atomic_store(ws_ptr<uint64_t>(p, p.wl.argkey), (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!p.step_from_ws) {  // publish this step's token/pos for launches that read them from the workspace
            uint32_t *ctrl = ws_ptr<uint32_t>(p, p.wl.ctrl);
            stc_u(ctrl + 3, (uint32_t)p.token);
            stc_u(ctrl + 4, (uint32_t)p.pos);
        }
    }
    switch (iv.op) {
        case OP_QKV: op_qkv(p, iv, lds, red); break;
        case OP_ATTN: op_attention(p, iv, lds); break;
        case OP_O: op_o(p, iv, lds); break;
        case OP_GATEUP: op_gateup(p, iv, lds, red); break;
        case OP_DOWN: op_down(p, iv, lds); break;
        case OP_LMHEAD: op_lmhead(p, iv, lds, red); break;
        default: break;
    }
}

}  // namespace mbk
