// bodies.h -- device bodies of the decode step (gfx950, wave64).
//
// Every body is a __device__ function run by one workgroup; the persistent
// kernel calls them in task-list order, the ablation kernel calls one
// interval per launch.  All executors produce bitwise identical results.
//
// Data exchange.  Each XCD of the chip has its own L2 and the L2s are not
// kept coherent with each other, so data handed from one workgroup to another
// goes through the memory side with device-scope (sc1) accesses.  Every
// activation vector handed between intervals (residual stream, queries, this
// step's keys and values, attention output, SwiGLU activations) is a vector of
// 8-byte entries {fp32 value, u32 tag} written with one 64-bit store; the tag
// names the (step, interval) that produced the value.  A reader polls the
// entries it needs until they carry the tag it expects, so data and
// completion arrive together: an interval's inputs cost one memory round trip
// after the producer's store, with no store drain and no grid barrier (the
// MegaBake article's roadmap, "Checking the 5.5x": per-phase event counters
// instead of grid barriers).  A counting grid barrier between intervals is
// kept as a mode.
//
// Reuse of a buffer is safe because of the data dependencies alone: a vector
// is overwritten only by an interval that (transitively) consumed every
// output of all readers of the previous version.  The residual stream is the
// one vector that is read and rewritten by the same operator (output and
// down projections add into it), so each workgroup reads only the residual
// rows it rewrites itself.
//
// Latency hiding.  While waves 0-1 poll an interval's inputs, waves 2-3 copy
// the NEXT interval's weight tiles (or the keys and values already in the
// cache) into one of two LDS staging buffers -- weight streaming across
// intervals (the article's prefetch of the next GEMM's weights while a block
// waits).  Tiles that do not fit stream from HBM through two register
// buffers used in turn.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace mbk {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kKvB = 4;        // attention: positions per lane per block (2 for G >= 5, see kv_batch)
constexpr int kPollWaves = 2;  // waves that poll an interval's inputs; the others stage the next interval
constexpr int kCh = 8;         // GEMV chunk: 16-byte loads per lane streamed from HBM at a time

// Positions per lane per attention block: fewer for large query groups, whose
// per-head state already takes most of the registers.
template <int G> constexpr int kv_batch() { return G >= 5 ? 2 : kKvB; }

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
    uint64_t *trace;          // phase timer [n_intervals][n_wg][4] or null
    MatGeom embed;            // packed tied embedding / LM head
    int32_t n_wg, n_intervals;
    int32_t H, nq, nkv, hd, I, V, S, NL;
    int32_t max_splits, gqa, attn_min_chunk;
    int32_t lds_tab, lds_rope, lds_xs, lds_xres, lds_bias, lds_ys, lds_pf;  // LDS offsets (floats)
    int32_t pf_bytes;         // size of ONE of the two LDS staging buffers
    float eps, scale;         // RMSNorm eps, 1/sqrt(head_dim)
    int32_t token, pos;       // token < 0: previous device argmax
    uint32_t seq;             // step number: tags of this step's activations
    int32_t step_from_ws;     // 1: read token/pos/seq from the workspace (graph replay)
    int32_t barrier;          // 1: counting grid barrier between intervals
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

MBK_DEV uint32_t ldc_u(const uint32_t *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MBK_DEV void stc_u(uint32_t *p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MBK_DEV uint32_t atom_add(uint32_t *p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

MBK_DEV auto rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
}
// 16-byte device-coherent load / store (sc1) at byte offset off from base.
MBK_DEV u32x4 ldc16(const void *base, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(rsrc(base), off, 0, 16); }
MBK_DEV void stc16(void *base, uint32_t off, u32x4 v) { __builtin_amdgcn_raw_buffer_store_b128(v, rsrc(base), off, 0, 16); }
MBK_DEV void stc_b16(void *base, uint32_t off, uint16_t v) {
    __builtin_amdgcn_raw_buffer_store_b16((short)v, rsrc(base), off, 0, 16);
}

template <class T> MBK_DEV T *ws_ptr(const Params &p, uint64_t off) { return (T *)(p.ws + off); }

MBK_DEV uint32_t ord_key(float f) {
    uint32_t b = __float_as_uint(f);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Phase timer: thread 0 of every workgroup stamps the device wall clock.
MBK_DEV void stamp(const Params &p, int ivi, int k) {
    if (p.trace && threadIdx.x == 0 && ivi >= 0)
        p.trace[((size_t)ivi * p.n_wg + blockIdx.x) * 4 + k] = wall_clock64();
}

// Error word: set when a bounded wait expires; every wait gives up soon after.
MBK_DEV void set_error(const Params &p) { stc_u(ws_ptr<uint32_t>(p, p.wl.ctrl), 1u); }
MBK_DEV bool aborted(const Params &p, int it) {
    return (it & 255) == 255 && ldc_u(ws_ptr<uint32_t>(p, p.wl.ctrl)) != 0u;
}

// ---- tagged activations --------------------------------------------------------------------------

MBK_DEV uint32_t step_seq(const Params &p) {
    return p.step_from_ws ? ldc_u(ws_ptr<uint32_t>(p, p.wl.ctrl) + 5) : p.seq;
}

// Tag of what interval ivi writes during step seq.  Nonzero (a zeroed
// workspace never matches) as the host keeps seq * n_intervals in range.
MBK_DEV uint32_t tag_of(const Params &p, uint32_t seq, int ivi) {
    return seq * (uint32_t)p.n_intervals + (uint32_t)ivi + 1u;
}

MBK_DEV void put(const Params &p, uint64_t base, int i, float v, uint32_t tag) {
    __hip_atomic_store(ws_ptr<uint64_t>(p, base) + i, ((uint64_t)tag << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// v[0..8) <- entries 8g..8g+7 of the tagged vector at base, once all of them
// carry `tag`.  Bounded: false when the wait expires or another wait did.
MBK_DEV bool poll8(const Params &p, uint64_t base, int g, uint32_t tag, float *v) {
    const uint32_t off = (uint32_t)(base + 64u * (uint32_t)g);
    for (int it = 0;; ++it) {
        const u32x4 a = ldc16(p.ws, off), b = ldc16(p.ws, off + 16u), c = ldc16(p.ws, off + 32u),
                    d = ldc16(p.ws, off + 48u);
        if (a.y == tag && a.w == tag && b.y == tag && b.w == tag && c.y == tag && c.w == tag && d.y == tag &&
            d.w == tag) {
            v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.z);
            v[2] = __uint_as_float(b.x); v[3] = __uint_as_float(b.z);
            v[4] = __uint_as_float(c.x); v[5] = __uint_as_float(c.z);
            v[6] = __uint_as_float(d.x); v[7] = __uint_as_float(d.z);
            return true;
        }
        if (it >= p.spin_limit) { set_error(p); return false; }
        if (aborted(p, it)) return false;
    }
}

// One entry of a tagged vector.
MBK_DEV bool poll1(const Params &p, uint64_t base, int i, uint32_t tag, float &v) {
    const uint64_t *e = ws_ptr<uint64_t>(p, base) + i;
    for (int it = 0;; ++it) {
        const uint64_t w = __hip_atomic_load(e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((uint32_t)(w >> 32) == tag) {
            v = __uint_as_float((uint32_t)w);
            return true;
        }
        if (it >= p.spin_limit) { set_error(p); return false; }
        if (aborted(p, it)) return false;
    }
}

// ---- grid barrier (barrier mode) -----------------------------------------------------------------
// Counting barrier with a monotonically growing arrival count (the pages'
// counting_grid_barrier: one add per block, then wait until the count
// reaches (ordinal + 1) * workers), arranged in two levels so the adds are
// spread over 8 counters: workgroup w adds to the counter of group w % 8; the
// last arrival of a group adds to the global counter, waits for all groups
// and then publishes the epoch on its group's release word, which the other
// members poll.  Every wait is bounded; on expiry the error word is set and
// the caller stops.

MBK_DEV bool spin_until(const Params &p, const uint32_t *w, uint32_t target) {
    for (int it = 0; (int32_t)(ldc_u(w) - target) < 0; ++it) {
        if (it >= p.spin_limit) { set_error(p); return false; }
        if (aborted(p, it)) return false;
    }
    return true;
}

// Arrival: every wave's stores must be complete first (on gfx9 loads and
// stores share one counter, so this also drains outstanding loads; staging
// of the next interval is therefore issued between arrival and waiting).
// Returns 1 in thread 0 when this workgroup arrived last in its group.
MBK_DEV int barrier_arrive(const Params &p, uint32_t epoch) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int last = 0;
    if (threadIdx.x == 0) {
        const int grp = blockIdx.x % kGroups;
        const uint32_t members = (uint32_t)((p.n_wg - grp + kGroups - 1) / kGroups);
        const uint32_t old = atom_add(ws_ptr<uint32_t>(p, p.wl.bar_group + 256u * grp), 1u);
        if (old == epoch * members - 1u) {
            atom_add(ws_ptr<uint32_t>(p, p.wl.bar_global), 1u);
            last = 1;
        }
    }
    return last;
}

// Wait (thread 0 spins, the workgroup joins at the end).  False on expiry.
MBK_DEV bool barrier_wait(const Params &p, uint32_t epoch, int last) {
    __shared__ int ok_s;
    if (threadIdx.x == 0) {
        const int grp = blockIdx.x % kGroups;
        const int ngroups = p.n_wg < kGroups ? p.n_wg : kGroups;
        uint32_t *rel = ws_ptr<uint32_t>(p, p.wl.bar_rel + 256u * grp);
        bool ok;
        if (last) {
            ok = spin_until(p, ws_ptr<uint32_t>(p, p.wl.bar_global), epoch * (uint32_t)ngroups);
            if (ok) stc_u(rel, epoch);
        } else {
            ok = spin_until(p, rel, epoch);
        }
        ok_s = ok;
    }
    __syncthreads();
    return ok_s != 0;
}

MBK_DEV bool grid_barrier(const Params &p, uint32_t epoch) { return barrier_wait(p, epoch, barrier_arrive(p, epoch)); }

// ---- reductions ----------------------------------------------------------------------------------
// Butterfly sums over groups of N consecutive lanes.  Steps inside 16 lanes
// use DPP moves: after the xor-1 and xor-2 steps every quad is uniform, so a
// half-row mirror (lane i <-> 7-i) pairs quad 0 with quad 1, and after that a
// row mirror (i <-> 15-i) pairs the two halves of a 16-lane row.  The 16- and
// 32-lane steps go through the LDS crossbar.

template <int CTRL> MBK_DEV float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

template <int N> MBK_DEV float group_sum(float v) {
    if constexpr (N >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (N >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (N >= 8) v += dpp<0x141>(v);   // row_half_mirror
    if constexpr (N >= 16) v += dpp<0x140>(v);  // row_mirror
    if constexpr (N >= 32) v += __shfl_xor(v, 16);
    if constexpr (N >= 64) v += __shfl_xor(v, 32);
    return v;
}

MBK_DEV float group_sum_n(float v, int n) {
    switch (n) {
        case 1: return v;
        case 2: return group_sum<2>(v);
        case 4: return group_sum<4>(v);
        case 8: return group_sum<8>(v);
        case 16: return group_sum<16>(v);
        case 32: return group_sum<32>(v);
        default: return group_sum<64>(v);
    }
}

// ---- step inputs and item placement --------------------------------------------------------------

MBK_DEV int step_token(const Params &p) {
    int t = p.step_from_ws ? (int)ldc_u(ws_ptr<uint32_t>(p, p.wl.ctrl) + 3) : p.token;
    if (t < 0) t = (int)ldc_u(ws_ptr<uint32_t>(p, p.wl.ctrl) + 1);
    return t;
}
MBK_DEV int step_pos(const Params &p) {
    return p.step_from_ws ? (int)ldc_u(ws_ptr<uint32_t>(p, p.wl.ctrl) + 4) : p.pos;
}

// Items (GEMV tiles, attention splits) of an interval run on workgroups
// (i + rot) % n_wg; first_item is the lowest item index of this workgroup.
MBK_DEV int first_item(const Params &p, const Interval &iv) {
    const uint32_t nwg = (uint32_t)p.n_wg;
    return (int)((blockIdx.x + nwg - (uint32_t)(iv.rot % p.n_wg)) % nwg);
}

// Rounds (one tile per wave each) needed to cover the interval's tiles.
MBK_DEV int gemv_rounds(const Params &p, const Interval &iv) {
    return (iv.n_items + kWaves * p.n_wg - 1) / (kWaves * p.n_wg);
}

MBK_DEV uint8_t *staging(const Params &p, float *lds, int ivi) {
    return (uint8_t *)(lds + p.lds_pf) + (size_t)(ivi & 1) * (size_t)p.pf_bytes;
}

// ---- GEMV input vectors --------------------------------------------------------------------------
// GEMV input vectors live in LDS as bf16 pairs: each 8-element group g is 32
// bytes, [hi pairs | lo pairs] with hi = bf16(x), lo = bf16(x - hi), so that
// hi + lo carries ~17 significant bits and the bf16 dot-product instruction
// (fp32 accumulation) consumes weights and activations without conversions.

MBK_DEV uint32_t pack2(uint16_t a, uint16_t b) { return (uint32_t)a | ((uint32_t)b << 16); }

MBK_DEV void split8(const float *v, u32x4 &h, u32x4 &l) {
    uint16_t hb[8], lb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        hb[e] = to_bf16(v[e]);
        lb[e] = to_bf16(v[e] - bf16f(hb[e]));
    }
    h = (u32x4){pack2(hb[0], hb[1]), pack2(hb[2], hb[3]), pack2(hb[4], hb[5]), pack2(hb[6], hb[7])};
    l = (u32x4){pack2(lb[0], lb[1]), pack2(lb[2], lb[3]), pack2(lb[4], lb[5]), pack2(lb[6], lb[7])};
}

MBK_DEV void unpack8(const u32x4 &w, float *v) {
    v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
    v[4] = bf_lo(w.z); v[5] = bf_hi(w.z); v[6] = bf_lo(w.w); v[7] = bf_hi(w.w);
}

MBK_DEV void store8(float *dst, const float *v) {
    *(float4 *)dst = make_float4(v[0], v[1], v[2], v[3]);
    *(float4 *)(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Phase 1 of an RMS-normalised input (threads [tid, nt)): xs[8g..8g+8) <- v * w
// (fp32) for the residual stream v (tagged, or the embedding row of `token`)
// and the bf16 norm weight w; returns this thread's part of sum(v^2).
MBK_DEV float norm_phase1(const Params &p, float *xs, bool from_embed, int token, uint32_t tag, uint64_t norm_off,
                          int K, int tid, int nt, bool &ok) {
    float ss = 0.f;
    for (int g = tid; g < K / 8; g += nt) {
        float v[8], w[8];
        if (from_embed) unpack8(*(const u32x4 *)(p.blob + row_group_offset(p.embed, token, g)), v);
        else if (!poll8(p, p.wl.x, g, tag, v)) { ok = false; return 0.f; }
        unpack8(*(const u32x4 *)(p.blob + norm_off + 16u * g), w);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ss += v[e] * v[e];
            v[e] *= w[e];
        }
        store8(xs + 8 * g, v);
    }
    return ss;
}

// Phase 2 (all threads): scale by r and split into hi/lo pairs in place.
MBK_DEV void norm_phase2(float *xs, float r, int K) {
    for (int g = threadIdx.x; g < K / 8; g += kThreads) {
        float v[8];
        const float4 a = *(const float4 *)(xs + 8 * g), b = *(const float4 *)(xs + 8 * g + 4);
        v[0] = a.x * r; v[1] = a.y * r; v[2] = a.z * r; v[3] = a.w * r;
        v[4] = b.x * r; v[5] = b.y * r; v[6] = b.z * r; v[7] = b.w * r;
        u32x4 h, l;
        split8(v, h, l);
        *(u32x4 *)(xs + 8 * g) = h;
        *(u32x4 *)(xs + 8 * g + 4) = l;
    }
}

// xs <- hi/lo pairs of the tagged vector at base (threads [tid, nt)).
MBK_DEV void poll_split(const Params &p, float *xs, uint64_t base, uint32_t tag, int K, int tid, int nt, bool &ok) {
    for (int g = tid; g < K / 8; g += nt) {
        float v[8];
        if (!poll8(p, base, g, tag, v)) { ok = false; return; }
        u32x4 h, l;
        split8(v, h, l);
        *(u32x4 *)(xs + 8 * g) = h;
        *(u32x4 *)(xs + 8 * g + 4) = l;
    }
}

// ---- GEMV --------------------------------------------------------------------------------------------
// A wave owns tiles first + wave*n_wg, + 4*n_wg, ... (round r holds one tile
// per wave).  The first rounds come from the LDS staging buffer; the rest are
// read from HBM in chunks of kCh steps (16-byte loads per lane; steps past IT
// re-read the last one, so every chunk issues exactly kCh loads and the
// compiler's in-order load counting keeps the next chunk in flight while the
// current one is consumed).  Lane l covers row l / L and input groups
// (l % L) + it * L; the row sum is reduced over its L lanes.  Row sums go to
// LDS (ys); the operator's epilogue then runs as a short loop over them, so
// the streaming loop exists once in the kernel's code.

// Rounds of tiles of this interval held in a staging buffer.
MBK_DEV int gemv_pf_rounds(const Params &p, const Interval &iv) {
    const int fit = p.pf_bytes / (kWaves * iv.mat.IT * 1024);
    return min(fit, gemv_rounds(p, iv));
}

MBK_DEV float dot2(uint32_t w, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), __builtin_bit_cast(bf16x2, x), acc, false);
}

// a += 8 weights (one 16-byte chunk) times input group xv (hi/lo pairs).
MBK_DEV void fma16(const u32x4 &w, const float *xv, float *a) {
    const u32x4 h = *(const u32x4 *)xv, l = *(const u32x4 *)(xv + 4);
    a[0] = dot2(w.x, h.x, a[0]);
    a[1] = dot2(w.y, h.y, a[1]);
    a[2] = dot2(w.z, h.z, a[2]);
    a[3] = dot2(w.w, h.w, a[3]);
    a[0] = dot2(w.x, l.x, a[0]);
    a[1] = dot2(w.y, l.y, a[1]);
    a[2] = dot2(w.z, l.z, a[2]);
    a[3] = dot2(w.w, l.w, a[3]);
}

MBK_DEV void load_chunk(const uint8_t *blob, const MatGeom &g, int64_t t, int c, int lane, u32x4 *w) {
    const uint8_t *base = blob + chunk_offset(g, t, 0, lane);
#pragma unroll
    for (int u = 0; u < kCh; ++u) {
        const int it = min(c * kCh + u, g.IT - 1);
        w[u] = ld_stream(base + (size_t)it * 1024u);
    }
}

MBK_DEV void fma_chunk(const MatGeom &g, int c, int kl, const float *xs, const u32x4 *w, float *a) {
#pragma unroll
    for (int u = 0; u < kCh; ++u) {
        const int it = c * kCh + u;
        if (it < g.IT) fma16(w[u], xs + (kl + it * g.L) * 8, a);
    }
}

// Stores the row sum of the wave's k-th tile: ys[(k * kWaves + wave) * RT + row].
MBK_DEV void finish_row(float *a, const MatGeom &g, int k, int lane, int wave, float *ys) {
    const float acc = group_sum_n((a[0] + a[1]) + (a[2] + a[3]), g.L);
    a[0] = a[1] = a[2] = a[3] = 0.f;
    if ((lane & (g.L - 1)) == 0) ys[((k * kWaves + wave) << g.lrt) + (lane >> (6 - g.lrt))] = acc;
}

// Copies this workgroup's first rounds of tiles into a staging buffer, using
// threads [tid, nt) of the workgroup.
MBK_DEV void stage_gemv(const Params &p, const Interval &iv, uint8_t *pf, int tid, int nt) {
    const MatGeom &g = iv.mat;
    const int npf = gemv_pf_rounds(p, iv);
    const int first = first_item(p, iv);
    const int per_slot = g.IT * 64;
    const int units = npf * kWaves * per_slot;
    constexpr int U = 8;
    for (int u0 = tid; u0 < units; u0 += U * nt) {
        u32x4 v[U];
        bool ok[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int u = u0 + k * nt;
            const int slot = u / per_slot, rem = u % per_slot;
            const int64_t t = first + (int64_t)slot * p.n_wg;  // slot = round * kWaves + wave
            ok[k] = u < units && t < iv.n_items;
            if (ok[k]) v[k] = ld_stream(p.blob + chunk_offset(g, t, rem / 64, rem % 64));
        }
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (ok[k]) *(u32x4 *)(pf + (size_t)(u0 + k * nt) * 16u) = v[k];
    }
}

// Row sums of all this workgroup's tiles of the interval into ys.  A (kCh
// registers) holds chunk 0 of the wave's first HBM tile, issued by
// gemv_start before the input phase.
MBK_DEV void gemv_rows(const Params &p, const Interval &iv, const float *xs, const uint8_t *pf, u32x4 *A, float *ys) {
    const MatGeom &g = iv.mat;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int kl = lane & (g.L - 1);
    const int first = first_item(p, iv);
    const int npf = gemv_pf_rounds(p, iv);
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < npf; ++r) {
        if (first + (int64_t)(wave + kWaves * r) * p.n_wg >= iv.n_items) break;
        const u32x4 *w = (const u32x4 *)(pf + (size_t)(r * kWaves + wave) * g.IT * 1024u) + lane;
        for (int it0 = 0; it0 < g.IT; it0 += kCh) {
#pragma unroll
            for (int u = 0; u < kCh; ++u)
                if (it0 + u < g.IT) fma16(w[(it0 + u) * 64], xs + (kl + (it0 + u) * g.L) * 8, a);
        }
        finish_row(a, g, r, lane, wave, ys);
    }
    int k = npf;
    int64_t t = first + (int64_t)(wave + kWaves * k) * p.n_wg;
    if (t >= iv.n_items) return;
    const int64_t T = (int64_t)kWaves * p.n_wg;
    const int nch = (g.IT + kCh - 1) / kCh;
    u32x4 B[kCh];
    int c = 0;
    for (;;) {
        int64_t tn = t;
        int cn = c + 1;
        if (cn == nch) { cn = 0; tn += T; }
        bool more = tn < iv.n_items;
        load_chunk(p.blob, g, more ? tn : t, more ? cn : c, lane, B);
        fma_chunk(g, c, kl, xs, A, a);
        if (c == nch - 1) finish_row(a, g, k++, lane, wave, ys);
        if (!more) return;
        t = tn;
        c = cn;
        tn = t;
        cn = c + 1;
        if (cn == nch) { cn = 0; tn += T; }
        more = tn < iv.n_items;
        load_chunk(p.blob, g, more ? tn : t, more ? cn : c, lane, A);
        fma_chunk(g, c, kl, xs, B, a);
        if (c == nch - 1) finish_row(a, g, k++, lane, wave, ys);
        if (!more) return;
        t = tn;
        c = cn;
    }
}

// Issues chunk 0 of this wave's first HBM tile into A.
MBK_DEV void gemv_start(const Params &p, const Interval &iv, u32x4 *A) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t t = first_item(p, iv) + (int64_t)(wave + kWaves * gemv_pf_rounds(p, iv)) * p.n_wg;
    if (t < iv.n_items) load_chunk(p.blob, iv.mat, t, 0, lane, A);
}

// Packed row of local row index i (ys index), or -1 if that slot holds no row.
MBK_DEV int local_row(const Params &p, const Interval &iv, int i) {
    const MatGeom &g = iv.mat;
    const int slot = i >> g.lrt;  // (round * kWaves + wave)
    const int64_t t = first_item(p, iv) + (int64_t)slot * p.n_wg;
    if (t >= iv.n_items) return -1;
    const int64_t r = (t << g.lrt) + (i & (g.RT - 1));
    return r < g.rows ? (int)r : -1;
}

MBK_DEV int local_rows(const Params &p, const Interval &iv) { return gemv_rounds(p, iv) * kWaves * iv.mat.RT; }

// ---- GEMV operators ------------------------------------------------------------------------------------

// Q/K/V: bias, RoPE on query/key pairs; queries and this step's keys/values
// published as tagged vectors, keys/values appended to the cache at slot pos.
MBK_DEV void epi_qkv(const Params &p, const Interval &iv, const float *lds, const float *ys, uint32_t tag) {
    const int pos = step_pos(p), hd = p.hd, Q = p.nq * hd, KVr = p.nkv * hd, half = hd / 2;
    const bool has_bias = iv.bias_off != ~(uint64_t)0;
    const float *bias = lds + p.lds_bias;
    const float2 *rope = (const float2 *)(lds + p.lds_rope);
    uint16_t *kc = p.kv + ((size_t)iv.layer * 2 + 0) * p.nkv * p.S * hd;
    uint16_t *vc = p.kv + ((size_t)iv.layer * 2 + 1) * p.nkv * p.S * hd;
    const int n = local_rows(p, iv);
    for (int i = threadIdx.x; i < n; i += kThreads) {
        const int prow = local_row(p, iv, i);
        if (prow < 0) continue;
        const RowSrc s = packed_row_source(MAT_QKV, prow, hd, Q, KVr);
        if (s.which == 2) {
            const float v = ys[i] + (has_bias ? bias[Q + KVr + s.row] : 0.f);
            const int j = s.row / hd, d = s.row % hd;
            put(p, p.wl.v, s.row, v, tag);
            stc_b16(vc, (uint32_t)((((size_t)j * p.S + pos) * hd + d) * 2u), to_bf16(v));
            continue;
        }
        if (prow & 1) continue;  // the odd row is the partner of this pair
        const int boff = s.which == 0 ? 0 : Q;
        const int h = s.row / hd, m = s.row % hd;  // m < hd/2
        float u = ys[i], w = ys[i + 1];
        if (has_bias) { u += bias[boff + s.row]; w += bias[boff + s.row + half]; }
        const float2 cs = rope[m];
        const float r0 = u * cs.x - w * cs.y, r1 = w * cs.x + u * cs.y;
        if (s.which == 0) {
            put(p, p.wl.q, h * hd + m, r0, tag);
            put(p, p.wl.q, h * hd + m + half, r1, tag);
        } else {
            put(p, p.wl.k, h * hd + m, r0, tag);
            put(p, p.wl.k, h * hd + m + half, r1, tag);
            const size_t base = ((size_t)h * p.S + pos) * hd;
            stc_b16(kc, (uint32_t)((base + m) * 2u), to_bf16(r0));
            stc_b16(kc, (uint32_t)((base + m + half) * 2u), to_bf16(r1));
        }
    }
}

// x[r] = residual[r] + y[r] (output and down projections); xres holds the
// residual of this workgroup's rows by local row index.
MBK_DEV void epi_residual(const Params &p, const Interval &iv, const float *lds, const float *ys, uint32_t tag) {
    const float *xres = lds + p.lds_xres;
    const int n = local_rows(p, iv);
    for (int i = threadIdx.x; i < n; i += kThreads) {
        const int r = local_row(p, iv, i);
        if (r >= 0) put(p, p.wl.x, r, xres[i] + ys[i], tag);
    }
}

// a = silu(gate) * up over the interleaved gate/up rows.
MBK_DEV void epi_swiglu(const Params &p, const Interval &iv, const float *ys, uint32_t tag) {
    const int n = local_rows(p, iv);
    for (int i = threadIdx.x; i < n; i += kThreads) {
        const int r = local_row(p, iv, i);
        if (r < 0 || (r & 1)) continue;
        const float g = ys[i];
        put(p, p.wl.a, r >> 1, __fdividef(g, 1.f + __expf(-g)) * ys[i + 1], tag);
    }
}

// Logits out; greedy argmax through one 64-bit atomic max per workgroup, the
// last workgroup to finish publishes the index.
MBK_DEV void epi_lmhead(const Params &p, const Interval &iv, const float *ys) {
    uint64_t best = 0;
    const int n = local_rows(p, iv);
    for (int i = threadIdx.x; i < n; i += kThreads) {
        const int r = local_row(p, iv, i);
        if (r < 0) continue;
        if (p.logits) p.logits[r] = ys[i];
        const uint64_t key = ((uint64_t)ord_key(ys[i]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)r);
        best = key > best ? key : best;
    }
    for (int m = 1; m < 64; m <<= 1) {
        const uint64_t o = ((uint64_t)__shfl_xor((uint32_t)(best >> 32), m) << 32) | __shfl_xor((uint32_t)best, m);
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

// Input phase of a GEMV interval, run by threads [tid, nt): vectors into LDS;
// returns this thread's part of the RMSNorm sum of squares.
MBK_DEV float gemv_inputs(const Params &p, const Interval &iv, int ivi, uint32_t seq, float *lds, int tid, int nt,
                          bool &ok) {
    float *xs = lds + p.lds_xs, *xres = lds + p.lds_xres;
    const uint32_t xtag = iv.x_src < 0 ? 0u : tag_of(p, seq, iv.x_src);
    const int token = iv.x_src < 0 ? step_token(p) : 0;
    switch (iv.op) {
        case OP_O:
        case OP_DOWN: {
            // residual rows this workgroup rewrites
            const int n = local_rows(p, iv);
            for (int i = tid; i < n; i += nt) {
                const int r = local_row(p, iv, i);
                if (r < 0) continue;
                if (iv.x_src < 0) {
                    const uint16_t *e = (const uint16_t *)(p.blob + row_group_offset(p.embed, token, r >> 3));
                    xres[i] = bf16f(e[r & 7]);
                } else if (!poll1(p, p.wl.x, r, xtag, xres[i])) {
                    ok = false;
                    return 0.f;
                }
            }
            if (iv.op == OP_O) poll_split(p, xs, p.wl.o, tag_of(p, seq, ivi - 1), p.nq * p.hd, tid, nt, ok);
            else poll_split(p, xs, p.wl.a, tag_of(p, seq, ivi - 1), p.I, tid, nt, ok);
            return 0.f;
        }
        case OP_QKV:
            if (iv.bias_off != ~(uint64_t)0) {
                const uint16_t *b = (const uint16_t *)(p.blob + iv.bias_off);
                float *bias = lds + p.lds_bias;
                for (int i = tid; i < (p.nq + 2 * p.nkv) * p.hd; i += nt) bias[i] = bf16f(b[i]);
            }
            return norm_phase1(p, xs, iv.x_src < 0, token, xtag, iv.norm_off, p.H, tid, nt, ok);
        default:  // gate/up and LM head: RMS-normalised residual stream
            return norm_phase1(p, xs, false, 0, xtag, iv.norm_off, p.H, tid, nt, ok);
    }
}

// Compute phase of a GEMV interval (all threads, inputs in LDS).
MBK_DEV void gemv_compute(const Params &p, const Interval &iv, int ivi, uint32_t seq, float *lds, const float *red,
                          u32x4 *A) {
    float *xs = lds + p.lds_xs;
    if (iv.op == OP_QKV || iv.op == OP_GATEUP || iv.op == OP_LMHEAD) {
        float tot = 0.f;
        for (int w = 0; w < kPollWaves; ++w) tot += red[w];
        norm_phase2(xs, rsqrtf(tot / (float)p.H + p.eps), p.H);
        __syncthreads();
    }
    float *ys = lds + p.lds_ys;
    gemv_rows(p, iv, xs, staging(p, lds, ivi), A, ys);
    __syncthreads();
    const uint32_t tag = tag_of(p, seq, ivi);
    switch (iv.op) {
        case OP_QKV: epi_qkv(p, iv, lds, ys, tag); break;
        case OP_O:
        case OP_DOWN: epi_residual(p, iv, lds, ys, tag); break;
        case OP_GATEUP: epi_swiglu(p, iv, ys, tag); break;
        default: epi_lmhead(p, iv, ys); break;
    }
}

// ---- attention ---------------------------------------------------------------------------------------
// Decode attention for KV head j over cached positions [t0, t1), the G query
// heads of the group packed together so each key and value is read once
// (README mirror, "Current status": flash decoding, query heads sharing a KV
// head packed at long context).

struct Split { int nsplit, t0, t1; };

MBK_DEV Split split_range(const Params &p, int s, int pos) {
    const int Lc = pos + 1;
    int chunk = (Lc + p.max_splits - 1) / p.max_splits;
    if (chunk < p.attn_min_chunk) chunk = p.attn_min_chunk;
    Split r;
    r.nsplit = (Lc + chunk - 1) / chunk;
    r.t0 = s * chunk;
    r.t1 = min(Lc, r.t0 + chunk);
    return r;
}

// End of the staged range [t0, end): cached positions before `pos` that fit.
MBK_DEV int attn_stage_end(const Params &p, const Split &sp, int pos) {
    const int cap = p.pf_bytes / (4 * p.hd);
    return max(sp.t0, min(min(sp.t1, pos), sp.t0 + cap));
}

MBK_DEV void lse_merge(float &m, float &l, float *acc, float m2, float l2, const float *acc2, int n) {
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;
    const float c1 = __expf(m - mn), c2 = __expf(m2 - mn);
    l = l * c1 + l2 * c2;
    for (int e = 0; e < n; ++e) acc[e] = acc[e] * c1 + acc2[e] * c2;
    m = mn;
}

MBK_DEV const uint16_t *kv_block(const Params &p, int layer, int which, int j) {
    return p.kv + (((size_t)layer * 2 + which) * p.nkv + j) * p.S * p.hd;
}

// Copies the staged positions of this workgroup's first attention item to a
// staging buffer (K rows then V rows, hd bf16 each), using threads [tid, nt).
// Only positions written by earlier steps are staged.
MBK_DEV void stage_attn(const Params &p, const Interval &iv, uint8_t *pf, int tid, int nt) {
    const int item = first_item(p, iv);
    if (item >= iv.n_items) return;
    const int pos = step_pos(p), j = item / p.max_splits, s = item % p.max_splits;
    const Split sp = split_range(p, s, pos);
    if (s >= sp.nsplit) return;
    const int npos = attn_stage_end(p, sp, pos) - sp.t0, row16 = p.hd / 8;
    const int half_units = npos * row16, units = 2 * half_units;
    const uint16_t *Kb = kv_block(p, iv.layer, 0, j), *Vb = kv_block(p, iv.layer, 1, j);
    constexpr int U = 8;
    for (int u0 = tid; u0 < units; u0 += U * nt) {
        u32x4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int u = u0 + k * nt;
            if (u < units) {
                const int which = u >= half_units, rem = u - which * half_units;
                v[k] = ldc16(which ? Vb : Kb, (uint32_t)((size_t)(sp.t0 + rem / row16) * p.hd * 2 + (rem % row16) * 16));
            }
        }
#pragma unroll
        for (int k = 0; k < U; ++k)
            if (u0 + k * nt < units) *(u32x4 *)(pf + (size_t)(u0 + k * nt) * 16u) = v[k];
    }
}

// Input phase of attention item `item` (threads [tid, nt)): the G queries of
// its KV head, pre-scaled, and the key and value appended this step, rounded
// to bf16 exactly as the cache holds them.  LDS layout at lds_xres:
// [G][hd] queries, [hd] key, [hd] value.
MBK_DEV void attn_inputs(const Params &p, int item, int ivi, uint32_t seq, float *lds, int tid, int nt, bool &ok) {
    const int pos = step_pos(p), j = item / p.max_splits, s = item % p.max_splits;
    if (s >= split_range(p, s, pos).nsplit) return;
    const int G = p.gqa, hd = p.hd, qg = G * hd / 8, kg = hd / 8;
    const uint32_t tag = tag_of(p, seq, ivi - 1);
    float *dst = lds + p.lds_xres;
    for (int g = tid; g < qg + 2 * kg; g += nt) {
        float v[8];
        if (g < qg) {
            if (!poll8(p, p.wl.q, j * qg + g, tag, v)) { ok = false; return; }
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= p.scale;
        } else {
            const bool key = g < qg + kg;
            if (!poll8(p, key ? p.wl.k : p.wl.v, j * kg + g - qg - (key ? 0 : kg), tag, v)) { ok = false; return; }
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = bf16f(to_bf16(v[e]));
        }
        store8(dst + 8 * g, v);
    }
}

// Attention over positions [t0, t1) for the G query heads of KV head j.
// Lane (slot, dl) handles positions t0 + wave*PPW + slot + i*4*PPW and head
// dims dl*8..dl*8+7.  Positions come in blocks of KB steps; per block each
// lane rescales its running (m, l, acc) once, so a position costs one
// exponential per head.  At the end every lane rescales to the workgroup-wide
// maximum of each head, so slots and waves combine by plain sums in LDS.
// qkv: inputs from attn_inputs.  Result: per head {M, L, acc[hd]} in out
// ([G][hd + 4], acc unnormalised).
template <int G>
MBK_DEV void attend_range(const Params &p, int layer, int j, const Split &sp, int pos, bool staged, const uint8_t *pf,
                          const float *qkv, float *out) {
    constexpr int KB = kv_batch<G>();
    const int hd = p.hd, LP = hd / 8, PPW = 64 / LP, per_it = kWaves * PPW;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int dl = lane % LP, slot = lane / LP;
    const int t0 = sp.t0, t1 = sp.t1;
    const int tend = staged ? attn_stage_end(p, sp, pos) : t0;  // [t0, tend) is in LDS
    const int npos = tend - t0;
    const uint16_t *Kb = kv_block(p, layer, 0, j), *Vb = kv_block(p, layer, 1, j);
    float qf[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float4 a = *(const float4 *)(qkv + h * hd + dl * 8), b = *(const float4 *)(qkv + h * hd + dl * 8 + 4);
        qf[h][0] = a.x; qf[h][1] = a.y; qf[h][2] = a.z; qf[h][3] = a.w;
        qf[h][4] = b.x; qf[h][5] = b.y; qf[h][6] = b.z; qf[h][7] = b.w;
    }
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }
    const int n_it = (t1 - t0 + per_it - 1) / per_it;
    for (int b = 0; b < n_it; b += KB) {
        float kf[KB][8], vf[KB][8];
        bool val[KB];
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            const int t = t0 + wave * PPW + slot + (b + u) * per_it;
            val[u] = t < t1;
            if (t < tend) {  // staged
                unpack8(*(const u32x4 *)(pf + ((size_t)(t - t0) * hd + dl * 8) * 2u), kf[u]);
                unpack8(*(const u32x4 *)(pf + ((size_t)(npos + t - t0) * hd + dl * 8) * 2u), vf[u]);
            } else if (t == pos) {  // appended this step
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    kf[u][e] = qkv[G * hd + dl * 8 + e];
                    vf[u][e] = qkv[(G + 1) * hd + dl * 8 + e];
                }
            } else if (t < t1) {  // cached by earlier steps, not staged
                const uint32_t off = (uint32_t)(((size_t)t * hd + dl * 8) * 2u);
                unpack8(ldc16(Kb, off), kf[u]);
                unpack8(ldc16(Vb, off), vf[u]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) kf[u][e] = vf[u][e] = 0.f;
            }
        }
        float sc[KB][G];
#pragma unroll
        for (int u = 0; u < KB; ++u) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d = fmaf(qf[h][e], kf[u][e], d);
                d = group_sum_n(d, LP);
                sc[u][h] = val[u] ? d : -INFINITY;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float bm = sc[0][h];
#pragma unroll
            for (int u = 1; u < KB; ++u) bm = fmaxf(bm, sc[u][h]);
            const float mn = fmaxf(m[h], bm);
            if (mn != -INFINITY && mn != m[h]) {
                const float c = __expf(m[h] - mn);
                l[h] *= c;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= c;
                m[h] = mn;
            }
        }
#pragma unroll
        for (int u = 0; u < KB; ++u) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float pw = val[u] ? __expf(sc[u][h] - m[h]) : 0.f;
                l[h] += pw;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pw, vf[u][e], acc[h][e]);
            }
        }
    }
    // workgroup-wide maximum per head: slots of the wave, then waves (LDS)
    const int stride = hd + 4;
    float *wmax = out + G * stride;   // [kWaves][G]
    float *part = wmax + kWaves * G;  // [kWaves * PPW][G][stride]
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float mm = m[h];
        for (int msk = LP; msk < 64; msk <<= 1) mm = fmaxf(mm, __shfl_xor(mm, msk));
        if (lane == 0) wmax[wave * G + h] = mm;
    }
    __syncthreads();
    const int contrib = wave * PPW + slot;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float M = wmax[h];
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, wmax[w * G + h]);
        const float f = m[h] == -INFINITY ? 0.f : __expf(m[h] - M);
        float *r = part + ((size_t)contrib * G + h) * stride;
        if (dl == 0) { r[0] = M; r[1] = l[h] * f; }
#pragma unroll
        for (int e = 0; e < 8; ++e) r[4 + dl * 8 + e] = acc[h][e] * f;
    }
    __syncthreads();
    const int nc = kWaves * PPW;
    for (int idx = threadIdx.x; idx < G * hd; idx += kThreads) {
        const int h = idx / hd, e = idx % hd;
        float ll = 0.f, aa = 0.f;
        for (int c = 0; c < nc; ++c) {
            const float *r = part + ((size_t)c * G + h) * stride;
            ll += r[1];
            aa += r[4 + e];
        }
        float *o = out + (size_t)h * stride;
        if (e == 0) { o[0] = part[h * stride]; o[1] = ll; }
        o[4 + e] = aa;
    }
    __syncthreads();
}

// One attention item: KV head j, split s of the cached context.  A single
// split writes o directly; with several, each split stores its partial and
// the last split to arrive (one atomic per split) merges all partials in
// split order, so the result does not depend on arrival order.
template <int G>
MBK_DEV void attention_item(const Params &p, int ivi, int layer, int j, int s, bool staged, float *lds, uint32_t tag) {
    const int pos = step_pos(p), hd = p.hd, stride = hd + 4;
    const Split sp = split_range(p, s, pos);
    if (s >= sp.nsplit) return;
    float *res = lds + p.lds_xs;  // [G][stride] + scratch
    attend_range<G>(p, layer, j, sp, pos, staged, staging(p, lds, ivi), lds + p.lds_xres, res);
    if (sp.nsplit == 1) {
        for (int idx = threadIdx.x; idx < G * hd; idx += kThreads) {
            const int h = idx / hd, e = idx % hd;
            const float *r = res + (size_t)h * stride;
            put(p, p.wl.o, (j * G + h) * hd + e, r[4 + e] / r[1], tag);
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
        const bool last = atom_add(cnt, 1u) == (uint32_t)sp.nsplit - 1u;
        if (last) {
            stc_u(cnt, 0u);
            __builtin_amdgcn_s_waitcnt(0);  // the reset lands before this group's output does
        }
        last_s = last;
    }
    __syncthreads();
    if (!last_s) return;
    // load every partial of head group j into LDS, then merge in split order
    float *all = res;  // [nsplit][G][stride]
    const uint64_t gbase = p.wl.part + ((uint64_t)(j * p.max_splits) * G) * stride * 4u;
    const int n16 = sp.nsplit * G * stride / 4;
    for (int idx = threadIdx.x; idx < n16; idx += kThreads)
        *(u32x4 *)(all + 4 * idx) = ldc16(p.ws, (uint32_t)(gbase + 16u * idx));
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * hd; idx += kThreads) {
        const int h = idx / hd, e = idx % hd;
        float mm = -INFINITY, ll = 0.f, aa = 0.f;
        for (int q = 0; q < sp.nsplit; ++q) {
            const float *r = all + ((size_t)q * G + h) * stride;
            lse_merge(mm, ll, &aa, r[0], r[1], &r[4 + e], 1);
        }
        put(p, p.wl.o, (j * G + h) * hd + e, aa / ll, tag);
    }
}

// Attention items of this workgroup.  The first item's inputs were loaded in
// the interval's input phase and its cached keys/values staged; further items
// (only when there are more items than workgroups) load their own.
template <int G>
MBK_DEV bool attention_compute(const Params &p, const Interval &iv, int ivi, uint32_t seq, float *lds) {
    const int first = first_item(p, iv);
    const uint32_t tag = tag_of(p, seq, ivi);
    for (int i = first; i < iv.n_items; i += p.n_wg) {
        if (i != first) {
            bool ok = true;
            attn_inputs(p, i, ivi, seq, lds, threadIdx.x, kThreads, ok);
            if (__syncthreads_or(!ok)) return false;
        }
        attention_item<G>(p, ivi, iv.layer, i / p.max_splits, i % p.max_splits, i == first, lds, tag);
        __syncthreads();
    }
    return true;
}

// ---- interval dispatch -------------------------------------------------------------------------------

// One-time per launch: the interval table and this step's RoPE row go to LDS.
MBK_DEV void load_static(const Params &p, float *lds) {
    const uint32_t *src = (const uint32_t *)p.iv;
    uint32_t *dst = (uint32_t *)(lds + p.lds_tab);
    const int nw = p.n_intervals * (int)(sizeof(Interval) / 4);
    for (int i = threadIdx.x; i < nw; i += kThreads) dst[i] = src[i];
    const int pos = step_pos(p), half = p.hd / 2;
    for (int i = threadIdx.x; i < 2 * half; i += kThreads) lds[p.lds_rope + i] = p.rope[(size_t)pos * 2 * half + i];
    __syncthreads();
}

// Descriptor of interval ivi from the LDS copy, forced into scalar registers.
MBK_DEV Interval interval_at(const Params &p, const float *lds, int ivi) {
    constexpr int nw = (int)(sizeof(Interval) / 4);
    const uint32_t *src = (const uint32_t *)(lds + p.lds_tab) + ivi * nw;
    uint32_t w[nw];
#pragma unroll
    for (int i = 0; i < nw; ++i) w[i] = __builtin_amdgcn_readfirstlane(src[i]);
    Interval v;
    __builtin_memcpy(&v, w, sizeof v);
    return v;
}

// Stages what interval ivi reads that does not depend on results of this
// step into staging buffer ivi & 1, using threads [tid, nt).
MBK_DEV void stage(const Params &p, float *lds, int ivi, int tid, int nt) {
    const Interval iv = interval_at(p, lds, ivi);
    if (iv.op == OP_ATTN) stage_attn(p, iv, staging(p, lds, ivi), tid, nt);
    else stage_gemv(p, iv, staging(p, lds, ivi), tid, nt);
}

// Runs interval ivi.  Waves 0-1 load its inputs while waves 2-3 stage
// interval `next` (-1: none).  False when a bounded wait expired.
template <int G>
MBK_DEV bool run_interval(const Params &p, int ivi, int next, float *lds, float *red) {
    const Interval iv = interval_at(p, lds, ivi);
    const uint32_t seq = step_seq(p);
    stamp(p, ivi, 0);
    if (ivi == 0 && blockIdx.x == 0 && threadIdx.x == 0) {
        __hip_atomic_store(ws_ptr<uint64_t>(p, p.wl.argkey), (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!p.step_from_ws) {  // this step's inputs, for launches that read them from the workspace
            uint32_t *ctrl = ws_ptr<uint32_t>(p, p.wl.ctrl);
            stc_u(ctrl + 3, (uint32_t)p.token);
            stc_u(ctrl + 4, (uint32_t)p.pos);
            stc_u(ctrl + 5, p.seq);
        }
    }
    const bool gemv = iv.op != OP_ATTN;
    const int first = first_item(p, iv);
    // every workgroup joins the LM head's argmax count, tiles or not
    const bool work = first < iv.n_items || iv.op == OP_LMHEAD;
    u32x4 A[kCh];
    if (gemv && work) gemv_start(p, iv, A);
    const int wave = threadIdx.x >> 6;
    bool ok = true;
    if (wave >= kPollWaves) {
        if (next >= 0) stage(p, lds, next, threadIdx.x - kPollWaves * 64, kThreads - kPollWaves * 64);
    } else if (work) {
        if (gemv) {
            float ss = gemv_inputs(p, iv, ivi, seq, lds, threadIdx.x, kPollWaves * 64, ok);
            ss = group_sum<64>(ss);
            if ((threadIdx.x & 63) == 0) red[wave] = ss;
        } else {
            attn_inputs(p, first, ivi, seq, lds, threadIdx.x, kPollWaves * 64, ok);
        }
    }
    if (__syncthreads_or(!ok)) return false;
    if (work) stamp(p, ivi, 1);
    if (work) {
        if (gemv) gemv_compute(p, iv, ivi, seq, lds, red, A);
        else if (!attention_compute<G>(p, iv, ivi, seq, lds)) return false;
    }
    __syncthreads();
    stamp(p, ivi, 2);
    return true;
}

}  // namespace mbk
